// kla_bwd.h -- launch descriptor of the backward pass (kla_bwd.hip), shared
// with the C-ABI front end.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "kla_internal.h"

namespace kla {

// Every pointer is a device pointer.  q, k, v, dO, dq, dk, dv in the input
// dtype; everything else fp32.  l0, eta0, dlT, detaT may be null (1, 0, 0, 0);
// gl0, geta0 may be null (not written).
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* a;
    const float* qn;
    const float* r;
    const float* l0;
    const float* eta0;
    const void* dO;
    const float* dlT;
    const float* detaT;
    // gradients (outputs) of q, k, v, a, qn, r, l0, eta0
    void* gq;
    void* gk;
    void* gv;
    float* ga;
    float* gqn;
    float* gr;
    float* gl0;
    float* geta0;
    float* ws;          // workspace, ws_stride floats per (b,h)
    size_t ws_stride;
    int B, H, T, dk, dv;
};

bool bwd_supported(int dk, int dv);
// Workspace floats per (b,h): the precision after every token, q dq per
// token (per key dim; summed over key dims when isotropic) and the diagonal
// qn partial, rounded up to 256 bytes.
size_t bwd_ws_stride(int B, int H, int T, int dk, int cov);
hipError_t launch_bwd(const BwdArgs& a, int dtype, int cov, hipStream_t s);

}  // namespace kla
