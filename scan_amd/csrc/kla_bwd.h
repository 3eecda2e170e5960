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
    // token-serial kernel run after the chunked one: when gate_nt > 0 a
    // workgroup works only if one of the gate_nt ints at ws + flag_off of its
    // (b,h) is set (a sequence the chunked kernels handed back)
    int gate_nt;
    size_t flag_off;
    // polls of the chunked reverse sweep's in-workgroup wait before it hands
    // the (b,h) back (KLA_BWD_SPIN overrides; 0 forces the hand-back)
    int spin;
};

// Workspace of the chunked backward (floats from the start of a (b,h)'s
// block).  The first 4 T dk + dk floats are the token-serial kernel's (its
// trajectory and the qn partial at 4 T dk, which both paths write), then
// the chunk-range flags of the row tiles, then the chunked kernels' own data:
// q.dq per token and key dim [T][dk], the row tiles' partials of dv [NT][T][dk]
// and dr [NT][T4], the precision at chunk starts [nch][dk], <detaT, eta_T> [dk].
struct BcLayout {
    size_t flags, q, dvp, drp, lst, z, total;
    int t4;
};
__host__ __device__ inline BcLayout bc_layout(int T, int D) {
    BcLayout L;
    const size_t td = (size_t)T * D;
    const int nt = D / 64, nch = (T + 15) / 16;
    L.t4 = (T + 3) / 4 * 4;
    L.flags = 4 * td + D;
    L.q = (L.flags + 4 + 63) / 64 * 64;
    L.dvp = L.q + td;
    L.drp = L.dvp + (size_t)nt * td;
    L.lst = L.drp + (size_t)nt * L.t4;
    L.z = L.lst + (size_t)nch * D;
    L.total = (L.z + D + 63) / 64 * 64;
    return L;
}

bool bwd_supported(int dk, int dv);
// Workspace floats per (b,h): the precision after every token, q dq per
// token (per key dim; summed over key dims when isotropic) and the diagonal
// qn partial, rounded up to 256 bytes; with the chunked kernels bc_layout's.
size_t bwd_ws_stride(int B, int H, int T, int dk, int cov, int dtype);
hipError_t launch_bwd(const BwdArgs& a, int dtype, int cov, hipStream_t s);

// The chunked backward on the matrix cores (kla_bwd_chunk.hip): bf16, T >= 1,
// diagonal with dk = dv in {64, 128} or isotropic with dk = dv = 64;
// KLA_BWD_IMPL=rows or plain turns it off.
bool bwd_chunk_supported(int dk, int dv, int cov, int dtype, int T);
// Its three launches (forward sweep, reverse sweep, dv/dr combine); the
// caller then runs the token-serial kernel gated on the flags.
hipError_t launch_bwd_chunk(const BwdArgs& a, int dtype, int cov, hipStream_t s);

}  // namespace kla
