// kla_internal.h -- launch descriptors shared by the C-ABI front end
// (kla_api.cpp) and the gfx950 kernels.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kla {

// Arguments of one forward launch.  Every pointer is a device pointer.
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* a;
    const float* qn;
    const float* r;
    const float* l0;    // may be null (l0 = 1)
    const float* eta0;  // may be null (eta0 = 0)
    void* o;
    float* lT;          // may be null
    float* etaT;        // may be null
    int B, H, T, dk, dv;
    int n_vtiles;       // workgroups per (b,h) along the value dim
    // diagonal wave-specialised kernel, bf16: run the precision as a
    // wavefront-level Mobius scan instead of the per-lane serial recursion
    bool chain_scan = false;

    // Fused block prologue (conv_w > 0, diagonal wave-specialised kernel):
    // q, k, v then hold the projections before the causal convolution, a the
    // decay's pre-activation za in the storage dtype, qn its pre-activation
    // zqn and r the pre-activation zr; the kernel forms
    // q = silu(conv(q)), ..., a = sigmoid(za), qn = softplus(zqn),
    // r = softplus(zr) + r_eps.
    int conv_w = 0;                       // taps W, 1..4 (0: no prologue)
    const float* conv_wt[3] = {};         // taps of q, k, v: [H, d, W]
    const float* conv_b[3] = {};          // biases [H, d] or null (zero)
    const void* conv_s[3] = {};           // states [B, H, W-1, d] or null (zero)
    float r_eps = 0.f;

    // Sequence split (diagonal, wave-specialised kernel only).  With nseg > 1
    // the workgroup of segment s handles tokens [s*seg_len, min(T,(s+1)*seg_len))
    // of its (b,h), starts from seg_l0 and a zero state, and leaves its local
    // result for the carry and correction passes.  nseg == 1 is the plain
    // forward and ignores the seg_* pointers.
    int nseg = 1;
    int seg_len = 0;
    const float* seg_l0 = nullptr;  // [BH, nseg, dk] precision before each segment
    float* seg_m = nullptr;         // [BH, nseg, dk, dv] local final mean state
    float* seg_d = nullptr;         // [BH, nseg, dk] total gate (decay) of each segment
    float* seg_lend = nullptr;      // [BH, dk] precision after the last segment
    void* seg_qhat = nullptr;       // q (.) gate product since segment start, in
                                    // 16-token tiles (qhat_tile_offset)
};

// Block prologue input x (q, k or v projections, [B,H,T,d] in TIn) at token
// t of sequence bh, channel c, as fp32: the row itself for t >= 0, before the
// sequence the convolution state row W-1+t ([B,H,W-1,d]) or zero.
template <typename TIn>
__device__ __forceinline__ float pro_x(const TIn* x, const void* st, int bh, int T, int W, int d, int t, int c) {
    if (t >= 0) return (float)x[((size_t)bh * T + t) * d + c];
    const int sr = W - 1 + t;
    return st && sr >= 0 ? (float)((const TIn*)st)[((size_t)bh * (W - 1) + sr) * d + c] : 0.f;
}

// Element offset of q-hat (token t of sequence bh, key dim i) in the tiled
// layout the correction pass reads: per (bh, 16-token tile, 32-dim block kb)
// 512 elements, lane (c16 = t % 16, g = i % 32 / 8) holding 8 consecutive
// dims at (g * 16 + c16) * 8, so one 64-lane 16-byte load covers a block.
__host__ __device__ inline size_t qhat_tile_offset(int bh, int T, int dk, int t, int i) {
    const size_t ntile = (size_t)(T + 15) / 16;
    return (((size_t)bh * ntile + t / 16) * (dk / 32) + i / 32) * 512 + ((i % 32) / 8 * 16 + t % 16) * 8 + i % 8;
}

// Segment lengths are multiples of kSegBlk tokens, the unit of the segment
// precision products.
constexpr int kSegBlk = 256;

// Workspace of the sequence split: every array above, 256-byte aligned.
struct SegWorkspace {
    size_t off_P, off_l0, off_d, off_lend, off_m, off_qhat, off_ok, bytes;
};
SegWorkspace seg_workspace(int B, int H, int T, int dk, int dv, int es, int nseg);
// Segments per (b,h) for a diagonal forward on the wave-specialised kernel
// (1 = no split).
int fwd_diag_nseg(int B, int H, int T, int dk, int dv, int nvt);
int fwd_diag_seg_len(int T, int nseg);
// The passes around the split forward (kla_fwd_seg.hip).
// ok: [BH, nseg, 2] flags (per 64 key dims), written by the warm-up and
// read by the exact passes.
hipError_t launch_seg_warm(const FwdArgs& a, int* ok, int dtype, hipStream_t s);
// The exact passes 1 and 2 (block products, then the precision carry by the
// last workgroup to finish); ok also holds their completion counter, after
// the flags, which the warm-up zeroes.
hipError_t launch_seg_mobius(const FwdArgs& a, float* P, int* ok, int dtype, hipStream_t s);
hipError_t launch_seg_carry_m(const FwdArgs& a, hipStream_t s);
hipError_t launch_seg_correct(const FwdArgs& a, int dtype, hipStream_t s);

// Device scratch of klaFwdNoAlloc (kla_noalloc.hip): the largest sequence-
// split workspace that entry point serves, and the address of the current
// device's copy (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);

struct StepArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* a;
    const float* qn;
    const float* r;
    float* l;
    float* eta;
    void* o;
    int B, H, dk, dv;
};

enum Dt { DT_F32 = 0, DT_BF16 = 1 };

// Each returns hipSuccess or the launch error.  Shapes were validated by the
// caller; the functions return hipErrorInvalidValue for a (dk, dv, dtype)
// combination they were not instantiated for.
hipError_t launch_fwd_diag(const FwdArgs& a, int dtype, hipStream_t s);
hipError_t launch_fwd_diag_pipe(const FwdArgs& a, int dtype, hipStream_t s);
bool fwd_diag_pipe_supported(int dk, int dv, int nvt, int dtype);
// Value tiles of the wave-specialised diagonal forward (0 = shape not built).
int fwd_diag_pipe_vtiles(int dk, int dv, int dtype);
hipError_t launch_fwd_iso(const FwdArgs& a, int dtype, hipStream_t s);
// Wave-specialised pipelined isotropic forward: bf16 dk = dv in {64, 128},
// fp32 dk = dv = 64, 64 or 32 value columns per workgroup.
bool fwd_iso_pipe_supported(int dk, int dv, int nvt, int dtype);
int fwd_iso_pipe_vtiles(int B, int H, int dk, int dv);
hipError_t launch_fwd_iso_pipe(const FwdArgs& a, int dtype, hipStream_t s);
hipError_t launch_step(const StepArgs& a, int dtype, int cov, hipStream_t s);
hipError_t launch_fwd_empty(const FwdArgs& a, int cov, hipStream_t s);

bool fwd_diag_supported(int dk, int dv, int dtype);
bool fwd_iso_supported(int dk, int dv, int dtype);
bool step_supported(int dk, int dv, int dtype, int cov);
// Value-dim tiles per (b,h) (workgroups per sequence) the forward uses.
int fwd_diag_vtiles(int B, int H, int T, int dk, int dv);
int fwd_iso_vtiles(int B, int H, int dk);

}  // namespace kla
