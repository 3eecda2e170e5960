// kla_step.hip -- gfx950 decode step: one token per (b,h), state in place.
//
// Sources: "Kalman Delta Networks: Uncertainty-aware Associative Memory"
// (abstract: constant-memory decoding; diagonal and isotropic variants) and
// "Kalman Linear Attention: Parallel Bayesian Filtering For Efficient Language
// Modelling and State Tracking" (gist.science explainer, method §1-§2).
//
// The same recurrence as the forward pass with T = 1, in information form:
//   lp = l / (a^2 + qn l),  l' = lp + b,  g = lp a / l,
//   eta'[i,:] = g eta[i,:] + (k_i / r) v,   o = sum_i (q_i / l'_i) eta'[i,:]
// (b = k_i^2 / r for the diagonal model, |k|^2 / (d_k r) for the isotropic
// one).  The step is bound by reading and writing the fp32 state eta once:
// each (b,h) is one workgroup whose threads stream rows of eta with 16-byte
// accesses and reduce the readout across row groups in LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kla_common.h"
#include "kla_internal.h"

namespace kla {
namespace {

constexpr int kStepThreads = 256;

template <typename TIn, int DK, int DV, bool ISO>
__global__ __launch_bounds__(kStepThreads) void kla_step_kernel(StepArgs p) {
    constexpr int NT = kStepThreads;
    constexpr int VQ = DV / 4;          // value quads per row
    constexpr int NRG = NT / VQ;        // row groups
    static_assert(NT % VQ == 0 && DK <= NT, "layout");
    __shared__ float gate[DK], kap[DK], qsc[DK];
    __shared__ f32x4 part[NRG][VQ];
    __shared__ float vsh[DV];
    __shared__ float red[NT / 64];

    const int tid = threadIdx.x;
    const int bh = blockIdx.x, h = bh % p.H;
    const TIn* q = (const TIn*)p.q + (size_t)bh * DK;
    const TIn* k = (const TIn*)p.k + (size_t)bh * DK;
    const TIn* v = (const TIn*)p.v + (size_t)bh * DV;
    const float r = p.r[bh];
    const float rho = 1.f / r;

    if (tid < DV) vsh[tid] = (float)v[tid];
    if constexpr (!ISO) {
        if (tid < DK) {
            const size_t si = (size_t)bh * DK + tid;
            const float l = p.l[si], a = p.a[si], qn = p.qn[(size_t)h * DK + tid];
            const float kv = (float)k[tid];
            const float lp = l / __builtin_fmaf(qn, l, a * a);
            const float ln = lp + kv * kv * rho;
            gate[tid] = lp * a / l;
            kap[tid] = kv * rho;
            qsc[tid] = (float)q[tid] / ln;
            p.l[si] = ln;
        }
    } else {
        float s = 0.f;
        if (tid < DK) {
            const float kv = (float)k[tid];
            s = kv * kv;
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) s += __shfl_xor(s, m, 64);
        if ((tid & 63) == 0) red[tid >> 6] = s;
        __syncthreads();
        float ksq = 0.f;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) ksq += red[w];
        const float l = p.l[bh], a = p.a[bh], qn = p.qn[bh];
        const float lp = l / __builtin_fmaf(qn, l, a * a);
        const float ln = lp + ksq * rho * (1.f / (float)DK);
        if (tid < DK) {
            gate[tid] = lp * a / l;
            kap[tid] = (float)k[tid] * rho;
            qsc[tid] = (float)q[tid] / ln;
        }
        __syncthreads();  // every thread has read l before it is overwritten
        if (tid == 0) p.l[bh] = ln;
    }
    __syncthreads();

    const int jq = tid % VQ, rg = tid / VQ;
    const f32x4 vv = *(const f32x4*)&vsh[4 * jq];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float* eta = p.eta + (size_t)bh * DK * DV;
    for (int i = rg; i < DK; i += NRG) {
        f32x4* row = (f32x4*)(eta + (size_t)i * DV) + jq;
        f32x4 e = *row;
        e = gate[i] * e + kap[i] * vv;
        *row = e;
        acc += qsc[i] * e;
    }
    part[rg][jq] = acc;
    __syncthreads();
    if (tid < VQ) {
        f32x4 s = part[0][tid];
        for (int g2 = 1; g2 < NRG; ++g2) s += part[g2][tid];
        TIn* o = (TIn*)p.o + (size_t)bh * DV;
        *(typename Quad<TIn>::V*)(o + 4 * tid) = Quad<TIn>::make(s);
    }
}

template <typename TIn, bool ISO>
hipError_t dispatch(const StepArgs& a, hipStream_t s) {
    if (a.dk != a.dv) return hipErrorInvalidValue;
    const dim3 grid(a.B * a.H), block(kStepThreads);
    switch (a.dk) {
        case 16: hipLaunchKernelGGL((kla_step_kernel<TIn, 16, 16, ISO>), grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL((kla_step_kernel<TIn, 32, 32, ISO>), grid, block, 0, s, a); break;
        case 64: hipLaunchKernelGGL((kla_step_kernel<TIn, 64, 64, ISO>), grid, block, 0, s, a); break;
        case 128: hipLaunchKernelGGL((kla_step_kernel<TIn, 128, 128, ISO>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool step_supported(int dk, int dv, int dtype, int cov) {
    (void)dtype;
    (void)cov;
    return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}

hipError_t launch_step(const StepArgs& a, int dtype, int cov, hipStream_t s) {
    if (dtype == DT_BF16)
        return cov ? dispatch<bf16, true>(a, s) : dispatch<bf16, false>(a, s);
    return cov ? dispatch<float, true>(a, s) : dispatch<float, false>(a, s);
}

}  // namespace kla

// ---------------------------------------------------------------- T == 0
// An empty sequence leaves the state untouched: lT = l0, etaT = eta0
// (l0 = 1, eta0 = 0 when not given).
namespace kla {
namespace {
__global__ void kla_fwd_empty_kernel(FwdArgs p, long long nl, long long neta) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (p.lT && i < nl) p.lT[i] = p.l0 ? p.l0[i] : 1.f;
    if (p.etaT && i < neta) p.etaT[i] = p.eta0 ? p.eta0[i] : 0.f;
}
}  // namespace

hipError_t launch_fwd_empty(const FwdArgs& a, int cov, hipStream_t s) {
    const long long bh = (long long)a.B * a.H;
    const long long nl = cov ? bh : bh * a.dk;
    const long long neta = bh * a.dk * a.dv;
    const long long n = nl > neta ? nl : neta;
    if (n == 0) return hipSuccess;
    const int blk = 256;
    hipLaunchKernelGGL(kla_fwd_empty_kernel, dim3((unsigned)((n + blk - 1) / blk)), dim3(blk), 0, s,
                       a, nl, neta);
    return hipGetLastError();
}
}  // namespace kla
