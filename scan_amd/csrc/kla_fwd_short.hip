// kla_fwd_short.hip -- gfx950 forward for short sequences (T <= 32): chunked
// prefill into cached states and multi-token decode at large batch.
//
// Sources: "Kalman Delta Networks: Uncertainty-aware Associative Memory"
// (abstract: constant-memory decoding; diagonal and isotropic variants) and
// "Kalman Linear Attention: Parallel Bayesian Filtering For Efficient Language
// Modelling and State Tracking" (gist.science explainer, method §1-§2).
//
// The recurrence of the forward pass, token by token in information form:
//   lp = l / (a^2 + qn l),  l' = lp + b,  g = lp a / l,
//   eta'[i,:] = g_i eta[i,:] + (k_i / r) v,   o = sum_i (q_i / l'_i) eta'[i,:]
// (b = k_i^2 / r for the diagonal model, |k|^2 / (d_k r) for the isotropic
// one; g and l are then scalars per head).
//
// With few tokens per (b,h) the forward is bound by the state: reading eta0
// and writing etaT (2 d_k d_v fp32 per (b,h)) outweighs the tokens.  The
// threads of a (b,h) keep its eta in registers for the whole sequence, each
// a slice (row group rg, value quad jq: rows rg*RPT .. rg*RPT+RPT-1 of
// columns 4jq..4jq+3), so the state crosses HBM once in each direction, in
// 16-byte accesses, and a thread reads its rows' coefficients as vectors.
// Tokens go in blocks of four.  The coefficients of a block (gates, k/r,
// q/l') are formed by one lane per key dim, with the hardware reciprocal
// (about 1 ulp), and staged in LDS; every thread
// applies the block's tokens to its rows and leaves a partial readout per
// token, and the partials are summed over row groups.  The next block's
// inputs are loaded while a block is applied, and its coefficients are staged
// before the block's outputs are stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kla_common.h"
#include "kla_short.h"

namespace kla {
namespace {

constexpr int kShortThreads = 256;
#ifndef KLA_SHORT_TB
#define KLA_SHORT_TB 4
#endif
constexpr int kShortTB = KLA_SHORT_TB;  // tokens per block

// Threads per (b,h): each thread holds at least four state rows of one value
// quad, so small heads share a workgroup (16 heads of d 16, 8 of d 32, 2 of
// d 64) and every workgroup carries about the same work.
template <int D>
struct ShortLayout {
    // state elements per thread, at least: 32 (16 at d16, where the v rows of
    // a block need 16 threads per head); more threads per head mean more LDS
    // traffic per element (coefficients, partials, row-group sums)
    static constexpr int EPT = D == 16 ? 16 : 32;
    static constexpr int NTH = D * D / EPT < kShortThreads ? D * D / EPT : kShortThreads;
    static constexpr int NH = kShortThreads / NTH;  // (b,h) per workgroup
    static constexpr int VQ = D / 4;                 // value quads per row
    static constexpr int RG = NTH / VQ;              // row groups of a (b,h)
    static constexpr int RPT = D / RG;               // rows per thread
    static_assert(RPT % 4 == 0 && kShortTB * VQ <= NTH && NTH * NH == kShortThreads, "layout");
};

// One buffer of each suffices: a block's coefficients are read (state
// update) before the first barrier of its iteration and the next block's are
// written after it; the partials are written before that barrier and read
// between it and the second.
template <int D, bool ISO>
struct ShortSm {
    static constexpr int NH = ShortLayout<D>::NH, NTH = ShortLayout<D>::NTH;
    // block coefficients per (b,h): gate per key dim (per head for iso), k/r
    // and q/l' per key dim, v rows
    alignas(16) float g[NH][kShortTB][ISO ? 4 : D];
    alignas(16) float kap[NH][kShortTB][D];
    alignas(16) float qs[NH][kShortTB][D];
    alignas(16) float v[NH][kShortTB][D];
    // partial readouts: one value quad per thread and token
    alignas(16) f32x4 part[NH][kShortTB][NTH];
    float red[kShortTB][kShortThreads / 64];  // iso, (b,h) over 4 waves: |k|^2 per wave
};

template <typename TIn, int D, bool ISO>
__global__ __launch_bounds__(kShortThreads) void kla_fwd_short_kernel(FwdArgs p) {
    typedef ShortLayout<D> Ly;
    constexpr int NT = kShortThreads, TB = kShortTB, NTH = Ly::NTH, NH = Ly::NH;
    constexpr int VQ = Ly::VQ, RG = Ly::RG, RPT = Ly::RPT;
    typedef typename Quad<TIn>::V QV;
    __shared__ ShortSm<D, ISO> sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = NH == 1 ? 0 : tid / NTH, lt = NH == 1 ? tid : tid % NTH;  // (b,h) in the workgroup, thread in it
    const int nbh = p.B * p.H, bh_ = NH == 1 ? (int)blockIdx.x : (int)blockIdx.x * NH + grp;
    const bool valid = NH == 1 || bh_ < nbh;
    const int bh = valid ? bh_ : nbh - 1;  // loads of a spare group stay in bounds
    const int h = bh % p.H;
    const int jq = lt % VQ, rg = lt / VQ;
    const size_t row0 = (size_t)bh * p.T;
    const TIn* q = (const TIn*)p.q;
    const TIn* k = (const TIn*)p.k;
    const TIn* v = (const TIn*)p.v;
    TIn* o = (TIn*)p.o;

    // the thread's slice of eta (information form)
    f32x4 e[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const size_t off = ((size_t)bh * D + rg * RPT + m) * D + 4 * jq;
        e[m] = p.eta0 ? *(const f32x4*)(p.eta0 + off) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // precision: of key dim lt (diag, lt < D) or of the head (iso, every
    // thread of the group runs the same scalar recursion)
    const bool kd = lt < D;
    const int kdim = kd ? lt : D - 1;
    float l;
    if constexpr (!ISO) l = p.l0 ? p.l0[(size_t)bh * D + kdim] : 1.f;
    else l = p.l0 ? p.l0[bh] : 1.f;
    const float qn_i = !ISO ? p.qn[(size_t)h * D + kdim] : 0.f;

    // raw inputs of a block.  Every load is unconditional, at an index
    // clamped into the sequence (the block's last token, key dim D-1).
    struct Raw {
        TIn k[TB], q[TB];
        float a[TB], r[TB], qn[TB];
        QV vq;
    };
    auto load = [&](int t0, Raw& x) {
        const int nb = p.T - t0 < TB ? p.T - t0 : TB;
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            const size_t t = row0 + t0 + (u < nb ? u : nb - 1), idx = t * D + kdim;
            x.k[u] = k[idx];
            x.q[u] = q[idx];
            x.r[u] = p.r[t];
            if constexpr (!ISO) {
                x.a[u] = p.a[idx];
                x.qn[u] = 0.f;
            } else {
                x.a[u] = p.a[t];
                x.qn[u] = p.qn[t];
            }
        }
        const int uv = lt / VQ < nb ? lt / VQ : nb - 1;
        x.vq = *(const QV*)(v + (row0 + t0 + uv) * D + 4 * jq);
    };
    // iso: |k_t|^2 of the group's head.  A group inside one wave sums with
    // lane exchanges; a group of four waves leaves one sum per wave in LDS.
    auto ksq_sum = [&](const Raw& x, int u) {
        const float kv = kd ? (float)x.k[u] : 0.f;
        float s = kv * kv;
        constexpr int W = NTH < 64 ? NTH : 64;
#pragma unroll
        for (int m = 1; m < W; m <<= 1) s += __shfl_xor(s, m, 64);
        return s;
    };
    auto ksq_waves = [&](const Raw& x) {
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            const float s = ksq_sum(x, u);
            if (lane == 0) sm.red[u][wave] = s;
        }
    };
    constexpr bool RED = ISO && NTH > 64;  // iso sums pass through LDS
    // coefficients of a block's tokens (and its v rows) into LDS; advances
    // the precision through the block
    auto coefs = [&](const Raw& x, int nb) {
        if constexpr (!ISO) {
            if (kd) {
#pragma unroll
                for (int u = 0; u < TB; ++u) {
                    if (u < nb) {
                        const float a = x.a[u], kv = (float)x.k[u];
                        const float rho = fast_rcp(x.r[u]);
                        const float rd = fast_rcp(__builtin_fmaf(qn_i, l, a * a));
                        const float ln = __builtin_fmaf(kv * kv, rho, l * rd);
                        sm.g[grp][u][lt] = a * rd;  // lp a / l with lp = l rd
                        sm.kap[grp][u][lt] = kv * rho;
                        sm.qs[grp][u][lt] = (float)x.q[u] * fast_rcp(ln);
                        l = ln;
                    }
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < TB; ++u) {
                float ksq = 0.f;
                if constexpr (RED) {
#pragma unroll
                    for (int w = 0; w < NTH / 64; ++w) ksq += sm.red[u][grp * (NTH / 64) + w];
                } else {
                    ksq = ksq_sum(x, u);
                }
                if (u < nb) {
                    const float a = x.a[u], rho = fast_rcp(x.r[u]);
                    const float rd = fast_rcp(__builtin_fmaf(x.qn[u], l, a * a));
                    const float ln = __builtin_fmaf(ksq * (1.f / (float)D), rho, l * rd);
                    if (lt == 0) sm.g[grp][u][0] = a * rd;  // lp a / l with lp = l rd
                    if (kd) {
                        sm.kap[grp][u][lt] = (float)x.k[u] * rho;
                        sm.qs[grp][u][lt] = (float)x.q[u] * fast_rcp(ln);
                    }
                    l = ln;
                }
            }
        }
        if (lt / VQ < nb) *(f32x4*)&sm.v[grp][lt / VQ][4 * jq] = Quad<TIn>::to_f32(x.vq);
    };
    // the compiler is kept from sinking a raw value's first use into a branch:
    // every register of the block is taken here, so the waits for its loads
    // are here too and none is left pending into the next block
    auto settle = [&](Raw& x) {
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            asm volatile("" : "+v"(x.k[u]), "+v"(x.q[u]), "+v"(x.a[u]), "+v"(x.r[u]));
            if constexpr (ISO) asm volatile("" : "+v"(x.qn[u]));
        }
        asm volatile("" : "+v"(x.vq));
    };

    {
        Raw x;
        load(0, x);
        settle(x);
        if constexpr (RED) {
            ksq_waves(x);
            lds_barrier();
        }
        coefs(x, p.T < TB ? p.T : TB);
        lds_barrier();
    }
    for (int t0 = 0; t0 < p.T; t0 += TB) {
        const int nb = p.T - t0 < TB ? p.T - t0 : TB;
        const bool more = t0 + TB < p.T;
        // the next block's inputs are in flight during this block's update
        Raw x;
        load(more ? t0 + TB : t0, x);
        // ---- this block's tokens on the thread's rows, partial readouts
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            if (u < nb) {
                const f32x4 vv = *(const f32x4*)&sm.v[grp][u][4 * jq];
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const int i0 = rg * RPT;
                const float gs = sm.g[grp][u][0];  // iso: the head's gate
#pragma unroll
                for (int m4 = 0; m4 < RPT; m4 += 4) {
                    f32x4 gv;
                    if constexpr (!ISO) gv = *(const f32x4*)&sm.g[grp][u][i0 + m4];
                    const f32x4 kv = *(const f32x4*)&sm.kap[grp][u][i0 + m4];
                    const f32x4 qv = *(const f32x4*)&sm.qs[grp][u][i0 + m4];
#pragma unroll
                    for (int x4 = 0; x4 < 4; ++x4) {
                        const float g = ISO ? gs : gv[x4];
                        e[m4 + x4] = g * e[m4 + x4] + kv[x4] * vv;
                        acc += qv[x4] * e[m4 + x4];
                    }
                }
                sm.part[grp][u][lt] = acc;
            }
        }
        settle(x);
        if constexpr (RED) ksq_waves(x);
        lds_barrier();
        // ---- readouts: sums over the row groups (one value quad per thread)
        const bool orow = lt < nb * VQ;
        f32x4 osum = {0.f, 0.f, 0.f, 0.f};
        if (orow) {
            osum = sm.part[grp][lt / VQ][jq];
#pragma unroll
            for (int r2 = 1; r2 < RG; ++r2) osum += sm.part[grp][lt / VQ][r2 * VQ + jq];
        }
        // ---- the next block's coefficients, then this block's outputs
        if (more) coefs(x, p.T - t0 - TB < TB ? p.T - t0 - TB : TB);
        if (orow && valid) *(QV*)(o + (row0 + t0 + lt / VQ) * D + 4 * jq) = Quad<TIn>::make(osum);
        lds_barrier();
    }
    // ---- final state
    if (!valid) return;
    if (p.etaT) {
#pragma unroll
        for (int m = 0; m < RPT; ++m) *(f32x4*)(p.etaT + ((size_t)bh * D + rg * RPT + m) * D + 4 * jq) = e[m];
    }
    if (p.lT) {
        if constexpr (!ISO) {
            if (kd) p.lT[(size_t)bh * D + lt] = l;
        } else if (lt == 0) {
            p.lT[bh] = l;
        }
    }
}

template <typename TIn, bool ISO>
hipError_t dispatch(const FwdArgs& a, hipStream_t s) {
    const dim3 block(kShortThreads);
    const int nbh = a.B * a.H;
    auto grid = [&](int nh) { return dim3((nbh + nh - 1) / nh); };
    switch (a.dk) {
        case 16: hipLaunchKernelGGL((kla_fwd_short_kernel<TIn, 16, ISO>), grid(ShortLayout<16>::NH), block, 0, s, a); break;
        case 32: hipLaunchKernelGGL((kla_fwd_short_kernel<TIn, 32, ISO>), grid(ShortLayout<32>::NH), block, 0, s, a); break;
        case 64: hipLaunchKernelGGL((kla_fwd_short_kernel<TIn, 64, ISO>), grid(ShortLayout<64>::NH), block, 0, s, a); break;
        case 128: hipLaunchKernelGGL((kla_fwd_short_kernel<TIn, 128, ISO>), grid(ShortLayout<128>::NH), block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool fwd_short_supported(int dk, int dv, int T) {
    return T >= 1 && T <= kShortTMax && dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}

hipError_t launch_fwd_short(const FwdArgs& a, int dtype, int cov, hipStream_t s) {
    if (!fwd_short_supported(a.dk, a.dv, a.T)) return hipErrorInvalidValue;
    if (dtype == DT_BF16) return cov ? dispatch<bf16, true>(a, s) : dispatch<bf16, false>(a, s);
    return cov ? dispatch<float, true>(a, s) : dispatch<float, false>(a, s);
}

}  // namespace kla
