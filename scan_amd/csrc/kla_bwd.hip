// kla_bwd.hip -- gfx950 backward pass of the KLA forward (diagonal and
// isotropic precision).
//
// Sources: "Kalman Linear Attention: Parallel Bayesian Filtering For Efficient
// Language Modelling and State Tracking" (fugumt abstract page: the filter is
// a primitive for parallel training; gist.science explainer, method §1-§3 for
// the recurrence) and "Kalman Delta Networks: Uncertainty-aware Associative
// Memory" (abstract: diagonal and isotropic variants).
//
// Forward, per (b,h), information form (key dim i, value column j):
//   D_t = a_t^2 + qn l_{t-1},  g_t = a_t / D_t,  l_t = l_{t-1} / D_t + k_t^2 / r_t
//   eta_t = g_t eta_{t-1} + (k_t / r_t) v_t^T,   o_t = sum_i (q_t[i] / l_t[i]) eta_t[i,:]
// Backward of L with the upstream dO = dL/do, dlT, detaT:
//   dq_t[i]   = S_t[i] / l_t[i],             S_t[i] = sum_j dO_t[j] eta_t[i,j]
//   ebar_t    = g_{t+1} ebar_{t+1} + (q_t / l_t) dO_t^T     (ebar_T = detaT, g_T = 1)
//   U_t[i]    = sum_j ebar_t[i,j] v_t[j],   dv_t[j] = sum_i ebar_t[i,j] k_t[i] / r_t
// The adjoint of log g_t needs sum_j ebar_t[i,j] eta_{t-1}[i,j], a per-token
// product of two dk x dv states.  It telescopes instead: with
// P_t = sum_j ebar_t[i,j] eta_t[i,j] one has P_{t-1} = P_t - kap_t U_t + q_{t-1} dq_{t-1},
// so  dlog g_t[i] = B[i] + sum_{s>=t} (q_s[i] dq_s[i] - kap_s[i] U_s[i]),
// B[i] = sum_j detaT[i,j] eta_T[i,j]  (kap = k / r), a reverse cumulative sum
// of per-token scalars.  Its terms nearly cancel when a token's write
// dominates the carried state (a small gate next to a large k v / r), so
// the states eta and ebar, their row sums, the cumulative sum and the
// precision recursion are carried in fp64 (the staged coefficients are fp32,
// the same values in both sweeps, so the state products are exact in fp64).  The precision adjoint is then one
// scalar reverse recursion per key dim (per head when isotropic):
//   lbar_t   += -q_t dq_t / l_t
//   dk_t      = U_t / r_t + lbar_t 2 k_t / r_t            (iso: 2 k_t[i] / (dk r_t))
//   dr_t      = -sum_i (kap_t[i] U_t[i] + lbar_t k_t[i]^2 / r_t) / r_t
//   da_t      = -lbar_t 2 a_t l_{t-1} / D_t^2 + dlog g_t (qn l_{t-1} - a_t^2) / (a_t D_t)
//   dqn      += -lbar_t l_{t-1}^2 / D_t^2 - dlog g_t l_{t-1} / D_t
//   lbar_{t-1} = lbar_t a_t^2 / D_t^2 - dlog g_t qn / D_t
// dl0 = lbar_{-1}, deta0 = g_0 ebar_0.
//
// One workgroup runs all of this for its (b,h) (small heads share a
// workgroup) in two sweeps over the tokens, the state slice of every thread
// in registers (rows rg*RPT.. of value quad jq):
//   sweep 1, forward: eta, dq, and per token l_t and q dq into the workspace;
//   sweep 2, backward: ebar, U, dv, the precision adjoint, dk, da, dr, dqn.
// Tokens go in blocks of TB; one lane per key dim forms the block's
// coefficients, every thread applies the block to its rows and leaves
// per-row and per-column partial sums in LDS, and the key-dim lanes and
// value-quad lanes sum them.  The diagonal qn is shared by the batch: each
// (b,h) leaves its partial in the workspace and a second kernel sums over b.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <type_traits>

#include "kla_bwd.h"
#include "kla_common.h"

namespace kla {
namespace {

constexpr int kBwdThreads = 256;

typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <int D>
struct BwdLayout {
    static constexpr int EPT = D == 16 ? 16 : 32;   // state elements per thread, at least
    static constexpr int NTH = D * D / EPT < kBwdThreads ? D * D / EPT : kBwdThreads;
    static constexpr int NH = kBwdThreads / NTH;    // (b,h) per workgroup
    static constexpr int VQ = D / 4;                // value quads per row
    static constexpr int RG = NTH / VQ;             // row groups
    static constexpr int RPT = D / RG;              // rows per thread
    static constexpr int TB = D == 128 ? 2 : 4;     // tokens per block (LDS of the row sums)
    static_assert(RPT % 4 == 0 && TB * VQ <= NTH && NTH * NH == kBwdThreads && D <= NTH, "layout");
};

template <int D>
struct BwdSm {
    typedef BwdLayout<D> Ly;
    static constexpr int NH = Ly::NH, NTH = Ly::NTH, VQ = Ly::VQ, TB = Ly::TB;
    // block coefficients per key dim: gate (of the next token in sweep 2),
    // k / r, q / l; the block's v and dO rows
    alignas(16) float g[NH][TB][D];
    alignas(16) float kap[NH][TB][D];
    alignas(16) float cq[NH][TB][D];
    alignas(16) float v[NH][TB][D];
    alignas(16) float dO[NH][TB][D];
    // per-row partial sums (over a thread's value quad): [token][quad][row];
    // rows padded by two doubles, so that the 32 value quads of a wave store
    // to different banks
    alignas(16) double rpart[NH][TB][VQ][D + 2];
    // per-column partial sums (over a thread's rows): one quad per thread
    alignas(16) f32x4 cpart[NH][TB][NTH];
    double red[NH][TB][2][2];  // cross-wave sums of the key-dim lanes
};

// Sum over the D key-dim lanes of a group, returned to every lane of the
// group.  Every thread of the workgroup calls it at the same point (lanes
// past the key dims pass 0): at D = 128 the two key-dim waves combine
// through LDS between workgroup barriers.
template <int D, int NH, int TB>
__device__ __forceinline__ double kdim_sum(double x, double (&red)[NH][TB][2][2], int grp, int u, int slot,
                                           int lt) {
    constexpr int W = D < 64 ? D : 64;
#pragma unroll
    for (int m = 1; m < W; m <<= 1) x += __shfl_xor(x, m, 64);
    if constexpr (D > 64) {
        if ((lt & 63) == 0 && lt < D) red[grp][u][lt >> 6][slot] = x;
        __syncthreads();
        x = red[grp][u][0][slot] + red[grp][u][1][slot];
        __syncthreads();
    }
    return x;
}

__device__ __forceinline__ f64x4 to_f64(f32x4 x) { return f64x4{x[0], x[1], x[2], x[3]}; }

// gate of one token from the precision before it, in fp64 (the same
// arithmetic in both sweeps, so the fp32 gates they stage match bit for bit);
// rd_out receives 1 / (a^2 + qn l)
__device__ __forceinline__ double gate_of(double a, double qn, double l, double* rd_out) {
    const double rd = 1. / __builtin_fma(qn, l, a * a);
    *rd_out = rd;
    return a * rd;
}

template <typename TIn, int D, bool ISO>
__global__ __launch_bounds__(kBwdThreads) void kla_bwd_kernel(BwdArgs p) {
    typedef BwdLayout<D> Ly;
    constexpr int TB = Ly::TB, NTH = Ly::NTH, NH = Ly::NH, VQ = Ly::VQ, RG = Ly::RG, RPT = Ly::RPT;
    constexpr int NL = ISO ? 1 : D;
    __shared__ BwdSm<D> sm;

    const int tid = threadIdx.x;
    const int grp = NH == 1 ? 0 : tid / NTH, lt = NH == 1 ? tid : tid % NTH;
    const int nbh = p.B * p.H, bh_ = NH == 1 ? (int)blockIdx.x : (int)blockIdx.x * NH + grp;
    // after the chunked kernels: only the (b,h) they handed back
    if (p.gate_nt > 0) {
        int any = 0;
        for (int g2 = 0; g2 < NH; ++g2) {
            const int b2 = NH == 1 ? (int)blockIdx.x : (int)blockIdx.x * NH + g2;
            if (b2 < nbh) {
                const int* fl = (const int*)(p.ws + (size_t)b2 * p.ws_stride + p.flag_off);
                for (int t2 = 0; t2 < p.gate_nt; ++t2) any |= fl[t2];
            }
        }
        if (!any) return;  // uniform over the workgroup
    }
    const bool valid = NH == 1 || bh_ < nbh;
    const int bh = valid ? bh_ : nbh - 1;  // a spare group stays in bounds and stores nothing
    const int h = bh % p.H;
    const int jq = lt % VQ, rg = lt / VQ;
    const int T = p.T;
    const size_t row0 = (size_t)bh * T;
    const TIn* q = (const TIn*)p.q;
    const TIn* k = (const TIn*)p.k;
    const TIn* v = (const TIn*)p.v;
    const TIn* dOg = (const TIn*)p.dO;
    const bool kd = lt < D;  // key-dim lane
    const int i = kd ? lt : D - 1;
    // workspace of this (b,h): l_t [T][NL] and q dq [T][NL] in fp64 (iso:
    // summed over key dims), then the diagonal qn partial [D] fp32
    double* wl = (double*)(p.ws + (size_t)bh * p.ws_stride);
    double* wqdq = wl + (size_t)T * NL;
    float* wdqn = (float*)(wqdq + (size_t)T * NL);

    const float qn_i = ISO ? 0.f : p.qn[(size_t)h * D + i];
    const double l_start = ISO ? (p.l0 ? p.l0[bh] : 1.f) : (p.l0 ? p.l0[(size_t)bh * D + i] : 1.f);

    // ---------------------------------------------------------------- sweep 1
    f64x4 e[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const size_t off = ((size_t)bh * D + rg * RPT + m) * D + 4 * jq;
        e[m] = p.eta0 ? to_f64(*(const f32x4*)(p.eta0 + off)) : f64x4{0., 0., 0., 0.};
    }
    double l = l_start;  // the precision recursion runs in fp64
    // stages v and dO rows (one value quad per thread) of tokens t0.. into LDS
    auto stage_rows = [&](int t0, int nb) {
        if (lt < TB * VQ && lt / VQ < nb) {
            const size_t t = row0 + t0 + lt / VQ;
            *(f32x4*)&sm.v[grp][lt / VQ][4 * jq] = Quad<TIn>::to_f32(*(const typename Quad<TIn>::V*)(v + t * D + 4 * jq));
            *(f32x4*)&sm.dO[grp][lt / VQ][4 * jq] = Quad<TIn>::to_f32(*(const typename Quad<TIn>::V*)(dOg + t * D + 4 * jq));
        }
    };
    // forward coefficients of a block (advances l): g, k/r into LDS, l_t into
    // the workspace
    auto fwd_coefs = [&](int t0, int nb) {
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            if (u < nb) {
                const size_t t = row0 + t0 + u;
                const double kv = (float)k[t * D + i];
                const double rt = p.r[t];
                double a, qn, b;
                if constexpr (ISO) {
                    a = p.a[t];
                    qn = p.qn[t];
                    b = kdim_sum<D, NH, TB>(kd ? kv * kv : 0., sm.red, grp, u, 0, lt) / ((double)D * rt);
                } else {
                    a = p.a[t * D + i];
                    qn = qn_i;
                    b = kv * kv / rt;
                }
                double rd;
                const double g = gate_of(a, qn, l, &rd);
                l = __builtin_fma(l, rd, b);
                if (kd) {
                    sm.g[grp][u][i] = (float)g;
                    sm.kap[grp][u][i] = (float)(kv / rt);
                    if ((!ISO || lt == 0) && valid) wl[(size_t)(t0 + u) * NL + (ISO ? 0 : i)] = l;
                }
            }
        }
    };
    if (T > 0) {
        stage_rows(0, T < TB ? T : TB);
        fwd_coefs(0, T < TB ? T : TB);
    }
    __syncthreads();
    for (int t0 = 0; t0 < T; t0 += TB) {
        const int nb = T - t0 < TB ? T - t0 : TB;
        // ---- the block on the thread's rows; per-row S partials
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            if (u < nb) {
                const f64x4 vv = to_f64(*(const f32x4*)&sm.v[grp][u][4 * jq]);
                const f64x4 dd = to_f64(*(const f32x4*)&sm.dO[grp][u][4 * jq]);
#pragma unroll
                for (int m4 = 0; m4 < RPT; m4 += 4) {
                    const f32x4 gv = *(const f32x4*)&sm.g[grp][u][rg * RPT + m4];
                    const f32x4 kv = *(const f32x4*)&sm.kap[grp][u][rg * RPT + m4];
                    double sp[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        e[m4 + x] = (double)gv[x] * e[m4 + x] + (double)kv[x] * vv;
                        const f64x4 pr = e[m4 + x] * dd;
                        sp[x] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
                    }
                    *(f64x2*)&sm.rpart[grp][u][jq][rg * RPT + m4] = f64x2{sp[0], sp[1]};
                    *(f64x2*)&sm.rpart[grp][u][jq][rg * RPT + m4 + 2] = f64x2{sp[2], sp[3]};
                }
            }
        }
        __syncthreads();
        // ---- dq of the block (key-dim lanes; the others compute along and
        // store nothing), then the next block's coefficients
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            if (u < nb) {
                double s = 0.;
#pragma unroll 8
                for (int x = 0; x < VQ; ++x) s += sm.rpart[grp][u][x][i];
                const size_t t = row0 + t0 + u;
                const double lt_ = wl[(size_t)(t0 + u) * NL + (ISO ? 0 : i)];
                const double qv = (float)q[t * D + i];
                const double dq = s / lt_;
                if (kd && valid) ((TIn*)p.gq)[t * D + i] = (TIn)(float)dq;
                // q dq with q / l rounded to fp32 exactly as sweep 2 stages it
                // for the readout adjoint, so the telescoping sum stays exact
                const double qdq = (double)(float)(qv / lt_) * s;
                if constexpr (ISO) {
                    const double tot = kdim_sum<D, NH, TB>(kd ? qdq : 0., sm.red, grp, u, 1, lt);
                    if (lt == 0 && valid) wqdq[t0 + u] = tot;
                } else {
                    if (kd && valid) wqdq[(size_t)(t0 + u) * D + i] = qdq;
                }
            }
        }
        const bool more = t0 + TB < T;
        if (more) {
            const int nb2 = T - t0 - TB < TB ? T - t0 - TB : TB;
            stage_rows(t0 + TB, nb2);
            fwd_coefs(t0 + TB, nb2);
        }
        __syncthreads();
    }
    // boundary term of the gate adjoint: B[i] = sum_j detaT[i,j] eta_T[i,j];
    // the state registers then take ebar_T = detaT
    double Bsum = 0.;
    {
#pragma unroll
        for (int m4 = 0; m4 < RPT; m4 += 4) {
            double sp[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const size_t off = ((size_t)bh * D + rg * RPT + m4 + x) * D + 4 * jq;
                const f64x4 dt = p.detaT ? to_f64(*(const f32x4*)(p.detaT + off)) : f64x4{0., 0., 0., 0.};
                const f64x4 pr = e[m4 + x] * dt;
                sp[x] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
                e[m4 + x] = dt;
            }
            *(f64x2*)&sm.rpart[grp][0][jq][rg * RPT + m4] = f64x2{sp[0], sp[1]};
            *(f64x2*)&sm.rpart[grp][0][jq][rg * RPT + m4 + 2] = f64x2{sp[2], sp[3]};
        }
        __syncthreads();
        if (kd) {
#pragma unroll 8
            for (int x = 0; x < VQ; ++x) Bsum += sm.rpart[grp][0][x][i];
        }
        if constexpr (ISO) Bsum = kdim_sum<D, NH, TB>(Bsum, sm.red, grp, 0, 0, lt);
        __syncthreads();
    }

    // ---------------------------------------------------------------- sweep 2
    double lbar = ISO ? (p.dlT ? p.dlT[bh] : 0.f) : (p.dlT ? p.dlT[(size_t)bh * D + i] : 0.f);
    double cum = Bsum;
    double dqn_acc = 0.;
    // backward coefficients of block [t0, t0+nb): gate of the token after
    // each (1 past the end), k/r, q/l; and the v, dO rows
    auto bwd_coefs = [&](int t0, int nb) {
        stage_rows(t0, nb);
        if (kd) {
#pragma unroll
            for (int u = 0; u < TB; ++u) {
                if (u < nb) {
                    const int t = t0 + u;
                    const size_t tt = row0 + t;
                    const double lt_ = wl[(size_t)t * NL + (ISO ? 0 : i)];
                    double gn = 1., rd;
                    if (t + 1 < T) {
                        const double an = ISO ? p.a[tt + 1] : p.a[(tt + 1) * D + i];
                        const double qnn = ISO ? p.qn[tt + 1] : qn_i;
                        gn = gate_of(an, qnn, lt_, &rd);
                    }
                    sm.g[grp][u][i] = (float)gn;
                    sm.kap[grp][u][i] = (float)((double)(float)k[tt * D + i] / (double)p.r[tt]);
                    sm.cq[grp][u][i] = (float)((double)(float)q[tt * D + i] / lt_);
                }
            }
        }
    };
    const int nblk = (T + TB - 1) / TB;
    if (T > 0) bwd_coefs((nblk - 1) * TB, T - (nblk - 1) * TB);
    __syncthreads();
    for (int blk = nblk - 1; blk >= 0; --blk) {
        const int t0 = blk * TB;
        const int nb = T - t0 < TB ? T - t0 : TB;
        // ---- ebar over the block's tokens, last first; U and dv partials
#pragma unroll
        for (int u = TB - 1; u >= 0; --u) {
            if (u < nb) {
                const f64x4 vv = to_f64(*(const f32x4*)&sm.v[grp][u][4 * jq]);
                const f64x4 dd = to_f64(*(const f32x4*)&sm.dO[grp][u][4 * jq]);
                f64x4 cs = {0., 0., 0., 0.};
#pragma unroll
                for (int m4 = 0; m4 < RPT; m4 += 4) {
                    const f32x4 gv = *(const f32x4*)&sm.g[grp][u][rg * RPT + m4];
                    const f32x4 cv = *(const f32x4*)&sm.cq[grp][u][rg * RPT + m4];
                    const f32x4 kv = *(const f32x4*)&sm.kap[grp][u][rg * RPT + m4];
                    double sp[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        e[m4 + x] = (double)gv[x] * e[m4 + x] + (double)cv[x] * dd;
                        const f64x4 pr = e[m4 + x] * vv;
                        sp[x] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
                        cs += (double)kv[x] * e[m4 + x];
                    }
                    *(f64x2*)&sm.rpart[grp][u][jq][rg * RPT + m4] = f64x2{sp[0], sp[1]};
                    *(f64x2*)&sm.rpart[grp][u][jq][rg * RPT + m4 + 2] = f64x2{sp[2], sp[3]};
                }
                sm.cpart[grp][u][lt] = f32x4{(float)cs[0], (float)cs[1], (float)cs[2], (float)cs[3]};
            }
        }
        __syncthreads();
        // ---- dv of the block (value-quad lanes)
        if (lt < TB * VQ && lt / VQ < nb) {
            const int u = lt / VQ;
            f32x4 s = sm.cpart[grp][u][jq];
#pragma unroll
            for (int r2 = 1; r2 < RG; ++r2) s += sm.cpart[grp][u][r2 * VQ + jq];
            if (valid) *(typename Quad<TIn>::V*)((TIn*)p.gv + (row0 + t0 + u) * D + 4 * jq) = Quad<TIn>::make(s);
        }
        // ---- the precision adjoint over the block (key-dim lanes; the others
        // compute along and store nothing), last first
#pragma unroll
        for (int u = TB - 1; u >= 0; --u) {
            if (u < nb) {
                const int t = t0 + u;
                const size_t tt = row0 + t;
                double Uv = 0.;
#pragma unroll 8
                for (int x = 0; x < VQ; ++x) Uv += sm.rpart[grp][u][x][i];
                const double kv = (float)k[tt * D + i];
                const double rt = p.r[tt];
                const double kap = (float)(kv / rt);  // the staged k/r of the state update
                const double lt_ = wl[(size_t)t * NL + (ISO ? 0 : i)];
                const double lprev = t == 0 ? l_start : wl[(size_t)(t - 1) * NL + (ISO ? 0 : i)];
                double a, qn, qdq, kU;
                if constexpr (ISO) {
                    a = p.a[tt];
                    qn = p.qn[tt];
                    qdq = wqdq[t];
                    kU = kdim_sum<D, NH, TB>(kd ? kap * Uv : 0., sm.red, grp, u, 0, lt);
                } else {
                    a = p.a[tt * D + i];
                    qn = qn_i;
                    qdq = wqdq[(size_t)t * D + i];
                    kU = kap * Uv;
                }
                lbar -= qdq / lt_;
                cum += qdq - kU;
                const double dlg = cum;
                const double den = a * a + qn * lprev;
                const double rd = 1. / den, rd2 = rd * rd;
                const double bscale = ISO ? 1. / (double)D : 1.;
                const double dk = Uv / rt + lbar * 2. * kv * bscale / rt;
                if (kd && valid) ((TIn*)p.gk)[tt * D + i] = (TIn)(float)dk;
                // dr: -(kap U + lbar b_i) / r, summed over key dims
                const double drp = -(kap * Uv + lbar * kv * kv * bscale / rt) / rt;
                const double dr = kdim_sum<D, NH, TB>(kd ? drp : 0., sm.red, grp, u, 1, lt);
                if (lt == 0 && valid) p.gr[tt] = (float)dr;
                const double da = -lbar * 2. * a * lprev * rd2 + dlg * (qn * lprev - a * a) * rd / a;
                const double dqn = -lbar * lprev * lprev * rd2 - dlg * lprev * rd;
                if constexpr (ISO) {
                    if (lt == 0 && valid) {
                        p.ga[tt] = (float)da;
                        p.gqn[tt] = (float)dqn;
                    }
                } else {
                    if (kd && valid) p.ga[tt * D + i] = (float)da;
                    dqn_acc += dqn;
                }
                lbar = lbar * a * a * rd2 - dlg * qn * rd;
            }
        }
        if (blk > 0) bwd_coefs(t0 - TB, TB);
        __syncthreads();
    }
    // ---- initial-state gradients: deta0 = g_0 ebar_0, dl0 = lbar_{-1}
    if (T > 0 && kd) {
        const double a0 = ISO ? p.a[row0] : p.a[row0 * D + i];
        const double qn0 = ISO ? p.qn[row0] : qn_i;
        double rd;
        sm.g[grp][0][i] = (float)gate_of(a0, qn0, l_start, &rd);
    }
    __syncthreads();
    if (!valid) return;
    if (p.geta0) {
#pragma unroll
        for (int m4 = 0; m4 < RPT; m4 += 4) {
            const f32x4 gv = T > 0 ? *(const f32x4*)&sm.g[grp][0][rg * RPT + m4] : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const f64x4 r4 = (double)gv[x] * e[m4 + x];
                *(f32x4*)(p.geta0 + ((size_t)bh * D + rg * RPT + m4 + x) * D + 4 * jq) =
                    f32x4{(float)r4[0], (float)r4[1], (float)r4[2], (float)r4[3]};
            }
        }
    }
    if (kd) {
        if (p.gl0 && (!ISO || lt == 0)) p.gl0[(size_t)bh * NL + (ISO ? 0 : i)] = (float)lbar;
        if (!ISO) wdqn[i] = (float)dqn_acc;
    }
}

// Diagonal precision: the same two sweeps with the global reads of a token
// block issued one block ahead.  The key-dim lanes load the next block's
// k, r, a, q (and, in sweep 2, the stored precisions and q dq) into
// registers before the current block's state update and turn them into the
// LDS coefficients after it; the staging lanes do the same for the v and dO
// rows.  The precisions of the current block stay in registers, and the
// per-token sum of dr over key dims is a wave reduction (the two waves of
// dk = 128 combine after the block's closing barrier).  The arithmetic and
// its order are those of kla_bwd_kernel.
// Reciprocal and quotient in fp64 for positive finite operands: the hardware
// reciprocal estimate refined by two Newton-Raphson steps, r <- r + r (1 - x r),
// and the quotient a r corrected once by its residual a - b q.  (The compiler's
// IEEE division sequence is several times longer; the backward's serial
// adjoint divides about a dozen times per token.)
__device__ __forceinline__ double rcp64(double x) {
    double r = __builtin_amdgcn_rcp(x);
    double e = __builtin_fma(-x, r, 1.0);
    r = __builtin_fma(r, e, r);
    e = __builtin_fma(-x, r, 1.0);
    return __builtin_fma(r, e, r);
}
__device__ __forceinline__ double div64(double a, double b) {
    const double r = rcp64(b);
    const double q = a * r;
    return __builtin_fma(__builtin_fma(-b, q, a), r, q);
}
// gate of one token from the precision before it (as gate_of)
__device__ __forceinline__ double gate_r(double a, double qn, double l, double* rd_out) {
    const double rd = rcp64(__builtin_fma(qn, l, a * a));
    *rd_out = rd;
    return a * rd;
}

// The key dims of a (b,h) may be split over NRG workgroups (RD rows each, all
// D value columns): the rows of the state, their precision chains and their
// gradients are independent, and only dv and dr sum over key dims; those
// workgroups leave partial sums in the workspace for kla_bwd_combine.  With
// few (b,h) this fills the GPU and divides the per-token state work.
template <int D, int NRG>
struct BwdRL {
    static constexpr int RD = D / NRG;                                    // rows per workgroup
    static constexpr int NTH = NRG == 1 ? BwdLayout<D>::NTH : kBwdThreads;
    static constexpr int NH = NRG == 1 ? BwdLayout<D>::NH : 1;            // (b,h) per workgroup
    static constexpr int VQ = D / 4;                                      // value quads per row
    static constexpr int RG = NTH / VQ;                                   // row groups
    static constexpr int RPT = RD / RG;                                   // rows per thread
    static constexpr int TB = NRG == 1 ? BwdLayout<D>::TB : 2 * NRG;      // tokens per block
    static_assert(RPT % 4 == 0 && TB * VQ <= NTH && NTH * NH == kBwdThreads && RD <= NTH, "layout");
};

template <class Ly, int D>
struct BwdSmR {
    static constexpr int NH = Ly::NH, NTH = Ly::NTH, VQ = Ly::VQ, TB = Ly::TB, RD = Ly::RD;
    alignas(16) float g[NH][TB][RD];
    alignas(16) float kap[NH][TB][RD];
    alignas(16) float cq[NH][TB][RD];
    alignas(16) float v[NH][TB][D];
    alignas(16) float dO[NH][TB][D];
    alignas(16) double rpart[NH][TB][VQ][RD + 2];
    alignas(16) f32x4 cpart[NH][TB][NTH];
};

// Rows of key dims per backward workgroup: all (1), or 1/2, 1/4 of dk = 128
// when there are fewer than 256 (b,h).  KLA_BWD_NRG=n overrides it.
int bwd_nrg_of(long long nbh, int dk, int cov) {
    const char* e = getenv("KLA_BWD_NRG");
    const int n = e && *e ? atoi(e) : 0;
    if (cov || dk != 128) return 1;
    if (n == 1 || n == 2 || n == 4) return n;
    return nbh >= 256 ? 1 : nbh >= 128 ? 2 : 4;
}

template <typename TIn, int D, int NRG>
__global__ __launch_bounds__(kBwdThreads) void kla_bwd_diag_kernel(BwdArgs p) {
    typedef BwdRL<D, NRG> Ly;
    typedef typename Quad<TIn>::V QV;
    constexpr int TB = Ly::TB, NTH = Ly::NTH, NH = Ly::NH, VQ = Ly::VQ, RG = Ly::RG, RPT = Ly::RPT;
    constexpr int RD = Ly::RD;
    constexpr int W = RD < 64 ? RD : 64;  // key-dim lanes per wave
    __shared__ BwdSmR<Ly, D> sm;
    __shared__ double drw[NH][TB][2];     // per-wave sums of dr (RD = 128)
    (void)RG;

    const int tid = threadIdx.x;
    const int grp = NH == 1 ? 0 : tid / NTH, lt = NH == 1 ? tid : tid % NTH;
    const int nbh = p.B * p.H;
    int bh_, rgp = 0;
    if constexpr (NRG == 1) {
        bh_ = NH == 1 ? (int)blockIdx.x : (int)blockIdx.x * NH + grp;
    } else if (nbh % 8 == 0) {
        // the row groups of a (b,h) on one XCD, where they share its v, dO rows
        const int x = blockIdx.x % 8, kx = blockIdx.x / 8;
        bh_ = (kx / NRG) * 8 + x;
        rgp = kx % NRG;
    } else {
        bh_ = blockIdx.x / NRG;
        rgp = blockIdx.x % NRG;
    }
    if constexpr (NRG == 1) {
        // after the chunked kernels: only the (b,h) they handed back
        if (p.gate_nt > 0) {
            int any = 0;
            for (int g2 = 0; g2 < NH; ++g2) {
                const int b2 = NH == 1 ? (int)blockIdx.x : (int)blockIdx.x * NH + g2;
                if (b2 < nbh) {
                    const int* fl = (const int*)(p.ws + (size_t)b2 * p.ws_stride + p.flag_off);
                    for (int t2 = 0; t2 < p.gate_nt; ++t2) any |= fl[t2];
                }
            }
            if (!any) return;  // uniform over the workgroup
        }
    }
    const bool valid = NH == 1 || bh_ < nbh;
    const int bh = valid ? bh_ : nbh - 1;  // a spare group stays in bounds and stores nothing
    const int h = bh % p.H;
    const int jq = lt % VQ, rg = lt / VQ;
    const int T = p.T;
    const size_t row0 = (size_t)bh * T;
    const TIn* q = (const TIn*)p.q;
    const TIn* k = (const TIn*)p.k;
    const TIn* v = (const TIn*)p.v;
    const TIn* dOg = (const TIn*)p.dO;
    const bool kd = lt < RD;           // key-dim lane
    const bool sl = lt < TB * VQ;      // staging lane: token lt / VQ, value quad jq
    const int il = kd ? lt : RD - 1;   // key dim in the workgroup's rows
    const int r0 = rgp * RD;
    const int i = r0 + il;             // key dim of the (b,h)
    double* wl = (double*)(p.ws + (size_t)bh * p.ws_stride);
    double* wqdq = wl + (size_t)T * D;
    float* wdqn = (float*)(wqdq + (size_t)T * D);
    // row-group partials of dv [NRG][T][D] and dr [NRG][T]
    float* wdv = wdqn + D;
    float* wdr = wdv + (size_t)NRG * T * D;

    const float qn_i = p.qn[(size_t)h * D + i];
    const double l_start = p.l0 ? p.l0[(size_t)bh * D + i] : 1.f;

    // raw inputs of one token block
    struct Raw {
        float k[TB], r[TB], a[TB], q[TB];   // key-dim lanes
        QV v, dO;                            // staging lanes
    };
    auto load_raw = [&](int t0, int nb, Raw& x) {
        if (kd) {
#pragma unroll
            for (int u = 0; u < TB; ++u) {
                const size_t t = row0 + t0 + (u < nb ? u : 0);
                x.k[u] = (float)k[t * D + i];
                x.r[u] = p.r[t];
                x.a[u] = p.a[t * D + i];
                x.q[u] = (float)q[t * D + i];
            }
        }
        if (sl && lt / VQ < nb) {
            const size_t t = row0 + t0 + lt / VQ;
            x.v = *(const QV*)(v + t * D + 4 * jq);
            x.dO = *(const QV*)(dOg + t * D + 4 * jq);
        }
    };
    // sum over the VQ value quads of one row's partials, in four independent
    // chains (the serial sum is a long dependent chain of fp64 adds)
    auto quad_sum = [&](const double* col) {
        double s4[4] = {0., 0., 0., 0.};
#pragma unroll
        for (int x = 0; x < VQ; ++x) s4[x % 4] += col[(size_t)x * (RD + 2)];
        return (s4[0] + s4[1]) + (s4[2] + s4[3]);
    };
    auto stage = [&](const Raw& x, int nb) {
        if (sl && lt / VQ < nb) {
            *(f32x4*)&sm.v[grp][lt / VQ][4 * jq] = Quad<TIn>::to_f32(x.v);
            *(f32x4*)&sm.dO[grp][lt / VQ][4 * jq] = Quad<TIn>::to_f32(x.dO);
        }
    };

    // ---------------------------------------------------------------- sweep 1
    f64x4 e[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const size_t off = ((size_t)bh * D + r0 + rg * RPT + m) * D + 4 * jq;
        e[m] = p.eta0 ? to_f64(*(const f32x4*)(p.eta0 + off)) : f64x4{0., 0., 0., 0.};
    }
    double l = l_start;  // the precision recursion runs in fp64
    double lb[TB];       // precisions after the current block's tokens
    float qb[TB];        // q of the current block's tokens
    // forward coefficients of a block from its raw inputs (advances l)
    auto fwd_coefs = [&](const Raw& x, int t0, int nb) {
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            if (u < nb) {
                const double kv = x.k[u], rt = x.r[u];
                double rd;
                const double g = gate_r(x.a[u], qn_i, l, &rd);
                l = __builtin_fma(l, rd, kv * kv * rcp64(rt));
                lb[u] = l;
                qb[u] = x.q[u];
                if (kd) {
                    sm.g[grp][u][il] = (float)g;
                    sm.kap[grp][u][il] = (float)div64(kv, rt);
                    if (valid) wl[(size_t)(t0 + u) * D + i] = l;
                }
            }
        }
        stage(x, nb);
    };
    Raw nx{};
    if (T > 0) {
        const int nb = T < TB ? T : TB;
        load_raw(0, nb, nx);
        fwd_coefs(nx, 0, nb);
    }
    lds_barrier();
    for (int t0 = 0; t0 < T; t0 += TB) {
        const int nb = T - t0 < TB ? T - t0 : TB;
        const bool more = t0 + TB < T;
        const int nb2 = more ? (T - t0 - TB < TB ? T - t0 - TB : TB) : 0;
        if (more) load_raw(t0 + TB, nb2, nx);
        // ---- the block on the thread's rows; per-row S partials
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            if (u < nb) {
                const f64x4 vv = to_f64(*(const f32x4*)&sm.v[grp][u][4 * jq]);
                const f64x4 dd = to_f64(*(const f32x4*)&sm.dO[grp][u][4 * jq]);
#pragma unroll
                for (int m4 = 0; m4 < RPT; m4 += 4) {
                    const f32x4 gv = *(const f32x4*)&sm.g[grp][u][rg * RPT + m4];
                    const f32x4 kv = *(const f32x4*)&sm.kap[grp][u][rg * RPT + m4];
                    double sp[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        e[m4 + x] = (double)gv[x] * e[m4 + x] + (double)kv[x] * vv;
                        const f64x4 pr = e[m4 + x] * dd;
                        sp[x] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
                    }
                    *(f64x2*)&sm.rpart[grp][u][jq][rg * RPT + m4] = f64x2{sp[0], sp[1]};
                    *(f64x2*)&sm.rpart[grp][u][jq][rg * RPT + m4 + 2] = f64x2{sp[2], sp[3]};
                }
            }
        }
        lds_barrier();
        // ---- dq of the block (key-dim lanes)
        if (kd) {
#pragma unroll
            for (int u = 0; u < TB; ++u) {
                if (u < nb) {
                    const double s = quad_sum(&sm.rpart[grp][u][0][il]);
                    const size_t t = row0 + t0 + u;
                    const double dq = div64(s, lb[u]);
                    if (valid) {
                        ((TIn*)p.gq)[t * D + i] = (TIn)(float)dq;
                        // q dq with q / l rounded to fp32 exactly as sweep 2
                        // stages it for the readout adjoint
                        wqdq[(size_t)(t0 + u) * D + i] = (double)(float)div64(qb[u], lb[u]) * s;
                    }
                }
            }
        }
        if (more) fwd_coefs(nx, t0 + TB, nb2);
        lds_barrier();
    }
    // boundary term of the gate adjoint: B[i] = sum_j detaT[i,j] eta_T[i,j];
    // the state registers then take ebar_T = detaT
    double Bsum = 0.;
    {
#pragma unroll
        for (int m4 = 0; m4 < RPT; m4 += 4) {
            double sp[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const size_t off = ((size_t)bh * D + r0 + rg * RPT + m4 + x) * D + 4 * jq;
                const f64x4 dt = p.detaT ? to_f64(*(const f32x4*)(p.detaT + off)) : f64x4{0., 0., 0., 0.};
                const f64x4 pr = e[m4 + x] * dt;
                sp[x] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
                e[m4 + x] = dt;
            }
            *(f64x2*)&sm.rpart[grp][0][jq][rg * RPT + m4] = f64x2{sp[0], sp[1]};
            *(f64x2*)&sm.rpart[grp][0][jq][rg * RPT + m4 + 2] = f64x2{sp[2], sp[3]};
        }
        __syncthreads();
        if (kd) Bsum = quad_sum(&sm.rpart[grp][0][0][il]);
        __syncthreads();
    }

    // ---------------------------------------------------------------- sweep 2
    double lbar = p.dlT ? p.dlT[(size_t)bh * D + i] : 0.f;
    double cum = Bsum;
    double dqn_acc = 0.;
    // raw inputs of a block for sweep 2: those of sweep 1, the stored
    // precisions (after each token, and before the block), the next token's
    // a and q dq
    struct Raw2 {
        Raw x;
        double lt[TB], lprev0, qdq[TB];
        float an[TB];
    };
    auto load_raw2 = [&](int t0, int nb, Raw2& y) {
        load_raw(t0, nb, y.x);
        if (kd) {
#pragma unroll
            for (int u = 0; u < TB; ++u) {
                const int t = t0 + (u < nb ? u : 0);
                y.lt[u] = wl[(size_t)t * D + i];
                y.qdq[u] = wqdq[(size_t)t * D + i];
                y.an[u] = t + 1 < T ? p.a[(row0 + t + 1) * D + i] : 0.f;
            }
            y.lprev0 = t0 == 0 ? l_start : wl[(size_t)(t0 - 1) * D + i];
        }
    };
    // the adjoint's inputs of the current block (registers)
    double c_lt[TB], c_lprev[TB], c_qdq[TB];
    float c_a[TB], c_k[TB], c_r[TB];
    // backward coefficients of a block: gate of the token after each (1 past
    // the end), k/r, q/l into LDS; its adjoint inputs into the registers
    auto bwd_coefs = [&](const Raw2& y, int t0, int nb) {
        stage(y.x, nb);
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            if (u < nb) {
                const int t = t0 + u;
                const double lt_ = y.lt[u];
                double gn = 1., rd;
                if (t + 1 < T) gn = gate_r(y.an[u], qn_i, lt_, &rd);
                if (kd) {
                    sm.g[grp][u][il] = (float)gn;
                    sm.kap[grp][u][il] = (float)div64(y.x.k[u], y.x.r[u]);
                    sm.cq[grp][u][il] = (float)div64(y.x.q[u], lt_);
                }
                c_lt[u] = lt_;
                c_lprev[u] = u == 0 ? y.lprev0 : y.lt[u - 1];
                c_qdq[u] = y.qdq[u];
                c_a[u] = y.x.a[u];
                c_k[u] = y.x.k[u];
                c_r[u] = y.x.r[u];
            }
        }
    };
    const int nblk = (T + TB - 1) / TB;
    Raw2 ny{};
    if (T > 0) {
        const int t0 = (nblk - 1) * TB;
        load_raw2(t0, T - t0, ny);
        bwd_coefs(ny, t0, T - t0);
    }
    lds_barrier();
    // dr of the previous block's tokens (dk = 128: the two waves' sums)
    auto store_dr = [&](int t0, int nb) {
        if constexpr (RD > 64) {
            if (tid < nb && valid) p.gr[row0 + t0 + tid] = (float)(drw[0][tid][0] + drw[0][tid][1]);
        }
    };
    int prev_t0 = -1, prev_nb = 0;
    for (int blk = nblk - 1; blk >= 0; --blk) {
        const int t0 = blk * TB;
        const int nb = T - t0 < TB ? T - t0 : TB;
        if (blk > 0) load_raw2(t0 - TB, TB, ny);
        if (prev_t0 >= 0) store_dr(prev_t0, prev_nb);
        // ---- ebar over the block's tokens, last first; U and dv partials
#pragma unroll
        for (int u = TB - 1; u >= 0; --u) {
            if (u < nb) {
                const f64x4 vv = to_f64(*(const f32x4*)&sm.v[grp][u][4 * jq]);
                const f64x4 dd = to_f64(*(const f32x4*)&sm.dO[grp][u][4 * jq]);
                f64x4 cs = {0., 0., 0., 0.};
#pragma unroll
                for (int m4 = 0; m4 < RPT; m4 += 4) {
                    const f32x4 gv = *(const f32x4*)&sm.g[grp][u][rg * RPT + m4];
                    const f32x4 cv = *(const f32x4*)&sm.cq[grp][u][rg * RPT + m4];
                    const f32x4 kv = *(const f32x4*)&sm.kap[grp][u][rg * RPT + m4];
                    double sp[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        e[m4 + x] = (double)gv[x] * e[m4 + x] + (double)cv[x] * dd;
                        const f64x4 pr = e[m4 + x] * vv;
                        sp[x] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
                        cs += (double)kv[x] * e[m4 + x];
                    }
                    *(f64x2*)&sm.rpart[grp][u][jq][rg * RPT + m4] = f64x2{sp[0], sp[1]};
                    *(f64x2*)&sm.rpart[grp][u][jq][rg * RPT + m4 + 2] = f64x2{sp[2], sp[3]};
                }
                sm.cpart[grp][u][lt] = f32x4{(float)cs[0], (float)cs[1], (float)cs[2], (float)cs[3]};
            }
        }
        lds_barrier();
        // ---- dv of the block (staging lanes)
        if (sl && lt / VQ < nb) {
            const int u = lt / VQ;
            f32x4 s = sm.cpart[grp][u][jq];
#pragma unroll
            for (int r2 = 1; r2 < Ly::RG; ++r2) s += sm.cpart[grp][u][r2 * VQ + jq];
            if (valid) {
                if constexpr (NRG == 1)
                    *(QV*)((TIn*)p.gv + (row0 + t0 + u) * D + 4 * jq) = Quad<TIn>::make(s);
                else
                    *(f32x4*)(wdv + ((size_t)rgp * T + t0 + u) * D + 4 * jq) = s;
            }
        }
        // ---- the precision adjoint over the block (key-dim lanes compute,
        // the dr sums run over every lane of a key-dim wave), last first
        if (lt < ((RD + 63) / 64) * 64) {
#pragma unroll
            for (int u = TB - 1; u >= 0; --u) {
                if (u < nb) {
                    const int t = t0 + u;
                    const size_t tt = row0 + t;
                    const double Uv = quad_sum(&sm.rpart[grp][u][0][il]);
                    const double kv = c_k[u];
                    const double rt = c_r[u];
                    const double kap = (float)div64(kv, rt);  // the staged k/r of the state update
                    const double rr = rcp64(rt);
                    const double lt_ = c_lt[u], lprev = c_lprev[u];
                    const double a = c_a[u], qn = qn_i, qdq = c_qdq[u];
                    const double kU = kap * Uv;
                    lbar -= qdq * rcp64(lt_);
                    cum += qdq - kU;
                    const double dlg = cum;
                    const double den = a * a + qn * lprev;
                    const double rd = rcp64(den), rd2 = rd * rd;
                    const double dk = (Uv + lbar * 2. * kv) * rr;
                    if (kd && valid) ((TIn*)p.gk)[tt * D + i] = (TIn)(float)dk;
                    // dr: -(kap U + lbar b_i) / r, summed over key dims
                    double dr = kd ? -(kap * Uv + lbar * kv * kv * rr) * rr : 0.;
#pragma unroll
                    for (int m = 1; m < W; m <<= 1) dr += __shfl_xor(dr, m, 64);
                    if constexpr (RD > 64) {
                        if ((lt & 63) == 0) drw[0][u][lt >> 6] = dr;
                    } else if constexpr (NRG == 1) {
                        if (lt == 0 && valid) p.gr[tt] = (float)dr;
                    } else {
                        if (lt == 0 && valid) wdr[(size_t)rgp * T + t] = (float)dr;
                    }
                    const double da = -lbar * 2. * a * lprev * rd2 + dlg * (qn * lprev - a * a) * rd * rcp64(a);
                    const double dqn = -lbar * lprev * lprev * rd2 - dlg * lprev * rd;
                    if (kd && valid) p.ga[tt * D + i] = (float)da;
                    dqn_acc += dqn;
                    lbar = lbar * a * a * rd2 - dlg * qn * rd;
                }
            }
        }
        if (blk > 0) bwd_coefs(ny, t0 - TB, TB);
        prev_t0 = t0;
        prev_nb = nb;
        lds_barrier();
    }
    if (prev_t0 >= 0) store_dr(prev_t0, prev_nb);
    // ---- initial-state gradients: deta0 = g_0 ebar_0, dl0 = lbar_{-1}
    if (T > 0 && kd) {
        double rd;
        sm.g[grp][0][il] = (float)gate_r(p.a[row0 * D + i], qn_i, l_start, &rd);
    }
    __syncthreads();
    if (!valid) return;
    if (p.geta0) {
#pragma unroll
        for (int m4 = 0; m4 < RPT; m4 += 4) {
            const f32x4 gv = T > 0 ? *(const f32x4*)&sm.g[grp][0][rg * RPT + m4] : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const f64x4 r4 = (double)gv[x] * e[m4 + x];
                *(f32x4*)(p.geta0 + ((size_t)bh * D + r0 + rg * RPT + m4 + x) * D + 4 * jq) =
                    f32x4{(float)r4[0], (float)r4[1], (float)r4[2], (float)r4[3]};
            }
        }
    }
    if (kd) {
        if (p.gl0) p.gl0[(size_t)bh * D + i] = (float)lbar;
        wdqn[i] = (float)dqn_acc;
    }
}

// Row-split diagonal backward at dk = dv = 128 with the per-token work of a
// token block spread over the four waves: wave w takes tokens w, w+4, ... of
// the block for every key dim of the workgroup (one lane per key dim).  Only
// the recursions stay serial: the precision l (sweep 1, wave 0) and the
// adjoints lbar, cum (sweep 2, wave 0), whose per-token coefficients the
// four waves form in parallel:
//   lbar_t = lbar_t' - qdq_t / l_t,   cum_t = cum_{t+1} + qdq_t - kap_t U_t,
//   lbar_{t-1}' = lbar_t a_t^2 rd_t^2 - cum_t qn rd_t        (rd_t = 1 / D_t)
// so each token's dk, da, dr, dqn follow from (lbar_t, cum_t) in parallel
// again.  Same arithmetic as kla_bwd_diag_kernel, in another order.
template <typename TIn, int NRG>
__global__ __launch_bounds__(kBwdThreads) void kla_bwd_rows_kernel(BwdArgs p) {
    constexpr int D = 128;
    typedef BwdRL<D, NRG> Ly;
    typedef typename Quad<TIn>::V QV;
    constexpr int TB = Ly::TB, NTH = Ly::NTH, VQ = Ly::VQ, RPT = Ly::RPT, RD = Ly::RD;
    constexpr int NWV = kBwdThreads / 64, TPW = TB / NWV;  // tokens per wave and block
    static_assert(Ly::NH == 1 && NTH == kBwdThreads && RD <= 64 && TB % NWV == 0, "row-split layout");
    __shared__ BwdSmR<Ly, D> sm;
    __shared__ double s_lt[2][TB][RD];      // sweep 1: l_t of the block, by block parity
    __shared__ double s_co[TB][4][RD];      // sweep 2: qdq/l, qdq - kap U, a^2 rd^2, qn rd
    __shared__ double s_lc[TB][2][RD];      // sweep 2: lbar_t, cum_t
    __shared__ float s_dqn[NWV][RD];

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int nbh = p.B * p.H;
    int bh, rgp;
    if (nbh % 8 == 0) {
        const int x = blockIdx.x % 8, kx = blockIdx.x / 8;
        bh = (kx / NRG) * 8 + x;
        rgp = kx % NRG;
    } else {
        bh = blockIdx.x / NRG;
        rgp = blockIdx.x % NRG;
    }
    const int h = bh % p.H;
    const int jq = tid % VQ, rg = tid / VQ;
    const int T = p.T;
    const size_t row0 = (size_t)bh * T;
    const TIn* q = (const TIn*)p.q;
    const TIn* k = (const TIn*)p.k;
    const TIn* v = (const TIn*)p.v;
    const TIn* dOg = (const TIn*)p.dO;
    const bool kd = lane < RD;             // key-dim lane (in every wave)
    const bool sl = tid < TB * VQ;         // staging lane: token tid / VQ, value quad jq
    const int il = kd ? lane : RD - 1;
    const int r0 = rgp * RD;
    const int i = r0 + il;
    double* wl = (double*)(p.ws + (size_t)bh * p.ws_stride);
    double* wqdq = wl + (size_t)T * D;
    float* wdqn = (float*)(wqdq + (size_t)T * D);
    float* wdv = wdqn + D;
    float* wdr = wdv + (size_t)NRG * T * D;

    const float qn_i = p.qn[(size_t)h * D + i];
    const double l_start = p.l0 ? p.l0[(size_t)bh * D + i] : 1.f;

    auto quad_sum = [&](const double* col) {
        double s4[4] = {0., 0., 0., 0.};
#pragma unroll
        for (int x = 0; x < VQ; ++x) s4[x % 4] += col[(size_t)x * (RD + 2)];
        return (s4[0] + s4[1]) + (s4[2] + s4[3]);
    };
    // the v and dO rows of a block (staging lanes)
    struct Rows {
        QV v, dO;
    };
    auto load_rows = [&](int t0, int nb, Rows& x) {
        if (sl && tid / VQ < nb) {
            const size_t t = row0 + t0 + tid / VQ;
            x.v = *(const QV*)(v + t * D + 4 * jq);
            x.dO = *(const QV*)(dOg + t * D + 4 * jq);
        }
    };
    auto stage_rows = [&](const Rows& x, int nb) {
        if (sl && tid / VQ < nb) {
            *(f32x4*)&sm.v[0][tid / VQ][4 * jq] = Quad<TIn>::to_f32(x.v);
            *(f32x4*)&sm.dO[0][tid / VQ][4 * jq] = Quad<TIn>::to_f32(x.dO);
        }
    };

    // ---------------------------------------------------------------- sweep 1
    f64x4 e[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const size_t off = ((size_t)bh * D + r0 + rg * RPT + m) * D + 4 * jq;
        e[m] = p.eta0 ? to_f64(*(const f32x4*)(p.eta0 + off)) : f64x4{0., 0., 0., 0.};
    }
    double l = l_start;  // wave 0: the precision recursion, fp64
    // raw inputs of a block: k, r, a of every token (wave 0, for the
    // recursion) and q of the wave's own tokens
    struct Raw1 {
        float k[TB], r[TB], a[TB], q[TPW];
        Rows rows;
    };
    auto load1 = [&](int t0, int nb, Raw1& x) {
        if (kd) {
            if (wv == 0) {
#pragma unroll
                for (int u = 0; u < TB; ++u) {
                    const size_t t = row0 + t0 + (u < nb ? u : 0);
                    x.k[u] = (float)k[t * D + i];
                    x.r[u] = p.r[t];
                    x.a[u] = p.a[t * D + i];
                }
            }
#pragma unroll
            for (int m = 0; m < TPW; ++m) {
                const int u = wv + NWV * m;
                x.q[m] = (float)q[(row0 + t0 + (u < nb ? u : 0)) * D + i];
            }
        }
        load_rows(t0, nb, x.rows);
    };
    // wave 0: the block's precisions (advances l), gates and k/r into LDS,
    // l_t into LDS (by parity) and the workspace
    auto fwd_coefs = [&](const Raw1& x, int t0, int nb, int par) {
        if (wv == 0) {
#pragma unroll
            for (int u = 0; u < TB; ++u) {
                if (u < nb) {
                    const double kv = x.k[u], rt = x.r[u];
                    double rd;
                    const double g = gate_r(x.a[u], qn_i, l, &rd);
                    l = __builtin_fma(l, rd, kv * kv * rcp64(rt));
                    if (kd) {
                        sm.g[0][u][il] = (float)g;
                        sm.kap[0][u][il] = (float)div64(kv, rt);
                        s_lt[par][u][il] = l;
                        wl[(size_t)(t0 + u) * D + i] = l;
                    }
                }
            }
        }
        stage_rows(x.rows, nb);
    };
    Raw1 n1{};
    float qb[TPW] = {};  // q of the wave's tokens of the current block
    if (T > 0) {
        const int nb = T < TB ? T : TB;
        load1(0, nb, n1);
        fwd_coefs(n1, 0, nb, 0);
#pragma unroll
        for (int m = 0; m < TPW; ++m) qb[m] = n1.q[m];
    }
    lds_barrier();
    for (int t0 = 0, bi = 0; t0 < T; t0 += TB, ++bi) {
        const int nb = T - t0 < TB ? T - t0 : TB;
        const bool more = t0 + TB < T;
        const int nb2 = more ? (T - t0 - TB < TB ? T - t0 - TB : TB) : 0;
        if (more) load1(t0 + TB, nb2, n1);
        // ---- the block on the thread's rows; per-row S partials
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            if (u < nb) {
                const f64x4 vv = to_f64(*(const f32x4*)&sm.v[0][u][4 * jq]);
                const f64x4 dd = to_f64(*(const f32x4*)&sm.dO[0][u][4 * jq]);
#pragma unroll
                for (int m4 = 0; m4 < RPT; m4 += 4) {
                    const f32x4 gv = *(const f32x4*)&sm.g[0][u][rg * RPT + m4];
                    const f32x4 kv = *(const f32x4*)&sm.kap[0][u][rg * RPT + m4];
                    double sp[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        e[m4 + x] = (double)gv[x] * e[m4 + x] + (double)kv[x] * vv;
                        const f64x4 pr = e[m4 + x] * dd;
                        sp[x] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
                    }
                    *(f64x2*)&sm.rpart[0][u][jq][rg * RPT + m4] = f64x2{sp[0], sp[1]};
                    *(f64x2*)&sm.rpart[0][u][jq][rg * RPT + m4 + 2] = f64x2{sp[2], sp[3]};
                }
            }
        }
        lds_barrier();
        // ---- dq of the wave's tokens
        if (kd) {
#pragma unroll
            for (int m = 0; m < TPW; ++m) {
                const int u = wv + NWV * m;
                if (u < nb) {
                    const double s = quad_sum(&sm.rpart[0][u][0][il]);
                    const double lb = s_lt[bi & 1][u][il];
                    const size_t t = row0 + t0 + u;
                    ((TIn*)p.gq)[t * D + i] = (TIn)(float)div64(s, lb);
                    // q dq with q / l rounded to fp32 exactly as sweep 2 stages it
                    wqdq[(size_t)(t0 + u) * D + i] = (double)(float)div64(qb[m], lb) * s;
                }
            }
        }
        if (more) {
            fwd_coefs(n1, t0 + TB, nb2, (bi + 1) & 1);
#pragma unroll
            for (int m = 0; m < TPW; ++m) qb[m] = n1.q[m];
        }
        lds_barrier();
    }
    // boundary term of the gate adjoint: B[i] = sum_j detaT[i,j] eta_T[i,j]
    double Bsum = 0.;
    {
#pragma unroll
        for (int m4 = 0; m4 < RPT; m4 += 4) {
            double sp[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const size_t off = ((size_t)bh * D + r0 + rg * RPT + m4 + x) * D + 4 * jq;
                const f64x4 dt = p.detaT ? to_f64(*(const f32x4*)(p.detaT + off)) : f64x4{0., 0., 0., 0.};
                const f64x4 pr = e[m4 + x] * dt;
                sp[x] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
                e[m4 + x] = dt;
            }
            *(f64x2*)&sm.rpart[0][0][jq][rg * RPT + m4] = f64x2{sp[0], sp[1]};
            *(f64x2*)&sm.rpart[0][0][jq][rg * RPT + m4 + 2] = f64x2{sp[2], sp[3]};
        }
        __syncthreads();  // also orders sweep 1's workspace stores before sweep 2's reads
        if (kd && wv == 0) Bsum = quad_sum(&sm.rpart[0][0][0][il]);
        __syncthreads();
    }

    // ---------------------------------------------------------------- sweep 2
    double lbar = p.dlT ? p.dlT[(size_t)bh * D + i] : 0.f;  // wave 0
    double cum = Bsum;                                        // wave 0
    double dqn_acc = 0.;                                      // per wave
    // inputs of the wave's tokens of a block
    struct Raw2 {
        float k[TPW], r[TPW], a[TPW], q[TPW], an[TPW];
        double lt[TPW], lp[TPW], qdq[TPW];
        Rows rows;
    };
    auto load2 = [&](int t0, int nb, Raw2& y) {
        if (kd) {
#pragma unroll
            for (int m = 0; m < TPW; ++m) {
                const int u = wv + NWV * m;
                const int t = t0 + (u < nb ? u : 0);
                const size_t tt = row0 + t;
                y.k[m] = (float)k[tt * D + i];
                y.r[m] = p.r[tt];
                y.a[m] = p.a[tt * D + i];
                y.q[m] = (float)q[tt * D + i];
                y.an[m] = t + 1 < T ? p.a[(tt + 1) * D + i] : 0.f;
                y.lt[m] = wl[(size_t)t * D + i];
                y.lp[m] = t == 0 ? l_start : wl[(size_t)(t - 1) * D + i];
                y.qdq[m] = wqdq[(size_t)t * D + i];
            }
        }
        load_rows(t0, nb, y.rows);
    };
    // the adjoint's inputs of the wave's tokens of the current block
    float c_k[TPW], c_r[TPW], c_a[TPW];
    double c_lt[TPW], c_lp[TPW], c_qdq[TPW];
    // backward coefficients of the wave's tokens: gate of the token after
    // (1 past the end), k/r, q/l into LDS; the adjoint inputs into registers
    auto bwd_coefs = [&](const Raw2& y, int t0, int nb) {
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int u = wv + NWV * m;
            if (u < nb) {
                double gn = 1., rd;
                if (t0 + u + 1 < T) gn = gate_r(y.an[m], qn_i, y.lt[m], &rd);
                if (kd) {
                    sm.g[0][u][il] = (float)gn;
                    sm.kap[0][u][il] = (float)div64(y.k[m], y.r[m]);
                    sm.cq[0][u][il] = (float)div64(y.q[m], y.lt[m]);
                }
                c_k[m] = y.k[m];
                c_r[m] = y.r[m];
                c_a[m] = y.a[m];
                c_lt[m] = y.lt[m];
                c_lp[m] = y.lp[m];
                c_qdq[m] = y.qdq[m];
            }
        }
        stage_rows(y.rows, nb);
    };
    const int nblk = (T + TB - 1) / TB;
    Raw2 n2{};
    if (T > 0) {
        const int t0 = (nblk - 1) * TB;
        load2(t0, T - t0, n2);
        bwd_coefs(n2, t0, T - t0);
    }
    lds_barrier();
    for (int blk = nblk - 1; blk >= 0; --blk) {
        const int t0 = blk * TB;
        const int nb = T - t0 < TB ? T - t0 : TB;
        if (blk > 0) load2(t0 - TB, TB, n2);
        // ---- ebar over the block's tokens, last first; U and dv partials
#pragma unroll
        for (int u = TB - 1; u >= 0; --u) {
            if (u < nb) {
                const f64x4 vv = to_f64(*(const f32x4*)&sm.v[0][u][4 * jq]);
                const f64x4 dd = to_f64(*(const f32x4*)&sm.dO[0][u][4 * jq]);
                f64x4 cs = {0., 0., 0., 0.};
#pragma unroll
                for (int m4 = 0; m4 < RPT; m4 += 4) {
                    const f32x4 gv = *(const f32x4*)&sm.g[0][u][rg * RPT + m4];
                    const f32x4 cv = *(const f32x4*)&sm.cq[0][u][rg * RPT + m4];
                    const f32x4 kv = *(const f32x4*)&sm.kap[0][u][rg * RPT + m4];
                    double sp[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        e[m4 + x] = (double)gv[x] * e[m4 + x] + (double)cv[x] * dd;
                        const f64x4 pr = e[m4 + x] * vv;
                        sp[x] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
                        cs += (double)kv[x] * e[m4 + x];
                    }
                    *(f64x2*)&sm.rpart[0][u][jq][rg * RPT + m4] = f64x2{sp[0], sp[1]};
                    *(f64x2*)&sm.rpart[0][u][jq][rg * RPT + m4 + 2] = f64x2{sp[2], sp[3]};
                }
                sm.cpart[0][u][tid] = f32x4{(float)cs[0], (float)cs[1], (float)cs[2], (float)cs[3]};
            }
        }
        lds_barrier();
        // ---- dv of the block (staging lanes); the per-token coefficients
        // of the adjoint recursions (each wave its tokens)
        if (sl && tid / VQ < nb) {
            const int u = tid / VQ;
            f32x4 s = sm.cpart[0][u][jq];
#pragma unroll
            for (int r2 = 1; r2 < Ly::RG; ++r2) s += sm.cpart[0][u][r2 * VQ + jq];
            *(f32x4*)(wdv + ((size_t)rgp * T + t0 + u) * D + 4 * jq) = s;
        }
        double Uv[TPW], kap[TPW], rr[TPW], rd[TPW];
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int u = wv + NWV * m;
            if (u < nb && kd) {
                Uv[m] = quad_sum(&sm.rpart[0][u][0][il]);
                kap[m] = (float)div64(c_k[m], c_r[m]);
                rr[m] = rcp64(c_r[m]);
                const double a = c_a[m];
                rd[m] = rcp64(a * a + (double)qn_i * c_lp[m]);
                s_co[u][0][il] = c_qdq[m] * rcp64(c_lt[m]);
                s_co[u][1][il] = c_qdq[m] - kap[m] * Uv[m];
                s_co[u][2][il] = a * a * rd[m] * rd[m];
                s_co[u][3][il] = (double)qn_i * rd[m];
            }
        }
        lds_barrier();
        // ---- the serial recursions (wave 0), last token first
        if (wv == 0 && kd) {
#pragma unroll
            for (int u = TB - 1; u >= 0; --u) {
                if (u < nb) {
                    lbar -= s_co[u][0][il];
                    cum += s_co[u][1][il];
                    s_lc[u][0][il] = lbar;
                    s_lc[u][1][il] = cum;
                    lbar = lbar * s_co[u][2][il] - cum * s_co[u][3][il];
                }
            }
        }
        lds_barrier();
        // ---- the gradients of the wave's tokens
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int u = wv + NWV * m;
            if (u < nb) {
                const size_t tt = row0 + t0 + u;
                const double lb = kd ? s_lc[u][0][il] : 0., dlg = kd ? s_lc[u][1][il] : 0.;
                const double kv = c_k[m], a = c_a[m], lprev = c_lp[m], qn = qn_i;
                const double rd2 = rd[m] * rd[m];
                if (kd) {
                    ((TIn*)p.gk)[tt * D + i] = (TIn)(float)((Uv[m] + lb * 2. * kv) * rr[m]);
                    p.ga[tt * D + i] = (float)(-lb * 2. * a * lprev * rd2 +
                                               dlg * (qn * lprev - a * a) * rd[m] * rcp64(a));
                    dqn_acc += -lb * lprev * lprev * rd2 - dlg * lprev * rd[m];
                }
                double dr = kd ? -(kap[m] * Uv[m] + lb * kv * kv * rr[m]) * rr[m] : 0.;
#pragma unroll
                for (int x = 1; x < (RD < 64 ? RD : 64); x <<= 1) dr += __shfl_xor(dr, x, 64);
                if (lane == 0) wdr[(size_t)rgp * T + t0 + u] = (float)dr;
            }
        }
        if (blk > 0) bwd_coefs(n2, t0 - TB, TB);
        lds_barrier();
    }
    // ---- initial-state gradients: deta0 = g_0 ebar_0, dl0 = lbar_{-1}; the
    // waves' dqn partials
    if (kd) s_dqn[wv][il] = (float)dqn_acc;
    if (T > 0 && kd && wv == 0) {
        double rdd;
        sm.g[0][0][il] = (float)gate_r(p.a[row0 * D + i], qn_i, l_start, &rdd);
    }
    __syncthreads();
    if (p.geta0) {
#pragma unroll
        for (int m4 = 0; m4 < RPT; m4 += 4) {
            const f32x4 gv = T > 0 ? *(const f32x4*)&sm.g[0][0][rg * RPT + m4] : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const f64x4 r4 = (double)gv[x] * e[m4 + x];
                *(f32x4*)(p.geta0 + ((size_t)bh * D + r0 + rg * RPT + m4 + x) * D + 4 * jq) =
                    f32x4{(float)r4[0], (float)r4[1], (float)r4[2], (float)r4[3]};
            }
        }
    }
    if (kd && wv == 0) {
        if (p.gl0) p.gl0[(size_t)bh * D + i] = (float)lbar;
        float sq = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NWV; ++w2) sq += s_dqn[w2][il];
        wdqn[i] = sq;
    }
}

// dv and dr of a row-split backward: the sums of the row groups' partials
// (in order of the group).  One thread per (b,h, token, value quad).
template <typename TIn, int NRG>
__global__ void kla_bwd_combine(BwdArgs p) {
    const int D = p.dv, VQ = D / 4;
    const size_t n = (size_t)p.B * p.H * p.T * VQ;
    const size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= n) return;
    const int jq = (int)(x % VQ);
    const size_t bt = x / VQ;
    const int t = (int)(bt % p.T);
    const int bh = (int)(bt / p.T);
    const float* wdv = p.ws + (size_t)bh * p.ws_stride + (size_t)p.T * p.dk * 4 + p.dk;
    const float* wdr = wdv + (size_t)NRG * p.T * D;
    f32x4 s = *(const f32x4*)(wdv + (size_t)t * D + 4 * jq);
#pragma unroll
    for (int g = 1; g < NRG; ++g) s += *(const f32x4*)(wdv + ((size_t)g * p.T + t) * D + 4 * jq);
    *(typename Quad<TIn>::V*)((TIn*)p.gv + bt * D + 4 * jq) = Quad<TIn>::make(s);
    if (jq == 0) {
        float r = wdr[t];
#pragma unroll
        for (int g = 1; g < NRG; ++g) r += wdr[(size_t)g * p.T + t];
        p.gr[bt] = r;
    }
}

// dqn[h, i] = sum over b of the per-(b,h) partials (in order of b).
__global__ void kla_bwd_dqn_sum(BwdArgs p) {
    const int n = p.H * p.dk;
    const int x = blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= n) return;
    const int h = x / p.dk, i = x % p.dk;
    const size_t off = (size_t)p.T * p.dk * 4;  // floats to the partial (after l_t and q dq, fp64)
    float s = 0.f;
    for (int b = 0; b < p.B; ++b) s += p.ws[(size_t)(b * p.H + h) * p.ws_stride + off + i];
    p.gqn[x] = s;
}

// The diagonal backward runs the prefetching kernel, the isotropic one the
// plain two-sweep kernel (KLA_BWD_IMPL=plain selects it for diagonal too).
bool bwd_plain() {
    const char* e = getenv("KLA_BWD_IMPL");
    return e && e[0] == 'p';
}

template <typename TIn, int D, bool ISO>
void launch_d(const BwdArgs& a, dim3 grid, dim3 block, hipStream_t s) {
    if constexpr ((D == 64 || (D == 128 && !ISO)) && std::is_same<TIn, bf16>::value) {
        if (bwd_chunk_supported(a.dk, a.dv, ISO ? 1 : 0, DT_BF16, a.T)) {
            // the chunked kernels, then the token-serial kernel for the (b,h)
            // whose decay products left the range of the chunk quotients
            if (launch_bwd_chunk(a, DT_BF16, ISO ? 1 : 0, s) != hipSuccess) return;
            BwdArgs f = a;
            f.gate_nt = D / 64;
            f.flag_off = bc_layout(a.T, D).flags;
            if constexpr (ISO)
                hipLaunchKernelGGL((kla_bwd_kernel<TIn, D, true>), grid, block, 0, s, f);
            else
                hipLaunchKernelGGL((kla_bwd_diag_kernel<TIn, D, 1>), grid, block, 0, s, f);
            return;
        }
    }
    if (ISO || bwd_plain()) {
        hipLaunchKernelGGL((kla_bwd_kernel<TIn, D, ISO>), grid, block, 0, s, a);
        return;
    }
    const int nbh = a.B * a.H;
    if constexpr (D == 128) {
        const int nrg = bwd_nrg_of(nbh, D, 0);
        if (nrg > 1) {
            const size_t n = (size_t)nbh * a.T * (D / 4);
            if (nrg == 2)
                hipLaunchKernelGGL((kla_bwd_rows_kernel<TIn, 2>), dim3(nbh * 2), block, 0, s, a);
            else
                hipLaunchKernelGGL((kla_bwd_rows_kernel<TIn, 4>), dim3(nbh * 4), block, 0, s, a);
            if (n > 0) {
                if (nrg == 2)
                    hipLaunchKernelGGL((kla_bwd_combine<TIn, 2>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
                else
                    hipLaunchKernelGGL((kla_bwd_combine<TIn, 4>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
            }
            return;
        }
    }
    hipLaunchKernelGGL((kla_bwd_diag_kernel<TIn, D, 1>), grid, block, 0, s, a);
}

template <typename TIn, bool ISO>
hipError_t dispatch(const BwdArgs& a, hipStream_t s) {
    const dim3 block(kBwdThreads);
    const int nbh = a.B * a.H;
    auto grid = [&](int nh) { return dim3((nbh + nh - 1) / nh); };
    if (nbh > 0) switch (a.dk) {
        case 16: launch_d<TIn, 16, ISO>(a, grid(BwdLayout<16>::NH), block, s); break;
        case 32: launch_d<TIn, 32, ISO>(a, grid(BwdLayout<32>::NH), block, s); break;
        case 64: launch_d<TIn, 64, ISO>(a, grid(BwdLayout<64>::NH), block, s); break;
        case 128: launch_d<TIn, 128, ISO>(a, grid(BwdLayout<128>::NH), block, s); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ISO) return e;
    const int n = a.H * a.dk;
    hipLaunchKernelGGL(kla_bwd_dqn_sum, dim3((n + 255) / 256), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool bwd_supported(int dk, int dv) { return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128); }

size_t bwd_ws_stride(int B, int H, int T, int dk, int cov, int dtype) {
    if (bwd_chunk_supported(dk, dk, cov, dtype, T)) return bc_layout(T, dk).total;
    const size_t nl = cov ? 1 : (size_t)dk;
    // l_t and q dq (fp64), the diagonal qn partial (fp32), and with a row
    // split the row groups' partials of dv [NRG][T][dv] and dr [NRG][T]
    size_t n = (size_t)T * nl * 4 + (cov ? 0 : (size_t)dk);
    const int nrg = bwd_plain() ? 1 : bwd_nrg_of((long long)B * H, dk, cov);
    if (nrg > 1) n += (size_t)nrg * T * dk + (size_t)nrg * T;
    return (n + 63) / 64 * 64;  // floats; 256-byte aligned per (b,h)
}

hipError_t launch_bwd(const BwdArgs& a, int dtype, int cov, hipStream_t s) {
    if (!bwd_supported(a.dk, a.dv)) return hipErrorInvalidValue;
    if (dtype == DT_BF16) return cov ? dispatch<bf16, true>(a, s) : dispatch<bf16, false>(a, s);
    return cov ? dispatch<float, true>(a, s) : dispatch<float, false>(a, s);
}

}  // namespace kla
