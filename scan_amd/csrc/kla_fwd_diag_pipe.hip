// kla_fwd_diag_pipe.hip -- gfx950 forward kernel, diagonal precision, for
// key dims 64 and 128: wave-specialised software pipeline.
//
// Sources: "Kalman Linear Attention: Parallel Bayesian Filtering For Efficient
// Language Modelling and State Tracking" (gist.science explainer, method §1-§3)
// and "Kalman Delta Networks: Uncertainty-aware Associative Memory" (abstract,
// diagonal variant).  The recurrence and the mean-form gated scan are the
// same as in kla_fwd_diag.hip:
//   lp = l/(a^2 + qn l),  l' = lp + k^2/r,
//   m_t = f_t (.) m_{t-1} + w_t v_t^T,  f = a lp / l',  w = k / (r l'),
//   o_t = q_t^T m_t.
//
// The precision recursion is sequential in t for each key dim, so one
// workgroup splits its waves by role and overlaps them chunk by chunk:
//   chain waves (one lane per key dim) run the precision recurrence of chunk
//     c+1 -- four dependent VALU ops per token -- and leave (a*lp, l) in LDS;
//   gate waves turn chunk c's precisions into gates and MFMA operands (every
//     lane owns two key dims and 8 tokens; the cumulative gate products cross
//     token groups with lane shuffles inside the wave, no barrier), then run
//     the chunk's MFMA work (causal S^T tiles, readout, state update) with the
//     fp32 state in accumulator registers.
// Two workgroup barriers per 32-token chunk.  Gate products that fall below
// 2^-64 inside a chunk trigger the exact sub-chunk split (rare, slow path).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kla_common.h"
#include "kla_internal.h"

namespace kla {
namespace {

constexpr float kFloor = 5.421010862427522e-20f;  // 2^-64

template <typename TIn, int DK_, int DV_>
struct PCfg {
    static constexpr int DK = DK_;
    static constexpr int DV = DV_;              // value columns of this workgroup
    static constexpr int C = 32;                // tokens per chunk
    static constexpr int NCW = DK / 64;         // chain waves
    static constexpr int NGW = 4;               // gate waves
    static constexpr int NW = NCW + NGW;
    static constexpr int NT = NW * 64;
    static constexpr int JT = DV / 16 / NGW;    // value tiles per gate wave
    static constexpr int IT = DK / 16;
    static constexpr int NB = C / 16;
    static constexpr int NIP = DK / 2;          // key-dim pairs
    static constexpr int NGRP = 256 / NIP;      // token groups (over all gate lanes)
    static constexpr int TPG = C / NGRP;        // tokens per group
    static constexpr int IPW = 64 / NGRP;       // key-dim pairs per gate wave
    static constexpr int PE = 16 / (int)sizeof(TIn);
    static constexpr int QS = DK + PE;
    static constexpr int CS = C + PE;
    static constexpr int VQ = DV / 4;
    static constexpr int VUNITS = (C / 2) * VQ;
    static constexpr int VPT = (VUNITS + 255) / 256;
    static_assert(DK == 64 || DK == 128, "pipelined kernel covers dk 64 and 128");
    static_assert(JT >= 1 && DV % (16 * NGW) == 0, "value tiles");
    static_assert(TPG >= 1 && C % NGRP == 0, "gate layout");
};

template <typename TIn, class K>
struct PSmem {
    f32x2 LP[2][K::C][K::DK];   // (a*lp, l) from the chain, by chunk parity
    TIn Q[K::C][K::QS];         // q^ = q G
    TIn W[K::C][K::QS];         // w^ = w / G
    TIn WT[K::DK][K::CS];       // w^ transposed
    TIn VT[K::DV][K::CS];       // v transposed
    float rho[2][K::C];         // 1/r_t by chunk parity
    float E[2][K::DK];          // pending end-of-subchunk state scale, by parity
    float sc[K::DK];            // state scale before a sub-chunk's readout
    float lT[K::DK];
    int L1;
    int bad[2];
};

// Pre-scale, readout and state update for tokens [ts, L1) of the chunk at t0.
template <typename TIn, class K>
__device__ __forceinline__ void pipe_mfma(PSmem<TIn, K>& sm, f32x4 (&accM)[K::IT][K::JT],
                                          const FwdArgs& p, int bh, int vt, int t0, int ts,
                                          int L1, int gw, int lane) {
    typedef Mma<TIn> M;
    const int c16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int it = 0; it < K::IT; ++it) {
        const f32x4 s = *(const f32x4*)&sm.sc[it * 16 + 4 * g];
#pragma unroll
        for (int jj = 0; jj < K::JT; ++jj) accM[it][jj] *= s;
    }
    typename M::K16 AM[K::IT][K::JT];
#pragma unroll
    for (int it = 0; it < K::IT; ++it)
#pragma unroll
        for (int jj = 0; jj < K::JT; ++jj) AM[it][jj] = M::from_acc(accM[it][jj]);

    const int tb0 = ts / 16, tb1 = (L1 + 15) / 16;
#pragma unroll
    for (int tau = 0; tau < K::NB; ++tau) {
        if (tau < tb0 || tau >= tb1) continue;
        typename M::K16 P[K::NB];
#pragma unroll
        for (int sig = 0; sig <= tau; ++sig) {
            if (sig < tb0) continue;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < K::DK / 32; ++kk)
                acc = M::mma32(M::ld32(&sm.W[sig * 16 + c16][kk * 32 + 8 * g]),
                               M::ld32(&sm.Q[tau * 16 + c16][kk * 32 + 8 * g]), acc);
            if (sig == tau) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * g + e > c16) acc[e] = 0.f;
            }
            P[sig] = M::from_acc(acc);
        }
        const int t = tau * 16 + c16;
        const bool store = (t >= ts) && (t < L1);
#pragma unroll
        for (int jj = 0; jj < K::JT; ++jj) {
            const int jt = gw * K::JT + jj;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int it = 0; it < K::IT; ++it)
                acc = M::mma16(AM[it][jj], M::ld16(&sm.Q[tau * 16 + c16][it * 16 + 4 * g]), acc);
#pragma unroll
            for (int sig = 0; sig <= tau; ++sig) {
                if (sig < tb0) continue;
                acc = M::mma16(M::ld16(&sm.VT[jt * 16 + c16][sig * 16 + 4 * g]), P[sig], acc);
            }
            if (store) {
                TIn* o = (TIn*)p.o;
                const size_t off = ((size_t)bh * p.T + t0 + t) * p.dv + (size_t)vt * K::DV +
                                   jt * 16 + 4 * g;
                *(typename Quad<TIn>::V*)(o + off) = Quad<TIn>::make(acc);
            }
        }
    }
#pragma unroll
    for (int it = 0; it < K::IT; ++it)
#pragma unroll
        for (int jj = 0; jj < K::JT; ++jj) {
            const int jt = gw * K::JT + jj;
            accM[it][jj] = M::mma32(M::ld32(&sm.WT[it * 16 + c16][8 * g]),
                                    M::ld32(&sm.VT[jt * 16 + c16][8 * g]), accM[it][jj]);
        }
}

// Store N consecutive values of T (16-byte aligned destination) as wide LDS writes.
template <typename T, int N>
__device__ __forceinline__ void store_row(T* dst, const T (&v)[N]) {
    constexpr int PER = 16 / (int)sizeof(T);   // values per 16-byte store
    if constexpr (N % PER == 0) {
#pragma unroll
        for (int b = 0; b < N / PER; ++b) {
            T tmp[PER];
#pragma unroll
            for (int e = 0; e < PER; ++e) tmp[e] = v[b * PER + e];
            *(f32x4*)(dst + b * PER) = __builtin_bit_cast(f32x4, tmp);
        }
    } else if constexpr ((N * (int)sizeof(T)) % 8 == 0) {
        constexpr int P8 = 8 / (int)sizeof(T);
#pragma unroll
        for (int b = 0; b < N / P8; ++b) {
            T tmp[P8];
#pragma unroll
            for (int e = 0; e < P8; ++e) tmp[e] = v[b * P8 + e];
            *(f32x2*)(dst + b * P8) = __builtin_bit_cast(f32x2, tmp);
        }
    } else {
#pragma unroll
        for (int e = 0; e < N; ++e) dst[e] = v[e];
    }
}

// Exclusive product over the token groups of one key-dim pair (lanes
// grp*IPW + ipl of the same wave).
template <class K>
__device__ __forceinline__ float group_exclusive_prod(float x, int grp) {
    float incl = x;
#pragma unroll
    for (int d = 1; d < K::NGRP; d <<= 1) {
        const float y = __shfl_up(incl, d * K::IPW, 64);
        if (grp >= d) incl *= y;
    }
    float excl = __shfl_up(incl, K::IPW, 64);
    return grp == 0 ? 1.f : excl;
}

// Chain role: one lane per key dim, precision recurrence one chunk ahead.
template <typename TIn, class K>
__device__ __forceinline__ void chain_role(PSmem<TIn, K>& sm, const FwdArgs& p, int bh, int vt,
                                           int wave, int lane) {
    constexpr int C = K::C, DK = K::DK;
    const int ci = wave * 64 + lane;
    const int h = bh % p.H;
    const size_t rowbase = (size_t)bh * p.T;
    const int nchunks = (p.T + C - 1) / C;
    const TIn* kp = (const TIn*)p.k;

    float cl = p.l0 ? p.l0[(size_t)bh * DK + ci] : 1.f;
    const float cqn = p.qn[(size_t)h * DK + ci];
    float ca[C], na[C];
    TIn ck[C], nk[C];
    float crho = 1.f, nrho = 1.f;   // r_t of lane t, turned into 1/r_t before use

    auto load = [&](int c, float (&a_)[C], TIn (&k_)[C], float& r_) {
        const int t0 = c * C;
        const int L = (p.T - t0) < C ? (p.T - t0) : C;
#pragma unroll
        for (int t = 0; t < C; ++t) {
            const int tt = t < L ? t : L - 1;   // clamp: every load stays in bounds
            const size_t off = (rowbase + t0 + tt) * DK + ci;
            a_[t] = p.a[off];
            k_[t] = kp[off];
        }
        r_ = p.r[rowbase + t0 + (lane < L ? lane : L - 1)];
    };
    // lp = l / (a^2 + qn l),  l' = lp + k^2 / r, over tokens [u0, u1) of chunk c
    auto run = [&](int c, int u0, int u1) {
        const int t0 = c * C;
        const int L = (p.T - t0) < C ? (p.T - t0) : C;
        const int par = c & 1;
#pragma unroll
        for (int t = 0; t < C; ++t) {
            if (t >= u0 && t < u1 && t < L) {
                const float rho =
                    __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, crho), t));
                const float a = ca[t], kv = (float)ck[t];
                const float b = kv * kv * rho;
                const float lp = cl * fast_rcp(__builtin_fmaf(cqn, cl, a * a));
                cl = lp + b;
                sm.LP[par][t][ci] = f32x2{a * lp, cl};
            }
        }
    };
    auto advance = [&]() {
#pragma unroll
        for (int t = 0; t < C; ++t) { ca[t] = na[t]; ck[t] = nk[t]; }
        crho = nrho;
    };

    sm.E[1][ci] = 1.f;
    if (wave == 0 && lane == 0) { sm.bad[0] = 0; sm.bad[1] = 0; }
    if (nchunks > 0) {
        load(0, ca, ck, crho);
        if (nchunks > 1) load(1, na, nk, nrho);
        crho = 1.f / crho;
        if (wave == 0 && lane < C) sm.rho[0][lane] = crho;
        run(0, 0, C);
        advance();
    }
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        const int L = (p.T - t0) < C ? (p.T - t0) : C;
        const int cp = c & 1;
        const bool has_next = c + 1 < nchunks;
        if (c + 2 < nchunks) load(c + 2, na, nk, nrho);
        if (has_next) {
            crho = 1.f / crho;
            if (wave == 0 && lane < C) sm.rho[cp ^ 1][lane] = crho;
            run(c + 1, 0, C / 2);
        }
        __syncthreads();                                         // X
        if (sm.bad[cp]) {                                        // mirror the split's barriers
            int ts = 0;
            while (ts < L) {
                __syncthreads();                                 // F1
                const int L1 = sm.L1;
                __syncthreads();                                 // F2
                ts = L1;
                __syncthreads();                                 // F3
                if (wave == 0 && lane == 0) sm.L1 = L;
                __syncthreads();                                 // F4
            }
        }
        if (has_next) {
            run(c + 1, C / 2, C);
            advance();
        }
        __syncthreads();                                         // Y
    }
    sm.lT[ci] = cl;
    if (p.lT && vt == 0) p.lT[(size_t)bh * DK + ci] = cl;
    __syncthreads();                                             // E
}

// Gate role: gates, MFMA operands, MFMA work for the current chunk.
template <typename TIn, class K>
__device__ __forceinline__ void gate_role(PSmem<TIn, K>& sm, const FwdArgs& p, int bh, int vt,
                                          int gw, int lane) {
    typedef Pair<TIn> PR;
    constexpr int C = K::C, DK = K::DK, DV = K::DV, TPG = K::TPG;
    const size_t rowbase = (size_t)bh * p.T;
    const int nchunks = (p.T + C - 1) / C;
    const int grp = lane / K::IPW, ipl = lane % K::IPW;
    const int ip = gw * K::IPW + ipl;               // key-dim pair
    const int c16 = lane & 15, g = lane >> 4;
    const int gtid = gw * 64 + lane;
    const TIn* qp = (const TIn*)p.q;
    const TIn* kp = (const TIn*)p.k;
    const TIn* vp = (const TIn*)p.v;

    typename PR::V gq[TPG], gk[TPG], nq[TPG], nk[TPG];
    typename Quad<TIn>::V gv[K::VPT][2], nv[K::VPT][2];
    auto load = [&](int c, typename PR::V (&q2)[TPG], typename PR::V (&k2)[TPG],
                    typename Quad<TIn>::V (&v4)[K::VPT][2]) {
        const int t0 = c * C;
        const int L = (p.T - t0) < C ? (p.T - t0) : C;
#pragma unroll
        for (int u = 0; u < TPG; ++u) {
            const int t = grp * TPG + u;
            const int tt = t < L ? t : L - 1;   // clamp: masked later, load stays in bounds
            const size_t off = (rowbase + t0 + tt) * DK + 2 * ip;
            q2[u] = *(const typename PR::V*)(qp + off);
            k2[u] = *(const typename PR::V*)(kp + off);
        }
#pragma unroll
        for (int x = 0; x < K::VPT; ++x) {
            const int unit = gtid + x * 256;
            const int tp = unit / K::VQ, jq = unit % K::VQ;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int t = 2 * tp + h2;
                const int tt = t < L ? t : L - 1;   // rows past the end meet zero weights
                const int jj = unit < K::VUNITS ? 4 * jq : 0;
                const size_t off = (rowbase + t0 + tt) * p.dv + (size_t)vt * DV + jj;
                v4[x][h2] = *(const typename Quad<TIn>::V*)(vp + off);
            }
        }
    };

    f32x4 accM[K::IT][K::JT];
#pragma unroll
    for (int it = 0; it < K::IT; ++it)
#pragma unroll
        for (int jj = 0; jj < K::JT; ++jj) {
            const int jt = gw * K::JT + jj;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = it * 16 + 4 * g + e;
                const int j = vt * DV + jt * 16 + c16;
                accM[it][jj][e] = p.eta0 ? p.eta0[((size_t)bh * DK + i) * p.dv + j] /
                                               (p.l0 ? p.l0[(size_t)bh * DK + i] : 1.f)
                                         : 0.f;
            }
        }
    if (nchunks > 0) load(0, gq, gk, gv);
    __syncthreads();

    int par = 0;  // E parity the next sub-chunk writes
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        const int L = (p.T - t0) < C ? (p.T - t0) : C;
        const int cp = c & 1;
        const bool has_next = c + 1 < nchunks;

        // ---------------- phase A: V^T, gates, operands
#pragma unroll
        for (int x = 0; x < K::VPT; ++x) {
            const int unit = gtid + x * 256;
            if (unit < K::VUNITS) {
                const int tp = unit / K::VQ, jq = unit % K::VQ;
                const f32x4 v0 = Quad<TIn>::to_f32(gv[x][0]), v1 = Quad<TIn>::to_f32(gv[x][1]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *(typename PR::V*)&sm.VT[4 * jq + e][2 * tp] = PR::make(v0[e], v1[e]);
            }
        }
        if (has_next) load(c + 1, nq, nk, nv);

        float f[TPG][2], w[TPG][2], G[TPG][2];
        float p0 = 1.f, p1 = 1.f;
#pragma unroll
        for (int u = 0; u < TPG; ++u) {
            const int t = grp * TPG + u;
            const f32x4 lp = *(const f32x4*)&sm.LP[cp][t][2 * ip];   // a*lp, l for 2 key dims
            const float rh = sm.rho[cp][t];
            const float rl0 = fast_rcp(lp[1]), rl1 = fast_rcp(lp[3]);
            f[u][0] = lp[0] * rl0;
            f[u][1] = lp[2] * rl1;
            w[u][0] = PR::lo(gk[u]) * rh * rl0;
            w[u][1] = PR::hi(gk[u]) * rh * rl1;
            if (t > 0 && t < L) { p0 *= f[u][0]; p1 *= f[u][1]; }
            G[u][0] = p0;
            G[u][1] = p1;
        }
        {
            const float e0 = group_exclusive_prod<K>(p0, grp);
            const float e1 = group_exclusive_prod<K>(p1, grp);
            bool badl = false;
            TIn wt0[TPG], wt1[TPG];
#pragma unroll
            for (int u = 0; u < TPG; ++u) {
                const int t = grp * TPG + u;
                const float g0 = G[u][0] * e0, g1 = G[u][1] * e1;
                const bool in = t < L;
                badl |= in && (g0 < kFloor || g1 < kFloor);
                float q0 = 0.f, q1 = 0.f, w0 = 0.f, w1 = 0.f;
                if (in) {
                    q0 = PR::lo(gq[u]) * g0;
                    q1 = PR::hi(gq[u]) * g1;
                    w0 = w[u][0] * fast_rcp(g0);
                    w1 = w[u][1] * fast_rcp(g1);
                }
                *(typename PR::V*)&sm.Q[t][2 * ip] = PR::make(q0, q1);
                *(typename PR::V*)&sm.W[t][2 * ip] = PR::make(w0, w1);
                wt0[u] = (TIn)w0;
                wt1[u] = (TIn)w1;
                if (t == 0) {
                    sm.sc[2 * ip] = sm.E[par ^ 1][2 * ip] * f[u][0];
                    sm.sc[2 * ip + 1] = sm.E[par ^ 1][2 * ip + 1] * f[u][1];
                }
                if (t == L - 1) {
                    sm.E[par][2 * ip] = g0;
                    sm.E[par][2 * ip + 1] = g1;
                }
            }
            store_row<TIn, TPG>(&sm.WT[2 * ip][grp * TPG], wt0);
            store_row<TIn, TPG>(&sm.WT[2 * ip + 1][grp * TPG], wt1);
            if (__builtin_amdgcn_ballot_w64(badl)) sm.bad[cp] = 1;
            if (gtid == 0) { sm.bad[cp ^ 1] = 0; sm.L1 = L; }
        }
        __syncthreads();                                         // X

        // ---------------- phase B: MFMA (or the exact split)
        if (!sm.bad[cp]) {
            pipe_mfma<TIn, K>(sm, accM, p, bh, vt, t0, 0, L, gw, lane);
            par ^= 1;
        } else {
            int ts = 0;
            while (ts < L) {
                float Gs[TPG][2];
                float s0 = 1.f, s1 = 1.f;
#pragma unroll
                for (int u = 0; u < TPG; ++u) {
                    const int t = grp * TPG + u;
                    if (t > ts && t < L) { s0 *= f[u][0]; s1 *= f[u][1]; }
                    Gs[u][0] = s0;
                    Gs[u][1] = s1;
                }
                const float e0 = group_exclusive_prod<K>(s0, grp);
                const float e1 = group_exclusive_prod<K>(s1, grp);
                int firstbad = L;
#pragma unroll
                for (int u = 0; u < TPG; ++u) {
                    const int t = grp * TPG + u;
                    Gs[u][0] *= e0;
                    Gs[u][1] *= e1;
                    if (t >= ts && t < L && (Gs[u][0] < kFloor || Gs[u][1] < kFloor))
                        firstbad = t < firstbad ? t : firstbad;
                }
                if (firstbad < L) atomicMin(&sm.L1, firstbad);
                __syncthreads();                                 // F1
                const int L1 = sm.L1;
                TIn wt0[TPG], wt1[TPG];
#pragma unroll
                for (int u = 0; u < TPG; ++u) {
                    const int t = grp * TPG + u;
                    const bool keep = (t >= ts) && (t < L1);
                    float q0 = 0.f, q1 = 0.f, w0 = 0.f, w1 = 0.f;
                    if (keep) {
                        q0 = PR::lo(gq[u]) * Gs[u][0];
                        q1 = PR::hi(gq[u]) * Gs[u][1];
                        w0 = w[u][0] * fast_rcp(Gs[u][0]);
                        w1 = w[u][1] * fast_rcp(Gs[u][1]);
                    }
                    *(typename PR::V*)&sm.Q[t][2 * ip] = PR::make(q0, q1);
                    *(typename PR::V*)&sm.W[t][2 * ip] = PR::make(w0, w1);
                    wt0[u] = (TIn)w0;
                    wt1[u] = (TIn)w1;
                    if (t == ts) {
                        sm.sc[2 * ip] = sm.E[par ^ 1][2 * ip] * f[u][0];
                        sm.sc[2 * ip + 1] = sm.E[par ^ 1][2 * ip + 1] * f[u][1];
                    }
                    if (t == L1 - 1) {
                        sm.E[par][2 * ip] = Gs[u][0];
                        sm.E[par][2 * ip + 1] = Gs[u][1];
                    }
                }
                store_row<TIn, TPG>(&sm.WT[2 * ip][grp * TPG], wt0);
                store_row<TIn, TPG>(&sm.WT[2 * ip + 1][grp * TPG], wt1);
                __syncthreads();                                 // F2
                pipe_mfma<TIn, K>(sm, accM, p, bh, vt, t0, ts, L1, gw, lane);
                par ^= 1;
                ts = L1;
                __syncthreads();                                 // F3
                __syncthreads();                                 // F4 (a chain lane resets L1)
            }
        }
        if (has_next) {
#pragma unroll
            for (int u = 0; u < TPG; ++u) { gq[u] = nq[u]; gk[u] = nk[u]; }
#pragma unroll
            for (int x = 0; x < K::VPT; ++x) { gv[x][0] = nv[x][0]; gv[x][1] = nv[x][1]; }
        }
        __syncthreads();                                         // Y
    }
    __syncthreads();                                             // E
    if (p.etaT) {
#pragma unroll
        for (int it = 0; it < K::IT; ++it)
#pragma unroll
            for (int jj = 0; jj < K::JT; ++jj) {
                const int jt = gw * K::JT + jj;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = it * 16 + 4 * g + e;
                    const int j = vt * DV + jt * 16 + c16;
                    p.etaT[((size_t)bh * DK + i) * p.dv + j] =
                        accM[it][jj][e] * sm.E[par ^ 1][i] * sm.lT[i];
                }
            }
    }
}

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__((PCfg<TIn, DK, DV>::NT)) void kla_fwd_diag_pipe_kernel(FwdArgs p) {
    typedef PCfg<TIn, DK, DV> K;
    __shared__ PSmem<TIn, K> sm;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int BH = p.B * p.H, nvt = p.n_vtiles;
    int bh, vt;
    {
        const int id = blockIdx.x;
        if (nvt > 1 && BH % 8 == 0) {   // all value tiles of a (b,h) on one XCD
            const int x = id % 8, kx = id / 8;
            bh = (kx / nvt) * 8 + x;
            vt = kx % nvt;
        } else {
            bh = id / nvt;
            vt = id % nvt;
        }
    }
    // Both roles execute the same sequence of workgroup barriers.
    if (wave < K::NCW)
        chain_role<TIn, K>(sm, p, bh, vt, wave, lane);
    else
        gate_role<TIn, K>(sm, p, bh, vt, wave - K::NCW, lane);
}

template <typename TIn, int DK, int DV>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
    typedef PCfg<TIn, DK, DV> K;
    const int nblk = a.B * a.H * a.n_vtiles;
    hipLaunchKernelGGL((kla_fwd_diag_pipe_kernel<TIn, DK, DV>), dim3(nblk), dim3(K::NT), 0, s, a);
    return hipGetLastError();
}

template <typename TIn>
hipError_t dispatch(const FwdArgs& a, hipStream_t s) {
    const int dvt = a.dv / a.n_vtiles;
    if (a.dk != a.dv || a.dv % a.n_vtiles) return hipErrorInvalidValue;
    if (a.dk == 128 && dvt == 128) return launch<TIn, 128, 128>(a, s);
    if (a.dk == 128 && dvt == 64) return launch<TIn, 128, 64>(a, s);
    if (a.dk == 64 && dvt == 64) return launch<TIn, 64, 64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace

bool fwd_diag_pipe_supported(int dk, int dv, int nvt) {
    if (dk != dv || dv % nvt) return false;
    const int dvt = dv / nvt;
    return (dk == 128 && (dvt == 128 || dvt == 64)) || (dk == 64 && dvt == 64);
}

hipError_t launch_fwd_diag_pipe(const FwdArgs& a, int dtype, hipStream_t s) {
    return dtype == DT_BF16 ? dispatch<bf16>(a, s) : dispatch<float>(a, s);
}

}  // namespace kla
