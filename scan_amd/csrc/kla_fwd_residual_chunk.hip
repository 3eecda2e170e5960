// kla_fwd_residual_chunk.hip -- gfx950 chunked forward of the residual-write
// variant ("Kalman Delta Networks: Uncertainty-aware Associative Memory",
// abstract: the Kalman gain weights a write of the residual; diagonal and
// isotropic approximations), on the matrix cores.
//
// Recurrence per (b,h) (the same as the block kernel of kla_fwd_residual.hip):
//   lp = l / (a^2 + qn l),  c = k / lp,  den = k.c + r,  g = c / den
//   u  = v - (a (.) m)^T k,  m = a (.) m + g u^T,  l = lp + k^2 / r,  o = m^T q
// Over a chunk of C = 16 tokens from the state M0 at its start, with
// Gam_t = a_1 ... a_t per key dim, K~ = Gam (.) K, Q~ = Gam (.) Q (rows per
// token), C^ = C / Gam and u'_s = u_s / den_s:
//   (a (.) m_{t-1})^T k_t = K~_t^T M0 + sum_{s<t} (K~_t . C^_s) u'_s
//   (diag(den) + strictlower(K~ C^T)) U' = V - K~ M0
//   O = Q~ M0 + lower(Q~ C^T) U'
//   M_C = Gam_C (.) M0 + E^T U',   E_s = (a_{s+1} ... a_C) (.) c_s
// Only the products with M0 and U' depend on the state.  The rest -- the
// precision chain, the Gram matrices K~ C^T and Q~ C^T, and the inverse
// T' = (diag(den) + strictlower(K~ C^T))^{-1} -- depends on the inputs only
// and runs one and two chunks ahead in other waves.
//
// Isotropic: the precision, decay and process noise are scalars per token,
// c = k / lp and den = |k|^2 / lp + r; the same chunk algebra with a scalar
// Gam_t.
//
// Roles (one workgroup per (b,h) and 64 value columns; tiles of one (b,h)
// run 8 workgroups apart, on one XCD):
// - chain waves (dk/64, one lane per key dim; isotropic: each forms |k_t|^2
//   over all key dims by a wave reduction and runs the scalar recursion in
//   every lane): the precision recursion and the rows of K~, Q~, C^, E and
//   Gam_C in LDS;
// - prep waves (2): the Gram matrices on the matrix cores (wave 0 K~ C^T,
//   wave 1 Q~ C^T), den = diag(K~ C^T) + r, and in wave 0 the inverse of the
//   unit lower triangular I + N, N = diag(den)^-1 strictlower(K~ C^T), by
//   forward substitution (a column per lane quad), scaled to T';
// - state waves (2, 32 value columns each as two 16-column groups): per
//   chunk [K~; Q~] M0, U' = T' (V - K~ M0), O = Q~ M0 + C' U' and the update,
//   the state in accumulator tiles for the whole sequence.
// Iteration j of the loop: chain on chunk j, prep on chunk j-1, state on
// chunk j-2, one workgroup barrier (LDS only) per iteration.
//
// C^ = c / Gam divides by the decay products.  A chain wave whose Gam leaves
// [2^-64, 2^64] within a chunk writes zero C^ rows for its key dims and
// instead forms their contribution to K~ C^T and Q~ C^T exactly, as sums of
// D(s,t) k_t c_s and D(s,t) q_t c_s with D(s,t) = a_{s+1} ... a_t (products
// only), which the prep waves add to the matrix-core Gram; its E rows then
// come from suffix products of the decays too (on the factorised path E is
// Gam_C C^).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "kla_common.h"
#include "kla_residual.h"

namespace kla {
namespace {

constexpr int kRC = 16;                 // tokens per chunk
constexpr int kRCP = kRC + 4;           // padded row of the [.][kRC] arrays
constexpr float kGamLo = 0x1p-64f, kGamHi = 0x1p64f;  // range of Gam for C^ = c / Gam
constexpr int kRcDVT = 64;              // value columns per workgroup

template <int D, bool ISO>
struct RcRoles {
    static constexpr int NCW = D / 64;  // chain waves
    static constexpr int NSW = 2;       // state waves
    static constexpr int NPW = 2;       // prep waves
    static constexpr int NW = NCW + NSW + NPW;
    // waves go round-robin over the four SIMDs: chain waves first, then the
    // state waves, so that the two never share a SIMD
    static constexpr int W_STATE = NCW, W_PREP = NCW + NSW;
};

// S: operand storage (bf16, or fp32 split into bf16 pairs at the read).
// Token-major rows are padded by 16 bytes and the [.][kRC] rows by 4 values,
// so that the 16 rows a fragment read touches fall in distinct banks.
template <typename S, int D, bool ISO>
struct RcSm {
    static constexpr int NCW = RcRoles<D, ISO>::NCW;
    static constexpr int DW = ISO ? D : 64;       // key dims staged per chain wave (isotropic: all, for |k|^2)
    static constexpr int PAD = 16 / (int)sizeof(S);
    static constexpr int KP = D + PAD;
    alignas(16) S kt[3][kRC][KP];                 // K~ rows
    alignas(16) S qt[3][kRC][KP];                 // Q~ rows
    alignas(16) S ch[2][kRC][KP];                 // C^ rows (zero off the factorisation)
    alignas(16) S e[3][D][kRCP];                  // E, key-dim-major
    alignas(16) S tp[2][kRC][kRCP];               // T'
    alignas(16) S cp[2][kRC][kRCP];               // C' = lower(Q~ C^T)
    alignas(16) float gc[3][D];                   // Gam_C
    alignas(16) float rr[2][kRC];                 // r of the chunk's tokens
    alignas(16) float gx[2][NCW][kRC][2 * kRC];   // exact sums [t][s] (K~ C^T, s <= t), [t][kRC + s] (Q~ C^T)
    alignas(16) float nt[kRC][4][4];              // N as [t][s % 4][s / 4]
    alignas(16) float dn[kRC];                    // den of the chunk's tokens
    // staging of a chunk's input rows (loaded into registers two chunks
    // ahead by the chain waves, one by the state waves): per chain wave its
    // key dims of k, q (and diagonal a); per state wave its 32 columns of v,
    // then of o
    alignas(16) S rk[NCW][kRC][DW + PAD];
    alignas(16) S rq[NCW][kRC][DW + PAD];
    alignas(16) float ra[NCW][kRC][ISO ? 4 : 64 + 4];   // diagonal decays
    alignas(16) S sv[2][kRC][32 + PAD];
    alignas(16) S ost[2][kRC][32 + PAD];
    int off[2][NCW];                              // chain wave off the factorisation
};

template <int CTRL>
__device__ __forceinline__ float dpp_q(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Two accumulator tiles as one K32 operand (slots 0-3 from lo, 4-7 from hi).
template <typename S>
__device__ __forceinline__ typename Frag<S>::V frag_acc(f32x4 lo, f32x4 hi) {
    if constexpr (std::is_same<S, bf16>::value) {
        typedef short s16x8 __attribute__((__vector_size__(16)));
        const s16x4 a = pack_bf16x4(lo[0], lo[1], lo[2], lo[3]);
        const s16x4 b = pack_bf16x4(hi[0], hi[1], hi[2], hi[3]);
        const s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        return __builtin_bit_cast(bf16x8, r);
    } else {
        return Frag<S>::from_acc(lo, hi);
    }
}

// LDS written by some lanes of a wave and then read by others of the same
// wave: order the accesses (the LDS executes a wave's instructions in order).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Rows [row, row + n) of a row-major [., D] array as a buffer resource of
// exactly those rows (loads past them read zero, stores past them are
// dropped).
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const T* base, size_t row, int n, int D) {
    return make_rsrc(base + row * D, n * D * (int)sizeof(T));
}

template <typename TIn, int D, bool ISO>
__global__ __launch_bounds__((RcRoles<D, ISO>::NW * 64)) void kla_fwd_residual_chunk_kernel(FwdArgs p) {
    typedef RcRoles<D, ISO> R;
    typedef TIn S;
    typedef RcSm<S, D, ISO> Sm;
    typedef Frag<S> F;     // K32 operands
    typedef Mma<TIn> MA;   // K16 operands
    constexpr int NVT = D / kRcDVT;
    constexpr int ES = (int)sizeof(TIn);
    __shared__ Sm sm;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int x8 = (int)blockIdx.x;
    const int vt = NVT == 1 ? 0 : (x8 / 8) % NVT;
    const int bh = NVT == 1 ? x8 : (x8 / (8 * NVT)) * 8 + x8 % 8;
    const int nbh = p.B * p.H;
    if (bh >= nbh) return;  // padding of the grid to the XCD pattern: the whole workgroup
    const int h = bh % p.H;
    const int T = p.T, nch = (T + kRC - 1) / kRC;
    const size_t row0 = (size_t)bh * T;
    auto nvalid = [&](int c) { return T - c * kRC < kRC ? T - c * kRC : kRC; };

    if (wave < R::NCW) {
      if constexpr (ISO) {
        // ---------------- chain (isotropic): lane holds key dim 64 cw + lane;
        // the precision, decay and process noise are scalars per token, the
        // same in every lane of every chain wave (each forms |k_t|^2 over all
        // key dims itself)
        constexpr int NDL = D / 64;
        const int cw = R::NCW == 1 ? 0 : wave, i = 64 * cw + lane;
        float l = p.l0 ? p.l0[bh] : 1.f;
        // a chunk's k rows (all key dims) and q rows (the wave's) as 16-byte
        // pieces: PRW / PRQ per row, NP / NQ per lane
        constexpr int PRW = D * ES / 16, NP = kRC * PRW / 64;
        constexpr int PRQ = 64 * ES / 16, NQ = kRC * PRQ / 64;
        struct RawI {
            i32x4 k[NP], q[NQ];
            float a, qn, r;  // of token lane % 16
        };
        auto load = [&](int c, RawI& x) {
            const int nv = nvalid(c);
            const size_t r0 = row0 + (size_t)c * kRC;
            const auto rk = rows_rsrc((const TIn*)p.k, r0, nv, D);
            const auto rq = rows_rsrc((const TIn*)p.q, r0, nv, D);
#pragma unroll
            for (int m = 0; m < NP; ++m) {
                const int pc = lane + 64 * m, t = pc / PRW, pe = pc % PRW;
                x.k[m] = buf_load<i32x4>(rk, t * D * ES + 16 * pe);
            }
#pragma unroll
            for (int m = 0; m < NQ; ++m) {
                const int pc = lane + 64 * m, t = pc / PRQ, pe = pc % PRQ;
                x.q[m] = buf_load<i32x4>(rq, (t * D + 64 * cw) * ES + 16 * pe);
            }
            x.a = buf_load<float>(make_rsrc(p.a + r0, nv * 4), (lane & 15) * 4);
            x.qn = buf_load<float>(make_rsrc(p.qn + r0, nv * 4), (lane & 15) * 4);
            x.r = buf_load<float>(make_rsrc(p.r + r0, nv * 4), (lane & 15) * 4);
        };
        auto stage = [&](const RawI& x) {
#pragma unroll
            for (int m = 0; m < NP; ++m) {
                const int pc = lane + 64 * m, t = pc / PRW, pe = pc % PRW;
                *(i32x4*)&sm.rk[cw][t][pe * (16 / ES)] = x.k[m];
            }
#pragma unroll
            for (int m = 0; m < NQ; ++m) {
                const int pc = lane + 64 * m, t = pc / PRQ, pe = pc % PRQ;
                *(i32x4*)&sm.rq[cw][t][pe * (16 / ES)] = x.q[m];
            }
        };
        auto uni = [&](float v, int u) {
            return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), u));
        };
        auto chain = [&](int c, float a_l, float qn_l, float r_l) {
            const int b3 = c % 3, b2 = c & 1;
            const int nv = nvalid(c);
            float kf[kRC], qf[kRC], ks[kRC];
#pragma unroll
            for (int u = 0; u < kRC; ++u) {
                qf[u] = (float)sm.rq[cw][u][lane];
                float kn = (float)sm.rk[cw][u][lane];
                kf[u] = kn;  // the wave's own key dim 64 cw + lane
                ks[u] = kn * kn;
#pragma unroll
                for (int m = 1; m < NDL; ++m) {
                    kn = (float)sm.rk[cw][u][lane + 64 * m];
                    kf[u] = cw == m ? kn : kf[u];
                    ks[u] = __builtin_fmaf(kn, kn, ks[u]);
                }
            }
            // token scalars (rows past the sequence's end: a = 1, r = 1, qn = 0)
            const bool lv = (lane & 15) < nv;
            const float av = lv ? a_l : 1.f, qv = lv ? qn_l : 0.f, rv = lv ? r_l : 1.f;
            if (cw == 0 && lane < kRC) sm.rr[b2][lane] = rv;
            const float irv = fast_rcp(rv) * (1.f / (float)D);
            // |k_t|^2 over the key dims: a reduce-scatter leaves token
            // 8 b5 + 4 b4 + 2 b3 + b2 in lanes with those lane bits
            int base = 0;
            reduce_scatter<kRC, 32>(ks, lane, base);
            float cv[kRC], chv[kRC];
            float gam = 1.f;
            bool ok = true;
#pragma unroll
            for (int u = 0; u < kRC; ++u) {
                const int ol = ((u >> 3) & 1) << 5 | ((u >> 2) & 1) << 4 | ((u >> 1) & 1) << 3 | (u & 1) << 2;
                const float ksq = uni(ks[0], ol), au = uni(av, u);
                const float lp = l * fast_rcp(__builtin_fmaf(uni(qv, u), l, au * au));
                l = u < nv ? __builtin_fmaf(ksq, uni(irv, u), lp) : l;
                gam *= au;
                ok = ok && gam >= kGamLo && gam <= kGamHi;
                cv[u] = kf[u] * fast_rcp(lp);
                chv[u] = cv[u] * fast_rcp(gam);
                sm.kt[b3][u][i] = (S)(gam * kf[u]);
                sm.qt[b3][u][i] = (S)(gam * qf[u]);
                sm.ch[b2][u][i] = (S)chv[u];
            }
            sm.gc[b3][i] = gam;
            const bool fac = __all(ok);
            {
                float ev[kRC];
                if (fac) {
#pragma unroll
                    for (int u = 0; u < kRC; ++u) ev[u] = gam * chv[u];
                } else {
                    float sfx = 1.f;
#pragma unroll
                    for (int u = kRC - 1; u >= 0; --u) {
                        ev[u] = sfx * cv[u];
                        sfx *= uni(av, u);
                    }
                }
#pragma unroll
                for (int u4 = 0; u4 < kRC; u4 += 4)
                    *(typename Quad<S>::V*)&sm.e[b3][i][u4] =
                        Quad<S>::make(f32x4{ev[u4], ev[u4 + 1], ev[u4 + 2], ev[u4 + 3]});
            }
            if (!fac) {
                // the wave's key dims, exactly: D(s,t) k_t c_s and D(s,t) q_t c_s
                // (s <= t), D a product of the scalar decays
#pragma unroll
                for (int u = 0; u < kRC; ++u) sm.ch[b2][u][i] = (S)0.f;
#pragma unroll
                for (int t = 0; t < kRC; ++t) {
                    float w[2 * kRC];
                    float dst = 1.f;
#pragma unroll
                    for (int s2 = kRC - 1; s2 >= 0; --s2) {
                        if (s2 > t) {
                            w[s2] = 0.f;
                            w[kRC + s2] = 0.f;
                            continue;
                        }
                        if (s2 < t) dst *= uni(av, s2 + 1);
                        w[s2] = dst * kf[t] * cv[s2];
                        w[kRC + s2] = dst * qf[t] * cv[s2];
                    }
                    int b = 0;
                    reduce_scatter<2 * kRC, 32>(w, lane, b);
                    if ((lane & 1) == 0) sm.gx[b2][cw][t][b] = w[0];
                }
            }
            if (lane == 0) sm.off[b2][cw] = fac ? 0 : 1;
        };

        RawI xa, xb;
        load(0, xa);
        if (nch > 1) load(1, xb);
        auto step = [&](int j, RawI& x) {
            if (j < nch) {
                stage(x);
                const float a_l = x.a, qn_l = x.qn, r_l = x.r;
                if (j + 2 < nch) load(j + 2, x);
                wave_lds_sync();
                chain(j, a_l, qn_l, r_l);
            }
            lds_barrier();
        };
        for (int j = 0; j < nch + 2; j += 2) {
            step(j, xa);
            if (j + 1 < nch + 2) step(j + 1, xb);
        }
        if (p.lT && vt == 0 && cw == 0 && lane == 0) p.lT[bh] = l;
      } else {
        // ---------------- chain: one lane per key dim
        const int cw = R::NCW == 1 ? 0 : wave, i = 64 * cw + lane;
        float l = p.l0 ? p.l0[(size_t)bh * D + i] : 1.f;
        const float qn = p.qn[(size_t)h * D + i];
        // a chunk's rows of the wave's 64 key dims, 16-byte pieces: lane l
        // loads token l/4, dims 16 (l%4) .. +15 of k, q and a, and r of token l%16
        const int lt = lane >> 2, ld = 16 * (lane & 3);
        constexpr int NKL = ES;  // 16-byte pieces of 16 values of k (or q)
        struct Raw {
            i32x4 k[NKL], q[NKL], a[4];
            float r;
        };
        auto load = [&](int c, Raw& x) {
            const int nv = nvalid(c);
            const size_t r0 = row0 + (size_t)c * kRC;
            const auto rk = rows_rsrc((const TIn*)p.k, r0, nv, D);
            const auto rq = rows_rsrc((const TIn*)p.q, r0, nv, D);
            const auto ra = rows_rsrc(p.a, r0, nv, D);
            const auto rr = make_rsrc(p.r + r0, nv * 4);
            const int ko = (lt * D + 64 * cw + ld) * ES;
#pragma unroll
            for (int h = 0; h < NKL; ++h) {
                x.k[h] = buf_load<i32x4>(rk, ko + 16 * h);
                x.q[h] = buf_load<i32x4>(rq, ko + 16 * h);
            }
#pragma unroll
            for (int h4 = 0; h4 < 4; ++h4) x.a[h4] = buf_load<i32x4>(ra, (lt * D + 64 * cw + ld + 4 * h4) * 4);
            x.r = buf_load<float>(rr, (lane & 15) * 4);
        };
        // rows past the sequence's end load as zero
        auto stage = [&](const Raw& x) {
#pragma unroll
            for (int h = 0; h < NKL; ++h) {
                *(i32x4*)&sm.rk[cw][lt][ld + (16 / ES) * h] = x.k[h];
                *(i32x4*)&sm.rq[cw][lt][ld + (16 / ES) * h] = x.q[h];
            }
#pragma unroll
            for (int h4 = 0; h4 < 4; ++h4) *(i32x4*)&sm.ra[cw][lt][ld + 4 * h4] = x.a[h4];
        };
        auto chain = [&](int c, float rlane) {
            const int b3 = c % 3, b2 = c & 1;
            float kf[kRC], qf[kRC], af[kRC], cv[kRC], gm[kRC];
            // every staged value first (one batch of LDS reads), then the
            // recursion; rows past the sequence's end hold zeros, their decay is 1
#pragma unroll
            for (int u = 0; u < kRC; ++u) {
                kf[u] = (float)sm.rk[cw][u][lane];
                qf[u] = (float)sm.rq[cw][u][lane];
                af[u] = sm.ra[cw][u][lane];
            }
            const int nv = nvalid(c);
#pragma unroll
            for (int u = 0; u < kRC; ++u) af[u] = u < nv ? af[u] : 1.f;
            const float rv = lane < nv ? rlane : 1.f;
            if (cw == 0 && lane < kRC) sm.rr[b2][lane] = rv;
            const float irl = fast_rcp(rv);
            float gam = 1.f;
            bool ok = true;
            float chv[kRC];  // C^ = c / Gam
#pragma unroll
            for (int u = 0; u < kRC; ++u) {
                const float ir = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, irl), u));
                const float lp = l * fast_rcp(__builtin_fmaf(qn, l, af[u] * af[u]));
                cv[u] = kf[u] * fast_rcp(lp);
                l = u < nv ? __builtin_fmaf(kf[u] * kf[u], ir, lp) : l;
                gam *= af[u];
                gm[u] = gam;
                ok = ok && gam >= kGamLo && gam <= kGamHi;
                chv[u] = cv[u] * fast_rcp(gam);
                sm.kt[b3][u][i] = (S)(gam * kf[u]);
                sm.qt[b3][u][i] = (S)(gam * qf[u]);
                sm.ch[b2][u][i] = (S)chv[u];
            }
            sm.gc[b3][i] = gam;
            const bool fac = __all(ok);
            auto put_e = [&](const float (&ev)[kRC]) {
#pragma unroll
                for (int u4 = 0; u4 < kRC; u4 += 4)
                    *(typename Quad<S>::V*)&sm.e[b3][i][u4] =
                        Quad<S>::make(f32x4{ev[u4], ev[u4 + 1], ev[u4 + 2], ev[u4 + 3]});
            };
            if (fac) {
                // E_s = Gam_C c_s / Gam_s
                float ev[kRC];
#pragma unroll
                for (int u = 0; u < kRC; ++u) ev[u] = gam * chv[u];
                put_e(ev);
            } else {
                // E by products of decays, C^ rows zero
                float ev[kRC];
                float sfx = 1.f;
#pragma unroll
                for (int u = kRC - 1; u >= 0; --u) {
                    ev[u] = sfx * cv[u];
                    sfx *= af[u];
                }
                put_e(ev);
#pragma unroll
                for (int u = 0; u < kRC; ++u) sm.ch[b2][u][i] = (S)0.f;
                // this wave's key dims, exactly: D(s,t) k_t c_s and D(s,t) q_t c_s (s <= t)
#pragma unroll
                for (int t = 0; t < kRC; ++t) {
                    float w[2 * kRC];
                    float dst = 1.f;
#pragma unroll
                    for (int s = kRC - 1; s >= 0; --s) {
                        if (s > t) {
                            w[s] = 0.f;
                            w[kRC + s] = 0.f;
                            continue;
                        }
                        if (s < t) dst *= af[s + 1];
                        w[s] = dst * kf[t] * cv[s];
                        w[kRC + s] = dst * qf[t] * cv[s];
                    }
                    int base = 0;
                    reduce_scatter<2 * kRC, 32>(w, lane, base);
                    if ((lane & 1) == 0) sm.gx[b2][cw][t][base] = w[0];
                }
            }
            if (lane == 0) sm.off[b2][cw] = fac ? 0 : 1;
        };

        // iteration j: stage chunk j (its loads were issued at iteration
        // j - 2), issue chunk j + 2's loads into the registers just staged,
        // run the chain on chunk j; two register sets in turn
        Raw xa, xb;
        load(0, xa);
        if (nch > 1) load(1, xb);
        auto step = [&](int j, Raw& x) {
            if (j < nch) {
                stage(x);
                const float rl = x.r;
                if (j + 2 < nch) load(j + 2, x);
                wave_lds_sync();
                chain(j, rl);
            }
            lds_barrier();
        };
        for (int j = 0; j < nch + 2; j += 2) {
            step(j, xa);
            if (j + 1 < nch + 2) step(j + 1, xb);
        }
        if (p.lT && vt == 0) p.lT[(size_t)bh * D + i] = l;
      }
    } else if (wave >= R::W_PREP) {
        // ---------------- prep: Gram matrices, den, the inverse
        const int pw = wave - R::W_PREP;
        const int cl = lane & 15, g4 = lane >> 4;
        auto prep = [&](int c) {
            const int b3 = c % 3, b2 = c & 1;
            const S* arow = pw == 0 ? &sm.kt[b3][cl][0] : &sm.qt[b3][cl][0];
            const S* brow = &sm.ch[b2][cl][0];
            f32x4 G = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < D / 32; ++kb) G = F::mma(F::ld(arow + 32 * kb, g4), F::ld(brow + 32 * kb, g4), G);
            // G: rows t = 4 g4 + e, column s = cl
            const int t0 = 4 * g4, s = cl;
#pragma unroll
            for (int cw = 0; cw < R::NCW; ++cw)
                if (sm.off[b2][cw]) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) G[e] += sm.gx[b2][cw][t0 + e][(pw == 0 ? 0 : kRC) + s];
                }
            if (pw == 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.cp[b2][t0 + e][s] = (S)(s <= t0 + e ? G[e] : 0.f);
                return;
            }
            // den_s = (K~ C^T)[s][s] + r_s, from the lanes holding the diagonal
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (s == t0 + e) sm.dn[s] = G[e] + sm.rr[b2][s];
            wave_lds_sync();
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sm.nt[t0 + e][s & 3][s >> 2] = s < t0 + e ? G[e] * fast_rcp(sm.dn[t0 + e]) : 0.f;
            wave_lds_sync();
            // S = (I + N)^-1 column j = lane / 4; lane phase ph holds rows ph + 4m
            const int j = lane >> 2, ph = lane & 3;
            float sv[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) sv[m] = ph + 4 * m == j ? 1.f : 0.f;
#pragma unroll
            for (int t = 1; t < kRC; ++t) {
                const f32x4 nr = *(const f32x4*)&sm.nt[t][ph][0];
                float part = nr[0] * sv[0];
#pragma unroll
                for (int m = 1; m < 4; ++m) part = __builtin_fmaf(nr[m], sv[m], part);
                part += dpp_q<0xB1>(part);  // quad_perm [1,0,3,2]
                part += dpp_q<0x4E>(part);  // quad_perm [2,3,0,1]
                if (ph == (t & 3) && t > j) sv[t >> 2] = -part;
            }
            const float rdj = fast_rcp(sm.dn[j]);
#pragma unroll
            for (int m = 0; m < 4; ++m) sm.tp[b2][ph + 4 * m][j] = (S)(sv[m] * rdj);
        };
        for (int j = 0; j < nch + 2; ++j) {
            if (j >= 1 && j - 1 < nch) prep(j - 1);
            lds_barrier();
        }
    } else {
        // ---------------- state: two 16-column groups per wave
        const int sw = wave - R::W_STATE;
        const int cl = lane & 15, g4 = lane >> 4;
        const int col0 = vt * kRcDVT + 32 * sw;  // the wave's first value column
        const int col = col0 + cl;               // + 16 g
        constexpr int NRT = D / 16;
        f32x4 M[2][NRT];
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) M[g][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (p.eta0) {
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        M[g][rt][e] = p.eta0[((size_t)bh * D + 16 * rt + 4 * g4 + e) * D + col + 16 * g];
        }
        // the state's loads land here, so that inside the loop the only
        // vector-memory operations in flight are the output stores
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        // 16-byte pieces of a chunk's 16 x 32 block of v (and of o): PR per
        // token row, PL per lane
        constexpr int PR = 32 * ES / 16, PL = kRC * PR / 64;
        i32x4 vr[PL];
        auto loadv = [&](int c) {
            const auto rs = rows_rsrc((const TIn*)p.v, row0 + (size_t)c * kRC, nvalid(c), D);
#pragma unroll
            for (int pl = 0; pl < PL; ++pl) {
                const int pc = lane + 64 * pl, tt = pc / PR, cq = pc % PR;
                vr[pl] = buf_load<i32x4>(rs, (tt * D + col0) * ES + 16 * cq);
            }
        };
        auto state = [&](int c) {
            const int b3 = c % 3, b2 = c & 1;
#pragma unroll
            for (int pl = 0; pl < PL; ++pl) {
                const int pc = lane + 64 * pl, tt = pc / PR, cq = pc % PR;
                *(i32x4*)&sm.sv[sw][tt][cq * (16 / ES)] = vr[pl];
            }
            if (c + 1 < nch) loadv(c + 1);
            f32x4 PK[2], PQ[2];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                PK[g] = f32x4{0.f, 0.f, 0.f, 0.f};
                PQ[g] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            const S* krow = &sm.kt[b3][cl][0];
            const S* qrow = &sm.qt[b3][cl][0];
#pragma unroll
            for (int kb = 0; kb < D / 32; ++kb) {
                const auto ak = F::ld(krow + 32 * kb, g4);
                const auto aq = F::ld(qrow + 32 * kb, g4);
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const auto bm = frag_acc<S>(M[g][2 * kb], M[g][2 * kb + 1]);
                    PK[g] = F::mma(ak, bm, PK[g]);
                    PQ[g] = F::mma(aq, bm, PQ[g]);
                }
            }
            wave_lds_sync();
            const auto at = MA::ld16(&sm.tp[b2][cl][4 * g4]);
            const auto ac = MA::ld16(&sm.cp[b2][cl][4 * g4]);
            typename MA::K16 ub[2];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                f32x4 X;
#pragma unroll
                for (int e = 0; e < 4; ++e) X[e] = (float)sm.sv[sw][4 * g4 + e][16 * g + cl] - PK[g][e];
                const f32x4 U = MA::mma16(at, MA::from_acc(X), f32x4{0.f, 0.f, 0.f, 0.f});
                ub[g] = MA::from_acc(U);
                const f32x4 O = MA::mma16(ac, ub[g], PQ[g]);
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.ost[sw][4 * g4 + e][16 * g + cl] = (S)O[e];
            }
            wave_lds_sync();
            {
                // the chunk's rows of o: stores past token T - 1 fall outside the resource
                const auto rs = rows_rsrc((TIn*)p.o, row0 + (size_t)c * kRC, nvalid(c), D);
#pragma unroll
                for (int pl = 0; pl < PL; ++pl) {
                    const int pc = lane + 64 * pl, tt = pc / PR, cq = pc % PR;
                    buf_store(*(const i32x4*)&sm.ost[sw][tt][cq * (16 / ES)], rs, (tt * D + col0) * ES + 16 * cq);
                }
            }
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const f32x4 gv = *(const f32x4*)&sm.gc[b3][16 * rt + 4 * g4];
                const auto ae = MA::ld16(&sm.e[b3][16 * rt + cl][4 * g4]);
#pragma unroll
                for (int g = 0; g < 2; ++g) M[g][rt] = MA::mma16(ae, ub[g], M[g][rt] * gv);
            }
        };
        loadv(0);
        for (int j = 0; j < nch + 2; ++j) {
            if (j >= 2) state(j - 2);
            lds_barrier();
        }
        if (p.etaT) {
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        p.etaT[((size_t)bh * D + 16 * rt + 4 * g4 + e) * D + col + 16 * g] = M[g][rt][e];
        }
    }
}

template <typename TIn, int D, bool ISO>
void launch(const FwdArgs& a, hipStream_t s) {
    constexpr int NVT = D / kRcDVT;
    const int nbh = a.B * a.H;
    const dim3 grid((unsigned)(NVT == 1 ? nbh : (nbh + 7) / 8 * 8 * NVT));
    hipLaunchKernelGGL((kla_fwd_residual_chunk_kernel<TIn, D, ISO>), grid, dim3(RcRoles<D, ISO>::NW * 64), 0, s, a);
}

template <typename TIn, bool ISO>
void launch_d(const FwdArgs& a, hipStream_t s) {
    if (a.dk == 64) launch<TIn, 64, ISO>(a, s);
    else launch<TIn, 128, ISO>(a, s);
}

}  // namespace

bool fwd_residual_chunk_supported(int dk, int dv, int cov, int dtype) {
    const char* env = getenv("KLA_RES_IMPL");
    if (env && env[0] == 'b') return false;  // KLA_RES_IMPL=block
    (void)cov;
    (void)dtype;
    return dk == dv && (dk == 64 || dk == 128);
}

hipError_t launch_fwd_residual_chunk(const FwdArgs& a, int dtype, int cov, hipStream_t s) {
    if (!fwd_residual_chunk_supported(a.dk, a.dv, cov, dtype) || a.T < 1) return hipErrorInvalidValue;
    if (dtype == DT_BF16) cov ? launch_d<bf16, true>(a, s) : launch_d<bf16, false>(a, s);
    else cov ? launch_d<float, true>(a, s) : launch_d<float, false>(a, s);
    return hipGetLastError();
}

}  // namespace kla
