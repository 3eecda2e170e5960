// kla_bwd_chunk.hip -- gfx950 chunked backward of the forward on the matrix
// cores (bf16 inputs; diagonal at dk = dv in {64, 128}, isotropic at 64).
//
// Sources: "Kalman Linear Attention: Parallel Bayesian Filtering For Efficient
// Language Modelling and State Tracking" (fugumt abstract page: the filter is
// a primitive for parallel training; gist.science explainer, method §1-§3 for
// the recurrence, §2 for evaluating it chunk by chunk).
//
// Forward per (b,h), information form (key dim i, value column j):
//   D_t = a_t^2 + qn l_{t-1},  g_t = a_t / D_t,  l_t = l_{t-1} / D_t + k_t^2 / r_t
//   eta_t = g_t eta_{t-1} + w_t v_t^T  (w = k / r),  o_t = eta_t^T qh_t  (qh = q / l)
// Over a chunk of C = 16 tokens, with G_t = g_1 ... g_t per key dim (from the
// chunk start) and A = G (.) qh (rows per token), the adjoint of kla_bwd.hip
// becomes:
//  forward sweep, from the state eta_in at the chunk start:
//   S = G (.) (dO eta_in^T + lower(dO V^T) (W / G)),  dq = S / l,  Q = qh (.) S
//   eta_out = G_C (.) (eta_in + (W / G)^T V)
//  reverse sweep, from the adjoint eps_out of the state after the chunk:
//   U = (1 / G) (.) (G_C (.) (V eps_out^T) + upper(V dO^T) A)
//   dv = (W / G) (G_C (.) eps_out) + upper((W / G) A^T) dO
//   eps_in = G_C (.) eps_out + A^T dO
//  (lower and upper keep the diagonal), then per token, last first,
//   dlog g_t = <detaT, eta_T> + sum_{s >= t} (Q_s - w_s U_s)
// and the scalar precision adjoint (lbar) of kla_bwd.hip, which gives dk, da,
// dr and the qn partial.  deta0 = eps_in of the first chunk, dl0 = lbar_{-1}.
//
// The matrix products run on bf16 MFMAs with every fp32 operand split into
// a bf16 pair (hi + lo; a product of two split operands takes three MFMAs,
// of a split and an exact bf16 input two): the adjoint of log g is a
// cumulative sum whose terms nearly cancel when the gates are small, so the
// per-token terms need about 2^-16 relative accuracy, not bf16's 2^-9.
//
// Two kernels, each with one workgroup per (b,h) and 64 key dims (dk 128: two
// row tiles, 8 workgroups apart so that they share an XCD and its v, dO):
// - kla_bwd_chunk_fwd: four matrix-core waves (16 key dims each, the state
//   rows eta[i][:] in accumulator tiles; each forms W / G, 1 / l and q / l of
//   its own tokens and key dims and checks the range of G) and a chain wave
//   one chunk ahead (the precision recursion, G, and l at chunk starts);
//   writes dq, Q, the chunk-start precisions, <detaT, eta_T> and the flag.
// - kla_bwd_chunk_rev: chunks last to first.  A chain wave recomputes the
//   chunk's precision from its start, splits A and W / G into bf16 pairs
//   once for all matrix-core waves and hands the precision adjoint g,
//   P = l_{t-1} / D and 1 / a.  Four matrix-core waves hold the adjoint
//   twice: eps[i][:] of 16 key dims for U and the update, and eps[:][j] of
//   D/4 value columns over the tile's 64 key dims for dv (the two products
//   contract it along different axes).  The precision-adjoint wave runs two
//   chunks behind the chain; at the start of each iteration it also forms
//   the chunk's two upper-triangular operands, which the matrix-core waves
//   take from LDS after a bounded wait on its flag.  With two row tiles dv
//   and dr leave per-tile partials that a third kernel sums; with one the
//   sweep writes them itself.
// Isotropic (one row tile): the precision, decay and process noise are
// scalars per token, written into every lane's row, so the matrix-core code
// is shared; the chain waves form |k_t|^2 over the key dims, the adjoint
// wave sums Q and w U over them and runs the scalar recursion.
// The quotients W / G and 1 / G need G in [2^-64, 2^64]: a (b,h) whose decay
// products leave that range in some chunk is flagged by the forward sweep,
// skipped by the reverse sweep and redone by the token-serial kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <type_traits>

#include "kla_bwd.h"
#include "kla_common.h"

namespace kla {
namespace {

constexpr int kBC = 16;          // tokens per chunk
constexpr int kBP = kBC + 4;     // padded [.][kBC] row
constexpr int kTM = 64 + 4;      // padded token-major row of the tile's 64 key dims
constexpr float kGLo = 0x1p-64f, kGHi = 0x1p64f;

typedef Mma<bf16> MB;  // exact bf16 operands, K16
typedef Frag<bf16> FB;  // exact bf16 operands, K32

__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// exact bf16 A times split B, and split A times exact B
__device__ __forceinline__ f32x4 mma_xs(s16x4 a, const SplitK16& b, f32x4 c) {
    return mfma16(a, b.hi, mfma16(a, b.lo, c));
}
__device__ __forceinline__ f32x4 mma_sx(const SplitK16& a, s16x4 b, f32x4 c) {
    return mfma16(a.hi, b, mfma16(a.lo, b, c));
}
__device__ __forceinline__ void buf_store_b16(bf16 v, __amdgpu_buffer_rsrc_t r, int voff) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, voff, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ float uni(float v, int u) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), u));
}

// LDS written by some lanes of a wave and then read by others of the same
// wave: order the accesses.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_of(const T* base, size_t row, int n, int D) {
    return make_rsrc(base + row * D, n * D * (int)sizeof(T));
}

// Workgroup -> ((b,h), row tile): the tiles of one (b,h) 8 workgroups apart.
template <int NT>
__device__ __forceinline__ void bc_place(int& bh, int& tile) {
    const int x8 = (int)blockIdx.x;
    tile = NT == 1 ? 0 : (x8 / 8) % NT;
    bh = NT == 1 ? x8 : (x8 / (8 * NT)) * 8 + x8 % 8;
}

// A chunk's rows of the tile's 64 key dims of k, q (bf16) and a (fp32), and r:
// lane l loads token l / 4, key dims 16 (l % 4) .. +15, and r of token l % 16;
// rows past the sequence's end read zero.  Staged into LDS by the chain wave
// and read back one key dim per lane.
struct ChainRaw {
    i32x4 k[2], q[2], a[4];
    float r, l;
    float as, qs;  // isotropic: a and qn of token lane % 16
};
struct ChainStage {
    alignas(16) bf16 rk[kBC][64 + 8];
    alignas(16) bf16 rq[kBC][64 + 8];
    alignas(16) float ra[kBC][kTM];
};
template <bool ISO>
__device__ __forceinline__ void chain_load(const BwdArgs& p, size_t row0, int c, int nv, int tile, int lane,
                                           ChainRaw& x) {
    const int D = p.dk, lt = lane >> 2, ld = 16 * (lane & 3);
    const size_t r0 = row0 + (size_t)c * kBC;
    const auto rk = rows_of((const bf16*)p.k, r0, nv, D);
    const auto rq = rows_of((const bf16*)p.q, r0, nv, D);
    const auto ra = rows_of(p.a, r0, ISO ? 0 : nv, D);
    const int ko = (lt * D + 64 * tile + ld) * 2;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        x.k[m] = buf_load<i32x4>(rk, ko + 16 * m);
        x.q[m] = buf_load<i32x4>(rq, ko + 16 * m);
    }
    if constexpr (ISO) {
        x.as = buf_load<float>(make_rsrc(p.a + r0, nv * 4), (lane & 15) * 4);
        x.qs = buf_load<float>(make_rsrc(p.qn + r0, nv * 4), (lane & 15) * 4);
    } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) x.a[m] = buf_load<i32x4>(ra, (lt * D + 64 * tile + ld + 4 * m) * 4);
    }
    x.r = buf_load<float>(make_rsrc(p.r + r0, nv * 4), (lane & 15) * 4);
}
template <bool ISO>
__device__ __forceinline__ void chain_stage(ChainStage& st, const ChainRaw& x, int lane) {
    const int lt = lane >> 2, ld = 16 * (lane & 3);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        *(i32x4*)&st.rk[lt][ld + 8 * m] = x.k[m];
        *(i32x4*)&st.rq[lt][ld + 8 * m] = x.q[m];
    }
    if constexpr (!ISO) {
#pragma unroll
        for (int m = 0; m < 4; ++m) *(i32x4*)&st.ra[lt][ld + 4 * m] = x.a[m];
    }
}

// The chain's per-token inputs: a, qn and k^2 (diagonal, per key dim) or the
// head's scalars a_t, qn_t and |k_t|^2 / dk (isotropic; |k|^2 summed over the
// wave's 64 key dims by a reduce-scatter, token u then held by lane
// 32 b3 + 16 b2 + 8 b1 + 4 b0 of u).  Tokens past the end: a = qn = 1.
template <bool ISO, int D>
__device__ __forceinline__ void chain_inputs(const ChainStage& st, int il, int lane, int nv, float qn_dim, float as,
                                             float qs, float (&kf)[kBC], float (&af)[kBC], float (&qv)[kBC],
                                             float (&kk)[kBC]) {
#pragma unroll
    for (int u = 0; u < kBC; ++u) kf[u] = (float)st.rk[u][il];
    if constexpr (ISO) {
        float ks[kBC];
#pragma unroll
        for (int u = 0; u < kBC; ++u) ks[u] = kf[u] * kf[u];
        int base = 0;
        reduce_scatter<kBC, 32>(ks, lane, base);
#pragma unroll
        for (int u = 0; u < kBC; ++u) {
            const int ol = ((u >> 3) & 1) << 5 | ((u >> 2) & 1) << 4 | ((u >> 1) & 1) << 3 | (u & 1) << 2;
            kk[u] = uni(ks[0], ol) * (1.f / (float)D);
            af[u] = u < nv ? uni(as, u) : 1.f;
            qv[u] = u < nv ? uni(qs, u) : 1.f;
        }
    } else {
#pragma unroll
        for (int u = 0; u < kBC; ++u) {
            af[u] = st.ra[u][il];
            qv[u] = qn_dim;
            kk[u] = kf[u] * kf[u];
        }
    }
}

// A chunk's 16 rows of dO and v in 16-byte pieces over the 256 lanes of the
// four matrix-core waves, mt = 64 w + lane for matrix-core wave w (dk 128:
// one piece of each per lane; dk 64: waves 0-1 dO, 2-3 v).
template <int D>
struct MmaRaw {
    static constexpr int PR = D * 2 / 16;         // pieces per row
    static constexpr int NP = 2 * kBC * PR / 256;  // pieces per lane
    i32x4 x[NP];
};
template <int D>
__device__ __forceinline__ void mma_load(const BwdArgs& p, size_t row0, int c, int nv, int mt, MmaRaw<D>& m) {
    typedef MmaRaw<D> R;
    const auto rd = rows_of((const bf16*)p.dO, row0 + (size_t)c * kBC, nv, D);
    const auto rv = rows_of((const bf16*)p.v, row0 + (size_t)c * kBC, nv, D);
#pragma unroll
    for (int u = 0; u < R::NP; ++u) {
        const int pc = mt + 256 * u;
        const int mat = __builtin_amdgcn_readfirstlane(pc / (kBC * R::PR));  // uniform per wave
        const int rem = pc % (kBC * R::PR), t = rem / R::PR, pe = rem % R::PR;
        m.x[u] = buf_load<i32x4>(mat == 0 ? rd : rv, t * D * 2 + 16 * pe);
    }
}
// Row-major dO and v.
template <int D>
__device__ __forceinline__ void mma_stage(const MmaRaw<D>& m, int mt, bf16 (*dO)[D + 8], bf16 (*vv)[D + 8]) {
    typedef MmaRaw<D> R;
#pragma unroll
    for (int u = 0; u < R::NP; ++u) {
        const int pc = mt + 256 * u;
        const int mat = pc / (kBC * R::PR);
        const int rem = pc % (kBC * R::PR), t = rem / R::PR, pe = rem % R::PR;
        *(i32x4*)(mat == 0 ? &dO[t][8 * pe] : &vv[t][8 * pe]) = m.x[u];
    }
}
// A K16 operand along tokens from a row-major [token][column] tile: the
// lane's column at rows 4g .. 4g + 3 (p = &tile[4g][column], S the row
// stride).  A transposed copy of the tile would cost scalar stores that all
// fall in one bank.
__device__ __forceinline__ s16x4 ld_col4(const bf16* p, int S) {
    return s16x4{__builtin_bit_cast(short, p[0]), __builtin_bit_cast(short, p[S]),
                 __builtin_bit_cast(short, p[2 * S]), __builtin_bit_cast(short, p[3 * S])};
}

// ============================================================ forward sweep
template <int D>
struct Bc1Sm {
    alignas(16) float gam[2][64][kBP];   // G, key-major, by chunk parity
    alignas(16) float lt[2][64][kBP];    // l_t
    alignas(16) float ir[2][kBC];        // 1 / r
    alignas(16) float ge[2][64];         // G_C
    ChainStage cs[2];                    // raw k, q (also read by the matrix-core waves), a
    alignas(16) bf16 dO[2][kBC][D + 8];
    alignas(16) bf16 vv[2][kBC][D + 8];
    alignas(16) float ost[4][2][kBC][16 + 4];
    int badw[4];                         // a matrix-core wave saw G out of range
};

template <int D, bool ISO>
__global__ __launch_bounds__(320) void kla_bwd_chunk_fwd(BwdArgs p) {
    constexpr int NT = D / 64, NJT = D / 16;
    __shared__ Bc1Sm<D> sm;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int bh, tile;
    bc_place<NT>(bh, tile);
    if (bh >= p.B * p.H) return;  // padding of the grid: the whole workgroup
    const int h = bh % p.H;
    const int T = p.T, nch = (T + kBC - 1) / kBC;
    const size_t row0 = (size_t)bh * T;
    const BcLayout L = bc_layout(T, D);
    float* ws = p.ws + (size_t)bh * p.ws_stride;
    auto nvalid = [&](int c) { return T - c * kBC < kBC ? T - c * kBC : kBC; };

    if (wave == 4) {
        // ---------------- chain: one lane per key dim
        const int il = lane, i = 64 * tile + il;
        // isotropic: one precision per head, the same in every lane
        float l = p.l0 ? p.l0[ISO ? (size_t)bh : (size_t)bh * D + i] : 1.f;
        const float qn = ISO ? 0.f : p.qn[(size_t)h * D + i];
        // the serial part only: the precision and G; the matrix-core waves
        // form W / G, 1 / l and q / l for their own tokens and check G's range
        auto chain = [&](int c, float rlane, float as, float qs) {
            const int b = c & 1, nv = nvalid(c);
            ws[L.lst + (size_t)c * D + i] = l;  // the precision before the chunk
            float kf[kBC], af[kBC], qv[kBC], kk[kBC];
            chain_inputs<ISO, D>(sm.cs[b], il, lane, nv, qn, as, qs, kf, af, qv, kk);
            const float irl = fast_rcp(lane < nv ? rlane : 1.f);
            if (lane < kBC) sm.ir[b][lane] = irl;
            float gam = 1.f;
            float vg[kBC], vl[kBC];
            // full chunks (all but perhaps the last) without the selects
            // for tokens past the end
            auto run = [&](auto full) {
#pragma unroll
                for (int u = 0; u < kBC; ++u) {
                    const bool in = decltype(full)::value || u < nv;
                    const float rd = fast_rcp(__builtin_fmaf(qv[u], l, af[u] * af[u]));
                    const float g = in ? af[u] * rd : 1.f;
                    l = in ? __builtin_fmaf(kk[u], uni(irl, u), l * rd) : l;
                    gam *= g;
                    vg[u] = gam;
                    vl[u] = l;
                }
            };
            if (nv == kBC) run(std::true_type{});
            else run(std::false_type{});
#pragma unroll
            for (int u = 0; u < kBC; u += 4) {
                *(f32x4*)&sm.gam[b][il][u] = f32x4{vg[u], vg[u + 1], vg[u + 2], vg[u + 3]};
                *(f32x4*)&sm.lt[b][il][u] = f32x4{vl[u], vl[u + 1], vl[u + 2], vl[u + 3]};
            }
            sm.ge[b][il] = gam;
        };
        ChainRaw x;
        chain_load<ISO>(p, row0, 0, nvalid(0), tile, lane, x);
        for (int it = 0; it <= nch; ++it) {
            if (it < nch) {
                chain_stage<ISO>(sm.cs[it & 1], x, lane);
                const float rl = x.r, as = x.as, qs = x.qs;
                if (it + 1 < nch) chain_load<ISO>(p, row0, it + 1, nvalid(it + 1), tile, lane, x);
                wave_sync();
                chain(it, rl, as, qs);
            }
            lds_barrier();
        }
        lds_barrier();  // the matrix-core waves' range checks are in
        if (lane == 0) ((int*)(ws + L.flags))[tile] = (sm.badw[0] | sm.badw[1] | sm.badw[2] | sm.badw[3]) ? 1 : 0;
        return;
    }

    // ---------------- matrix-core waves: key dims 64 tile + 16 w + c16
    const int w = wave, c16 = lane & 15, g = lane >> 4, mt = 64 * w + lane;
    const int il = 16 * w + c16, ig = 64 * tile + il;
    f32x4 eta[NJT];  // eta[ig][16 jt + 4 g + e]
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt)
        eta[jt] = p.eta0 ? *(const f32x4*)&p.eta0[((size_t)bh * D + ig) * D + 16 * jt + 4 * g] : zero4();
    MmaRaw<D> mr;
    bool bad = false;  // G of the lane's tokens and key dim left [2^-64, 2^64]
    auto step = [&](int c) {
        const int b = c & 1, nv = nvalid(c);
        // X = dO eta_in^T, the state tiles as the B operand (K16 over value columns)
        // (two accumulators, so that consecutive MFMAs do not wait on each other)
        f32x4 Xacc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
            const s16x4 df = MB::ld16(&sm.dO[b][c16][16 * jt + 4 * g]);
            const SplitK16 es = split4(eta[jt]);
            Xacc[2 * (jt & 1)] = mfma16(df, es.hi, Xacc[2 * (jt & 1)]);
            Xacc[2 * (jt & 1) + 1] = mfma16(df, es.lo, Xacc[2 * (jt & 1) + 1]);
        }
        const f32x4 X = (Xacc[0] + Xacc[2]) + (Xacc[1] + Xacc[3]);
        // M^T[s][t] = v_s . dO_t; lane holds M[t = c16][s = 4g + e]: the A
        // operand of lower(M) (W / G) as it stands
        f32x4 Mt = zero4();
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb)
            Mt = FB::mma(FB::ld(&sm.vv[b][c16][32 * kb], g), FB::ld(&sm.dO[b][c16][32 * kb], g), Mt);
#pragma unroll
        for (int e = 0; e < 4; ++e) Mt[e] = 4 * g + e <= c16 ? Mt[e] : 0.f;
        // the lane's tokens t = 4g + e of key dim il: W / G, 1 / l, q / l
        // (rows past the end: k = q = 0)
        const f32x4 gm = *(const f32x4*)&sm.gam[b][il][4 * g];
        const f32x4 lv = *(const f32x4*)&sm.lt[b][il][4 * g];
#pragma unroll
        for (int e = 0; e < 4; ++e) bad = bad || !(gm[e] >= kGLo && gm[e] <= kGHi);
        const f32x4 irv = *(const f32x4*)&sm.ir[b][4 * g];
        f32x4 wgv, rlv, qhv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wgv[e] = (float)sm.cs[b].rk[4 * g + e][il] * irv[e] * fast_rcp(gm[e]);
            rlv[e] = fast_rcp(lv[e]);
            qhv[e] = (float)sm.cs[b].rq[4 * g + e][il] * rlv[e];
        }
        const SplitK16 wgs = split4(wgv);
        const f32x4 Y = Mma<float>::mma16(split4(Mt), wgs, zero4());
        // S = G (.) (X + Y); lane holds t = 4g + e, key dim il
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float S = gm[e] * (X[e] + Y[e]);
            sm.ost[w][0][4 * g + e][c16] = S * rlv[e];
            sm.ost[w][1][4 * g + e][c16] = S * qhv[e];
        }
        wave_sync();
        {
            // dq (bf16) and Q (fp32) rows of the wave's 16 key dims; rows past
            // the end fall outside the resources
            const int rr = lane >> 2, cc = 4 * (lane & 3);
            const f32x4 d4 = *(const f32x4*)&sm.ost[w][0][rr][cc];
            const f32x4 q4 = *(const f32x4*)&sm.ost[w][1][rr][cc];
            const auto rdq = rows_of((bf16*)p.gq, row0 + (size_t)c * kBC, nv, D);
            buf_store(Quad<bf16>::make(d4), rdq, (rr * D + 64 * tile + 16 * w + cc) * 2);
            const auto rq = rows_of(ws + L.q, (size_t)c * kBC, nv, D);
            buf_store(q4, rq, (rr * D + 64 * tile + 16 * w + cc) * 4);
        }
        // eta_out = G_C (.) (eta_in + (W / G)^T V)
        const float gev = sm.ge[b][il];
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) eta[jt] = mma_xs(ld_col4(&sm.vv[b][4 * g][16 * jt + c16], D + 8), wgs, eta[jt]) * gev;
    };
    mma_load<D>(p, row0, 0, nvalid(0), mt, mr);
    for (int it = 0; it <= nch; ++it) {
        if (it < nch) mma_stage<D>(mr, mt, sm.dO[it & 1], sm.vv[it & 1]);
        if (it + 1 < nch) mma_load<D>(p, row0, it + 1, nvalid(it + 1), mt, mr);
        if (it >= 1) step(it - 1);
        lds_barrier();
    }
    // <detaT, eta_T> of the lane's key dim
    float z = 0.f;
    if (p.detaT) {
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
            const f32x4 d = *(const f32x4*)&p.detaT[((size_t)bh * D + ig) * D + 16 * jt + 4 * g];
#pragma unroll
            for (int e = 0; e < 4; ++e) z = __builtin_fmaf(d[e], eta[jt][e], z);
        }
    }
    z += __shfl_xor(z, 16, 64);
    z += __shfl_xor(z, 32, 64);
    if (g == 0) ws[L.z + ig] = z;
    const int wb = __any(bad ? 1 : 0);
    if (lane == 0) sm.badw[w] = wb;
    lds_barrier();  // the chain wave writes the flag
}

// ============================================================ reverse sweep
template <int D>
struct Bc2Sm {
    // for the matrix-core waves, by chunk parity
    // (A = G qh and W / G as bf16 pairs hi + lo, split once by the chain wave)
    alignas(16) float rgam[2][64][kBP];       // 1 / G, key-major
    alignas(16) bf16 akh[2][64][kBC + 8];     // A, key-major
    alignas(16) bf16 akl[2][64][kBC + 8];
    alignas(16) bf16 ath[2][kBC][64 + 8];     // A, token-major
    alignas(16) bf16 atl[2][kBC][64 + 8];
    alignas(16) bf16 wth[2][kBC][64 + 8];     // W / G, token-major
    alignas(16) bf16 wtl[2][kBC][64 + 8];
    alignas(16) float ge[2][64];          // G_C
    // for the precision adjoint, by chunk mod 3
    alignas(16) float lg[3][64][kBP];     // g = a / D (1 past the end), key-major
    alignas(16) float lP[3][64][kBP];     // P = l_{t-1} / D
    alignas(16) float lia[3][64][kBP];    // 1 / a (1 past the end)
    alignas(16) float lw[3][64][kBP];     // w = k / r
    alignas(16) float lk[3][64][kBP];     // k
    alignas(16) float ir[3][kBC];         // 1 / r
    alignas(16) float lks[3][kBC];        // isotropic: |k|^2 / dk
    alignas(16) float lqn[3][kBC];        // isotropic: qn
    alignas(16) float ub[2][64][kBP];     // U, key-major, by chunk parity
    // the chunk's upper(V dO^T) and upper((W / G) A^T) as split K16 operands
    // [t][s], formed once by the adjoint wave for the matrix-core waves
    alignas(16) bf16 mvh[kBC][kBC + 4];
    alignas(16) bf16 mvl[kBC][kBC + 4];
    alignas(16) bf16 wdh[kBC][kBC + 4];
    alignas(16) bf16 wdl[kBC][kBC + 4];
    int hand;                             // chunk + 1 once they are written
    ChainStage cs;
    alignas(16) bf16 dO[2][kBC][D + 8];
    alignas(16) bf16 vv[2][kBC][D + 8];
};

template <int D, bool ISO>
__global__ __launch_bounds__(384) void kla_bwd_chunk_rev(BwdArgs p) {
    constexpr int NT = D / 64, NJT = D / 16, JW = D / 4, NJB = JW / 16;
    __shared__ Bc2Sm<D> sm;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int bh, tile;
    bc_place<NT>(bh, tile);
    if (bh >= p.B * p.H) return;
    const int h = bh % p.H;
    const int T = p.T, nch = (T + kBC - 1) / kBC;
    const size_t row0 = (size_t)bh * T;
    const BcLayout L = bc_layout(T, D);
    float* ws = p.ws + (size_t)bh * p.ws_stride;
    {
        // a (b,h) the forward sweep flagged goes to the token-serial kernel
        const int* fl = (const int*)(ws + L.flags);
        int bad = 0;
#pragma unroll
        for (int t2 = 0; t2 < NT; ++t2) bad |= fl[t2];
        if (bad) return;  // uniform over the workgroup
    }
    if (threadIdx.x == 0) sm.hand = 0;  // seen by the others after the first barrier
    auto nvalid = [&](int c) { return T - c * kBC < kBC ? T - c * kBC : kBC; };

    // waves go round-robin over the four SIMDs: the matrix-core waves are
    // 0, 1, 4, 5 (two to a SIMD), the chain wave 2 and the adjoint wave 3
    // each have a SIMD of their own
    if (wave == 2) {
        // ---------------- chain: the chunk's precision again, from its start
        const int il = lane, i = 64 * tile + il;
        const float qn = ISO ? 0.f : p.qn[(size_t)h * D + i];
        auto chain = [&](int c, float rlane, float l, float as, float qs) {
            const int b2 = c & 1, b3 = c % 3, nv = nvalid(c);
            float kf[kBC], qf[kBC], af[kBC], qv[kBC], kk[kBC];
            chain_inputs<ISO, D>(sm.cs, il, lane, nv, qn, as, qs, kf, af, qv, kk);
#pragma unroll
            for (int u = 0; u < kBC; ++u) qf[u] = (float)sm.cs.rq[u][il];
            const float irl = fast_rcp(lane < nv ? rlane : 1.f);
            if (lane < kBC) sm.ir[b3][lane] = irl;
            if constexpr (ISO) {
                if (lane == 0) {
#pragma unroll
                    for (int u = 0; u < kBC; u += 4) {
                        *(f32x4*)&sm.lks[b3][u] = f32x4{kk[u], kk[u + 1], kk[u + 2], kk[u + 3]};
                        *(f32x4*)&sm.lqn[b3][u] = f32x4{qv[u], qv[u + 1], qv[u + 2], qv[u + 3]};
                    }
                }
            }
            // 1 / G as a running product of D / a (the reciprocal of a is
            // needed by the precision adjoint anyway)
            float gam = 1.f, rg = 1.f;
            float vr[kBC], vg[kBC], vP[kBC], vi[kBC], vw[kBC];
            bf16 vah[kBC], val[kBC];
            auto run = [&](auto full) {
#pragma unroll
                for (int u = 0; u < kBC; ++u) {
                    const bool in = decltype(full)::value || u < nv;
                    const float ir = uni(irl, u);
                    const float Dn = __builtin_fmaf(qv[u], l, af[u] * af[u]);
                    const float rd = fast_rcp(Dn);
                    const float ia = fast_rcp(in ? af[u] : 1.f);
                    const float g = in ? af[u] * rd : 1.f;
                    const float P = l * rd;
                    vg[u] = g;
                    vP[u] = P;
                    vi[u] = ia;
                    l = in ? __builtin_fmaf(kk[u], ir, P) : l;
                    gam *= g;
                    rg *= in ? Dn * ia : 1.f;
                    const float wv = kf[u] * ir;
                    vw[u] = wv;
                    const float A = gam * (qf[u] * fast_rcp(l));
                    const float W = wv * rg;
                    const bf16 ah = (bf16)A, wh = (bf16)W;
                    const bf16 al = (bf16)(A - (float)ah), wl = (bf16)(W - (float)wh);
                    vr[u] = rg;
                    vah[u] = ah;
                    val[u] = al;
                    sm.ath[b2][u][il] = ah;
                    sm.atl[b2][u][il] = al;
                    sm.wth[b2][u][il] = wh;
                    sm.wtl[b2][u][il] = wl;
                }
            };
            if (nv == kBC) run(std::true_type{});
            else run(std::false_type{});
#pragma unroll
            for (int u = 0; u < kBC; u += 4) {
                *(f32x4*)&sm.lg[b3][il][u] = f32x4{vg[u], vg[u + 1], vg[u + 2], vg[u + 3]};
                *(f32x4*)&sm.lP[b3][il][u] = f32x4{vP[u], vP[u + 1], vP[u + 2], vP[u + 3]};
                *(f32x4*)&sm.lia[b3][il][u] = f32x4{vi[u], vi[u + 1], vi[u + 2], vi[u + 3]};
                *(f32x4*)&sm.lk[b3][il][u] = f32x4{kf[u], kf[u + 1], kf[u + 2], kf[u + 3]};
                *(f32x4*)&sm.lw[b3][il][u] = f32x4{vw[u], vw[u + 1], vw[u + 2], vw[u + 3]};
                *(f32x4*)&sm.rgam[b2][il][u] = f32x4{vr[u], vr[u + 1], vr[u + 2], vr[u + 3]};
                *(bf16x4*)&sm.akh[b2][il][u] = bf16x4{vah[u], vah[u + 1], vah[u + 2], vah[u + 3]};
                *(bf16x4*)&sm.akl[b2][il][u] = bf16x4{val[u], val[u + 1], val[u + 2], val[u + 3]};
            }
            sm.ge[b2][il] = gam;
        };
        ChainRaw x;
        auto load = [&](int c) {
            chain_load<ISO>(p, row0, c, nvalid(c), tile, lane, x);
            x.l = ws[L.lst + (size_t)c * D + i];
        };
        load(nch - 1);
        for (int it = 0; it < nch + 2; ++it) {
            if (it < nch) {
                const int c = nch - 1 - it;
                chain_stage<ISO>(sm.cs, x, lane);
                const float rl = x.r, lc = x.l, as = x.as, qs = x.qs;
                if (c >= 1) load(c - 1);
                wave_sync();
                chain(c, rl, lc, as, qs);
            }
            lds_barrier();
        }
        return;
    }

    if (wave == 3) {
        // ---------------- precision adjoint, two chunks behind the chain
        const int il = lane, i = 64 * tile + il;
        const float qn = ISO ? 0.f : p.qn[(size_t)h * D + i];
        // isotropic: lbar and dlog g are the head's scalars (the same in every
        // lane), dlog g summing <detaT, eta_T> over the key dims
        float lbar = p.dlT ? p.dlT[ISO ? (size_t)bh : (size_t)bh * D + i] : 0.f;
        float cum = ws[L.z + i];
        if constexpr (ISO) {
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) cum += __shfl_xor(cum, m, 64);
        }
        float dqn = 0.f;
        float qv[kBC];
        auto loadq = [&](int c) {
            const auto rq = rows_of(ws + L.q, (size_t)c * kBC, nvalid(c), D);
#pragma unroll
            for (int u = 0; u < kBC; ++u) qv[u] = buf_load<float>(rq, (u * D + i) * 4);
        };
        // Branch-free over the chunk (a store inside a branch makes the
        // compiler wait for every earlier memory operation): tokens past the
        // end hold a = 1, k = 0, U = 0, Q = 0, leave lbar, cum and the qn
        // partial unchanged, and their stores fall outside the resources.
        // The chunk's rows are read at once and everything that does not
        // depend on the recursion is formed outside its loop.
        auto adj = [&](int c) {
            const int b2 = c & 1, b3 = c % 3, nv = nvalid(c);
            float q2[kBC], gv[kBC], Pv[kBC], iav[kBC], wv[kBC], kv[kBC], Uv[kBC], irv[kBC];
#pragma unroll
            for (int u = 0; u < kBC; u += 4) {
                const f32x4 g4 = *(const f32x4*)&sm.lg[b3][il][u], p4 = *(const f32x4*)&sm.lP[b3][il][u];
                const f32x4 i4 = *(const f32x4*)&sm.lia[b3][il][u], w4 = *(const f32x4*)&sm.lw[b3][il][u];
                const f32x4 k4 = *(const f32x4*)&sm.lk[b3][il][u];
                const f32x4 u4 = *(const f32x4*)&sm.ub[b2][il][u], r4 = *(const f32x4*)&sm.ir[b3][u];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    gv[u + e] = g4[e];
                    Pv[u + e] = p4[e];
                    iav[u + e] = i4[e];
                    wv[u + e] = w4[e];
                    kv[u + e] = k4[e];
                    Uv[u + e] = u4[e];
                    irv[u + e] = r4[e];
                }
            }
#pragma unroll
            for (int u = 0; u < kBC; ++u) q2[u] = qv[u];
            if constexpr (ISO) {
                // the per-token sums over the key dims of Q and w U: a
                // reduce-scatter leaves entry v (v < 16: Q of token v, else
                // w U of token v - 16) in lane 32 b4 + 16 b3 + 8 b2 + 4 b1 + 2 b0
                float sv[2 * kBC];
#pragma unroll
                for (int u = 0; u < kBC; ++u) {
                    sv[u] = q2[u];
                    sv[kBC + u] = wv[u] * Uv[u];
                }
                int base = 0;
                reduce_scatter<2 * kBC, 32>(sv, lane, base);
                auto lane_of = [](int v) {
                    return ((v >> 4) & 1) << 5 | ((v >> 3) & 1) << 4 | ((v >> 2) & 1) << 3 | ((v >> 1) & 1) << 2 |
                           (v & 1) << 1;
                };
                float sQ[kBC], sR[kBC], ks[kBC], qt[kBC], rl[kBC];
#pragma unroll
                for (int u = 0; u < kBC; u += 4) {
                    const f32x4 k4 = *(const f32x4*)&sm.lks[b3][u], q4 = *(const f32x4*)&sm.lqn[b3][u];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ks[u + e] = k4[e];
                        qt[u + e] = q4[e];
                    }
                }
#pragma unroll
                for (int u = 0; u < kBC; ++u) {
                    sQ[u] = uni(sv[0], lane_of(u));
                    sR[u] = uni(sv[0], lane_of(kBC + u));
                    rl[u] = fast_rcp(__builtin_fmaf(ks[u], irv[u], Pv[u]));  // 1 / l_t
                }
                float lb[kBC], cm[kBC];
#pragma unroll
                for (int u = kBC - 1; u >= 0; --u) {
                    cum += sQ[u] - sR[u];
                    lbar = __builtin_fmaf(-sQ[u], rl[u], lbar);
                    lb[u] = lbar;
                    cm[u] = cum;
                    const float lnext = __builtin_fmaf(lbar, gv[u] * gv[u], -cum * (qt[u] * gv[u] * iav[u]));
                    lbar = u < nv ? lnext : lbar;
                }
                const auto rgk = rows_of((bf16*)p.gk, row0 + (size_t)c * kBC, nv, D);
                // per-token outputs (a, qn and r of the head): every lane stores
                // the same value
                const auto rga = rows_of(p.ga, row0 + (size_t)c * kBC, nv, 1);
                const auto rgq = rows_of(p.gqn, row0 + (size_t)c * kBC, nv, 1);
                const auto rdr = rows_of(p.gr, row0 + (size_t)c * kBC, nv, 1);  // one row tile: dr itself
#pragma unroll
                for (int u = 0; u < kBC; ++u) {
                    const float lbu = lb[u], cmu = cm[u], g = gv[u], P = Pv[u];
                    buf_store_b16((bf16)(__builtin_fmaf(2.f * lbu * (1.f / (float)D), kv[u], Uv[u]) * irv[u]), rgk,
                                  (u * D + i) * 2);
                    buf_store(-irv[u] * __builtin_fmaf(lbu * ks[u], irv[u], sR[u]), rdr, u * 4);
                    buf_store(__builtin_fmaf(-2.f * lbu, g * P, cmu * __builtin_fmaf(-2.f, g, iav[u])), rga, u * 4);
                    buf_store(-__builtin_fmaf(lbu * P, P, cmu * P), rgq, u * 4);
                }
            } else {
                // with g = a / D and P = l_{t-1} / D: l_t = P + k w, a^2 / D^2 = g^2,
                // qn / D = qn g / a, a l_{t-1} / D^2 = g P
                float rl[kBC];
#pragma unroll
                for (int u = 0; u < kBC; ++u) rl[u] = fast_rcp(__builtin_fmaf(kv[u], wv[u], Pv[u]));  // 1 / l_t
                // the recursion, last token first: dlog g_t (cum) and lbar
                float lb[kBC], cm[kBC];
#pragma unroll
                for (int u = kBC - 1; u >= 0; --u) {
                    cum = __builtin_fmaf(-wv[u], Uv[u], cum + q2[u]);
                    lbar = __builtin_fmaf(-q2[u], rl[u], lbar);
                    lb[u] = lbar;
                    cm[u] = cum;
                    const float lnext = __builtin_fmaf(lbar, gv[u] * gv[u], -cum * (qn * gv[u] * iav[u]));
                    lbar = u < nv ? lnext : lbar;
                }
                const auto rgk = rows_of((bf16*)p.gk, row0 + (size_t)c * kBC, nv, D);
                const auto rga = rows_of(p.ga, row0 + (size_t)c * kBC, nv, D);
                float dr[kBC];
#pragma unroll
                for (int u = 0; u < kBC; ++u) {
                    const float lbu = lb[u], cmu = cm[u], g = gv[u], P = Pv[u];
                    buf_store_b16((bf16)(__builtin_fmaf(2.f * lbu, kv[u], Uv[u]) * irv[u]), rgk, (u * D + i) * 2);
                    dr[u] = -wv[u] * __builtin_fmaf(lbu, kv[u], Uv[u]) * irv[u];
                    // da = -2 lbar a l_{t-1} / D^2 + dlog g (qn l_{t-1} - a^2) / (a D)
                    buf_store(__builtin_fmaf(-2.f * lbu, g * P, cmu * __builtin_fmaf(-2.f, g, iav[u])), rga, (u * D + i) * 4);
                    const float dqt = __builtin_fmaf(lbu * P, P, cmu * P);
                    dqn -= u < nv ? dqt : 0.f;
                }
                // dr of the tile's key dims: a reduce-scatter leaves token
                // 8 b5 + 4 b4 + 2 b3 + b2 (lane bits) summed over the 64 lanes,
                // the same in the four lanes of a quad
                int base = 0;
                reduce_scatter<kBC, 32>(dr, lane, base);
                if constexpr (NT == 1)
                    buf_store(dr[0], rows_of(p.gr, row0 + (size_t)c * kBC, nv, 1), base * 4);
                else
                    buf_store(dr[0], rows_of(ws + L.drp + (size_t)tile * L.t4, (size_t)c * kBC, nv, 1), base * 4);
            }
            if (c >= 1) loadq(c - 1);  // lands during the next iteration
        };
        // The chunk's two upper-triangular operands (the same for every
        // matrix-core wave): lane (c16, g) holds rows t = c16, columns
        // s = 4g + e of the accumulators, which is its K16 operand slot.
        auto tri = [&](int c) {
            const int b = c & 1, c16 = lane & 15, g = lane >> 4;
            f32x4 Mt = zero4();
#pragma unroll
            for (int kb = 0; kb < D / 32; ++kb)
                Mt = FB::mma(FB::ld(&sm.dO[b][c16][32 * kb], g), FB::ld(&sm.vv[b][c16][32 * kb], g), Mt);
            f32x4 Wt = zero4();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const SplitK32 xa = {FB::ld(&sm.ath[b][c16][32 * kb], g), FB::ld(&sm.atl[b][c16][32 * kb], g)};
                const SplitK32 xw = {FB::ld(&sm.wth[b][c16][32 * kb], g), FB::ld(&sm.wtl[b][c16][32 * kb], g)};
                Wt = Mma<float>::mma32(xa, xw, Wt);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Mt[e] = 4 * g + e >= c16 ? Mt[e] : 0.f;
                Wt[e] = 4 * g + e >= c16 ? Wt[e] : 0.f;
            }
            const SplitK16 ms = split4(Mt), wsp = split4(Wt);
            *(s16x4*)&sm.mvh[c16][4 * g] = ms.hi;
            *(s16x4*)&sm.mvl[c16][4 * g] = ms.lo;
            *(s16x4*)&sm.wdh[c16][4 * g] = wsp.hi;
            *(s16x4*)&sm.wdl[c16][4 * g] = wsp.lo;
            __hip_atomic_store(&sm.hand, c + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        };
        loadq(nch - 1);
        for (int it = 0; it < nch + 2; ++it) {
            if (it >= 1 && it <= nch) tri(nch - it);
            if (it >= 2) adj(nch + 1 - it);
            lds_barrier();
        }
        if constexpr (ISO) {
            if (p.gl0 && lane == 0) p.gl0[bh] = lbar;
        } else {
            if (p.gl0) p.gl0[(size_t)bh * D + i] = lbar;
            ws[(size_t)4 * T * D + i] = dqn;  // this (b,h)'s qn partial
        }
        (void)dqn;
        return;
    }

    // ---------------- matrix-core waves
    const int w = wave < 2 ? wave : wave - 2, c16 = lane & 15, g = lane >> 4, mt = 64 * w + lane;
    const int il = 16 * w + c16, ig = 64 * tile + il;
    const int jw0 = JW * w;
    f32x4 eA[NJT];       // eps[ig][16 jt + 4 g + e]
    f32x4 eB[4][NJB];    // eps[64 tile + 16 ib + 4 g + e][jw0 + 16 jb + c16]
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt)
        eA[jt] = p.detaT ? *(const f32x4*)&p.detaT[((size_t)bh * D + ig) * D + 16 * jt + 4 * g] : zero4();
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                eB[ib][jb][e] = p.detaT ? p.detaT[((size_t)bh * D + 64 * tile + 16 * ib + 4 * g + e) * D + jw0 +
                                                  16 * jb + c16]
                                        : 0.f;
    MmaRaw<D> mr;
    auto step = [&](int c) {
        const int b = c & 1, nv = nvalid(c);
        // P1 = V eps^T over value columns (state tiles as the B operand)
        // (four accumulators, hi and lo products in separate ones, so that
        // consecutive MFMAs do not wait on each other)
        f32x4 Pacc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
            const s16x4 vf = MB::ld16(&sm.vv[b][c16][16 * jt + 4 * g]);
            const SplitK16 es = split4(eA[jt]);
            Pacc[2 * (jt & 1)] = mfma16(vf, es.hi, Pacc[2 * (jt & 1)]);
            Pacc[2 * (jt & 1) + 1] = mfma16(vf, es.lo, Pacc[2 * (jt & 1) + 1]);
        }
        const f32x4 P1 = (Pacc[0] + Pacc[2]) + (Pacc[1] + Pacc[3]);
        // the adjoint wave's upper(V dO^T) and upper((W / G) A^T) of this
        // chunk: a bounded wait on its flag (within the workgroup, which it
        // always reaches first thing in the iteration); should it ever run
        // out, the (b,h) is handed to the token-serial kernel
        {
            int n = 0;
            while (__hip_atomic_load(&sm.hand, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != c + 1 && n < p.spin) {
                __builtin_amdgcn_s_sleep(1);
                ++n;
            }
            if (n >= p.spin) ((int*)(ws + L.flags))[tile] = 1;
        }
        const SplitK16 as = {MB::ld16(&sm.akh[b][il][4 * g]), MB::ld16(&sm.akl[b][il][4 * g])};  // A[s][il]
        const f32x4 P2 = Mma<float>::mma16(SplitK16{MB::ld16(&sm.mvh[c16][4 * g]), MB::ld16(&sm.mvl[c16][4 * g])}, as,
                                           zero4());
        // U = (1 / G) (.) (G_C P1 + P2), key-major for the adjoint wave
        {
            const f32x4 rg = *(const f32x4*)&sm.rgam[b][il][4 * g];
            const float gev = sm.ge[b][il];
            f32x4 U;
#pragma unroll
            for (int e = 0; e < 4; ++e) U[e] = rg[e] * __builtin_fmaf(gev, P1[e], P2[e]);
            *(f32x4*)&sm.ub[b][il][4 * g] = U;
        }
        const SplitK16 wd = {MB::ld16(&sm.wdh[c16][4 * g]), MB::ld16(&sm.wdl[c16][4 * g])};
        // G_C (.) eps on the rows of the value-column copy
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            const f32x4 gr = *(const f32x4*)&sm.ge[b][16 * ib + 4 * g];
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) eB[ib][jb] *= gr;
        }
        // dv = (W / G) (G_C (.) eps) + upper((W / G) A^T) dO for the wave's columns
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            // one accumulator per key-dim block (three MFMAs each), the upper
            // triangle's two in a fifth
            f32x4 dacc[4];
#pragma unroll
            for (int ib = 0; ib < 4; ++ib)
                dacc[ib] = Mma<float>::mma16(SplitK16{MB::ld16(&sm.wth[b][c16][16 * ib + 4 * g]),
                                                      MB::ld16(&sm.wtl[b][c16][16 * ib + 4 * g])},
                                             split4(eB[ib][jb]), zero4());
            const f32x4 du = mma_sx(wd, ld_col4(&sm.dO[b][4 * g][jw0 + 16 * jb + c16], D + 8), zero4());
            const f32x4 dv = ((dacc[0] + dacc[1]) + (dacc[2] + dacc[3])) + du;
            // straight from the accumulator: rows 4g + e, 16 consecutive
            // columns per row (rows past the end are dropped); with one row
            // tile dv itself, with two the tile's partial for the combine pass
            if constexpr (NT == 1) {
                const auto rg = rows_of((bf16*)p.gv, row0 + (size_t)c * kBC, nv, D);
#pragma unroll
                for (int e = 0; e < 4; ++e) buf_store_b16((bf16)dv[e], rg, ((4 * g + e) * D + jw0 + 16 * jb + c16) * 2);
            } else {
                const auto rs = rows_of(ws + L.dvp + (size_t)tile * T * D, (size_t)c * kBC, nv, D);
#pragma unroll
                for (int e = 0; e < 4; ++e) buf_store(dv[e], rs, ((4 * g + e) * D + jw0 + 16 * jb + c16) * 4);
            }
        }
        // eps_in = G_C (.) eps_out + A^T dO, both copies
        {
            const float gev = sm.ge[b][il];
#pragma unroll
            for (int jt = 0; jt < NJT; ++jt) eA[jt] = mma_xs(ld_col4(&sm.dO[b][4 * g][16 * jt + c16], D + 8), as, eA[jt] * gev);
        }
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            const SplitK16 ak = {MB::ld16(&sm.akh[b][16 * ib + c16][4 * g]), MB::ld16(&sm.akl[b][16 * ib + c16][4 * g])};
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
                eB[ib][jb] = mma_sx(ak, ld_col4(&sm.dO[b][4 * g][jw0 + 16 * jb + c16], D + 8), eB[ib][jb]);
        }
    };
    mma_load<D>(p, row0, nch - 1, nvalid(nch - 1), mt, mr);
    for (int it = 0; it < nch + 2; ++it) {
        if (it < nch) {
            const int c = nch - 1 - it;
            mma_stage<D>(mr, mt, sm.dO[c & 1], sm.vv[c & 1]);
            if (c >= 1) mma_load<D>(p, row0, c - 1, nvalid(c - 1), mt, mr);
        }
        if (it >= 1 && it <= nch) step(nch - it);
        lds_barrier();
    }
    if (p.geta0) {
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) *(f32x4*)&p.geta0[((size_t)bh * D + ig) * D + 16 * jt + 4 * g] = eA[jt];
    }
}

// dv and dr with two or more row tiles: the sums of the tiles' partials (in
// tile order).  One thread per (b,h, token, value quad).
template <int NT>
__global__ void kla_bwd_chunk_combine(BwdArgs p) {
    const int D = p.dv, VQ = D / 4;
    const size_t n = (size_t)p.B * p.H * p.T * VQ;
    const size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= n) return;
    const int jq = (int)(x % VQ);
    const size_t bt = x / VQ;
    const int t = (int)(bt % p.T);
    const size_t bh = bt / p.T;
    const BcLayout L = bc_layout(p.T, D);
    const float* ws = p.ws + bh * p.ws_stride;
    f32x4 s = *(const f32x4*)(ws + L.dvp + (size_t)t * D + 4 * jq);
#pragma unroll
    for (int tl = 1; tl < NT; ++tl) s += *(const f32x4*)(ws + L.dvp + ((size_t)tl * p.T + t) * D + 4 * jq);
    *(typename Quad<bf16>::V*)((bf16*)p.gv + bt * D + 4 * jq) = Quad<bf16>::make(s);
    if (jq == 0) {
        float r = ws[L.drp + t];
#pragma unroll
        for (int tl = 1; tl < NT; ++tl) r += ws[L.drp + (size_t)tl * L.t4 + t];
        p.gr[bt] = r;
    }
}

template <int D, bool ISO>
void launch(const BwdArgs& a, hipStream_t s) {
    constexpr int NT = D / 64;
    const int nbh = a.B * a.H;
    const dim3 grid((unsigned)(NT == 1 ? nbh : (nbh + 7) / 8 * 8 * NT));
    hipLaunchKernelGGL((kla_bwd_chunk_fwd<D, ISO>), grid, dim3(320), 0, s, a);
    hipLaunchKernelGGL((kla_bwd_chunk_rev<D, ISO>), grid, dim3(384), 0, s, a);
    if constexpr (NT > 1) {  // one row tile writes dv and dr itself
        const size_t n = (size_t)nbh * a.T * (D / 4);
        hipLaunchKernelGGL((kla_bwd_chunk_combine<NT>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    }
}

}  // namespace

bool bwd_chunk_supported(int dk, int dv, int cov, int dtype, int T) {
    const char* e = getenv("KLA_BWD_IMPL");
    if (e && (e[0] == 'r' || e[0] == 'p')) return false;  // KLA_BWD_IMPL=rows / plain
    if (dtype != DT_BF16 || dk != dv || T < 1) return false;
    // isotropic: the head's sums over key dims stay in one workgroup
    return cov ? dk == 64 : (dk == 64 || dk == 128);
}

hipError_t launch_bwd_chunk(const BwdArgs& a, int dtype, int cov, hipStream_t s) {
    if (!bwd_chunk_supported(a.dk, a.dv, cov, dtype, a.T) || a.B * a.H == 0) return hipErrorInvalidValue;
    BwdArgs b = a;
    const char* e = getenv("KLA_BWD_SPIN");
    if (e && *e) b.spin = atoi(e) < 0 ? 0 : atoi(e);
    if (cov) launch<64, true>(b, s);
    else if (a.dk == 64) launch<64, false>(b, s);
    else launch<128, false>(b, s);
    return hipGetLastError();
}

}  // namespace kla
