// kla_fwd_residual.hip -- gfx950 forward of the residual-write variant: the
// Kalman gain weights a write of the residual v - m_pred^T k (the delta-style
// write of "Kalman Delta Networks: Uncertainty-aware Associative Memory",
// abstract; diagonal and isotropic approximations).
//
// Recurrence per (b,h), state (l, m) with m the posterior mean (dk x dv):
//   lp = l / (a^2 + qn l),  m_pred = a (.) m               (row i scaled by a_i)
//   g  = P k / (k^T P k + r),  P = diag(1/lp)               (iso: P = I/lp)
//   m  = m_pred + g (v - m_pred^T k)^T,  l = lp + k^2/r     (iso: lp + |k|^2/(dk r))
//   o  = m^T q
// The precision is the Mobius map of the KLA forward; the mean write couples
// the key dims through the prediction m_pred^T k.
//
// Tokens go in blocks of n <= 4.  With G_t the product of the block's decays
// through token t and D(s,t) = a_{s+1} ... a_t (products only, no division),
// the block's residuals u_t and outputs follow from the state M0 at its start:
//   u_t = v_t - P_t - sum_{s<t} A[t][s] u_s,   P_t = (G_t k_t)^T M0
//   o_t = O_t + sum_{s<=t} C[t][s] u_s,         O_t = (G_t q_t)^T M0
//   M_end = G_end (.) M0 + sum_s (D(s,end) g_s) u_s^T
// with A[t][s] = sum_i D(s,t)_i k_t,i g_s,i and C[t][s] = sum_i D(s,t)_i q_t,i g_s,i.
// A and C (20 key-dim sums per four-token block, 72 per eight) depend on the inputs only, so they are
// formed for the next block while the current one runs.
//
// Two layouts of the state M, both in registers for the whole sequence:
// - thread rows (d 16 / 32, and d 128 with many (b,h)), as in the
//   short-sequence kernel: row group rg, value quad jq per thread, small
//   heads sharing a workgroup.  Per block: (1) every thread forms its rows'
//   partial predictions and readouts against M0; barrier; (4) partials are
//   summed over the row groups (and the next block's coefficients are
//   finished); barrier; (6) one thread per value quad solves the 4x4
//   unit-lower-triangular system for the residuals and writes the outputs;
//   barrier; (8) every thread updates its rows.
// - matrix cores (MM: d 64, and d 128 with few (b,h), 64-column tiles): each
//   wave keeps 16 columns as MFMA accumulator tiles; predictions, readouts
//   and the update are MFMA passes within the wave (see ResLayout), with two
//   barriers per block for the coefficient pipeline only.  Blocks hold eight
//   tokens at d 128 and four at d 64.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "kla_common.h"
#include "kla_residual.h"

namespace kla {
namespace {

constexpr int kResThreads = 256;
constexpr int kResTB = 4;                          // tokens per block (thread rows)
constexpr int kResTBM = 8;                         // tokens per block (matrix cores, d 128)
constexpr int kNP = kResTB * (kResTB + 1) / 2;     // token pairs s <= t (thread rows)
constexpr int kNS = 32;                            // 2*kNP sums, padded to a power of two
template <bool MM, int D> constexpr int res_tb() { return MM && D >= 128 ? kResTBM : kResTB; }
template <bool MM, int D> constexpr int res_np() { return res_tb<MM, D>() * (res_tb<MM, D>() + 1) / 2; }
__device__ __forceinline__ constexpr int pidx(int t, int s) { return t * (t + 1) / 2 + s; }

// An f32x4 as the K16 operand of Mma<T>: bf16 by a vector conversion (two
// values per instruction), split pairs for fp32.
template <typename T>
__device__ __forceinline__ typename Mma<T>::K16 k16(f32x4 x) {
    if constexpr (std::is_same<T, bf16>::value) {
        return __builtin_bit_cast(s16x4, __builtin_convertvector(x, bf16x4));
    } else {
        return Mma<T>::from_acc(x);
    }
}

// A (b,h) may be split by value columns into tiles of DVT columns: the
// residual write couples the key dims, not the value columns, so each tile
// runs on its own (the key-dim sums are formed in every tile).
//
// MM (d 64 / 128, 64-column tiles): the matrix-core layout.  Each of the four
// waves owns 16 value columns of the tile as D/16 accumulator tiles (lane l:
// key dims 16 rt + 4 (l/16) + e, column l%16), which is also the B operand
// of a 16-wide contraction over key dims.  The block's predictions and
// readouts are then one pass of MFMAs per wave, with the block's eight G_t k_t
// and eight G_t q_t stacked as the 16 rows of the A operand, and the state update is a
// second pass with the residuals as the B operand: nothing is summed across
// waves, and one barrier fewer is needed per block.
template <int D, int DVT, bool MM>
struct ResLayout {
    static constexpr int EPT = D == 16 ? 16 : 32;  // state elements per thread, at least
    static constexpr int NTH = MM ? kResThreads : D * DVT / EPT < kResThreads ? D * DVT / EPT : kResThreads;
    static constexpr int NH = kResThreads / NTH;   // (b,h, value tile) per workgroup
    static constexpr int VQ = DVT / 4;             // value quads per row of the tile
    static constexpr int RG = MM ? 1 : NTH / VQ;   // row groups of a (b,h)
    static constexpr int RPT = MM ? 4 : D / RG;    // rows per thread
    static constexpr int KW = D < 64 ? D : 64;     // key-dim lanes per wave
    static_assert(RPT % 4 == 0 && res_tb<MM, D>() * VQ <= NTH && NTH * NH == kResThreads && NTH % D == 0 &&
                      (KW == 16 || KW == 32 || KW == 64) && (!MM || (DVT == 64 && D >= 64)),
                  "layout");
};

// Coefficient buffers alternate by block parity: block b+1's are written
// after the first barrier of block b, when every thread has finished block
// b-1's state update, the last reader of that buffer.
template <int D, int DVT, bool MM>
struct ResSm {
    static constexpr int NH = ResLayout<D, DVT, MM>::NH, NTH = ResLayout<D, DVT, MM>::NTH;
    static constexpr int X = MM ? 1 : 0;  // arrays only the thread-row layout uses shrink to one entry
    static constexpr int TB = res_tb<MM, D>();
    alignas(16) float kt[2][NH][TB][D];   // G_t k_t
    alignas(16) float qt[2][NH][TB][D];   // G_t q_t
    alignas(16) float e[2][NH][MM ? D : TB][MM ? TB : D];  // D(s,end) g_s ([i][s] for MM)
    alignas(16) float gn[2][NH][D];           // G_end
    alignas(16) float v[2][NH][TB][DVT];
    alignas(16) float A[2][NH][TB][TB];  // [t][s], s < t
    alignas(16) float C[2][NH][TB][TB];  // [t][s], s <= t
    alignas(16) f32x4 part[2][NH][X ? 1 : kResTB][X ? 1 : NTH];  // prediction / readout partials
    alignas(16) float pr[2][NH][X ? 1 : kResTB][X ? 4 : DVT];  // their sums over the row groups
    alignas(16) float u[NH][X ? 1 : kResTB][X ? 4 : DVT];      // residuals
    // the key-dim sums of each reduction unit: thread rows, 2*kNP (padded to
    // kNS) per group's key-dim lanes or, at d 128, per wave; matrix cores,
    // one set of NP sums per wave
    float sums[kResThreads / 16][MM ? 40 : kNS];
};

template <typename TIn, int D, int DVT, bool ISO, bool MM>
__global__ __launch_bounds__(kResThreads) void kla_fwd_residual_kernel(FwdArgs p) {
    typedef ResLayout<D, DVT, MM> Ly;
    constexpr int NVT = D / DVT;
    constexpr int TB = res_tb<MM, D>(), NTH = Ly::NTH, NH = Ly::NH, VQ = Ly::VQ, RG = Ly::RG, RPT = Ly::RPT;
    constexpr int NP = res_np<MM, D>();  // token pairs s <= t of a block
    constexpr int KW = Ly::KW;
    constexpr bool RED = D > 64;  // key dims of a head span two waves
    typedef typename Quad<TIn>::V QV;
    __shared__ ResSm<D, DVT, MM> sm;
    typedef Mma<TIn> MA;  // bf16 operands, or split bf16 pairs for fp32 inputs

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = NH == 1 ? 0 : tid / NTH, lt = NH == 1 ? tid : tid % NTH;
    // Value tiles of one (b,h) run 8 workgroups apart, on the same XCD
    // (workgroups go round-robin over the 8 XCDs), so the second tile's reads
    // of k, q, a and r hit that XCD's L2.
    const int x8 = (int)blockIdx.x;
    const int vt = NVT == 1 ? 0 : (x8 / 8) % NVT;
    const int hb = NVT == 1 ? x8 : (x8 / (8 * NVT)) * 8 + x8 % 8;
    const int nbh = p.B * p.H;
    if (NVT > 1 && hb >= (nbh + NH - 1) / NH) return;  // padding of the grid to the XCD pattern
    const int bh_ = NH == 1 ? hb : hb * NH + grp;
    const bool valid = NH == 1 || bh_ < nbh;
    const int bh = valid ? bh_ : nbh - 1;  // a spare group loads in bounds and stores nothing
    const int h = bh % p.H;
    const int col0 = vt * DVT;  // first value column of the tile
    const int jq = lt % VQ, rg = lt / VQ, i0 = rg * RPT;
    const bool kd = lt < D;  // key-dim lane
    // MM: every lane holds a key dim (lane lt: dim lt % D); waves 0 .. D/64-1
    // form the key sums of the coefficient step and the next D/64 waves the
    // query sums, so each set reduces half of the values
    const int kdim = MM ? lt % D : kd ? lt : D - 1;
    constexpr int NKW = D / 64 > 0 ? D / 64 : 1;  // MM: waves per key-dim set
    const int role = MM ? wave / NKW : 0;          // MM: 0 key sums, 1 query sums, 2+ none
    // MM: waves 3 and 0 stage the v rows, wave 3 writes A and C (waves 0-1
    // write the per-key-dim coefficients); vlt is the lane's index for the v rows
    const int vlt = MM ? (lt + 64) % NTH : lt;
    const size_t row0 = (size_t)bh * p.T;
    const TIn* q = (const TIn*)p.q;
    const TIn* k = (const TIn*)p.k;
    const TIn* v = (const TIn*)p.v;
    TIn* o = (TIn*)p.o;

    // the thread's slice of the mean state: RPT rows of one value quad, or
    // (MM) D/16 accumulator tiles of the wave's 16 columns
    constexpr int NM = MM ? D / 16 : RPT;
    const int wcol = col0 + 16 * wave + (lane & 15);  // MM: the lane's value column
    f32x4 M[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        if constexpr (MM) {
#pragma unroll
            for (int x4 = 0; x4 < 4; ++x4)
                M[m][x4] = p.eta0 ? p.eta0[((size_t)bh * D + 16 * m + 4 * (lane >> 4) + x4) * D + wcol] : 0.f;
        } else {
            const size_t off = ((size_t)bh * D + i0 + m) * D + col0 + 4 * jq;
            M[m] = p.eta0 ? *(const f32x4*)(p.eta0 + off) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    float l;  // precision of key dim kdim (diag) or of the head (iso)
    if constexpr (!ISO) l = p.l0 ? p.l0[(size_t)bh * D + kdim] : 1.f;
    else l = p.l0 ? p.l0[bh] : 1.f;
    const float qn_i = !ISO ? p.qn[(size_t)h * D + kdim] : 0.f;

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
        const int uv = vlt / VQ < nb ? vlt / VQ : nb - 1;
        x.vq = *(const QV*)(v + (row0 + t0 + uv) * D + col0 + 4 * (vlt % VQ));
    };
    auto settle = [&](Raw& x) {
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            asm volatile("" : "+v"(x.k[u]), "+v"(x.q[u]), "+v"(x.a[u]), "+v"(x.r[u]));
            if constexpr (ISO) asm volatile("" : "+v"(x.qn[u]));
        }
        asm volatile("" : "+v"(x.vq));
    };

    // ---- a block's coefficients, in two steps around a barrier
    // Pre: per key-dim lane, the block's gains up to their common divisor and
    // the NP key and NP query sums (diag: k_t.D(s,t).k_s/lp_s and q_t.D(s,t).k_s/lp_s;
    // iso: k_t.k_s and q_t.k_s), reduced over the wave's key-dim lanes.
    struct Pre {
        float kf[TB], qf[TB], c[TB], cum[TB];  // k, q, k/lp (diag), G_t (diag)
        float lp[TB];                           // diag: predicted precision
        float sum[2 * NP];                      // [0,NP): k-sums, [NP,2NP): q-sums
    };
    auto pre = [&](const Raw& x, int nb, Pre& P) {
        float dec[TB];
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            const bool on = u < nb && (MM || kd);
            P.kf[u] = on ? (float)x.k[u] : 0.f;
            P.qf[u] = on ? (float)x.q[u] : 0.f;
            dec[u] = u < nb ? x.a[u] : 1.f;
        }
        if constexpr (!ISO) {
            float g = 1.f;
#pragma unroll
            for (int u = 0; u < TB; ++u) {
                const float rd = fast_rcp(__builtin_fmaf(qn_i, l, dec[u] * dec[u]));
                const float lp = l * rd;
                P.lp[u] = lp;
                P.c[u] = P.kf[u] * fast_rcp(lp);
                g *= dec[u];
                P.cum[u] = g;
                if (u < nb) l = __builtin_fmaf(P.kf[u] * P.kf[u], fast_rcp(x.r[u]), lp);
            }
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                float dst = 1.f;  // D(s,t) for s = t, t-1, ...
#pragma unroll
                for (int s = t; s >= 0; --s) {
                    if (s < t) dst *= dec[s + 1];
                    P.sum[pidx(t, s)] = dst * P.kf[t] * P.c[s];
                    P.sum[NP + pidx(t, s)] = dst * P.qf[t] * P.c[s];
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < TB; ++t)
#pragma unroll
                for (int s = 0; s <= t; ++s) {
                    P.sum[pidx(t, s)] = P.kf[t] * P.kf[s];
                    P.sum[NP + pidx(t, s)] = P.qf[t] * P.kf[s];
                }
        }
        // Reduce-scatter over the KW key-dim lanes: at each exchange a lane
        // keeps one half of its values (chosen by its lane bit), sends the
        // other half to its partner and adds the partner's copy of the kept
        // half.  After log2(kNS) halvings each lane holds one value summed
        // over 32 lanes (two values over 16 at KW = 16); a last full exchange
        // completes KW = 64.  The owners write the sums to LDS.
        if constexpr (MM) {
            // the wave's set of NP sums: up to 16 padded to 16 (one value per
            // 4 lanes); 36 as 32 (one per 2 lanes) and 4 (one per 16 lanes)
            constexpr int NV = NP <= 16 ? 16 : 32;
            constexpr int NR = NP <= 16 ? 0 : 4;
            static_assert(NP <= NV + NR, "sums per set");
            float w[NV];
#pragma unroll
            for (int j = 0; j < NV; ++j) w[j] = j < NP ? (role == 0 ? P.sum[j] : P.sum[NP + j]) : 0.f;
            int base = 0;
            reduce_scatter<NV, 32>(w, lane, base);
            if (role <= 1 && (lane & (64 / NV - 1)) == 0) sm.sums[wave][base] = w[0];
            if constexpr (NR > 0) {
                float w2[NR];
#pragma unroll
                for (int j = 0; j < NR; ++j)
                    w2[j] = NV + j < NP ? (role == 0 ? P.sum[NV + j] : P.sum[NP + NV + j]) : 0.f;
                int b2 = 0;
                reduce_scatter<NR, 32>(w2, lane, b2);
                if (role <= 1 && (lane & (64 / NR - 1)) == 0) sm.sums[wave][NV + b2] = w2[0];
            }
        } else {
            float w[kNS];
#pragma unroll
            for (int j = 0; j < kNS; ++j) w[j] = j < 2 * kNP ? P.sum[j] : 0.f;
            int base = 0;
            reduce_scatter<kNS, KW / 2>(w, lane, base);
            // owners: lane holds values base .. base+NOUT-1 of its unit
            constexpr int NOUT = kNS / KW > 0 ? kNS / KW : 1;
            const int unit = RED ? wave : grp;
            const bool owner = kd && (KW < 64 || (lane & 1) == 0);
            if (owner) {
#pragma unroll
                for (int j = 0; j < NOUT; ++j) sm.sums[unit][base + j] = w[j];
            }
        }
    };
    // Finish (after a barrier): the whole-head sums, the gains' divisors and
    // the coefficients of buffer c.
    auto finish = [&](const Raw& x, int nb, Pre& P, int c) {
        if constexpr (MM) {
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                float sk = 0.f, sq = 0.f;
#pragma unroll
                for (int w = 0; w < NKW; ++w) {
                    sk += sm.sums[w][j];
                    sq += sm.sums[NKW + w][j];
                }
                P.sum[j] = sk;
                P.sum[NP + j] = sq;
            }
        } else if constexpr (RED) {
            // the head's key dims are the group's first two waves
            const int w0 = grp * (NTH / 64);
#pragma unroll
            for (int j = 0; j < 2 * kNP; ++j) P.sum[j] = sm.sums[w0][j] + sm.sums[w0 + 1][j];
        } else {
#pragma unroll
            for (int j = 0; j < 2 * kNP; ++j) P.sum[j] = sm.sums[grp][j];
        }
        float dec[TB], inv[TB], cum[TB];
        float scale[TB];  // iso: 1 / lp_s (the gain is k_s / (lp_s (s_s + r_s)))
#pragma unroll
        for (int u = 0; u < TB; ++u) dec[u] = u < nb ? x.a[u] : 1.f;
        if constexpr (!ISO) {
#pragma unroll
            for (int u = 0; u < TB; ++u) {
                inv[u] = fast_rcp(P.sum[pidx(u, u)] + x.r[u]);
                scale[u] = 1.f;
                cum[u] = P.cum[u];
            }
        } else {
            float g = 1.f;
#pragma unroll
            for (int u = 0; u < TB; ++u) {
                const float ksq = P.sum[pidx(u, u)];
                const float rd = fast_rcp(__builtin_fmaf(x.qn[u], l, dec[u] * dec[u]));
                const float lp = l * rd, rlp = fast_rcp(lp);
                inv[u] = fast_rcp(__builtin_fmaf(ksq, rlp, x.r[u]));
                scale[u] = rlp;
                if (u < nb) l = __builtin_fmaf(ksq * (1.f / (float)D), fast_rcp(x.r[u]), lp);
                g *= dec[u];
                cum[u] = g;
            }
        }
        float gend = 1.f;  // G at the block's last token
#pragma unroll
        for (int u = 0; u < TB; ++u)
            if (u == nb - 1) gend = cum[u];
        if (kd) {
#pragma unroll
            for (int u = 0; u < TB; ++u) {
                // D(u, end) g_u: decays after token u through the block's end
                float after = 1.f;
#pragma unroll
                for (int w = u + 1; w < TB; ++w)
                    if (w < nb) after *= dec[w];
                const float gu = (ISO ? P.kf[u] * scale[u] : P.c[u]) * inv[u];
                if constexpr (MM) sm.e[c][grp][lt][u] = after * gu;
                else sm.e[c][grp][u][lt] = after * gu;
                sm.kt[c][grp][u][lt] = cum[u] * P.kf[u];
                sm.qt[c][grp][u][lt] = cum[u] * P.qf[u];
            }
            sm.gn[c][grp][lt] = gend;
        }
        if (lt == (MM ? NTH - 1 : 0)) {
            static_assert(TB % 4 == 0, "rows of A and C are written as f32x4 pieces");
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                float ar[TB], cr[TB];
                float dst = 1.f;
#pragma unroll
                for (int s = TB - 1; s >= 0; --s) {
                    if (s > t) {
                        ar[s] = 0.f;
                        cr[s] = 0.f;
                        continue;
                    }
                    if (s < t) dst *= dec[s + 1];
                    const float w = (ISO ? dst * scale[s] : 1.f) * inv[s];
                    ar[s] = s < t ? w * P.sum[pidx(t, s)] : 0.f;
                    cr[s] = w * P.sum[NP + pidx(t, s)];
                }
#pragma unroll
                for (int s4 = 0; s4 < TB; s4 += 4) {
                    *(f32x4*)&sm.A[c][grp][t][s4] = f32x4{ar[s4], ar[s4 + 1], ar[s4 + 2], ar[s4 + 3]};
                    *(f32x4*)&sm.C[c][grp][t][s4] = f32x4{cr[s4], cr[s4 + 1], cr[s4 + 2], cr[s4 + 3]};
                }
            }
        }
        if (vlt / VQ < nb) *(f32x4*)&sm.v[c][grp][vlt / VQ][4 * (vlt % VQ)] = Quad<TIn>::to_f32(x.vq);
    };

    {
        Raw x;
        load(0, x);
        settle(x);
        Pre P;
        const int nb0 = p.T < TB ? p.T : TB;
        pre(x, nb0, P);
        lds_barrier();
        finish(x, nb0, P, 0);
        lds_barrier();
    }
    int c = 0;
    for (int t0 = 0; t0 < p.T; t0 += TB, c ^= 1) {
        const int nb = p.T - t0 < TB ? p.T - t0 : TB;
        const bool more = t0 + TB < p.T;
        const int nbn = more ? (p.T - t0 - TB < TB ? p.T - t0 - TB : TB) : 0;
        Raw x;
        load(more ? t0 + TB : t0, x);
        if constexpr (MM) {
            // (1) predictions (slots 0 .. TB-1: G_t k_t) and readouts (slots
            // TB .. 2TB-1: G_t q_t) of the block's tokens against M0, over the
            // key-dim tiles
            const int slot = lane & 15, kq = lane >> 4;
            const float* arow = slot < TB ? &sm.kt[c][0][slot][0] : &sm.qt[c][0][(slot - TB) & (TB - 1)][0];
            f32x4 po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int rt = 0; rt < D / 16; ++rt) {
                // read by every lane (no branch, so the reads run ahead), zero in unused slots
                f32x4 av = *(const f32x4*)(arow + 16 * rt + 4 * kq);
                if (slot >= 2 * TB) av = f32x4{0.f, 0.f, 0.f, 0.f};
                po = MA::mma16(k16<TIn>(av), k16<TIn>(M[rt]), po);
            }
            // (2) residuals and outputs: lane j < 16 of the wave solves column
            // 16 wave + j; row r of the product sits in lane j + 16 (r/4),
            // element r%4
            float pt[TB], o0[TB];
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                pt[t] = t < 4 ? po[t] : __shfl(po[t % 4], lane + 16 * (t / 4), 64);
                o0[t] = __shfl(po[(TB + t) % 4], lane + 16 * ((TB + t) / 4), 64);
            }
            float uv[TB];
#pragma unroll
            for (int t = 0; t < TB; ++t) uv[t] = 0.f;
            if (lane < 16) {
#pragma unroll
                for (int t = 0; t < TB; ++t) {
                    if (t < nb) {
                        float ut = sm.v[c][0][t][16 * wave + lane] - pt[t];
#pragma unroll
                        for (int s2 = 0; s2 < t; ++s2) ut -= sm.A[c][0][t][s2] * uv[s2];
                        uv[t] = ut;
                        float ot = o0[t];
#pragma unroll
                        for (int s2 = 0; s2 <= t; ++s2) ot += sm.C[c][0][t][s2] * uv[s2];
                        if (valid) o[(row0 + t0 + t) * D + wcol] = (TIn)ot;
                    }
                }
            }
            // (3) the state at the block's end: M = G_end (.) M + E U, with E
            // (key dims x tokens) the A operand and the residuals the B
            // operand (tokens 4 kq .. 4 kq + 3 in lanes 16 kq .. 16 kq + 15)
            f32x4 uq = {uv[0], uv[1], uv[2], uv[3]};
            if constexpr (TB == 8) {
                f32x4 hi;
#pragma unroll
                for (int e = 0; e < 4; ++e) hi[e] = __shfl(uv[4 + e], (lane + 48) & 63, 64);
                if (lane >= 16) uq = hi;
                if (lane >= 32) uq = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            const auto ub = k16<TIn>(uq);
#pragma unroll
            for (int rt = 0; rt < D / 16; ++rt) {
                const f32x4 gv = *(const f32x4*)&sm.gn[c][0][16 * rt + 4 * kq];
                M[rt] *= gv;
                f32x4 ev = *(const f32x4*)&sm.e[c][0][16 * rt + slot][4 * (kq & (TB / 4 - 1))];
                if (kq >= TB / 4) ev = f32x4{0.f, 0.f, 0.f, 0.f};
                M[rt] = MA::mma16(k16<TIn>(ev), ub, M[rt]);
            }
            // (4) the next block's coefficients
            settle(x);
            Pre P;
            if (more) pre(x, nbn, P);
            lds_barrier();
            if (more) finish(x, nbn, P, c ^ 1);
            lds_barrier();
        } else {
            // (1) partial predictions and readouts of the block's tokens against M0
    #pragma unroll
            for (int u = 0; u < TB; ++u) {
                if (u < nb) {
                    f32x4 ap = {0.f, 0.f, 0.f, 0.f}, ao = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                    for (int m4 = 0; m4 < RPT; m4 += 4) {
                        const f32x4 kv = *(const f32x4*)&sm.kt[c][grp][u][i0 + m4];
                        const f32x4 qv = *(const f32x4*)&sm.qt[c][grp][u][i0 + m4];
    #pragma unroll
                        for (int x4 = 0; x4 < 4; ++x4) {
                            ap += kv[x4] * M[m4 + x4];
                            ao += qv[x4] * M[m4 + x4];
                        }
                    }
                    sm.part[0][grp][u][lt] = ap;
                    sm.part[1][grp][u][lt] = ao;
                }
            }
            // (2) the next block's key-dim sums
            settle(x);
            Pre P;
            if (more) pre(x, nbn, P);
            lds_barrier();
            // (4) sums over the row groups; the next block's coefficients
            for (int w = lt; w < 2 * nb * VQ; w += NTH) {
                const int kind = w / (nb * VQ), rem = w % (nb * VQ), u = rem / VQ, j4 = rem % VQ;
                f32x4 s = sm.part[kind][grp][u][j4];
    #pragma unroll
                for (int r2 = 1; r2 < RG; ++r2) s += sm.part[kind][grp][u][r2 * VQ + j4];
                *(f32x4*)&sm.pr[kind][grp][u][4 * j4] = s;
            }
            if (more) finish(x, nbn, P, c ^ 1);
            lds_barrier();
            // (6) residuals and outputs, one thread per value quad
            if (lt < VQ) {
                f32x4 us[TB];
    #pragma unroll
                for (int t = 0; t < TB; ++t) {
                    if (t < nb) {
                        f32x4 ut = *(const f32x4*)&sm.v[c][grp][t][4 * lt] - *(const f32x4*)&sm.pr[0][grp][t][4 * lt];
    #pragma unroll
                        for (int s = 0; s < t; ++s) ut -= sm.A[c][grp][t][s] * us[s];
                        us[t] = ut;
                        f32x4 ot = *(const f32x4*)&sm.pr[1][grp][t][4 * lt];
    #pragma unroll
                        for (int s = 0; s <= t; ++s) ot += sm.C[c][grp][t][s] * us[s];
                        *(f32x4*)&sm.u[grp][t][4 * lt] = ut;
                        if (valid) *(QV*)(o + (row0 + t0 + t) * D + col0 + 4 * lt) = Quad<TIn>::make(ot);
                    }
                }
            }
            lds_barrier();
            // (8) the state at the block's end
    #pragma unroll
            for (int m4 = 0; m4 < RPT; m4 += 4) {
                const f32x4 gv = *(const f32x4*)&sm.gn[c][grp][i0 + m4];
    #pragma unroll
                for (int x4 = 0; x4 < 4; ++x4) M[m4 + x4] *= gv[x4];
            }
    #pragma unroll
            for (int u = 0; u < TB; ++u) {
                if (u < nb) {
                    const f32x4 uu = *(const f32x4*)&sm.u[grp][u][4 * jq];
    #pragma unroll
                    for (int m4 = 0; m4 < RPT; m4 += 4) {
                        const f32x4 ev = *(const f32x4*)&sm.e[c][grp][u][i0 + m4];
    #pragma unroll
                        for (int x4 = 0; x4 < 4; ++x4) M[m4 + x4] += ev[x4] * uu;
                    }
                }
            }
        }
    }
    if (!valid) return;
    if (p.etaT) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if constexpr (MM) {
#pragma unroll
                for (int x4 = 0; x4 < 4; ++x4)
                    p.etaT[((size_t)bh * D + 16 * m + 4 * (lane >> 4) + x4) * D + wcol] = M[m][x4];
            } else {
                *(f32x4*)(p.etaT + ((size_t)bh * D + i0 + m) * D + col0 + 4 * jq) = M[m];
            }
        }
    }
    if (p.lT && vt == 0) {
        if constexpr (!ISO) {
            if (kd) p.lT[(size_t)bh * D + lt] = l;
        } else if (lt == 0) {
            p.lT[bh] = l;
        }
    }
}

template <typename TIn, int D, int DVT, bool ISO, bool MM = false>
void launch(const FwdArgs& a, hipStream_t s) {
    typedef ResLayout<D, DVT, MM> Ly;
    const int nbh = a.B * a.H, ngroups = (nbh + Ly::NH - 1) / Ly::NH;
    constexpr int NVT = D / DVT;
    const dim3 grid((unsigned)(NVT == 1 ? ngroups : (ngroups + 7) / 8 * 8 * NVT));
    hipLaunchKernelGGL((kla_fwd_residual_kernel<TIn, D, DVT, ISO, MM>), grid, dim3(kResThreads), 0, s, a);
}

// KLA_RES_MM=0 keeps 64-column tiles on the thread-row layout.
bool res_mm() {
    const char* env = getenv("KLA_RES_MM");
    return !(env && env[0] == '0');
}

template <typename TIn, bool ISO>
hipError_t dispatch(const FwdArgs& a, hipStream_t s) {
    const int nvt = a.n_vtiles;
    const bool mm = res_mm();  // matrix-core layout for 64-column tiles
    switch (a.dk) {
        case 16: launch<TIn, 16, 16, ISO>(a, s); break;
        case 32: launch<TIn, 32, 32, ISO>(a, s); break;
        case 64:
            if (nvt == 2) launch<TIn, 64, 32, ISO>(a, s);
            else if (mm) launch<TIn, 64, 64, ISO, true>(a, s);
            else launch<TIn, 64, 64, ISO>(a, s);
            break;
        case 128:
            if (nvt == 2 && mm) launch<TIn, 128, 64, ISO, true>(a, s);
            else if (nvt == 2) launch<TIn, 128, 64, ISO>(a, s);
            else launch<TIn, 128, 128, ISO>(a, s);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool fwd_residual_supported(int dk, int dv) {
    return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}

int fwd_residual_vtiles(int B, int H, int dk) {
    // two value tiles for d 64 / 128 while there are fewer (b,h) than about
    // two workgroups per CU
    const long long nbh = (long long)B * H;
    // 64-column tiles on the matrix cores: the whole head at d 64; two tiles
    // at d 128 while there are fewer (b,h) than about two workgroups per CU
    // (beyond that the second tile's repeated key-dim sums cost more than
    // the matrix cores save)
    if (res_mm()) return dk == 128 ? (nbh < 512 ? 2 : 1) : 1;
    return dk >= 64 && nbh < 512 ? 2 : 1;
}

hipError_t launch_fwd_residual(const FwdArgs& a, int dtype, int cov, hipStream_t s) {
    if (!fwd_residual_supported(a.dk, a.dv) || a.T < 1) return hipErrorInvalidValue;
    if (fwd_residual_chunk_supported(a.dk, a.dv, cov, dtype)) return launch_fwd_residual_chunk(a, dtype, cov, s);
    if (a.n_vtiles != 1 && !(a.n_vtiles == 2 && a.dk >= 64)) return hipErrorInvalidValue;
    if (dtype == DT_BF16) return cov ? dispatch<bf16, true>(a, s) : dispatch<bf16, false>(a, s);
    return cov ? dispatch<float, true>(a, s) : dispatch<float, false>(a, s);
}

}  // namespace kla
