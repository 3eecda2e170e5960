// kla_fwd_diag_pipe.hip -- gfx950 forward kernel, diagonal precision,
// three-role software pipeline (key dims 64 and 128).
//
// Sources: "Kalman Linear Attention: Parallel Bayesian Filtering For Efficient
// Language Modelling and State Tracking" (gist.science explainer, method §1-§3)
// and "Kalman Delta Networks: Uncertainty-aware Associative Memory" (abstract,
// diagonal variant).  Per (b,h) and key dim i:
//   lp = l/(a^2 + qn l),  l' = lp + k^2/r                          (precision)
//   m_t = f_t (.) m_{t-1} + w_t v_t^T,  f = a lp / l',  w = k/(r l')  (mean)
//   o_t = q_t^T m_t
// (the information-form update divided by l'; every gate f lies in (0, 1]).
//
// One workgroup owns one (b,h) and DV value columns and walks the sequence in
// 32-token chunks.  Its waves have three roles that work on three different
// chunks at once and meet at ONE workgroup barrier per chunk:
//   chain waves  (one lane per key dim) run the sequential precision recursion
//                of chunk c+2: four dependent VALU ops per token.  They write
//                (a*lp, l) to LDS and flag the chunk if some cumulative gate
//                product inside it drops below 2^-64.  A second chain role
//                (chain_role_scan, selected at launch) computes the same
//                chunk as a wavefront-level Mobius scan over lanes that own
//                4 key dims x 8 tokens;
//   gate waves   turn chunk c+1's precisions into gates f, w and cumulative
//                products G (lanes own 2 key dims x 8 tokens at dk 128, x 4
//                at dk 64; the products cross token groups with DPP row
//                shifts), and write the MFMA operands q^ = q G, w^ = w / G
//                (or, for a flagged chunk, the raw fp32 gates).  They request
//                the next chunk's rows after their work, the chain waves at
//                the start of theirs;
//   MMA waves    own the fp32 state m (accumulator registers) and run chunk
//                c: causal S^T = W^ Q^^T tiles, O^T = m^T Q^^T + V^T P^T,
//                m += W^^T V.  All products use 16x16x32 MFMAs: the K index of
//                an operand fragment is permuted so that two stacked 16x16
//                accumulator tiles form one K=32 operand without LDS.
//                A flagged chunk is applied token by token (exact, slower).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kla_common.h"
#include "kla_internal.h"

namespace kla {
namespace {

constexpr float kFloor = 5.421010862427522e-20f;  // 2^-64

template <typename TIn, int DK_, int DV_>
struct P3 {
    static constexpr int DK = DK_;
    static constexpr int DV = DV_;
    static constexpr int C = 32;                 // tokens per chunk
    static constexpr int NCW = DK / 64;          // chain waves
    static constexpr int NMW = DV / 32;          // MMA waves
    static constexpr int JT = 2;                 // 16-column value tiles per MMA wave
    // The gates of a chunk are cut into four groups of key-dim pairs (virtual
    // gate waves).  With 64 value columns four gate waves take one group
    // each; with 128 the four MMA waves leave room for two, which take two
    // groups each, one after the other.
    static constexpr int NGW = DV == 128 ? 2 : 4;  // gate waves
    static constexpr int NVG = 4 / NGW;            // groups per gate wave
    static constexpr int NW = NCW + NMW + NGW;
    static constexpr int NT = 64 * NW;
    static constexpr int IT = DK / 16;           // 16-row tiles of the state
    static constexpr int KB = DK / 32;           // K=32 blocks over the key dim
    static constexpr int NIP = DK / 2;           // key-dim pairs
    static constexpr int NGRP = 256 / NIP;       // token groups
    static constexpr int TPG = C / NGRP;         // tokens per group
    static constexpr int IPW = 64 / NGRP;        // key-dim pairs per group
    static constexpr int PE = 16 / (int)sizeof(TIn);
    static constexpr int QS = DK + PE;           // row stride of Q^, W^
    static constexpr int CS = C + PE;            // row stride of W^T, V^T
    static constexpr int LPS = DK + 2;           // row stride of the chain buffer
    static constexpr int VQ = DV / 4;
    static constexpr int VUNITS = (C / 2) * VQ;
    static constexpr int VPT = VUNITS / 256;
    // chain and gate waves keep NBC / NBG chunks of inputs in registers and
    // load NBC-1 / NBG-1 chunks ahead; every role runs a multiple of UNR
    // pipeline steps
    static constexpr int NBC = 2;
    static constexpr int NBG = 2;
    static constexpr int UNR = NBC * NBG / (NBC == NBG ? NBC : 1);
    static_assert(DK == 64 || DK == 128, "key dims 64 and 128");
    static_assert(DV % 32 == 0 && VUNITS % 256 == 0, "value tiles");
};

template <typename TIn, class K>
struct OpFac {
    TIn Q[K::C][K::QS];
    TIn W[K::C][K::QS];
    TIn WT[K::DK][K::CS];
};
template <class K>
struct OpRaw {
    float f[K::C][K::DK];
    float w[K::C][K::DK];
};

template <typename TIn, class K>
struct S3 {
    f32x2 LP[2][K::C][K::LPS];   // (a*lp, l) by chunk parity
    union {
        OpFac<TIn, K> fac;
        OpRaw<K> raw;
    } op[2];                      // MFMA operands (or raw gates) by chunk parity
    TIn VT[2][K::DV][K::CS];      // v^T by chunk parity
    alignas(16) float rho[2][K::C];  // 1/r_t by chunk parity
    alignas(16) float sc[2][K::DK];  // state scale before the chunk's readout
    alignas(16) float E[2][K::DK];   // end-of-chunk gate product (pending state scale)
    float lT[K::DK];
    alignas(16) float Wc[2][K::DK];  // sequence split: gate product from the segment
                                     // start through token 0 of the chunk
    alignas(16) float WcM[2][K::DK];  // the same, handed by the gate waves to the
                                      // MMA waves (with the block prologue, bf16:
                                      // they store q-hat)
    int bad[4];                   // chunk needs the exact token-by-token path
};

// Block prologue: convolution taps (right-aligned into four) and biases of
// q (all key dims) and v (the workgroup's value columns), for the gate waves.
template <class K>
struct PTaps {
    f32x4 qw[K::DK], vw[K::DV];
    float qb[K::DK], vb[K::DV];
};
struct NoTaps {};

// LDS layouts are permuted so that the lanes of one gate-wave access spread
// over the banks, while every 8/16-byte operand group stays contiguous and
// the MFMA waves' addresses stay loop-invariant:
//   LP row t:     (a*lp, l) of key dim i at column i ^ lp_swz(t)
//   Q^, W^:       token t at row qw_row<K>(t) (swaps 4-row or 2-row blocks
//                 in the second half of the chunk)
//   V^T row j:    4-token group c of the chunk at group c ^ vt_swz<K>(j),
//                 uniform over the 16 rows of an MFMA tile
__device__ __forceinline__ int lp_swz(int t) { return ((t >> 3) & 3) << 3; }
template <class K>
__device__ __forceinline__ int qw_row(int t) { return t ^ (((t >> 4) & 1) << (K::DK == 128 ? 2 : 1)); }
template <class K>
__device__ __forceinline__ int vt_swz(int j) { return (((j >> 4) * (128 / K::DV)) & 7) << 2; }

template <int N>
__device__ __forceinline__ float dpp_row_shr(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, false));
}

// Exclusive product over the NGRP consecutive lanes (token groups) of a key-dim pair.
template <class K>
__device__ __forceinline__ float group_excl_prod(float x, int grp) {
    float y = dpp_row_shr<1>(x);
    if (grp >= 1) x *= y;
    y = dpp_row_shr<2>(x);
    if (grp >= 2) x *= y;
    if constexpr (K::NGRP > 4) {
        y = dpp_row_shr<4>(x);
        if (grp >= 4) x *= y;
    }
    y = dpp_row_shr<1>(x);
    return grp == 0 ? 1.f : y;
}

template <typename T, int N>
__device__ __forceinline__ void store_row(T* dst, const T (&v)[N]) {
    constexpr int PER = 16 / (int)sizeof(T);
    if constexpr (N % PER == 0) {
#pragma unroll
        for (int b = 0; b < N / PER; ++b) {
            T tmp[PER];
#pragma unroll
            for (int e = 0; e < PER; ++e) tmp[e] = v[b * PER + e];
            *(f32x4*)(dst + b * PER) = __builtin_bit_cast(f32x4, tmp);
        }
    } else {
        constexpr int P8 = 8 / (int)sizeof(T);
        static_assert(N % P8 == 0, "row store");
#pragma unroll
        for (int b = 0; b < N / P8; ++b) {
            T tmp[P8];
#pragma unroll
            for (int e = 0; e < P8; ++e) tmp[e] = v[b * P8 + e];
            *(f32x2*)(dst + b * P8) = __builtin_bit_cast(f32x2, tmp);
        }
    }
}

// Wait until at most N vector-memory operations of this wave are in flight
// (expcnt and lgkmcnt left at their maxima; the counter holds at most 63).
// Called at the top of a pipeline step, before the step issues its loads, with
// N = the loads of the one chunk issued after the current chunk's: the current
// chunk's registers then need no further waits, however many loads follow.
template <int N>
__device__ __forceinline__ void wait_loads() {
    constexpr int n = N < 63 ? N : 63;
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Pipeline steps of every role: nchunks + 2, rounded up to a multiple of UNR.
template <class K>
__device__ __forceinline__ int pipe_steps(int nchunks) {
    return (nchunks + 2 + K::UNR - 1) / K::UNR * K::UNR;
}

__device__ __forceinline__ int chunk_len(int T, int c, int C) {
    const int n = T - c * C;
    return n < C ? n : C;
}

// Token span of one workgroup: the whole sequence, or one segment of it.
struct Span {
    int seg;   // segment index (0 without a split)
    int T0;    // first token
    int TL;    // tokens
    bool last; // last segment of the (b,h)
};

// ------------------------------------------------------------------ chain role
template <typename TIn, class K, bool SEG, bool PRO>
__device__ void chain_role(S3<TIn, K>& sm, const FwdArgs& p, const Span& sp, int bh, int vt, int cw,
                           int lane) {
    constexpr int C = K::C, DK = K::DK;
    const int i = cw * 64 + lane;
    const size_t rowbase = (size_t)bh * p.T + sp.T0;
    const int nchunks = (sp.TL + C - 1) / C;
    const int nsteps = pipe_steps<K>(nchunks);
    const TIn* kp = (const TIn*)p.k;
    // The chain waves form the gates f, w themselves (instead of the gate
    // waves) with the block prologue, whose gate waves have no k, and with
    // 128-column tiles, whose two gate waves would otherwise bound the step.
    constexpr bool CG = PRO || K::DV == 128;

    float l = SEG ? p.seg_l0[((size_t)bh * p.nseg + sp.seg) * DK + i]
                  : (p.l0 ? p.l0[(size_t)bh * DK + i] : 1.f);
    float qn = p.qn[(size_t)(bh % p.H) * DK + i];
    // Block prologue: qn = softplus(zqn); k = silu(conv(x)) from the taps of
    // key dim i and a window of the three x values before the token (from
    // the convolution state before token 0)
    float kw[4] = {0.f, 0.f, 0.f, 0.f}, kb = 0.f, kx1 = 0.f, kx2 = 0.f, kx3 = 0.f;
    if constexpr (PRO) {
        qn = act_softplus(qn);
        const int W = p.conv_w;
        const size_t ch = (size_t)(bh % p.H) * DK + i;
        load_taps4(kw, p.conv_wt[1] + ch * W, W);
        if (p.conv_b[1]) kb = p.conv_b[1][ch];
        // the x rows before the span's first token (segments after the first:
        // the sequence's own rows)
        kx1 = pro_x(kp, p.conv_s[1], bh, p.T, W, DK, sp.T0 - 1, i);
        kx2 = pro_x(kp, p.conv_s[1], bh, p.T, W, DK, sp.T0 - 2, i);
        kx3 = pro_x(kp, p.conv_s[1], bh, p.T, W, DK, sp.T0 - 3, i);
    }
    float wrun = 1.f;  // sequence split: gate product from the segment start
    // One chunk of inputs per buffer; NBC buffers rotate, so a chunk's loads
    // are issued NBC-1 iterations before their first use.
    constexpr int NB = K::NBC, D = NB - 1;
    struct Buf {
        // a, or with the prologue the bits of za like those of k
        typename std::conditional<PRO, unsigned, float>::type a[C];
        unsigned k[C];  // bits of k (or of its x), zero-extended (bf16 values sit in the low half)
        float r;        // r (or zr) of token `lane` of the chunk
    };
    Buf b[NB];
    auto bits_f = [](unsigned u) { return __builtin_bit_cast(float, sizeof(TIn) == 2 ? u << 16 : u); };

    // Rows of a and k are read through buffer resources over one chunk's
    // rows, so rows past T (the tail of the last chunk, chunks past the end)
    // read as zero.  At dk = 64 the resources cover 4 KiB windows, whose row
    // offsets are immediates: register offsets for the rows past 4 KiB spill
    // the chain role there.  At dk = 128 one resource per chunk and input is
    // faster (measured).
    constexpr int ARB = DK * (PRO ? (int)sizeof(TIn) : 4), KRB = DK * (int)sizeof(TIn);  // row bytes
    constexpr bool WIN = DK < 128;
    constexpr int ARW = WIN && 4096 / ARB < C ? 4096 / ARB : C;  // rows per resource
    constexpr int KRW = WIN && 4096 / KRB < C ? 4096 / KRB : C;
    const char* abase = (const char*)p.a + rowbase * ARB;
    const char* kbase = (const char*)(kp + rowbase * DK);
    const char* rbase = (const char*)(p.r + rowbase);
    auto rows_left = [&](int t, int cap) {
        const int n = sp.TL - t;
        return n < 0 ? 0 : (n < cap ? n : cap);
    };
    auto load = [&](int c, Buf& b) {
        const int t0 = c * C, rows = rows_left(t0, C);
        const char* a0 = abase + (size_t)t0 * ARB;
        const char* k0 = kbase + (size_t)t0 * KRB;
#pragma unroll
        for (int w = 0; w < C / ARW; ++w) {
            const int n = rows - w * ARW;
            const auto rs = make_rsrc(a0 + w * ARW * ARB, (n < 0 ? 0 : (n < ARW ? n : ARW)) * ARB);
#pragma unroll
            for (int t = 0; t < ARW; ++t) {
                if constexpr (!PRO)
                    b.a[w * ARW + t] = buf_load<float>(rs, i * 4 + t * ARB);
                else if constexpr (sizeof(TIn) == 2)
                    b.a[w * ARW + t] = (unsigned)buf_load<unsigned short>(rs, i * 2 + t * ARB);
                else
                    b.a[w * ARW + t] = buf_load<unsigned>(rs, i * 4 + t * ARB);
            }
        }
#pragma unroll
        for (int w = 0; w < C / KRW; ++w) {
            const int n = rows - w * KRW;
            const auto rs = make_rsrc(k0 + w * KRW * KRB, (n < 0 ? 0 : (n < KRW ? n : KRW)) * KRB);
#pragma unroll
            for (int t = 0; t < KRW; ++t)
                b.k[w * KRW + t] = sizeof(TIn) == 2 ? (unsigned)buf_load<unsigned short>(rs, i * 2 + t * KRB)
                                                    : buf_load<unsigned>(rs, i * 4 + t * KRB);
        }
        b.r = buf_load<float>(make_rsrc(rbase + (size_t)t0 * 4, rows * 4), lane * 4);
    };
    auto step = [&](int c, Buf& cur, Buf& nxt) {
        const int cc = c + 2;  // chunk scanned in this iteration
        wait_loads<(D - 1) * (2 * C + 1)>();
        if (nchunks > 0) load(cc + D, nxt);
        if (cc < nchunks) {
            const int L = chunk_len(sp.TL, cc, C), par = cc & 1;
            const float rho = lane < L ? 1.f / (PRO ? act_softplus(cur.r) + p.r_eps : cur.r) : 0.f;
            if (cw == 0 && lane < C) sm.rho[par][lane] = rho;
            float f0 = 1.f;  // gate of token 0 of the chunk (sequence split)
            // full chunks take a copy of the scan without per-token tests
            auto scan = [&](auto full) {
                constexpr bool FULL = decltype(full)::value;
                float num = 1.f, den = 1.f, G = 1.f;
#pragma unroll
                for (int t = 0; t < C; ++t) {
                    if (FULL || t < L) {
                        const float rt = __builtin_bit_cast(
                            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rho), t));
                        float a, kv;
                        if constexpr (PRO) {
                            a = act_sigmoid(bits_f(cur.a[t]));
                            const float x0 = bits_f(cur.k[t]);
                            kv = act_silu(conv4(kw, kb, x0, kx1, kx2, kx3));
                            kx3 = kx2;
                            kx2 = kx1;
                            kx1 = x0;
                        } else {
                            a = cur.a[t];
                            kv = bits_f(cur.k[t]);
                        }
                        const float lp = l * fast_rcp(__builtin_fmaf(qn, l, a * a));
                        l = __builtin_fmaf(kv * kv, rt, lp);
                        const float alp = a * lp;
                        if constexpr (CG) {
                            // the gates themselves: the gate waves have no k
                            const float rl = fast_rcp(l);
                            sm.LP[par][t][i ^ lp_swz(t)] = f32x2{alp * rl, kv * rt * rl};
                        } else {
                            sm.LP[par][t][i ^ lp_swz(t)] = f32x2{alp, l};
                        }
                        if (t >= 1) { num *= alp; den *= l; }
                        if (SEG && t == 0) { f0 = alp * fast_rcp(l); }
                    }
                    if (t % 8 == 7) { G *= num * fast_rcp(den); num = 1.f; den = 1.f; }
                }
                return G * num * fast_rcp(den);
            };
            const float G = L == C ? scan(std::true_type{}) : scan(std::false_type{});
            if (__builtin_amdgcn_ballot_w64(G < kFloor)) sm.bad[cc & 3] = 1;
            if constexpr (SEG) {
                const float wc = wrun * f0;  // through token 0
                sm.Wc[par][i] = wc;
                wrun = wc * G;                                // through the chunk's end
            }
        }
        lds_barrier();
    };

    if (nchunks > 0) {
#pragma unroll
        for (int j = 0; j < D; ++j) load(j, b[j]);
    }
    // step c scans chunk c+2 from buffer (c+2) mod NB and loads chunk c+2+D
    for (int c = -2; c < nsteps - 2; c += NB) {
#pragma unroll
        for (int s = 0; s < NB; ++s) step(c + s, b[s], b[(s + D) % NB]);
    }
    sm.lT[i] = l;
    if (sp.last && p.lT && vt == 0) p.lT[(size_t)bh * DK + i] = l;
    if constexpr (SEG) {
        if (vt == 0) {
            p.seg_d[((size_t)bh * p.nseg + sp.seg) * DK + i] = wrun;
            if (sp.last) p.seg_lend[(size_t)bh * DK + i] = l;
        }
    }
    lds_barrier();
}

// ------------------------------------------------------------------ chain role, wavefront-level Mobius scan
// The precision map of one token, l -> ((1 + b qn) l + b a^2) / (qn l + a^2)
// with b = k^2 / r, is the 2x2 projective matrix [[1 + b qn, b a^2], [qn, a^2]]
// = [[1, b], [0, 1]] [[1, 0], [qn, a^2]]; maps compose as matrix products and
// any positive multiple of a matrix is the same map.
struct Mob {
    float p11, p12, p21, p22;
};

__device__ __forceinline__ Mob mob_identity() { return Mob{1.f, 0.f, 0.f, 1.f}; }

// P <- M(b, a^2, qn) P (the token after the ones P already holds)
__device__ __forceinline__ void mob_push(Mob& P, float b, float a2, float qn) {
    const float r1 = __builtin_fmaf(qn, P.p11, a2 * P.p21);
    const float r2 = __builtin_fmaf(qn, P.p12, a2 * P.p22);
    P.p11 = __builtin_fmaf(b, r1, P.p11);
    P.p12 = __builtin_fmaf(b, r2, P.p12);
    P.p21 = r1;
    P.p22 = r2;
}

// the map of Y followed by X, i.e. X Y
__device__ __forceinline__ Mob mob_mul(const Mob& X, const Mob& Y) {
    return Mob{__builtin_fmaf(X.p11, Y.p11, X.p12 * Y.p21), __builtin_fmaf(X.p11, Y.p12, X.p12 * Y.p22),
               __builtin_fmaf(X.p21, Y.p11, X.p22 * Y.p21), __builtin_fmaf(X.p21, Y.p12, X.p22 * Y.p22)};
}

// divides by the entry sum (the entries are non-negative)
__device__ __forceinline__ void mob_norm(Mob& P) {
    const float s = fast_rcp((P.p11 + P.p12) + (P.p21 + P.p22));
    P.p11 *= s;
    P.p12 *= s;
    P.p21 *= s;
    P.p22 *= s;
}

__device__ __forceinline__ Mob mob_shfl_up(const Mob& P, int delta) {
    return Mob{__shfl_up(P.p11, delta, 64), __shfl_up(P.p12, delta, 64), __shfl_up(P.p21, delta, 64),
               __shfl_up(P.p22, delta, 64)};
}

// Chain waves: the precision of chunk c+2, as a wavefront-level Mobius scan.
// Lane (dq = lane % 16, tg = lane / 16) owns key dims i0..i0+3 (i0 = 64 cw +
// 4 dq) and tokens 8 tg .. 8 tg + 7 of the chunk.  Each lane composes its
// eight tokens' maps for its four key dims; a scan over the four token groups
// (lane shifts of 16 and 32) gives every group the map of the tokens before
// it, which applied to the chunk's carried precision gives the group's
// starting precision; then each lane runs the recursion over its eight
// tokens, writes (a lp, l) to LDS and forms its share of the chunk's gate
// product.  Rows arrive as 16-byte (a) and 8/16-byte (k) loads, 18 per lane
// and chunk, one chunk ahead.
template <typename TIn, class K, bool SEG>
__device__ void chain_role_scan(S3<TIn, K>& sm, const FwdArgs& p, const Span& sp, int bh, int vt, int cw,
                           int lane) {
    constexpr int C = K::C, DK = K::DK, TPL = 8;  // tokens per lane
    static_assert(C == 4 * TPL, "four token groups of eight");
    typedef typename Quad<TIn>::V QV;
    const int dq = lane & 15, tg = lane >> 4;
    const int i0 = cw * 64 + 4 * dq;
    const size_t rowbase = (size_t)bh * p.T + sp.T0;
    const int nchunks = (sp.TL + C - 1) / C;
    const int nsteps = pipe_steps<K>(nchunks);
    const TIn* kp = (const TIn*)p.k;

    float lin[4], qn[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = i0 + e;
        lin[e] = SEG ? p.seg_l0[((size_t)bh * p.nseg + sp.seg) * DK + i] : (p.l0 ? p.l0[(size_t)bh * DK + i] : 1.f);
        qn[e] = p.qn[(size_t)(bh % p.H) * DK + i];
    }
    float wrun[4] = {1.f, 1.f, 1.f, 1.f};  // sequence split: gate product from the segment start
    constexpr int NB = K::NBC, D = NB - 1;
    struct Buf {
        f32x4 a[TPL];  // a of the lane's four key dims, per token
        QV k[TPL];     // k likewise
        f32x4 r[2];    // r of the lane's eight tokens
    };
    constexpr int NLD = 2 * TPL + 2;  // loads per chunk
    Buf b[NB];
    constexpr int ES = (int)sizeof(TIn), ARB = DK * 4, KRB = DK * ES;  // row bytes
    const char* abase = (const char*)(p.a + rowbase * DK);
    const char* kbase = (const char*)(kp + rowbase * DK);
    const char* rbase = (const char*)(p.r + rowbase);
    const int aoff = TPL * tg * ARB + i0 * 4, koff = TPL * tg * KRB + i0 * ES, roff = TPL * tg * 4;
    auto load = [&](int c, Buf& bf) {
        const int t0 = c * C, n = sp.TL - t0;
        const int rows = n < 0 ? 0 : (n < C ? n : C);
        // rows past the segment's end read as zero
        const auto ra = make_rsrc(abase + (size_t)t0 * ARB, rows * ARB);
        const auto rk = make_rsrc(kbase + (size_t)t0 * KRB, rows * KRB);
        const auto rr = make_rsrc(rbase + (size_t)t0 * 4, rows * 4);
#pragma unroll
        for (int u = 0; u < TPL; ++u) {
            bf.a[u] = buf_load<f32x4>(ra, aoff + u * ARB);
            bf.k[u] = buf_load<QV>(rk, koff + u * KRB);
        }
        bf.r[0] = buf_load<f32x4>(rr, roff);
        bf.r[1] = buf_load<f32x4>(rr, roff + 16);
    };
    auto step = [&](int c, Buf& cur, Buf& nxt) {
        const int cc = c + 2;  // chunk scanned in this iteration
        wait_loads<(D - 1) * NLD>();
        if (nchunks > 0) load(cc + D, nxt);
        if (cc < nchunks) {
            const int L = chunk_len(sp.TL, cc, C), par = cc & 1;
            const int tb = TPL * tg;  // the lane's first token
            float rho[TPL];
#pragma unroll
            for (int u = 0; u < TPL; ++u) rho[u] = tb + u < L ? fast_rcp(cur.r[u / 4][u % 4]) : 0.f;
            if (cw == 0 && dq == 0) {
                *(f32x4*)&sm.rho[par][tb] = f32x4{rho[0], rho[1], rho[2], rho[3]};
                *(f32x4*)&sm.rho[par][tb + 4] = f32x4{rho[4], rho[5], rho[6], rho[7]};
            }
            float f0[4] = {1.f, 1.f, 1.f, 1.f}, Gp[4] = {1.f, 1.f, 1.f, 1.f}, lfin[4];
            // full chunks take a copy without per-token tests
            auto scan = [&](auto full) {
                constexpr bool FULL = decltype(full)::value;
                // ---- this lane's eight maps, composed per key dim
                Mob P[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) P[e] = mob_identity();
#pragma unroll
                for (int u = 0; u < TPL; ++u) {
                    if (FULL || tb + u < L) {
                        const f32x4 kv = Quad<TIn>::to_f32(cur.k[u]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float a = cur.a[u][e];
                            mob_push(P[e], kv[e] * kv[e] * rho[u], a * a, qn[e]);
                        }
                    }
                    if (u == TPL / 2 - 1) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) mob_norm(P[e]);
                    }
                }
                // ---- scan over the four token groups: the map of every token
                // before the group, applied to the chunk's carried precision
                float ls[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    mob_norm(P[e]);
                    Mob Y = mob_shfl_up(P[e], 16);
                    if (tg >= 1) P[e] = mob_mul(P[e], Y);
                    mob_norm(P[e]);
                    Y = mob_shfl_up(P[e], 32);
                    if (tg >= 2) P[e] = mob_mul(P[e], Y);
                    Mob E = mob_shfl_up(P[e], 16);
                    if (tg == 0) E = mob_identity();
                    ls[e] = __builtin_fmaf(E.p11, lin[e], E.p12) * fast_rcp(__builtin_fmaf(E.p21, lin[e], E.p22));
                }
                // ---- the recursion over the lane's tokens
                float num[4] = {1.f, 1.f, 1.f, 1.f}, den[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
                for (int u = 0; u < TPL; ++u) {
                    const int t = tb + u;
                    if (FULL || t < L) {
                        const f32x4 kv = Quad<TIn>::to_f32(cur.k[u]);
                        float alp[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float a = cur.a[u][e];
                            const float lp = ls[e] * fast_rcp(__builtin_fmaf(qn[e], ls[e], a * a));
                            ls[e] = __builtin_fmaf(kv[e] * kv[e], rho[u], lp);
                            alp[e] = a * lp;
                            if (t >= 1) {
                                num[e] *= alp[e];
                                den[e] *= ls[e];
                            } else {
                                f0[e] = alp[e] * fast_rcp(ls[e]);
                            }
                        }
                        const int j = i0 ^ lp_swz(t);
                        *(f32x4*)&sm.LP[par][t][j] = f32x4{alp[0], ls[0], alp[1], ls[1]};
                        *(f32x4*)&sm.LP[par][t][j + 2] = f32x4{alp[2], ls[2], alp[3], ls[3]};
                    }
                    if (u == TPL / 2 - 1) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            Gp[e] *= num[e] * fast_rcp(den[e]);
                            num[e] = 1.f;
                            den[e] = 1.f;
                        }
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Gp[e] *= num[e] * fast_rcp(den[e]);
                    lfin[e] = ls[e];
                }
            };
            if (L == C) scan(std::true_type{});
            else scan(std::false_type{});
            // the chunk's gate product (tokens 1..), the precision it leaves
            // (after the last group), and token 0's gate, in every lane of the
            // key-dim quad
            float G[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                G[e] = Gp[e] * __shfl_xor(Gp[e], 16, 64);
                G[e] *= __shfl_xor(G[e], 32, 64);
                lin[e] = __shfl(lfin[e], 48 + dq, 64);
                f0[e] = __shfl(f0[e], dq, 64);
            }
            const bool low = G[0] < kFloor || G[1] < kFloor || G[2] < kFloor || G[3] < kFloor;
            if (__builtin_amdgcn_ballot_w64(low)) sm.bad[cc & 3] = 1;
            if constexpr (SEG) {
                f32x4 wc;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wc[e] = wrun[e] * f0[e];  // through token 0
                    wrun[e] = wc[e] * G[e];   // through the chunk's end
                }
                if (tg == 0) *(f32x4*)&sm.Wc[par][i0] = wc;
            }
        }
        lds_barrier();
    };

    if (nchunks > 0) {
#pragma unroll
        for (int j = 0; j < D; ++j) load(j, b[j]);
    }
    // step c scans chunk c+2 from buffer (c+2) mod NB and loads chunk c+2+D
    for (int c = -2; c < nsteps - 2; c += NB) {
#pragma unroll
        for (int s = 0; s < NB; ++s) step(c + s, b[s], b[(s + D) % NB]);
    }
    if (tg == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = i0 + e;
            sm.lT[i] = lin[e];
            if (sp.last && p.lT && vt == 0) p.lT[(size_t)bh * DK + i] = lin[e];
            if constexpr (SEG) {
                if (vt == 0) {
                    p.seg_d[((size_t)bh * p.nseg + sp.seg) * DK + i] = wrun[e];
                    if (sp.last) p.seg_lend[(size_t)bh * DK + i] = lin[e];
                }
            }
        }
    }
    lds_barrier();
}

// a lane's 4- or 8-byte value from lane src of the wave
template <typename V>
__device__ __forceinline__ V shfl_val(V v, int src) {
    if constexpr (sizeof(V) == 4) {
        return __builtin_bit_cast(V, __shfl(__builtin_bit_cast(int, v), src, 64));
    } else {
        static_assert(sizeof(V) == 8, "4 or 8 bytes");
        i32x2 x = __builtin_bit_cast(i32x2, v);
        x[0] = __shfl(x[0], src, 64);
        x[1] = __shfl(x[1], src, 64);
        return __builtin_bit_cast(V, x);
    }
}

// ------------------------------------------------------------------ gate role
template <typename TIn, class K, bool SEG, bool PRO, class TAPS>
__device__ void gate_role(S3<TIn, K>& sm, TAPS& taps, const FwdArgs& p, const Span& sp, int bh, int vt, int gw,
                          int lane) {
    typedef Pair<TIn> PR;
    typedef typename Quad<TIn>::V QV;
    constexpr int C = K::C, DK = K::DK, DV = K::DV, TPG = K::TPG;
    const size_t rowbase = (size_t)bh * p.T + sp.T0;
    const int nchunks = (sp.TL + C - 1) / C;
    // sequence split: segments after the first also write q (.) (gate product
    // since the segment start) for the correction pass (one value-tile
    // workgroup writes it)
    const bool wq = SEG && sp.seg > 0 && vt == 0;
    const int nsteps = pipe_steps<K>(nchunks);
    const int grp = lane % K::NGRP, ipl = lane / K::NGRP;
    // group h of this wave is virtual gate wave gw + h * NGW
    constexpr int NV = K::NVG;
    static_assert(NV == 1 || !PRO, "the block prologue runs with four gate waves");
    int ipv[NV], gtv[NV];
#pragma unroll
    for (int h = 0; h < NV; ++h) {
        ipv[h] = (gw + h * K::NGW) * K::IPW + ipl;
        gtv[h] = (gw + h * K::NGW) * 64 + lane;
    }
    const int ip = ipv[0];
    const int gtid = gtv[0];
    const TIn* qp = (const TIn*)p.q;
    const TIn* kp = (const TIn*)p.k;
    const TIn* vp = (const TIn*)p.v;

    struct Buf {
        typename PR::V q[TPG], k[TPG];
        QV v[K::VPT][2];
        QV vh[K::VPT][3];  // block prologue: the three v rows before the unit's tokens
    };
    constexpr int NB = K::NBG, D = NB - 1;
    // With two groups per wave each group keeps one buffer, refilled with
    // the next chunk's rows once the step has used it (two in-flight chunks
    // for both groups would not fit in the registers).
    constexpr int NBUF = NV == 1 ? NB : 1;
    Buf b[NBUF][NV];
    // with the block prologue or 128-column tiles the chain waves form f
    // and w, and the gate waves read no k
    constexpr bool CG = PRO || K::DV == 128;
    // sequence split with the block prologue, bf16: the MMA waves store
    // q-hat, which leaves the gate waves (the convolution of q and v is theirs)
    // more of the step (measured 7% faster on the B1 H16 T32768 block; without
    // the prologue 3-4% slower, and with 128-column tiles it spilled the chain
    // waves' registers)
    constexpr bool QM = SEG && PRO && std::is_same<TIn, bf16>::value && K::DV == 64;
    constexpr int NLD = (PRO ? TPG + 5 * K::VPT : CG ? TPG + 2 * K::VPT : 2 * TPG + 2 * K::VPT);  // loads per chunk
    // The next chunk's rows are requested after the step's work: at the step
    // start they queue with the chain waves' requests, which are on the
    // critical path (measured 8% faster on the LM-layer shape, 4% on the
    // split long-context forward).
    // Each chunk is read through buffer resources spanning its rows, so rows
    // past T read as zero; a lane's token rows are immediates from its offset.
    constexpr int ES = (int)sizeof(TIn), QRB = DK * ES;
    const int VRB = p.dv * ES;
    const char* qbase = (const char*)(qp + rowbase * DK);
    const char* kbase = (const char*)(kp + rowbase * DK);
    const char* vbase = (const char*)(vp + rowbase * p.dv);
    int qoffv[NV], voffv[NV][K::VPT][2];
#pragma unroll
    for (int h = 0; h < NV; ++h) {
        qoffv[h] = grp * TPG * QRB + 2 * ipv[h] * ES;
#pragma unroll
        for (int x = 0; x < K::VPT; ++x) {
            const int unit = gtv[h] + x * 256;
            const int tp = unit / K::VQ, jq = unit % K::VQ;
            voffv[h][x][0] = 2 * tp * VRB + (vt * DV + 4 * jq) * ES;
            voffv[h][x][1] = voffv[h][x][0] + VRB;
        }
    }
    // Block prologue: the chain waves form k and the gates f, w; the gate
    // waves form q and v.  They stage the taps and biases in LDS (read from
    // the first gated chunk on, after the pipeline's first barrier).  The
    // three x rows of q before a lane's first token come from the lane of the
    // previous token group, and for the first group from the last group's
    // rows of the previous chunk, kept in pq (before token 0: the convolution
    // state).  The three v rows before a unit's tokens are loaded with it.
    typename PR::V pq[3];
    if constexpr (PRO) {
        const int W = p.conv_w, h = bh % p.H;
        for (int x = gtid; x < DK; x += 256) {
            const size_t ch = (size_t)h * DK + x;
            float w4[4];
            load_taps4(w4, p.conv_wt[0] + ch * W, W);
            taps.qw[x] = f32x4{w4[0], w4[1], w4[2], w4[3]};
            taps.qb[x] = p.conv_b[0] ? p.conv_b[0][ch] : 0.f;
        }
        for (int x = gtid; x < DV; x += 256) {
            const size_t ch = (size_t)h * p.dv + vt * DV + x;
            float w4[4];
            load_taps4(w4, p.conv_wt[2] + ch * W, W);
            taps.vw[x] = f32x4{w4[0], w4[1], w4[2], w4[3]};
            taps.vb[x] = p.conv_b[2] ? p.conv_b[2][ch] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 3; ++j)  // token T0 + j - 3
            pq[j] = PR::make(pro_x(qp, p.conv_s[0], bh, p.T, W, DK, sp.T0 + j - 3, 2 * ip),
                             pro_x(qp, p.conv_s[0], bh, p.T, W, DK, sp.T0 + j - 3, 2 * ip + 1));
    }
    auto load = [&](int c, Buf& bf, int h) {
        const int qoff = qoffv[h];
        const auto& voff = voffv[h];
        const int t0 = c * C, n = sp.TL - t0;
        const int rows = n < 0 ? 0 : (n < C ? n : C);
        const auto rq = make_rsrc(qbase + (size_t)t0 * QRB, rows * QRB);
        const auto rk = make_rsrc(kbase + (size_t)t0 * QRB, rows * QRB);
        const auto rv = make_rsrc(vbase + (size_t)t0 * VRB, rows * VRB);
#pragma unroll
        for (int u = 0; u < TPG; ++u) {
            bf.q[u] = buf_load<typename PR::V>(rq, qoff + u * QRB);
            if constexpr (!CG) bf.k[u] = buf_load<typename PR::V>(rk, qoff + u * QRB);
        }
#pragma unroll
        for (int x = 0; x < K::VPT; ++x)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) bf.v[x][h2] = buf_load<QV>(rv, voff[x][h2]);
        if constexpr (PRO) {
            // rows t0-3 .. of the span, clipped to the sequence start and the
            // span end: rows before token 0 of the sequence read as zero (the
            // state is added at the first chunk)
            const int h0 = sp.T0 + t0 >= 3 ? t0 - 3 : -sp.T0;
            const int hend = t0 + rows < sp.TL ? t0 + rows : sp.TL;
            const auto rh = make_rsrc(vbase + (ptrdiff_t)h0 * VRB, (hend > h0 ? hend - h0 : 0) * VRB);
#pragma unroll
            for (int x = 0; x < K::VPT; ++x)
#pragma unroll
                for (int j = 0; j < 3; ++j) bf.vh[x][j] = buf_load<QV>(rh, voff[x][0] + (j - 3 + t0 - h0) * VRB);
        }
    };

    auto step = [&](int c, Buf (&curs)[NV], Buf (&nxts)[NV]) {
        const int cg = c + 1;  // chunk gated in this iteration
        wait_loads<(D - 1) * NLD * NV>();
#pragma unroll
        for (int h = 0; h < NV; ++h) {
        const int ip = ipv[h], gtid = gtv[h], gwv = gw + h * K::NGW;
        Buf& cur = curs[h];
        if (cg >= 0 && cg < nchunks) {
            const int L = chunk_len(sp.TL, cg, C), par = cg & 1;
            // V^T of the chunk
#pragma unroll
            for (int x = 0; x < K::VPT; ++x) {
                const int unit = gtid + x * 256;
                const int tp = unit / K::VQ, jq = unit % K::VQ;
                f32x4 v0 = Quad<TIn>::to_f32(cur.v[x][0]), v1 = Quad<TIn>::to_f32(cur.v[x][1]);
                if constexpr (PRO) {
                    f32x4 h[3];
#pragma unroll
                    for (int j = 0; j < 3; ++j) h[j] = Quad<TIn>::to_f32(cur.vh[x][j]);
                    if (cg == 0 && sp.T0 == 0 && p.conv_s[2]) {
                        // the first chunk: rows before token 0 from the state
                        const int W = p.conv_w;
#pragma unroll
                        for (int j = 0; j < 3; ++j) {
                            const int sr = W - 1 + 2 * tp - 3 + j;
                            if (2 * tp - 3 + j < 0 && sr >= 0)
                                h[j] += Quad<TIn>::to_f32(*(const QV*)((const TIn*)p.conv_s[2] +
                                                                      ((size_t)bh * (W - 1) + sr) * p.dv +
                                                                      vt * DV + 4 * jq));
                        }
                    }
                    const bool in0 = 2 * tp < L, in1 = 2 * tp + 1 < L;
                    f32x4 y0, y1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const f32x4 w4 = taps.vw[4 * jq + e];
                        const float b = taps.vb[4 * jq + e];
                        y0[e] = in0 ? act_silu(conv4(w4, b, v0[e], h[2][e], h[1][e], h[0][e])) : 0.f;
                        y1[e] = in1 ? act_silu(conv4(w4, b, v1[e], v0[e], h[2][e], h[1][e])) : 0.f;
                    }
                    v0 = y0;
                    v1 = y1;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *(typename PR::V*)&sm.VT[par][4 * jq + e][(2 * tp) ^ vt_swz<K>(4 * jq + e)] =
                        PR::make(v0[e], v1[e]);
            }
            // q of the lane's tokens: the loaded rows, or with the block
            // prologue their convolution and SiLU (the three earlier rows from
            // the lane of the previous token group)
            typename PR::V hq[3];
            if constexpr (PRO) {
                const int src = grp > 0 ? lane - 1 : lane + K::NGRP - 1;
#pragma unroll
                for (int j = 0; j < 3; ++j) hq[j] = shfl_val(grp == K::NGRP - 1 ? pq[j] : cur.q[TPG - 3 + j], src);
#pragma unroll
                for (int j = 0; j < 3; ++j) pq[j] = cur.q[TPG - 3 + j];
            }
            // value e (0: key dim 2ip, 1: 2ip+1) of row j of a window whose
            // rows 0..2 are the halo h and 3.. the lane's tokens
            auto xw = [&](const typename PR::V* rows, const typename PR::V (&h)[3], int j, int e) {
                const typename PR::V v = j < 3 ? h[j] : rows[j - 3];
                return e ? PR::hi(v) : PR::lo(v);
            };
            auto qval = [&](int u, int e) -> float {
                if constexpr (PRO) {
                    const int c = 2 * ip + e;
                    return act_silu(conv4(taps.qw[c], taps.qb[c], xw(cur.q, hq, 3 + u, e), xw(cur.q, hq, 2 + u, e),
                                          xw(cur.q, hq, 1 + u, e), xw(cur.q, hq, u, e)));
                } else {
                    return e ? PR::hi(cur.q[u]) : PR::lo(cur.q[u]);
                }
            };
            // gates
            float f[TPG][2], w[TPG][2];
#pragma unroll
            for (int u = 0; u < TPG; ++u) {
                const int t = grp * TPG + u;
                // a*lp, l (two key dims); or f, w from the chain waves
                const f32x4 lq = *(const f32x4*)&sm.LP[par][t][(2 * ip) ^ lp_swz(t)];
                if constexpr (CG) {
                    f[u][0] = lq[0];
                    w[u][0] = lq[1];
                    f[u][1] = lq[2];
                    w[u][1] = lq[3];
                } else {
                    const float rh = sm.rho[par][t];
                    const float rl0 = fast_rcp(lq[1]), rl1 = fast_rcp(lq[3]);
                    f[u][0] = lq[0] * rl0;
                    f[u][1] = lq[2] * rl1;
                    w[u][0] = PR::lo(cur.k[u]) * rh * rl0;
                    w[u][1] = PR::hi(cur.k[u]) * rh * rl1;
                }
            }
            const float* Eprev = sm.E[par ^ 1];
            const float wc0 = SEG ? sm.Wc[par][2 * ip] : 1.f, wc1 = SEG ? sm.Wc[par][2 * ip + 1] : 1.f;
            // q-hat rows of this chunk (range 0 when not written)
            // (16-token tiles: the chunk start is a multiple of 16 tokens)
            const auto rqh = SEG && wq ? make_rsrc((const TIn*)p.seg_qhat +
                                                       qhat_tile_offset(bh, p.T, DK, sp.T0 + cg * C, 0),
                                                   (L + 15) / 16 * 16 * DK * (int)sizeof(TIn))
                                       : make_rsrc(p.q, 0);
            // element offset of (token t of the chunk, key dims 2ip, 2ip+1) there
            auto qho = [&](int t, int i) {
                return ((t / 16) * (DK / 32) + i / 32) * 512 + (i % 32 / 8 * 16 + t % 16) * 8 + i % 8;
            };
            // eight key dims of q-hat from a row of Q^ (LDS) and Wc, as one
            // 16-byte store (two for fp32)
            auto store_qhat8 = [&](const TIn* qr, f32x4 c0, f32x4 c1, int off) {
                typedef typename Quad<TIn>::V QV;
                const QV b0 = Quad<TIn>::make(Quad<TIn>::to_f32(*(const QV*)qr) * c0);
                const QV b1 = Quad<TIn>::make(Quad<TIn>::to_f32(*(const QV*)(qr + 4)) * c1);
                if constexpr (sizeof(TIn) == 2) {
                    struct alignas(16) Two { QV x, y; };
                    buf_store(__builtin_bit_cast(f32x4, Two{b0, b1}), rqh, off);
                } else {
                    buf_store(b0, rqh, off);
                    buf_store(b1, rqh, off + 16);
                }
            };
            // Factorised operands.  Full chunks take a copy with no per-token
            // tests, so the whole step is one basic block the compiler can
            // schedule; only the lanes holding token 0 or the last token
            // store the state prescale and the chunk-end gate.
            auto fac = [&](auto full) {
                constexpr bool FULL = decltype(full)::value;
                float G[TPG][2];
                float p0 = 1.f, p1 = 1.f;
#pragma unroll
                for (int u = 0; u < TPG; ++u) {
                    const int t = grp * TPG + u;
                    const bool inc = FULL ? (u > 0 || grp > 0) : (t > 0 && t < L);
                    p0 *= inc ? f[u][0] : 1.f;
                    p1 *= inc ? f[u][1] : 1.f;
                    G[u][0] = p0;
                    G[u][1] = p1;
                }
                const float e0 = group_excl_prod<K>(p0, grp), e1 = group_excl_prod<K>(p1, grp);
                TIn wt0[TPG], wt1[TPG];
                float gl0 = 1.f, gl1 = 1.f;
#pragma unroll
                for (int u = 0; u < TPG; ++u) {
                    const int t = grp * TPG + u;
                    const float g0 = G[u][0] * e0, g1 = G[u][1] * e1;
                    const bool in = FULL || t < L;
                    const float q0 = in ? qval(u, 0) * g0 : 0.f;
                    const float q1 = in ? qval(u, 1) * g1 : 0.f;
                    const float w0 = in ? w[u][0] * fast_rcp(g0) : 0.f;
                    const float w1 = in ? w[u][1] * fast_rcp(g1) : 0.f;
                    *(typename PR::V*)&sm.op[par].fac.Q[qw_row<K>(t)][2 * ip] = PR::make(q0, q1);
                    *(typename PR::V*)&sm.op[par].fac.W[qw_row<K>(t)][2 * ip] = PR::make(w0, w1);
                    wt0[u] = (TIn)w0;
                    wt1[u] = (TIn)w1;
                    if (!FULL && t == L - 1) { gl0 = g0; gl1 = g1; }
                    if (FULL && u == TPG - 1) { gl0 = g0; gl1 = g1; }
                }
                store_row<TIn, TPG>(&sm.op[par].fac.WT[2 * ip][grp * TPG], wt0);
                store_row<TIn, TPG>(&sm.op[par].fac.WT[2 * ip + 1][grp * TPG], wt1);
                if (grp == 0) *(f32x2*)&sm.sc[par][2 * ip] =
                    f32x2{Eprev[2 * ip] * f[0][0], Eprev[2 * ip + 1] * f[0][1]};
                const int gend = FULL ? K::NGRP - 1 : (L - 1) / TPG;
                if (grp == gend) *(f32x2*)&sm.E[par][2 * ip] = f32x2{gl0, gl1};
            };
            if (!__builtin_amdgcn_readfirstlane(sm.bad[cg & 3])) {
                if (L == C) fac(std::true_type{});
                else fac(std::false_type{});
                if constexpr (QM) {
                    // the MMA waves store q-hat from their Q^ fragments
                    if (grp == 0) *(f32x2*)&sm.WcM[par][2 * ip] = f32x2{wc0, wc1};
                } else if constexpr (SEG) {
                    if (wq) {
                        // q-hat = Q^ (.) Wc, read back from this wave's own
                        // block of Q^ (all tokens, its 2 IPW key dims) as 8
                        // consecutive key dims of one token per lane, so
                        // that each lane writes whole 16-byte pieces of the
                        // tiled layout (rows past L hold zeros)
                        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
                        __builtin_amdgcn_wave_barrier();
                        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
                        for (int x = 0; x < K::IPW / 8; ++x) {
                            const int pid = x * 64 + lane, t = pid % C;
                            const int i0 = gwv * 2 * K::IPW + 8 * (pid / C);
                            const f32x4 c0 = *(const f32x4*)&sm.Wc[par][i0];
                            const f32x4 c1 = *(const f32x4*)&sm.Wc[par][i0 + 4];
                            store_qhat8(&sm.op[par].fac.Q[qw_row<K>(t)][i0], c0, c1,
                                        qho(t, i0) * (int)sizeof(TIn));
                        }
                    }
                }
            } else {
                if constexpr (SEG) {
                    if (wq) {
                        // q (.) gate product for the correction pass, from the
                        // chunk-start products of this path's raw gates
                        float p0 = 1.f, p1 = 1.f;
                        float G[TPG][2];
#pragma unroll
                        for (int u = 0; u < TPG; ++u) {
                            const int t = grp * TPG + u;
                            const bool inc = t > 0 && t < L;
                            p0 *= inc ? f[u][0] : 1.f;
                            p1 *= inc ? f[u][1] : 1.f;
                            G[u][0] = p0;
                            G[u][1] = p1;
                        }
                        const float e0 = group_excl_prod<K>(p0, grp), e1 = group_excl_prod<K>(p1, grp);
#pragma unroll
                        for (int u = 0; u < TPG; ++u) {
                            const int t = grp * TPG + u;
                            const float q0 = qval(u, 0) * G[u][0] * e0 * wc0;
                            const float q1 = qval(u, 1) * G[u][1] * e1 * wc1;
                            buf_store(PR::make(q0, q1), rqh, qho(t, 2 * ip) * (int)sizeof(TIn));
                        }
                    }
                }
                // flagged chunk: raw fp32 gates for the token-by-token path
#pragma unroll
                for (int u = 0; u < TPG; ++u) {
                    const int t = grp * TPG + u;
                    const bool in = t < L;
                    *(f32x2*)&sm.op[par].raw.f[t][2 * ip] = f32x2{in ? f[u][0] : 1.f, in ? f[u][1] : 1.f};
                    *(f32x2*)&sm.op[par].raw.w[t][2 * ip] = f32x2{in ? w[u][0] : 0.f, in ? w[u][1] : 0.f};
                    if (t == 0) {
                        sm.sc[par][2 * ip] = Eprev[2 * ip];
                        sm.sc[par][2 * ip + 1] = Eprev[2 * ip + 1];
                    }
                    if (t == L - 1) {
                        sm.E[par][2 * ip] = 1.f;
                        sm.E[par][2 * ip + 1] = 1.f;
                    }
                }
            }
        }
        }
        if (nchunks > 0) {
#pragma unroll
            for (int h = 0; h < NV; ++h) load(cg + D, nxts[h], h);
        }
        lds_barrier();
    };

#pragma unroll
    for (int h = 0; h < NV; ++h)
        if (gtv[h] < DK) sm.E[1][gtv[h]] = 1.f;
    // step c gates chunk c+1 from buffer (c+1) mod NB and loads chunk c+1+D;
    // the first step only loads
    if (nchunks > 0) {
#pragma unroll
        for (int j = 0; j < D - 1; ++j)
#pragma unroll
            for (int h = 0; h < NV; ++h) load(j, b[j % NBUF][h], h);
    }
    if constexpr (NBUF == 1) {
        for (int c = -2; c < nsteps - 2; ++c) step(c, b[0], b[0]);
    } else {
        for (int c = -2; c < nsteps - 2; c += NB) {
#pragma unroll
            for (int s = 0; s < NB; ++s) step(c + s, b[(s + NB - 1) % NB], b[(s + NB - 2) % NB]);
        }
    }
    lds_barrier();
}

// ------------------------------------------------------------------ MMA role
template <typename TIn, class K, bool SEG, bool PRO>
__device__ void mma_role(S3<TIn, K>& sm, const FwdArgs& p, const Span& sp, int bh, int vt, int mw,
                         int lane) {
    typedef Frag<TIn> F;
    typedef typename F::V FV;
    constexpr int C = K::C, DK = K::DK, DV = K::DV, IT = K::IT, JT = K::JT, KB = K::KB;
    // sequence split with the block prologue, bf16: these waves store q-hat
    constexpr bool QM = SEG && PRO && std::is_same<TIn, bf16>::value && K::DV == 64;
    const size_t rowbase = (size_t)bh * p.T + sp.T0;
    const int nchunks = (sp.TL + C - 1) / C;
    const int nsteps = pipe_steps<K>(nchunks);
    const int c16 = lane & 15, g = lane >> 4;
    const bool has_eta0 = p.eta0 && sp.seg == 0;  // later segments start from a zero state
    TIn* op = (TIn*)p.o;
    const TIn* qp = (const TIn*)p.q;

    f32x4 acc[IT][JT];
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int jj = 0; jj < JT; ++jj) {
            const int j = vt * DV + (mw * JT + jj) * 16 + c16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = it * 16 + 4 * g + e;
                acc[it][jj][e] = has_eta0 ? p.eta0[((size_t)bh * DK + i) * p.dv + j] /
                                                (p.l0 ? p.l0[(size_t)bh * DK + i] : 1.f)
                                          : 0.f;
            }
        }

    auto step = [&](int c) {
        if (c >= 0 && c < nchunks) {
            const int L = chunk_len(sp.TL, c, C), par = c & 1, t0 = c * C;
            const bool bad = __builtin_amdgcn_readfirstlane(sm.bad[c & 3]);
            if (mw == 0 && lane == 0 && c >= 1) sm.bad[(c - 1) & 3] = 0;
            // m <- sc (.) m
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const f32x4 s = *(const f32x4*)&sm.sc[par][it * 16 + 4 * g];
#pragma unroll
                for (int jj = 0; jj < JT; ++jj) acc[it][jj] *= s;
            }
            if (!bad) {
                const OpFac<TIn, K>& o = sm.op[par].fac;
                // o rows of this chunk; rows past T fall outside the range
                const auto ro = make_rsrc(op + (rowbase + t0) * p.dv, L * p.dv * (int)sizeof(TIn));
                FV Qf[2][KB], Vf[JT];
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int kk = 0; kk < KB; ++kk)
                        Qf[b][kk] = F::ld(&o.Q[qw_row<K>(b * 16 + c16)][kk * 32], g);
#pragma unroll
                for (int jj = 0; jj < JT; ++jj) {
                    const int j = (mw * JT + jj) * 16 + c16, sw = vt_swz<K>(j);
                    Vf[jj] = F::ld2(&sm.VT[par][j][(4 * g) ^ sw], &sm.VT[par][j][(16 + 4 * g) ^ sw]);
                }
                // causal S^T tiles (sigma, tau)
                f32x4 s00 = {0.f, 0.f, 0.f, 0.f}, s01 = s00, s11 = s00;
#pragma unroll
                for (int kk = 0; kk < KB; ++kk) {
                    const FV w0 = F::ld(&o.W[qw_row<K>(c16)][kk * 32], g);
                    const FV w1 = F::ld(&o.W[qw_row<K>(16 + c16)][kk * 32], g);
                    s00 = F::mma(w0, Qf[0][kk], s00);
                    s01 = F::mma(w0, Qf[1][kk], s01);
                    s11 = F::mma(w1, Qf[1][kk], s11);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (4 * g + e > c16) { s00[e] = 0.f; s11[e] = 0.f; }
                }
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const FV P0 = F::from_acc(s00, zero), P1 = F::from_acc(s01, s11);
                // readout O^T = m^T Q^^T + V^T P^T, the state as the A operand
#pragma unroll
                for (int jj = 0; jj < JT; ++jj) {
                    f32x4 out0 = {0.f, 0.f, 0.f, 0.f}, out1 = out0;
#pragma unroll
                    for (int kk = 0; kk < KB; ++kk) {
                        const FV am = F::from_acc(acc[2 * kk][jj], acc[2 * kk + 1][jj]);
                        out0 = F::mma(am, Qf[0][kk], out0);
                        out1 = F::mma(am, Qf[1][kk], out1);
                    }
                    out0 = F::mma(Vf[jj], P0, out0);
                    out1 = F::mma(Vf[jj], P1, out1);
                    const int col = vt * DV + (mw * JT + jj) * 16 + 4 * g;
                    buf_store(Quad<TIn>::make(out0), ro, (c16 * p.dv + col) * (int)sizeof(TIn));
                    buf_store(Quad<TIn>::make(out1), ro, ((16 + c16) * p.dv + col) * (int)sizeof(TIn));
                }
                // m += W^^T V
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    const FV wt = F::ld(&o.WT[it * 16 + c16][0], g);
#pragma unroll
                    for (int jj = 0; jj < JT; ++jj) acc[it][jj] = F::mma(wt, Vf[jj], acc[it][jj]);
                }
                // Sequence split, bf16: q-hat = Q^ (.) Wc for the correction pass,
                // from the Q^ fragments (the MMA waves that share the chain
                // waves' SIMDs, which have issue slots to spare).  Lanes g and
                // g^1 swap a half so that each holds 8 consecutive key dims,
                // the tiled layout's 16-byte piece: the same values the gate
                // waves would store (bf16 Q^ times Wc, rounded once more).
                if constexpr (QM) {
                    if (sp.seg > 0 && vt == 0 && mw < 2) {
                        const auto rqh = make_rsrc((const TIn*)p.seg_qhat +
                                                       qhat_tile_offset(bh, p.T, DK, sp.T0 + t0, 0),
                                                   (L + 15) / 16 * 16 * DK * (int)sizeof(TIn));
                        const int odd = g & 1, gn = odd ? 2 + (g >> 1) : (g >> 1);
#pragma unroll
                        for (int b = 0; b < 2; ++b)
#pragma unroll
                            for (int kk = 0; kk < KB; ++kk) {
                                if (kk % 2 != mw) continue;
                                typedef unsigned u32x4 __attribute__((__vector_size__(16)));
                                const u32x4 u = __builtin_bit_cast(u32x4, Qf[b][kk]);
                                // slots 0-3: dims 4g.., 4-7: dims 16+4g..
                                const unsigned x0 = odd ? u[0] : u[2], x1 = odd ? u[1] : u[3];
                                const unsigned y0 = (unsigned)__shfl_xor((int)x0, 16, 64);
                                const unsigned y1 = (unsigned)__shfl_xor((int)x1, 16, 64);
                                const u32x4 nat = odd ? u32x4{y0, y1, u[2], u[3]} : u32x4{u[0], u[1], y0, y1};
                                const int i0 = kk * 32 + 8 * gn;
                                const f32x4 w0 = *(const f32x4*)&sm.WcM[par][i0];
                                const f32x4 w1 = *(const f32x4*)&sm.WcM[par][i0 + 4];
                                const f32x4 lo = f32x4{__builtin_bit_cast(float, nat[0] << 16),
                                                       __builtin_bit_cast(float, nat[0] & 0xffff0000u),
                                                       __builtin_bit_cast(float, nat[1] << 16),
                                                       __builtin_bit_cast(float, nat[1] & 0xffff0000u)} * w0;
                                const f32x4 hi = f32x4{__builtin_bit_cast(float, nat[2] << 16),
                                                       __builtin_bit_cast(float, nat[2] & 0xffff0000u),
                                                       __builtin_bit_cast(float, nat[3] << 16),
                                                       __builtin_bit_cast(float, nat[3] & 0xffff0000u)} * w1;
                                struct alignas(16) Two { typename Quad<TIn>::V x, y; };
                                buf_store(__builtin_bit_cast(f32x4, Two{Quad<TIn>::make(lo), Quad<TIn>::make(hi)}),
                                          rqh, ((b * KB + kk) * 512 + (gn * 16 + c16) * 8) * (int)sizeof(TIn));
                            }
                    }
                }
            } else {
                // exact path: m <- f_t (.) m + w_t v_t^T, o_t = q_t^T m, token by token
                const OpRaw<K>& o = sm.op[par].raw;
                // one 16-column tile at a time: updating every tile per token
                // raised the register demand of the whole role
#pragma unroll
                for (int jj = 0; jj < JT; ++jj) {
                    const int j = (mw * JT + jj) * 16 + c16;
#pragma unroll 1
                    for (int t = 0; t < L; ++t) {
                        const float vj = (float)sm.VT[par][j][t ^ vt_swz<K>(j)];
                        float part = 0.f;
#pragma unroll
                        for (int it = 0; it < IT; ++it) {
                            const f32x4 fi = *(const f32x4*)&o.f[t][it * 16 + 4 * g];
                            const f32x4 wi = *(const f32x4*)&o.w[t][it * 16 + 4 * g];
                            const f32x4 qi = Quad<TIn>::to_f32(
                                *(const typename Quad<TIn>::V*)(qp + (rowbase + t0 + t) * DK + it * 16 + 4 * g));
                            acc[it][jj] = fi * acc[it][jj] + wi * vj;
#pragma unroll
                            for (int e = 0; e < 4; ++e) part += qi[e] * acc[it][jj][e];
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        part += __shfl_xor(part, 16, 64);
                        part += __shfl_xor(part, 32, 64);
                        if (g == 0) op[(rowbase + t0 + t) * p.dv + (size_t)vt * DV + j] = (TIn)part;
                    }
                }
            }
        }
        lds_barrier();
    };
    for (int c = -2; c < nsteps - 2; ++c) step(c);
    lds_barrier();
    // final state: the stored state times the pending chunk gate is the mean
    // state; the information form multiplies it by the precision
    float* dst = SEG ? p.seg_m + ((size_t)bh * p.nseg + sp.seg) * DK * p.dv : p.etaT + (size_t)bh * DK * p.dv;
    if ((SEG || p.etaT) && nchunks > 0) {
        const int lp = (nchunks - 1) & 1;
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
            for (int jj = 0; jj < JT; ++jj) {
                const int j = vt * DV + (mw * JT + jj) * 16 + c16;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = it * 16 + 4 * g + e;
                    dst[(size_t)i * p.dv + j] = acc[it][jj][e] * sm.E[lp][i] * (SEG ? 1.f : sm.lT[i]);
                }
            }
    }
}

template <typename TIn, int DK, int DV, bool SEG, bool SCAN, bool PRO>
__global__ __launch_bounds__((P3<TIn, DK, DV>::NT)) void kla_fwd_diag_pipe_kernel(FwdArgs p) {
    static_assert(!(SCAN && PRO), "the block prologue runs with the serial chain");
    typedef P3<TIn, DK, DV> K;
    __shared__ S3<TIn, K> sm;
    __shared__ typename std::conditional<PRO, PTaps<K>, NoTaps>::type taps;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int BH = p.B * p.H, nvt = p.n_vtiles, nseg = SEG ? p.nseg : 1;
    const int nu = nvt * nseg;  // workgroups per (b,h): value tiles x segments
    int bh, u;
    {
        const int id = blockIdx.x;
        if (nu > 1 && BH % 8 == 0) {   // all workgroups of a (b,h) on one XCD
            const int x = id % 8, kx = id / 8;
            bh = (kx / nu) * 8 + x;
            u = kx % nu;
        } else {
            bh = id / nu;
            u = id % nu;
        }
    }
    const int vt = u % nvt;
    Span sp;
    sp.seg = u / nvt;
    sp.T0 = SEG ? sp.seg * p.seg_len : 0;
    sp.TL = SEG ? (p.T - sp.T0 < p.seg_len ? p.T - sp.T0 : p.seg_len) : p.T;
    sp.last = sp.seg == nseg - 1;
    if (threadIdx.x < 4) sm.bad[threadIdx.x] = 0;
    lds_barrier();
    // All roles run the same number of pipeline steps (nchunks + 2, rounded
    // up to a multiple of UNR) with one barrier each, then one more.
    // Waves w and w+4 of a workgroup share a SIMD.  The chain waves, whose
    // scan is one long dependency chain, take waves 0.. and share their SIMDs
    // with the MMA waves (4..), whose VALU load is the lightest; the gate
    // waves fill the rest and pair with each other.  The chain waves also
    // win issue ties on their SIMD.
    static_assert(K::NCW <= 4 && K::NW >= 4 + K::NMW, "wave placement");
    if (wave < K::NCW) {
        __builtin_amdgcn_s_setprio(2);
        if constexpr (SCAN) chain_role_scan<TIn, K, SEG>(sm, p, sp, bh, vt, wave, lane);
        else chain_role<TIn, K, SEG, PRO>(sm, p, sp, bh, vt, wave, lane);
    } else if (wave < 4) {
        gate_role<TIn, K, SEG, PRO>(sm, taps, p, sp, bh, vt, wave - K::NCW, lane);
    } else if (wave < 4 + K::NMW) {
        mma_role<TIn, K, SEG, PRO>(sm, p, sp, bh, vt, wave - 4, lane);
    } else {
        gate_role<TIn, K, SEG, PRO>(sm, taps, p, sp, bh, vt, 4 - K::NCW + (wave - 4 - K::NMW), lane);
    }
}

template <typename TIn, int DK, int DV, bool SCAN>
hipError_t launch_chain(const FwdArgs& a, hipStream_t s) {
    typedef P3<TIn, DK, DV> K;
    if (a.nseg > 1) {
        const int nblk = a.B * a.H * a.n_vtiles * a.nseg;
        hipLaunchKernelGGL((kla_fwd_diag_pipe_kernel<TIn, DK, DV, true, SCAN, false>), dim3(nblk), dim3(K::NT), 0,
                           s, a);
    } else {
        const int nblk = a.B * a.H * a.n_vtiles;
        hipLaunchKernelGGL((kla_fwd_diag_pipe_kernel<TIn, DK, DV, false, SCAN, false>), dim3(nblk), dim3(K::NT),
                           0, s, a);
    }
    return hipGetLastError();
}

// the serial chain by default; the wavefront-level scan chain on request
// (bf16 inputs: the fp32 build of the scan chain spills); the block prologue
// (unsplit, serial chain) when conv_w is set
template <typename TIn, int DK, int DV>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
    if constexpr (DV == 128) {
        // 128-column tiles: the plain forward only (serial chain)
        if (a.conv_w > 0 || a.chain_scan) return hipErrorInvalidValue;
        return launch_chain<TIn, DK, DV, false>(a, s);
    } else {
        if (a.conv_w > 0) {
            typedef P3<TIn, DK, DV> K;
            if (a.nseg > 1) {
                const int nblk = a.B * a.H * a.n_vtiles * a.nseg;
                hipLaunchKernelGGL((kla_fwd_diag_pipe_kernel<TIn, DK, DV, true, false, true>), dim3(nblk),
                                   dim3(K::NT), 0, s, a);
            } else {
                const int nblk = a.B * a.H * a.n_vtiles;
                hipLaunchKernelGGL((kla_fwd_diag_pipe_kernel<TIn, DK, DV, false, false, true>), dim3(nblk),
                                   dim3(K::NT), 0, s, a);
            }
            return hipGetLastError();
        }
        if constexpr (std::is_same<TIn, bf16>::value) {
            if (a.chain_scan) return launch_chain<TIn, DK, DV, true>(a, s);
        }
        return launch_chain<TIn, DK, DV, false>(a, s);
    }
}

}  // namespace

bool fwd_diag_pipe_supported(int dk, int dv, int nvt, int dtype) {
    if (dk != dv || nvt < 1 || dv % nvt) return false;
    const int dvt = dv / nvt;
    if (dvt == 128) return dk == 128 && dtype == DT_BF16;
    return dvt == 64 && (dk == 64 || (dk == 128 && dtype == DT_BF16));
}

int fwd_diag_pipe_vtiles(int dk, int dv, int dtype) {
    // 64-column tiles: measured faster than wider ones (register pressure)
    // and than 32-column tiles of the single-role kernel
    return dv % 64 == 0 && fwd_diag_pipe_supported(dk, dv, dv / 64, dtype) ? dv / 64 : 0;
}

hipError_t launch_fwd_diag_pipe(const FwdArgs& a, int dtype, hipStream_t s) {
    if (!fwd_diag_pipe_supported(a.dk, a.dv, a.n_vtiles, dtype)) return hipErrorInvalidValue;
    const int dvt = a.dv / a.n_vtiles;
    if (dtype == DT_BF16 && dvt == 128) return launch<bf16, 128, 128>(a, s);
    if (dtype == DT_BF16) return a.dk == 128 ? launch<bf16, 128, 64>(a, s) : launch<bf16, 64, 64>(a, s);
    return launch<float, 64, 64>(a, s);
}

}  // namespace kla
