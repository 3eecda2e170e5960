// kla_fwd_iso_pipe.hip -- wave-specialised, pipelined isotropic KLA forward
// for gfx950 (dk = 64 / 128, 64 value columns per workgroup).
//
// Method: "Kalman Linear Attention: Parallel Bayesian Filtering For Efficient
// Language Modelling and State Tracking" (technical summary > method §1-§3)
// with the isotropic variant of "Kalman Delta Networks: Uncertainty-aware
// Associative Memory" (abstract): one precision scalar l per head, per-token
// decay a_t and process noise qn_t, precision increment
// b_t = |k_t|^2 / (dk r_t).  The precision map l -> ((1+b qn) l + b a^2) /
// (qn l + a^2) is a 2x2 projective (Mobius) matrix, so a chunk's precisions
// come from a prefix product of matrices.  The memory runs in mean form,
// m_t = f_t m_{t-1} + c_t k_t v_t^T with f_t = a_t lp_t / l_t, c_t = 1/(r_t l_t),
// o_t = q_t^T m_t.
//
// One workgroup owns one (b,h) and 64 value columns.  Three wave roles run a
// software pipeline over chunks of C = 64 tokens with one LDS-only barrier
// per step s:
//   * staging waves (4) write chunk s's q, k rows, k^T and v^T into LDS
//     buffer s mod 2 and load chunk s+2;
//   * the scan wave (1) scans chunk s: |k_t|^2 from its own loads, the
//     Mobius prefix over the 64 tokens (DPP Hillis-Steele, one token per
//     lane), the gates and their log2 prefix Gamma, and per-token scale
//     factors for the MMA waves;
//   * MMA waves (4, 16 value columns each) finish chunk s-1: causal
//     S = K Q^T tiles scaled by c_s 2^(Gamma_t - Gamma_s), the readout
//     O = f_0 2^Gamma_t (q_t^T M) + P V, and M <- f_0 2^Gamma_end M + K^T (w V).
//
// The scale 2^(Gamma_t - Gamma_s) is split at the chunk's mid point into a
// per-t and a per-s factor (each within 2^(+-Gamma_end/2)); a chunk whose
// total log2 decay is below -200 uses exp2 of the difference per element.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kla_common.h"
#include "kla_internal.h"

namespace kla {
namespace {

template <typename TIn, int DK_, int DV_>
struct IP {
    static constexpr int DK = DK_;
    static constexpr int DV = DV_;                 // value columns per workgroup
    static constexpr int C = 64;                   // tokens per chunk
    static constexpr int NSW = 4;                  // staging waves
    static constexpr int NMW = DV / 16;            // MMA waves (16 columns each)
    // bf16 dk = 64: a P wave forms the scaled causal score tiles of a chunk
    // once, one step ahead of the MMA waves, which then read them from LDS;
    // the chunk buffers rotate over three chunks.  Otherwise every MMA wave
    // forms them itself and two chunk buffers rotate.
    static constexpr bool PW = DK == 64 && sizeof(TIn) == 2;
    static constexpr int NCB = PW ? 3 : 2;         // chunk buffers
    // matrix-core operands: fp32 as split bf16 pairs, except with 64-column
    // tiles, where the pairs' extra registers spill (measured slower)
    static constexpr bool F32MMA = sizeof(TIn) == 4 && DV == 64;
    typedef typename std::conditional<F32MMA, MmaF32, Mma<TIn>>::type M;
    typedef typename std::conditional<F32MMA, FragF32, Frag<TIn>>::type F;
    static constexpr int NW = NSW + 1 + (PW ? 1 : 0) + NMW;
    static constexpr int NT = 64 * NW;
    static constexpr int ES = (int)sizeof(TIn);
    static constexpr int PE = 16 / ES;             // row padding (16 bytes)
    static constexpr int QS = DK + PE;             // row stride of Q, K
    static constexpr int CS = C + PE;              // row stride of K^T, V^T
    static constexpr int OCT = 16 / ES;            // values per 16-byte load
    static constexpr int KOCT = DK / 8;            // 8-value groups per q/k row
    static constexpr int QKU = (C / 2) * KOCT;     // (token pair, 8-group) units
    static constexpr int QKPL = QKU / (64 * NSW);  // units per staging lane
    static constexpr int VQ = DV / 4;              // 4-value groups per v row
    static constexpr int VU = (C / 2) * VQ;
    static constexpr int VPL = VU / (64 * NSW);
    static constexpr int IT = DK / 16;
    static constexpr int NBS = DK * ES <= 128 ? 3 : 2;  // scan-wave load buffers
    static constexpr int KR = DK * ES / 16;        // 16-byte loads per k row
    static constexpr int BUFV = 4 * QKPL * (8 * ES / 4) + VPL * 2 * (4 * ES / 4);  // VGPRs per buffer
    // (at least 3: the staging waves also form the key norms of the chunk
    // after the one they stage)
    static constexpr int NSB = 120 / BUFV < 3 ? 3 : (120 / BUFV > 5 ? 5 : 120 / BUFV);
    static_assert(QKU % (64 * NSW) == 0 && VU % (64 * NSW) == 0, "unit split");
};

template <typename TIn, class K>
struct ChunkBuf {
    TIn Q[K::C][K::QS];
    TIn Kr[K::C][K::QS];
    TIn KT[K::DK][K::CS];
    TIn VT[K::DV][K::CS];
};

struct alignas(16) ScanOut {
    float e[64];      // 2^(Gamma_t - Gamma_mid)
    float ei[64];     // c_s 2^(Gamma_mid - Gamma_s)
    float fc[64];     // f_0 2^Gamma_t: decay of the incoming state at t
    float wsc[64];    // c_s 2^(Gamma_end - Gamma_s): weight of token s in the update
    float gam[64];    // Gamma_t (for chunks with a very wide decay range)
    float cs[64];     // c_s
    float fcend;      // f_0 2^Gamma_end
    int wide;         // use exp2 of Gamma differences per element
    float pad[2];
};

template <typename TIn, class K>
struct IsoSm {
    ChunkBuf<TIn, K> buf[K::NCB];
    ScanOut sc[K::NCB];
    // scaled causal score tiles (t-tile tau, s-tile sig <= tau) of a chunk as
    // MFMA B fragments, one per lane (P wave only)
    typename K::M::K16 P[K::PW ? 2 : 1][10][K::PW ? 64 : 1];
    float ksq[2][64];  // |k_t|^2 of a chunk, from the staging waves
    float lT;
};

// Value e (0..7) of an 8-value group held as 16-byte words (one word of bf16,
// two of fp32).
template <typename TIn>
__device__ __forceinline__ float get8(const f32x4* w, int e) {
    if constexpr (sizeof(TIn) == 2) return (float)__builtin_bit_cast(bf16x8, w[0])[e];
    else return w[e >> 2][e & 3];
}

// bf16 pair (value e of word a, value e of word b) from two rows held as raw
// 32-bit words: low halves for even e, high halves for odd e (one v_perm).
__device__ __forceinline__ unsigned bf16_pair(unsigned a, unsigned b, int odd) {
    return __builtin_amdgcn_perm(b, a, odd ? 0x07060302u : 0x05040100u);
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- DPP scans
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp(float old, float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                 __builtin_bit_cast(int, x), CTRL,
                                                                 ROWS, 0xF, false));
}

// One Hillis-Steele step of the inclusive prefix product P_t = M_t ... M_0
// (later tokens on the left), renormalised by the entry sum (a positive
// multiple of a Mobius matrix is the same map).
template <int CTRL, int ROWS>
__device__ __forceinline__ void mat_step(float& m00, float& m01, float& m10, float& m11) {
    const float y00 = dpp<CTRL, ROWS>(1.f, m00), y01 = dpp<CTRL, ROWS>(0.f, m01);
    const float y10 = dpp<CTRL, ROWS>(0.f, m10), y11 = dpp<CTRL, ROWS>(1.f, m11);
    const float n00 = m00 * y00 + m01 * y10, n01 = m00 * y01 + m01 * y11;
    const float n10 = m10 * y00 + m11 * y10, n11 = m10 * y01 + m11 * y11;
    const float s = fast_rcp(n00 + n01 + n10 + n11);
    m00 = n00 * s;
    m01 = n01 * s;
    m10 = n10 * s;
    m11 = n11 * s;
}

__device__ __forceinline__ void mat_scan(float& m00, float& m01, float& m10, float& m11) {
    mat_step<0x111, 0xF>(m00, m01, m10, m11);  // row_shr:1
    mat_step<0x112, 0xF>(m00, m01, m10, m11);  // row_shr:2
    mat_step<0x114, 0xF>(m00, m01, m10, m11);  // row_shr:4
    mat_step<0x118, 0xF>(m00, m01, m10, m11);  // row_shr:8
    mat_step<0x142, 0xA>(m00, m01, m10, m11);  // row_bcast:15 into rows 1, 3
    mat_step<0x143, 0xC>(m00, m01, m10, m11);  // row_bcast:31 into rows 2, 3
}

__device__ __forceinline__ float sum_scan(float x) {
    x += dpp<0x111, 0xF>(0.f, x);
    x += dpp<0x112, 0xF>(0.f, x);
    x += dpp<0x114, 0xF>(0.f, x);
    x += dpp<0x118, 0xF>(0.f, x);
    x += dpp<0x142, 0xA>(0.f, x);
    x += dpp<0x143, 0xC>(0.f, x);
    return x;
}

__device__ __forceinline__ float lane_bcast(float x, int src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), src));
}

// Pipeline steps: every role runs the same number of barrier steps.  A role
// that rotates NB register buffers runs a multiple of NB steps in its loop
// (work is guarded per step, the barrier is not), then pads to the common total.
__device__ __forceinline__ int round_up(int n, int m) { return (n + m - 1) / m * m; }

template <class K>
__device__ __forceinline__ int total_steps(int nchunks) {
    const int n = nchunks + 1 + (K::PW ? 1 : 0);  // the MMA waves finish chunk s-1 (s-2 with a P wave)
    const int a = round_up(n, K::NSB), b = round_up(n, K::NBS);
    return a > b ? a : b;
}

// Sum of x over each group of G consecutive lanes (G = 8 or 16), in every lane
// of the group.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp<0xB1, 0xF>(0.f, x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E, 0xF>(0.f, x);   // quad_perm [2,3,0,1]
    x += dpp<0x141, 0xF>(0.f, x);  // row_half_mirror
    if constexpr (G == 16) x += dpp<0x140, 0xF>(0.f, x);  // row_mirror
    return x;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    constexpr int n = N < 63 ? N : 63;
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// ------------------------------------------------------------ staging role
template <typename TIn, class K>
__device__ void stage_role(IsoSm<TIn, K>& sm, const FwdArgs& p, int bh, int vt, int sw, int lane) {
    constexpr int C = K::C, DK = K::DK, ES = K::ES;
    constexpr int WPO = 8 * ES / 16;  // 16-byte words per 8-value group
    typedef typename Quad<TIn>::V QV;
    // a 4-value group of v as raw words (register arrays of 8-byte bf16
    // vectors are not kept in registers by the compiler)
    typedef typename std::conditional<sizeof(TIn) == 2, f32x2, f32x4>::type VW;
    const int nchunks = (p.T + C - 1) / C;
    const int sl = sw * 64 + lane;
    const size_t rowbase = (size_t)bh * p.T;
    const char* qb = (const char*)((const TIn*)p.q + rowbase * DK);
    const char* kb = (const char*)((const TIn*)p.k + rowbase * DK);
    const char* vb = (const char*)((const TIn*)p.v + rowbase * p.dv);
    const int VRB = p.dv * ES;

    struct Regs {
        f32x4 q[K::QKPL][2][WPO], k[K::QKPL][2][WPO];
        VW v[K::VPL][2];
    };
    constexpr int NB = K::NSB;
    Regs r[NB];
    int qoff[K::QKPL], voff[K::VPL];
#pragma unroll
    for (int x = 0; x < K::QKPL; ++x) {
        const int u = sl + x * 64 * K::NSW, tp = u / K::KOCT, oc = u % K::KOCT;
        qoff[x] = (2 * tp * DK + 8 * oc) * ES;
    }
#pragma unroll
    for (int x = 0; x < K::VPL; ++x) {
        const int u = sl + x * 64 * K::NSW, tp = u / K::VQ, jq = u % K::VQ;
        voff[x] = 2 * tp * VRB + (vt * K::DV + 4 * jq) * ES;
    }
    auto load = [&](int c, Regs& g) {
        const int t0 = c * C, n = p.T - t0;
        const int rows = n < 0 ? 0 : (n < C ? n : C);
        const auto rq = make_rsrc(qb + (size_t)t0 * DK * ES, rows * DK * ES);
        const auto rk = make_rsrc(kb + (size_t)t0 * DK * ES, rows * DK * ES);
        const auto rv = make_rsrc(vb + (size_t)t0 * VRB, rows * VRB);
#pragma unroll
        for (int x = 0; x < K::QKPL; ++x)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int w = 0; w < WPO; ++w) {
                    g.q[x][h][w] = buf_load<f32x4>(rq, qoff[x] + h * DK * ES + 16 * w);
                    g.k[x][h][w] = buf_load<f32x4>(rk, qoff[x] + h * DK * ES + 16 * w);
                }
#pragma unroll
        for (int x = 0; x < K::VPL; ++x)
#pragma unroll
            for (int h = 0; h < 2; ++h) g.v[x][h] = buf_load<VW>(rv, voff[x] + h * VRB);
    };
    auto stage = [&](int c, const Regs& g) {
        ChunkBuf<TIn, K>& B = sm.buf[c % K::NCB];
#pragma unroll
        for (int x = 0; x < K::QKPL; ++x) {
            const int u = sl + x * 64 * K::NSW, tp = u / K::KOCT, oc = u % K::KOCT;
            const int t = 2 * tp;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int w = 0; w < WPO; ++w) {
                    *(f32x4*)&B.Q[t + h][8 * oc + w * (16 / ES)] = g.q[x][h][w];
                    *(f32x4*)&B.Kr[t + h][8 * oc + w * (16 / ES)] = g.k[x][h][w];
                }
            if constexpr (sizeof(TIn) == 2) {
                const u32x4 k0 = __builtin_bit_cast(u32x4, g.k[x][0][0]);
                const u32x4 k1 = __builtin_bit_cast(u32x4, g.k[x][1][0]);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *(unsigned*)&B.KT[8 * oc + e][t] = bf16_pair(k0[e >> 1], k1[e >> 1], e & 1);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *(typename Pair<TIn>::V*)&B.KT[8 * oc + e][t] =
                        Pair<TIn>::make(get8<TIn>(g.k[x][0], e), get8<TIn>(g.k[x][1], e));
            }
        }
#pragma unroll
        for (int x = 0; x < K::VPL; ++x) {
            const int u = sl + x * 64 * K::NSW, tp = u / K::VQ, jq = u % K::VQ;
            if constexpr (sizeof(TIn) == 2) {
                const u32x2 v0 = __builtin_bit_cast(u32x2, g.v[x][0]);
                const u32x2 v1 = __builtin_bit_cast(u32x2, g.v[x][1]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *(unsigned*)&B.VT[4 * jq + e][2 * tp] = bf16_pair(v0[e >> 1], v1[e >> 1], e & 1);
            } else {
                const f32x4 v0 = Quad<TIn>::to_f32(__builtin_bit_cast(QV, g.v[x][0]));
                const f32x4 v1 = Quad<TIn>::to_f32(__builtin_bit_cast(QV, g.v[x][1]));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *(typename Pair<TIn>::V*)&B.VT[4 * jq + e][2 * tp] = Pair<TIn>::make(v0[e], v1[e]);
            }
        }
    };
    // |k_t|^2 of chunk c for the scan wave: each unit sums its 8 dims of two
    // tokens, the KOCT units of a token pair are consecutive lanes
    auto norms = [&](int c, const Regs& g) {
        float* ks = sm.ksq[c & 1];
#pragma unroll
        for (int x = 0; x < K::QKPL; ++x) {
            const int u = sl + x * 64 * K::NSW, tp = u / K::KOCT, oc = u % K::KOCT;
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float k0 = get8<TIn>(g.k[x][0], e), k1 = get8<TIn>(g.k[x][1], e);
                s0 = __builtin_fmaf(k0, k0, s0);
                s1 = __builtin_fmaf(k1, k1, s1);
            }
            s0 = group_sum<K::KOCT>(s0);
            s1 = group_sum<K::KOCT>(s1);
            if (oc == 0) *(f32x2*)&ks[2 * tp] = f32x2{s0, s1};
        }
    };
    static_assert(K::KOCT == 8 || K::KOCT == 16, "key-norm groups");
    static_assert(NB >= 3, "the next chunk's rows must be loaded a step ahead");
    constexpr int NLD = 4 * WPO * K::QKPL + 2 * K::VPL;
#pragma unroll
    for (int j = 0; j < NB - 1; ++j) load(j, r[j]);
    // chunk 0's norms before the pipeline's first step (all roles pass one
    // extra barrier here)
    wait_vm<(NB - 2) * NLD>();
    norms(0, r[0]);
    lds_barrier();
    // step s stages chunk s from buffer s mod NB, forms the norms of chunk
    // s+1 and loads chunk s+NB-1
    const int nloop = round_up(nchunks + 1, NB);
    for (int s0 = 0; s0 < nloop; s0 += NB) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int s = s0 + j;
            wait_vm<(NB - 3) * NLD>();
            if (s < nchunks) stage(s, r[j]);
            if (s + 1 < nchunks) norms(s + 1, r[(j + 1) % NB]);
            load(s + NB - 1, r[(j + NB - 1) % NB]);
            lds_barrier();
        }
    }
    for (int s = nloop; s < total_steps<K>(nchunks); ++s) lds_barrier();
}

// ---------------------------------------------------------------- scan role
template <typename TIn, class K>
__device__ void scan_role(IsoSm<TIn, K>& sm, const FwdArgs& p, int bh, int vt, int lane) {
    constexpr int C = K::C, DK = K::DK, NB = K::NBS;
    const int nchunks = (p.T + C - 1) / C;
    const size_t rowbase = (size_t)bh * p.T;
    const char* ab = (const char*)(p.a + rowbase);
    const char* qnb = (const char*)(p.qn + rowbase);
    const char* rb = (const char*)(p.r + rowbase);

    struct Regs {
        float a, qn, r;
    };
    Regs rg[NB];
    auto load = [&](int c, Regs& g) {
        const int t0 = c * C, n = p.T - t0;
        const int rows = n < 0 ? 0 : (n < C ? n : C);
        g.a = buf_load<float>(make_rsrc(ab + (size_t)t0 * 4, rows * 4), lane * 4);
        g.qn = buf_load<float>(make_rsrc(qnb + (size_t)t0 * 4, rows * 4), lane * 4);
        g.r = buf_load<float>(make_rsrc(rb + (size_t)t0 * 4, rows * 4), lane * 4);
    };
    float lc = p.l0 ? p.l0[bh] : 1.f;
    auto scan = [&](int c, const Regs& g) {
        ScanOut& o = sm.sc[c % K::NCB];
        const int t = lane;
        const int L = (p.T - c * C) < C ? (p.T - c * C) : C;
        const bool in = t < L;
        const float ksq = sm.ksq[c & 1][t];  // from the staging waves
        const float rho = in ? 1.f / g.r : 0.f;
        const float b = ksq * rho * (1.f / (float)DK);
        const float a2 = g.a * g.a;
        float m00 = in ? __builtin_fmaf(b, g.qn, 1.f) : 1.f, m01 = in ? b * a2 : 0.f;
        float m10 = in ? g.qn : 0.f, m11 = in ? a2 : 1.f;
        mat_scan(m00, m01, m10, m11);
        const float lt = __builtin_fmaf(m00, lc, m01) / __builtin_fmaf(m10, lc, m11);
        const float lprev = dpp<0x138, 0xF>(lc, lt);  // wave_shr:1, lane 0 gets the carry
        const float lp = lprev * fast_rcp(__builtin_fmaf(g.qn, lprev, a2));
        const float rl = fast_rcp(lt);
        const float f = in ? g.a * lp * rl : 1.f;
        const float cc = rho * rl;
        const float gam = sum_scan((in && t >= 1) ? fast_log2(f) : 0.f);
        const float gend = lane_bcast(gam, L - 1);
        const float f0 = lane_bcast(f, 0);
        const float gmid = 0.5f * gend;
        o.e[t] = fast_exp2(gam - gmid);
        o.ei[t] = cc * fast_exp2(gmid - gam);
        o.fc[t] = f0 * fast_exp2(gam);
        o.wsc[t] = cc * fast_exp2(gend - gam);
        o.gam[t] = gam;
        o.cs[t] = cc;
        if (lane == 0) {
            o.fcend = f0 * fast_exp2(gend);
            o.wide = gend < -200.f;
        }
        lc = lane_bcast(lt, L - 1);
    };
    constexpr int NLD = 3;
#pragma unroll
    for (int j = 0; j < NB - 1; ++j) load(j, rg[j]);
    lds_barrier();  // chunk 0's key norms
    const int nloop = round_up(nchunks + 1, NB);
    for (int s0 = 0; s0 < nloop; s0 += NB) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int s = s0 + j;
            wait_vm<(NB - 2) * NLD>();
            if (s < nchunks) scan(s, rg[j]);
            load(s + NB - 1, rg[(j + NB - 1) % NB]);
            lds_barrier();
        }
    }
    for (int s = nloop; s < total_steps<K>(nchunks); ++s) lds_barrier();
    if (lane == 0) sm.lT = lc;
    if (p.lT && vt == 0 && lane == 0) p.lT[bh] = lc;
    lds_barrier();
}

// Scaled causal score tiles of token tile tau of a chunk: for every s-tile
// sig <= tau, S[s,t] = k_s . q_t times c_s 2^(Gamma_t - Gamma_s), zero for
// s > t, as K=16 MFMA B fragments.  kfrag(sig, kk) gives the K=32 fragment of
// k rows sig*16.. at dims kk*32..; Qf the q fragments of the tile's tokens.
template <typename TIn, class K, bool WIDE, class KF>
__device__ __forceinline__ void score_tiles(const ScanOut& so, KF kfrag,
                                            const typename K::F::V (&Qf)[K::DK / 32], int tau,
                                            int c16, int g, typename K::M::K16 (&P)[K::C / 16]) {
    typedef typename K::F F;
    typedef typename K::M M;
    constexpr int KB = K::DK / 32, NT16 = K::C / 16;
    const int t = tau * 16 + c16;
    f32x4 S[NT16];
#pragma unroll
    for (int sig = 0; sig <= tau; ++sig) {
        S[sig] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) S[sig] = F::mma(kfrag(sig, kk), Qf[kk], S[sig]);
    }
    const float et = so.e[t], gt = so.gam[t];
#pragma unroll
    for (int sig = 0; sig <= tau; ++sig) {
        f32x4 sv = S[sig];
        if constexpr (!WIDE) {
            const f32x4 ei = *(const f32x4*)&so.ei[sig * 16 + 4 * g];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = sv[e] * ei[e] * et;
                sv[e] = (sig < tau || 4 * g + e <= c16) ? v : 0.f;
            }
        } else {
            const f32x4 gs = *(const f32x4*)&so.gam[sig * 16 + 4 * g];
            const f32x4 cs = *(const f32x4*)&so.cs[sig * 16 + 4 * g];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = sv[e] * cs[e] * fast_exp2(gt - gs[e]);
                sv[e] = (sig < tau || 4 * g + e <= c16) ? v : 0.f;
            }
        }
        P[sig] = M::from_acc(sv);
    }
}

// ------------------------------------------------------------------- P role
// With PW: step s forms the score tiles of chunk s-1 into P[(s-1) & 1].
template <typename TIn, class K>
__device__ void p_role(IsoSm<TIn, K>& sm, const FwdArgs& p, int lane) {
    typedef typename K::F F;
    typedef typename F::V FV;
    constexpr int C = K::C, DK = K::DK, KB = DK / 32, NT16 = C / 16;
    const int nchunks = (p.T + C - 1) / C;
    const int c16 = lane & 15, g = lane >> 4;
    auto pchunk = [&](int c, auto wide_t) {
        constexpr bool WIDE = decltype(wide_t)::value;
        const ChunkBuf<TIn, K>& B = sm.buf[c % K::NCB];
        const ScanOut& so = sm.sc[c % K::NCB];
        typename K::M::K16(*out)[64] = sm.P[c & 1];
        FV Kf[NT16][KB];
#pragma unroll
        for (int sig = 0; sig < NT16; ++sig)
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) Kf[sig][kk] = F::ld(&B.Kr[sig * 16 + c16][kk * 32], g);
#pragma unroll
        for (int tau = 0; tau < NT16; ++tau) {
            FV Qf[KB];
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) Qf[kk] = F::ld(&B.Q[tau * 16 + c16][kk * 32], g);
            typename K::M::K16 P[NT16];
            score_tiles<TIn, K, WIDE>(so, [&](int sig, int kk) { return Kf[sig][kk]; }, Qf, tau, c16, g, P);
#pragma unroll
            for (int sig = 0; sig <= tau; ++sig) out[tau * (tau + 1) / 2 + sig][lane] = P[sig];
        }
    };
    lds_barrier();  // chunk 0's key norms
    for (int s = 0; s < total_steps<K>(nchunks); ++s) {
        if (s >= 1 && s <= nchunks) {
            if (__builtin_amdgcn_readfirstlane(sm.sc[(s - 1) % K::NCB].wide)) pchunk(s - 1, std::true_type{});
            else pchunk(s - 1, std::false_type{});
        }
        lds_barrier();
    }
    lds_barrier();
}

// ----------------------------------------------------------------- MMA role
template <typename TIn, class K>
__device__ void mma_role(IsoSm<TIn, K>& sm, const FwdArgs& p, int bh, int vt, int mw, int lane) {
    typedef typename K::M M;
    constexpr int C = K::C, DK = K::DK, IT = K::IT;
    const int nchunks = (p.T + C - 1) / C;
    const int c16 = lane & 15, g = lane >> 4;
    const int jrow = mw * 16 + c16;                 // this lane's value column in the tile
    const size_t rowbase = (size_t)bh * p.T;
    TIn* op = (TIn*)p.o;

    f32x4 accM[IT];
    {
        const float il = p.l0 ? 1.f / p.l0[bh] : 1.f;
        const int j = vt * K::DV + jrow;
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = it * 16 + 4 * g + e;
                accM[it][e] = p.eta0 ? p.eta0[((size_t)bh * DK + i) * p.dv + j] * il : 0.f;
            }
    }

    auto chunk = [&](int c, auto wide_t) {
        constexpr bool WIDE = decltype(wide_t)::value;
        typedef typename K::F F;
        typedef typename F::V FV;
        constexpr int KB = DK / 32, NT16 = C / 16;
        constexpr bool KHOIST = DK <= 64;  // keep every K tile's fragments in registers
        const ChunkBuf<TIn, K>& B = sm.buf[c % K::NCB];
        const ScanOut& so = sm.sc[c % K::NCB];
        const int t0 = c * C;
        const int L = (p.T - t0) < C ? (p.T - t0) : C;
        // o rows of this chunk, range-checked so rows past T are not written
        const auto ro = make_rsrc(op + (rowbase + t0) * p.dv, L * p.dv * (int)sizeof(TIn));
        // the incoming state as K=32 A operands (two accumulator tiles each)
        FV AM[KB];
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) AM[kk] = F::from_acc(accM[2 * kk], accM[2 * kk + 1]);
        FV Kf[KHOIST && !K::PW ? NT16 : 1][KB];
        if constexpr (KHOIST && !K::PW) {
#pragma unroll
            for (int sig = 0; sig < NT16; ++sig)
#pragma unroll
                for (int kk = 0; kk < KB; ++kk) Kf[sig][kk] = F::ld(&B.Kr[sig * 16 + c16][kk * 32], g);
        }
#pragma unroll
        for (int tau = 0; tau < NT16; ++tau) {
            const int t = tau * 16 + c16;
            FV Qf[KB];
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) Qf[kk] = F::ld(&B.Q[t][kk * 32], g);
            // the state readout and the scaled causal score tiles
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) acc = F::mma(AM[kk], Qf[kk], acc);
            typename M::K16 P[NT16];
            if constexpr (K::PW) {
#pragma unroll
                for (int sig = 0; sig <= tau; ++sig) P[sig] = sm.P[c & 1][tau * (tau + 1) / 2 + sig][lane];
            } else {
                score_tiles<TIn, K, WIDE>(
                    so,
                    [&](int sig, int kk) {
                        if constexpr (KHOIST) return Kf[KHOIST ? sig : 0][kk];
                        else return F::ld(&B.Kr[sig * 16 + c16][kk * 32], g);
                    },
                    Qf, tau, c16, g, P);
            }
            acc *= so.fc[t];
#pragma unroll
            for (int sig = 0; sig <= tau; ++sig)
                acc = M::mma16(M::ld16(&B.VT[jrow][sig * 16 + 4 * g]), P[sig], acc);
            buf_store(Quad<TIn>::make(acc), ro,
                      (t * p.dv + vt * K::DV + mw * 16 + 4 * g) * (int)sizeof(TIn));
        }
        // state update: M <- fcend M + K^T diag(wsc) V
        const float fe = so.fcend;
#pragma unroll
        for (int it = 0; it < IT; ++it) accM[it] *= fe;
#pragma unroll
        for (int kb = 0; kb < C / 32; ++kb) {
            const f32x4 w0 = *(const f32x4*)&so.wsc[kb * 32 + 8 * g];
            const f32x4 w1 = *(const f32x4*)&so.wsc[kb * 32 + 8 * g + 4];
            typename M::K32 vf;
            if constexpr (sizeof(TIn) == 2) {
                vf = M::ld32(&B.VT[jrow][kb * 32 + 8 * g]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vf[e] = (bf16)((float)vf[e] * w0[e]);
                    vf[e + 4] = (bf16)((float)vf[e + 4] * w1[e]);
                }
            } else {
                const float* vr = &B.VT[jrow][kb * 32 + 8 * g];
                vf = M::make32(*(const f32x4*)vr * w0, *(const f32x4*)(vr + 4) * w1);
            }
#pragma unroll
            for (int it = 0; it < IT; ++it)
                accM[it] = M::mma32(M::ld32(&B.KT[it * 16 + c16][kb * 32 + 8 * g]), vf, accM[it]);
        }
    };
    constexpr int LAG = K::PW ? 2 : 1;  // chunk finished in step s: s - LAG
    lds_barrier();                      // chunk 0's key norms
    for (int s = 0; s < total_steps<K>(nchunks); ++s) {
        if (s >= LAG && s < nchunks + LAG) {
            if (K::PW) chunk(s - LAG, std::false_type{});  // the P wave handled the range
            else if (__builtin_amdgcn_readfirstlane(sm.sc[(s - LAG) % K::NCB].wide))
                chunk(s - LAG, std::true_type{});
            else
                chunk(s - LAG, std::false_type{});
        }
        lds_barrier();
    }
    lds_barrier();
    if (p.etaT) {
        const float lT = sm.lT;
        const int j = vt * K::DV + jrow;
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = it * 16 + 4 * g + e;
                p.etaT[((size_t)bh * DK + i) * p.dv + j] = accM[it][e] * lT;
            }
    }
}

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__((IP<TIn, DK, DV>::NT)) void kla_fwd_iso_pipe_kernel(FwdArgs p) {
    typedef IP<TIn, DK, DV> K;
    __shared__ IsoSm<TIn, K> sm;
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
    // Every role runs total_steps() pipeline steps with one barrier each,
    // then one more barrier before the final state is read.
    if (wave < K::NSW) {
        stage_role<TIn, K>(sm, p, bh, vt, wave, lane);
        lds_barrier();
    } else if (wave == K::NSW) {
        scan_role<TIn, K>(sm, p, bh, vt, lane);
    } else {
        if constexpr (K::PW) {
            if (wave == K::NSW + 1) {
                p_role<TIn, K>(sm, p, lane);
                return;
            }
        }
        mma_role<TIn, K>(sm, p, bh, vt, wave - K::NSW - 1 - (K::PW ? 1 : 0), lane);
    }
}

template <typename TIn, int DK, int DV>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
    typedef IP<TIn, DK, DV> K;
    const int nblk = a.B * a.H * a.n_vtiles;
    hipLaunchKernelGGL((kla_fwd_iso_pipe_kernel<TIn, DK, DV>), dim3(nblk), dim3(K::NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool fwd_iso_pipe_supported(int dk, int dv, int nvt, int dtype) {
    if (dk != dv || nvt < 1 || dv % nvt) return false;
    const int dvt = dv / nvt;
    if (dvt != 64 && dvt != 32) return false;
    return dtype == DT_BF16 ? (dk == 64 || dk == 128) : dk == 64;
}

int fwd_iso_pipe_vtiles(int B, int H, int dk, int dv) {
    // 32-column tiles when 64-column tiles would leave most CUs idle
    const long long bh = (long long)B * H;
    return (bh * (dv / 64) < 256 && dk <= 64) ? dv / 32 : dv / 64;
}

hipError_t launch_fwd_iso_pipe(const FwdArgs& a, int dtype, hipStream_t s) {
    if (!fwd_iso_pipe_supported(a.dk, a.dv, a.n_vtiles, dtype)) return hipErrorInvalidValue;
    const bool wide = a.dv / a.n_vtiles == 64;
    if (dtype == DT_BF16) {
        if (a.dk == 64) return wide ? launch<bf16, 64, 64>(a, s) : launch<bf16, 64, 32>(a, s);
        return wide ? launch<bf16, 128, 64>(a, s) : launch<bf16, 128, 32>(a, s);
    }
    return wide ? launch<float, 64, 64>(a, s) : launch<float, 64, 32>(a, s);
}

}  // namespace kla
