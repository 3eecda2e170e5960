// kla_fwd_iso.hip -- gfx950 forward kernel, isotropic precision.
//
// Sources: "Kalman Delta Networks: Uncertainty-aware Associative Memory"
// (abstract: isotropic variant, one uncertainty scalar per head, Mobius
// uncertainty recurrence with an associative scan) and "Kalman Linear
// Attention: Parallel Bayesian Filtering For Efficient Language Modelling and
// State Tracking" (gist.science explainer, method §2: the precision map is a
// Mobius transformation, compositions are associative, so the precision path
// is a parallel prefix scan; the mean update is affine once it is known).
//
// Per (b,h) the precision is one scalar: l -> ((1 + b qn) l + b a^2)/(qn l + a^2)
// with per-token a_t, qn_t and b_t = |k_t|^2 / (d_k r_t).  One wave scans a
// 64-token chunk: lane t forms the 2x2 map M_t, a Hillis-Steele scan over the
// lanes gives the prefix products P_t = M_t ... M_0 (renormalised: the map is
// projective), and l_t = P_t(l_carry).  Only one evaluation per chunk sits on
// the sequential path.  The mean m = eta / l then follows
//   m_t = f_t m_{t-1} + c_t k_t v_t^T,  f = a lp / l_t,  c = 1 / (r_t l_t),
// with a scalar gate per token, so the chunk's decay matrix
// D[s,t] = prod_{u=s+1..t} f_u = exp2(Gamma_t - Gamma_s) is formed entry-wise
// (every entry <= 1, no range problem) and q, k feed the MFMA unscaled.
// The barriers order LDS only, so the next chunk's loads stay in flight
// across them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kla_common.h"
#include "kla_internal.h"

namespace kla {
namespace {

template <typename TIn, int DK_, int DV_>
struct IsoCfg {
    static constexpr int DK = DK_;
    static constexpr int DV = DV_;             // value columns owned by the workgroup
    static constexpr int C = 64;               // tokens per chunk = one wave of lanes
    static constexpr int NW = DV / 16;         // one 16-column tile per wave
    static constexpr int NT = NW * 64;
    static constexpr int IT = DK / 16;
    static constexpr int NB = C / 16;
    static constexpr int PE = 16 / (int)sizeof(TIn);
    static constexpr int QS = DK + PE;
    static constexpr int CS = C + PE;
    static constexpr int KOCT = DK / 8;        // 8-value units per q/k row
    static constexpr int KUNITS = C * KOCT;
    static constexpr int KPT = (KUNITS + NT - 1) / NT;
    static constexpr int VQ = DV / 4;
    static constexpr int VUNITS = (C / 2) * VQ;
    static constexpr int VPT = (VUNITS + NT - 1) / NT;
    static constexpr int TUNITS = (C / 2) * KOCT;  // (token pair, key oct) for K~^T
    static constexpr int TPT = (TUNITS + NT - 1) / NT;
    static_assert(NW >= 1 && NW <= 4, "1..4 waves");
    static_assert(64 % KOCT == 0 && NT % KOCT == 0, "k^2 reduction stays inside a wave");
};

template <typename TIn, class K>
struct IsoSmem {
    TIn Q[K::C][K::QS];
    TIn Kk[K::C][K::QS];
    TIn KT[K::DK][K::CS];   // k_s[i] * c_s * D[s, end]
    TIn VT[K::DV][K::CS];
    float ksq[K::C];        // |k_t|^2
    float gam[K::C];        // Gamma_t = sum_{u=1..t} log2 f_u
    float cs[K::C];         // c_t = 1/(r_t l_t), zero past the chunk end
    float fc[K::C];         // f_0 * exp2(Gamma_t): state decay seen by token t
    float ksc[K::C];        // c_t * exp2(Gamma_end - Gamma_t)
    float fcend;            // f_0 * exp2(Gamma_end)
    float lcar;             // precision carry
};

template <typename TIn, class K>
struct IsoRegs {
    typename Oct<TIn>::V q[K::KPT];
    typename Oct<TIn>::V k[K::KPT];
    typename Quad<TIn>::V v[K::VPT][2];
    float a, qn, r;         // per-token scalars (wave 0, lane = token)
};

template <typename TIn, class K>
__device__ __forceinline__ void iso_load(IsoRegs<TIn, K>& R, const FwdArgs& p, int bh, int vt,
                                         int t0, int L, int tid) {
    typedef typename Oct<TIn>::V O8;
    const TIn* q = (const TIn*)p.q;
    const TIn* k = (const TIn*)p.k;
    const TIn* v = (const TIn*)p.v;
    const size_t row0 = (size_t)bh * p.T + t0;
#pragma unroll
    for (int x = 0; x < K::KPT; ++x) {
        const int unit = tid + x * K::NT;
        const int t = unit / K::KOCT, oc = unit % K::KOCT;
        if (unit < K::KUNITS && t < L) {
            const size_t off = (row0 + t) * K::DK + 8 * oc;
            R.q[x] = *(const O8*)(q + off);
            R.k[x] = *(const O8*)(k + off);
        } else {
            R.q[x] = Oct<TIn>::zero();
            R.k[x] = Oct<TIn>::zero();
        }
    }
#pragma unroll
    for (int x = 0; x < K::VPT; ++x) {
        const int unit = tid + x * K::NT;
        const int tp = unit / K::VQ, jq = unit % K::VQ;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int t = 2 * tp + h2;
            if (unit < K::VUNITS && t < L) {
                const size_t off = (row0 + t) * p.dv + (size_t)vt * K::DV + 4 * jq;
                R.v[x][h2] = *(const typename Quad<TIn>::V*)(v + off);
            } else {
                R.v[x][h2] = Quad<TIn>::zero();
            }
        }
    }
    if (tid < K::C) {
        const bool in = tid < L;
        R.a = in ? p.a[row0 + tid] : 1.f;
        R.qn = in ? p.qn[row0 + tid] : 0.f;
        R.r = in ? p.r[row0 + tid] : 1.f;
    }
}

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__((IsoCfg<TIn, DK, DV>::NT)) void kla_fwd_iso_kernel(FwdArgs p) {
    typedef IsoCfg<TIn, DK, DV> K;
    typedef MmaFor<TIn, K::DK> M;
    __shared__ IsoSmem<TIn, K> sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4;

    const int BH = p.B * p.H, nvt = p.n_vtiles;
    int bh, vt;
    {
        const int id = blockIdx.x;
        if (nvt > 1 && BH % 8 == 0) {   // keep the value tiles of one (b,h) on one XCD
            const int x = id % 8, kx = id / 8;
            bh = (kx / nvt) * 8 + x;
            vt = kx % nvt;
        } else {
            bh = id / nvt;
            vt = id % nvt;
        }
    }

    if (tid == 0) sm.lcar = p.l0 ? p.l0[bh] : 1.f;
    lds_barrier();
    // state m0 = eta0 / l0, wave owns value tile `wave`: lane holds rows 4g+e, column c16
    f32x4 accM[K::IT];
    {
        const float il = 1.f / sm.lcar;
        const int j = vt * DV + wave * 16 + c16;
#pragma unroll
        for (int it = 0; it < K::IT; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = it * 16 + 4 * g + e;
                accM[it][e] = p.eta0 ? p.eta0[((size_t)bh * DK + i) * p.dv + j] * il : 0.f;
            }
    }

    IsoRegs<TIn, K> cur;
    if (p.T > 0) iso_load<TIn, K>(cur, p, bh, vt, 0, p.T < K::C ? p.T : K::C, tid);

    for (int t0 = 0; t0 < p.T; t0 += K::C) {
        const int L = (p.T - t0) < K::C ? (p.T - t0) : K::C;

        // ---- stage q, k rows, V^T, |k_t|^2
#pragma unroll
        for (int x = 0; x < K::KPT; ++x) {
            const int unit = tid + x * K::NT;
            const int t = unit / K::KOCT, oc = unit % K::KOCT;
            float s = 0.f;
            if (unit < K::KUNITS) {
                *(typename Oct<TIn>::V*)&sm.Q[t][8 * oc] = cur.q[x];
                *(typename Oct<TIn>::V*)&sm.Kk[t][8 * oc] = cur.k[x];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float kv = Oct<TIn>::get(cur.k[x], e);
                    s += kv * kv;
                }
            }
#pragma unroll
            for (int m = 1; m < K::KOCT; m <<= 1) s += __shfl_xor(s, m, 64);
            if (unit < K::KUNITS && oc == 0) sm.ksq[t] = s;
        }
#pragma unroll
        for (int x = 0; x < K::VPT; ++x) {
            const int unit = tid + x * K::NT;
            if (unit < K::VUNITS) {
                const int tp = unit / K::VQ, jq = unit % K::VQ;
                const f32x4 v0 = Quad<TIn>::to_f32(cur.v[x][0]);
                const f32x4 v1 = Quad<TIn>::to_f32(cur.v[x][1]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *(typename Pair<TIn>::V*)&sm.VT[4 * jq + e][2 * tp] = Pair<TIn>::make(v0[e], v1[e]);
            }
        }
        const float a_t = cur.a, qn_t = cur.qn, r_t = cur.r;
        IsoRegs<TIn, K> nxt;
        const int t0n = t0 + K::C;
        if (t0n < p.T) iso_load<TIn, K>(nxt, p, bh, vt, t0n, (p.T - t0n) < K::C ? (p.T - t0n) : K::C, tid);
        lds_barrier();

        // ---- precision scan and gates: wave 0, lane = token
        if (wave == 0) {
            const int t = lane;
            const bool in = t < L;
            const float rho = 1.f / r_t;
            const float b = sm.ksq[t] * rho * (1.f / (float)DK);
            const float a2 = a_t * a_t;
            float m00 = in ? 1.f + b * qn_t : 1.f, m01 = in ? b * a2 : 0.f;
            float m10 = in ? qn_t : 0.f, m11 = in ? a2 : 1.f;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const float o00 = __shfl_up(m00, d, 64), o01 = __shfl_up(m01, d, 64);
                const float o10 = __shfl_up(m10, d, 64), o11 = __shfl_up(m11, d, 64);
                if (lane >= d) {
                    const float n00 = m00 * o00 + m01 * o10, n01 = m00 * o01 + m01 * o11;
                    const float n10 = m10 * o00 + m11 * o10, n11 = m10 * o01 + m11 * o11;
                    const float s = fast_rcp(n00 + n01 + n10 + n11);
                    m00 = n00 * s; m01 = n01 * s; m10 = n10 * s; m11 = n11 * s;
                }
            }
            const float lc = sm.lcar;
            const float lt = (m00 * lc + m01) / (m10 * lc + m11);
            float lprev = __shfl_up(lt, 1, 64);
            if (lane == 0) lprev = lc;
            const float lp = lprev / __builtin_fmaf(qn_t, lprev, a2);
            const float rl = 1.f / lt;
            const float f = a_t * lp * rl;
            const float c = in ? rho * rl : 0.f;
            float x = (in && t >= 1) ? fast_log2(f) : 0.f;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const float y = __shfl_up(x, d, 64);
                if (lane >= d) x += y;
            }
            const float gend = __shfl(x, L - 1, 64);
            const float f0 = __shfl(f, 0, 64);
            sm.gam[t] = x;
            sm.cs[t] = c;
            sm.fc[t] = f0 * fast_exp2(x);
            sm.ksc[t] = in ? c * fast_exp2(gend - x) : 0.f;
            const float lend = __shfl(lt, L - 1, 64);
            if (lane == 0) {
                sm.fcend = f0 * fast_exp2(gend);
                sm.lcar = lend;
            }
        }
        lds_barrier();

        // ---- K~^T[i][s] = k_s[i] * c_s * exp2(Gamma_end - Gamma_s)
#pragma unroll
        for (int x = 0; x < K::TPT; ++x) {
            const int unit = tid + x * K::NT;
            if (unit < K::TUNITS) {
                const int sp = unit / K::KOCT, oc = unit % K::KOCT;
                const int s0 = 2 * sp;
                const float k0 = sm.ksc[s0], k1 = sm.ksc[s0 + 1];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x0 = (float)sm.Kk[s0][8 * oc + e] * k0;
                    const float x1 = (float)sm.Kk[s0 + 1][8 * oc + e] * k1;
                    *(typename Pair<TIn>::V*)&sm.KT[8 * oc + e][s0] = Pair<TIn>::make(x0, x1);
                }
            }
        }
        lds_barrier();

        // ---- MFMA: readout and state update for this wave's value tile
        typename M::K16 AM[K::IT];
#pragma unroll
        for (int it = 0; it < K::IT; ++it) AM[it] = M::from_acc(accM[it]);
        const int jrow = wave * 16 + c16;
        const int nblk = (L + 15) / 16;
        for (int tau = 0; tau < nblk; ++tau) {
            const int t = tau * 16 + c16;
            const float gt = sm.gam[t];
            typename M::K16 P[K::NB];
#pragma unroll
            for (int sig = 0; sig < K::NB; ++sig) {
                if (sig > tau) continue;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if constexpr (DK >= 32) {
#pragma unroll
                    for (int kk = 0; kk < DK / 32; ++kk)
                        acc = M::mma32(M::ld32(&sm.Kk[sig * 16 + c16][kk * 32 + 8 * g]),
                                       M::ld32(&sm.Q[tau * 16 + c16][kk * 32 + 8 * g]), acc);
                } else {
                    acc = M::mma16(M::ld16(&sm.Kk[sig * 16 + c16][4 * g]),
                                   M::ld16(&sm.Q[tau * 16 + c16][4 * g]), acc);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = sig * 16 + 4 * g + e;
                    acc[e] = (s <= t) ? acc[e] * sm.cs[s] * fast_exp2(gt - sm.gam[s]) : 0.f;
                }
                P[sig] = M::from_acc(acc);
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int it = 0; it < K::IT; ++it)
                acc = M::mma16(AM[it], M::ld16(&sm.Q[tau * 16 + c16][it * 16 + 4 * g]), acc);
            acc *= sm.fc[t];
#pragma unroll
            for (int sig = 0; sig < K::NB; ++sig) {
                if (sig > tau) continue;
                acc = M::mma16(M::ld16(&sm.VT[jrow][sig * 16 + 4 * g]), P[sig], acc);
            }
            if (t < L) {
                TIn* o = (TIn*)p.o;
                const size_t off = ((size_t)bh * p.T + t0 + t) * p.dv + (size_t)vt * DV + wave * 16 + 4 * g;
                *(typename Quad<TIn>::V*)(o + off) = Quad<TIn>::make(acc);
            }
        }
        const float fe = sm.fcend;
#pragma unroll
        for (int it = 0; it < K::IT; ++it) {
            accM[it] *= fe;
#pragma unroll
            for (int sc = 0; sc < K::C / 32; ++sc)
                accM[it] = M::mma32(M::ld32(&sm.KT[it * 16 + c16][sc * 32 + 8 * g]),
                                    M::ld32(&sm.VT[jrow][sc * 32 + 8 * g]), accM[it]);
        }
        lds_barrier();
        cur = nxt;
    }

    if (p.etaT) {
        const float lT = sm.lcar;
        const int j = vt * DV + wave * 16 + c16;
#pragma unroll
        for (int it = 0; it < K::IT; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = it * 16 + 4 * g + e;
                p.etaT[((size_t)bh * DK + i) * p.dv + j] = accM[it][e] * lT;
            }
    }
    if (p.lT && vt == 0 && tid == 0) p.lT[bh] = sm.lcar;
}

template <typename TIn, int DK, int DV>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
    typedef IsoCfg<TIn, DK, DV> K;
    const int nblk = a.B * a.H * a.n_vtiles;
    hipLaunchKernelGGL((kla_fwd_iso_kernel<TIn, DK, DV>), dim3(nblk), dim3(K::NT), 0, s, a);
    return hipGetLastError();
}

template <typename TIn>
hipError_t dispatch(const FwdArgs& a, hipStream_t s) {
    const int dvt = a.dv / a.n_vtiles;
    if (a.dk != a.dv) return hipErrorInvalidValue;
    switch (a.dk) {
        case 16: if (dvt == 16) return launch<TIn, 16, 16>(a, s); break;
        case 32:
            if (dvt == 32) return launch<TIn, 32, 32>(a, s);
            if (dvt == 16) return launch<TIn, 32, 16>(a, s);
            break;
        case 64:
            if (dvt == 64) return launch<TIn, 64, 64>(a, s);
            if (dvt == 32) return launch<TIn, 64, 32>(a, s);
            if (dvt == 16) return launch<TIn, 64, 16>(a, s);
            break;
        case 128:
            if (dvt == 64) return launch<TIn, 128, 64>(a, s);
            if (dvt == 32) return launch<TIn, 128, 32>(a, s);
            if (dvt == 16) return launch<TIn, 128, 16>(a, s);
            break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool fwd_iso_supported(int dk, int dv, int dtype) {
    (void)dtype;
    return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}

int fwd_iso_vtiles(int B, int H, int dk) {
    const long long bh = (long long)B * H;
    int nvt = dk > 64 ? dk / 64 : 1;                      // at most 64 columns per workgroup
    while (bh * nvt < 512 && dk / (nvt * 2) >= 16) nvt *= 2;  // fill the CUs
    return nvt;
}

hipError_t launch_fwd_iso(const FwdArgs& a, int dtype, hipStream_t s) {
    return dtype == DT_BF16 ? dispatch<bf16>(a, s) : dispatch<float>(a, s);
}

}  // namespace kla
