// kla_fwd_diag.hip -- gfx950 forward kernel, diagonal precision.
//
// Sources: "Kalman Linear Attention: Parallel Bayesian Filtering For Efficient
// Language Modelling and State Tracking" (gist.science explainer, method §1-§4)
// and "Kalman Delta Networks: Uncertainty-aware Associative Memory" (abstract,
// diagonal variant).
//
// Per (b,h) and key dim i the filter is
//   lp = l/(a^2 + qn l);  l' = lp + k^2/r                       (precision)
// and the posterior mean m = eta/l (one row per key dim) follows the gated
// linear recurrence that the precision ratios define (method §3, forget and
// write gates from precision ratios):
//   m_t = f_t (.) m_{t-1} + w_t v_t^T,  f = a lp / l',  w = k / (r l'),
//   o_t = q_t^T m_t.
// This is the information-form update eta' = (lp a / l) eta + k v / r divided
// by l' (method §2: the mean update is affine once the precision path is
// known).  The mean form keeps every gate in (0, 1], so cumulative gates only
// decay, which is what the chunked factorisation below relies on.
//
// One workgroup owns one (b,h) and one tile of value columns and walks the
// sequence in chunks of C tokens:
//   stage    coalesced loads of q,k,a,r,v; a^2 and b = k^2/r to LDS; V^T to LDS
//   chain    one lane per key dim runs the precision recurrence over the chunk
//            (4 VALU ops per token; the carry stays in LDS between chunks)
//   gates    all lanes: f, w, chunk-local cumulative gates G_t (product of f
//            after the chunk's first token), q^ = q G, w^ = w / G
//   mfma     S^T = W^ Q^^T (causal 16x16 tiles), O^T = M^T Q^^T + V^T P^T,
//            M += W^^T V; M is the fp32 state in accumulator registers
// The barriers order LDS only: __syncthreads() would also wait for the loads
// of the next chunk issued before it, which are meant to stay in flight.
// Every factor of the factorisation is bounded: G in [2^-64, 1].  If a gate
// product inside a chunk would fall below 2^-64, the chunk is cut there and
// the rest is processed as a new sub-chunk (exact, only slower).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kla_common.h"
#include "kla_internal.h"

namespace kla {
namespace {

constexpr float kGateFloor = 5.421010862427522e-20f;  // 2^-64

// ---------------------------------------------------------------- config
template <typename TIn, int DK_, int DV_, int C_>
struct Cfg {
    static constexpr int DK = DK_;            // key dim (all of it per workgroup)
    static constexpr int DV = DV_;            // value columns owned by the workgroup
    static constexpr int C = C_;              // tokens per chunk
    static constexpr int NW = (DV / 16 < 4) ? DV / 16 : 4;
    static constexpr int NT = NW * 64;
    static constexpr int JT = DV / 16 / NW;   // 16-column tiles per wave
    static constexpr int IT = DK / 16;        // 16-row tiles of the state
    static constexpr int NB = C / 16;         // 16-token blocks per chunk
    static constexpr int NIP = DK / 2;        // key-dim pairs
    static constexpr int NG = NT / NIP;       // token groups in the gate phase
    static constexpr int TPG = C / NG;        // tokens per group
    static constexpr int PE = 16 / (int)sizeof(TIn);  // 16-byte row padding
    static constexpr int QS = DK + PE;        // row stride of Q^, W^
    static constexpr int CS = C + PE;         // row stride of W^T, V^T
    static constexpr int VQ = DV / 4;         // value quads per token row
    static constexpr int VUNITS = (C / 2) * VQ;  // (token pair, value quad) units
    static constexpr int VPT = (VUNITS + NT - 1) / NT;
    static_assert(NT >= DK, "one chain lane per key dim");
    static_assert(NT % NIP == 0 && C % NG == 0 && TPG >= 1, "gate-phase layout");
    static_assert(C % 32 == 0 && DK % 16 == 0 && DV % 16 == 0, "tile shapes");
    static_assert(DV / 16 % NW == 0, "value tiles per wave");
};

// LDS.  The chain buffer AB is dead once the gate phase has read it, so the
// MFMA operands Q^, W^, W^T live in the same bytes.
template <typename TIn, class K>
struct Smem {
    union {
        f32x2 AB[K::C][K::DK];  // (a^2, b) in, (lp, l) out of the chain
        struct {
            TIn Q[K::C][K::QS];
            TIn W[K::C][K::QS];
            TIn WT[K::DK][K::CS];
        } op;
    } u;
    TIn VT[K::DV][K::CS];
    alignas(8) float gtot[K::NG][K::DK];
    float E[2][K::DK];   // pending end-of-subchunk state scale, by parity
    float sc[K::DK];     // state scale applied before a sub-chunk's readout
    float lcar[K::DK];   // precision carry between chunks
    int L1;
};

// Registers holding one chunk of HBM inputs for one thread.
template <typename TIn, class K>
struct ChunkRegs {
    typename Pair<TIn>::V q[K::TPG];
    typename Pair<TIn>::V k[K::TPG];
    f32x2 a[K::TPG];
    typename Quad<TIn>::V v[K::VPT][2];
    float r[K::TPG];  // r of the lane's gate-phase tokens
};

template <typename TIn, class K>
__device__ __forceinline__ void load_chunk(ChunkRegs<TIn, K>& R, const FwdArgs& p, int bh,
                                           int vt, int t0, int L, int tid) {
    typedef typename Pair<TIn>::V P2;
    const int ip = tid % K::NIP, grp = tid / K::NIP;
    const TIn* q = (const TIn*)p.q;
    const TIn* k = (const TIn*)p.k;
    const size_t row0 = (size_t)bh * p.T + t0;
#pragma unroll
    for (int u = 0; u < K::TPG; ++u) {
        const int t = grp * K::TPG + u;
        if (t < L) {
            const size_t off = (row0 + t) * K::DK + 2 * ip;
            R.q[u] = *(const P2*)(q + off);
            R.k[u] = *(const P2*)(k + off);
            R.a[u] = *(const f32x2*)(p.a + off);
        } else {
            R.q[u] = Pair<TIn>::zero();
            R.k[u] = Pair<TIn>::zero();
            R.a[u] = f32x2{1.f, 1.f};
        }
    }
    const TIn* v = (const TIn*)p.v;
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
#pragma unroll
    for (int u = 0; u < K::TPG; ++u) {
        const int t = grp * K::TPG + u;
        R.r[u] = t < L ? p.r[row0 + t] : 1.f;
    }
}

// Pre-scale of the state, its bf16 (or fp32) A-operand, readout, state update.
// FULL: the sub-chunk is the whole chunk (ts = 0, L1 = C), so the token-block
// loop has compile-time bounds and unrolls into one schedulable block.
template <typename TIn, class K, bool FULL>
__device__ __forceinline__ void mfma_subchunk(Smem<TIn, K>& sm, f32x4 (&accM)[K::IT][K::JT],
                                              const FwdArgs& p, int bh, int vt, int t0,
                                              int ts, int L1, int wave, int lane) {
    typedef MmaFor<TIn, K::DK> M;
    const int c16 = lane & 15, g = lane >> 4;

    // 1. m <- (pending end scale * first-token gate) (.) m, row-wise.
#pragma unroll
    for (int it = 0; it < K::IT; ++it) {
        const f32x4 s = *(const f32x4*)&sm.sc[it * 16 + 4 * g];
#pragma unroll
        for (int jj = 0; jj < K::JT; ++jj) accM[it][jj] *= s;
    }
    // 2. state as the A operand of O^T = M^T Q^^T (accumulator layout == A layout).
    typename M::K16 AM[K::IT][K::JT];
#pragma unroll
    for (int it = 0; it < K::IT; ++it)
#pragma unroll
        for (int jj = 0; jj < K::JT; ++jj) AM[it][jj] = M::from_acc(accM[it][jj]);

    // 3-4. per 16-token block: causal S^T tiles, then O^T tiles.
    const int tb0 = FULL ? 0 : ts / 16, tb1 = FULL ? K::NB : (L1 + 15) / 16;
#pragma unroll
    for (int tau = tb0; tau < tb1; ++tau) {
        typename M::K16 P[K::NB];
#pragma unroll
        for (int sig = 0; sig < K::NB; ++sig) {
            if (sig > tau || sig < tb0) continue;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if constexpr (K::DK >= 32) {
#pragma unroll
                for (int kk = 0; kk < K::DK / 32; ++kk) {
                    typename M::K32 a = M::ld32(&sm.u.op.W[sig * 16 + c16][kk * 32 + 8 * g]);
                    typename M::K32 b = M::ld32(&sm.u.op.Q[tau * 16 + c16][kk * 32 + 8 * g]);
                    acc = M::mma32(a, b, acc);
                }
            } else {
                typename M::K16 a = M::ld16(&sm.u.op.W[sig * 16 + c16][4 * g]);
                typename M::K16 b = M::ld16(&sm.u.op.Q[tau * 16 + c16][4 * g]);
                acc = M::mma16(a, b, acc);
            }
            if (sig == tau) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * g + e > c16) acc[e] = 0.f;
            }
            P[sig] = M::from_acc(acc);
        }
        const int t = tau * 16 + c16;
        const bool store = FULL || ((t >= ts) && (t < L1));
#pragma unroll
        for (int jj = 0; jj < K::JT; ++jj) {
            const int jt = wave * K::JT + jj;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int it = 0; it < K::IT; ++it) {
                typename M::K16 b = M::ld16(&sm.u.op.Q[tau * 16 + c16][it * 16 + 4 * g]);
                acc = M::mma16(AM[it][jj], b, acc);
            }
#pragma unroll
            for (int sig = 0; sig < K::NB; ++sig) {
                if (sig > tau || sig < tb0) continue;
                typename M::K16 a = M::ld16(&sm.VT[jt * 16 + c16][sig * 16 + 4 * g]);
                acc = M::mma16(a, P[sig], acc);
            }
            if (store) {
                TIn* o = (TIn*)p.o;
                const size_t off = ((size_t)bh * p.T + t0 + t) * p.dv + (size_t)vt * K::DV +
                                   jt * 16 + 4 * g;
                *(typename Quad<TIn>::V*)(o + off) = Quad<TIn>::make(acc);
            }
        }
    }

    // 5. m += W^^T V  (rows of W^ outside [ts, L1) are zero).
#pragma unroll
    for (int it = 0; it < K::IT; ++it)
#pragma unroll
        for (int jj = 0; jj < K::JT; ++jj) {
            const int jt = wave * K::JT + jj;
#pragma unroll
            for (int sc = 0; sc < K::C / 32; ++sc) {
                typename M::K32 a = M::ld32(&sm.u.op.WT[it * 16 + c16][sc * 32 + 8 * g]);
                typename M::K32 b = M::ld32(&sm.VT[jt * 16 + c16][sc * 32 + 8 * g]);
                accM[it][jj] = M::mma32(a, b, accM[it][jj]);
            }
        }
}

template <typename TIn, int DK, int DV, int C>
__global__ __launch_bounds__((Cfg<TIn, DK, DV, C>::NT)) void kla_fwd_diag_kernel(FwdArgs p) {
    typedef Cfg<TIn, DK, DV, C> K;
    typedef Pair<TIn> PR;
    __shared__ Smem<TIn, K> sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4;

    // Workgroup -> (b,h, value tile).  Dispatch is round-robin over the 8
    // XCDs; keep all value tiles of one (b,h) on one XCD so the q/k/a reads
    // they share hit the same L2.
    const int BH = p.B * p.H, nvt = p.n_vtiles;
    int bh, vt;
    {
        const int id = blockIdx.x;
        if (nvt > 1 && BH % 8 == 0) {
            const int x = id % 8, kx = id / 8;
            bh = (kx / nvt) * 8 + x;
            vt = kx % nvt;
        } else {
            bh = id / nvt;
            vt = id % nvt;
        }
    }
    const int h = bh % p.H;
    const int ip = tid % K::NIP, grp = tid / K::NIP;

    // ---- initial state: precision carry and mean m0 = eta0 / l0
    if (tid < DK) {
        sm.lcar[tid] = p.l0 ? p.l0[(size_t)bh * DK + tid] : 1.f;
        sm.E[1][tid] = 1.f;
    }
    lds_barrier();
    f32x4 accM[K::IT][K::JT];
#pragma unroll
    for (int it = 0; it < K::IT; ++it)
#pragma unroll
        for (int jj = 0; jj < K::JT; ++jj) {
            const int jt = wave * K::JT + jj;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = it * 16 + 4 * g + e;
                const int j = vt * DV + jt * 16 + c16;
                accM[it][jj][e] =
                    p.eta0 ? p.eta0[((size_t)bh * DK + i) * p.dv + j] / sm.lcar[i] : 0.f;
            }
        }
    const float qn_i = (tid < DK) ? p.qn[(size_t)h * DK + tid] : 0.f;

    int par = 0;  // parity of the E buffer the next sub-chunk writes
    ChunkRegs<TIn, K> cur;
    if (p.T > 0) load_chunk<TIn, K>(cur, p, bh, vt, 0, p.T < C ? p.T : C, tid);

    for (int t0 = 0; t0 < p.T; t0 += C) {
        const int L = (p.T - t0) < C ? (p.T - t0) : C;

        // ---- stage: (a^2, b) for the chain, V^T.  Each lane divides 1/r for
        // its own tokens, which saves a barrier and an LDS round trip.
        float rho[K::TPG];
#pragma unroll
        for (int u = 0; u < K::TPG; ++u) rho[u] = 1.f / cur.r[u];
#pragma unroll
        for (int u = 0; u < K::TPG; ++u) {
            const int t = grp * K::TPG + u;
            const float rh = rho[u];
            const float k0 = PR::lo(cur.k[u]), k1 = PR::hi(cur.k[u]);
            const f32x2 av = cur.a[u];
            f32x4 ab = {av[0] * av[0], k0 * k0 * rh, av[1] * av[1], k1 * k1 * rh};
            *(f32x4*)&sm.u.AB[t][2 * ip] = ab;
        }
#pragma unroll
        for (int x = 0; x < K::VPT; ++x) {
            const int unit = tid + x * K::NT;
            if (unit < K::VUNITS) {
                const int tp = unit / K::VQ, jq = unit % K::VQ;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    typename PR::V pr = PR::make((float)cur.v[x][0][e], (float)cur.v[x][1][e]);
                    *(typename PR::V*)&sm.VT[4 * jq + e][2 * tp] = pr;
                }
            }
        }
        if (tid == 0) sm.L1 = L;
        lds_barrier();

        // ---- chain: one lane per key dim, sequential over the chunk
        if (tid < DK) {
            float l = sm.lcar[tid];
            auto link = [&](int t) {
                const f32x2 ab = sm.u.AB[t][tid];
                const float lp = l * fast_rcp(__builtin_fmaf(qn_i, l, ab[0]));
                l = lp + ab[1];
                sm.u.AB[t][tid] = f32x2{lp, l};
            };
            if (L == C) {
                // full chunk: unrolled, so the LDS reads run ahead of the chain
#pragma unroll
                for (int t = 0; t < C; ++t) link(t);
            } else {
                for (int t = 0; t < L; ++t) link(t);
            }
            sm.lcar[tid] = l;
        }
        lds_barrier();

        // ---- gates (a): f = a lp / l, w = k / (r l)
        float f[K::TPG][2], w[K::TPG][2];
#pragma unroll
        for (int u = 0; u < K::TPG; ++u) {
            const int t = grp * K::TPG + u;
            const f32x4 pl = *(const f32x4*)&sm.u.AB[t][2 * ip];  // lp0, l0, lp1, l1
            const float rl0 = fast_rcp(pl[1]), rl1 = fast_rcp(pl[3]);
            f[u][0] = cur.a[u][0] * pl[0] * rl0;
            f[u][1] = cur.a[u][1] * pl[2] * rl1;
            const float rh = rho[u];
            w[u][0] = PR::lo(cur.k[u]) * rh * rl0;
            w[u][1] = PR::hi(cur.k[u]) * rh * rl1;
        }

        // ---- sub-chunks (one unless a gate product drops below 2^-64)
        int ts = 0;
        while (ts < L) {
            // (b) group products of f over tokens (ts, L)
            float G[K::TPG][2];
            float p0 = 1.f, p1 = 1.f;
#pragma unroll
            for (int u = 0; u < K::TPG; ++u) {
                const int t = grp * K::TPG + u;
                if (t > ts && t < L) { p0 *= f[u][0]; p1 *= f[u][1]; }
                G[u][0] = p0;
                G[u][1] = p1;
            }
            // previous readers of gtot / sm.L1: the last sub-chunk (the first
            // sub-chunk's were in the previous chunk, several barriers ago)
            if (ts > 0) lds_barrier();
            *(f32x2*)&sm.gtot[grp][2 * ip] = f32x2{p0, p1};
            lds_barrier();
            // (c) cumulative gates, range check; all group totals are read at once
            float pre0 = 1.f, pre1 = 1.f;
#pragma unroll
            for (int gg = 0; gg < K::NG - 1; ++gg) {
                const f32x2 gv = *(const f32x2*)&sm.gtot[gg][2 * ip];
                if (gg < grp) {
                    pre0 *= gv[0];
                    pre1 *= gv[1];
                }
            }
            int firstbad = L;
#pragma unroll
            for (int u = 0; u < K::TPG; ++u) {
                const int t = grp * K::TPG + u;
                G[u][0] *= pre0;
                G[u][1] *= pre1;
                if (t >= ts && t < L && (G[u][0] < kGateFloor || G[u][1] < kGateFloor))
                    firstbad = t < firstbad ? t : firstbad;
            }
            if (firstbad < L) atomicMin(&sm.L1, firstbad);
            lds_barrier();
            const int L1 = sm.L1;
            // (d) operands of this sub-chunk; zero outside [ts, L1)
            TIn wt0[K::TPG], wt1[K::TPG];
#pragma unroll
            for (int u = 0; u < K::TPG; ++u) {
                const int t = grp * K::TPG + u;
                const bool keep = (t >= ts) && (t < L1);
                float q0 = 0.f, q1 = 0.f, w0 = 0.f, w1 = 0.f;
                if (keep) {
                    q0 = PR::lo(cur.q[u]) * G[u][0];
                    q1 = PR::hi(cur.q[u]) * G[u][1];
                    w0 = w[u][0] * fast_rcp(G[u][0]);
                    w1 = w[u][1] * fast_rcp(G[u][1]);
                }
                *(typename PR::V*)&sm.u.op.Q[t][2 * ip] = PR::make(q0, q1);
                *(typename PR::V*)&sm.u.op.W[t][2 * ip] = PR::make(w0, w1);
                wt0[u] = (TIn)w0;
                wt1[u] = (TIn)w1;
                if (t == ts) {
                    sm.sc[2 * ip] = sm.E[par ^ 1][2 * ip] * f[u][0];
                    sm.sc[2 * ip + 1] = sm.E[par ^ 1][2 * ip + 1] * f[u][1];
                }
                if (t == L1 - 1) {
                    sm.E[par][2 * ip] = G[u][0];
                    sm.E[par][2 * ip + 1] = G[u][1];
                }
            }
#pragma unroll
            for (int u = 0; u < K::TPG; ++u) {
                sm.u.op.WT[2 * ip][grp * K::TPG + u] = wt0[u];
                sm.u.op.WT[2 * ip + 1][grp * K::TPG + u] = wt1[u];
            }
            lds_barrier();

            if (ts == 0 && L1 == C)
                mfma_subchunk<TIn, K, true>(sm, accM, p, bh, vt, t0, ts, L1, wave, lane);
            else
                mfma_subchunk<TIn, K, false>(sm, accM, p, bh, vt, t0, ts, L1, wave, lane);

            par ^= 1;
            ts = L1;
            if (ts < L) {
                lds_barrier();  // all waves done reading this sub-chunk's operands
                if (tid == 0) sm.L1 = L;
            }
        }
        // Prefetch the next chunk at the end of this one.  Requested at the
        // stage, the loads queued ahead of the chain's critical path; requested
        // by the waves that idle through the chain, they slowed the workgroups
        // sharing the CU (both measured).
        const int t0n = t0 + C;
        if (t0n < p.T) load_chunk<TIn, K>(cur, p, bh, vt, t0n, (p.T - t0n) < C ? (p.T - t0n) : C, tid);
        lds_barrier();  // LDS free for the next chunk's stage
    }

    // ---- epilogue: m <- pending scale (.) m;  etaT = lT (.) m;  lT
    if (p.etaT) {
#pragma unroll
        for (int it = 0; it < K::IT; ++it)
#pragma unroll
            for (int jj = 0; jj < K::JT; ++jj) {
                const int jt = wave * K::JT + jj;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = it * 16 + 4 * g + e;
                    const int j = vt * DV + jt * 16 + c16;
                    p.etaT[((size_t)bh * DK + i) * p.dv + j] =
                        accM[it][jj][e] * sm.E[par ^ 1][i] * sm.lcar[i];
                }
            }
    }
    if (p.lT && vt == 0 && tid < DK) p.lT[(size_t)bh * DK + tid] = sm.lcar[tid];
}

template <typename TIn, int DK, int DV, int C>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
    typedef Cfg<TIn, DK, DV, C> K;
    const int nblk = a.B * a.H * a.n_vtiles;
    hipLaunchKernelGGL((kla_fwd_diag_kernel<TIn, DK, DV, C>), dim3(nblk), dim3(K::NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool fwd_diag_supported(int dk, int dv, int dtype) {
    (void)dtype;
    return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}

int fwd_diag_vtiles(int B, int H, int T, int dk, int dv) {
    (void)T;
    (void)dv;
    // Fewer than one (b,h) per CU: split the value columns in two.
    if ((long long)B * H < 256 && dk >= 64) return 2;
    return 1;
}

hipError_t launch_fwd_diag(const FwdArgs& a, int dtype, hipStream_t s) {
    constexpr int C = 32;
    const int nvt = a.n_vtiles;
    if (a.dk != a.dv) return hipErrorInvalidValue;
    if (dtype == DT_BF16) {
        switch (a.dk) {
            case 16: if (nvt == 1) return launch<bf16, 16, 16, C>(a, s); break;
            case 32: if (nvt == 1) return launch<bf16, 32, 32, C>(a, s); break;
            case 64:
                if (nvt == 1) return launch<bf16, 64, 64, C>(a, s);
                if (nvt == 2) return launch<bf16, 64, 32, C>(a, s);
                break;
            case 128:
                if (nvt == 1) return launch<bf16, 128, 128, C>(a, s);
                if (nvt == 2) return launch<bf16, 128, 64, C>(a, s);
                break;
        }
    } else {
        switch (a.dk) {
            case 16: if (nvt == 1) return launch<float, 16, 16, C>(a, s); break;
            case 32: if (nvt == 1) return launch<float, 32, 32, C>(a, s); break;
            case 64:
                if (nvt == 1) return launch<float, 64, 64, C>(a, s);
                if (nvt == 2) return launch<float, 64, 32, C>(a, s);
                break;
            case 128:
                if (nvt == 1) return launch<float, 128, 128, C>(a, s);
                if (nvt == 2) return launch<float, 128, 64, C>(a, s);
                break;
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace kla
