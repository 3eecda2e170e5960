// kla_fwd_seg.hip -- the passes around a sequence-split diagonal KLA forward
// for gfx950.
//
// Method: "Kalman Linear Attention: Parallel Bayesian Filtering For Efficient
// Language Modelling and State Tracking" (technical summary > method §2): the
// precision update is a Mobius map, so the map of a whole segment of tokens is
// the product of the segments' 2x2 matrices, and the precision entering every
// segment follows from a short scan over segment products.  The mean state is
// affine in the incoming state (m_t = f_t m_{t-1} + w_t v_t^T), so each
// segment can run from a zero state and be corrected afterwards.
//
// With nseg segments per (b,h) the forward runs:
//   0. kla_seg_warm:     the precision entering each segment from the map
//                        of the kWarm tokens before it, applied to both
//                        extreme precisions (0 and +inf); a (b,h) where the
//                        two agree at every key dim and segment start skips
//                        passes 1 and 2;
//   1. kla_seg_mobius:   the product of the precision matrices of every
//                        block of kSegBlk tokens before the last segment, per
//                        key dim;
//   2. the precision entering each segment (a walk over the block
//      products), exact from the caller's l0, run by the last workgroup of
//      pass 1 to finish;
//   3. the wave-specialised forward on every segment (local outputs, local
//      final mean state, the segment's total gate, and q (.) gate product);
//   4. kla_seg_carry_m:  the mean state entering each segment, and etaT;
//   5. kla_seg_correct:  o_t += (q_t (.) G_t)^T M_in for every later segment.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kla_common.h"
#include "kla_internal.h"

namespace kla {
namespace {

__device__ __forceinline__ size_t seg_row(const FwdArgs& p, int bh, int s) {
    return (size_t)bh * p.nseg + s;
}

__device__ __forceinline__ int seg_blocks(const FwdArgs& p) {
    return (p.nseg - 1) * (p.seg_len / kSegBlk);
}

// True when the warm-up settled the precision entering every segment of
// (b,h) bh; the exact passes then leave it alone.
// (The flags are read without an early exit, so that the loads overlap.)
__device__ __forceinline__ bool seg_warm_ok(const FwdArgs& p, const int* ok, int bh) {
    const int* f = ok + seg_row(p, bh, 0) * 2;
    int all = 1;
    for (int x = 2; x < 2 * p.nseg; ++x)
        all &= (x % 2 == 0 || p.dk == 128) ? f[x] : 1;
    return all != 0;
}

// Every (b,h) settled by the warm-up, checked by the whole workgroup at once
// (one flag per thread, a workgroup vote) when the flags fit; the launches
// that only handle unsettled ones then end at once.
__device__ __forceinline__ bool seg_all_warm_ok(const FwdArgs& p, const int* ok) {
    const int per = 2 * p.nseg, n = p.B * p.H * per;
    if (n > (int)blockDim.x) return false;  // too many: checked per (b,h)
    int good = 1;
    const int x = (int)threadIdx.x;
    if (x < n) {
        const int bh = x / per, k = x % per;
        if (k >= 2 && (k % 2 == 0 || p.dk == 128)) good = ok[seg_row(p, bh, 0) * 2 + k];
    }
    return __syncthreads_and(good) != 0;
}

// Scale a positive 2x2 map by a power of two (exact; the map is unchanged)
// so that its entries sum to [1, 2).
__device__ __forceinline__ void mob_renorm(double& p00, double& p01, double& p10, double& p11) {
    const int e = __builtin_amdgcn_frexp_exp((p00 + p01) + (p10 + p11));
    p00 = __builtin_amdgcn_ldexp(p00, 1 - e);
    p01 = __builtin_amdgcn_ldexp(p01, 1 - e);
    p10 = __builtin_amdgcn_ldexp(p10, 1 - e);
    p11 = __builtin_amdgcn_ldexp(p11, 1 - e);
}

// -------------------------------------------------- 0. precision warm-up
// Every token's precision map x -> x / (qn x + a^2) + k^2 / r is increasing
// and contracting, so the precision after a run of tokens hardly depends on
// where the run started: the run's composed map P sends the extreme starts 0
// and +inf to P(0) = p01/p11 and P(inf) = p00/p10, which enclose the true
// precision, and once they agree to 2^-20 (relative) their midpoint is the
// precision to within 2^-21.  The kWarm tokens before each segment start are
// composed in fp64 (rounding far below that bound; each token's b and a^2
// are rounded to fp32 as in the forward's chain), kWarmRun tokens per thread
// and the runs in order; when the window reaches the sequence start
// the map is applied to the caller's l0 instead (exact).  One workgroup per
// (b,h, segment s >= 1, 64 key dims), one wave per run.  The (b,h, s, group)
// flag is set only when every key dim of the group converged; a (b,h) with
// any flag clear takes the exact passes 1 and 2 instead.
constexpr int kWarm = 512;
constexpr int kWarmRun = 32;
constexpr int kWarmRuns = kWarm / kWarmRun;

template <typename TIn, int DK, bool PRO>
__global__ __launch_bounds__(64 * kWarmRuns) void kla_seg_warm(FwdArgs p, int* ok) {
    __shared__ double sP[kWarmRuns][4][64];
    constexpr int G = DK / 64;
    int x = blockIdx.x;
    const int g = x % G;
    x /= G;
    const int s = 1 + x % (p.nseg - 1), bh = x / (p.nseg - 1);
    const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
    const int i = g * 64 + lane;
    const int h = bh % p.H;
    const int bnd = s * p.seg_len;
    // the counter of the exact passes' workgroups (launched next) starts at 0
    if (blockIdx.x == 0 && threadIdx.x == 0) ok[(size_t)p.B * p.H * p.nseg * 2] = 0;
    const int n = bnd < kWarm ? bnd : kWarm;  // a multiple of kSegBlk
    const int t0 = bnd - n;
    const double qn = PRO ? act_softplus(p.qn[(size_t)h * DK + i]) : p.qn[(size_t)h * DK + i];
    // P = M_last ... M_first with M_t = [[1 + b qn, b a^2], [qn, a^2]]
    double p00 = 1.0, p01 = 0.0, p10 = 0.0, p11 = 1.0;
    if (j * kWarmRun < n) {  // uniform over the wave
        const int tr = t0 + j * kWarmRun;  // the run's first token
        const size_t row = (size_t)bh * p.T + tr;
        // a (with the block prologue: its pre-activation, in the input dtype)
        constexpr int AES = PRO ? (int)sizeof(TIn) : 4;
        const auto ra = make_rsrc((const char*)p.a + row * DK * AES, kWarmRun * DK * AES);
        const auto rk = make_rsrc((const TIn*)p.k + row * DK, kWarmRun * DK * (int)sizeof(TIn));
        // the token's row offset goes in the scalar offset, the lane's column
        // in the vector offset
        float av[kWarmRun], kv[kWarmRun];
#pragma unroll
        for (int u = 0; u < kWarmRun; ++u) {
            if constexpr (AES == 2)
                av[u] = __builtin_bit_cast(
                    float, (unsigned)(unsigned short)__builtin_amdgcn_raw_buffer_load_b16(ra, i * 2, u * DK * 2, 0)
                               << 16);
            else
                av[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, i * 4, u * DK * 4, 0));
            if constexpr (sizeof(TIn) == 2)
                kv[u] = __builtin_bit_cast(
                    float, (unsigned)(unsigned short)__builtin_amdgcn_raw_buffer_load_b16(rk, i * 2, u * DK * 2, 0)
                               << 16);
            else
                kv[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rk, i * 4, u * DK * 4, 0));
        }
        // block prologue: k = silu(conv(x)) from the taps of key dim i and the
        // three x values before each token
        float kw[4] = {0.f, 0.f, 0.f, 0.f}, kb = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
        if constexpr (PRO) {
            const int W = p.conv_w;
            const size_t ch = (size_t)h * DK + i;
            load_taps4(kw, p.conv_wt[1] + ch * W, W);
            if (p.conv_b[1]) kb = p.conv_b[1][ch];
            x1 = pro_x((const TIn*)p.k, p.conv_s[1], bh, p.T, W, DK, tr - 1, i);
            x2 = pro_x((const TIn*)p.k, p.conv_s[1], bh, p.T, W, DK, tr - 2, i);
            x3 = pro_x((const TIn*)p.k, p.conv_s[1], bh, p.T, W, DK, tr - 3, i);
        }
        // 1/r once per token (lane u holds token u of the run).  b and a^2 are
        // rounded to fp32 like the forward's own chain; the composition that
        // follows is fp64.
        const float rraw = p.r[row + (lane % kWarmRun)];
        const float rho_l = 1.f / (PRO ? act_softplus(rraw) + p.r_eps : rraw);
#pragma unroll
        for (int u = 0; u < kWarmRun; ++u) {
            const float rt = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rho_l), u));
            float af = av[u], kf = kv[u];
            if constexpr (PRO) {
                af = act_sigmoid(av[u]);
                kf = act_silu(conv4(kw, kb, kv[u], x1, x2, x3));
                x3 = x2;
                x2 = x1;
                x1 = kv[u];
            }
            const double a2 = (double)(af * af);
            const double b = (double)(kf * kf * rt);
            const double m00 = __builtin_fma(b, qn, 1.0), m01 = b * a2;
            const double n00 = m00 * p00 + m01 * p10, n01 = m00 * p01 + m01 * p11;
            const double n10 = qn * p00 + a2 * p10, n11 = qn * p01 + a2 * p11;
            p00 = n00; p01 = n01; p10 = n10; p11 = n11;
            if (u % 8 == 7) mob_renorm(p00, p01, p10, p11);
        }
    }
    sP[j][0][lane] = p00;
    sP[j][1][lane] = p01;
    sP[j][2][lane] = p10;
    sP[j][3][lane] = p11;
    __syncthreads();
    if (j != 0) return;
    for (int u = 1; u < kWarmRuns; ++u) {  // later runs on the left
        const double m00 = sP[u][0][lane], m01 = sP[u][1][lane];
        const double m10 = sP[u][2][lane], m11 = sP[u][3][lane];
        const double n00 = m00 * p00 + m01 * p10, n01 = m00 * p01 + m01 * p11;
        const double n10 = m10 * p00 + m11 * p10, n11 = m10 * p01 + m11 * p11;
        p00 = n00; p01 = n01; p10 = n10; p11 = n11;
        mob_renorm(p00, p01, p10, p11);
    }
    const float l_in = p.l0 ? p.l0[(size_t)bh * DK + i] : 1.f;
    float* l0out = const_cast<float*>(p.seg_l0);
    if (s == 1) l0out[seg_row(p, bh, 0) * DK + i] = l_in;
    double l;
    bool good;
    if (t0 == 0) {
        l = (p00 * l_in + p01) / (p10 * l_in + p11);
        good = true;
    } else {
        const double lo = p01 / p11, hi = p00 / p10;
        l = 0.5 * (lo + hi);
        good = __builtin_fabs(hi - lo) <= 0x1p-20 * lo;  // false for NaN (qn = 0)
    }
    l0out[seg_row(p, bh, s) * DK + i] = (float)l;
    const unsigned long long bad = __builtin_amdgcn_ballot_w64(!good);
    if (lane == 0) ok[seg_row(p, bh, s) * 2 + g] = bad == 0;
}

// -------------------------------------------------- 1. block products
// One workgroup per (b,h, block of kSegBlk tokens) at a time; NSUB threads per
// key dim each compose a contiguous run of the block, then the runs are
// combined in order.  Workgroups of 512 threads, so that several share a CU,
// and 16 tokens of loads in flight per thread keep enough reads outstanding.
constexpr int kMobThreads = 512;
constexpr int kMobGrid = 1024;

template <typename TIn, int DK, bool PRO>
__device__ __forceinline__ void mobius_block(const FwdArgs& p, float* P, f32x4 (*sP)[DK], int i, int sub,
                                             int nb, int bh, int s) {
    constexpr int NSUB = kMobThreads / DK;
    const int h = bh % p.H;
    const int T0 = s * kSegBlk;
    constexpr int sl = kSegBlk / NSUB;
    const int tb = T0 + sub * sl;  // blocks before the last segment are full
    const float qn = PRO ? act_softplus(p.qn[(size_t)h * DK + i]) : p.qn[(size_t)h * DK + i];
    // a (with the block prologue: its pre-activation, in the input dtype)
    constexpr int AES = PRO ? (int)sizeof(TIn) : 4;
    const char* ap = (const char*)p.a + ((size_t)bh * p.T * DK + i) * AES;
    const TIn* kp = (const TIn*)p.k + (size_t)bh * p.T * DK + i;
    const float* rp = p.r + (size_t)bh * p.T;
    // P = M_t ... M_tb, later tokens on the left
    float p00 = 1.f, p01 = 0.f, p10 = 0.f, p11 = 1.f;
    auto step = [&](float a, float kv, float rho) {
        const float b = kv * kv * rho, a2 = a * a;
        const float m00 = __builtin_fmaf(b, qn, 1.f), m01 = b * a2, m10 = qn, m11 = a2;
        const float n00 = m00 * p00 + m01 * p10, n01 = m00 * p01 + m01 * p11;
        const float n10 = m10 * p00 + m11 * p10, n11 = m10 * p01 + m11 * p11;
        p00 = n00; p01 = n01; p10 = n10; p11 = n11;
    };
    // All lanes of a wave walk the same tokens (64 consecutive key dims of
    // one run), so 1/r is computed once per token: lane u divides for token
    // tb + u and the steps read it back by lane.
    constexpr int TB = 8;  // tokens per load batch
    static_assert(sl <= 64 && sl % TB == 0 && DK % 64 == 0, "run layout");
    const int lane = threadIdx.x & 63;
    const float rho_l = lane < sl ? 1.f / (PRO ? act_softplus(rp[tb + lane]) + p.r_eps : rp[tb + lane]) : 0.f;
    // block prologue: k = silu(conv(x)) from the taps of key dim i and the
    // three x values before each token
    float kw[4] = {0.f, 0.f, 0.f, 0.f}, kb = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
    if constexpr (PRO) {
        const int W = p.conv_w;
        const size_t ch = (size_t)h * DK + i;
        load_taps4(kw, p.conv_wt[1] + ch * W, W);
        if (p.conv_b[1]) kb = p.conv_b[1][ch];
        x1 = pro_x((const TIn*)p.k, p.conv_s[1], bh, p.T, W, DK, tb - 1, i);
        x2 = pro_x((const TIn*)p.k, p.conv_s[1], bh, p.T, W, DK, tb - 2, i);
        x3 = pro_x((const TIn*)p.k, p.conv_s[1], bh, p.T, W, DK, tb - 3, i);
    }
    // batches of TB tokens, the next batch's loads in flight during the
    // current batch's steps
    struct Batch {
        float a[TB], kv[TB];
    };
    // the run's rows of a and k through buffer resources (offsets from the
    // run start, so the per-token offsets are immediates or a few registers)
    const auto ra = make_rsrc(ap - (size_t)i * AES + (size_t)tb * DK * AES, sl * DK * AES);
    const auto rk = make_rsrc(kp - i + (size_t)tb * DK, sl * DK * (int)sizeof(TIn));
    auto load = [&](int t8, Batch& x) {
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            if constexpr (AES == 2)
                x.a[u] = __builtin_bit_cast(
                    float, (unsigned)buf_load<unsigned short>(ra, ((t8 + u) * DK + i) * 2) << 16);
            else
                x.a[u] = buf_load<float>(ra, ((t8 + u) * DK + i) * 4);
            if constexpr (sizeof(TIn) == 2)
                x.kv[u] = __builtin_bit_cast(
                    float, (unsigned)buf_load<unsigned short>(rk, ((t8 + u) * DK + i) * 2) << 16);
            else
                x.kv[u] = buf_load<float>(rk, ((t8 + u) * DK + i) * 4);
        }
    };
    auto run = [&](int t8, const Batch& x) {
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            const float rho = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rho_l), t8 + u));
            if constexpr (PRO) {
                const float kf = act_silu(conv4(kw, kb, x.kv[u], x1, x2, x3));
                x3 = x2;
                x2 = x1;
                x1 = x.kv[u];
                step(act_sigmoid(x.a[u]), kf, rho);
            } else {
                step(x.a[u], x.kv[u], rho);
            }
            if (u % 4 == 3) {
                const float sc = fast_rcp(p00 + p01 + p10 + p11);  // positive rescale: same map
                p00 *= sc; p01 *= sc; p10 *= sc; p11 *= sc;
            }
        }
    };
    Batch b0, b1;
    load(0, b0);
#pragma unroll 1
    for (int t8 = 0; t8 < sl; t8 += 2 * TB) {
        if (t8 + TB < sl) load(t8 + TB, b1);
        run(t8, b0);
        if (t8 + TB >= sl) break;
        if (t8 + 2 * TB < sl) load(t8 + 2 * TB, b0);
        run(t8 + TB, b1);
    }
    sP[sub][i] = f32x4{p00, p01, p10, p11};
    __syncthreads();
    if (sub == 0) {
        f32x4 q = sP[0][i];
        for (int u = 1; u < NSUB; ++u) {
            const f32x4 m = sP[u][i];  // later run on the left
            f32x4 n;
            n[0] = m[0] * q[0] + m[1] * q[2];
            n[1] = m[0] * q[1] + m[1] * q[3];
            n[2] = m[2] * q[0] + m[3] * q[2];
            n[3] = m[2] * q[1] + m[3] * q[3];
            const float sc = fast_rcp(n[0] + n[1] + n[2] + n[3]);
            q = n * sc;
        }
        *(f32x4*)&P[(((size_t)bh * nb + s) * DK + i) * 4] = q;
    }
}

__device__ void seg_carry_l_one(const FwdArgs& p, const float* P, const int* ok, int x);

template <typename TIn, int DK, bool PRO>
__global__ __launch_bounds__(kMobThreads) void kla_seg_mobius(FwdArgs p, float* P, int* ok) {
    constexpr int NSUB = kMobThreads / DK;
    __shared__ f32x4 sP[NSUB][DK];
    const int i = threadIdx.x % DK, sub = threadIdx.x / DK;
    const int nb = seg_blocks(p);
    if (seg_all_warm_ok(p, ok)) return;  // uniform over the workgroup
    // at most kMobGrid workgroups stride over the blocks
    for (int blk = blockIdx.x; blk < p.B * p.H * nb; blk += gridDim.x) {
        const int bh = blk / nb, s = blk % nb;
        if (seg_warm_ok(p, ok, bh)) continue;  // uniform over the workgroup
        mobius_block<TIn, DK, PRO>(p, P, sP, i, sub, nb, bh, s);
        __syncthreads();  // sP is reused by the next block
    }
    // The last workgroup to finish (counted after its block matrices are
    // released) runs pass 2, the precision carry, which needs all of them:
    // one launch instead of two, and no workgroup waits for another.
    __shared__ int last;
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        last = atomicAdd(ok + (size_t)p.B * p.H * p.nseg * 2, 1) == (int)gridDim.x - 1;
    }
    __syncthreads();
    if (!last) return;
    __threadfence();
    for (int x = threadIdx.x; x < p.B * p.H * p.dk; x += blockDim.x) seg_carry_l_one(p, P, ok, x);
}

// -------------------------------------------------- 2. precision carry
// Entry x = (b,h, key dim) of a (b,h) the warm-up left unsettled: the
// precision entering each segment from the caller's l0, composing the block
// matrices of each segment eight loads at a time.  Run by the last workgroup
// of pass 1 (below), once every block matrix is written.
__device__ void seg_carry_l_one(const FwdArgs& p, const float* P, const int* ok, int x) {
    const int bh = x / p.dk, i = x % p.dk;
    if (seg_warm_ok(p, ok, bh)) return;
    float l = p.l0 ? p.l0[x] : 1.f;
    float* out = const_cast<float*>(p.seg_l0);
    const int nb = seg_blocks(p), per = p.seg_len / kSegBlk;
    const f32x4* Pb = (const f32x4*)P + (size_t)bh * nb * p.dk + i;
    for (int s = 0; s < p.nseg; ++s) {
        out[seg_row(p, bh, s) * p.dk + i] = l;
        if (s + 1 == p.nseg) break;
        // the segment's map: its block matrices composed (later on the left),
        // eight independent loads at a time
        f32x4 q = {1.f, 0.f, 0.f, 1.f};
        for (int b0 = s * per; b0 < (s + 1) * per; b0 += 8) {
            f32x4 m[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                m[u] = b0 + u < (s + 1) * per ? Pb[(size_t)(b0 + u) * p.dk] : f32x4{1.f, 0.f, 0.f, 1.f};
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                f32x4 n;
                n[0] = m[u][0] * q[0] + m[u][1] * q[2];
                n[1] = m[u][0] * q[1] + m[u][1] * q[3];
                n[2] = m[u][2] * q[0] + m[u][3] * q[2];
                n[3] = m[u][2] * q[1] + m[u][3] * q[3];
                q = n * fast_rcp(n[0] + n[1] + n[2] + n[3]);
            }
        }
        l = __builtin_fmaf(q[0], l, q[1]) / __builtin_fmaf(q[2], l, q[3]);
    }
}

// -------------------------------------------------- 4. state carry
// Segment 0 ran from the caller's state, later ones from zero, so the state
// entering segment s (s >= 1) is M_s = d_{s-1} M_{s-1} + Mloc_{s-1} with
// M_0 = 0; it overwrites slot s-1 (already consumed).  etaT = lT (.) M_nseg.
__global__ void kla_seg_carry_m(FwdArgs p) {
    const size_t n = (size_t)p.B * p.H * p.dk * p.dv;
    const size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= n) return;
    const int j = (int)(x % p.dv);
    const int i = (int)((x / p.dv) % p.dk);
    const int bh = (int)(x / ((size_t)p.dv * p.dk));
    // Eight segments at a time: their local states and decays are all read
    // before any slot is rewritten (slot s-1 is rewritten only after segment
    // s-1 has been read), so the reads of a batch are in flight together
    // instead of one round trip per segment.
    constexpr int NB = 8;
    const size_t slot0 = (size_t)bh * p.nseg * p.dk * p.dv + (size_t)i * p.dv + j;
    const size_t sstride = (size_t)p.dk * p.dv;
    float m = 0.f;
    for (int s0 = 0; s0 < p.nseg; s0 += NB) {
        float ml[NB], d[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int s = s0 + u;
            ml[u] = s < p.nseg ? p.seg_m[slot0 + (size_t)s * sstride] : 0.f;
            d[u] = s < p.nseg ? p.seg_d[seg_row(p, bh, s) * p.dk + i] : 1.f;
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int s = s0 + u;
            if (s < p.nseg) {
                if (s >= 1) p.seg_m[slot0 + (size_t)(s - 1) * sstride] = m;  // M entering segment s
                m = __builtin_fmaf(d[u], m, ml[u]);
            }
        }
    }
    if (p.etaT) p.etaT[x] = m * p.seg_lend[(size_t)bh * p.dk + i];
}

// -------------------------------------------------- 5. output correction
// o_t += sum_i qhat_t[i] M_s[i,:] for the tokens of segment s >= 1.  One
// workgroup per (b,h, segment, kCorrBlk-token block); M_s^T is staged once in
// LDS as the A operand, every wave then runs 16-token tiles.  The q-hat rows
// are read as MFMA B fragments (16 bytes per lane, K in natural order, the A
// fragments likewise); the output rows are read and written with whole-row
// 16-byte accesses and moved to and from the accumulator layout through a
// small LDS tile of the wave.  The next tile's loads are in flight while the
// current one is multiplied.
constexpr int kCorrBlk = 512;

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(256) void kla_seg_correct(FwdArgs p) {
    typedef Frag<TIn> F;
    typedef typename F::V FV;
    typedef typename Quad<TIn>::V QV;
    constexpr int PE = 16 / (int)sizeof(TIn), MS = DK + PE, OS = DV + PE, ES = (int)sizeof(TIn);
    constexpr int KB = DK / 32, JB = DV / 16;
    constexpr int OL = 16 * DV * ES / 1024;  // 16-byte loads per lane for one tile of o
    constexpr int RL = DV * ES / 16;         // lanes per o row
    static_assert(OL >= 1 && 16 * DV * ES % 1024 == 0, "tile of o");
    __shared__ TIn MT[DV][MS];
    __shared__ TIn OT[4][16][OS];
    const int nlater = p.nseg - 1;
    const int nblk = (p.seg_len + kCorrBlk - 1) / kCorrBlk;
    int id = blockIdx.x;
    const int blk = id % nblk;
    id /= nblk;
    const int s = 1 + id % nlater;
    const int bh = id / nlater;
    const int T0 = s * p.seg_len;
    int TL = p.T - T0;
    if (TL > p.seg_len) TL = p.seg_len;
    const int tb = blk * kCorrBlk;
    if (tb >= TL) return;  // uniform over the workgroup
    // stage M_s^T (M_s lives in slot s-1): every thread issues all of its
    // 16-byte loads before the first LDS write
    {
        constexpr int NV = DK * DV / 4 / 256;
        const f32x4* M = (const f32x4*)(p.seg_m + seg_row(p, bh, s - 1) * DK * DV);
        f32x4 mv[NV];
#pragma unroll
        for (int u = 0; u < NV; ++u) mv[u] = M[threadIdx.x + u * 256];
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int x = 4 * (threadIdx.x + u * 256), i = x / DV, j = x % DV;
#pragma unroll
            for (int e = 0; e < 4; ++e) MT[j + e][i] = (TIn)mv[u][e];
        }
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c16 = lane & 15, g = lane >> 4;
    const size_t row0 = (size_t)bh * p.T + T0 + tb;
    const int rows = TL - tb < kCorrBlk ? TL - tb : kCorrBlk;
    // q-hat tiles of this block (segment and block starts are multiples of 16)
    const TIn* qh = (const TIn*)p.seg_qhat + qhat_tile_offset(bh, p.T, DK, T0 + tb, 0);
    TIn* o = (TIn*)p.o + row0 * p.dv;
    const auto ro = make_rsrc(o, rows * p.dv * ES);
    TIn(*ot)[OS] = OT[wave];
    // K = 32 fragment with slot e holding k = 8g + e
    auto ldn = [&](const TIn* row) { return F::ld2(row + 8 * g, row + 8 * g + 4); };
    struct Tile {
        FV q[KB];     // q-hat of token tt + c16 (rows past the block end: padding, dropped)
        f32x4 o[OL];  // o rows of the tile, whole rows (zero past the block end)
    };
    auto load = [&](int tt, Tile& x) {
        const TIn* qt = qh + (size_t)(tt / 16) * KB * 512 + lane * 8;
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) x.q[kk] = F::ld2(qt + kk * 512, qt + kk * 512 + 4);
#pragma unroll
        for (int u = 0; u < OL; ++u) x.o[u] = buf_load<f32x4>(ro, tt * p.dv * ES + (lane + 64 * u) * 16);
    };
    auto run = [&](int tt, const Tile& x) {
        // o rows into the accumulator layout: lane (c16, g) takes o[tt+c16][jt*16+4g .. +3]
#pragma unroll
        for (int u = 0; u < OL; ++u) {
            const int f = lane + 64 * u;
            *(f32x4*)&ot[f / RL][(f % RL) * PE] = x.o[u];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        // M^T fragments are read from LDS for every tile: keeping all of them
        // in registers would cap the waves per SIMD, and with them the loads
        // in flight that bound this pass
        int mo = c16 * MS;
        asm volatile("" : "+v"(mo));
        const TIn* mrow = &MT[0][0] + mo;
#pragma unroll
        for (int jt = 0; jt < JB; ++jt) {
            TIn* cell = &ot[c16][jt * 16 + 4 * g];
            f32x4 acc = Quad<TIn>::to_f32(*(const QV*)cell);
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) acc = F::mma(ldn(mrow + jt * 16 * MS + kk * 32), x.q[kk], acc);
            *(QV*)cell = Quad<TIn>::make(acc);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
        for (int u = 0; u < OL; ++u) {
            const int f = lane + 64 * u;
            buf_store(*(const f32x4*)&ot[f / RL][(f % RL) * PE], ro, tt * p.dv * ES + f * 16);
        }
    };
    Tile b0, b1;
    int tt = wave * 16;
    if (tt < rows) load(tt, b0);
    for (; tt < rows; tt += 128) {
        if (tt + 64 < rows) load(tt + 64, b1);
        run(tt, b0);
        if (tt + 64 >= rows) break;
        if (tt + 128 < rows) load(tt + 128, b0);
        run(tt + 64, b1);
    }
}

template <typename TIn>
hipError_t launch_warm_t(const FwdArgs& a, int* ok, hipStream_t s) {
    const int nblk = a.B * a.H * (a.nseg - 1) * (a.dk / 64);
    const bool pro = a.conv_w > 0;
    if (a.dk == 128 && pro)
        hipLaunchKernelGGL((kla_seg_warm<TIn, 128, true>), dim3(nblk), dim3(64 * kWarmRuns), 0, s, a, ok);
    else if (a.dk == 128)
        hipLaunchKernelGGL((kla_seg_warm<TIn, 128, false>), dim3(nblk), dim3(64 * kWarmRuns), 0, s, a, ok);
    else if (a.dk == 64 && pro)
        hipLaunchKernelGGL((kla_seg_warm<TIn, 64, true>), dim3(nblk), dim3(64 * kWarmRuns), 0, s, a, ok);
    else if (a.dk == 64)
        hipLaunchKernelGGL((kla_seg_warm<TIn, 64, false>), dim3(nblk), dim3(64 * kWarmRuns), 0, s, a, ok);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_mobius_t(const FwdArgs& a, float* P, int* ok, hipStream_t s) {
    int nblk = a.B * a.H * (a.nseg - 1) * (a.seg_len / kSegBlk);
    if (nblk > kMobGrid) nblk = kMobGrid;
    const bool pro = a.conv_w > 0;
    if (a.dk == 128 && pro)
        hipLaunchKernelGGL((kla_seg_mobius<TIn, 128, true>), dim3(nblk), dim3(kMobThreads), 0, s, a, P, ok);
    else if (a.dk == 128)
        hipLaunchKernelGGL((kla_seg_mobius<TIn, 128, false>), dim3(nblk), dim3(kMobThreads), 0, s, a, P, ok);
    else if (a.dk == 64 && pro)
        hipLaunchKernelGGL((kla_seg_mobius<TIn, 64, true>), dim3(nblk), dim3(kMobThreads), 0, s, a, P, ok);
    else if (a.dk == 64)
        hipLaunchKernelGGL((kla_seg_mobius<TIn, 64, false>), dim3(nblk), dim3(kMobThreads), 0, s, a, P, ok);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_correct_t(const FwdArgs& a, hipStream_t s) {
    const int nblk = a.B * a.H * (a.nseg - 1) * ((a.seg_len + kCorrBlk - 1) / kCorrBlk);
    if (a.dk == 128 && a.dv == 128)
        hipLaunchKernelGGL((kla_seg_correct<TIn, 128, 128>), dim3(nblk), dim3(256), 0, s, a);
    else if (a.dk == 128 && a.dv == 64)
        hipLaunchKernelGGL((kla_seg_correct<TIn, 128, 64>), dim3(nblk), dim3(256), 0, s, a);
    else if (a.dk == 64 && a.dv == 64)
        hipLaunchKernelGGL((kla_seg_correct<TIn, 64, 64>), dim3(nblk), dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

SegWorkspace seg_workspace(int B, int H, int T, int dk, int dv, int es, int nseg) {
    const size_t bh = (size_t)B * H;
    SegWorkspace w;
    size_t o = 0;
    w.off_P = o;    o += align256(bh * (size_t)(T / kSegBlk + 1) * dk * 4 * sizeof(float));
    w.off_l0 = o;   o += align256(bh * nseg * dk * sizeof(float));
    w.off_d = o;    o += align256(bh * nseg * dk * sizeof(float));
    w.off_lend = o; o += align256(bh * dk * sizeof(float));
    w.off_m = o;    o += align256(bh * nseg * dk * dv * sizeof(float));
    w.off_qhat = o; o += align256(bh * (size_t)((T + 15) / 16 * 16) * dk * es);
    w.off_ok = o;   o += align256((bh * nseg * 2 + 1) * sizeof(int));  // flags, then the pass-1 counter
    w.bytes = o;
    return w;
}

int fwd_diag_nseg(int B, int H, int T, int dk, int dv, int nvt) {
    (void)dv;
    if (dk != 64 && dk != 128) return 1;
    const long long units = (long long)B * H * nvt;
    if (units >= 192 || T < 2048) return 1;
    int n = (int)((256 + units - 1) / units);
    if (n > T / 1024) n = T / 1024;
    // the extra passes cost about what a workgroup spends on 1,500 tokens:
    // split only when a workgroup saves more than that
    if (n < 2 || T - T / n < 1536) return 1;
    return n;
}

int fwd_diag_seg_len(int T, int nseg) {
    const int l = (T + nseg - 1) / nseg;
    return (l + kSegBlk - 1) / kSegBlk * kSegBlk;
}

hipError_t launch_seg_warm(const FwdArgs& a, int* ok, int dtype, hipStream_t s) {
    return dtype == DT_BF16 ? launch_warm_t<bf16>(a, ok, s) : launch_warm_t<float>(a, ok, s);
}

hipError_t launch_seg_mobius(const FwdArgs& a, float* P, int* ok, int dtype, hipStream_t s) {
    return dtype == DT_BF16 ? launch_mobius_t<bf16>(a, P, ok, s) : launch_mobius_t<float>(a, P, ok, s);
}


hipError_t launch_seg_carry_m(const FwdArgs& a, hipStream_t s) {
    const size_t n = (size_t)a.B * a.H * a.dk * a.dv;
    hipLaunchKernelGGL(kla_seg_carry_m, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_seg_correct(const FwdArgs& a, int dtype, hipStream_t s) {
    return dtype == DT_BF16 ? launch_correct_t<bf16>(a, s) : launch_correct_t<float>(a, s);
}

}  // namespace kla
