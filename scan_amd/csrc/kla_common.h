// kla_common.h -- gfx950 vector types and MFMA operand helpers shared by the
// forward and decode kernels of this library.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

namespace kla {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef bf16 bf16x4 __attribute__((__vector_size__(8)));
typedef bf16 bf16x2 __attribute__((__vector_size__(4)));
typedef short s16x4 __attribute__((__vector_size__(8)));
typedef float f32x4 __attribute__((__vector_size__(16)));
typedef float f32x2 __attribute__((__vector_size__(8)));

// Four fp32 values rounded (RNE) to bf16 and packed, two per conversion
// instruction (a two-element vector conversion maps to v_cvt_pk_bf16_f32;
// element-wise casts of a four-element vector were emitted one value per
// instruction plus a permute).
__device__ __forceinline__ s16x4 pack_bf16x4(float x0, float x1, float x2, float x3) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    const b2 lo = __builtin_convertvector((f2){x0, x1}, b2);
    const b2 hi = __builtin_convertvector((f2){x2, x3}, b2);
    return __builtin_bit_cast(s16x4, (u2){__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)});
}

// A "K32 step" contracts 32 values of the shared dimension with one
// 16x16 output tile; every lane holds 8 consecutive values of its row (A) or
// column (B).  A "K16 step" holds 4.  Both operands of one step are loaded
// with the same lane/slot -> k mapping, so the products pair up regardless of
// the instruction's internal K order.  The 16x16 accumulator layout (lane l
// holds rows 4*(l/16)+e, column l%16) equals the K16 A/B operand layout, so
// an accumulator can feed the next product without passing through LDS.
template <typename T>
struct Mma;

template <>
struct Mma<bf16> {
    typedef bf16x8 K32;
    typedef s16x4 K16;
    static __device__ __forceinline__ K32 ld32(const bf16* p) { return *(const bf16x8*)p; }
    static __device__ __forceinline__ K16 ld16(const bf16* p) { return *(const s16x4*)p; }
    static __device__ __forceinline__ f32x4 mma32(K32 a, K32 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma16(K16 a, K16 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ K16 from_acc(f32x4 x) { return pack_bf16x4(x[0], x[1], x[2], x[3]); }
};

// fp32 operands run on the bf16 matrix cores as split pairs: x = hi + lo
// with hi = bf16(x) and lo = bf16(x - hi), and a product as
// hi*hi + hi*lo + lo*hi, accumulated in fp32 (the dropped lo*lo and the
// rounding of lo are about 2^-17 of |x y| each).  gfx950 has no xf32 MFMA,
// and three bf16 MFMAs take about a fifth of the time of the fp32 MFMAs
// covering the same K.
struct SplitK32 { bf16x8 hi, lo; };
struct SplitK16 { s16x4 hi, lo; };

// hi = bf16(x) (round to nearest even) for a pair, two per conversion
// instruction; the hi values back as floats by a shift or a mask of the
// packed word; lo = bf16(x - hi) likewise (x - hi is exact).
__device__ __forceinline__ void split_pair(float x0, float x1, unsigned& hi, unsigned& lo) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    hi = __builtin_bit_cast(unsigned, __builtin_convertvector((f2){x0, x1}, b2));
    const float h0 = __builtin_bit_cast(float, hi << 16), h1 = __builtin_bit_cast(float, hi & 0xffff0000u);
    lo = __builtin_bit_cast(unsigned, __builtin_convertvector((f2){x0 - h0, x1 - h1}, b2));
}

__device__ __forceinline__ SplitK32 split8(f32x4 a, f32x4 b) {  // slots 0-3 from a, 4-7 from b
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    unsigned h0, h1, h2, h3, l0, l1, l2, l3;
    split_pair(a[0], a[1], h0, l0);
    split_pair(a[2], a[3], h1, l1);
    split_pair(b[0], b[1], h2, l2);
    split_pair(b[2], b[3], h3, l3);
    SplitK32 r;
    r.hi = __builtin_bit_cast(bf16x8, (u4){h0, h1, h2, h3});
    r.lo = __builtin_bit_cast(bf16x8, (u4){l0, l1, l2, l3});
    return r;
}

__device__ __forceinline__ SplitK16 split4(f32x4 a) {
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    unsigned h0, h1, l0, l1;
    split_pair(a[0], a[1], h0, l0);
    split_pair(a[2], a[3], h1, l1);
    SplitK16 r;
    r.hi = __builtin_bit_cast(s16x4, (u2){h0, h1});
    r.lo = __builtin_bit_cast(s16x4, (u2){l0, l1});
    return r;
}

template <>
struct Mma<float> {
    typedef SplitK32 K32;
    typedef SplitK16 K16;
    static __device__ __forceinline__ K32 make32(f32x4 a, f32x4 b) { return split8(a, b); }
    static __device__ __forceinline__ K32 ld32(const float* p) {
        return split8(*(const f32x4*)p, *(const f32x4*)(p + 4));
    }
    static __device__ __forceinline__ K16 ld16(const float* p) { return split4(*(const f32x4*)p); }
    static __device__ __forceinline__ f32x4 mma32(K32 a, K32 b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma16(K16 a, K16 b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.lo, b.hi, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.lo, c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.hi, c, 0, 0, 0);
    }
    static __device__ __forceinline__ K16 from_acc(f32x4 x) { return split4(x); }
};

// The fp32 MFMAs themselves, same interface as Mma<float>: faster than the
// split pairs where the operands are re-read for every product, as in the
// single-role kernels at large dk.
struct MmaF32 {
    struct K32 { f32x4 lo, hi; };
    typedef f32x4 K16;
    static __device__ __forceinline__ K32 make32(f32x4 a, f32x4 b) { return K32{a, b}; }
    static __device__ __forceinline__ K32 ld32(const float* p) {
        return K32{*(const f32x4*)p, *(const f32x4*)(p + 4)};
    }
    static __device__ __forceinline__ K16 ld16(const float* p) { return *(const f32x4*)p; }
    static __device__ __forceinline__ f32x4 mma32(K32 a, K32 b, f32x4 c) {
#pragma unroll
        for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[e], b.lo[e], c, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[e], b.hi[e], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ f32x4 mma16(K16 a, K16 b, f32x4 c) {
#pragma unroll
        for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ K16 from_acc(f32x4 x) { return x; }
};

// Matrix-core operands for the single-role kernels: split pairs for fp32 at
// dk 32 and 64, the fp32 MFMAs at dk 16 and 128 (measured).
template <typename TIn, int DK>
using MmaFor = typename std::conditional<std::is_same<TIn, float>::value && (DK <= 16 || DK >= 128), MmaF32,
                                         Mma<TIn>>::type;

// Eight bf16/f32 values forming one K=32 operand fragment: slots 0-3 hold
// k = 4g..4g+3 of the first 16-block, slots 4-7 the same of the second.
template <typename T> struct Frag;
template <> struct Frag<bf16> {
    typedef bf16x8 V;
    static __device__ __forceinline__ V ld(const bf16* row, int g) { return ld2(row + 4 * g, row + 16 + 4 * g); }
    // slots 0-3 from `lo`, 4-7 from `hi` (for swizzled rows)
    static __device__ __forceinline__ V ld2(const bf16* lo_p, const bf16* hi_p) {
        const s16x4 lo = *(const s16x4*)lo_p;
        const s16x4 hi = *(const s16x4*)hi_p;
        typedef short s16x8 __attribute__((__vector_size__(16)));
        s16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(V, r);
    }
    static __device__ __forceinline__ V from_acc(f32x4 lo, f32x4 hi) {
        V r = {(bf16)lo[0], (bf16)lo[1], (bf16)lo[2], (bf16)lo[3],
               (bf16)hi[0], (bf16)hi[1], (bf16)hi[2], (bf16)hi[3]};
        return r;
    }
    static __device__ __forceinline__ f32x4 mma(V a, V b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Frag<float> {
    typedef SplitK32 V;  // split bf16 pairs, see Mma<float>
    static __device__ __forceinline__ V ld(const float* row, int g) { return ld2(row + 4 * g, row + 16 + 4 * g); }
    static __device__ __forceinline__ V ld2(const float* lo_p, const float* hi_p) {
        return split8(*(const f32x4*)lo_p, *(const f32x4*)hi_p);
    }
    static __device__ __forceinline__ V from_acc(f32x4 lo, f32x4 hi) { return split8(lo, hi); }
    static __device__ __forceinline__ f32x4 mma(V a, V b, f32x4 c) { return Mma<float>::mma32(a, b, c); }
};

// K=32 fragments for the fp32 MFMAs themselves (slot order as Frag<bf16>).
struct FragF32 {
    struct V { f32x4 lo, hi; };
    static __device__ __forceinline__ V ld(const float* row, int g) { return ld2(row + 4 * g, row + 16 + 4 * g); }
    static __device__ __forceinline__ V ld2(const float* lo_p, const float* hi_p) {
        return V{*(const f32x4*)lo_p, *(const f32x4*)hi_p};
    }
    static __device__ __forceinline__ V from_acc(f32x4 lo, f32x4 hi) { return V{lo, hi}; }
    static __device__ __forceinline__ f32x4 mma(V a, V b, f32x4 c) {
        return MmaF32::mma32(MmaF32::K32{a.lo, a.hi}, MmaF32::K32{b.lo, b.hi}, c);
    }
};

// Two consecutive values of the input dtype, as loaded from / stored to HBM.
template <typename T> struct Pair;
template <> struct Pair<bf16> {
    typedef bf16x2 V;
    static __device__ __forceinline__ float lo(V v) { return (float)v[0]; }
    static __device__ __forceinline__ float hi(V v) { return (float)v[1]; }
    static __device__ __forceinline__ V make(float a, float b) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(V, __builtin_convertvector((f2){a, b}, b2));  // one v_cvt_pk_bf16_f32
    }
    static __device__ __forceinline__ V zero() { V r = {(bf16)0.f, (bf16)0.f}; return r; }
};
template <> struct Pair<float> {
    typedef f32x2 V;
    static __device__ __forceinline__ float lo(V v) { return v[0]; }
    static __device__ __forceinline__ float hi(V v) { return v[1]; }
    static __device__ __forceinline__ V make(float a, float b) { V r = {a, b}; return r; }
    static __device__ __forceinline__ V zero() { V r = {0.f, 0.f}; return r; }
};

// Four consecutive values (a row fragment, an output store).
template <typename T> struct Quad;
template <> struct Quad<bf16> {
    typedef bf16x4 V;
    static __device__ __forceinline__ V make(f32x4 x) {
        return __builtin_bit_cast(V, pack_bf16x4(x[0], x[1], x[2], x[3]));
    }
    static __device__ __forceinline__ f32x4 to_f32(V v) {
        return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    }
    static __device__ __forceinline__ V zero() { return make(f32x4{0.f, 0.f, 0.f, 0.f}); }
};
template <> struct Quad<float> {
    typedef f32x4 V;
    static __device__ __forceinline__ V make(f32x4 x) { return x; }
    static __device__ __forceinline__ f32x4 to_f32(V v) { return v; }
    static __device__ __forceinline__ V zero() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
};

// Eight consecutive values (16 bytes of bf16, 32 bytes of fp32).
template <typename T> struct Oct;
template <> struct Oct<bf16> {
    typedef bf16x8 V;
    static __device__ __forceinline__ float get(const V& v, int e) { return (float)v[e]; }
    static __device__ __forceinline__ V zero() {
        V r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = (bf16)0.f;
        return r;
    }
};
template <> struct Oct<float> {
    struct V { f32x4 lo, hi; };
    static __device__ __forceinline__ float get(const V& v, int e) { return e < 4 ? v.lo[e] : v.hi[e - 4]; }
    static __device__ __forceinline__ V zero() { V r; r.lo = f32x4{0.f, 0.f, 0.f, 0.f}; r.hi = r.lo; return r; }
};

// Range-checked loads through a buffer resource.  The descriptor holds a
// 48-bit base, stride 0, a byte range and the gfx9-family format word; a load
// whose (vector offset + immediate offset) falls at or past the range reads
// zero, so chunk tails need no clamped addresses.  Per-token row offsets are
// compile-time constants and fold into the 12-bit immediate field.
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// The base and range must be the same in every lane (they are read from the
// first active lane, which keeps the descriptor in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    const unsigned long long a = (unsigned long long)base;
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)a);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32));
    void* b = (void*)(((unsigned long long)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

template <typename V>
__device__ __forceinline__ V buf_load(__amdgpu_buffer_rsrc_t r, int voff) {
    if constexpr (sizeof(V) == 2) {
        return __builtin_bit_cast(V, (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0));
    } else if constexpr (sizeof(V) == 4) {
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
    } else if constexpr (sizeof(V) == 8) {
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0));
    } else {
        static_assert(sizeof(V) == 16, "2, 4, 8 or 16 bytes");
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
    }
}

// Range-checked store through a buffer resource: a store whose offset falls at
// or past the resource's byte range is dropped, so tails need no branch.
template <typename V>
__device__ __forceinline__ void buf_store(V v, __amdgpu_buffer_rsrc_t r, int voff) {
    if constexpr (sizeof(V) == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, voff, 0, 0);
    } else if constexpr (sizeof(V) == 8) {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, v), r, voff, 0, 0);
    } else {
        static_assert(sizeof(V) == 16, "4, 8 or 16 bytes");
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, voff, 0, 0);
    }
}

// Workgroup barrier that orders LDS only.  __syncthreads() also releases
// global memory, which on gfx9 waits for every vector-memory load in flight
// (vmcnt(0)) and so drains any prefetch at each barrier; waves that exchange
// data only through LDS need just lgkmcnt(0) before the s_barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One exchange of the reduce-scatter over lane mask M of the N values a lane
// still holds: the lane keeps the half chosen by its lane bit, sends the
// other half to its partner and adds the partner's copy of the kept half
// (N == 1: a plain exchange-and-add).  base accumulates the index of the
// first kept value.
template <int N, int M>
__device__ __forceinline__ void reduce_scatter(float* w, int lane, int& base) {
    if constexpr (M >= 1) {
        if constexpr (N > 1) {
            constexpr int H = N / 2;
            const bool hi = (lane & M) != 0;
#pragma unroll
            for (int j = 0; j < H; ++j) {
                const float keep = hi ? w[H + j] : w[j];
                const float send = hi ? w[j] : w[H + j];
                w[j] = keep + __shfl_xor(send, M, 64);
            }
            base += hi ? H : 0;
            reduce_scatter<H, M / 2>(w, lane, base);
        } else {
            w[0] += __shfl_xor(w[0], M, 64);
            reduce_scatter<N, M / 2>(w, lane, base);
        }
    }
}

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Activations of the fused block prologue, in fp32 from the hardware exp2,
// log2 and reciprocal (a few ulp).
constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
__device__ __forceinline__ float act_sigmoid(float x) { return fast_rcp(1.f + fast_exp2(-x * kLog2e)); }
__device__ __forceinline__ float act_silu(float x) { return x * act_sigmoid(x); }
// softplus(x) = max(x, 0) + log1p(e), e = exp(-|x|).  log1p(e) = log(u) e /
// (u - 1) with u = 1 + e rounded, which keeps the relative accuracy of the
// logarithm for small e (Goldberg's log1p identity); e itself once u rounds
// to 1.
__device__ __forceinline__ float act_softplus(float x) {
    const float e = fast_exp2(-__builtin_fabsf(x) * kLog2e);
    const float u = 1.f + e;
    const float l1p = u == 1.f ? e : fast_log2(u) * kLn2 * e / (u - 1.f);
    return __builtin_fmaxf(x, 0.f) + l1p;
}
// One channel of a causal depthwise convolution of up to four taps: w[3] on
// the current token's x0, w[2] on x1 (one token back) ... w[0] on x3.
template <typename W4>
__device__ __forceinline__ float conv4(const W4& w, float b, float x0, float x1, float x2, float x3) {
    return __builtin_fmaf(w[3], x0, __builtin_fmaf(w[2], x1, __builtin_fmaf(w[1], x2, __builtin_fmaf(w[0], x3, b))));
}
// The taps of one channel, right-aligned into four (zero for absent taps).
__device__ __forceinline__ void load_taps4(float (&w)[4], const float* src, int width) {
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = j >= 4 - width ? src[j - (4 - width)] : 0.f;
}

}  // namespace kla
