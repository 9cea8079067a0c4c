// rlk_device.h -- device-side building blocks shared by the forward, backward
// and softcap kernels (gfx950, wave64).
//
// Element -> lane map.  A row of V logits is cut into chunks of 8 consecutive
// elements (one 16-byte load for bf16, two for fp32).  In a workgroup of
// BLOCK threads, lane `tid` owns chunks tid, tid + BLOCK, tid + 2 BLOCK, ...,
// consumed in groups of U chunks.  This map, the group size, the per-lane
// accumulation order and the reduction tree depend only on V and on the
// compile-time BLOCK and U: never on N, on the row stride, on the pointer
// alignment or on the dtype.  So every row's result is deterministic and
// batch-invariant, and an fp32 and a bf16 row holding the same values give
// identical statistics.
//
// Online statistics in base 2 (the single-read scheme of the review comment
// on "Add Triton kernels for vocab-parallel logprobs, entropy and KL",
// DeepSpeed pull request 8838, re-derived here with exp2):
//   a_v  = the statistic input of logit x_v: x_v itself, or with the softcap
//          one of the two forms of cap_value below;
//   sc   = its scale, so that y_v log2(e) = a_v sc + (a constant of the row);
//   mL   = m sc with m the running maximum of a (a rounded constant that is
//          used consistently everywhere, so its rounding cancels), or the
//          fixed reference 0 of the fixed cap form;
//   t_v  = a_v sc - mL (one FMA), S = sum 2^t_v, W = sum 2^t_v t_v.
//   When the maximum grows by d = mL_old - mL_new (< 0):
//          S <- 2^d S,  W <- 2^d (W + d S).
//   Then log p_v = ln2 (t_v - log2 S) and the entropy is
//          H = ln2 (log2 S - W / S).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rlk_launch.h"

namespace rlk {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kClampT = -256.0f;  // 2^-256 is 0 in fp32: clamping t below it is exact
constexpr int kChunk = 8;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float pos_inf() { return __builtin_inff(); }
__device__ __forceinline__ float qnan() { return __builtin_nanf(""); }

// Raw hardware exp2 / reciprocal (v_exp_f32, v_rcp_f32, about 1 ulp).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ---------------------------------------------------------------- dtypes

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct F32 {
    using storage = float;
    static constexpr int kBytes = 4;
};
struct BF16 {
    using storage = uint16_t;
    static constexpr int kBytes = 2;
};
struct F16 {
    using storage = _Float16;
    static constexpr int kBytes = 2;
};
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Round-to-nearest-even pack (v_cvt_pk_bf16_f32 on gfx950; NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v;
    v.x = static_cast<__bf16>(lo);
    v.y = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Cache hints for the bulk row traffic.  Every logit is touched once per
// kernel: an operand larger than the Infinity Cache streams through
// non-temporal loads (NT), which keep it from evicting other data, while one
// that fits is read with ordinary loads, which find what the previous kernel
// left in the cache (kCachedReadBytes).  Stores are non-temporal (a
// compile-time switch).
#ifndef RLK_NT_STORE
#define RLK_NT_STORE 1
#endif
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool NT, typename V>
__device__ __forceinline__ V ld16(const V* p) {
    if (NT) return __builtin_nontemporal_load(p);
    return *p;
}
template <typename V>
__device__ __forceinline__ void st16(V* p, V v) {
    if (RLK_NT_STORE)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// Load one full chunk of 8 elements from a 16-byte aligned address.
template <bool NT>
__device__ __forceinline__ void load_chunk(const float* p, float (&f)[kChunk]) {
    const f32x4 a = ld16<NT>(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = ld16<NT>(reinterpret_cast<const f32x4*>(p) + 1);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
template <bool NT>
__device__ __forceinline__ void load_chunk(const uint16_t* p, float (&f)[kChunk]) {
    const u32x4 w = ld16<NT>(reinterpret_cast<const u32x4*>(p));
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
    f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
    f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}
template <bool NT>
__device__ __forceinline__ void load_chunk(const _Float16* p, float (&f)[kChunk]) {
    const u32x4 w = ld16<NT>(reinterpret_cast<const u32x4*>(p));
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f16x2_t h = __builtin_bit_cast(f16x2_t, ws[i]);
        f[2 * i] = static_cast<float>(h.x);
        f[2 * i + 1] = static_cast<float>(h.y);
    }
}
__device__ __forceinline__ float load_one(const float* p) { return *p; }
__device__ __forceinline__ float load_one(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load_one(const _Float16* p) { return static_cast<float>(*p); }

// Store one full chunk of 8 values to a 16-byte aligned address.
__device__ __forceinline__ void store_chunk(float* p, const float (&f)[kChunk]) {
    const f32x4 a = {f[0], f[1], f[2], f[3]};
    const f32x4 b = {f[4], f[5], f[6], f[7]};
    st16(reinterpret_cast<f32x4*>(p), a);
    st16(reinterpret_cast<f32x4*>(p) + 1, b);
}
__device__ __forceinline__ void store_chunk(uint16_t* p, const float (&f)[kChunk]) {
    const u32x4 w = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                     pack_bf16x2(f[6], f[7])};
    st16(reinterpret_cast<u32x4*>(p), w);
}
// Round-to-nearest-even fp16 pack (overflow gives +-inf, NaN stays NaN).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2_t v;
    v.x = static_cast<_Float16>(lo);
    v.y = static_cast<_Float16>(hi);
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ void store_chunk(_Float16* p, const float (&f)[kChunk]) {
    const u32x4 w = {pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3]), pack_f16x2(f[4], f[5]),
                     pack_f16x2(f[6], f[7])};
    st16(reinterpret_cast<u32x4*>(p), w);
}
__device__ __forceinline__ void store_one(float* p, float f) { *p = f; }
__device__ __forceinline__ void store_one(uint16_t* p, float f) { *p = f32_to_bf16(f); }
__device__ __forceinline__ void store_one(_Float16* p, float f) { *p = static_cast<_Float16>(f); }

// ---------------------------------------------------------------- softcap
//
// "Final Logit Softcap", Summary: y = c tanh(x / c), dy/dx = 1 - tanh^2.
//
// Fused prologue form.  With r = 1 / (1 + 2^(k x)), k = -2 log2(e) / c:
//   tanh(x / c) = 2 r - 1   and   1 - tanh^2(x / c) = 4 r (1 - r),
// so y log2(e) = sc r - c log2(e) with sc = 2 c log2(e).  Two forms of the
// statistic input (CapMode in rlk_launch.h):
//   online: a = r with the scale sc; the constant -c log2(e) is common to
//           every logit of the row and cancels exactly in t = y log2(e) - max;
//   fixed:  a = t = (y - c) log2(e) = sc (r - 1) = -sc / (1 + 2^(-k x))
//           itself (scale 1, reference 0), one FMA and a reciprocal away
//           from the exponential: -1 / (1/sc + 2^(-k x) / sc).
// Both ends are exact (x = +inf: r = 1, t = 0; x = -inf: r = 0, i.e.
// y = -c; slope 0 at both).  The absolute error of a is about 1e-7 (online)
// or 1e-7 sc (fixed); the softmax depends only on absolute errors of y.
struct CapArgs {
    float k;     // -2 log2(e) / c
    float isc;   // fixed form: 1 / sc
    float span;  // fixed form, backward: w where 2^(-k x) = 0, i.e. rcp(isc) (fixed_span)
    const float* tab = nullptr;  // table forms: sc/2 + t(|x|) by 16-bit magnitude (LDS)
    float half = 0.0f;           // odd forms: sc/2
};

// Table forms.  With w(x) = sc / (1 + 2^(-k x)), w(x) + w(-x) = sc, so
// t(x) + sc/2 = sc/2 - w(x) is odd in x: its value at |x| with the sign bit
// of x.  hi16 holds the 16-bit pattern in bits 31..16; a NaN pattern reads
// a NaN entry, +-inf read +-sc/2.
// The magnitude of m with the sign bit of s.
__device__ __forceinline__ float with_sign(float m, uint32_t s) {
    return __uint_as_float((s & 0x80000000u) | (__float_as_uint(m) & 0x7fffffffu));
}
// The table holds magnitudes (sign bits clear: tab_entry), so a lookup only
// ors in the sign bit of x, with the bits of with_sign(entry, x).
__device__ __forceinline__ float tab_entry(float v) { return fabsf(v); }
__device__ __forceinline__ float tab_lookup(const float* tab, uint32_t hi16) {
    return __uint_as_float((hi16 & 0x80000000u) | __float_as_uint(tab[(hi16 >> 16) & 0x7fffu]));
}
template <typename S>
__device__ __forceinline__ float from_bits16(uint32_t b);
template <>
__device__ __forceinline__ float from_bits16<uint16_t>(uint32_t b) {
    return __uint_as_float(b << 16);
}
template <>
__device__ __forceinline__ float from_bits16<_Float16>(uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

template <int CAP>
__device__ __forceinline__ float cap_value(float x, CapArgs c) {
    if (CAP == kCapOnline) return rcp(1.0f + ex2(x * c.k));
    if (CAP == kCapFixed) return -rcp(__builtin_fmaf(ex2(-(x * c.k)), c.isc, c.isc));
    if (CAP == kCapFixedOdd)
        return with_sign(c.half + cap_value<kCapFixed>(fabsf(x), c), __float_as_uint(x));
    // x is a bf16 / fp16 value widened to float: back to its 16-bit pattern
    if (CAP == kCapTableB) return tab_lookup(c.tab, __float_as_uint(x));
    if (CAP == kCapTableH)
        return tab_lookup(c.tab, static_cast<uint32_t>(__builtin_bit_cast(
                                     uint16_t, static_cast<_Float16>(x))) << 16);
    return x;
}

// Statistic input a and the slope 1 - tanh^2 up to a factor fixed per cap
// (slope_factor): s = r (1 - r) in the online form.  Fixed form: with
// q = 2^(-k x) and w = sc / (1 + q) (so a = -w), sc (1 - r) = w and
// sc r = sc - w, so s = (sc - w) w = r (1 - r) sc^2, with sc taken as the
// very w of q = 0 (c.span = fixed_span): s is exactly 0 at x = -inf
// (q = 0, w = span) and at x = +inf (q = inf, w = 0), and a NaN x stays NaN
// through w.  Towards x = -inf the difference keeps its absolute accuracy
// (about 2^-23 sc^2 in s, 2^-21 in the slope), not a relative one; the
// gradient's error bounds are absolute there.
template <int CAP>
__device__ __forceinline__ float cap_value_slope(float x, CapArgs c, float& s) {
    if (CAP == kCapOnline) {
        const float r = rcp(1.0f + ex2(x * c.k));
        s = __builtin_fmaf(-r, r, r);
        return r;
    }
    if (CAP == kCapFixed) {
        const float q = ex2(-(x * c.k));
        const float w = rcp(__builtin_fmaf(q, c.isc, c.isc));
        s = (c.span - w) * w;
        return -w;
    }
    s = 1.0f;
    return x;
}

// The fixed form's span for cap_value_slope: its w at q = 0, by the same
// reciprocal, so that the slope vanishes exactly there.
__device__ __forceinline__ float fixed_span(float isc) { return rcp(__builtin_fmaf(0.0f, isc, isc)); }

// The slope is slope_factor * s: 4 (online form), 4 / sc^2 (fixed form).
template <int CAP>
__device__ __forceinline__ float slope_factor(CapArgs c) {
    return CAP == kCapFixed ? 4.0f * c.isc * c.isc : 4.0f;
}

// Standalone form, accurate in RELATIVE terms (the output y itself is
// compared at 1e-5 relative).  For |u| < 0.55 an odd polynomial
// u + u^3 P(u^2) whose five coefficients were fitted to tanh on [0, 0.55]
// (weighted least squares, max relative error 7e-8 in fp32 Horner form);
// above, tanh|u| = (1 - e) / (1 + e) with e = 2^(-2 log2(e) |u|) <= 1/3 and
// the slope 4 e / (1 + e)^2 (no cancellation near saturation).
__device__ __forceinline__ float tanh_precise(float u, float* slope) {
    const float au = fabsf(u);
    const float u2 = u * u;
    float p = -6.0180192813277245e-03f;
    p = __builtin_fmaf(p, u2, 2.0877523347735405e-02f);
    p = __builtin_fmaf(p, u2, -5.3801555186510086e-02f);
    p = __builtin_fmaf(p, u2, 1.3332062959671020e-01f);
    p = __builtin_fmaf(p, u2, -3.3333301544189453e-01f);
    const float ts = __builtin_fmaf(u * u2, p, u);
    const float e = ex2(-2.0f * kLog2e * au);
    const float r = rcp(1.0f + e);
    const float tl = __builtin_copysignf(__builtin_fmaf(-e, r, r), u);
    const bool small = au < 0.55f;
    *slope = small ? __builtin_fmaf(-ts, ts, 1.0f) : 4.0f * e * r * r;
    return small ? ts : tl;
}

// ------------------------------------------------------ row streaming
//
// A group is U chunks of 8 elements for lane tid: chunk (g0 + u BLOCK + tid).
// Fast groups (every chunk inside the row, 16-byte aligned rows) are loaded
// as raw 16-byte vectors and kept packed until they are consumed, so the
// next group's loads can be in flight while the current one is computed.
template <typename S, int U>
struct RawGroup;
template <int U>
struct RawGroup<uint16_t, U> {
    u32x4 v[U];
};
template <int U>
struct RawGroup<float, U> {
    f32x4 v[U][2];
};
template <int U>
struct RawGroup<_Float16, U> {
    u32x4 v[U];
};

// Lane of the calling thread among the BLOCK threads that walk one row.
// MULTI: the workgroup walks several rows side by side, BLOCK threads each
// (the table forward); otherwise the workgroup is BLOCK threads.
template <int BLOCK, bool MULTI>
__device__ __forceinline__ int row_lane() {
    static_assert((BLOCK & (BLOCK - 1)) == 0, "BLOCK must be a power of two");
    return MULTI ? static_cast<int>(threadIdx.x) & (BLOCK - 1) : static_cast<int>(threadIdx.x);
}
// The table forms run in the multi-row workgroup.
constexpr bool multi_row(int CAP) { return CAP == kCapTableB || CAP == kCapTableH; }

template <int BLOCK, int U, bool NT, bool MULTI = false>
__device__ __forceinline__ void raw_load(const uint16_t* __restrict__ row, int64_t g0,
                                         RawGroup<uint16_t, U>& r) {
#pragma unroll
    for (int u = 0; u < U; ++u)
        r.v[u] = ld16<NT>(reinterpret_cast<const u32x4*>(
            row + (g0 + u * BLOCK + row_lane<BLOCK, MULTI>()) * kChunk));
}
template <int BLOCK, int U, bool NT, bool MULTI = false>
__device__ __forceinline__ void raw_load(const _Float16* __restrict__ row, int64_t g0,
                                         RawGroup<_Float16, U>& r) {
#pragma unroll
    for (int u = 0; u < U; ++u)
        r.v[u] = ld16<NT>(reinterpret_cast<const u32x4*>(
            row + (g0 + u * BLOCK + row_lane<BLOCK, MULTI>()) * kChunk));
}
// fp32 pieces hold quads: chunk slot u of lane t is quads t and BLOCK + t of
// the slot's BLOCK chunks (piece_col), so that each load covers 1 KB per wave.
template <int BLOCK, int U, bool NT, bool MULTI = false>
__device__ __forceinline__ void raw_load(const float* __restrict__ row, int64_t g0,
                                         RawGroup<float, U>& r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const f32x4* p = reinterpret_cast<const f32x4*>(row + (g0 + u * BLOCK) * kChunk) +
                         row_lane<BLOCK, MULTI>();
        r.v[u][0] = ld16<NT>(p);
        r.v[u][1] = ld16<NT>(p + BLOCK);
    }
}

// Column (from the piece's first chunk g0) of value e of chunk slot u that
// lane t holds in a one-shot backward piece.  16-bit logits: chunk g0 + u
// BLOCK + t, its 8 values side by side.  fp32 logits in a full piece (QUADS):
// values 0..3 are quad t and values 4..7 quad BLOCK + t of the slot's 2 BLOCK
// quads, so each of a wave's two 16-byte loads or stores per slot covers 1 KB
// contiguous; a chunk's two quads side by side would make each store write
// every other 16 bytes (the fp32 backward then moved 3.3x fewer bytes per
// second).  Partial pieces keep the chunk layout (tail_values, store_group).
template <int BLOCK, bool QUADS>
__device__ __forceinline__ int64_t piece_col(int64_t g0, int u, int t, int e) {
    if (QUADS) {
        const int64_t q0 = (g0 + static_cast<int64_t>(u) * BLOCK) * kChunk + 4 * t;
        return e < 4 ? q0 + e : q0 + 4 * BLOCK + (e - 4);
    }
    return (g0 + static_cast<int64_t>(u) * BLOCK + t) * kChunk + e;
}
template <typename S, bool FULL>
constexpr bool piece_quads() {
    return FULL && sizeof(S) == 4;
}
// Inverse of piece_col: the lane-order index (u BLOCK + t) kChunk + e of the
// value at column c of the piece (0 <= c < BLOCK U kChunk).
template <int BLOCK, bool QUADS>
__device__ __forceinline__ int piece_slot(int c) {
    if (!QUADS) return c;
    const int q = c >> 2, r = q % (2 * BLOCK);
    const int half = r >= BLOCK ? 1 : 0;
    return ((q / (2 * BLOCK)) * BLOCK + (r - half * BLOCK)) * kChunk + half * 4 + (c & 3);
}
// The row walks (for_each_group, for_each_group2) read their full groups
// through a buffer resource per group: its base is the group's first byte,
// the same for every lane of a wave (each wave walks one row; readfirstlane
// keeps it in scalar registers), its range the group's bytes, and each lane
// adds a 32-bit offset, so a group costs no 64-bit vector address arithmetic
// (the KL forward's loop lost 2% of its VALU instructions).  The policy bit
// nt (2) is the non-temporal load's; a range shorter than the group (bytes)
// reads 0 beyond it.  The backward's one-shot pieces keep
// raw_load's global loads, with which they measured faster (logprobs
// backward, bf16 [8192, 151936]: 743 us against 761 us).
template <typename S>
__device__ __forceinline__ void* wave_base(const S* p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    return reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
}
template <int BLOCK, int U, typename S>
constexpr int group_bytes() {
    return BLOCK * U * kChunk * static_cast<int>(sizeof(S));
}
template <typename S>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t group_rsrc(const S* row, int64_t g0, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(wave_base(row + g0 * kChunk), 0, bytes, 0x00020000);
}
template <int BLOCK, bool MULTI, typename S>
__device__ __forceinline__ int lane_offset(int u) {
    return (u * BLOCK + row_lane<BLOCK, MULTI>()) * kChunk * static_cast<int>(sizeof(S));
}
template <int BLOCK, int U, bool NT, bool MULTI = false>
__device__ __forceinline__ void raw_load_walk(const uint16_t* __restrict__ row, int64_t g0,
                                              RawGroup<uint16_t, U>& r,
                                              int bytes = group_bytes<BLOCK, U, uint16_t>()) {
    const __amdgpu_buffer_rsrc_t rs = group_rsrc(row, g0, bytes);
#pragma unroll
    for (int u = 0; u < U; ++u)
        r.v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rs, lane_offset<BLOCK, MULTI, uint16_t>(u), 0,
                                               NT ? 2 : 0));
}
template <int BLOCK, int U, bool NT, bool MULTI = false>
__device__ __forceinline__ void raw_load_walk(const _Float16* __restrict__ row, int64_t g0,
                                              RawGroup<_Float16, U>& r,
                                              int bytes = group_bytes<BLOCK, U, _Float16>()) {
    const __amdgpu_buffer_rsrc_t rs = group_rsrc(row, g0, bytes);
#pragma unroll
    for (int u = 0; u < U; ++u)
        r.v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rs, lane_offset<BLOCK, MULTI, _Float16>(u), 0,
                                               NT ? 2 : 0));
}
// fp32 walks.  A lane's chunk is 32 bytes, so its two halves side by side
// would make each of the wave's two loads read every other 16 bytes over
// 2 KB (a read-only probe over fp32 rows: 5.7 TB/s against 7.0 TB/s for
// contiguous 16-byte words).  Instead each load reads 1 KB of the wave's 64
// chunks contiguous: the first load chunks 0..31, lanes 0..31 their first
// and lanes 32..63 their second halves, the second load chunks 32..63 alike.
// One lane-32 swap per dword (raw_unpack of a WalkF32) then gives every lane
// both halves of its own chunk, the element-to-lane map of the 16-bit walks
// (so fp32 and 16-bit rows of the same values still give the same bits).
// Every lane of the wave takes part (whole waves walk a row).
template <int U>
struct WalkF32 {
    f32x4 v[U][2];
};
template <typename S, int U>
struct WalkGroupT {
    using type = RawGroup<S, U>;
};
template <int U>
struct WalkGroupT<float, U> {
    using type = WalkF32<U>;
};
template <typename S, int U>
using WalkGroup = typename WalkGroupT<S, U>::type;
template <int BLOCK, int U, bool NT, bool MULTI = false>
__device__ __forceinline__ void raw_load_walk(const float* __restrict__ row, int64_t g0,
                                              WalkF32<U>& r,
                                              int bytes = group_bytes<BLOCK, U, float>()) {
    const __amdgpu_buffer_rsrc_t rs = group_rsrc(row, g0, bytes);
    const int t = row_lane<BLOCK, MULTI>(), l = t & 63;
    // chunk (t - l) + (l & 31) of the slot, half l >> 5; then 32 chunks on
    const int lane_off = ((t - l) + (l & 31)) * kChunk * 4 + (l >> 5) * 16;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int off = u * BLOCK * kChunk * 4 + lane_off;
        r.v[u][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rs, off, 0, NT ? 2 : 0));
        r.v[u][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rs, off + 32 * kChunk * 4, 0, NT ? 2 : 0));
    }
}
template <int U>
__device__ __forceinline__ void raw_unpack(const RawGroup<uint16_t, U>& r, float (&a)[U][kChunk]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        a[u][0] = bf16_lo(r.v[u].x); a[u][1] = bf16_hi(r.v[u].x);
        a[u][2] = bf16_lo(r.v[u].y); a[u][3] = bf16_hi(r.v[u].y);
        a[u][4] = bf16_lo(r.v[u].z); a[u][5] = bf16_hi(r.v[u].z);
        a[u][6] = bf16_lo(r.v[u].w); a[u][7] = bf16_hi(r.v[u].w);
    }
}
template <int U>
__device__ __forceinline__ void raw_unpack(const RawGroup<_Float16, U>& r, float (&a)[U][kChunk]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t ws[4] = {r.v[u].x, r.v[u].y, r.v[u].z, r.v[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f16x2_t h = __builtin_bit_cast(f16x2_t, ws[i]);
            a[u][2 * i] = static_cast<float>(h.x);
            a[u][2 * i + 1] = static_cast<float>(h.y);
        }
    }
}
template <int U>
__device__ __forceinline__ void raw_unpack(const RawGroup<float, U>& r, float (&a)[U][kChunk]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        a[u][0] = r.v[u][0].x; a[u][1] = r.v[u][0].y; a[u][2] = r.v[u][0].z; a[u][3] = r.v[u][0].w;
        a[u][4] = r.v[u][1].x; a[u][5] = r.v[u][1].y; a[u][6] = r.v[u][1].z; a[u][7] = r.v[u][1].w;
    }
}
// Lane m < 32 loaded the first half of chunk m and lane m + 32 its second
// half (first load); lane m - 32 the first and lane m the second half of
// chunk m >= 32 (second load): the swap of lanes 32..63 of the first with
// lanes 0..31 of the second gives each lane its chunk's halves in order.
template <int U>
__device__ __forceinline__ void raw_unpack(const WalkF32<U>& r, float (&a)[U][kChunk]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float p[4] = {r.v[u][0].x, r.v[u][0].y, r.v[u][0].z, r.v[u][0].w};
        const float q[4] = {r.v[u][1].x, r.v[u][1].y, r.v[u][1].z, r.v[u][1].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[i]),
                                                            __float_as_uint(q[i]), false, false);
            a[u][i] = __uint_as_float(w[0]);
            a[u][4 + i] = __uint_as_float(w[1]);
        }
    }
}
// Values of one group that is not a full aligned group (the row's tail, or
// every group of a row that is not 16-byte aligned).  Chunks that lie wholly
// inside an aligned row still use one vector load; the remaining elements are
// loaded from clamped (always valid) addresses without branches, so all loads
// are in flight together, and slots beyond V become -inf (they contribute
// exactly 0; consumers clamp t before any 0 * t in tail groups).  With a
// cap the in-range values are mapped to their statistic input (cap_value)
// while padding stays -inf.
template <int BLOCK, int U, typename S, int CAP, bool ALIGNED, bool NT>
__device__ __forceinline__ void tail_values(const S* __restrict__ row, int64_t V, int64_t nfull,
                                            int64_t g0, CapArgs ca, float (&a)[U][kChunk]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t c = g0 + u * BLOCK + row_lane<BLOCK, multi_row(CAP)>();
        if (ALIGNED && c < nfull) {
            load_chunk<NT>(row + c * kChunk, a[u]);
            if (CAP != kCapNone) {
#pragma unroll
                for (int e = 0; e < kChunk; ++e) a[u][e] = cap_value<CAP>(a[u][e], ca);
            }
        } else if (c * kChunk >= V) {
#pragma unroll
            for (int e = 0; e < kChunk; ++e) a[u][e] = neg_inf();
        } else {
            float v[kChunk];
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                const int64_t col = c * kChunk + e;
                v[e] = load_one(row + (col < V ? col : V - 1));
            }
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                const int64_t col = c * kChunk + e;
                const float w = cap_value<CAP>(v[e], ca);
                a[u][e] = col < V ? w : neg_inf();
            }
        }
    }
}
// Fast-group counterpart: unpack the raw vectors (and apply the cap).
// G: RawGroup (pieces) or WalkGroup (row walks).
template <int U, typename S, int CAP, typename G>
__device__ __forceinline__ void fast_values(const G& r, CapArgs ca, float (&a)[U][kChunk]) {
    if constexpr (CAP == kCapTableB || CAP == kCapTableH) {
        static_assert(sizeof(S) == 2, "table forms read 16-bit logits");
        // straight from the packed words: element 2i in the low half
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t ws[4] = {r.v[u].x, r.v[u].y, r.v[u].z, r.v[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[u][2 * i] = tab_lookup(ca.tab, ws[i] << 16);
                a[u][2 * i + 1] = tab_lookup(ca.tab, ws[i]);
            }
        }
        return;
    }
    raw_unpack(r, a);
    if (CAP != kCapNone) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < kChunk; ++e) a[u][e] = cap_value<CAP>(a[u][e], ca);
    }
}

// Walk a row group by group, calling f(g0, full, a) with the values of each
// group in order.  Full aligned groups are loaded as raw 16-byte vectors; with
// PIPE two register buffers alternate so that the next group's loads are in
// flight while the current group is consumed.  The order in which f sees the
// groups, and the values, are the same for every path.
//
// The last group of an aligned row of whole chunks (V a multiple of 8) that
// does not fill a group is read the same way, through a resource that ends
// at the row's end: its chunks are each wholly inside the row or wholly
// beyond it (read as 0, then set to -inf, as tail_values does), so it is
// prefetched behind the last full group instead of being loaded after it,
// and f receives the values tail_values would give (full = false).  (The
// two-row walk below keeps tail_values for that group: the prefetch took
// the KL forward from 116 to 136 VGPRs and measured 1.4% slower.)
//
// gbeg / gend restrict the walk to the groups [gbeg, gend) of the row (a
// column segment); -1 for gend means "to the end of the row".
template <int BLOCK, int U, bool MULTI>
__device__ __forceinline__ void beyond_row(int64_t g0, int64_t nchunks, float (&a)[U][kChunk]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (g0 + u * BLOCK + row_lane<BLOCK, MULTI>() >= nchunks) {
#pragma unroll
            for (int e = 0; e < kChunk; ++e) a[u][e] = neg_inf();
        }
}
template <int BLOCK, int U, typename S, int CAP, bool ALIGNED, bool PIPE, bool NT, typename F>
__device__ __forceinline__ void for_each_group(const S* __restrict__ row, int64_t V, CapArgs k, F&& f,
                                               int64_t gbeg = 0, int64_t gend = -1) {
    constexpr bool MULTI = multi_row(CAP);
    const int64_t step = (int64_t)U * BLOCK;
    const int64_t nchunks = (V + kChunk - 1) / kChunk, nfull = V / kChunk;
    const int64_t ngroups = (nchunks + step - 1) / step;
    if (gend < 0 || gend > ngroups) gend = ngroups;
    const int64_t nfg_row = ALIGNED ? nfull / step : 0;  // full aligned groups of the row
    const int64_t nfg = nfg_row < gend ? nfg_row : gend;
    // the row's last group, partial, read like a full one
    const bool last_raw =
        ALIGNED && nfull == nchunks && nfg_row < ngroups && gend == ngroups && gbeg <= nfg_row;
    const int64_t nraw = nfg + (last_raw ? 1 : 0);
    const int last_bytes =
        last_raw ? static_cast<int>((nchunks - nfg_row * step) * kChunk * sizeof(S)) : 0;
    // (g beyond the walk: a resource of no bytes, which reads 0 and touches
    // no memory; see the loop below)
    auto load = [&](int64_t g, WalkGroup<S, U>& r) {
        raw_load_walk<BLOCK, U, NT, MULTI>(
            row, g * step, r, g < nfg ? group_bytes<BLOCK, U, S>() : (g < nraw ? last_bytes : 0));
    };
    auto full = [&](int64_t g, const WalkGroup<S, U>& r) {
        float a[U][kChunk];
        fast_values<U, S, CAP>(r, k, a);
        f(g * step, true, a);
    };
    auto last = [&](int64_t g, const WalkGroup<S, U>& r) {
        float a[U][kChunk];
        fast_values<U, S, CAP>(r, k, a);
        beyond_row<BLOCK, U, MULTI>(g * step, nchunks, a);
        f(g * step, false, a);
    };
    int64_t gi = gbeg;
    if (PIPE && gi < nraw) {
        WalkGroup<S, U> A, B;
        load(gi, A);
        // The next-but-one group is loaded unconditionally (an empty range
        // past the walk): behind a branch, the compiler's wait for the
        // current group merged both paths and also waited for the loads
        // just issued.  The scheduling barriers keep each group's loads
        // ahead of the other group's consumption, which the scheduler
        // otherwise hoisted above them: two groups stay in flight.
        for (; gi + 1 < nfg; gi += 2) {
            load(gi + 1, B);
            __builtin_amdgcn_sched_barrier(0);
            full(gi, A);
            load(gi + 2, A);
            __builtin_amdgcn_sched_barrier(0);
            full(gi + 1, B);
        }
        if (gi + 1 == nfg) {  // one full group left (in A); the last one behind it
            if (last_raw) load(nfg, B);
            full(gi, A);
            ++gi;
        } else if (last_raw) {  // gi == nfg: the last group is in A
            B = A;
        }
        if (last_raw) {
            last(gi, B);
            ++gi;
        }
    } else {
        for (; gi < nraw; ++gi) {
            WalkGroup<S, U> A;
            load(gi, A);
            if (gi < nfg)
                full(gi, A);
            else
                last(gi, A);
        }
    }
    for (; gi < gend; ++gi) {
        float a[U][kChunk];
        tail_values<BLOCK, U, S, CAP, ALIGNED, NT>(row, V, nfull, gi * step, k, a);
        f(gi * step, false, a);
    }
}

// Same walk over two rows in lockstep (KL: policy and reference).
template <int BLOCK, int U, typename S, int CAPA, int CAPB, bool ALIGNED, bool PIPE, bool NT,
          typename F>
__device__ __forceinline__ void for_each_group2(const S* __restrict__ ra, const S* __restrict__ rb,
                                                int64_t V, CapArgs ka, CapArgs kb, F&& f,
                                                int64_t gbeg = 0, int64_t gend = -1) {
    const int64_t step = (int64_t)U * BLOCK;
    const int64_t nchunks = (V + kChunk - 1) / kChunk, nfull = V / kChunk;
    const int64_t ngroups = (nchunks + step - 1) / step;
    if (gend < 0 || gend > ngroups) gend = ngroups;
    const int64_t nfg_row = ALIGNED ? nfull / step : 0;
    const int64_t nfg = nfg_row < gend ? nfg_row : gend;
    int64_t gi = gbeg;
    if (PIPE && gi < nfg) {
        WalkGroup<S, U> A0, B0, A1, B1;
        raw_load_walk<BLOCK, U, NT>(ra, gi * step, A0);
        raw_load_walk<BLOCK, U, NT>(rb, gi * step, B0);
        // unconditional loads and scheduling barriers as in for_each_group
        for (; gi + 1 < nfg; gi += 2) {
            raw_load_walk<BLOCK, U, NT>(ra, (gi + 1) * step, A1);
            raw_load_walk<BLOCK, U, NT>(rb, (gi + 1) * step, B1);
            __builtin_amdgcn_sched_barrier(0);
            {
                float a[U][kChunk], b[U][kChunk];
                fast_values<U, S, CAPA>(A0, ka, a);
                fast_values<U, S, CAPB>(B0, kb, b);
                f(gi * step, true, a, b);
            }
            const int next = gi + 2 < nfg ? group_bytes<BLOCK, U, S>() : 0;
            raw_load_walk<BLOCK, U, NT>(ra, (gi + 2) * step, A0, next);
            raw_load_walk<BLOCK, U, NT>(rb, (gi + 2) * step, B0, next);
            __builtin_amdgcn_sched_barrier(0);
            {
                float a[U][kChunk], b[U][kChunk];
                fast_values<U, S, CAPA>(A1, ka, a);
                fast_values<U, S, CAPB>(B1, kb, b);
                f((gi + 1) * step, true, a, b);
            }
        }
        if (gi < nfg) {
            float a[U][kChunk], b[U][kChunk];
            fast_values<U, S, CAPA>(A0, ka, a);
            fast_values<U, S, CAPB>(B0, kb, b);
            f(gi * step, true, a, b);
            ++gi;
        }
    } else {
        for (; gi < nfg; ++gi) {
            WalkGroup<S, U> A, B;
            raw_load_walk<BLOCK, U, NT>(ra, gi * step, A);
            raw_load_walk<BLOCK, U, NT>(rb, gi * step, B);
            float a[U][kChunk], b[U][kChunk];
            fast_values<U, S, CAPA>(A, ka, a);
            fast_values<U, S, CAPB>(B, kb, b);
            f(gi * step, true, a, b);
        }
    }
    for (; gi < gend; ++gi) {
        float a[U][kChunk], b[U][kChunk];
        tail_values<BLOCK, U, S, CAPA, ALIGNED, NT>(ra, V, nfull, gi * step, ka, a);
        tail_values<BLOCK, U, S, CAPB, ALIGNED, NT>(rb, V, nfull, gi * step, kb, b);
        f(gi * step, false, a, b);
    }
}

// Stores of a full piece (every chunk inside an aligned row) through a buffer
// resource whose base is the piece's first element, with cache policy CPOL.
// Offsets are relative to the piece, so rows of any length fit the 32-bit
// offsets.  Two policies are used (kCpolStream, kCpolWriteThrough below).
constexpr int kCpolStream = 2;             // nt
constexpr int kCpolWriteThrough = 16 | 2;  // sc1 | nt: system scope, streaming
// With CUT, the first `skip` chunks of the piece are not stored: their offset
// is the end of the buffer, where its range check drops the stores.  fp32
// pieces are stored in quads (piece_col).
template <int BLOCK, int U, typename S, int CPOL, bool CUT = false>
__device__ __forceinline__ void store_piece(S* __restrict__ piece, const float (&v)[U][kChunk],
                                            uint32_t skip = 0) {
    constexpr uint32_t kChunkBytes = kChunk * sizeof(S);
    constexpr uint32_t kBytes = BLOCK * U * kChunkBytes;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(static_cast<void*>(piece), 0, kBytes, 0x00020000);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (sizeof(S) == 4) {
            // quads 2 u BLOCK + t and (2 u + 1) BLOCK + t; with CUT the
            // first 2 skip quads are dropped
            const uint32_t q0 = 2 * u * BLOCK + threadIdx.x, q1 = q0 + BLOCK;
            const uint32_t off0 = (!CUT || q0 >= 2 * skip) ? q0 * 16u : kBytes;
            const uint32_t off1 = (!CUT || q1 >= 2 * skip) ? q1 * 16u : kBytes;
            const u32x4 a = {__float_as_uint(v[u][0]), __float_as_uint(v[u][1]),
                             __float_as_uint(v[u][2]), __float_as_uint(v[u][3])};
            const u32x4 b = {__float_as_uint(v[u][4]), __float_as_uint(v[u][5]),
                             __float_as_uint(v[u][6]), __float_as_uint(v[u][7])};
            __builtin_amdgcn_raw_buffer_store_b128(a, rs, off0, 0, CPOL);
            __builtin_amdgcn_raw_buffer_store_b128(b, rs, off1, 0, CPOL);
        } else {
            const uint32_t ci = u * BLOCK + threadIdx.x;
            const uint32_t off = (!CUT || ci >= skip) ? ci * kChunkBytes : kBytes;
            u32x4 w;
            if constexpr (std::is_same_v<S, uint16_t>)
                w = u32x4{pack_bf16x2(v[u][0], v[u][1]), pack_bf16x2(v[u][2], v[u][3]),
                          pack_bf16x2(v[u][4], v[u][5]), pack_bf16x2(v[u][6], v[u][7])};
            else
                w = u32x4{pack_f16x2(v[u][0], v[u][1]), pack_f16x2(v[u][2], v[u][3]),
                          pack_f16x2(v[u][4], v[u][5]), pack_f16x2(v[u][6], v[u][7])};
            __builtin_amdgcn_raw_buffer_store_b128(w, rs, off, 0, CPOL);
        }
    }
}

// Stores of a full fp32 group of a row walk in the layout of its loads
// (raw_load_walk): the lane-32 swap undoes raw_unpack's, so each of the
// wave's two stores per chunk slot writes 1 KB contiguous.  Every lane of
// the wave takes part.
template <int BLOCK, int U>
__device__ __forceinline__ void store_walk_f32(float* __restrict__ row, int64_t g0,
                                               const float (&v)[U][kChunk]) {
    const __amdgpu_buffer_rsrc_t rs = group_rsrc(row, g0, group_bytes<BLOCK, U, float>());
    const int t = row_lane<BLOCK, false>(), l = t & 63;
    const int lane_off = ((t - l) + (l & 31)) * kChunk * 4 + (l >> 5) * 16;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        uint32_t p[4], q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[u][i]),
                                                            __float_as_uint(v[u][4 + i]), false,
                                                            false);
            p[i] = w[0];
            q[i] = w[1];
        }
        const int off = u * BLOCK * kChunk * 4 + lane_off;
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{p[0], p[1], p[2], p[3]}, rs, off, 0,
                                               RLK_NT_STORE ? 2 : 0);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{q[0], q[1], q[2], q[3]}, rs,
                                               off + 32 * kChunk * 4, 0, RLK_NT_STORE ? 2 : 0);
    }
}

// Store a group of results.  Full aligned groups use 16-byte stores; in
// other groups, whole in-range chunks of an aligned row still do, and the
// remaining elements are stored one by one (nothing beyond V is written).
// With CUT, chunks before `cut` are not stored.
template <int BLOCK, int U, typename S, bool ALIGNED, bool CUT = false>
__device__ __forceinline__ void store_group(S* __restrict__ row, int64_t V, int64_t g0, bool full,
                                            const float (&v)[U][kChunk], int64_t cut = 0) {
    const int64_t nfull = V / kChunk;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t c = g0 + u * BLOCK + (int)threadIdx.x;
        if (CUT && c < cut) continue;
        if (ALIGNED && (full || c < nfull)) {
            store_chunk(row + c * kChunk, v[u]);
        } else {
#pragma unroll
            for (int e = 0; e < kChunk; ++e)
                if (c * kChunk + e < V) store_one(row + c * kChunk + e, v[u][e]);
        }
    }
}

// ------------------------------------------------------- online statistics

// Running statistics of one tensor row (per lane, then merged).
//   m: max of a (-inf while nothing finite has been seen), mL = m sc
//   (0 while m = -inf, so t stays -inf instead of NaN), S, W as above.
struct Stat1 {
    float m, mL, S, W;
};

// FIXED (kCapFixed): the reference is the bound 0 of every t from the start
// (m = mL = 0) and never moves.
template <bool FIXED = false>
__device__ __forceinline__ Stat1 stat1_init() {
    return {FIXED ? 0.0f : neg_inf(), 0.0f, 0.0f, 0.0f};
}

// Merge two partial states (exact up to rounding; empty parts drop out).
template <bool WITH_W>
__device__ __forceinline__ Stat1 stat1_merge(const Stat1& A, const Stat1& B) {
    if (A.m == neg_inf()) return B;
    if (B.m == neg_inf()) return A;
    const bool a_big = A.m >= B.m;
    Stat1 o;
    o.m = a_big ? A.m : B.m;
    o.mL = a_big ? A.mL : B.mL;
    const float dA = A.mL - o.mL, dB = B.mL - o.mL;  // <= 0, finite
    const float sA = ex2(dA), sB = ex2(dB);
    o.S = A.S * sA + B.S * sB;
    o.W = WITH_W ? sA * __builtin_fmaf(dA, A.S, A.W) + sB * __builtin_fmaf(dB, B.S, B.W) : 0.0f;
    return o;
}

// Statistics of a KL row pair: a side (policy) and b side (reference).
//   W = sum 2^ta (ta - tb)  (reverse: weights from the policy) or
//   W = sum 2^tb (tb - ta)  (forward: weights from the reference);
//   flag = max (reverse) / min (forward) of ta - tb: +inf / -inf exactly
//   when one side is finite where the other is -inf (support mismatch).
struct StatKL {
    float ma, mLa, Sa, mb, mLb, Sb, W, flag;
};

template <bool REVERSE, bool FIXA = false, bool FIXB = false>
__device__ __forceinline__ StatKL statkl_init() {
    return {FIXA ? 0.0f : neg_inf(), 0.0f, 0.0f, FIXB ? 0.0f : neg_inf(), 0.0f, 0.0f, 0.0f,
            REVERSE ? neg_inf() : pos_inf()};
}

template <bool REVERSE>
__device__ __forceinline__ StatKL statkl_merge(const StatKL& A, const StatKL& B) {
    StatKL o;
    o.flag = REVERSE ? fmaxf(A.flag, B.flag) : fminf(A.flag, B.flag);
    // a side
    const bool a_empty_A = A.ma == neg_inf(), a_empty_B = B.ma == neg_inf();
    const bool a_big = A.ma >= B.ma;
    o.ma = a_big ? A.ma : B.ma;
    o.mLa = a_empty_A ? B.mLa : (a_empty_B ? A.mLa : (a_big ? A.mLa : B.mLa));
    const float dA = a_empty_A ? 0.0f : A.mLa - o.mLa;
    const float dB = a_empty_B ? 0.0f : B.mLa - o.mLa;
    const float saA = a_empty_A ? 0.0f : ex2(dA), saB = a_empty_B ? 0.0f : ex2(dB);
    // b side
    const bool b_empty_A = A.mb == neg_inf(), b_empty_B = B.mb == neg_inf();
    const bool b_big = A.mb >= B.mb;
    o.mb = b_big ? A.mb : B.mb;
    o.mLb = b_empty_A ? B.mLb : (b_empty_B ? A.mLb : (b_big ? A.mLb : B.mLb));
    const float eA = b_empty_A ? 0.0f : A.mLb - o.mLb;
    const float eB = b_empty_B ? 0.0f : B.mLb - o.mLb;
    const float sbA = b_empty_A ? 0.0f : ex2(eA), sbB = b_empty_B ? 0.0f : ex2(eB);
    o.Sa = A.Sa * saA + B.Sa * saB;
    o.Sb = A.Sb * sbA + B.Sb * sbB;
    // A part with no finite weight carries W = 0 (or a mismatch, which
    // overrides the value anyway): drop it instead of scaling 0 by garbage.
    float wA, wB;
    if (REVERSE) {
        wA = (a_empty_A || b_empty_A) ? 0.0f : saA * __builtin_fmaf(dA - eA, A.Sa, A.W);
        wB = (a_empty_B || b_empty_B) ? 0.0f : saB * __builtin_fmaf(dB - eB, B.Sa, B.W);
    } else {
        wA = (a_empty_A || b_empty_A) ? 0.0f : sbA * __builtin_fmaf(eA - dA, A.Sb, A.W);
        wB = (a_empty_B || b_empty_B) ? 0.0f : sbB * __builtin_fmaf(eB - dB, B.Sb, B.W);
    }
    o.W = wA + wB;
    return o;
}

// Both KL directions of one row pair at once: the shared sums and maxima,
// W of each direction and both mismatch flags.  The two directions' views are
// exactly the single-direction states (same operations in the same order).
struct StatKL2 {
    float ma, mLa, Sa, mb, mLb, Sb, Wr, Wf, fmax, fmin;
};

template <bool FIXA = false, bool FIXB = false>
__device__ __forceinline__ StatKL2 statkl2_init() {
    return {FIXA ? 0.0f : neg_inf(), 0.0f, 0.0f, FIXB ? 0.0f : neg_inf(), 0.0f, 0.0f, 0.0f, 0.0f,
            neg_inf(), pos_inf()};
}
__device__ __forceinline__ StatKL kl_view_rev(const StatKL2& s) {
    return {s.ma, s.mLa, s.Sa, s.mb, s.mLb, s.Sb, s.Wr, s.fmax};
}
__device__ __forceinline__ StatKL kl_view_fwd(const StatKL2& s) {
    return {s.ma, s.mLa, s.Sa, s.mb, s.mLb, s.Sb, s.Wf, s.fmin};
}
__device__ __forceinline__ StatKL2 statkl2_merge(const StatKL2& A, const StatKL2& B) {
    const StatKL r = statkl_merge<true>(kl_view_rev(A), kl_view_rev(B));
    const StatKL f = statkl_merge<false>(kl_view_fwd(A), kl_view_fwd(B));
    return {r.ma, r.mLa, r.Sa, r.mb, r.mLb, r.Sb, r.W, f.W, r.flag, f.flag};
}

// ---------------------------------------------------- wave64 shuffles

__device__ __forceinline__ float shfl_xor(float v, int mask) {
    return __shfl_xor(v, mask, 64);
}

// Wave64 butterflies on lane moves that stay in registers: DPP quad
// permutations (lane ^ 1, lane ^ 2), the half-row and row mirrors (lane i
// with 7 - i and 15 - i: after the steps before, the same pairs of partial
// results as lane ^ 4 and lane ^ 8) and the 16- and 32-lane swaps.  Each step
// combines two values with a commutative operation, so every lane ends with
// the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <typename OP>
__device__ __forceinline__ float wave_fold(float v, OP op) {
    v = op(v, dpp_move<0xB1>(v));   // quad_perm [1, 0, 3, 2]
    v = op(v, dpp_move<0x4E>(v));   // quad_perm [2, 3, 0, 1]
    v = op(v, dpp_move<0x141>(v));  // row_half_mirror
    v = op(v, dpp_move<0x140>(v));  // row_mirror
    const auto h = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = op(__uint_as_float(h[0]), __uint_as_float(h[1]));
    const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return op(__uint_as_float(w[0]), __uint_as_float(w[1]));
}

// A wave's state: the maximum first (with its reference: mL = m * scale
// grows with m), then each lane's sums rescaled to it once, then plain
// sums.  Two butterflies of max and add replace a chain of rescaling merges
// (each step waiting for a shuffle, an exponential and its products); the
// tree is fixed, so the result is the same for every batch.
// The first N lanes of each group of N (N = 1, 2, 4, 8 or 16) folded with
// the first steps of wave_fold.
template <int N, typename OP>
__device__ __forceinline__ float lanes_fold(float v, OP op) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "a power of two up to a row");
    if (N >= 2) v = op(v, dpp_move<0xB1>(v));
    if (N >= 4) v = op(v, dpp_move<0x4E>(v));
    if (N >= 8) v = op(v, dpp_move<0x141>(v));
    if (N >= 16) v = op(v, dpp_move<0x140>(v));
    return v;
}
template <bool WITH_W, typename FOLD>
__device__ __forceinline__ Stat1 stat1_fold(Stat1 s, FOLD fold) {
    const auto mx = [](float a, float b) { return fmaxf(a, b); };
    const auto add = [](float a, float b) { return a + b; };
    const bool empty = s.m == neg_inf();
    const float M = fold(s.m, mx);
    const float ML = fold(empty ? neg_inf() : s.mL, mx);
    if (M == neg_inf()) return s;  // every lane folded is empty (and holds the same)
    const float d = s.mL - ML;     // <= 0
    const float sc = empty ? 0.0f : ex2(d);
    const float S = fold(s.S * sc, add);
    const float W = WITH_W ? fold(empty ? 0.0f : sc * __builtin_fmaf(d, s.S, s.W), add) : 0.0f;
    return {M, ML, S, W};
}
template <bool WITH_W>
__device__ __forceinline__ Stat1 wave_reduce(Stat1 s) {
    return stat1_fold<WITH_W>(s, [](float v, auto op) { return wave_fold(v, op); });
}
// The NW waves' states of a workgroup (red[0..NW)), combined the same way
// by the first NW lanes of the wave that calls it (lane 0 holds the result).
template <int NW, bool WITH_W>
__device__ __forceinline__ Stat1 waves_reduce(const Stat1* red, int lane) {
    return stat1_fold<WITH_W>(red[lane & (NW - 1)],
                              [](float v, auto op) { return lanes_fold<NW>(v, op); });
}

// A wave's KL state, as wave_reduce: both sides' maxima and the flag first,
// then each lane's sums rescaled once (a lane with an empty side carries no
// W, as in statkl_merge), then plain sums.
struct KLScale {
    bool ea, eb;
    float da, db, sa, sb;
};
template <typename FOLD>
__device__ __forceinline__ KLScale kl_scale(float ma, float mLa, float mb, float mLb, float& MLa,
                                            float& MLb, FOLD fold) {
    const auto mx = [](float a, float b) { return fmaxf(a, b); };
    KLScale k;
    k.ea = ma == neg_inf();
    k.eb = mb == neg_inf();
    MLa = fold(k.ea ? neg_inf() : mLa, mx);
    MLb = fold(k.eb ? neg_inf() : mLb, mx);
    k.da = k.ea ? 0.0f : mLa - MLa;
    k.db = k.eb ? 0.0f : mLb - MLb;
    k.sa = k.ea ? 0.0f : ex2(k.da);
    k.sb = k.eb ? 0.0f : ex2(k.db);
    return k;
}
template <bool REVERSE>
__device__ __forceinline__ float kl_w(const KLScale& k, float Sa, float Sb, float W) {
    if (k.ea || k.eb) return 0.0f;
    return REVERSE ? k.sa * __builtin_fmaf(k.da - k.db, Sa, W)
                   : k.sb * __builtin_fmaf(k.db - k.da, Sb, W);
}
template <bool REVERSE, typename FOLD>
__device__ __forceinline__ StatKL statkl_fold(StatKL s, FOLD fold) {
    const auto mx = [](float a, float b) { return fmaxf(a, b); };
    const auto mn = [](float a, float b) { return fminf(a, b); };
    const auto add = [](float a, float b) { return a + b; };
    float MLa, MLb;
    const KLScale k = kl_scale(s.ma, s.mLa, s.mb, s.mLb, MLa, MLb, fold);
    StatKL o;
    o.ma = fold(s.ma, mx);
    o.mb = fold(s.mb, mx);
    o.mLa = o.ma == neg_inf() ? s.mLa : MLa;  // (every lane empty: its own, the same)
    o.mLb = o.mb == neg_inf() ? s.mLb : MLb;
    o.flag = REVERSE ? fold(s.flag, mx) : fold(s.flag, mn);
    o.Sa = fold(s.Sa * k.sa, add);
    o.Sb = fold(s.Sb * k.sb, add);
    o.W = fold(kl_w<REVERSE>(k, s.Sa, s.Sb, s.W), add);
    return o;
}
template <bool REVERSE>
__device__ __forceinline__ StatKL wave_reduce_kl(StatKL s) {
    return statkl_fold<REVERSE>(s, [](float v, auto op) { return wave_fold(v, op); });
}
template <int NW, bool REVERSE>
__device__ __forceinline__ StatKL waves_reduce_kl(const StatKL* red, int lane) {
    return statkl_fold<REVERSE>(red[lane & (NW - 1)],
                                [](float v, auto op) { return lanes_fold<NW>(v, op); });
}

// Both directions: the very operations of statkl_fold for each.
template <typename FOLD>
__device__ __forceinline__ StatKL2 statkl2_fold(StatKL2 s, FOLD fold) {
    const auto mx = [](float a, float b) { return fmaxf(a, b); };
    const auto mn = [](float a, float b) { return fminf(a, b); };
    const auto add = [](float a, float b) { return a + b; };
    float MLa, MLb;
    const KLScale k = kl_scale(s.ma, s.mLa, s.mb, s.mLb, MLa, MLb, fold);
    StatKL2 o;
    o.ma = fold(s.ma, mx);
    o.mb = fold(s.mb, mx);
    o.mLa = o.ma == neg_inf() ? s.mLa : MLa;
    o.mLb = o.mb == neg_inf() ? s.mLb : MLb;
    o.fmax = fold(s.fmax, mx);
    o.fmin = fold(s.fmin, mn);
    o.Sa = fold(s.Sa * k.sa, add);
    o.Sb = fold(s.Sb * k.sb, add);
    o.Wr = fold(kl_w<true>(k, s.Sa, s.Sb, s.Wr), add);
    o.Wf = fold(kl_w<false>(k, s.Sa, s.Sb, s.Wf), add);
    return o;
}
__device__ __forceinline__ StatKL2 wave_reduce_kl2(StatKL2 s) {
    return statkl2_fold(s, [](float v, auto op) { return wave_fold(v, op); });
}
template <int NW>
__device__ __forceinline__ StatKL2 waves_reduce_kl2(const StatKL2* red, int lane) {
    return statkl2_fold(red[lane & (NW - 1)],
                        [](float v, auto op) { return lanes_fold<NW>(v, op); });
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += shfl_xor(v, off);
    return v;
}

// ----------------------------------------------------------- row record

// Per-row record written by a forward call and read by its backward call.
// 32 bytes per row, 16-byte aligned.
struct alignas(16) RowStats {
    float mLa, log2Sa;  // first (or only) tensor: scaled max, log2 of the sum
    float mLb, log2Sb;  // KL reference tensor
    float value;        // entropy H, or KL D (natural log units)
    uint32_t flags;     // kFlag* bits
    float pad0, pad1;
};
constexpr uint32_t kFlagEmptyA = 1u, kFlagEmptyB = 2u, kFlagMismatch = 4u;

// Row state of one vocabulary shard (32 bytes per row), exported before the
// heads are finalized so that P shards can be folded in rank order with the
// same merges as the in-kernel tree (the cross-shard step of "Add Triton
// kernels for vocab-parallel logprobs, entropy and KL", Changes: local
// statistics rescaled to the global maximum).
struct alignas(16) PartialRec {
    float ma, mLa, Sa, W, mb, mLb, Sb, flag;
};

__device__ __forceinline__ PartialRec to_partial(const Stat1& s) {
    return {s.m, s.mL, s.S, s.W, 0.0f, 0.0f, 0.0f, 0.0f};
}
__device__ __forceinline__ PartialRec to_partial(const StatKL& s) {
    return {s.ma, s.mLa, s.Sa, s.W, s.mb, s.mLb, s.Sb, s.flag};
}
__device__ __forceinline__ Stat1 stat1_of(const PartialRec& r) { return {r.ma, r.mLa, r.Sa, r.W}; }
__device__ __forceinline__ StatKL statkl_of(const PartialRec& r) {
    return {r.ma, r.mLa, r.Sa, r.mb, r.mLb, r.Sb, r.W, r.flag};
}

// Heads and row record from a row's final single-tensor state:
// logsumexp = ln2 (mL + log2 S), entropy H = ln2 (log2 S - W / S); an empty
// row (every logit -inf) has log2 S = -inf and H = NaN.
template <bool WITH_W>
__device__ __forceinline__ RowStats finalize1(const Stat1& r) {
    const bool empty = r.m == neg_inf();
    const float log2S = log2f(r.S);  // -inf for an empty row
    RowStats rs;
    rs.mLa = r.mL;
    rs.log2Sa = log2S;
    rs.mLb = 0.0f;
    rs.log2Sb = 0.0f;
    rs.flags = empty ? kFlagEmptyA : 0u;
    rs.value = WITH_W ? (empty ? qnan() : kLn2 * (log2S - r.W / r.S)) : 0.0f;
    rs.pad0 = rs.pad1 = 0.0f;
    return rs;
}

// KL(A||B) = ln2 (W / S_A - log2 S_A + log2 S_B) (reverse: A = policy), NaN
// if either row is empty, +inf on a support mismatch.
template <bool REVERSE>
__device__ __forceinline__ RowStats finalize_kl(const StatKL& r) {
    const bool empty_a = r.ma == neg_inf(), empty_b = r.mb == neg_inf();
    const bool mismatch = REVERSE ? r.flag == pos_inf() : r.flag == neg_inf();
    const float log2Sa = log2f(r.Sa), log2Sb = log2f(r.Sb);
    const float D = REVERSE ? kLn2 * (r.W / r.Sa - log2Sa + log2Sb)
                            : kLn2 * (r.W / r.Sb - log2Sb + log2Sa);
    RowStats rs;
    rs.mLa = r.mLa;
    rs.log2Sa = log2Sa;
    rs.mLb = r.mLb;
    rs.log2Sb = log2Sb;
    rs.value = (empty_a || empty_b) ? qnan() : (mismatch ? pos_inf() : D);
    rs.flags = (empty_a ? kFlagEmptyA : 0u) | (empty_b ? kFlagEmptyB : 0u) |
               (mismatch ? kFlagMismatch : 0u);
    rs.pad0 = rs.pad1 = 0.0f;
    return rs;
}

// log p of a target from its statistic input a and the row record.
__device__ __forceinline__ float target_logp(float a, float sc, const RowStats& rs) {
    return (__builtin_fmaf(a, sc, -rs.mLa) - rs.log2Sa) * kLn2;
}

}  // namespace rlk
