// rlk_softcap.hip -- standalone elementwise final-logit softcap.
//
// "Final Logit Softcap" (RL-Kernel operator documentation), Summary and Tensor
// and Precision Contract: y = c tanh(x / c) with the cap a runtime argument,
// fp32 internal math and one trailing cast; the backward recomputes tanh from
// the saved input and returns g_y (1 - tanh^2(x / c)) in the input dtype.
// 64-bit element offsets throughout (the contract removes the 2^31 limit).
// x / c is evaluated as x * (1 / c) with 1 / c rounded once on the host.
#include "rlk_device.h"
#include "rlk_launch.h"

namespace rlk {

constexpr int kCapBlock = 256;

// Four consecutive values (a quad) at an aligned address: 16 bytes of
// fp32, 8 bytes of a 16-bit type.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <bool NT>
__device__ __forceinline__ void load_quad(const float* p, float (&f)[4]) {
    const f32x4 a = ld16<NT>(reinterpret_cast<const f32x4*>(p));
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
}
template <bool NT>
__device__ __forceinline__ void load_quad(const uint16_t* p, float (&f)[4]) {
    const u32x2 w = ld16<NT>(reinterpret_cast<const u32x2*>(p));
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
    f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
}
template <bool NT>
__device__ __forceinline__ void load_quad(const _Float16* p, float (&f)[4]) {
    const u32x2 w = ld16<NT>(reinterpret_cast<const u32x2*>(p));
    const uint32_t ws[2] = {w.x, w.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const f16x2_t h = __builtin_bit_cast(f16x2_t, ws[i]);
        f[2 * i] = static_cast<float>(h.x);
        f[2 * i + 1] = static_cast<float>(h.y);
    }
}
__device__ __forceinline__ void store_quad(float* p, const float (&f)[4]) {
    st16(reinterpret_cast<f32x4*>(p), f32x4{f[0], f[1], f[2], f[3]});
}
__device__ __forceinline__ void store_quad(uint16_t* p, const float (&f)[4]) {
    st16(reinterpret_cast<u32x2*>(p), u32x2{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])});
}
__device__ __forceinline__ void store_quad(_Float16* p, const float (&f)[4]) {
    st16(reinterpret_cast<u32x2*>(p), u32x2{pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3])});
}

// Each workgroup iteration covers a span of kCapBlock chunks.  When an fp32
// tensor takes part (QUADS), a full span of an aligned call gives lane t its
// quads t and kCapBlock + t, so every load and store of a wave is contiguous
// (a lane's 8-value chunk puts a wave's fp32 accesses 32 bytes apart: fp32 ->
// fp32 at 2^29 values 5.4 TB/s, 6.3 TB/s in quads).  Otherwise, and in the
// last span, lane t takes chunk t of the span (16 bytes of a 16-bit type:
// bf16 -> bf16 measured 5% slower in 8-byte quads), element by element past n.
template <typename TX, typename TY, bool ALIGNED>
__global__ __launch_bounds__(kCapBlock) void softcap_fwd_kernel(const void* xv, void* yv,
                                                                 int64_t n, float c, float inv_c) {
    using SX = typename TX::storage;
    using SY = typename TY::storage;
    const SX* __restrict__ x = static_cast<const SX*>(xv);
    SY* __restrict__ y = static_cast<SY*>(yv);
    constexpr bool QUADS = sizeof(SX) == 4 || sizeof(SY) == 4;
    const int64_t nchunks = (n + kChunk - 1) / kChunk;
    const int64_t stride = (int64_t)gridDim.x * kCapBlock;
    for (int64_t cb = (int64_t)blockIdx.x * kCapBlock; cb < nchunks; cb += stride) {
        const int64_t s0 = cb * kChunk;
        if (QUADS && ALIGNED && s0 + kCapBlock * kChunk <= n) {
            const int64_t i0 = s0 + 4 * threadIdx.x, i1 = i0 + 4 * kCapBlock;
            float f[2][4];
            load_quad<true>(x + i0, f[0]);
            load_quad<true>(x + i1, f[1]);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float sl;
                    f[h][e] = c * tanh_precise(f[h][e] * inv_c, &sl);
                }
            store_quad(y + i0, f[0]);
            store_quad(y + i1, f[1]);
            continue;
        }
        const int64_t ch = cb + threadIdx.x;
        if (ch >= nchunks) continue;
        const int64_t i0 = ch * kChunk;
        float f[kChunk];
        if (ALIGNED && i0 + kChunk <= n) {
            load_chunk<true>(x + i0, f);
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                float sl;
                f[e] = c * tanh_precise(f[e] * inv_c, &sl);
            }
            store_chunk(y + i0, f);
        } else {
            for (int e = 0; e < kChunk && i0 + e < n; ++e) {
                float sl;
                store_one(y + i0 + e, c * tanh_precise(load_one(x + i0 + e) * inv_c, &sl));
            }
        }
    }
}

template <typename TX, bool ALIGNED>
__global__ __launch_bounds__(kCapBlock) void softcap_bwd_kernel(const void* xv, const float* gy,
                                                                 void* gxv, int64_t n,
                                                                 float inv_c) {
    using SX = typename TX::storage;
    const SX* __restrict__ x = static_cast<const SX*>(xv);
    SX* __restrict__ gx = static_cast<SX*>(gxv);
    constexpr bool QUADS = sizeof(SX) == 4;  // (the fp32 g_y alone does not pay)
    const int64_t nchunks = (n + kChunk - 1) / kChunk;
    const int64_t stride = (int64_t)gridDim.x * kCapBlock;
    for (int64_t cb = (int64_t)blockIdx.x * kCapBlock; cb < nchunks; cb += stride) {
        const int64_t s0 = cb * kChunk;
        if (QUADS && ALIGNED && s0 + kCapBlock * kChunk <= n) {
            const int64_t i0 = s0 + 4 * threadIdx.x, i1 = i0 + 4 * kCapBlock;
            float f[2][4], g[2][4];
            load_quad<true>(x + i0, f[0]);
            load_quad<true>(x + i1, f[1]);
            load_quad<true>(gy + i0, g[0]);
            load_quad<true>(gy + i1, g[1]);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float sl;
                    (void)tanh_precise(f[h][e] * inv_c, &sl);
                    f[h][e] = g[h][e] * sl;
                }
            store_quad(gx + i0, f[0]);
            store_quad(gx + i1, f[1]);
            continue;
        }
        const int64_t ch = cb + threadIdx.x;
        if (ch >= nchunks) continue;
        const int64_t i0 = ch * kChunk;
        float f[kChunk], g[kChunk];
        if (ALIGNED && i0 + kChunk <= n) {
            load_chunk<true>(x + i0, f);
            load_chunk<true>(gy + i0, g);
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                float sl;
                (void)tanh_precise(f[e] * inv_c, &sl);
                f[e] = g[e] * sl;
            }
            store_chunk(gx + i0, f);
        } else {
            for (int e = 0; e < kChunk && i0 + e < n; ++e) {
                float sl;
                (void)tanh_precise(load_one(x + i0 + e) * inv_c, &sl);
                store_one(gx + i0 + e, gy[i0 + e] * sl);
            }
        }
    }
}

static int cap_grid(int64_t n) {
    const int64_t chunks = (n + kChunk - 1) / kChunk;
    const int64_t blocks = (chunks + kCapBlock - 1) / kCapBlock;
    return static_cast<int>(blocks < kMaxGrid ? blocks : kMaxGrid);
}

template <typename TX, typename TY>
static hipError_t cap_fwd_al(const void* x, void* y, int64_t n, float c, bool al, hipStream_t s) {
    const float inv_c = 1.0f / c;
    if (al)
        hipLaunchKernelGGL((softcap_fwd_kernel<TX, TY, true>), dim3(cap_grid(n)), dim3(kCapBlock),
                           0, s, x, y, n, c, inv_c);
    else
        hipLaunchKernelGGL((softcap_fwd_kernel<TX, TY, false>), dim3(cap_grid(n)),
                           dim3(kCapBlock), 0, s, x, y, n, c, inv_c);
    return hipGetLastError();
}

template <typename TX>
static hipError_t cap_fwd_y(const void* x, void* y, int y_dtype, int64_t n, float c, bool al,
                            hipStream_t s) {
    if (y_dtype == 0) return cap_fwd_al<TX, F32>(x, y, n, c, al, s);
    if (y_dtype == 1) return cap_fwd_al<TX, BF16>(x, y, n, c, al, s);
    return cap_fwd_al<TX, F16>(x, y, n, c, al, s);
}

hipError_t launch_softcap_fwd(const void* x, int x_dtype, void* y, int y_dtype, int64_t n,
                              float cap, bool aligned, hipStream_t stream) {
    if (x_dtype == 0) return cap_fwd_y<F32>(x, y, y_dtype, n, cap, aligned, stream);
    if (x_dtype == 1) return cap_fwd_y<BF16>(x, y, y_dtype, n, cap, aligned, stream);
    return cap_fwd_y<F16>(x, y, y_dtype, n, cap, aligned, stream);
}

template <typename TX>
static hipError_t cap_bwd_al(const void* x, const float* gy, void* gx, int64_t n, float inv_c,
                             bool al, hipStream_t s) {
    const dim3 grid(cap_grid(n)), block(kCapBlock);
    if (al)
        hipLaunchKernelGGL((softcap_bwd_kernel<TX, true>), grid, block, 0, s, x, gy, gx, n, inv_c);
    else
        hipLaunchKernelGGL((softcap_bwd_kernel<TX, false>), grid, block, 0, s, x, gy, gx, n, inv_c);
    return hipGetLastError();
}

hipError_t launch_softcap_bwd(const void* x, int x_dtype, const float* gy, void* gx, int64_t n,
                              float cap, bool aligned, hipStream_t stream) {
    const float inv_c = 1.0f / cap;
    if (x_dtype == 0) return cap_bwd_al<F32>(x, gy, gx, n, inv_c, aligned, stream);
    if (x_dtype == 1) return cap_bwd_al<BF16>(x, gy, gx, n, inv_c, aligned, stream);
    return cap_bwd_al<F16>(x, gy, gx, n, inv_c, aligned, stream);
}

}  // namespace rlk
