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

template <typename TX, typename TY, bool ALIGNED>
__global__ __launch_bounds__(kCapBlock) void softcap_fwd_kernel(const void* xv, void* yv,
                                                                 int64_t n, float c, float inv_c) {
    using SX = typename TX::storage;
    using SY = typename TY::storage;
    const SX* __restrict__ x = static_cast<const SX*>(xv);
    SY* __restrict__ y = static_cast<SY*>(yv);
    const int64_t nchunks = (n + kChunk - 1) / kChunk;
    const int64_t stride = (int64_t)gridDim.x * kCapBlock;
    for (int64_t ch = (int64_t)blockIdx.x * kCapBlock + threadIdx.x; ch < nchunks; ch += stride) {
        const int64_t i0 = ch * kChunk;
        float f[kChunk];
        if (ALIGNED && i0 + kChunk <= n) {
            load_chunk<true>(x + i0, f);
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                float s;
                f[e] = c * tanh_precise(f[e] * inv_c, &s);
            }
            store_chunk(y + i0, f);
        } else {
            for (int e = 0; e < kChunk && i0 + e < n; ++e) {
                float s;
                store_one(y + i0 + e, c * tanh_precise(load_one(x + i0 + e) * inv_c, &s));
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
    const int64_t nchunks = (n + kChunk - 1) / kChunk;
    const int64_t stride = (int64_t)gridDim.x * kCapBlock;
    for (int64_t ch = (int64_t)blockIdx.x * kCapBlock + threadIdx.x; ch < nchunks; ch += stride) {
        const int64_t i0 = ch * kChunk;
        float f[kChunk], g[kChunk];
        if (ALIGNED && i0 + kChunk <= n) {
            load_chunk<true>(x + i0, f);
            load_chunk<true>(gy + i0, g);
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                float s;
                (void)tanh_precise(f[e] * inv_c, &s);
                f[e] = g[e] * s;
            }
            store_chunk(gx + i0, f);
        } else {
            for (int e = 0; e < kChunk && i0 + e < n; ++e) {
                float s;
                (void)tanh_precise(load_one(x + i0 + e) * inv_c, &s);
                store_one(gx + i0 + e, gy[i0 + e] * s);
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
