// issue_rate.hip -- VALU issue-rate probe: how often a SIMD issues a wave64
// FMA, v_exp_f32 or v_rcp_f32 when every lane runs 8 independent chains of
// the same operation (no dependency stalls at 8 waves per SIMD).  The ratio
// prices the transcendentals of the cap and the softmax against ordinary
// instructions in the kernels' VALU budgets.  Measurement infrastructure
// only (linked into libceiling.so, loaded by the benchmark).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kChains = 8;

template <int OP>
__global__ __launch_bounds__(256) void issue_kernel(float* __restrict__ out, int iters, float a) {
    float v[kChains];
#pragma unroll
    for (int i = 0; i < kChains; ++i) v[i] = a + 0.001f * static_cast<float>(threadIdx.x + i);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kChains; ++i) {
            if (OP == 0) v[i] = __builtin_fmaf(v[i], 0.999f, 0.0001f);
            if (OP == 1) v[i] = __builtin_amdgcn_exp2f(v[i]);
            if (OP == 2) v[i] = __builtin_amdgcn_rcpf(v[i]);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kChains; ++i) s += v[i];
    out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = s;  // one float per thread
}

}  // namespace

extern "C" {

// Operations per lane of one launch of issue_rate_run (kChains chains x iters).
int issue_rate_chains(void) { return kChains; }

// Launch the probe for op 0 (fma), 1 (exp2) or 2 (rcp): `blocks` workgroups
// of 256 threads, each thread writing one float of `out` (blocks * 256
// floats).  Returns 0, -1 for an unknown op or bad sizes, or the launch error.
int issue_rate_run(int op, int blocks, int iters, float* out, void* stream) {
    if (blocks <= 0 || iters <= 0) return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (op) {
        case 0: hipLaunchKernelGGL(issue_kernel<0>, dim3(blocks), dim3(256), 0, s, out, iters, 0.5f); break;
        case 1: hipLaunchKernelGGL(issue_kernel<1>, dim3(blocks), dim3(256), 0, s, out, iters, -0.5f); break;
        case 2: hipLaunchKernelGGL(issue_kernel<2>, dim3(blocks), dim3(256), 0, s, out, iters, 1.5f); break;
        default: return -1;
    }
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
