// rlk_launch.h -- kernel parameter blocks and the internal launchers that the
// C ABI (rlk_api.cpp) calls after it has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlk {

// Heads of the fused row kernels.
enum Head : int { kHeadLogp = 0, kHeadEntropy = 1, kHeadKLReverse = 2, kHeadKLForward = 3 };

// Launch shape of the row kernels: one workgroup of kBlock threads per row
// (grid-stride over rows), each lane consuming kUnroll chunks of 8 elements
// per group.  These constants fix the reduction tree, so they are the same
// for every N.
constexpr int kBlock = 256;
constexpr int kUnroll1 = 4;   // single-tensor heads (logp, entropy)
constexpr int kUnrollKL = 2;  // KL reads two tensors per group
constexpr int kMaxGrid = 1 << 20;

struct FwdParams {
    const void* x;   // logits (KL: policy)
    const void* y;   // KL reference (else unused)
    int64_t N, V, ldx, ldy;
    const int64_t* targets;  // logp: [N, k]
    int64_t k;
    float kx, ky;    // softcap multiplier -2 log2(e) / c (unused when off)
    float scx, scy;  // log2(e), or c log2(e) when the softcap is on
    float* out;      // logp [N, k], entropy [N] or KL [N]
    void* stats;     // RowStats [N]
};

struct BwdParams {
    const void* x;
    const void* y;
    int64_t N, V, ldx, ldy;
    const int64_t* targets;
    int64_t k;
    float kx, ky, scx, scy;
    const void* stats;
    const float* g;  // upstream gradient: [N, k] (logp) or [N]
    void* gx;        // gradient w.r.t. x, [N, V] contiguous, logits dtype
};

// dtype codes follow rlk_dtype (0 fp32, 1 bf16).
hipError_t launch_fwd(int head, int dtype, bool cap_x, bool cap_y, bool aligned,
                      const FwdParams& p, hipStream_t stream);
hipError_t launch_bwd(int head, int dtype, bool cap_x, bool cap_y, bool aligned,
                      const BwdParams& p, hipStream_t stream);
hipError_t launch_softcap_fwd(const void* x, int x_dtype, void* y, int y_dtype, int64_t n,
                              float cap, bool aligned, hipStream_t stream);
hipError_t launch_softcap_bwd(const void* x, int x_dtype, const float* gy, void* gx, int64_t n,
                              float cap, bool aligned, hipStream_t stream);

inline int row_grid(int64_t N) { return static_cast<int>(N < kMaxGrid ? N : kMaxGrid); }

}  // namespace rlk
