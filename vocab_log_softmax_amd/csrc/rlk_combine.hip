// rlk_combine.hip -- deterministic P-way combine of vocabulary-shard records.
//
// "Add Triton kernels for vocab-parallel logprobs, entropy and KL" (DeepSpeed
// pull request 8838), Changes and the review comment: with the vocabulary
// split across ranks, each rank computes its local max, sum of exponentials
// and weighted sum in one read; they are then rescaled to the global max and
// added, and the support-mismatch flag travels with the max.  Here the shard
// records (PartialRec) are folded in rank order with the same merges the row
// kernels use inside a workgroup, so the result is deterministic and the same
// on every rank that folds the same gathered records.  The heads and the row
// record for the backward are then finalized exactly as in a plain forward.
#include "rlk_device.h"
#include "rlk_launch.h"

namespace rlk {

constexpr int kCombineBlock = 128;

template <int HEAD>
__global__ __launch_bounds__(kCombineBlock) void combine_kernel(CombineParams q) {
    constexpr bool KL = HEAD == kHeadKLReverse || HEAD == kHeadKLForward;
    constexpr bool WITH_W = HEAD == kHeadEntropy;
    const PartialRec* part = static_cast<const PartialRec*>(q.part);
    RowStats* stats = static_cast<RowStats*>(q.stats);
    const int64_t stride = (int64_t)gridDim.x * kCombineBlock;
    for (int64_t row = (int64_t)blockIdx.x * kCombineBlock + threadIdx.x; row < q.N;
         row += stride) {
        RowStats rs;
        if (KL) {
            StatKL acc = statkl_of(part[row]);
            for (int s = 1; s < q.P; ++s)
                acc = statkl_merge<HEAD == kHeadKLReverse>(acc, statkl_of(part[s * q.N + row]));
            rs = finalize_kl<HEAD == kHeadKLReverse>(acc);
            q.out[row] = rs.value;
        } else {
            Stat1 acc = stat1_of(part[row]);
            for (int s = 1; s < q.P; ++s)
                acc = stat1_merge<WITH_W>(acc, stat1_of(part[s * q.N + row]));
            rs = finalize1<WITH_W>(acc);
            if (HEAD == kHeadEntropy) q.out[row] = rs.value;
        }
        stats[row] = rs;
        if (HEAD == kHeadLogp) {
            for (int64_t j = 0; j < q.k; ++j) {
                const int64_t t = q.targets[row * q.k + j];
                float o = 0.0f;
                if (t >= 0 && t < q.vtotal) {
                    int s = 0;
                    while (s + 1 < q.P && t >= q.bounds[s + 1]) ++s;  // owning shard
                    o = target_logp(q.tvals[(s * q.N + row) * q.k + j], q.sc, rs);
                }
                q.out[row * q.k + j] = o;
            }
        }
    }
}

hipError_t launch_combine(int head, const CombineParams& q, hipStream_t stream) {
    const int64_t blocks = (q.N + kCombineBlock - 1) / kCombineBlock;
    const dim3 grid(static_cast<unsigned>(blocks < kMaxGrid ? blocks : kMaxGrid));
    const dim3 block(kCombineBlock);
    switch (head) {
        case kHeadLogp:
            hipLaunchKernelGGL(combine_kernel<kHeadLogp>, grid, block, 0, stream, q);
            break;
        case kHeadEntropy:
            hipLaunchKernelGGL(combine_kernel<kHeadEntropy>, grid, block, 0, stream, q);
            break;
        case kHeadKLReverse:
            hipLaunchKernelGGL(combine_kernel<kHeadKLReverse>, grid, block, 0, stream, q);
            break;
        case kHeadKLForward:
            hipLaunchKernelGGL(combine_kernel<kHeadKLForward>, grid, block, 0, stream, q);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rlk
