// rlk_fwd_f16.hip -- forward row kernels instantiated for f16 logits
// (one translation unit per dtype so the library builds in parallel).
#include "rlk_fwd_kernels.h"

namespace rlk {

hipError_t launch_fwd_f16(int head, int cap_x, int cap_y, bool aligned,
                           const FwdParams& p, hipStream_t stream) {
    return fwd_dispatch_cap<F16>(head, cap_x, cap_y, aligned, p, stream);
}

}  // namespace rlk
