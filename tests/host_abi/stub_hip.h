// stub_hip.h -- the fake HIP runtime's registry and launch log (host-only
// sanitizer build of the C ABI; see stub_hip.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_launch.h"

namespace stub {

constexpr int kDevices = 2;
enum Kind { kNone = 0, kFwd, kBwd, kSoftcapFwd, kSoftcapBwd, kCombine };

struct Log {
    int launches = 0;
    int hip_calls = 0;
    int set_device_calls = 0;
    int range_errors = 0;
    int kind = kNone;
    int dtype = -1, dtype_y = -1, head = -1, cap_x = -1, cap_y = -1, device = -1;
    bool aligned = false;
    int64_t n = 0;
    float cap = 0.0f;
    rlk::FwdParams fwd{};
    rlk::BwdParams bwd{};
    rlk::CombineParams comb{};
};
extern Log g_log;

// A fake allocation of `size` bytes on device `dev` (or pinned host memory).
// The address is 4096-byte aligned and never dereferenced.
void* fake_alloc(size_t size, int dev = 0, bool host = false);
void reset_log();
int current_device();
void set_current_device(int d);

}  // namespace stub
