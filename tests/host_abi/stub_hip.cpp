// stub_hip.cpp -- a fake HIP runtime and recording launchers for the host-only
// build of rlk_api.cpp (tests/test_host_sanitize.py).
//
// The C ABI's host code (validation, device binding, kernel parameters) is
// compiled with g++ under AddressSanitizer and UBSan and linked against this
// file instead of the HIP runtime and the kernels.  "Device memory" is a set
// of registered address ranges that are never dereferenced; each launcher
// records its arguments and checks that every byte the kernel would touch
// (from the sizes, row maps and pointers it was given) lies inside one
// registered allocation of the device that is current at the launch.
#include "stub_hip.h"

#include <cstdio>
#include <cstdlib>
#include <vector>

namespace stub {

namespace {
struct Alloc {
    uintptr_t base;
    size_t size;
    int dev;
    bool host;
};
std::vector<Alloc> g_allocs;
uintptr_t g_next = uintptr_t(0x100000000000ull);
int g_cur = 0;
}  // namespace

Log g_log;

void* fake_alloc(size_t size, int dev, bool host) {
    const uintptr_t base = g_next;
    g_next += (size + 4095u) / 4096u * 4096u + 4096u;  // a gap between allocations
    g_allocs.push_back({base, size, dev, host});
    return reinterpret_cast<void*>(base);
}

void reset_log() { g_log = Log{}; }
int current_device() { return g_cur; }
void set_current_device(int d) { g_cur = d; }

static const Alloc* find(uintptr_t p) {
    for (const Alloc& a : g_allocs)
        if (p >= a.base && p < a.base + (a.size ? a.size : 1)) return &a;
    return nullptr;
}

// Every byte of [p, p + n) inside one device allocation of the current device.
static void need(const void* p, uint64_t n, const char* what) {
    if (n == 0) return;
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    const Alloc* a = find(b);
    if (!a || a->host || a->dev != g_cur || b + n > a->base + a->size) {
        std::fprintf(stderr, "launch touches %s outside its allocation: [%#llx, +%llu) dev %d\n",
                     what, (unsigned long long)b, (unsigned long long)n, g_cur);
        ++g_log.range_errors;
    }
}

// Rows 0..N-1 of V elements at `base` through the row map.
static void need_rows(const void* base, const rlk::RowMap& m, int64_t N, int64_t V, int64_t es,
                      const char* what) {
    if (N <= 0 || V <= 0) return;
    for (int64_t i = 0; i < N; ++i) {
        const int64_t off = m.offset(i);
        need(static_cast<const char*>(base) + off * es, static_cast<uint64_t>(V * es), what);
        if (g_log.range_errors) return;
    }
}

static int64_t es_of(int dtype) { return dtype == 0 ? 4 : 2; }

static void fwd(int dtype, int head, int cx, int cy, bool al, const rlk::FwdParams& p) {
    ++g_log.launches;
    g_log.kind = kFwd;
    g_log.dtype = dtype;
    g_log.head = head;
    g_log.cap_x = cx;
    g_log.cap_y = cy;
    g_log.aligned = al;
    g_log.fwd = p;
    g_log.device = g_cur;
    const int64_t es = es_of(dtype);
    const bool kl = head >= rlk::kHeadKLReverse;
    need_rows(p.x, p.mx, p.N, p.V, es, "x");
    if (kl) need_rows(p.y, p.my, p.N, p.V, es, "y");
    const int64_t k = head == rlk::kHeadLogp ? p.k : 1;
    if (head == rlk::kHeadLogp) need(p.targets, 8ull * p.N * k, "targets");
    if (p.part) {
        need(p.part, 32ull * p.N, "partial records");
        if (head == rlk::kHeadLogp) need(p.tvals, 4ull * p.N * k, "target values");
    } else {
        need(p.out, 4ull * p.N * k, "out");
        need(p.stats, 32ull * p.N, "stats");
        if (head == rlk::kHeadKLBoth) {
            need(p.out2, 4ull * p.N, "out2");
            need(p.stats2, 32ull * p.N, "stats2");
        }
    }
}

static void bwd(int dtype, int head, int cx, int cy, bool al, const rlk::BwdParams& p) {
    ++g_log.launches;
    g_log.kind = kBwd;
    g_log.dtype = dtype;
    g_log.head = head;
    g_log.cap_x = cx;
    g_log.cap_y = cy;
    g_log.aligned = al;
    g_log.bwd = p;
    g_log.device = g_cur;
    const int64_t es = es_of(dtype);
    const bool kl = head >= rlk::kHeadKLReverse;
    need_rows(p.x, p.mx, p.N, p.V, es, "x");
    if (kl) need_rows(p.y, p.my, p.N, p.V, es, "y");
    need_rows(p.gx, p.mg, p.N, p.V, es, "gradient");
    need(p.stats, 32ull * p.N, "stats");
    if (head == rlk::kHeadLogp) {
        need(p.targets, 8ull * p.N * p.k, "targets");
        need(p.g, 4ull * p.N * p.k, "upstream gradient");
    } else {
        need(p.g, 4ull * p.N, "upstream gradient");
    }
}

}  // namespace stub

using stub::g_log;

namespace rlk {

hipError_t launch_fwd_f32(int h, int cx, int cy, bool al, const FwdParams& p, hipStream_t) {
    stub::fwd(0, h, cx, cy, al, p);
    return hipSuccess;
}
hipError_t launch_fwd_bf16(int h, int cx, int cy, bool al, const FwdParams& p, hipStream_t) {
    stub::fwd(1, h, cx, cy, al, p);
    return hipSuccess;
}
hipError_t launch_fwd_f16(int h, int cx, int cy, bool al, const FwdParams& p, hipStream_t) {
    stub::fwd(2, h, cx, cy, al, p);
    return hipSuccess;
}
hipError_t launch_bwd_f32(int h, int cx, int cy, bool al, const BwdParams& p, hipStream_t) {
    stub::bwd(0, h, cx, cy, al, p);
    return hipSuccess;
}
hipError_t launch_bwd_bf16(int h, int cx, int cy, bool al, const BwdParams& p, hipStream_t) {
    stub::bwd(1, h, cx, cy, al, p);
    return hipSuccess;
}
hipError_t launch_bwd_f16(int h, int cx, int cy, bool al, const BwdParams& p, hipStream_t) {
    stub::bwd(2, h, cx, cy, al, p);
    return hipSuccess;
}

hipError_t launch_softcap_fwd(const void* x, int xd, void* y, int yd, int64_t n, float cap,
                              bool al, hipStream_t) {
    ++g_log.launches;
    g_log.kind = stub::kSoftcapFwd;
    g_log.dtype = xd;
    g_log.dtype_y = yd;
    g_log.n = n;
    g_log.cap = cap;
    g_log.aligned = al;
    g_log.device = stub::current_device();
    stub::need(x, static_cast<uint64_t>(n) * stub::es_of(xd), "softcap x");
    stub::need(y, static_cast<uint64_t>(n) * stub::es_of(yd), "softcap y");
    return hipSuccess;
}

hipError_t launch_softcap_bwd(const void* x, int xd, const float* gy, void* gx, int64_t n,
                              float cap, bool al, hipStream_t) {
    ++g_log.launches;
    g_log.kind = stub::kSoftcapBwd;
    g_log.dtype = xd;
    g_log.n = n;
    g_log.cap = cap;
    g_log.aligned = al;
    g_log.device = stub::current_device();
    stub::need(x, static_cast<uint64_t>(n) * stub::es_of(xd), "softcap x");
    stub::need(gy, static_cast<uint64_t>(n) * 4u, "softcap grad_y");
    stub::need(gx, static_cast<uint64_t>(n) * stub::es_of(xd), "softcap grad_x");
    return hipSuccess;
}

hipError_t launch_combine(int head, const CombineParams& q, hipStream_t) {
    ++g_log.launches;
    g_log.kind = stub::kCombine;
    g_log.head = head;
    g_log.comb = q;
    g_log.device = stub::current_device();
    const uint64_t P = static_cast<uint64_t>(q.P), N = static_cast<uint64_t>(q.N);
    stub::need(q.part, 32u * P * N, "partial records");
    stub::need(q.out, 4u * N * static_cast<uint64_t>(q.k), "out");
    stub::need(q.stats, 32u * N, "stats");
    if (head == kHeadLogp) {
        stub::need(q.targets, 8u * N * static_cast<uint64_t>(q.k), "targets");
        stub::need(q.tvals, 4u * P * N * static_cast<uint64_t>(q.k), "target values");
    }
    return hipSuccess;
}

}  // namespace rlk

// ------------------------------------------------------------ fake runtime

extern "C" {

hipError_t hipPointerGetAttributes(hipPointerAttribute_t* attr, const void* ptr) {
    ++g_log.hip_calls;
    const stub::Alloc* a = stub::find(reinterpret_cast<uintptr_t>(ptr));
    if (!a) return hipErrorInvalidValue;
    attr->type = a->host ? hipMemoryTypeHost : hipMemoryTypeDevice;
    attr->device = a->dev;
    attr->devicePointer = a->host ? nullptr : const_cast<void*>(ptr);
    attr->hostPointer = a->host ? const_cast<void*>(ptr) : nullptr;
    attr->isManaged = 0;
    attr->allocationFlags = 0;
    return hipSuccess;
}

hipError_t hipGetDevice(int* d) {
    ++g_log.hip_calls;
    *d = stub::g_cur;
    return hipSuccess;
}

hipError_t hipSetDevice(int d) {
    ++g_log.hip_calls;
    if (d < 0 || d >= stub::kDevices) return hipErrorInvalidDevice;
    ++g_log.set_device_calls;
    stub::g_cur = d;
    return hipSuccess;
}

hipError_t hipGetLastError(void) { return hipSuccess; }

const char* hipGetErrorString(hipError_t) { return "fake runtime error"; }

}  // extern "C"
