// rlk_api.cpp -- the C ABI declared in include/rlk.h: host-side argument
// validation, device binding and the launches.
//
// Validation happens entirely on the host before any HIP call, so a bad
// argument never reaches a kernel ("Final Logit Softcap", Tensor and Precision
// Contract: an invalid cap is rejected up front rather than turning into NaN
// inside a kernel).  Empty inputs return before any HIP call.  The launch
// goes to the device that owns the tensors, not to whichever device happens
// to be current (the device-guard lesson of RL-Kernel pull requests 495 and
// 507), and the caller's current device is restored.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "rlk.h"
#include "rlk_launch.h"

namespace {

thread_local char g_err[512] = "";

rlk_status fail(rlk_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

rlk_status ok() {
    g_err[0] = '\0';
    return RLK_OK;
}

bool dtype_ok(int d) { return d == RLK_F32 || d == RLK_BF16 || d == RLK_F16; }
int64_t esize(int d) { return d == RLK_F32 ? 4 : 2; }

// A fused-head cap: 0 = off, otherwise finite and > 0.
rlk_status check_head_cap(float c, const char* name) {
    if (c == 0.0f) return RLK_OK;
    if (!std::isfinite(c) || !(c > 0.0f))
        return fail(RLK_ERR_ARG, "%s must be 0 (off) or finite and > 0, got %g", name, (double)c);
    return RLK_OK;
}

rlk_status check_matrix(int64_t N, int64_t V, int64_t ld, int64_t es, const char* name) {
    if (N < 0) return fail(RLK_ERR_SHAPE, "N must be >= 0, got %lld", (long long)N);
    if (V < 1) return fail(RLK_ERR_SHAPE, "V must be >= 1, got %lld", (long long)V);
    if (V > INT32_MAX) return fail(RLK_ERR_SHAPE, "V must be < 2^31, got %lld", (long long)V);
    if (ld < V)
        return fail(RLK_ERR_SHAPE, "%s row stride %lld is smaller than V = %lld", name,
                    (long long)ld, (long long)V);
    if (N > 0 && ld > INT64_MAX / es / N)
        return fail(RLK_ERR_SHAPE, "%s: N * ld overflows 64-bit offsets", name);
    return RLK_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Softcap constants of the row kernels (rlk::CapMode): k = -2 log2(e) / c
// gives r = 1 / (1 + 2^(k x)); the statistic input is x with scale log2(e)
// (cap off), r with scale 2 c log2(e) (online form) or t = (y - c) log2(e)
// itself with scale 1 (fixed form, caps with kCapFixedMinScale <=
// 2 c log2(e) <= kCapFixedMaxScale), whose kernels also take 1 / (2 c log2(e)).
// A forward call, its backward and the shard combine all derive the mode from
// the same c.
constexpr double kLog2eD = 1.44269504088896340736;
int cap_mode(float c) {
    if (c == 0.0f) return rlk::kCapNone;
    const double sc = 2.0 * c * kLog2eD;
    return sc >= rlk::kCapFixedMinScale && sc <= rlk::kCapFixedMaxScale ? rlk::kCapFixed
                                                                         : rlk::kCapOnline;
}
float cap_k(float c) { return c != 0.0f ? static_cast<float>(-2.0 * kLog2eD / c) : 0.0f; }
float cap_sc(float c) {
    switch (cap_mode(c)) {
        case rlk::kCapFixed: return 1.0f;
        case rlk::kCapOnline: return static_cast<float>(2.0 * c * kLog2eD);
        default: return static_cast<float>(kLog2eD);
    }
}
float cap_isc(float c) {
    return cap_mode(c) == rlk::kCapFixed ? static_cast<float>(1.0 / (2.0 * c * kLog2eD)) : 0.0f;
}

// Device that owns `ptr` (device or managed memory only).
rlk_status pointer_device(const void* ptr, const char* name, int* dev) {
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, ptr);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(RLK_ERR_DEVICE, "%s is not a HIP allocation (%s)", name, hipGetErrorString(e));
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
        return fail(RLK_ERR_DEVICE, "%s is not device memory", name);
    *dev = attr.device;
    return RLK_OK;
}

// Binds the device owning every listed pointer for the lifetime of the
// object and restores the caller's device afterwards.
class DeviceBinding {
  public:
    rlk_status bind(std::initializer_list<std::pair<const void*, const char*>> ptrs) {
        int dev = -1;
        for (const auto& pn : ptrs) {
            if (pn.first == nullptr) continue;
            int d = -1;
            rlk_status s = pointer_device(pn.first, pn.second, &d);
            if (s != RLK_OK) return s;
            if (dev < 0)
                dev = d;
            else if (d != dev)
                return fail(RLK_ERR_DEVICE, "%s is on device %d but the first tensor is on %d",
                            pn.second, d, dev);
        }
        if (dev < 0) return fail(RLK_ERR_DEVICE, "no device pointer given");
        if (hipGetDevice(&prev_) != hipSuccess) {
            (void)hipGetLastError();
            return fail(RLK_ERR_DEVICE, "hipGetDevice failed");
        }
        if (prev_ != dev) {
            if (hipSetDevice(dev) != hipSuccess) {
                (void)hipGetLastError();
                return fail(RLK_ERR_DEVICE, "hipSetDevice(%d) failed", dev);
            }
            switched_ = true;
        }
        return RLK_OK;
    }
    ~DeviceBinding() {
        if (switched_) (void)hipSetDevice(prev_);
    }

  private:
    int prev_ = -1;
    bool switched_ = false;
};

rlk_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(RLK_ERR_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int rlk_abi_version(void) { return RLK_ABI_VERSION; }

size_t rlk_stats_bytes(rlk_head head, int64_t N, int64_t V) {
    (void)V;
    if (N <= 0 || static_cast<uint64_t>(N) > SIZE_MAX / 32u) return 0;
    if (head != RLK_HEAD_LOGP && head != RLK_HEAD_ENTROPY && head != RLK_HEAD_KL) return 0;
    return static_cast<size_t>(N) * 32u;
}

const char* rlk_status_str(rlk_status s) {
    switch (s) {
        case RLK_OK: return "RLK_OK";
        case RLK_ERR_ARG: return "RLK_ERR_ARG";
        case RLK_ERR_DTYPE: return "RLK_ERR_DTYPE";
        case RLK_ERR_SHAPE: return "RLK_ERR_SHAPE";
        case RLK_ERR_DEVICE: return "RLK_ERR_DEVICE";
        case RLK_ERR_LAUNCH: return "RLK_ERR_LAUNCH";
    }
    return "RLK_ERR_UNKNOWN";
}

const char* rlk_last_error(void) { return g_err; }

// ------------------------------------------------------------- softcap

rlk_status rlk_softcap_fwd(const void* x, rlk_dtype x_dtype, void* y, rlk_dtype y_dtype,
                           int64_t n, float cap, void* stream) {
    if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype))
        return fail(RLK_ERR_DTYPE, "softcap dtypes must be RLK_F32, RLK_BF16 or RLK_F16");
    if (!std::isfinite(cap) || !(cap > 0.0f))
        return fail(RLK_ERR_ARG, "softcap cap must be finite and > 0, got %g", (double)cap);
    if (n < 0) return fail(RLK_ERR_SHAPE, "n must be >= 0, got %lld", (long long)n);
    if (n == 0) return ok();
    if (!x || !y) return fail(RLK_ERR_ARG, "x and y must be non-null when n > 0");
    DeviceBinding dev;
    rlk_status s = dev.bind({{x, "x"}, {y, "y"}});
    if (s != RLK_OK) return s;
    const bool al = aligned16(x) && aligned16(y);
    return launched(rlk::launch_softcap_fwd(x, x_dtype, y, y_dtype, n, cap, al,
                                            static_cast<hipStream_t>(stream)),
                    "softcap_fwd");
}

rlk_status rlk_softcap_bwd(const void* x, rlk_dtype x_dtype, const float* grad_y, void* grad_x,
                           int64_t n, float cap, void* stream) {
    if (!dtype_ok(x_dtype)) return fail(RLK_ERR_DTYPE, "x dtype must be RLK_F32, RLK_BF16 or RLK_F16");
    if (!std::isfinite(cap) || !(cap > 0.0f))
        return fail(RLK_ERR_ARG, "softcap cap must be finite and > 0, got %g", (double)cap);
    if (n < 0) return fail(RLK_ERR_SHAPE, "n must be >= 0, got %lld", (long long)n);
    if (n == 0) return ok();
    if (!x || !grad_y || !grad_x) return fail(RLK_ERR_ARG, "null pointer with n > 0");
    DeviceBinding dev;
    rlk_status s = dev.bind({{x, "x"}, {grad_y, "grad_y"}, {grad_x, "grad_x"}});
    if (s != RLK_OK) return s;
    const bool al = aligned16(x) && aligned16(grad_y) && aligned16(grad_x);
    return launched(rlk::launch_softcap_bwd(x, x_dtype, grad_y, grad_x, n, cap, al,
                                            static_cast<hipStream_t>(stream)),
                    "softcap_bwd");
}

// ------------------------------------------------------------ row layouts

}  // extern "C"

namespace {

using rlk::RowMap;

RowMap plain_rows(int64_t N, int64_t ld) { return RowMap{N > 0 ? N : 1, 0, ld}; }

// Validate a row layout of N rows of V elements (es bytes each).  `output`:
// the rows are written, so they must not overlap.
rlk_status check_rows(const rlk_rows* r, int64_t N, int64_t V, int64_t es, const char* name,
                      bool output, RowMap* m) {
    if (!r) return fail(RLK_ERR_ARG, "%s: layout pointer is null", name);
    const int64_t T = r->rows_per_batch, sb = r->batch_stride, st = r->row_stride;
    if (T < 1) return fail(RLK_ERR_SHAPE, "%s: rows_per_batch must be >= 1", name);
    if (sb < 0 || st < 0) return fail(RLK_ERR_SHAPE, "%s: strides must be >= 0", name);
    const int64_t B = N > 0 ? (N - 1) / T + 1 : 0;  // batches (no N + T - 1 overflow)
    if (N > 0) {
        // the last element touched: (B-1) sb + (min(N,T)-1) st + V - 1 must fit
        const int64_t tmax = (N < T ? N : T) - 1;
        const long double last = (long double)(B - 1) * sb + (long double)tmax * st + V;
        if (last * es > (long double)INT64_MAX)
            return fail(RLK_ERR_SHAPE, "%s: layout overflows 64-bit offsets", name);
    }
    if (output && N > 1) {
        const int64_t Tn = N < T ? N : T;
        const bool rows_ok = Tn == 1 || st >= V;
        const bool batch_major = B == 1 || sb >= (Tn - 1) * st + V;
        const bool time_major = Tn == 1 || st >= (B - 1) * sb + V;
        if (!((rows_ok && batch_major) || (sb >= V && time_major)))
            return fail(RLK_ERR_SHAPE, "%s: output rows overlap", name);
    }
    // (input rows may overlap: a broadcast view is read, never written)
    *m = RowMap{T, sb, st};
    return RLK_OK;
}

bool rows_aligned(const void* base, const RowMap& m, int64_t es) {
    return aligned16(base) && (m.st * es) % 16 == 0 && (m.sb * es) % 16 == 0;
}

rlk_status logp_fwd_impl(const void* logits, rlk_dtype dtype, int64_t N, int64_t V,
                         const RowMap& mx, const int64_t* targets, int64_t k, float softcap,
                         float* logp, void* stats, void* stream) {
    if (N == 0) return ok();
    if (!logits || !targets || !logp || !stats)
        return fail(RLK_ERR_ARG, "logits, targets, logp and stats must be non-null when N > 0");
    DeviceBinding dev;
    rlk_status s = dev.bind({{logits, "logits"}, {targets, "targets"}, {logp, "logp"},
                             {stats, "stats"}});
    if (s != RLK_OK) return s;
    rlk::FwdParams p{};
    p.x = logits;
    p.N = N;
    p.V = V;
    p.vtotal = V;
    p.mx = mx;
    p.my = mx;
    p.targets = targets;
    p.k = k;
    p.kx = cap_k(softcap);
    p.scx = cap_sc(softcap);
    p.ix = cap_isc(softcap);
    p.out = logp;
    p.stats = stats;
    const bool al = rows_aligned(logits, mx, esize(dtype));
    return launched(rlk::launch_fwd(rlk::kHeadLogp, dtype, cap_mode(softcap), rlk::kCapNone, al, p,
                                    static_cast<hipStream_t>(stream)),
                    "logp_fwd");
}

rlk_status logp_bwd_impl(const void* logits, rlk_dtype dtype, int64_t N, int64_t V,
                         const RowMap& mx, const int64_t* targets, int64_t k, float softcap,
                         const void* stats, const float* grad_logp, void* grad_logits,
                         const RowMap& mg, void* stream) {
    if (N == 0) return ok();
    if (!logits || !targets || !stats || !grad_logp || !grad_logits)
        return fail(RLK_ERR_ARG, "null pointer with N > 0");
    DeviceBinding dev;
    rlk_status s = dev.bind({{logits, "logits"}, {targets, "targets"}, {stats, "stats"},
                             {grad_logp, "grad_logp"}, {grad_logits, "grad_logits"}});
    if (s != RLK_OK) return s;
    rlk::BwdParams p{};
    p.x = logits;
    p.N = N;
    p.V = V;
    p.vtotal = V;
    p.mx = mx;
    p.my = mx;
    p.mg = mg;
    p.targets = targets;
    p.k = k;
    p.kx = cap_k(softcap);
    p.scx = cap_sc(softcap);
    p.ix = cap_isc(softcap);
    p.stats = stats;
    p.g = grad_logp;
    p.gx = grad_logits;
    const int64_t es = esize(dtype);
    const bool al = rows_aligned(logits, mx, es) && rows_aligned(grad_logits, mg, es);
    return launched(rlk::launch_bwd(rlk::kHeadLogp, dtype, cap_mode(softcap), rlk::kCapNone, al, p,
                                    static_cast<hipStream_t>(stream)),
                    "logp_bwd");
}

rlk_status entropy_fwd_impl(const void* logits, rlk_dtype dtype, int64_t N, int64_t V,
                            const RowMap& mx, float softcap, float* entropy, void* stats,
                            void* stream) {
    if (N == 0) return ok();
    if (!logits || !entropy || !stats)
        return fail(RLK_ERR_ARG, "logits, entropy and stats must be non-null when N > 0");
    DeviceBinding dev;
    rlk_status s = dev.bind({{logits, "logits"}, {entropy, "entropy"}, {stats, "stats"}});
    if (s != RLK_OK) return s;
    rlk::FwdParams p{};
    p.x = logits;
    p.N = N;
    p.V = V;
    p.vtotal = V;
    p.mx = mx;
    p.my = mx;
    p.k = 1;
    p.kx = cap_k(softcap);
    p.scx = cap_sc(softcap);
    p.ix = cap_isc(softcap);
    p.out = entropy;
    p.stats = stats;
    const bool al = rows_aligned(logits, mx, esize(dtype));
    return launched(rlk::launch_fwd(rlk::kHeadEntropy, dtype, cap_mode(softcap), rlk::kCapNone, al, p,
                                    static_cast<hipStream_t>(stream)),
                    "entropy_fwd");
}

rlk_status entropy_bwd_impl(const void* logits, rlk_dtype dtype, int64_t N, int64_t V,
                            const RowMap& mx, float softcap, const void* stats,
                            const float* grad_entropy, void* grad_logits, const RowMap& mg,
                            void* stream) {
    if (N == 0) return ok();
    if (!logits || !stats || !grad_entropy || !grad_logits)
        return fail(RLK_ERR_ARG, "null pointer with N > 0");
    DeviceBinding dev;
    rlk_status s = dev.bind({{logits, "logits"}, {stats, "stats"},
                             {grad_entropy, "grad_entropy"}, {grad_logits, "grad_logits"}});
    if (s != RLK_OK) return s;
    rlk::BwdParams p{};
    p.x = logits;
    p.N = N;
    p.V = V;
    p.vtotal = V;
    p.mx = mx;
    p.my = mx;
    p.mg = mg;
    p.k = 1;
    p.kx = cap_k(softcap);
    p.scx = cap_sc(softcap);
    p.ix = cap_isc(softcap);
    p.stats = stats;
    p.g = grad_entropy;
    p.gx = grad_logits;
    const int64_t es = esize(dtype);
    const bool al = rows_aligned(logits, mx, es) && rows_aligned(grad_logits, mg, es);
    return launched(rlk::launch_bwd(rlk::kHeadEntropy, dtype, cap_mode(softcap), rlk::kCapNone, al, p,
                                    static_cast<hipStream_t>(stream)),
                    "entropy_bwd");
}

// One KL direction (kl2 == nullptr), or both from one read of the pair:
// reverse KL to (kl, stats) and forward KL to (kl2, stats2).
rlk_status kl_fwd_impl(const void* policy, const void* ref, rlk_dtype dtype, int64_t N, int64_t V,
                       const RowMap& mp, const RowMap& mr, rlk_kl_dir dir, float cp, float cr,
                       float* kl, void* stats, float* kl2, void* stats2, void* stream) {
    const bool both = kl2 != nullptr || stats2 != nullptr;
    if (N == 0) return ok();
    if (!policy || !ref || !kl || !stats || (both && (!kl2 || !stats2)))
        return fail(RLK_ERR_ARG, "policy, ref, outputs and row records must be non-null when N > 0");
    DeviceBinding dev;
    rlk_status s = dev.bind({{policy, "policy"}, {ref, "ref"}, {kl, "kl"}, {stats, "stats"},
                             {kl2, "kl_forward"}, {stats2, "stats_forward"}});
    if (s != RLK_OK) return s;
    rlk::FwdParams p{};
    p.x = policy;
    p.y = ref;
    p.N = N;
    p.V = V;
    p.vtotal = V;
    p.mx = mp;
    p.my = mr;
    p.k = 1;
    p.kx = cap_k(cp);
    p.ky = cap_k(cr);
    p.scx = cap_sc(cp);
    p.ix = cap_isc(cp);
    p.scy = cap_sc(cr);
    p.iy = cap_isc(cr);
    p.out = kl;
    p.stats = stats;
    p.out2 = kl2;
    p.stats2 = stats2;
    const int64_t es = esize(dtype);
    const bool al = rows_aligned(policy, mp, es) && rows_aligned(ref, mr, es);
    const int head = both                    ? rlk::kHeadKLBoth
                     : dir == RLK_KL_REVERSE ? rlk::kHeadKLReverse
                                             : rlk::kHeadKLForward;
    return launched(rlk::launch_fwd(head, dtype, cap_mode(cp), cap_mode(cr), al, p,
                                    static_cast<hipStream_t>(stream)),
                    both ? "kl_fwd_both" : "kl_fwd");
}

// Gradient of the KL w.r.t. the policy, or (wrt_ref) w.r.t. the reference.
// The reference gradient of one direction is the policy gradient of the other
// direction with the two tensors swapped (KL(P||R) is the forward KL of the
// pair policy R, reference P), so it runs the same kernels with the operands,
// the caps and the two sides of the row record exchanged.
rlk_status kl_bwd_impl(const void* policy, const void* ref, rlk_dtype dtype, int64_t N, int64_t V,
                       const RowMap& mp, const RowMap& mr, rlk_kl_dir dir, float cp, float cr,
                       const void* stats, const float* grad_kl, void* grad_out,
                       const RowMap& mg, bool wrt_ref, void* stream) {
    if (N == 0) return ok();
    if (!policy || !ref || !stats || !grad_kl || !grad_out)
        return fail(RLK_ERR_ARG, "null pointer with N > 0");
    const char* gname = wrt_ref ? "grad_ref" : "grad_policy";
    DeviceBinding dev;
    rlk_status s = dev.bind({{policy, "policy"}, {ref, "ref"}, {stats, "stats"},
                             {grad_kl, "grad_kl"}, {grad_out, gname}});
    if (s != RLK_OK) return s;
    rlk::BwdParams p{};
    p.x = wrt_ref ? ref : policy;
    p.y = wrt_ref ? policy : ref;
    p.N = N;
    p.V = V;
    p.vtotal = V;
    p.mx = wrt_ref ? mr : mp;
    p.my = wrt_ref ? mp : mr;
    p.mg = mg;
    p.k = 1;
    const float cx = wrt_ref ? cr : cp, cy = wrt_ref ? cp : cr;
    p.kx = cap_k(cx);
    p.ky = cap_k(cy);
    p.scx = cap_sc(cx);
    p.ix = cap_isc(cx);
    p.scy = cap_sc(cy);
    p.iy = cap_isc(cy);
    p.stats = stats;
    p.swap = wrt_ref ? 1 : 0;
    p.g = grad_kl;
    p.gx = grad_out;
    const int64_t es = esize(dtype);
    const bool al = rows_aligned(policy, mp, es) && rows_aligned(ref, mr, es) &&
                    rows_aligned(grad_out, mg, es);
    const bool reverse = (dir == RLK_KL_REVERSE) != wrt_ref;
    const int head = reverse ? rlk::kHeadKLReverse : rlk::kHeadKLForward;
    return launched(rlk::launch_bwd(head, dtype, cap_mode(cx), cap_mode(cy), al, p,
                                    static_cast<hipStream_t>(stream)),
                    wrt_ref ? "kl_bwd_ref" : "kl_bwd");
}

rlk_status check_common(rlk_dtype dtype, int64_t N, int64_t V, float cap, const char* capname) {
    if (!dtype_ok(dtype))
        return fail(RLK_ERR_DTYPE, "logits dtype must be RLK_F32, RLK_BF16 or RLK_F16");
    if (N < 0) return fail(RLK_ERR_SHAPE, "N must be >= 0, got %lld", (long long)N);
    if (V < 1) return fail(RLK_ERR_SHAPE, "V must be >= 1, got %lld", (long long)V);
    if (V > INT32_MAX) return fail(RLK_ERR_SHAPE, "V must be < 2^31, got %lld", (long long)V);
    return check_head_cap(cap, capname);
}

rlk_status check_k(int64_t N, int64_t k) {
    if (k < 1 || k > RLK_MAX_TOPK)
        return fail(RLK_ERR_SHAPE, "k must be in [1, %d], got %lld", RLK_MAX_TOPK, (long long)k);
    if (N > 0 && k > INT64_MAX / N) return fail(RLK_ERR_SHAPE, "N * k overflows");
    return RLK_OK;
}

rlk_status check_dir(rlk_kl_dir dir) {
    if (dir != RLK_KL_REVERSE && dir != RLK_KL_FORWARD)
        return fail(RLK_ERR_ARG, "dir must be RLK_KL_REVERSE or RLK_KL_FORWARD, got %d", (int)dir);
    return RLK_OK;
}

// A vocabulary shard: columns [v0, v0 + V_shard) of rows of width V_total,
// stored with row stride ld.  An empty shard (V_shard = 0) is allowed.
rlk_status check_shard(int64_t N, int64_t V_shard, int64_t ld, int64_t v0, int64_t V_total,
                       int64_t es, const char* name) {
    if (N < 0) return fail(RLK_ERR_SHAPE, "N must be >= 0, got %lld", (long long)N);
    if (V_shard < 0) return fail(RLK_ERR_SHAPE, "%s: V_shard must be >= 0", name);
    if (v0 < 0 || v0 + V_shard > V_total)
        return fail(RLK_ERR_SHAPE, "%s: shard [%lld, %lld) is outside [0, %lld)", name,
                    (long long)v0, (long long)(v0 + V_shard), (long long)V_total);
    if (V_shard > 0 && ld < V_shard)
        return fail(RLK_ERR_SHAPE, "%s: row stride %lld is smaller than V_shard = %lld", name,
                    (long long)ld, (long long)V_shard);
    if (N > 0 && V_shard > 0 && ld > INT64_MAX / es / N)
        return fail(RLK_ERR_SHAPE, "%s: N * ld overflows 64-bit offsets", name);
    return RLK_OK;
}

#define RLK_TRY(expr)                          \
    do {                                       \
        const rlk_status s_ = (expr);          \
        if (s_ != RLK_OK) return s_;           \
    } while (0)

}  // namespace

extern "C" {

// ------------------------------------------------------------ logprobs

rlk_status rlk_logp_fwd(const void* logits, rlk_dtype dtype, int64_t N, int64_t V, int64_t ld,
                        const int64_t* targets, int64_t k, float softcap, float* logp,
                        void* stats, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap, "softcap"));
    RLK_TRY(check_matrix(N, V, ld, esize(dtype), "logits"));
    RLK_TRY(check_k(N, k));
    return logp_fwd_impl(logits, dtype, N, V, plain_rows(N, ld), targets, k, softcap, logp, stats,
                         stream);
}

rlk_status rlk_logp_bwd(const void* logits, rlk_dtype dtype, int64_t N, int64_t V, int64_t ld,
                        const int64_t* targets, int64_t k, float softcap, const void* stats,
                        const float* grad_logp, void* grad_logits, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap, "softcap"));
    RLK_TRY(check_matrix(N, V, ld, esize(dtype), "logits"));
    RLK_TRY(check_k(N, k));
    return logp_bwd_impl(logits, dtype, N, V, plain_rows(N, ld), targets, k, softcap, stats,
                         grad_logp, grad_logits, plain_rows(N, V), stream);
}

rlk_status rlk_logp_fwd_strided(const void* logits, rlk_dtype dtype, int64_t N, int64_t V,
                                const rlk_rows* rows, const int64_t* targets, int64_t k,
                                float softcap, float* logp, void* stats, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap, "softcap"));
    RowMap mx;
    RLK_TRY(check_rows(rows, N, V, esize(dtype), "logits", false, &mx));
    RLK_TRY(check_k(N, k));
    return logp_fwd_impl(logits, dtype, N, V, mx, targets, k, softcap, logp, stats, stream);
}

rlk_status rlk_logp_bwd_strided(const void* logits, rlk_dtype dtype, int64_t N, int64_t V,
                                const rlk_rows* rows, const int64_t* targets, int64_t k,
                                float softcap, const void* stats, const float* grad_logp,
                                void* grad_logits, const rlk_rows* grad_rows, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap, "softcap"));
    RowMap mx, mg;
    RLK_TRY(check_rows(rows, N, V, esize(dtype), "logits", false, &mx));
    RLK_TRY(check_rows(grad_rows, N, V, esize(dtype), "grad_logits", true, &mg));
    RLK_TRY(check_k(N, k));
    return logp_bwd_impl(logits, dtype, N, V, mx, targets, k, softcap, stats, grad_logp,
                         grad_logits, mg, stream);
}

// -------------------------------------------------------------- entropy

rlk_status rlk_entropy_fwd(const void* logits, rlk_dtype dtype, int64_t N, int64_t V, int64_t ld,
                           float softcap, float* entropy, void* stats, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap, "softcap"));
    RLK_TRY(check_matrix(N, V, ld, esize(dtype), "logits"));
    return entropy_fwd_impl(logits, dtype, N, V, plain_rows(N, ld), softcap, entropy, stats,
                            stream);
}

rlk_status rlk_entropy_bwd(const void* logits, rlk_dtype dtype, int64_t N, int64_t V, int64_t ld,
                           float softcap, const void* stats, const float* grad_entropy,
                           void* grad_logits, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap, "softcap"));
    RLK_TRY(check_matrix(N, V, ld, esize(dtype), "logits"));
    return entropy_bwd_impl(logits, dtype, N, V, plain_rows(N, ld), softcap, stats, grad_entropy,
                            grad_logits, plain_rows(N, V), stream);
}

rlk_status rlk_entropy_fwd_strided(const void* logits, rlk_dtype dtype, int64_t N, int64_t V,
                                   const rlk_rows* rows, float softcap, float* entropy,
                                   void* stats, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap, "softcap"));
    RowMap mx;
    RLK_TRY(check_rows(rows, N, V, esize(dtype), "logits", false, &mx));
    return entropy_fwd_impl(logits, dtype, N, V, mx, softcap, entropy, stats, stream);
}

rlk_status rlk_entropy_bwd_strided(const void* logits, rlk_dtype dtype, int64_t N, int64_t V,
                                   const rlk_rows* rows, float softcap, const void* stats,
                                   const float* grad_entropy, void* grad_logits,
                                   const rlk_rows* grad_rows, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap, "softcap"));
    RowMap mx, mg;
    RLK_TRY(check_rows(rows, N, V, esize(dtype), "logits", false, &mx));
    RLK_TRY(check_rows(grad_rows, N, V, esize(dtype), "grad_logits", true, &mg));
    return entropy_bwd_impl(logits, dtype, N, V, mx, softcap, stats, grad_entropy, grad_logits,
                            mg, stream);
}

// ------------------------------------------------------------------- KL

rlk_status rlk_kl_fwd(const void* policy, const void* ref, rlk_dtype dtype, int64_t N, int64_t V,
                      int64_t ld_policy, int64_t ld_ref, rlk_kl_dir dir, float softcap_policy,
                      float softcap_ref, float* kl, void* stats, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap_policy, "softcap_policy"));
    RLK_TRY(check_head_cap(softcap_ref, "softcap_ref"));
    RLK_TRY(check_matrix(N, V, ld_policy, esize(dtype), "policy"));
    RLK_TRY(check_matrix(N, V, ld_ref, esize(dtype), "ref"));
    RLK_TRY(check_dir(dir));
    return kl_fwd_impl(policy, ref, dtype, N, V, plain_rows(N, ld_policy), plain_rows(N, ld_ref),
                       dir, softcap_policy, softcap_ref, kl, stats, nullptr, nullptr, stream);
}

rlk_status rlk_kl_fwd_both(const void* policy, const void* ref, rlk_dtype dtype, int64_t N,
                           int64_t V, int64_t ld_policy, int64_t ld_ref, float softcap_policy,
                           float softcap_ref, float* kl_reverse, void* stats_reverse,
                           float* kl_forward, void* stats_forward, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap_policy, "softcap_policy"));
    RLK_TRY(check_head_cap(softcap_ref, "softcap_ref"));
    RLK_TRY(check_matrix(N, V, ld_policy, esize(dtype), "policy"));
    RLK_TRY(check_matrix(N, V, ld_ref, esize(dtype), "ref"));
    if (N > 0 && (!kl_forward || !stats_forward))
        return fail(RLK_ERR_ARG, "kl_forward and stats_forward must be non-null when N > 0");
    return kl_fwd_impl(policy, ref, dtype, N, V, plain_rows(N, ld_policy), plain_rows(N, ld_ref),
                       RLK_KL_REVERSE, softcap_policy, softcap_ref, kl_reverse, stats_reverse,
                       kl_forward, stats_forward, stream);
}

rlk_status rlk_kl_bwd(const void* policy, const void* ref, rlk_dtype dtype, int64_t N, int64_t V,
                      int64_t ld_policy, int64_t ld_ref, rlk_kl_dir dir, float softcap_policy,
                      float softcap_ref, const void* stats, const float* grad_kl,
                      void* grad_policy, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap_policy, "softcap_policy"));
    RLK_TRY(check_head_cap(softcap_ref, "softcap_ref"));
    RLK_TRY(check_matrix(N, V, ld_policy, esize(dtype), "policy"));
    RLK_TRY(check_matrix(N, V, ld_ref, esize(dtype), "ref"));
    RLK_TRY(check_dir(dir));
    return kl_bwd_impl(policy, ref, dtype, N, V, plain_rows(N, ld_policy), plain_rows(N, ld_ref),
                       dir, softcap_policy, softcap_ref, stats, grad_kl, grad_policy,
                       plain_rows(N, V), false, stream);
}

rlk_status rlk_kl_fwd_strided(const void* policy, const void* ref, rlk_dtype dtype, int64_t N,
                              int64_t V, const rlk_rows* policy_rows, const rlk_rows* ref_rows,
                              rlk_kl_dir dir, float softcap_policy, float softcap_ref, float* kl,
                              void* stats, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap_policy, "softcap_policy"));
    RLK_TRY(check_head_cap(softcap_ref, "softcap_ref"));
    RowMap mp, mr;
    RLK_TRY(check_rows(policy_rows, N, V, esize(dtype), "policy", false, &mp));
    RLK_TRY(check_rows(ref_rows, N, V, esize(dtype), "ref", false, &mr));
    RLK_TRY(check_dir(dir));
    return kl_fwd_impl(policy, ref, dtype, N, V, mp, mr, dir, softcap_policy, softcap_ref, kl,
                       stats, nullptr, nullptr, stream);
}

rlk_status rlk_kl_fwd_both_strided(const void* policy, const void* ref, rlk_dtype dtype,
                                   int64_t N, int64_t V, const rlk_rows* policy_rows,
                                   const rlk_rows* ref_rows, float softcap_policy,
                                   float softcap_ref, float* kl_reverse, void* stats_reverse,
                                   float* kl_forward, void* stats_forward, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap_policy, "softcap_policy"));
    RLK_TRY(check_head_cap(softcap_ref, "softcap_ref"));
    RowMap mp, mr;
    RLK_TRY(check_rows(policy_rows, N, V, esize(dtype), "policy", false, &mp));
    RLK_TRY(check_rows(ref_rows, N, V, esize(dtype), "ref", false, &mr));
    if (N > 0 && (!kl_forward || !stats_forward))
        return fail(RLK_ERR_ARG, "kl_forward and stats_forward must be non-null when N > 0");
    return kl_fwd_impl(policy, ref, dtype, N, V, mp, mr, RLK_KL_REVERSE, softcap_policy,
                       softcap_ref, kl_reverse, stats_reverse, kl_forward, stats_forward, stream);
}

rlk_status rlk_kl_bwd_strided(const void* policy, const void* ref, rlk_dtype dtype, int64_t N,
                              int64_t V, const rlk_rows* policy_rows, const rlk_rows* ref_rows,
                              rlk_kl_dir dir, float softcap_policy, float softcap_ref,
                              const void* stats, const float* grad_kl, void* grad_policy,
                              const rlk_rows* grad_rows, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap_policy, "softcap_policy"));
    RLK_TRY(check_head_cap(softcap_ref, "softcap_ref"));
    RowMap mp, mr, mg;
    RLK_TRY(check_rows(policy_rows, N, V, esize(dtype), "policy", false, &mp));
    RLK_TRY(check_rows(ref_rows, N, V, esize(dtype), "ref", false, &mr));
    RLK_TRY(check_rows(grad_rows, N, V, esize(dtype), "grad_policy", true, &mg));
    RLK_TRY(check_dir(dir));
    return kl_bwd_impl(policy, ref, dtype, N, V, mp, mr, dir, softcap_policy, softcap_ref, stats,
                       grad_kl, grad_policy, mg, false, stream);
}

rlk_status rlk_kl_bwd_ref(const void* policy, const void* ref, rlk_dtype dtype, int64_t N,
                          int64_t V, int64_t ld_policy, int64_t ld_ref, rlk_kl_dir dir,
                          float softcap_policy, float softcap_ref, const void* stats,
                          const float* grad_kl, void* grad_ref, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap_policy, "softcap_policy"));
    RLK_TRY(check_head_cap(softcap_ref, "softcap_ref"));
    RLK_TRY(check_matrix(N, V, ld_policy, esize(dtype), "policy"));
    RLK_TRY(check_matrix(N, V, ld_ref, esize(dtype), "ref"));
    RLK_TRY(check_dir(dir));
    return kl_bwd_impl(policy, ref, dtype, N, V, plain_rows(N, ld_policy), plain_rows(N, ld_ref),
                       dir, softcap_policy, softcap_ref, stats, grad_kl, grad_ref,
                       plain_rows(N, V), true, stream);
}

rlk_status rlk_kl_bwd_ref_strided(const void* policy, const void* ref, rlk_dtype dtype, int64_t N,
                                  int64_t V, const rlk_rows* policy_rows,
                                  const rlk_rows* ref_rows, rlk_kl_dir dir, float softcap_policy,
                                  float softcap_ref, const void* stats, const float* grad_kl,
                                  void* grad_ref, const rlk_rows* grad_rows, void* stream) {
    RLK_TRY(check_common(dtype, N, V, softcap_policy, "softcap_policy"));
    RLK_TRY(check_head_cap(softcap_ref, "softcap_ref"));
    RowMap mp, mr, mg;
    RLK_TRY(check_rows(policy_rows, N, V, esize(dtype), "policy", false, &mp));
    RLK_TRY(check_rows(ref_rows, N, V, esize(dtype), "ref", false, &mr));
    RLK_TRY(check_rows(grad_rows, N, V, esize(dtype), "grad_ref", true, &mg));
    RLK_TRY(check_dir(dir));
    return kl_bwd_impl(policy, ref, dtype, N, V, mp, mr, dir, softcap_policy, softcap_ref, stats,
                       grad_kl, grad_ref, mg, true, stream);
}

// ------------------------------------------------- vocabulary shards

size_t rlk_partial_bytes(int64_t N) {
    if (N <= 0 || static_cast<uint64_t>(N) > SIZE_MAX / 32u) return 0;
    return static_cast<size_t>(N) * 32u;
}

rlk_status rlk_logp_fwd_partial(const void* logits, rlk_dtype dtype, int64_t N, int64_t V_shard,
                                int64_t ld, int64_t v0, int64_t V_total, const int64_t* targets,
                                int64_t k, float softcap, void* partial, float* target_vals,
                                void* stream) {
    RLK_TRY(check_common(dtype, N, V_total, softcap, "softcap"));
    RLK_TRY(check_shard(N, V_shard, ld, v0, V_total, esize(dtype), "logits"));
    RLK_TRY(check_k(N, k));
    if (N == 0) return ok();
    if ((!logits && V_shard > 0) || !targets || !partial || !target_vals)
        return fail(RLK_ERR_ARG, "null pointer with N > 0");
    DeviceBinding dev;
    RLK_TRY(dev.bind({{logits, "logits"}, {targets, "targets"}, {partial, "partial"},
                      {target_vals, "target_vals"}}));
    rlk::FwdParams p{};
    p.x = logits;
    p.N = N;
    p.V = V_shard;
    p.mx = plain_rows(N, ld);
    p.my = p.mx;
    p.targets = targets;
    p.k = k;
    p.kx = cap_k(softcap);
    p.scx = cap_sc(softcap);
    p.ix = cap_isc(softcap);
    p.v0 = v0;
    p.vtotal = V_total;
    p.part = partial;
    p.tvals = target_vals;
    const bool al = rows_aligned(logits, p.mx, esize(dtype));
    return launched(rlk::launch_fwd(rlk::kHeadLogp, dtype, cap_mode(softcap), rlk::kCapNone, al, p,
                                    static_cast<hipStream_t>(stream)),
                    "logp_fwd_partial");
}

rlk_status rlk_entropy_fwd_partial(const void* logits, rlk_dtype dtype, int64_t N,
                                   int64_t V_shard, int64_t ld, float softcap, void* partial,
                                   void* stream) {
    RLK_TRY(check_common(dtype, N, V_shard > 0 ? V_shard : 1, softcap, "softcap"));
    RLK_TRY(check_shard(N, V_shard, ld, 0, V_shard, esize(dtype), "logits"));
    if (N == 0) return ok();
    if ((!logits && V_shard > 0) || !partial) return fail(RLK_ERR_ARG, "null pointer with N > 0");
    DeviceBinding dev;
    RLK_TRY(dev.bind({{logits, "logits"}, {partial, "partial"}}));
    rlk::FwdParams p{};
    p.x = logits;
    p.N = N;
    p.V = V_shard;
    p.vtotal = V_shard;
    p.mx = plain_rows(N, ld);
    p.my = p.mx;
    p.k = 1;
    p.kx = cap_k(softcap);
    p.scx = cap_sc(softcap);
    p.ix = cap_isc(softcap);
    p.part = partial;
    const bool al = rows_aligned(logits, p.mx, esize(dtype));
    return launched(rlk::launch_fwd(rlk::kHeadEntropy, dtype, cap_mode(softcap), rlk::kCapNone, al, p,
                                    static_cast<hipStream_t>(stream)),
                    "entropy_fwd_partial");
}

rlk_status rlk_kl_fwd_partial(const void* policy, const void* ref, rlk_dtype dtype, int64_t N,
                              int64_t V_shard, int64_t ld_policy, int64_t ld_ref, rlk_kl_dir dir,
                              float softcap_policy, float softcap_ref, void* partial,
                              void* stream) {
    RLK_TRY(check_common(dtype, N, V_shard > 0 ? V_shard : 1, softcap_policy, "softcap_policy"));
    RLK_TRY(check_head_cap(softcap_ref, "softcap_ref"));
    RLK_TRY(check_shard(N, V_shard, ld_policy, 0, V_shard, esize(dtype), "policy"));
    RLK_TRY(check_shard(N, V_shard, ld_ref, 0, V_shard, esize(dtype), "ref"));
    RLK_TRY(check_dir(dir));
    if (N == 0) return ok();
    if (((!policy || !ref) && V_shard > 0) || !partial)
        return fail(RLK_ERR_ARG, "null pointer with N > 0");
    DeviceBinding dev;
    RLK_TRY(dev.bind({{policy, "policy"}, {ref, "ref"}, {partial, "partial"}}));
    rlk::FwdParams p{};
    p.x = policy;
    p.y = ref;
    p.N = N;
    p.V = V_shard;
    p.vtotal = V_shard;
    p.mx = plain_rows(N, ld_policy);
    p.my = plain_rows(N, ld_ref);
    p.k = 1;
    p.kx = cap_k(softcap_policy);
    p.ky = cap_k(softcap_ref);
    p.scx = cap_sc(softcap_policy);
    p.ix = cap_isc(softcap_policy);
    p.scy = cap_sc(softcap_ref);
    p.iy = cap_isc(softcap_ref);
    p.part = partial;
    const int64_t es = esize(dtype);
    const bool al = rows_aligned(policy, p.mx, es) && rows_aligned(ref, p.my, es);
    const int head = dir == RLK_KL_REVERSE ? rlk::kHeadKLReverse : rlk::kHeadKLForward;
    return launched(rlk::launch_fwd(head, dtype, cap_mode(softcap_policy), cap_mode(softcap_ref), al,
                                    p, static_cast<hipStream_t>(stream)),
                    "kl_fwd_partial");
}

rlk_status rlk_combine(rlk_head head, rlk_kl_dir dir, int64_t P, const int64_t* bounds, int64_t N,
                       const void* partials, const int64_t* targets, int64_t k,
                       const float* target_vals, float softcap, float* out, void* stats,
                       void* stream) {
    if (head != RLK_HEAD_LOGP && head != RLK_HEAD_ENTROPY && head != RLK_HEAD_KL)
        return fail(RLK_ERR_ARG, "unknown head %d", (int)head);
    if (head == RLK_HEAD_KL) RLK_TRY(check_dir(dir));
    if (P < 1 || P > RLK_MAX_SHARDS)
        return fail(RLK_ERR_SHAPE, "P must be in [1, %d], got %lld", RLK_MAX_SHARDS, (long long)P);
    if (!bounds) return fail(RLK_ERR_ARG, "bounds (host array of P + 1 columns) is null");
    if (bounds[0] != 0) return fail(RLK_ERR_SHAPE, "bounds[0] must be 0");
    for (int64_t s = 0; s < P; ++s)
        if (bounds[s + 1] < bounds[s]) return fail(RLK_ERR_SHAPE, "bounds must not decrease");
    const int64_t V_total = bounds[P];
    if (V_total < 1 || V_total > INT32_MAX)
        return fail(RLK_ERR_SHAPE, "the vocabulary width bounds[P] must be in [1, 2^31)");
    if (N < 0) return fail(RLK_ERR_SHAPE, "N must be >= 0");
    if (head == RLK_HEAD_LOGP) {
        RLK_TRY(check_k(N, k));
        RLK_TRY(check_head_cap(softcap, "softcap"));
    }
    if (N > 0 && P > INT64_MAX / N) return fail(RLK_ERR_SHAPE, "P * N overflows");
    if (N == 0) return ok();
    if (!partials || !out || !stats) return fail(RLK_ERR_ARG, "null pointer with N > 0");
    if (head == RLK_HEAD_LOGP && (!targets || !target_vals))
        return fail(RLK_ERR_ARG, "logprobs combine needs targets and target_vals");
    DeviceBinding dev;
    RLK_TRY(dev.bind({{partials, "partials"}, {out, "out"}, {stats, "stats"},
                      {head == RLK_HEAD_LOGP ? targets : nullptr, "targets"},
                      {head == RLK_HEAD_LOGP ? target_vals : nullptr, "target_vals"}}));
    rlk::CombineParams q{};
    q.P = static_cast<int>(P);
    q.N = N;
    q.k = head == RLK_HEAD_LOGP ? k : 1;
    q.vtotal = V_total;
    for (int64_t s = 0; s <= P; ++s) q.bounds[s] = bounds[s];
    q.part = partials;
    q.targets = targets;
    q.tvals = target_vals;
    q.sc = cap_sc(softcap);
    q.out = out;
    q.stats = stats;
    const int h = head == RLK_HEAD_LOGP      ? rlk::kHeadLogp
                  : head == RLK_HEAD_ENTROPY ? rlk::kHeadEntropy
                  : dir == RLK_KL_REVERSE    ? rlk::kHeadKLReverse
                                             : rlk::kHeadKLForward;
    return launched(rlk::launch_combine(h, q, static_cast<hipStream_t>(stream)), "combine");
}

rlk_status rlk_logp_bwd_shard(const void* logits, rlk_dtype dtype, int64_t N, int64_t V_shard,
                              int64_t ld, int64_t v0, int64_t V_total, const int64_t* targets,
                              int64_t k, float softcap, const void* stats,
                              const float* grad_logp, void* grad_logits, void* stream) {
    RLK_TRY(check_common(dtype, N, V_total, softcap, "softcap"));
    RLK_TRY(check_shard(N, V_shard, ld, v0, V_total, esize(dtype), "logits"));
    RLK_TRY(check_k(N, k));
    if (N == 0 || V_shard == 0) return ok();
    if (!logits || !targets || !stats || !grad_logp || !grad_logits)
        return fail(RLK_ERR_ARG, "null pointer with N > 0");
    DeviceBinding dev;
    RLK_TRY(dev.bind({{logits, "logits"}, {targets, "targets"}, {stats, "stats"},
                      {grad_logp, "grad_logp"}, {grad_logits, "grad_logits"}}));
    rlk::BwdParams p{};
    p.x = logits;
    p.N = N;
    p.V = V_shard;
    p.v0 = v0;
    p.vtotal = V_total;
    p.mx = plain_rows(N, ld);
    p.my = p.mx;
    p.mg = plain_rows(N, V_shard);
    p.targets = targets;
    p.k = k;
    p.kx = cap_k(softcap);
    p.scx = cap_sc(softcap);
    p.ix = cap_isc(softcap);
    p.stats = stats;
    p.g = grad_logp;
    p.gx = grad_logits;
    const int64_t es = esize(dtype);
    const bool al = rows_aligned(logits, p.mx, es) && rows_aligned(grad_logits, p.mg, es);
    return launched(rlk::launch_bwd(rlk::kHeadLogp, dtype, cap_mode(softcap), rlk::kCapNone, al, p,
                                    static_cast<hipStream_t>(stream)),
                    "logp_bwd_shard");
}

}  // extern "C"
