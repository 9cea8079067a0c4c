// driver.cpp -- drives every C ABI entry point of the host-only build
// (rlk_api.cpp + stub_hip.cpp) under AddressSanitizer and UBSan.
//
// For each call it checks the status, that failures happen before any HIP
// call, that a successful call launches exactly once on the device owning
// the tensors (and restores the caller's device), the kernel parameters the
// host derived (sizes, caps, row maps, shard bounds, alignment), and that the
// launch stays inside the fake allocations.  The input-validation cases follow
// the boundary's documented errors (include/rlk.h): null pointers, V = 0,
// k outside [1, 4096], row strides below V, 64-bit offset overflow, overlapping
// gradient rows, invalid caps and directions, mixed devices, host memory,
// shard and combine bounds.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>

#include "rlk.h"
#include "stub_hip.h"

using stub::g_log;

static int g_checks = 0, g_failed = 0;

#define CHECK(cond)                                                                    \
    do {                                                                               \
        ++g_checks;                                                                    \
        if (!(cond)) {                                                                 \
            ++g_failed;                                                                \
            std::fprintf(stderr, "%s:%d: CHECK failed: %s (last error: %s)\n", __FILE__, \
                         __LINE__, #cond, rlk_last_error());                           \
        }                                                                              \
    } while (0)

// A call that must fail with `st` before touching the runtime.
#define EXPECT_FAIL(st, call)                                  \
    do {                                                       \
        stub::reset_log();                                     \
        const rlk_status s_ = (call);                          \
        CHECK(s_ == (st));                                     \
        CHECK(g_log.launches == 0);                            \
        CHECK(std::strlen(rlk_last_error()) > 0);              \
        if ((st) != RLK_ERR_DEVICE) CHECK(g_log.hip_calls == 0); \
    } while (0)

// A call that must succeed with one launch on `dev`, leaving the caller's
// device current and staying inside the allocations.
#define EXPECT_LAUNCH(dev, call)                         \
    do {                                                 \
        stub::reset_log();                               \
        const int cur_ = stub::current_device();         \
        const rlk_status s_ = (call);                    \
        CHECK(s_ == RLK_OK);                             \
        CHECK(g_log.launches == 1);                      \
        CHECK(g_log.device == (dev));                    \
        CHECK(g_log.range_errors == 0);                  \
        CHECK(stub::current_device() == cur_);           \
        CHECK(rlk_last_error()[0] == '\0');              \
    } while (0)

// N = 0 (or n = 0): OK with no HIP call at all.
#define EXPECT_EMPTY(call)              \
    do {                                \
        stub::reset_log();              \
        CHECK((call) == RLK_OK);        \
        CHECK(g_log.hip_calls == 0);    \
        CHECK(g_log.launches == 0);     \
    } while (0)

static const float kNaN = std::numeric_limits<float>::quiet_NaN();
static const float kInf = std::numeric_limits<float>::infinity();

static int64_t es(rlk_dtype d) { return d == RLK_F32 ? 4 : 2; }

static void test_status_and_sizes() {
    const rlk_status all[] = {RLK_OK, RLK_ERR_ARG, RLK_ERR_DTYPE, RLK_ERR_SHAPE, RLK_ERR_DEVICE,
                              RLK_ERR_LAUNCH};
    for (rlk_status s : all) CHECK(std::strncmp(rlk_status_str(s), "RLK_", 4) == 0);
    CHECK(std::strcmp(rlk_status_str(static_cast<rlk_status>(99)), "RLK_ERR_UNKNOWN") == 0);
    CHECK(rlk_abi_version() == RLK_ABI_VERSION);
    CHECK(rlk_stats_bytes(RLK_HEAD_LOGP, 10, 100) == 320);
    CHECK(rlk_stats_bytes(RLK_HEAD_KL, 0, 100) == 0);
    CHECK(rlk_stats_bytes(RLK_HEAD_ENTROPY, -5, 100) == 0);
    CHECK(rlk_stats_bytes(static_cast<rlk_head>(7), 10, 100) == 0);
    // sizes that do not fit size_t are 0, never a wrapped small value
    CHECK(rlk_stats_bytes(RLK_HEAD_LOGP, INT64_MAX, 100) == 0);
    CHECK(rlk_stats_bytes(RLK_HEAD_LOGP, (int64_t(1) << 59) + 1, 100) == 0);
    CHECK(rlk_partial_bytes(7) == 224);
    CHECK(rlk_partial_bytes(0) == 0);
    CHECK(rlk_partial_bytes(INT64_MAX) == 0);
}

static void test_softcap() {
    const int64_t n = 1000;
    for (rlk_dtype xd : {RLK_F32, RLK_BF16, RLK_F16})
        for (rlk_dtype yd : {RLK_F32, RLK_BF16, RLK_F16}) {
            void* x = stub::fake_alloc(n * es(xd));
            void* y = stub::fake_alloc(n * es(yd));
            float* gy = static_cast<float*>(stub::fake_alloc(n * 4));
            void* gx = stub::fake_alloc(n * es(xd));
            EXPECT_LAUNCH(0, rlk_softcap_fwd(x, xd, y, yd, n, 30.0f, nullptr));
            CHECK(g_log.kind == stub::kSoftcapFwd && g_log.n == n && g_log.cap == 30.0f);
            CHECK(g_log.dtype == xd && g_log.dtype_y == yd && g_log.aligned);
            EXPECT_LAUNCH(0, rlk_softcap_bwd(x, xd, gy, gx, n, 20.0f, nullptr));
            CHECK(g_log.kind == stub::kSoftcapBwd && g_log.n == n);
            // misaligned y: still launched, with the element path
            EXPECT_LAUNCH(0, rlk_softcap_fwd(x, xd, static_cast<char*>(y) + es(yd), yd, n - 1,
                                             30.0f, nullptr));
            CHECK(!g_log.aligned);
        }
    void* x = stub::fake_alloc(4000);
    void* y = stub::fake_alloc(4000);
    EXPECT_EMPTY(rlk_softcap_fwd(nullptr, RLK_F32, nullptr, RLK_F32, 0, 30.0f, nullptr));
    EXPECT_FAIL(RLK_ERR_ARG, rlk_softcap_fwd(x, RLK_F32, y, RLK_F32, 10, 0.0f, nullptr));
    EXPECT_FAIL(RLK_ERR_ARG, rlk_softcap_fwd(x, RLK_F32, y, RLK_F32, 10, -1.0f, nullptr));
    EXPECT_FAIL(RLK_ERR_ARG, rlk_softcap_fwd(x, RLK_F32, y, RLK_F32, 10, kNaN, nullptr));
    EXPECT_FAIL(RLK_ERR_ARG, rlk_softcap_bwd(x, RLK_F32, (float*)y, y, 10, kInf, nullptr));
    EXPECT_FAIL(RLK_ERR_DTYPE, rlk_softcap_fwd(x, static_cast<rlk_dtype>(3), y, RLK_F32, 10, 30.0f,
                                                nullptr));
    EXPECT_FAIL(RLK_ERR_SHAPE, rlk_softcap_fwd(x, RLK_F32, y, RLK_F32, -1, 30.0f, nullptr));
    EXPECT_FAIL(RLK_ERR_ARG, rlk_softcap_fwd(nullptr, RLK_F32, y, RLK_F32, 10, 30.0f, nullptr));
}

static void test_logp() {
    const int64_t N = 37, V = 1031, ld = 1040, k = 5;
    for (rlk_dtype d : {RLK_F32, RLK_BF16, RLK_F16}) {
        void* x = stub::fake_alloc(N * ld * es(d));
        int64_t* t = static_cast<int64_t*>(stub::fake_alloc(N * k * 8));
        float* out = static_cast<float*>(stub::fake_alloc(N * k * 4));
        void* st = stub::fake_alloc(rlk_stats_bytes(RLK_HEAD_LOGP, N, V));
        float* g = static_cast<float*>(stub::fake_alloc(N * k * 4));
        void* gx = stub::fake_alloc(N * V * es(d));
        for (float cap : {0.0f, 20.0f, 30.0f, 50.0f, 1e-7f}) {
            EXPECT_LAUNCH(0, rlk_logp_fwd(x, d, N, V, ld, t, k, cap, out, st, nullptr));
            CHECK(g_log.kind == stub::kFwd && g_log.head == rlk::kHeadLogp && g_log.dtype == d);
            CHECK(g_log.fwd.N == N && g_log.fwd.V == V && g_log.fwd.k == k);
            CHECK(g_log.fwd.v0 == 0 && g_log.fwd.vtotal == V && g_log.fwd.part == nullptr);
            CHECK(g_log.fwd.mx.st == ld && g_log.fwd.mx.sb == 0 && g_log.fwd.mx.T == N);
            // cap forms: none, fixed (2 c log2 e <= 120), online above or below 2^-16
            const int want = cap == 0.0f ? rlk::kCapNone
                             : (2.0 * cap * 1.4426950408889634 <= 120.0 &&
                                2.0 * cap * 1.4426950408889634 >= 1.0 / 65536)
                                 ? rlk::kCapFixed
                                 : rlk::kCapOnline;
            CHECK(g_log.cap_x == want);
            if (want == rlk::kCapFixed)
                CHECK(std::fabs(g_log.fwd.ix * 2.0 * cap * 1.4426950408889634 - 1.0) < 1e-6);
            if (cap != 0.0f) CHECK(std::fabs(g_log.fwd.kx * cap / -2.8853900817779268 - 1.0) < 1e-6);
            // ld * es is a multiple of 16 for fp32 (4160) and 16-bit (2080)
            CHECK(g_log.aligned);
            EXPECT_LAUNCH(0, rlk_logp_bwd(x, d, N, V, ld, t, k, cap, st, g, gx, nullptr));
            CHECK(g_log.kind == stub::kBwd && g_log.bwd.mg.st == V && g_log.bwd.k == k);
            if (want == rlk::kCapFixed)
                CHECK(std::fabs(g_log.bwd.ix * 2.0 * cap * 1.4426950408889634 - 1.0) < 1e-6);
        }
        // the row stride decides the alignment: ld = 1033 is not 16-byte aligned
        EXPECT_LAUNCH(0, rlk_logp_fwd(x, d, N, V, 1033, t, k, 0.0f, out, st, nullptr));
        CHECK(!g_log.aligned);
        EXPECT_EMPTY(rlk_logp_fwd(nullptr, d, 0, V, V, nullptr, k, 0.0f, nullptr, nullptr, nullptr));
        EXPECT_EMPTY(rlk_logp_bwd(nullptr, d, 0, V, V, nullptr, k, 0.0f, nullptr, nullptr, nullptr,
                                  nullptr));
        EXPECT_FAIL(RLK_ERR_SHAPE, rlk_logp_fwd(x, d, N, 0, ld, t, k, 0.0f, out, st, nullptr));
        EXPECT_FAIL(RLK_ERR_SHAPE, rlk_logp_fwd(x, d, -1, V, ld, t, k, 0.0f, out, st, nullptr));
        EXPECT_FAIL(RLK_ERR_SHAPE, rlk_logp_fwd(x, d, N, V, V - 1, t, k, 0.0f, out, st, nullptr));
        EXPECT_FAIL(RLK_ERR_SHAPE,
                    rlk_logp_fwd(x, d, N, int64_t(1) << 31, int64_t(1) << 31, t, k, 0.0f, out, st,
                                 nullptr));
        EXPECT_FAIL(RLK_ERR_SHAPE, rlk_logp_fwd(x, d, N, V, ld, t, 0, 0.0f, out, st, nullptr));
        EXPECT_FAIL(RLK_ERR_SHAPE,
                    rlk_logp_fwd(x, d, N, V, ld, t, RLK_MAX_TOPK + 1, 0.0f, out, st, nullptr));
        // N * ld elements overflow 64-bit byte offsets
        EXPECT_FAIL(RLK_ERR_SHAPE, rlk_logp_fwd(x, d, int64_t(1) << 40, V, int64_t(1) << 30, t, 1,
                                                0.0f, out, st, nullptr));
        EXPECT_FAIL(RLK_ERR_SHAPE, rlk_logp_bwd(x, d, INT64_MAX / 2, V, V, t, 1, 0.0f, st, g, gx,
                                                nullptr));
        for (float bad : {kNaN, kInf, -kInf, -30.0f})
            EXPECT_FAIL(RLK_ERR_ARG, rlk_logp_fwd(x, d, N, V, ld, t, k, bad, out, st, nullptr));
        EXPECT_FAIL(RLK_ERR_ARG, rlk_logp_fwd(x, d, N, V, ld, nullptr, k, 0.0f, out, st, nullptr));
        EXPECT_FAIL(RLK_ERR_ARG, rlk_logp_fwd(x, d, N, V, ld, t, k, 0.0f, out, nullptr, nullptr));
        EXPECT_FAIL(RLK_ERR_ARG,
                    rlk_logp_bwd(x, d, N, V, ld, t, k, 0.0f, st, nullptr, gx, nullptr));
    }
    EXPECT_FAIL(RLK_ERR_DTYPE, rlk_logp_fwd(nullptr, static_cast<rlk_dtype>(-1), 1, 1, 1, nullptr,
                                            1, 0.0f, nullptr, nullptr, nullptr));
}

static void test_devices() {
    const int64_t N = 8, V = 64;
    void* x0 = stub::fake_alloc(N * V * 2, 0);
    void* x1 = stub::fake_alloc(N * V * 2, 1);
    void* h1 = stub::fake_alloc(64, 1);
    float* H1 = static_cast<float*>(stub::fake_alloc(N * 4, 1));
    void* s1 = stub::fake_alloc(N * 32, 1);
    void* hostmem = stub::fake_alloc(N * V * 2, 0, /*host=*/true);
    char unregistered[64];
    (void)h1;
    // tensors on device 1 while device 0 is current: the launch runs on 1
    // and device 0 is current again afterwards
    stub::set_current_device(0);
    EXPECT_LAUNCH(1, rlk_entropy_fwd(x1, RLK_BF16, N, V, V, 0.0f, H1, s1, nullptr));
    CHECK(g_log.set_device_calls == 2);
    // already current: no switch
    stub::set_current_device(1);
    EXPECT_LAUNCH(1, rlk_entropy_fwd(x1, RLK_BF16, N, V, V, 0.0f, H1, s1, nullptr));
    CHECK(g_log.set_device_calls == 0);
    stub::set_current_device(0);
    // mixed devices, host memory, memory HIP does not know
    EXPECT_FAIL(RLK_ERR_DEVICE, rlk_entropy_fwd(x0, RLK_BF16, N, V, V, 0.0f, H1, s1, nullptr));
    EXPECT_FAIL(RLK_ERR_DEVICE,
                rlk_entropy_fwd(hostmem, RLK_BF16, N, V, V, 0.0f, H1, s1, nullptr));
    EXPECT_FAIL(RLK_ERR_DEVICE,
                rlk_entropy_fwd(unregistered, RLK_BF16, N, V, V, 0.0f, H1, s1, nullptr));
    CHECK(stub::current_device() == 0);
}

static void test_entropy_kl() {
    const int64_t N = 19, V = 4097;
    for (rlk_dtype d : {RLK_F32, RLK_BF16, RLK_F16}) {
        void* a = stub::fake_alloc(N * V * es(d));
        void* b = stub::fake_alloc(N * V * es(d));
        float* o = static_cast<float*>(stub::fake_alloc(N * 4));
        float* o2 = static_cast<float*>(stub::fake_alloc(N * 4));
        void* st = stub::fake_alloc(rlk_stats_bytes(RLK_HEAD_KL, N, V));
        void* st2 = stub::fake_alloc(rlk_stats_bytes(RLK_HEAD_KL, N, V));
        float* g = static_cast<float*>(stub::fake_alloc(N * 4));
        void* gx = stub::fake_alloc(N * V * es(d));
        EXPECT_LAUNCH(0, rlk_entropy_fwd(a, d, N, V, V, 30.0f, o, st, nullptr));
        CHECK(g_log.head == rlk::kHeadEntropy && g_log.cap_x == rlk::kCapFixed);
        CHECK(!g_log.aligned || (V * es(d)) % 16 == 0);
        EXPECT_LAUNCH(0, rlk_entropy_bwd(a, d, N, V, V, 30.0f, st, g, gx, nullptr));
        for (rlk_kl_dir dir : {RLK_KL_REVERSE, RLK_KL_FORWARD}) {
            EXPECT_LAUNCH(0, rlk_kl_fwd(a, b, d, N, V, V, V, dir, 0.0f, 45.0f, o, st, nullptr));
            CHECK(g_log.head == (dir == RLK_KL_REVERSE ? rlk::kHeadKLReverse
                                                       : rlk::kHeadKLForward));
            CHECK(g_log.cap_x == rlk::kCapNone && g_log.cap_y == rlk::kCapOnline);
            CHECK(g_log.fwd.x == a && g_log.fwd.y == b);
            EXPECT_LAUNCH(0, rlk_kl_bwd(a, b, d, N, V, V, V, dir, 0.0f, 45.0f, st, g, gx, nullptr));
            CHECK(g_log.bwd.x == a && g_log.bwd.y == b && g_log.bwd.swap == 0);
            // the reference gradient: operands, caps and record sides exchanged,
            // the other direction's kernel
            EXPECT_LAUNCH(0, rlk_kl_bwd_ref(a, b, d, N, V, V, V, dir, 0.0f, 45.0f, st, g, gx,
                                            nullptr));
            CHECK(g_log.bwd.x == b && g_log.bwd.y == a && g_log.bwd.swap == 1);
            CHECK(g_log.cap_x == rlk::kCapOnline && g_log.cap_y == rlk::kCapNone);
            CHECK(g_log.head == (dir == RLK_KL_REVERSE ? rlk::kHeadKLForward
                                                       : rlk::kHeadKLReverse));
            EXPECT_FAIL(RLK_ERR_ARG, rlk_kl_fwd(a, b, d, N, V, V, V, dir, 0.0f, kNaN, o, st,
                                                nullptr));
        }
        EXPECT_LAUNCH(0, rlk_kl_fwd_both(a, b, d, N, V, V, V, 0.0f, 0.0f, o, st, o2, st2, nullptr));
        CHECK(g_log.head == rlk::kHeadKLBoth && g_log.fwd.out2 == o2 && g_log.fwd.stats2 == st2);
        EXPECT_FAIL(RLK_ERR_ARG,
                    rlk_kl_fwd_both(a, b, d, N, V, V, V, 0.0f, 0.0f, o, st, nullptr, st2, nullptr));
        EXPECT_FAIL(RLK_ERR_ARG, rlk_kl_fwd(a, b, d, N, V, V, V, static_cast<rlk_kl_dir>(2), 0.0f,
                                            0.0f, o, st, nullptr));
        EXPECT_FAIL(RLK_ERR_SHAPE,
                    rlk_kl_fwd(a, b, d, N, V, V, V - 1, RLK_KL_REVERSE, 0.0f, 0.0f, o, st, nullptr));
        EXPECT_FAIL(RLK_ERR_ARG, rlk_kl_bwd(a, nullptr, d, N, V, V, V, RLK_KL_REVERSE, 0.0f, 0.0f,
                                            st, g, gx, nullptr));
        EXPECT_EMPTY(rlk_kl_bwd_ref(nullptr, nullptr, d, 0, V, V, V, RLK_KL_FORWARD, 0.0f, 0.0f,
                                    nullptr, nullptr, nullptr, nullptr));
    }
}

static void test_strided() {
    // logits[:, :-1] of a contiguous [B, T + 1, V] tensor, read in place, and
    // its gradient written into grad[:, :-1] of a buffer of the same shape
    const int64_t B = 3, T = 5, V = 1000, N = B * T;
    const rlk_rows view{T, (T + 1) * V, V};
    for (rlk_dtype d : {RLK_F32, RLK_BF16}) {
        void* x = stub::fake_alloc(B * (T + 1) * V * es(d));
        void* gx = stub::fake_alloc(B * (T + 1) * V * es(d));
        int64_t* t = static_cast<int64_t*>(stub::fake_alloc(N * 8));
        float* o = static_cast<float*>(stub::fake_alloc(N * 4));
        float* g = static_cast<float*>(stub::fake_alloc(N * 4));
        void* st = stub::fake_alloc(rlk_stats_bytes(RLK_HEAD_LOGP, N, V));
        EXPECT_LAUNCH(0, rlk_logp_fwd_strided(x, d, N, V, &view, t, 1, 0.0f, o, st, nullptr));
        CHECK(g_log.fwd.mx.T == T && g_log.fwd.mx.sb == (T + 1) * V && g_log.fwd.mx.st == V);
        EXPECT_LAUNCH(0, rlk_logp_bwd_strided(x, d, N, V, &view, t, 1, 0.0f, st, g, gx, &view,
                                              nullptr));
        EXPECT_LAUNCH(0, rlk_entropy_bwd_strided(x, d, N, V, &view, 0.0f, st, g, gx, &view,
                                                 nullptr));
        // time-major rows (sb < st) are a valid non-overlapping output layout
        const rlk_rows tm{T, V, B * V};
        EXPECT_LAUNCH(0, rlk_entropy_bwd_strided(x, d, N, V, &tm, 0.0f, st, g, gx, &tm, nullptr));
        // a broadcast input (every row the same) may be read, never written
        const rlk_rows bcast{T, 0, 0};
        EXPECT_LAUNCH(0, rlk_entropy_fwd_strided(x, d, N, V, &bcast, 0.0f, o, st, nullptr));
        EXPECT_FAIL(RLK_ERR_SHAPE, rlk_entropy_bwd_strided(x, d, N, V, &view, 0.0f, st, g, gx,
                                                           &bcast, nullptr));
        const rlk_rows overlap{T, (T + 1) * V, V - 1};
        EXPECT_FAIL(RLK_ERR_SHAPE, rlk_logp_bwd_strided(x, d, N, V, &view, t, 1, 0.0f, st, g, gx,
                                                        &overlap, nullptr));
        const rlk_rows zero_t{0, V, V}, neg{T, -1, V};
        EXPECT_FAIL(RLK_ERR_SHAPE,
                    rlk_logp_fwd_strided(x, d, N, V, &zero_t, t, 1, 0.0f, o, st, nullptr));
        EXPECT_FAIL(RLK_ERR_SHAPE, rlk_logp_fwd_strided(x, d, N, V, &neg, t, 1, 0.0f, o, st, nullptr));
        EXPECT_FAIL(RLK_ERR_ARG, rlk_logp_fwd_strided(x, d, N, V, nullptr, t, 1, 0.0f, o, st,
                                                      nullptr));
        // the last row's offset overflows 64-bit byte offsets
        const rlk_rows huge{1, INT64_MAX / 4, V};
        EXPECT_FAIL(RLK_ERR_SHAPE, rlk_logp_fwd_strided(x, d, 4, V, &huge, t, 1, 0.0f, o, st,
                                                        nullptr));
        const rlk_rows huge_t{INT64_MAX, 0, INT64_MAX / 4};
        EXPECT_FAIL(RLK_ERR_SHAPE, rlk_entropy_fwd_strided(x, d, 3, V, &huge_t, 0.0f, o, st,
                                                           nullptr));
        // KL views: both inputs strided, the gradient into a strided buffer
        EXPECT_LAUNCH(0, rlk_kl_fwd_strided(x, x, d, N, V, &view, &view, RLK_KL_FORWARD, 0.0f,
                                            0.0f, o, st, nullptr));
        EXPECT_LAUNCH(0, rlk_kl_bwd_ref_strided(x, x, d, N, V, &view, &view, RLK_KL_FORWARD, 0.0f,
                                                0.0f, st, g, gx, &view, nullptr));
    }
}

static void test_shards() {
    const int64_t N = 11, Vt = 3001, k = 3;
    const int64_t bounds[] = {0, 1000, 1000, 2500, Vt};  // an empty shard
    const int64_t P = 4;
    int64_t* t = static_cast<int64_t*>(stub::fake_alloc(N * k * 8));
    void* part = stub::fake_alloc(P * N * 32);
    float* tv = static_cast<float*>(stub::fake_alloc(P * N * k * 4));
    float* o = static_cast<float*>(stub::fake_alloc(N * k * 4));
    void* st = stub::fake_alloc(N * 32);
    float* g = static_cast<float*>(stub::fake_alloc(N * k * 4));
    for (int64_t s = 0; s < P; ++s) {
        const int64_t v0 = bounds[s], Vs = bounds[s + 1] - bounds[s];
        void* x = Vs ? stub::fake_alloc(N * Vs * 2) : nullptr;
        void* gx = Vs ? stub::fake_alloc(N * Vs * 2) : nullptr;
        char* ps = static_cast<char*>(part) + s * N * 32;
        float* tvs = tv + s * N * k;
        EXPECT_LAUNCH(0, rlk_logp_fwd_partial(x, RLK_BF16, N, Vs, Vs ? Vs : 1, v0, Vt, t, k, 20.0f,
                                              ps, tvs, nullptr));
        CHECK(g_log.fwd.v0 == v0 && g_log.fwd.vtotal == Vt && g_log.fwd.V == Vs);
        CHECK(g_log.fwd.part == ps && g_log.fwd.tvals == tvs);
        EXPECT_LAUNCH(0, rlk_entropy_fwd_partial(x, RLK_BF16, N, Vs, Vs ? Vs : 1, 0.0f, ps,
                                                 nullptr));
        if (Vs) {
            EXPECT_LAUNCH(0, rlk_logp_bwd_shard(x, RLK_BF16, N, Vs, Vs, v0, Vt, t, k, 20.0f, st, g,
                                                gx, nullptr));
            CHECK(g_log.bwd.v0 == v0 && g_log.bwd.vtotal == Vt);
        } else {
            EXPECT_EMPTY(rlk_logp_bwd_shard(nullptr, RLK_BF16, N, 0, 1, v0, Vt, t, k, 20.0f, st, g,
                                            nullptr, nullptr));
        }
    }
    EXPECT_LAUNCH(0, rlk_combine(RLK_HEAD_LOGP, RLK_KL_REVERSE, P, bounds, N, part, t, k, tv,
                                 20.0f, o, st, nullptr));
    CHECK(g_log.kind == stub::kCombine && g_log.comb.P == P && g_log.comb.vtotal == Vt);
    for (int64_t s = 0; s <= P; ++s) CHECK(g_log.comb.bounds[s] == bounds[s]);
    EXPECT_LAUNCH(0, rlk_combine(RLK_HEAD_KL, RLK_KL_FORWARD, P, bounds, N, part, nullptr, 1,
                                 nullptr, 0.0f, o, st, nullptr));
    CHECK(g_log.head == rlk::kHeadKLForward);
    // shard and combine bounds
    void* x = stub::fake_alloc(N * 1000 * 2);
    EXPECT_FAIL(RLK_ERR_SHAPE, rlk_logp_fwd_partial(x, RLK_BF16, N, 1000, 1000, -1, Vt, t, k, 0.0f,
                                                    part, tv, nullptr));
    EXPECT_FAIL(RLK_ERR_SHAPE, rlk_logp_fwd_partial(x, RLK_BF16, N, 1000, 1000, 2002, Vt, t, k,
                                                    0.0f, part, tv, nullptr));
    EXPECT_FAIL(RLK_ERR_SHAPE, rlk_logp_fwd_partial(x, RLK_BF16, N, 1000, 999, 0, Vt, t, k, 0.0f,
                                                    part, tv, nullptr));
    EXPECT_FAIL(RLK_ERR_SHAPE, rlk_entropy_fwd_partial(x, RLK_BF16, N, -3, 1000, 0.0f, part,
                                                       nullptr));
    EXPECT_FAIL(RLK_ERR_SHAPE, rlk_logp_bwd_shard(x, RLK_BF16, INT64_MAX / 1000, 1000, 1000, 0, Vt,
                                                  t, 1, 0.0f, st, g, x, nullptr));
    const int64_t bad0[] = {1, 10}, dec[] = {0, 10, 5}, wide[] = {0, int64_t(1) << 31};
    EXPECT_FAIL(RLK_ERR_SHAPE, rlk_combine(RLK_HEAD_ENTROPY, RLK_KL_REVERSE, 0, bounds, N, part,
                                           nullptr, 1, nullptr, 0.0f, o, st, nullptr));
    EXPECT_FAIL(RLK_ERR_SHAPE, rlk_combine(RLK_HEAD_ENTROPY, RLK_KL_REVERSE, RLK_MAX_SHARDS + 1,
                                           bounds, N, part, nullptr, 1, nullptr, 0.0f, o, st,
                                           nullptr));
    EXPECT_FAIL(RLK_ERR_SHAPE, rlk_combine(RLK_HEAD_ENTROPY, RLK_KL_REVERSE, 1, bad0, N, part,
                                           nullptr, 1, nullptr, 0.0f, o, st, nullptr));
    EXPECT_FAIL(RLK_ERR_SHAPE, rlk_combine(RLK_HEAD_ENTROPY, RLK_KL_REVERSE, 2, dec, N, part,
                                           nullptr, 1, nullptr, 0.0f, o, st, nullptr));
    EXPECT_FAIL(RLK_ERR_SHAPE, rlk_combine(RLK_HEAD_ENTROPY, RLK_KL_REVERSE, 1, wide, N, part,
                                           nullptr, 1, nullptr, 0.0f, o, st, nullptr));
    EXPECT_FAIL(RLK_ERR_ARG, rlk_combine(RLK_HEAD_ENTROPY, RLK_KL_REVERSE, 1, nullptr, N, part,
                                         nullptr, 1, nullptr, 0.0f, o, st, nullptr));
    EXPECT_FAIL(RLK_ERR_ARG, rlk_combine(static_cast<rlk_head>(5), RLK_KL_REVERSE, 1, bounds, N,
                                         part, nullptr, 1, nullptr, 0.0f, o, st, nullptr));
    EXPECT_FAIL(RLK_ERR_ARG, rlk_combine(RLK_HEAD_LOGP, RLK_KL_REVERSE, P, bounds, N, part,
                                         nullptr, k, tv, 0.0f, o, st, nullptr));
    EXPECT_FAIL(RLK_ERR_SHAPE, rlk_combine(RLK_HEAD_LOGP, RLK_KL_REVERSE, P, bounds,
                                           INT64_MAX / 2, part, t, k, tv, 0.0f, o, st, nullptr));
}

int main() {
    test_status_and_sizes();
    test_softcap();
    test_logp();
    test_devices();
    test_entropy_kl();
    test_strided();
    test_shards();
    std::printf("host ABI driver: %d checks, %d failed\n", g_checks, g_failed);
    return g_failed ? 1 : 0;
}
