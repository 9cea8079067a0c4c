// rlk_launch.h -- kernel parameter blocks and the internal launchers that the
// C ABI (rlk_api.cpp) calls after it has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlk {

// Heads of the fused row kernels.
// kHeadKLBoth: forward only, both KL directions from one read of the pair.
enum Head : int {
    kHeadLogp = 0,
    kHeadEntropy = 1,
    kHeadKLReverse = 2,
    kHeadKLForward = 3,
    kHeadKLBoth = 4
};

// Softcap modes of one logits tensor (host-chosen from the cap c, the same
// for a forward call, its backward and the shard combine):
//   kCapNone   no cap; statistic input a = x, scale log2(e);
//   kCapOnline a = r = 1 / (1 + 2^(k x)), scale 2 c log2(e), running max;
//   kCapFixed  a = t = (y - c) log2(e) = -1 / (1/sc + 2^(-k x)/sc) in one FMA
//              and a reciprocal, scale 1, reference 0 (no running max).
// t of the fixed mode lies in [-2 c log2(e), 0], so for caps with
// 2 c log2(e) <= kCapFixedMaxScale every 2^t is a normal float and the sums
// need no rescaling; larger caps take the online mode.  So do caps with
// 2 c log2(e) < kCapFixedMinScale: the fixed form's backward scales its slope
// by 1 / (2 c log2(e))^2, which must stay far from overflow.
enum CapMode : int { kCapNone = 0, kCapOnline = 1, kCapFixed = 2 };
// Device-side forms of kCapFixed in the logprobs / entropy forward (never
// passed in from the host): the statistic input is t + sc/2, odd in x, with
// the reference at -sc/2 instead of 0 -- computed as sc/2 + t(|x|) with the
// sign of x (kCapFixedOdd), or read from an LDS table of sc/2 + t(|x|) over
// the 2^15 magnitudes of bf16 / fp16 bit patterns (fwd1_tab_kernel).  The
// two give the same bits for the same value, whatever its dtype.
enum CapFormMode : int { kCapTableB = 3, kCapTableH = 4, kCapFixedOdd = 5 };
constexpr int kTabSize = 1 << 15;  // 16-bit magnitudes
constexpr int kTabRows = 4;        // rows side by side in one table workgroup
constexpr int kTabGrid = 256;      // table workgroups at most: one per CU
#ifndef RLK_CAP_TABLE
#define RLK_CAP_TABLE 1
#endif
constexpr bool kUseCapTable = RLK_CAP_TABLE != 0;
// Row widths from which the fixed cap's logprobs / entropy forward takes the
// odd form (measured on bf16 rows: the table kernel walks kTabRows rows in
// lockstep per CU, which pays only for long rows; entropy spends more VALU
// per logit than logprobs and gains from shorter rows on).
constexpr int64_t kOddMinColsEntropy = 65536;
constexpr int64_t kOddMinColsLogp = 196608;
inline int64_t odd_form_min_cols(int head) {
    return head == kHeadEntropy ? kOddMinColsEntropy : kOddMinColsLogp;
}
constexpr float kCapFixedMaxScale = 120.0f;
constexpr float kCapFixedMinScale = 1.0f / 65536.0f;

// Launch shape of the forward row kernels: one workgroup per row (grid-stride
// over rows), each lane consuming groups of U chunks of 8 elements.  These
// constants fix the reduction tree, so they are the same for every N (the
// batch-invariance guarantee).  The backward is elementwise given the row
// record, so its shape is free; it is tuned for the read+write stream.
// (Overridable at compile time for launch-shape sweeps.)
#ifndef RLK_BLOCK
#define RLK_BLOCK 256
#endif
#ifndef RLK_UNROLL1
#define RLK_UNROLL1 4
#endif
#ifndef RLK_UNROLL_KL
#define RLK_UNROLL_KL 2
#endif
#ifndef RLK_BWD_BLOCK_TOPK
#define RLK_BWD_BLOCK_TOPK 512
#endif
#ifndef RLK_BWD_UNROLL_TOPK
#define RLK_BWD_UNROLL_TOPK 2
#endif
// Backward in one-shot pieces (every workgroup handles BLOCK chunks of one
// row and exits) for every head except logprobs with more than a few slots
// (wide pieces below; beyond 256 slots the row kernel takes the _TOPK shape).
#ifndef RLK_BWD_PIECE_BLOCK
#define RLK_BWD_PIECE_BLOCK 256
#endif
// Chunks per lane of the wide top-k pieces (logprobs, 4 < k <= 256).
#ifndef RLK_BWD_WIDE_UNROLL
#define RLK_BWD_WIDE_UNROLL 4
#endif
constexpr int kBwdWideUnroll = RLK_BWD_WIDE_UNROLL;
#ifndef RLK_FWD_PIPE
#define RLK_FWD_PIPE 1
#endif
#ifndef RLK_BWD_PIPE
#define RLK_BWD_PIPE 0
#endif
constexpr bool kFwdPipe = RLK_FWD_PIPE;
constexpr bool kBwdPipe = RLK_BWD_PIPE;
constexpr int kBwdPieceBlock = RLK_BWD_PIECE_BLOCK;
// Chunks per lane of a piece.  One (4 KB of bf16 per workgroup) is the
// fastest for every head, the VALU-heavy capped ones included: two or four
// amortise the per-piece setup but lengthen each workgroup's life.
#ifndef RLK_BWD_PIECE_UNROLL
#define RLK_BWD_PIECE_UNROLL 1
#endif
constexpr int kBwdPieceUnroll = RLK_BWD_PIECE_UNROLL;
// Minimum waves per SIMD requested from the register allocator (0: none).
#ifndef RLK_WAVES_PER_EU
#define RLK_WAVES_PER_EU 0
#endif
#if RLK_WAVES_PER_EU > 0
#define RLK_OCCUPANCY __attribute__((amdgpu_waves_per_eu(RLK_WAVES_PER_EU)))
#else
#define RLK_OCCUPANCY
#endif
constexpr int kBlock = RLK_BLOCK;
constexpr int kUnroll1 = RLK_UNROLL1;    // forward, single-tensor heads
constexpr int kUnrollKL = RLK_UNROLL_KL;  // forward, KL (two tensors per group)
constexpr int kBwdBlockTopk = RLK_BWD_BLOCK_TOPK;  // logprobs backward with wide top-k
constexpr int kBwdUnrollTopk = RLK_BWD_UNROLL_TOPK;
// Resident one-shot pieces per CU.  A piece issues all its loads at once, so
// the pieces resident on a CU set its bytes in flight, and past a point more
// of them only add DRAM conflicts.  Measured on the read+write stream
// (bf16 / fp32 [.., 151936] logprobs and entropy, KL [.., 75968]; 256 lanes x
// 16 bytes of each operand per piece): moving 8 KB per piece (16-bit
// logprobs, entropy) is best with all the 8 the registers allow (6: +10%);
// 12 KB (16-bit KL) with 6 (-2 to -3%; 7: +1%); 16 KB (fp32 logprobs,
// entropy) with 4 (-10%); 24 KB (fp32 KL) with 3 (-5 to -7%).  The limit is
// set by dynamic LDS that the kernel does not use.
constexpr int kLdsPerCu = 160 * 1024;  // LDS per CU
constexpr int kLdsGranule = 512;       // its allocation unit
inline unsigned lds_for_wgs_per_cu(int w) {
    // the least multiple of the granule of which w + 1 do not fit
    return w >= 8 ? 0u
                  : static_cast<unsigned>((kLdsPerCu / (w + 1) / kLdsGranule + 1) * kLdsGranule);
}
template <int ESIZE, bool KL>
constexpr int piece_wgs_per_cu() {
    return ESIZE == 4 ? (KL ? 3 : 4) : (KL ? 6 : 8);
}
// Wide top-k pieces (16 KB of 16-bit logits read and written, 32 KB of fp32):
// the capped 16-bit backward needs every resident wave for its arithmetic
// (top-256 + cap 20, bf16 [2048, 262144]: 5 per CU +9%); fp32 ones are best
// with 2 per CU (k = 64, fp32 [2048, 151936]: -11%; top-256 + cap 20, fp32
// [1024, 262144]: -5%).  (Their static LDS only adds to the dynamic part.)
template <int ESIZE>
constexpr int wide_wgs_per_cu() {
    return ESIZE == 4 ? 2 : 8;
}

// Few rows: a narrow shape whose rows are also split into column segments,
// so that there are enough workgroups to cover the chip.
constexpr int kBwdBlockSmall = 256;
constexpr int kBwdUnrollSmall = 1;
constexpr int64_t kBwdSmallRows = 512;      // below this many rows
constexpr int64_t kBwdTargetItems = 2048;   // aim for this many (row, segment) items
// A call whose operands (N x V logits, two tensors for KL) are at most this
// many bytes reads them with ordinary loads: the previous kernel usually left
// them in the 256 MB Infinity Cache, where non-temporal loads measured slower
// (logprobs fp32 [64, 32000], fwd+bwd: 12.8 -> 10.2 us); larger operands
// stream with non-temporal loads (bf16 [8192, 151936]: forward 0.366 ms
// against 0.406 ms with ordinary loads).
constexpr int64_t kCachedReadBytes = int64_t(256) << 20;
inline bool stream_reads(int64_t N, int64_t V, int64_t esize, int64_t tensors) {
    const int64_t row = V * esize * tensors;
    return row > 0 && N > kCachedReadBytes / row;
}
// Top-k slots per lane whose target loads and gathers a logprobs forward
// issues together.
constexpr int kTopkBatch = 4;
// Largest grid in workgroups: a dispatch counts work-items in 32 bits, and
// blocks are at most 1024 threads.
constexpr int kMaxGrid = (1 << 22) - 1;

// Row i of a (possibly two-stride) view starts at element
// (i / T) * sb + (i % T) * st: a [B, T, V] view with strides (sb, st, 1).
// A plain [N, V] matrix with row stride ld is {T = N, sb = 0, st = ld}.
struct RowMap {
    int64_t T, sb, st;
    __host__ __device__ int64_t offset(int64_t i) const {
        if (i < T) return i * st;  // first (or only) batch: no division
        if (((i | T) >> 32) == 0) {  // 32-bit division when both fit
            const int64_t b = static_cast<uint32_t>(i) / static_cast<uint32_t>(T);
            return b * sb + (i - b * T) * st;
        }
        const int64_t b = i / T;
        return b * sb + (i - b * T) * st;
    }
};

struct FwdParams {
    const void* x;   // logits (KL: policy)
    const void* y;   // KL reference (else unused)
    int64_t N, V;
    RowMap mx, my;   // row layouts of x and y
    const int64_t* targets;  // logp: [N, k]
    int64_t k;
    float kx, ky;    // softcap multiplier -2 log2(e) / c (unused when off)
    float scx, scy;  // statistic scale: log2(e), 2 c log2(e) (online cap) or 1 (fixed cap)
    float ix, iy;    // fixed cap: 1 / (2 c log2(e)) (else unused)
    float* out;      // logp [N, k], entropy [N] or KL [N]
    void* stats;     // RowStats [N]
    // Vocabulary shard: the columns of x are [v0, v0 + V) of a row of width
    // vtotal (plain call: v0 = 0, vtotal = V).  With `part` set, the kernel
    // writes the shard's PartialRec [N] (and, for logprobs, the statistic
    // input of every target it owns into tvals [N, k]) instead of the heads.
    int64_t v0, vtotal;
    void* part;
    float* tvals;
    // kHeadKLBoth: the forward-KL output and row record (out / stats hold
    // the reverse KL).
    float* out2;
    void* stats2;
};

struct BwdParams {
    const void* x;
    const void* y;
    int64_t N, V;
    RowMap mx, my, mg;  // row layouts of x, y and of the gradient output
    const int64_t* targets;
    int64_t k;
    float kx, ky, scx, scy, ix, iy;
    const void* stats;
    const float* g;  // upstream gradient: [N, k] (logp) or [N]
    void* gx;        // gradient w.r.t. x, [N, V] contiguous, logits dtype
    int64_t split;   // column segments per row (one workgroup each), >= 1
    int64_t v0, vtotal;  // vocabulary shard of x (plain call: 0, V)
    int swap;            // KL: x is the record's b side (reference gradient)
    int wt;              // full pieces store with the write-through policy
};

// Gradients at least this large cannot stay in the 256 MB Infinity Cache:
// their full pieces are stored write-through (sc1 nt), which streams ~3%
// faster; smaller ones keep plain streaming stores, whose lines stay cached
// for the caller (a 16 MB gradient's backward took 9.1 us write-through and
// 5.1 us without).
constexpr uint64_t kWriteThroughBytes = uint64_t(256) << 20;

constexpr int kMaxShards = 64;

struct CombineParams {
    int P;
    int64_t N, k, vtotal;
    int64_t bounds[kMaxShards + 1];  // shard s owns columns [bounds[s], bounds[s+1])
    const void* part;                // PartialRec [P, N]
    const int64_t* targets;          // logp: [N, k]
    const float* tvals;              // logp: [P, N, k]
    float sc;                        // statistic scale of the logits (as FwdParams::scx)
    float* out;
    void* stats;
};

hipError_t launch_combine(int head, const CombineParams& q, hipStream_t stream);

// Per-dtype row-kernel launchers (rlk_fwd_<dtype>.hip, rlk_bwd_<dtype>.hip).
// cap_x / cap_y: CapMode of each tensor.
hipError_t launch_fwd_f32(int head, int cap_x, int cap_y, bool aligned, const FwdParams& p,
                          hipStream_t stream);
hipError_t launch_fwd_bf16(int head, int cap_x, int cap_y, bool aligned, const FwdParams& p,
                           hipStream_t stream);
hipError_t launch_fwd_f16(int head, int cap_x, int cap_y, bool aligned, const FwdParams& p,
                          hipStream_t stream);
hipError_t launch_bwd_f32(int head, int cap_x, int cap_y, bool aligned, const BwdParams& p,
                          hipStream_t stream);
hipError_t launch_bwd_bf16(int head, int cap_x, int cap_y, bool aligned, const BwdParams& p,
                           hipStream_t stream);
hipError_t launch_bwd_f16(int head, int cap_x, int cap_y, bool aligned, const BwdParams& p,
                          hipStream_t stream);

// dtype codes follow rlk_dtype (0 fp32, 1 bf16, 2 fp16).
inline hipError_t launch_fwd(int head, int dtype, int cap_x, int cap_y, bool aligned,
                             const FwdParams& p, hipStream_t stream) {
    if (dtype == 0) return launch_fwd_f32(head, cap_x, cap_y, aligned, p, stream);
    if (dtype == 1) return launch_fwd_bf16(head, cap_x, cap_y, aligned, p, stream);
    return launch_fwd_f16(head, cap_x, cap_y, aligned, p, stream);
}
inline hipError_t launch_bwd(int head, int dtype, int cap_x, int cap_y, bool aligned,
                             const BwdParams& p, hipStream_t stream) {
    if (dtype == 0) return launch_bwd_f32(head, cap_x, cap_y, aligned, p, stream);
    if (dtype == 1) return launch_bwd_bf16(head, cap_x, cap_y, aligned, p, stream);
    return launch_bwd_f16(head, cap_x, cap_y, aligned, p, stream);
}
hipError_t launch_softcap_fwd(const void* x, int x_dtype, void* y, int y_dtype, int64_t n,
                              float cap, bool aligned, hipStream_t stream);
hipError_t launch_softcap_bwd(const void* x, int x_dtype, const float* gy, void* gx, int64_t n,
                              float cap, bool aligned, hipStream_t stream);

inline int row_grid(int64_t N) { return static_cast<int>(N < kMaxGrid ? N : kMaxGrid); }

}  // namespace rlk
