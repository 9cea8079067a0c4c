// rlk_bwd_kernels.h -- fused zero-workspace backward kernels.
//
// "perf(logp): fused zero-workspace backward for the generic CUDA fused logp"
// (RL-Kernel pull request 495), Summary: the gradient g (onehot - softmax) is
// written straight in the logits dtype with no [N, V] fp32 temporary; rows
// whose targets are all outside [0, V) get an exactly zero gradient (Behavior
// changes).  Here the softmax is not recomputed from two more passes: the
// forward saved (max log2 e, log2 S) per row, so each logit is read once and
// each gradient written once, and p takes its exponent from the very same
// FMA as the forward.
//
// Heads (all times the upstream g of the row and, with a softcap, the
// derivative 1 - tanh^2 of "Final Logit Softcap", Summary):
//   logprobs: h_v - p_v G, with the top-k one-hot sums h added in fp32 before
//             the single cast ("Add Triton kernels for vocab-parallel
//             logprobs, entropy and KL", Changes);
//   entropy:  -p_v (log p_v + H);
//   reverse KL(P||R): p_v (log p_v - log q_v - D);
//   forward KL(R||P): p_v - q_v;
// and w.r.t. the reference, with the operands and the record's sides
// exchanged (KL(P||R) is the forward KL of the pair policy R, reference P):
//   reverse KL(P||R): q_v - p_v;  forward KL(R||P): q_v (log q_v - log p_v - D).
#pragma once

#include "rlk_device.h"
#include "rlk_launch.h"

namespace rlk {

// Lanes that sum the upstream gradient of the k slots (fixed tree).
constexpr int kGLanes = 256;
// Longest per-piece slot list that bwd_wide_kernel searches entry by entry;
// a longer one is sorted first.
constexpr int kWideScanMax = 16;

// Row modes.
enum : int { kModeNormal = 0, kModeZero = 1, kModeNaN = 2, kModeMismatch = 3 };

// Which flags a record can carry, by the cap forms of its sides.  Every
// forward starts a fixed-form side's reference at 0, so that side is never
// empty (an all-NaN row of it yields NaN values through the arithmetic);
// a capped logit is never -inf, so reverse KL flags no support mismatch
// when both sides are capped.  The backward tests only the flags that can
// be set.
template <int CAP>
constexpr bool can_be_empty() {
    return CAP != kCapFixed;
}
template <int CAPA, int CAPB>
constexpr bool can_mismatch() {
    return CAPA == kCapNone || CAPB == kCapNone;
}

// The record with its a and b sides exchanged (gradient w.r.t. the KL
// reference: the operands are exchanged too).
__device__ __forceinline__ void swap_sides(RowStats& rs) {
    const float m = rs.mLa, l = rs.log2Sa;
    rs.mLa = rs.mLb;
    rs.log2Sa = rs.log2Sb;
    rs.mLb = m;
    rs.log2Sb = l;
}

// Per-row coefficients of grad_elem.  With t = y log2 e - mL (the exponent
// of the forward's FMA), p = 2^t / S, so the row's 1 / S = 2^-log2 S (as the
// record holds it) and the log2 S shift of log p are folded into the
// coefficients once per row instead of subtracted per element:
//   logp        A = -G / S                          o = A 2^t
//   entropy     A = -g ln2 / S, B = -g (H - ln2 log2 S) / S
//                                                   o = 2^t (A t + B)
//   reverse KL  A = g ln2 / S_a, B = -g (D + ln2 (log2 S_a - log2 S_b)) / S_a
//                                                   o = 2^ta (A (ta - tb) + B)
//   forward KL  A = g / S_a, B = g / S_b             o = A 2^ta - B 2^tb
// (with the cap, the slope's constant factor cf = slope_factor is folded in
// as well).
template <int HEAD, int CAPA>
__device__ __forceinline__ void row_coeffs(const RowStats& rs, float G, float g_row, float cf,
                                           float& A, float& B) {
    const float f = CAPA != kCapNone ? cf : 1.0f;
    float a0 = 0.0f, b0 = 0.0f;
    if (HEAD == kHeadLogp) {
        a0 = -f * G;
    } else if (HEAD == kHeadEntropy) {
        a0 = -f * g_row * kLn2;
        b0 = -f * g_row * rs.value;
    } else if (HEAD == kHeadKLReverse) {
        a0 = f * g_row * kLn2;
        b0 = -f * g_row * rs.value;
    } else {
        a0 = f * g_row;
    }
    const float inv_sa = ex2(-rs.log2Sa);
    A = a0 * inv_sa;
    if (HEAD == kHeadLogp)
        B = 0.0f;
    else if (HEAD == kHeadEntropy)
        B = __builtin_fmaf(-a0, rs.log2Sa, b0) * inv_sa;
    else if (HEAD == kHeadKLReverse)
        B = __builtin_fmaf(-a0, rs.log2Sa - rs.log2Sb, b0) * inv_sa;
    else
        B = a0 * ex2(-rs.log2Sb);
}

// With a fixed-form cap, S can be as small as 2^-kCapFixedMaxScale and 1 / S
// would overflow the row coefficients: that side's log2 S moves into its
// exponent reference instead (mL is 0 there), so every exponent of it is
// log2 p <= 0 and its 1 / S factor is 1.
template <int CAPA, int CAPB, bool KL>
__device__ __forceinline__ void fixed_refs(RowStats& rs) {
    if (CAPA == kCapFixed) {
        rs.mLa += rs.log2Sa;
        rs.log2Sa = 0.0f;
    }
    if (KL && CAPB == kCapFixed) {
        rs.mLb += rs.log2Sb;
        rs.log2Sb = 0.0f;
    }
}

// A gradient as the rounded fp32 value it is.  The empty asm operand hides
// how it was computed from the conversion to a 16-bit gradient, which the
// compiler would otherwise fuse with a last product on some store paths
// (v_fma_mix: one rounding instead of two) and not on others, so that the
// bits would depend on the path.  It emits no instruction.
__device__ __forceinline__ float rounded(float v) {
    __asm__("" : "+v"(v));
    return v;
}

// Gradient of one element from its statistic inputs (a; b for KL), the
// cap's slope s up to its factor (cap_value_slope) and the row's record and
// coefficients; the exponent t comes from the forward's own FMA.
template <int HEAD, int CAPA>
__device__ __forceinline__ float grad_elem(float a, float s, float b, const RowStats& rs, float A,
                                           float B, float scx, float scy) {
    constexpr bool C = CAPA != kCapNone;
    const float ta = __builtin_fmaf(a, scx, -rs.mLa);
    float o;
    if (HEAD == kHeadLogp) {
        o = A * ex2(ta);
    } else if (HEAD == kHeadEntropy) {
        const float tc = C ? ta : fmaxf(ta, kClampT);
        o = ex2(tc) * __builtin_fmaf(A, tc, B);
    } else {
        const float tb = __builtin_fmaf(b, scy, -rs.mLb);
        if (HEAD == kHeadKLReverse) {
            const float l = C ? ta - tb : fmaxf(ta - tb, kClampT);
            o = ex2(ta) * __builtin_fmaf(A, l, B);
        } else {
            // two rounded products and their difference, never contracted to
            // an FMA: equal distributions give exactly 0
#pragma clang fp contract(off)
            o = A * ex2(ta) - B * ex2(tb);
        }
    }
    if (C) o *= s;  // the slope's factor is in A, B
    return rounded(o);
}

// Logprobs gradient at a target column: h - p G (h: the column's summed
// upstream gradients), times the cap's slope cf s.
template <int CAPA>
__device__ __forceinline__ float target_grad(float a, float s, float cf, const RowStats& rs,
                                             float G, float h, float scx) {
    const float pt = ex2(__builtin_fmaf(a, scx, -rs.mLa) - rs.log2Sa);
    const float v = __builtin_fmaf(-pt, G, h);
    return rounded(CAPA != kCapNone ? v * (cf * s) : v);
}

// Slots of bwd_topk_kernel: the sort keys are padded to a power of two.
__host__ __device__ inline int topk_pad(int64_t k) {
    int n = 2;
    while (n < k) n <<= 1;
    return n;
}

// Dynamic LDS of bwd_topk_kernel: kpad 64-bit sort keys, then k fp32 g.
inline size_t topk_lds_bytes(int64_t k) {
    return static_cast<size_t>(topk_pad(k)) * sizeof(uint64_t) +
           static_cast<size_t>(k) * sizeof(float);
}

// Logprobs with k > kGLanes: one workgroup per (row, column segment), visited
// last-first (the end of the forward's stream is what the Infinity Cache
// still holds).  The k slots are staged in LDS and G is summed in a tree
// fixed by kGLanes (slot j by lane j mod kGLanes, in order), not by BLOCK.
// After the bulk pass a barrier orders the target columns' one-hot rewrites
// after the bulk stores of the same addresses.  The rewrites find duplicate
// ids by sorting the keys (local column, slot) of the row's local slots in
// LDS (bitonic, O(k log^2 k) compare-exchanges over the workgroup): the
// first key of each column's run sums the run's g, which the sort leaves in
// slot order, and writes the column once.
template <int BLOCK, int U, typename T, int CAPA, bool ALIGNED, bool NT>
__global__ __launch_bounds__(BLOCK) RLK_OCCUPANCY void bwd_topk_kernel(BwdParams p) {
    using S = typename T::storage;
    static_assert(BLOCK >= kGLanes, "the G tree needs kGLanes threads");
    // (local column << 32 | slot) of the local slots, all ones for the rest
    // and the padding [kpad]; then fp32 g [k]
    extern __shared__ uint64_t smem_topk[];
    __shared__ float red_g[kGLanes / 64];
    __shared__ float red_n[kGLanes / 64];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t step = (int64_t)U * BLOCK;
    const int64_t nchunks = (p.V + kChunk - 1) / kChunk, nfull = p.V / kChunk;
    const int64_t ngroups = (nchunks + step - 1) / step;
    const int64_t gps = (ngroups + p.split - 1) / p.split;  // groups per column segment
    const RowStats* stats = static_cast<const RowStats*>(p.stats);
    const int kpad = topk_pad(p.k);
    constexpr uint64_t kNoKey = ~0ull;
    uint64_t* keys = smem_topk;
    float* gg = reinterpret_cast<float*>(smem_topk + kpad);
    const CapArgs ca{p.kx, p.ix, CAPA == kCapFixed ? fixed_span(p.ix) : 0.0f};
    const float cf = slope_factor<CAPA>(ca);

    for (int64_t it = blockIdx.x; it < p.N * p.split; it += gridDim.x) {
        const int64_t rit = it / p.split, seg = it - rit * p.split;
        const int64_t row = p.N - 1 - rit;
        const int64_t gbeg = seg * gps, gend = gbeg + gps < ngroups ? gbeg + gps : ngroups;
        const int64_t cbeg = gbeg * step * kChunk, cend = gend * step * kChunk;  // columns
        const S* __restrict__ xa = static_cast<const S*>(p.x) + p.mx.offset(row);
        S* __restrict__ gx = static_cast<S*>(p.gx) + p.mg.offset(row);
        RowStats rs = stats[row];
        fixed_refs<CAPA, kCapNone, false>(rs);

        // Stage the slots: g, and the key of each slot local to this
        // vocabulary shard (plain call: every valid slot).
        float part = 0.0f, cnt = 0.0f;
        if (tid < kGLanes) {
            for (int64_t j = tid; j < p.k; j += kGLanes) {
                const int64_t t = p.targets[row * p.k + j];
                const bool valid = t >= 0 && t < p.vtotal;
                const bool local = t >= p.v0 && t < p.v0 + p.V;
                const float g = p.g[row * p.k + j];
                keys[j] = local ? (static_cast<uint64_t>(t - p.v0) << 32) | static_cast<uint64_t>(j)
                                : kNoKey;
                gg[j] = g;
                if (valid) {
                    part += g;
                    cnt += 1.0f;
                }
            }
        }
        for (int j = static_cast<int>(p.k) + tid; j < kpad; j += BLOCK) keys[j] = kNoKey;
        part = wave_sum(part);
        cnt = wave_sum(cnt);
        if (lane == 0 && wid < kGLanes / 64) {
            red_g[wid] = part;
            red_n[wid] = cnt;
        }
        __syncthreads();
        float n = red_n[0], G = red_g[0];
#pragma unroll
        for (int w = 1; w < kGLanes / 64; ++w) {
            G += red_g[w];
            n += red_n[w];
        }
        const int mode = n == 0.0f ? kModeZero
                         : (can_be_empty<CAPA>() && (rs.flags & kFlagEmptyA)) ? kModeNaN
                                                                               : kModeNormal;

        if (mode == kModeNormal) {
            float A, B;
            row_coeffs<kHeadLogp, CAPA>(rs, G, 0.0f, cf, A, B);
            for_each_group<BLOCK, U, S, kCapNone, ALIGNED, kBwdPipe, NT>(
                xa, p.V, CapArgs{},
                [&](int64_t g0, bool full, const float (&x)[U][kChunk]) {
                    float v[U][kChunk];
#pragma unroll
                    for (int u = 0; u < U; ++u)
#pragma unroll
                        for (int e = 0; e < kChunk; ++e) {
                            float s4;
                            const float a = cap_value_slope<CAPA>(x[u][e], ca, s4);
                            v[u][e] = grad_elem<kHeadLogp, CAPA>(a, s4, 0.0f, rs, A, B, p.scx,
                                                                 p.scy);
                        }
                    if constexpr (sizeof(S) == 4 && ALIGNED) {
                        if (full) {  // uniform: the walk's full groups
                            store_walk_f32<BLOCK, U>(gx, g0, v);
                            return;
                        }
                    }
                    store_group<BLOCK, U, S, ALIGNED>(gx, p.V, g0, full, v);
                },
                gbeg, gend);
            // Sort the keys: a column's slots become one run, in slot order.
            for (int size = 2; size <= kpad; size <<= 1) {
                for (int stride = size >> 1; stride > 0; stride >>= 1) {
                    __syncthreads();
                    for (int i = tid; i < kpad / 2; i += BLOCK) {
                        const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
                        const uint64_t a = keys[lo], b = keys[hi];
                        if ((a > b) == ((lo & size) == 0)) {
                            keys[lo] = b;
                            keys[hi] = a;
                        }
                    }
                }
            }
            // (the last barrier of the sort also orders the rewrites after
            // the bulk stores)
            __syncthreads();
            // Target columns of this segment: the bulk value becomes the
            // one-hot term, written by the first slot of the column's run,
            // which sums the run's g in slot order.
            for (int i = tid; i < p.k; i += BLOCK) {
                const uint64_t key = keys[i];
                if (key == kNoKey) continue;
                const int64_t t = static_cast<int64_t>(key >> 32);
                if (t < cbeg || t >= cend) continue;
                if (i > 0 && (keys[i - 1] >> 32) == (key >> 32)) continue;
                float h = 0.0f;
                for (int r = i; r < p.k && (keys[r] >> 32) == (key >> 32); ++r)
                    h += gg[static_cast<uint32_t>(keys[r])];
                float s4;
                const float a = cap_value_slope<CAPA>(load_one(xa + t), ca, s4);
                store_one(gx + t, target_grad<CAPA>(a, s4, cf, rs, G, h, p.scx));
            }
        } else {
            const float fill = mode == kModeZero ? 0.0f : qnan();
            float v[U][kChunk];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < kChunk; ++e) v[u][e] = fill;
            for (int64_t g0 = gbeg * step; g0 < gend * step; g0 += step)
                store_group<BLOCK, U, S, ALIGNED>(gx, p.V, g0, g0 + step <= nfull, v);
        }
        __syncthreads();
    }
}

// Logprobs calls with at most this many slots per row take the piece kernel
// (up to kGLanes slots bwd_wide_kernel, more bwd_topk_kernel).
constexpr int kPieceMaxK = 4;

// One-shot pieces: every workgroup computes the gradient of U chunks per lane
// (BLOCK x U x 8 columns) of one row and exits.  Its loads are issued before
// anything else, there is no barrier, no LDS and no loop, and a workgroup's
// stores never hold up the next load: on this part such a stream of short
// workgroups moves noticeably more bytes per second than row-long loops.
// Full pieces (every chunk inside an aligned row) load raw 16-byte vectors
// with no branch between them.  Logprobs slots (k <= kPieceMaxK) are read by
// every lane: G is summed in the association of bwd_topk_kernel's tree, and
// target columns take target_grad, so all backward kernels give the same bits.
template <int BLOCK, int U, typename T, int HEAD, int CAPA, int CAPB, bool ALIGNED, bool FULL,
          bool NT, bool CUT = false>
__device__ __forceinline__ void piece(const BwdParams& p, int64_t row, int64_t g0,
                                      int64_t cut = 0) {
    using S = typename T::storage;
    constexpr bool KL = HEAD == kHeadKLReverse || HEAD == kHeadKLForward;
    const int64_t nfull = p.V / kChunk;
    const RowStats* stats = static_cast<const RowStats*>(p.stats);
    const S* __restrict__ xa = static_cast<const S*>(p.x) + p.mx.offset(row);
    S* __restrict__ gx = static_cast<S*>(p.gx) + p.mg.offset(row);

    // raw logits of x (the cap and its slope are taken per element),
    // statistic inputs of y
    float x[U][kChunk], b[U][kChunk];
    RawGroup<S, U> rx, ry;
    const CapArgs cb{p.ky, p.iy};
    const S* __restrict__ xb = KL ? static_cast<const S*>(p.y) + p.my.offset(row) : nullptr;
    // A tail piece reads the row's record and upstream gradient first: its
    // logit loads end in waits (tail_values), and the record's loads would
    // otherwise each add a round trip after them (the tail piece then took
    // three times as long as a full one).  Full pieces read them after the
    // logits, as scalar loads that overlap the logits' latency.
    RowStats rs;
    float g_row = 0.0f;
    if (!FULL) {
        rs = stats[row];
        if (HEAD != kHeadLogp) g_row = p.g[row];
    }
    if (FULL) {
        raw_load<BLOCK, U, NT>(xa, g0, rx);
        if (KL) raw_load<BLOCK, U, NT>(xb, g0, ry);
    } else {
        tail_values<BLOCK, U, S, kCapNone, ALIGNED, NT>(xa, p.V, nfull, g0, CapArgs{}, x);
        if (KL) tail_values<BLOCK, U, S, CAPB, ALIGNED, NT>(xb, p.V, nfull, g0, cb, b);
    }
    const CapArgs ca{p.kx, p.ix, CAPA == kCapFixed ? fixed_span(p.ix) : 0.0f};
    const float cf = slope_factor<CAPA>(ca);

    if (FULL) {
        rs = stats[row];
        if (HEAD != kHeadLogp) g_row = p.g[row];
    }
    if (KL && p.swap) swap_sides(rs);
    fixed_refs<CAPA, CAPB, KL>(rs);

    int mode = kModeNormal;
    float G = 0.0f;
    int64_t tl[kPieceMaxK];  // local column of each slot, -1 if none
    bool hit = false;        // some slot's column lies in this piece (uniform)
    float gs[kPieceMaxK];
    if (HEAD == kHeadLogp) {
        // Slot j < k: valid if 0 <= t < V_total, local column t - v0 if in
        // [0, V); each range test is one unsigned compare.  (Issuing the
        // four slot loads together before any use, forced through an empty
        // asm statement, measured slower here.)
        float sv[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // valid slots' g, zeros beyond k
        int nvalid = 0;
#pragma unroll
        for (int j = 0; j < kPieceMaxK; ++j) {
            tl[j] = -1;
            gs[j] = 0.0f;
            if (j < p.k) {
                const int64_t t = p.targets[row * p.k + j];
                const float g = p.g[row * p.k + j];
                const uint64_t c = static_cast<uint64_t>(t) - static_cast<uint64_t>(p.v0);
                const bool valid = static_cast<uint64_t>(t) < static_cast<uint64_t>(p.vtotal);
                tl[j] = c < static_cast<uint64_t>(p.V) ? static_cast<int64_t>(c) : -1;
                hit |= c - static_cast<uint64_t>(g0 * kChunk) <
                       static_cast<uint64_t>(BLOCK * U * kChunk);
                gs[j] = g;
                if (valid) {
                    sv[j] = g;
                    ++nvalid;
                }
            }
        }
        // bwd_topk_kernel's wave64 butterfly over lanes 0..3 holding the slots
        G = (sv[0] + sv[2]) + (sv[1] + sv[3]);
        if (nvalid == 0)
            mode = kModeZero;
        else if (can_be_empty<CAPA>() && (rs.flags & kFlagEmptyA))
            mode = kModeNaN;
    } else if (HEAD == kHeadEntropy) {
        if (can_be_empty<CAPA>() && (rs.flags & kFlagEmptyA)) mode = kModeNaN;
    } else {
        // (the reference gradient exchanges the sides: both are tested)
        if ((can_be_empty<CAPA>() || can_be_empty<CAPB>()) &&
            (rs.flags & (kFlagEmptyA | kFlagEmptyB)))
            mode = kModeNaN;
        else if (HEAD == kHeadKLReverse && can_mismatch<CAPA, CAPB>() &&
                 (rs.flags & kFlagMismatch))
            mode = kModeMismatch;
    }
    if (FULL) {
        raw_unpack(rx, x);
        if (KL) fast_values<U, S, CAPB>(ry, cb, b);
    }

    // Entropy and KL compute the bulk values for every row and replace them
    // afterwards in the rare rows that need others: their mode comes from the
    // record's flags alone, and with a mode branch around the computation the
    // compiler moved the logits' loads into it, behind a wait for the flags.
    // (Logprobs' mode also needs the slots, which are read after the logits.)
    constexpr bool UNCOND = HEAD != kHeadLogp;
    float v[U][kChunk];
    if (UNCOND || mode == kModeNormal) {
        float A, B;
        row_coeffs<HEAD, CAPA>(rs, G, g_row, cf, A, B);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float a[kChunk], s4[kChunk];
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                a[e] = cap_value_slope<CAPA>(x[u][e], ca, s4[e]);
                v[u][e] = grad_elem<HEAD, CAPA>(a[e], s4[e], KL ? b[u][e] : 0.0f, rs, A, B,
                                                p.scx, p.scy);
            }
            if (HEAD == kHeadLogp && hit) {
                // one-hot terms: a slot whose column falls in this lane's chunk
                // (most pieces hold no target column and skip this); values
                // 0..3 sit at columns lo.., 4..7 at hi.. (piece_col)
                constexpr bool Q = piece_quads<S, FULL>();
                const int64_t lo = piece_col<BLOCK, Q>(g0, u, threadIdx.x, 0);
                const int64_t hi = piece_col<BLOCK, Q>(g0, u, threadIdx.x, 4);
                bool any = false;
#pragma unroll
                for (int j = 0; j < kPieceMaxK; ++j)
                    any |= Q ? (tl[j] >= lo && tl[j] < lo + 4) || (tl[j] >= hi && tl[j] < hi + 4)
                             : tl[j] >= lo && tl[j] < lo + kChunk;
                if (any) {
#pragma unroll
                    for (int e = 0; e < kChunk; ++e) {
                        const int64_t col = e < 4 ? lo + e : hi + (e - 4);
                        float h = 0.0f;
                        bool match = false;
#pragma unroll
                        for (int j = 0; j < kPieceMaxK; ++j)
                            if (tl[j] == col) {
                                h += gs[j];
                                match = true;
                            }
                        if (match) v[u][e] = target_grad<CAPA>(a[e], s4[e], cf, rs, G, h, p.scx);
                    }
                }
            }
        }
    }
    if (mode == kModeMismatch) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < kChunk; ++e)
                v[u][e] = (CAPA == kCapNone && x[u][e] == neg_inf()) ? 0.0f : qnan();
    } else if (mode != kModeNormal) {
        const float fill = mode == kModeZero ? 0.0f : qnan();
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < kChunk; ++e) v[u][e] = fill;
    }
    const uint32_t skip = CUT ? static_cast<uint32_t>(cut - g0) : 0u;
    if (FULL && p.wt)
        store_piece<BLOCK, U, S, kCpolWriteThrough, CUT>(gx + g0 * kChunk, v, skip);
    else if (FULL)
        store_piece<BLOCK, U, S, kCpolStream, CUT>(gx + g0 * kChunk, v, skip);
    else
        store_group<BLOCK, U, S, ALIGNED, CUT>(gx, p.V, g0, false, v, cut);
}

// grid (pieces of a row, rows): consecutive workgroups take consecutive
// pieces of a row, so the chip sweeps the matrix front to back; rows run
// last-first (see bwd_topk_kernel).
template <int BLOCK, int U, typename T, int HEAD, int CAPA, int CAPB, bool ALIGNED, bool NT>
__global__ __launch_bounds__(BLOCK) void bwd_piece_kernel(BwdParams p, int64_t rbase) {
    const int64_t row = p.N - 1 - (rbase + static_cast<int64_t>(blockIdx.y));
    const int64_t g0 = static_cast<int64_t>(blockIdx.x) * (BLOCK * U);  // first chunk
    if (ALIGNED && g0 + BLOCK * U <= p.V / kChunk)
        piece<BLOCK, U, T, HEAD, CAPA, CAPB, ALIGNED, true, NT>(p, row, g0);
    else
        piece<BLOCK, U, T, HEAD, CAPA, CAPB, ALIGNED, false, NT>(p, row, g0);
}

// The last piece of each row (one workgroup per row, grid (1, rows)), moved
// back to end at the row's end: it takes the full-piece path, recomputes the
// columns it shares with the piece before it and stores only its own.  Used
// for aligned rows of whole chunks whose tail is at least half a piece (see
// last_piece_apart).
template <int BLOCK, int U, typename T, int HEAD, int CAPA, int CAPB, bool NT>
__global__ __launch_bounds__(BLOCK) void bwd_last_piece_kernel(BwdParams p, int64_t rbase) {
    const int64_t row = p.N - 1 - (rbase + static_cast<int64_t>(blockIdx.y));
    const int64_t nfull = p.V / kChunk;
    const int64_t cut = nfull / (BLOCK * U) * (BLOCK * U);
    piece<BLOCK, U, T, HEAD, CAPA, CAPB, true, true, NT, true>(p, row, nfull - BLOCK * U, cut);
}

// Logprobs with kPieceMaxK < k <= kGLanes: one-shot pieces of kGLanes lanes
// x U chunks (2048 U columns) of one row.  Each lane reads one slot: G and the
// valid count take bwd_topk_kernel's tree (slot j in lane j, wave butterfly,
// the four waves in order), so both kernels give the same bits.  The slots
// whose column falls in the piece are compacted into LDS in slot order
// (ballot ranks, per-wave offsets) and marked in a bitmap of one byte per
// chunk; a lane whose chunk has a marked column sums that column's slots from
// the list in slot order (bwd_topk_kernel's one-hot sum) and writes the
// target gradient in place of the bulk value.  A short list is searched entry
// by entry; a long one (a small V puts many targets in one piece) is sorted by
// (column, slot) first, and each marked chunk starts at its first key, so a
// column costs a few reads instead of a pass over the list.  Every column is
// computed once and stored once, the data loads are issued first, and the
// piece exits after its stores: the slot work (k 12-byte records, mostly from
// L2) is spread over 4 KB U of logits.
// FULL: every chunk of the piece lies inside an aligned row, so its loads are
// raw 16-byte vectors issued back to back without branches (tail_values'
// per-chunk branches would make the compiler wait for each load in turn).
// LDS of a wide piece, declared once per kernel (the full and tail forms of
// the piece are two instantiations of wide_piece and share it).
template <int U>
struct WideLds {
    static constexpr int NW = kGLanes / 64, PC = kGLanes * U;
    // one byte per chunk, lane-major: word t holds lane t's U chunks (byte
    // u: the columns of chunk slot u marked), so a lane reads its marks once
    uint32_t bits[kGLanes];
    // (the column's lane-order index in the piece, piece_slot; g as bits) in
    // slot order, padded to a multiple of 4 entries with (-1, +0) so that the
    // search reads 4 entries per step (8 per step measured slower: the kernel
    // then needs 88 VGPRs instead of 80, 5 waves per SIMD instead of 6)
    alignas(16) int2 list[kGLanes];
    // A list longer than kWideScanMax entries (many targets per piece: a small
    // V or a large k) is searched through its keys (lane-order index << 16 |
    // list index) sorted in LDS and the first sorted position of each marked
    // chunk.
    uint32_t skey[kGLanes];
    uint16_t cstart[PC];
    // A short list without repeated columns (no duplicate ids in the piece,
    // the common case) is not searched: each marked column's list position
    // sits in head (written only for marked columns, so never cleared)
    uint8_t head[PC * kChunk];
    int dup;  // some column is marked by more than one slot
    float red_g[NW], red_n[NW];
    int red_c[NW];
};

template <int U, typename T, int CAPA, bool ALIGNED, bool FULL, bool NT, bool CUT = false>
__device__ __forceinline__ void wide_piece(const BwdParams& p, WideLds<U>& L, int64_t row,
                                           int64_t g0, int64_t cut = 0) {
    using S = typename T::storage;
    constexpr int BLOCK = kGLanes, NW = kGLanes / 64;
    constexpr int PC = BLOCK * U;  // chunks per piece
    static_assert(U <= 4, "a lane's chunk marks fill one word");
    static_assert(kGLanes <= 256, "list positions fit head's bytes");
    uint32_t(&bits)[kGLanes] = L.bits;
    int2(&list)[kGLanes] = L.list;
    uint32_t(&skey)[kGLanes] = L.skey;
    uint16_t(&cstart)[PC] = L.cstart;
    uint8_t(&head)[PC * kChunk] = L.head;
    int& dup = L.dup;
    float(&red_g)[NW] = L.red_g;
    float(&red_n)[NW] = L.red_n;
    int(&red_c)[NW] = L.red_c;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t nfull = p.V / kChunk;
    const RowStats* stats = static_cast<const RowStats*>(p.stats);
    const S* __restrict__ xa = static_cast<const S*>(p.x) + p.mx.offset(row);
    S* __restrict__ gx = static_cast<S*>(p.gx) + p.mg.offset(row);

    // The slot loads go first (mostly L2 hits): loads complete in order, so
    // G, the list and both barriers then overlap the logits' HBM latency.
    int64_t t = -1;
    float gj = 0.0f;
    if (tid < p.k) {
        t = p.targets[row * p.k + tid];
        gj = p.g[row * p.k + tid];
    }
    RawGroup<S, U> raw;
    float x[U][kChunk];
    if (FULL)
        raw_load<BLOCK, U, NT>(xa, g0, raw);
    else
        tail_values<BLOCK, U, S, kCapNone, ALIGNED, NT>(xa, p.V, nfull, g0, CapArgs{}, x);
    RowStats rs = stats[row];
    fixed_refs<CAPA, kCapNone, false>(rs);

    float part = 0.0f, cnt = 0.0f;
    bool mine = false;  // slot tid names a column of this piece
    int pcol = 0;
    if (tid < p.k) {
        if (t >= 0 && t < p.vtotal) {
            part += gj;
            cnt = 1.0f;
        }
        const int64_t c = t - p.v0 - g0 * kChunk;
        mine = t >= p.v0 && t < p.v0 + p.V && c >= 0 && c < static_cast<int64_t>(PC) * kChunk;
        // the list and bitmap index values in lane order (piece_slot)
        pcol = piece_slot<BLOCK, piece_quads<S, FULL>()>(static_cast<int>(c));
    }
    bits[tid] = 0u;
    if (tid == 0) dup = 0;
    part = wave_sum(part);
    cnt = wave_sum(cnt);
    const uint64_t m = __ballot(mine);
    if (lane == 0) {
        red_g[wid] = part;
        red_n[wid] = cnt;
        red_c[wid] = __popcll(m);
    }
    __syncthreads();
    float G = red_g[0], n = red_n[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        G += red_g[w];
        n += red_n[w];
    }
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        base += w < wid ? red_c[w] : 0;
        total += red_c[w];
    }
    if (mine) {
        const int rank = __popcll(m & ((1ull << lane) - 1ull));
        list[base + rank] = make_int2(pcol, __float_as_int(gj));
        head[pcol] = static_cast<uint8_t>(base + rank);
        const int ci = pcol / kChunk;
        const uint32_t bit = 1u << ((ci / BLOCK) * 8 + pcol % kChunk);
        if (atomicOr(&bits[ci % BLOCK], bit) & bit) dup = 1;
    }
    if (tid >= total && tid < ((total + 3) & ~3)) list[tid] = make_int2(-1, 0);
    if (total > 0) __syncthreads();  // uniform: the list and bitmap are complete
    const bool sorted = total > kWideScanMax;  // uniform
    if (sorted) {
        int pad = 2;
        while (pad < total) pad <<= 1;
        if (tid < pad)
            skey[tid] = tid < total ? (static_cast<uint32_t>(list[tid].x) << 16) |
                                          static_cast<uint32_t>(tid)
                                    : 0xffffffffu;
        for (int size = 2; size <= pad; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                __syncthreads();
                if (tid < pad / 2) {
                    const int lo = 2 * tid - (tid & (stride - 1)), hi = lo + stride;
                    const uint32_t ka = skey[lo], kb = skey[hi];
                    if ((ka > kb) == ((lo & size) == 0)) {
                        skey[lo] = kb;
                        skey[hi] = ka;
                    }
                }
            }
        }
        __syncthreads();
        if (tid < total) {
            const uint32_t c = skey[tid] >> 19;  // chunk of the key's column
            if (tid == 0 || (skey[tid - 1] >> 19) != c) cstart[c] = static_cast<uint16_t>(tid);
        }
        __syncthreads();
    }
    const int mode = n == 0.0f ? kModeZero
                     : (can_be_empty<CAPA>() && (rs.flags & kFlagEmptyA)) ? kModeNaN
                                                                           : kModeNormal;
    if (FULL) raw_unpack(raw, x);

    float v[U][kChunk];
    if (mode == kModeNormal) {
        const CapArgs ca{p.kx, p.ix, CAPA == kCapFixed ? fixed_span(p.ix) : 0.0f};
        const float cf = slope_factor<CAPA>(ca);
        float A, B;
        row_coeffs<kHeadLogp, CAPA>(rs, G, 0.0f, cf, A, B);
        const uint32_t marks = total > 0 ? bits[tid] : 0u;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ci = u * BLOCK + tid;
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                float s4;
                const float a = cap_value_slope<CAPA>(x[u][e], ca, s4);
                v[u][e] = grad_elem<kHeadLogp, CAPA>(a, s4, 0.0f, rs, A, B, p.scx, p.scy);
            }
            // (a target column takes its statistic input and slope again
            // from x: keeping them for all 8 columns costs registers)
            const uint32_t mark = (marks >> (u * 8)) & 0xffu;
            if (mark) {  // rare: a target column in this chunk
                // one pass per marked column (its value picked by selects),
                // not a test of all 8 with the search repeated in each
                uint32_t mk = mark;
                do {
                    const int e = __builtin_ctz(mk);
                    mk &= mk - 1u;
                    const int col = ci * kChunk + e;
                    float h = 0.0f;
                    if (!sorted && !dup) {
                        // the column's one slot (h = +0 + g, as the scan
                        // below would sum it)
                        h += __int_as_float(list[head[col]].y);
                    } else if (sorted) {
                        // the chunk's keys follow cstart in (column, slot)
                        // order: the column's g are summed in slot order
                        for (int r = cstart[ci]; r < total; ++r) {
                            const uint32_t key = skey[r];
                            const int kc = static_cast<int>(key >> 16);
                            if (kc > col) break;
                            if (kc == col) h += __int_as_float(list[key & 0xffffu].y);
                        }
                    } else {
                        // the matching slots' g in slot order; adding +0 for
                        // the others leaves every partial sum's bits unchanged
                        // (h starts at +0 and a sum is never -0 in
                        // round-to-nearest)
                        const int4* l4 = reinterpret_cast<const int4*>(list);
                        for (int j = 0; j < total; j += 4) {
                            const int4 l0 = l4[j >> 1], l1 = l4[(j >> 1) + 1];
                            h += l0.x == col ? __int_as_float(l0.y) : 0.0f;
                            h += l0.z == col ? __int_as_float(l0.w) : 0.0f;
                            h += l1.x == col ? __int_as_float(l1.y) : 0.0f;
                            h += l1.z == col ? __int_as_float(l1.w) : 0.0f;
                        }
                    }
                    float xe = x[u][0];
#pragma unroll
                    for (int i = 1; i < kChunk; ++i) xe = e == i ? x[u][i] : xe;
                    float s4;
                    const float a = cap_value_slope<CAPA>(xe, ca, s4);
                    const float tg = target_grad<CAPA>(a, s4, cf, rs, G, h, p.scx);
#pragma unroll
                    for (int i = 0; i < kChunk; ++i) v[u][i] = e == i ? tg : v[u][i];
                } while (mk);
            }
        }
    } else {
        const float fill = mode == kModeZero ? 0.0f : qnan();
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < kChunk; ++e) v[u][e] = fill;
    }
    // (plain streaming stores: the sc1 policy of store_piece measured slower
    // for these 16 KB pieces)
    if constexpr (piece_quads<S, FULL>())
        store_piece<BLOCK, U, S, kCpolStream, CUT>(gx + g0 * kChunk, v,
                                                   CUT ? static_cast<uint32_t>(cut - g0) : 0u);
    else
        store_group<BLOCK, U, S, ALIGNED, CUT>(gx, p.V, g0, FULL, v, cut);
}

template <int U, typename T, int CAPA, bool ALIGNED, bool NT>
__device__ __forceinline__ void wide_pieces(const BwdParams& p, int64_t rbase) {
    const int64_t row = p.N - 1 - (rbase + static_cast<int64_t>(blockIdx.y));
    const int64_t g0 = static_cast<int64_t>(blockIdx.x) * (kGLanes * U);
    __shared__ WideLds<U> L;
    if (ALIGNED && g0 + kGLanes * U <= p.V / kChunk)
        wide_piece<U, T, CAPA, ALIGNED, true, NT>(p, L, row, g0);
    else
        wide_piece<U, T, CAPA, ALIGNED, false, NT>(p, L, row, g0);
}

// Rows with 16-byte aligned starts: held to 72 VGPRs, seven waves per SIMD
// (top-256 + cap 20 bf16 [2048, 262144]: 418 -> 399 us against six waves at
// 76 VGPRs; eight waves spill and were slower for k = 16 and 64).
template <int U, typename T, int CAPA, bool NT>
__global__ __launch_bounds__(kGLanes) __attribute__((amdgpu_waves_per_eu(7))) void bwd_wide_kernel(
    BwdParams p, int64_t rbase) {
    wide_pieces<U, T, CAPA, true, NT>(p, rbase);
}

// Other rows (element loads) keep the registers they need.
template <int U, typename T, int CAPA, bool NT>
__global__ __launch_bounds__(kGLanes) void bwd_wide_kernel_unaligned(BwdParams p, int64_t rbase) {
    wide_pieces<U, T, CAPA, false, NT>(p, rbase);
}

// The last wide piece of each row, as bwd_last_piece_kernel.
template <int U, typename T, int CAPA, bool NT>
__global__ __launch_bounds__(kGLanes) __attribute__((amdgpu_waves_per_eu(6))) void
bwd_wide_last_kernel(BwdParams p, int64_t rbase) {
    const int64_t row = p.N - 1 - (rbase + static_cast<int64_t>(blockIdx.y));
    const int64_t nfull = p.V / kChunk;
    const int64_t cut = nfull / (kGLanes * U) * (kGLanes * U);
    __shared__ WideLds<U> L;
    wide_piece<U, T, CAPA, true, true, NT, true>(p, L, row, nfull - kGLanes * U, cut);
}

// ------------------------------------------------------------- dispatch
//
// The backward is elementwise given the row record (and G has a fixed tree),
// so its launch shape does not change any result and is chosen per call:
// one-shot 256-thread pieces for entropy, KL and logprobs with k <= 4;
// one-shot wide pieces (256 lanes x kBwdWideUnroll chunks, half that where a
// piece would hold few targets) for logprobs with k <= kGLanes; for wider top-k bwd_topk_kernel with 512-thread workgroups
// (fewer idle lanes during each row's fix-up), or, for fewer than
// kBwdSmallRows rows, 256-thread workgroups with the rows cut into column
// segments.

// Targets per full wide piece (on average) up to which the half-size pieces
// are used.
constexpr int64_t kWideFewTargets = 5;
constexpr int kBwdWideUnrollHalf = kBwdWideUnroll > 1 ? kBwdWideUnroll / 2 : 1;

// Rows per piece launch (the grid's second dimension is limited to 65536).
constexpr int64_t kPieceRowsPerLaunch = 65536;

// Whether the last piece of each row (pc chunks per piece) runs apart, moved
// back to end at the row's end (bwd_last_piece_kernel), in a second launch:
// for aligned rows of whole chunks, fewer than 16 pieces long, whose tail is
// at least half a piece, in a call of at least 64 MiB of logits.  The tail
// path would cost about three full pieces (branching loads); with a shorter
// tail the recomputed shared part, in a longer row or a smaller call the
// second launch cost more than that (logprobs bf16 backward, k = 1
// [16384, 32000]: 378 -> 332 us, k = 4: 482 -> 332 us; but [4096, 128256],
// 62 pieces: 308 us either way, and fp32 [64, 32000]: 5.5 -> 8.4 us).
inline bool last_piece_apart(bool aligned, int64_t N, int64_t V, int64_t esize, int64_t pc) {
    const int64_t nfull = V / kChunk;
    return aligned && V % kChunk == 0 && nfull >= pc && nfull / pc < 16 &&
           2 * (nfull % pc) >= pc && N * V * esize >= (int64_t(64) << 20);
}

template <typename T, int HEAD, int CAPX, int CAPY, bool AL, bool NT>
inline hipError_t bwd_piece_launch(const BwdParams& p0, hipStream_t s) {
    BwdParams p = p0;
    p.wt = static_cast<uint64_t>(p.N) * static_cast<uint64_t>(p.V) * T::kBytes >=
           kWriteThroughBytes;
    constexpr int U = kBwdPieceUnroll;
    constexpr int64_t pc = static_cast<int64_t>(kBwdPieceBlock) * U;
    const bool apart = last_piece_apart(AL, p.N, p.V, T::kBytes, pc);
    const int64_t pieces = apart ? p.V / kChunk / pc : ((p.V + kChunk - 1) / kChunk + pc - 1) / pc;
    constexpr bool KL = HEAD == kHeadKLReverse || HEAD == kHeadKLForward;
    const unsigned lds = lds_for_wgs_per_cu(piece_wgs_per_cu<T::kBytes, KL>());
    for (int64_t r0 = 0; r0 < p.N; r0 += kPieceRowsPerLaunch) {
        const int64_t rows = p.N - r0 < kPieceRowsPerLaunch ? p.N - r0 : kPieceRowsPerLaunch;
        const dim3 grid(static_cast<unsigned>(pieces), static_cast<unsigned>(rows));
        hipLaunchKernelGGL((bwd_piece_kernel<kBwdPieceBlock, U, T, HEAD, CAPX, CAPY, AL, NT>), grid,
                           dim3(kBwdPieceBlock), lds, s, p, r0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if constexpr (AL) {
            if (apart) {
                hipLaunchKernelGGL(
                    (bwd_last_piece_kernel<kBwdPieceBlock, U, T, HEAD, CAPX, CAPY, NT>),
                    dim3(1, static_cast<unsigned>(rows)), dim3(kBwdPieceBlock), 0, s, p, r0);
                e = hipGetLastError();
                if (e != hipSuccess) return e;
            }
        }
    }
    return hipSuccess;
}

template <int U, typename T, int CAPX, bool AL, bool NT>
inline hipError_t bwd_wide_launch(const BwdParams& p, hipStream_t s) {
    constexpr int64_t pc = static_cast<int64_t>(kGLanes) * U;
    const bool apart = last_piece_apart(AL, p.N, p.V, T::kBytes, pc);
    const int64_t pieces = apart ? p.V / kChunk / pc : ((p.V + kChunk - 1) / kChunk + pc - 1) / pc;
    for (int64_t r0 = 0; r0 < p.N; r0 += kPieceRowsPerLaunch) {
        const int64_t rows = p.N - r0 < kPieceRowsPerLaunch ? p.N - r0 : kPieceRowsPerLaunch;
        const dim3 grid(static_cast<unsigned>(pieces), static_cast<unsigned>(rows));
        if constexpr (AL)
            hipLaunchKernelGGL((bwd_wide_kernel<U, T, CAPX, NT>), grid, dim3(kGLanes),
                               lds_for_wgs_per_cu(wide_wgs_per_cu<T::kBytes>()), s, p, r0);
        else
            hipLaunchKernelGGL((bwd_wide_kernel_unaligned<U, T, CAPX, NT>), grid,
                               dim3(kGLanes), 0, s, p, r0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if constexpr (AL) {
            if (apart) {
                hipLaunchKernelGGL((bwd_wide_last_kernel<U, T, CAPX, NT>),
                                   dim3(1, static_cast<unsigned>(rows)), dim3(kGLanes), 0, s, p,
                                   r0);
                e = hipGetLastError();
                if (e != hipSuccess) return e;
            }
        }
    }
    return hipSuccess;
}

template <int BB, int U, typename T, int CAPX, bool AL, bool NT>
inline hipError_t bwd_topk_launch(const BwdParams& p, hipStream_t s) {
    const size_t lds = topk_lds_bytes(p.k);
    hipLaunchKernelGGL((bwd_topk_kernel<BB, U, T, CAPX, AL, NT>), dim3(row_grid(p.N * p.split)),
                       dim3(BB), lds, s, p);
    return hipGetLastError();
}

template <typename T, int CAPX, int CAPY, bool AL, bool NT>
inline hipError_t bwd_dispatch_al(int head, const BwdParams& p0, hipStream_t s) {
    switch (head) {
        case kHeadEntropy:
            return bwd_piece_launch<T, kHeadEntropy, CAPX, kCapNone, AL, NT>(p0, s);
        case kHeadKLReverse:
            return bwd_piece_launch<T, kHeadKLReverse, CAPX, CAPY, AL, NT>(p0, s);
        case kHeadKLForward:
            return bwd_piece_launch<T, kHeadKLForward, CAPX, CAPY, AL, NT>(p0, s);
        case kHeadLogp:
            break;
        default:
            return hipErrorInvalidValue;
    }
    if (p0.k <= kPieceMaxK) return bwd_piece_launch<T, kHeadLogp, CAPX, kCapNone, AL, NT>(p0, s);
    if (p0.k <= kGLanes) {
        // Half-size pieces where a full one would hold few targets: their
        // slot staging then costs less than the shorter pieces stream faster
        // (k = 16 at [4096, 32000] -5%, k = 64 at [8192, 151936] -4%; with 8
        // targets per full piece, c5's shape, +8%).
        if (p0.k * kGLanes * kBwdWideUnroll * kChunk <= kWideFewTargets * p0.V)
            return bwd_wide_launch<kBwdWideUnrollHalf, T, CAPX, AL, NT>(p0, s);
        return bwd_wide_launch<kBwdWideUnroll, T, CAPX, AL, NT>(p0, s);
    }
    BwdParams p = p0;
    if (p.N < kBwdSmallRows) {
        // Few rows: narrow workgroups, each row cut into column segments.
        const int64_t step = (int64_t)kBwdUnrollSmall * kBwdBlockSmall;
        const int64_t ngroups = ((p.V + kChunk - 1) / kChunk + step - 1) / step;
        const int64_t split = (kBwdTargetItems + p.N - 1) / p.N;
        p.split = split < ngroups ? split : (ngroups > 0 ? ngroups : 1);
        return bwd_topk_launch<kBwdBlockSmall, kBwdUnrollSmall, T, CAPX, AL, NT>(p, s);
    }
    p.split = 1;
    return bwd_topk_launch<kBwdBlockTopk, kBwdUnrollTopk, T, CAPX, AL, NT>(p, s);
}

// Rows that are not 16-byte aligned read every element with ordinary loads,
// so only aligned rows choose between streaming and cached loads.
template <typename T, int CAPX, int CAPY>
inline hipError_t bwd_dispatch_a(int head, bool al, const BwdParams& p, hipStream_t s) {
    if (!al) return bwd_dispatch_al<T, CAPX, CAPY, false, true>(head, p, s);
    const bool kl = head == kHeadKLReverse || head == kHeadKLForward;
    return stream_reads(p.N, p.V, T::kBytes, kl ? 2 : 1)
               ? bwd_dispatch_al<T, CAPX, CAPY, true, true>(head, p, s)
               : bwd_dispatch_al<T, CAPX, CAPY, true, false>(head, p, s);
}

template <typename T, int CAPX>
inline hipError_t bwd_dispatch_cy(int head, int cy, bool al, const BwdParams& p, hipStream_t s) {
    if (cy == kCapOnline) return bwd_dispatch_a<T, CAPX, kCapOnline>(head, al, p, s);
    if (cy == kCapFixed) return bwd_dispatch_a<T, CAPX, kCapFixed>(head, al, p, s);
    return bwd_dispatch_a<T, CAPX, kCapNone>(head, al, p, s);
}

template <typename T>
inline hipError_t bwd_dispatch_cap(int head, int cx, int cy, bool al, const BwdParams& p,
                                   hipStream_t s) {
    const bool kl = head == kHeadKLReverse || head == kHeadKLForward;
    if (!kl) cy = kCapNone;
    if (cx == kCapOnline) return bwd_dispatch_cy<T, kCapOnline>(head, cy, al, p, s);
    if (cx == kCapFixed) return bwd_dispatch_cy<T, kCapFixed>(head, cy, al, p, s);
    return bwd_dispatch_cy<T, kCapNone>(head, cy, al, p, s);
}

}  // namespace rlk
