// rlk_fwd_kernels.h -- forward row kernels: one read of each logit, online
// statistics, head outputs and the per-row record for the backward.
//
// Single-read statistics follow the review comment on the entropy / KL
// forward of "Add Triton kernels for vocab-parallel logprobs, entropy and
// KL" (DeepSpeed pull request 8838), which proposes a single pass over the
// logits in place of the first version's two: the running max, the sum of exponentials and a probability-weighted sum of
// centred logits, all rescaled when the max grows, give
//   entropy  H = log S - W / S,
//   KL(A||B) = W / S_A - log S_A + log S_B,
// and a support-mismatch flag decided on the logits.  The logprobs head reads
// the target logit (prefetched when the row starts) and subtracts the row's
// logsumexp (pull request 495, Behavior changes: targets outside [0, V)
// give 0).
//
// Streaming: one workgroup per row; lane tid consumes groups of U chunks of 8
// logits with 16-byte nontemporal loads (for_each_group in rlk_device.h).
#pragma once

#include "rlk_device.h"
#include "rlk_launch.h"

namespace rlk {

// Fold one group into a single-tensor state.  CLAMP keeps 0 * (-inf) out of
// W where -inf can occur: masked logits (never with the softcap) and the
// padding of a row's tail group.  FIXED: a is already t (fixed cap form), the
// reference never moves.
template <int U, bool WITH_W, bool CLAMP, bool FIXED = false>
__device__ __forceinline__ void update1(Stat1& st, const float (&a)[U][kChunk], float sc) {
    float gm = a[0][0];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < kChunk; ++e) gm = fmaxf(gm, a[u][e]);
    if (!FIXED && gm > st.m) {
        const float mLn = gm * sc;
        if (st.m != neg_inf()) {
            const float d = st.mL - mLn;
            const float s = ex2(d);
            if (WITH_W) st.W = s * __builtin_fmaf(d, st.S, st.W);
            st.S *= s;
        }
        st.m = gm;
        st.mL = mLn;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
            float t = FIXED ? a[u][e] : __builtin_fmaf(a[u][e], sc, -st.mL);
            if (CLAMP) t = fmaxf(t, kClampT);
            const float ex = ex2(t);
            st.S += ex;
            if (WITH_W) st.W = __builtin_fmaf(ex, t, st.W);
        }
}

// Fold one group into a KL state (a: policy, b: reference).  FIXA / FIXB:
// that side's values are already t (fixed cap form).
template <int U, bool REVERSE, bool FIXA = false, bool FIXB = false>
__device__ __forceinline__ void update_kl(StatKL& st, const float (&a)[U][kChunk],
                                          const float (&b)[U][kChunk], float sca, float scb) {
    float gma = a[0][0], gmb = b[0][0];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
            gma = fmaxf(gma, a[u][e]);
            gmb = fmaxf(gmb, b[u][e]);
        }
    if (!FIXA && gma > st.ma) {
        const float mLn = gma * sca;
        if (st.ma != neg_inf()) {
            const float d = st.mLa - mLn;
            const float s = ex2(d);
            if (REVERSE)
                st.W = s * __builtin_fmaf(d, st.Sa, st.W);
            else
                st.W = __builtin_fmaf(-d, st.Sb, st.W);
            st.Sa *= s;
        }
        st.ma = gma;
        st.mLa = mLn;
    }
    if (!FIXB && gmb > st.mb) {
        const float mLn = gmb * scb;
        if (st.mb != neg_inf()) {
            const float d = st.mLb - mLn;
            const float s = ex2(d);
            if (REVERSE)
                st.W = __builtin_fmaf(-d, st.Sa, st.W);
            else
                st.W = s * __builtin_fmaf(d, st.Sb, st.W);
            st.Sb *= s;
        }
        st.mb = gmb;
        st.mLb = mLn;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
            const float ta = FIXA ? a[u][e] : __builtin_fmaf(a[u][e], sca, -st.mLa);
            const float tb = FIXB ? b[u][e] : __builtin_fmaf(b[u][e], scb, -st.mLb);
            const float ea = ex2(ta), eb = ex2(tb);
            st.Sa += ea;
            st.Sb += eb;
            const float d = ta - tb;
            if (REVERSE) {
                st.flag = fmaxf(st.flag, d);
                st.W = __builtin_fmaf(ea, fmaxf(d, kClampT), st.W);
            } else {
                st.flag = fminf(st.flag, d);
                st.W = __builtin_fmaf(eb, fmaxf(-d, kClampT), st.W);
            }
        }
}

// Fold one group into the two-direction KL state: each direction's W and
// flag see the very operations of update_kl<U, true> / update_kl<U, false>.
template <int U, bool FIXA = false, bool FIXB = false>
__device__ __forceinline__ void update_kl2(StatKL2& st, const float (&a)[U][kChunk],
                                           const float (&b)[U][kChunk], float sca, float scb) {
    float gma = a[0][0], gmb = b[0][0];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
            gma = fmaxf(gma, a[u][e]);
            gmb = fmaxf(gmb, b[u][e]);
        }
    if (!FIXA && gma > st.ma) {
        const float mLn = gma * sca;
        if (st.ma != neg_inf()) {
            const float d = st.mLa - mLn;
            const float s = ex2(d);
            st.Wr = s * __builtin_fmaf(d, st.Sa, st.Wr);
            st.Wf = __builtin_fmaf(-d, st.Sb, st.Wf);
            st.Sa *= s;
        }
        st.ma = gma;
        st.mLa = mLn;
    }
    if (!FIXB && gmb > st.mb) {
        const float mLn = gmb * scb;
        if (st.mb != neg_inf()) {
            const float d = st.mLb - mLn;
            const float s = ex2(d);
            st.Wr = __builtin_fmaf(-d, st.Sa, st.Wr);
            st.Wf = s * __builtin_fmaf(d, st.Sb, st.Wf);
            st.Sb *= s;
        }
        st.mb = gmb;
        st.mLb = mLn;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
            const float ta = FIXA ? a[u][e] : __builtin_fmaf(a[u][e], sca, -st.mLa);
            const float tb = FIXB ? b[u][e] : __builtin_fmaf(b[u][e], scb, -st.mLb);
            const float ea = ex2(ta), eb = ex2(tb);
            st.Sa += ea;
            st.Sb += eb;
            const float d = ta - tb;
            st.fmax = fmaxf(st.fmax, d);
            st.Wr = __builtin_fmaf(ea, fmaxf(d, kClampT), st.Wr);
            st.fmin = fminf(st.fmin, d);
            st.Wf = __builtin_fmaf(eb, fmaxf(-d, kClampT), st.Wf);
        }
}

// One target slot's output: the statistic input of a target this shard owns
// (shard call) or the slot's logprob, 0 for a target outside [0, V).
template <int CAP>
__device__ __forceinline__ void slot_out(const FwdParams& p, int64_t row, int64_t j, int64_t t,
                                         float xv, CapArgs ca, const RowStats& rs) {
    const bool local = t >= p.v0 && t < p.v0 + p.V;
    const float a = local ? cap_value<CAP>(xv, ca) : 0.0f;
    if (p.part)
        p.tvals[row * p.k + j] = a;
    else
        p.out[row * p.k + j] = (t >= 0 && t < p.vtotal) ? target_logp(a, p.scx, rs) : 0.0f;
}

// Logprobs / entropy forward: one workgroup per row.
template <int BLOCK, int U, typename T, int HEAD, int CAP, bool ALIGNED, bool NT, bool ODD = false>
__global__ __launch_bounds__(BLOCK) RLK_OCCUPANCY void fwd1_kernel(FwdParams p) {
    using S = typename T::storage;
    constexpr bool WITH_W = HEAD == kHeadEntropy;
    constexpr bool FIX = CAP == kCapFixed;
    constexpr bool CLAMP = WITH_W && CAP == kCapNone;  // full groups; tail groups always clamp
    // ODD: the fixed form's statistics take the odd form (reference -sc/2),
    // the same bits as fwd1_tab_kernel's table; targets keep the direct form
    static_assert(!ODD || FIX, "the odd form is a form of the fixed cap");
    constexpr int CAPS = ODD ? kCapFixedOdd : CAP;
    CapArgs ca{p.kx, p.ix};
    if (ODD) ca.half = 0.5f / p.ix;
    constexpr int NW = BLOCK / 64;
    __shared__ Stat1 red[NW];
    __shared__ float bc[2];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    RowStats* stats = static_cast<RowStats*>(p.stats);
    for (int64_t row = blockIdx.x; row < p.N; row += gridDim.x) {
        const S* __restrict__ x = static_cast<const S*>(p.x) + p.mx.offset(row);
        // This lane's first target slot, read now; its logit (if this shard
        // owns the column) is gathered once the walk's first group has
        // arrived (gather_first), behind the loads then in flight: gathered
        // here, its address would hold back the row's first loads by a
        // memory round trip.
        int64_t t0 = -1;
        float xt0 = 0.0f;
        if (HEAD == kHeadLogp && tid < p.k) t0 = p.targets[row * p.k + tid];
        bool gathered = HEAD != kHeadLogp;
        auto gather_first = [&]() {
            if (gathered) return;
            gathered = true;
            // (the empty asm keeps the address arithmetic here: hoisted out
            // of the walk, its wait for t0 held back the next group's loads)
            int64_t t = t0;
            __asm__ volatile("" : "+v"(t));
            if (tid < p.k && t >= p.v0 && t < p.v0 + p.V) xt0 = load_one(x + (t - p.v0));
        };
        Stat1 st = stat1_init<FIX>();
        if (ODD) st.mL = -ca.half;
        for_each_group<BLOCK, U, S, CAPS, ALIGNED, kFwdPipe, NT>(
            x, p.V, ca,
            [&](int64_t, bool full, const float (&a)[U][kChunk]) {
                gather_first();
                if (full)
                    update1<U, WITH_W, CLAMP, FIX>(st, a, p.scx);
                else
                    update1<U, WITH_W, WITH_W, FIX>(st, a, p.scx);
            });
        // The gathered logit is waited for here, where the walk's own loads
        // have arrived, and not at its use below, behind the record's store.
        if (HEAD == kHeadLogp) __asm__ volatile("" : "+v"(xt0));
        st = wave_reduce<WITH_W>(st);
        if (lane == 0) red[wid] = st;
        __syncthreads();
        Stat1 r{};
        if (wid == 0) r = waves_reduce<NW, WITH_W>(red, lane);
        if (tid == 0) {
            if (p.part) {
                static_cast<PartialRec*>(p.part)[row] = to_partial(r);
            } else {
                const RowStats rs = finalize1<WITH_W>(r);
                if (HEAD == kHeadEntropy) p.out[row] = rs.value;
                stats[row] = rs;
                bc[0] = rs.mLa;
                bc[1] = rs.log2Sa;
            }
        }
        __syncthreads();
        if (HEAD == kHeadLogp) {
            RowStats rs;
            rs.mLa = bc[0];
            rs.log2Sa = bc[1];
            if (p.k <= BLOCK) {
                // Every slot is a lane's prefetched first one: no load here,
                // hence no wait, which would also wait for the record's store
                // above (one counter covers loads and stores).
                if (tid < p.k) slot_out<CAP>(p, row, tid, t0, xt0, ca, rs);
            } else {
                // Slots beyond the prefetched first one, kTopkBatch per lane
                // at a time: their target loads are issued together, then
                // their gathers, so a lane waits twice per batch instead of
                // twice per slot.
                for (int64_t j0 = tid; j0 < p.k; j0 += static_cast<int64_t>(BLOCK) * kTopkBatch) {
                    int64_t t[kTopkBatch];
                    float xv[kTopkBatch];
#pragma unroll
                    for (int b = 0; b < kTopkBatch; ++b) {
                        const int64_t j = j0 + static_cast<int64_t>(b) * BLOCK;
                        t[b] = j == tid ? t0 : (j < p.k ? p.targets[row * p.k + j] : -1);
                    }
#pragma unroll
                    for (int b = 0; b < kTopkBatch; ++b) {
                        const int64_t j = j0 + static_cast<int64_t>(b) * BLOCK;
                        const bool local = t[b] >= p.v0 && t[b] < p.v0 + p.V;
                        xv[b] = j == tid ? xt0 : (local ? load_one(x + (t[b] - p.v0)) : 0.0f);
                    }
#pragma unroll
                    for (int b = 0; b < kTopkBatch; ++b) {
                        const int64_t j = j0 + static_cast<int64_t>(b) * BLOCK;
                        if (j >= p.k) break;
                        slot_out<CAP>(p, row, j, t[b], xv[b], ca, rs);
                    }
                }
            }
        }
        __syncthreads();
    }
}

// KL forward (either direction): one workgroup per row pair.
// Logprobs / entropy forward of 16-bit logits under the fixed-form cap.  A
// 16-bit logit has 2^15 magnitudes and t(x) + sc/2 is odd in x (tab_lookup),
// so a 128 KB LDS table of sc/2 + t(|x|), built once per workgroup, and the
// logit's sign bit give every statistic input, shifted by sc/2 (reference
// -sc/2), where the direct form spends an exponential, an FMA and a
// reciprocal per logit.  Every path of the row walk (full, tail and
// unaligned groups) reads the table, so a row's values do not depend on how
// it is laid out or batched.  The table fills a CU's LDS: one workgroup of
// kTabRows x BLOCK threads walks up to kTabRows rows side by side (rpw,
// fewer when N is small so that the rows still spread over the CUs), each
// row as fwd1_kernel walks it (its own BLOCK threads, waves and reduction),
// so the bits do not depend on rpw.  The targets' values keep the direct
// form (target_logp subtracts the record's reference).
template <int U, typename T, int HEAD, bool ALIGNED, bool NT>
__global__ __launch_bounds__(kTabRows* kBlock) void fwd1_tab_kernel(FwdParams p, int rpw) {
    constexpr int BLOCK = kBlock;
    using S = typename T::storage;
    static_assert(sizeof(S) == 2, "table forms read 16-bit logits");
    constexpr int TAB = std::is_same<S, uint16_t>::value ? kCapTableB : kCapTableH;
    constexpr bool WITH_W = HEAD == kHeadEntropy;
    constexpr int NW = BLOCK / 64;
    __shared__ float tab[kTabSize];
    __shared__ Stat1 red[kTabRows][NW];
    __shared__ float bc[kTabRows][2];
    const int sub = threadIdx.x / BLOCK, tid = threadIdx.x % BLOCK, lane = tid & 63,
              wid = tid >> 6;
    CapArgs cf{p.kx, p.ix};
    const float half = 0.5f / p.ix;
    cf.half = half;
    // Where 2^(-k |x|) overflows (nearly half of the bf16 magnitudes) the
    // direct form gives -1 / inf = -0 and the entry is exactly sc/2: those
    // entries skip the exponential and the reciprocal (same bits).
    for (int i = threadIdx.x; i < kTabSize; i += kTabRows * BLOCK) {
        const float v = from_bits16<S>(static_cast<uint32_t>(i));
        tab[i] = tab_entry(-(v * cf.k) >= 128.0f ? half : half + cap_value<kCapFixed>(v, cf));
    }
    CapArgs ct = cf;
    ct.tab = tab;
    __syncthreads();
    RowStats* stats = static_cast<RowStats*>(p.stats);
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * rpw; base < p.N;
         base += static_cast<int64_t>(gridDim.x) * rpw) {
        const int64_t row = base + sub;
        const bool live = sub < rpw && row < p.N;
        const S* __restrict__ x = static_cast<const S*>(p.x) + p.mx.offset(live ? row : 0);
        int64_t t0 = -1;
        float xt0 = 0.0f;
        if (live) {
            // (the target's logit is gathered behind the first group, as in
            // fwd1_kernel)
            if (HEAD == kHeadLogp && tid < p.k) t0 = p.targets[row * p.k + tid];
            bool gathered = HEAD != kHeadLogp;
            Stat1 st{0.0f, -half, 0.0f, 0.0f};
            for_each_group<BLOCK, U, S, TAB, ALIGNED, kFwdPipe, NT>(
                x, p.V, ct, [&](int64_t, bool full, const float (&a)[U][kChunk]) {
                    if (!gathered) {
                        gathered = true;
                        int64_t t = t0;
                        __asm__ volatile("" : "+v"(t));
                        if (tid < p.k && t >= p.v0 && t < p.v0 + p.V)
                            xt0 = load_one(x + (t - p.v0));
                    }
                    if (full)
                        update1<U, WITH_W, false, true>(st, a, p.scx);
                    else
                        update1<U, WITH_W, WITH_W, true>(st, a, p.scx);
                });
            if (HEAD == kHeadLogp) __asm__ volatile("" : "+v"(xt0));  // (as in fwd1_kernel)
            st = wave_reduce<WITH_W>(st);
            if (lane == 0) red[sub][wid] = st;
        }
        __syncthreads();
        Stat1 r{};
        if (live && wid == 0) r = waves_reduce<NW, WITH_W>(red[sub], lane);
        if (live && tid == 0) {
            if (p.part) {
                static_cast<PartialRec*>(p.part)[row] = to_partial(r);
            } else {
                const RowStats rs = finalize1<WITH_W>(r);
                if (HEAD == kHeadEntropy) p.out[row] = rs.value;
                stats[row] = rs;
                bc[sub][0] = rs.mLa;
                bc[sub][1] = rs.log2Sa;
            }
        }
        // Next pass: red[sub] is rewritten after this barrier, which its
        // readers (wave 0 of the row) pass after reading it; bc[sub] after the
        // next pass's first barrier, which its readers pass after reading it.
        __syncthreads();
        if (live && HEAD == kHeadLogp) {
            RowStats rs;
            rs.mLa = bc[sub][0];
            rs.log2Sa = bc[sub][1];
            if (p.k <= BLOCK) {
                // (as in fwd1_kernel: no load, no wait)
                if (tid < p.k) slot_out<kCapFixed>(p, row, tid, t0, xt0, cf, rs);
            } else {
                for (int64_t j0 = tid; j0 < p.k; j0 += static_cast<int64_t>(BLOCK) * kTopkBatch) {
                    int64_t t[kTopkBatch];
                    float xv[kTopkBatch];
#pragma unroll
                    for (int b = 0; b < kTopkBatch; ++b) {
                        const int64_t j = j0 + static_cast<int64_t>(b) * BLOCK;
                        t[b] = j == tid ? t0 : (j < p.k ? p.targets[row * p.k + j] : -1);
                    }
#pragma unroll
                    for (int b = 0; b < kTopkBatch; ++b) {
                        const int64_t j = j0 + static_cast<int64_t>(b) * BLOCK;
                        const bool local = t[b] >= p.v0 && t[b] < p.v0 + p.V;
                        xv[b] = j == tid ? xt0 : (local ? load_one(x + (t[b] - p.v0)) : 0.0f);
                    }
#pragma unroll
                    for (int b = 0; b < kTopkBatch; ++b) {
                        const int64_t j = j0 + static_cast<int64_t>(b) * BLOCK;
                        if (j >= p.k) break;
                        slot_out<kCapFixed>(p, row, j, t[b], xv[b], cf, rs);
                    }
                }
            }
        }
    }
}

template <int BLOCK, int U, typename T, bool REVERSE, int CAPA, int CAPB, bool ALIGNED, bool NT>
__global__ __launch_bounds__(BLOCK) RLK_OCCUPANCY void fwdkl_kernel(FwdParams p) {
    constexpr bool FIXA = CAPA == kCapFixed, FIXB = CAPB == kCapFixed;
    using S = typename T::storage;
    constexpr int NW = BLOCK / 64;
    __shared__ StatKL red[NW];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    RowStats* stats = static_cast<RowStats*>(p.stats);
    for (int64_t row = blockIdx.x; row < p.N; row += gridDim.x) {
        const S* __restrict__ xa = static_cast<const S*>(p.x) + p.mx.offset(row);
        const S* __restrict__ xb = static_cast<const S*>(p.y) + p.my.offset(row);
        StatKL st = statkl_init<REVERSE, FIXA, FIXB>();
        for_each_group2<BLOCK, U, S, CAPA, CAPB, ALIGNED, kFwdPipe, NT>(
            xa, xb, p.V, CapArgs{p.kx, p.ix}, CapArgs{p.ky, p.iy},
            [&](int64_t, bool, const float (&a)[U][kChunk], const float (&b)[U][kChunk]) {
                update_kl<U, REVERSE, FIXA, FIXB>(st, a, b, p.scx, p.scy);
            });
        st = wave_reduce_kl<REVERSE>(st);
        if (lane == 0) red[wid] = st;
        __syncthreads();
        StatKL r{};
        if (wid == 0) r = waves_reduce_kl<NW, REVERSE>(red, lane);
        if (tid == 0) {
            if (p.part) {
                static_cast<PartialRec*>(p.part)[row] = to_partial(r);
            } else {
                const RowStats rs = finalize_kl<REVERSE>(r);
                stats[row] = rs;
                p.out[row] = rs.value;
            }
        }
        __syncthreads();
    }
}

// Both KL directions from one read of the pair: reverse KL to out / stats,
// forward KL to out2 / stats2, each bit-identical to its one-direction call.
template <int BLOCK, int U, typename T, int CAPA, int CAPB, bool ALIGNED, bool NT>
__global__ __launch_bounds__(BLOCK) RLK_OCCUPANCY void fwdkl2_kernel(FwdParams p) {
    constexpr bool FIXA = CAPA == kCapFixed, FIXB = CAPB == kCapFixed;
    using S = typename T::storage;
    constexpr int NW = BLOCK / 64;
    __shared__ StatKL2 red[NW];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    RowStats* stats = static_cast<RowStats*>(p.stats);
    RowStats* stats2 = static_cast<RowStats*>(p.stats2);
    for (int64_t row = blockIdx.x; row < p.N; row += gridDim.x) {
        const S* __restrict__ xa = static_cast<const S*>(p.x) + p.mx.offset(row);
        const S* __restrict__ xb = static_cast<const S*>(p.y) + p.my.offset(row);
        StatKL2 st = statkl2_init<FIXA, FIXB>();
        for_each_group2<BLOCK, U, S, CAPA, CAPB, ALIGNED, kFwdPipe, NT>(
            xa, xb, p.V, CapArgs{p.kx, p.ix}, CapArgs{p.ky, p.iy},
            [&](int64_t, bool, const float (&a)[U][kChunk], const float (&b)[U][kChunk]) {
                update_kl2<U, FIXA, FIXB>(st, a, b, p.scx, p.scy);
            });
        st = wave_reduce_kl2(st);
        if (lane == 0) red[wid] = st;
        __syncthreads();
        StatKL2 r{};
        if (wid == 0) r = waves_reduce_kl2<NW>(red, lane);
        if (tid == 0) {
            const RowStats rr = finalize_kl<true>(kl_view_rev(r));
            const RowStats rf = finalize_kl<false>(kl_view_fwd(r));
            stats[row] = rr;
            p.out[row] = rr.value;
            stats2[row] = rf;
            p.out2[row] = rf.value;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------- dispatch

// Logprobs / entropy forward.  Under the fixed cap, rows of at least
// odd_form_min_cols(HEAD) columns take the odd form: 16-bit logits from the
// LDS table once there are kTabRows rows per CU, else (and fp32) computed;
// the two give the same bits, so the choice may follow N.  Which form a row
// takes depends on its width, head and cap only, never on N or its layout.
template <typename T, int HEAD, int CAP, bool AL, bool NT>
inline void fwd1_launch(const FwdParams& p, hipStream_t s) {
    const dim3 grid(row_grid(p.N)), block(kBlock);
    if constexpr (CAP == kCapFixed) {
        if (kUseCapTable && p.V >= odd_form_min_cols(HEAD)) {
            if constexpr (T::kBytes == 2) {
                if (p.N >= static_cast<int64_t>(kTabRows) * kTabGrid) {
                    // rows per workgroup: kTabRows once every CU has a row
                    const int64_t rpw64 = (p.N + kTabGrid - 1) / kTabGrid;
                    const int rpw = static_cast<int>(rpw64 < kTabRows ? rpw64 : kTabRows);
                    const int64_t wgs = (p.N + rpw - 1) / rpw;
                    hipLaunchKernelGGL((fwd1_tab_kernel<kUnroll1, T, HEAD, AL, NT>),
                                       dim3(static_cast<int>(wgs < kTabGrid ? wgs : kTabGrid)),
                                       dim3(kTabRows * kBlock), 0, s, p, rpw);
                    return;
                }
            }
            hipLaunchKernelGGL((fwd1_kernel<kBlock, kUnroll1, T, HEAD, CAP, AL, NT, true>), grid,
                               block, 0, s, p);
            return;
        }
    }
    hipLaunchKernelGGL((fwd1_kernel<kBlock, kUnroll1, T, HEAD, CAP, AL, NT>), grid, block, 0, s, p);
}

template <typename T, int CAPX, int CAPY, bool AL, bool NT>
inline hipError_t fwd_dispatch_head(int head, const FwdParams& p, hipStream_t s) {
    const dim3 grid(row_grid(p.N)), block(kBlock);
    switch (head) {
        case kHeadLogp:
            fwd1_launch<T, kHeadLogp, CAPX, AL, NT>(p, s);
            break;
        case kHeadEntropy:
            fwd1_launch<T, kHeadEntropy, CAPX, AL, NT>(p, s);
            break;
        case kHeadKLReverse:
            hipLaunchKernelGGL((fwdkl_kernel<kBlock, kUnrollKL, T, true, CAPX, CAPY, AL, NT>), grid,
                               block, 0, s, p);
            break;
        case kHeadKLForward:
            hipLaunchKernelGGL((fwdkl_kernel<kBlock, kUnrollKL, T, false, CAPX, CAPY, AL, NT>), grid,
                               block, 0, s, p);
            break;
        case kHeadKLBoth:
            hipLaunchKernelGGL((fwdkl2_kernel<kBlock, kUnrollKL, T, CAPX, CAPY, AL, NT>), grid, block,
                               0, s, p);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Rows that are not 16-byte aligned read every element with ordinary loads,
// so only aligned rows choose between streaming and cached loads.
template <typename T, int CAPX, int CAPY>
inline hipError_t fwd_dispatch_al(int head, bool al, const FwdParams& p, hipStream_t s) {
    if (!al) return fwd_dispatch_head<T, CAPX, CAPY, false, true>(head, p, s);
    const bool kl = head == kHeadKLReverse || head == kHeadKLForward || head == kHeadKLBoth;
    return stream_reads(p.N, p.V, T::kBytes, kl ? 2 : 1)
               ? fwd_dispatch_head<T, CAPX, CAPY, true, true>(head, p, s)
               : fwd_dispatch_head<T, CAPX, CAPY, true, false>(head, p, s);
}

template <typename T, int CAPX>
inline hipError_t fwd_dispatch_cy(int head, int cy, bool al, const FwdParams& p, hipStream_t s) {
    if (cy == kCapOnline) return fwd_dispatch_al<T, CAPX, kCapOnline>(head, al, p, s);
    if (cy == kCapFixed) return fwd_dispatch_al<T, CAPX, kCapFixed>(head, al, p, s);
    return fwd_dispatch_al<T, CAPX, kCapNone>(head, al, p, s);
}

template <typename T>
inline hipError_t fwd_dispatch_cap(int head, int cx, int cy, bool al, const FwdParams& p,
                                   hipStream_t s) {
    const bool kl = head == kHeadKLReverse || head == kHeadKLForward || head == kHeadKLBoth;
    if (!kl) cy = kCapNone;  // the second cap only exists for KL
    if (cx == kCapOnline) return fwd_dispatch_cy<T, kCapOnline>(head, cy, al, p, s);
    if (cx == kCapFixed) return fwd_dispatch_cy<T, kCapFixed>(head, cy, al, p, s);
    return fwd_dispatch_cy<T, kCapNone>(head, cy, al, p, s);
}

}  // namespace rlk
