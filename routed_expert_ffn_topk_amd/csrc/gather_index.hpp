// Gather index: the per-expert slot lists that drive the gather of HiNa-MoE
// §4.1 (each expert's routed tokens form one small matrix), as a stable
// counting sort of the n slots by expert id.  Device building blocks shared
// by the stand-alone index kernels and the gate/up product, which builds the
// index in its own prologue for decode-sized batches.
#pragma once

#include <climits>
#include <cstdint>

#include "common.hpp"

namespace moe {

constexpr int kMaxExperts = 1024;          // matches MOE_FFN_MAX_EXPERTS

struct GlobalIds {
    const int32_t* p;
    __device__ int operator()(int s) const { return p[s]; }
};
struct LdsIds {
    const int* p;
    __device__ int operator()(int s) const { return p[s]; }
};

// ---------------------------------------------------------------------------
// Gather index: stable counting sort of the n slots by expert.  Writes
// counts, offsets (exclusive prefix), the ascending lists of active experts
// (split by token count between the small-m and the tiled product), and
// sorted_slot (expert-major, slot order within an expert).  Slots with ids
// outside [0, E) are left out and counted in meta[1].
// ---------------------------------------------------------------------------

// The experts' offsets (exclusive scan of cnt[]) and lists, by wave 0 alone
// (each lane owns a run of up to 16 consecutive experts).  Experts with more
// than m_split slots go to the large list (the tiled product), the other
// active ones to the active list (the small-m product).  base[] receives the
// offsets.
__device__ __forceinline__ void scan_experts(const int* cnt, int E, int m_split, int nbad,
                                             int* base, int32_t* __restrict__ meta,
                                             int32_t* __restrict__ counts,
                                             int32_t* __restrict__ offsets,
                                             int32_t* __restrict__ active,
                                             int32_t* __restrict__ large) {
    const int lane = threadIdx.x;
    const int per = (E + kWave - 1) / kWave;
    const int e0 = min(E, lane * per), e1 = min(E, e0 + per);
    int lc = 0, la = 0, ll = 0;
    for (int e = e0; e < e1; ++e) {
        lc += cnt[e];
        la += cnt[e] > 0 && cnt[e] <= m_split;
        ll += cnt[e] > m_split;
    }
    const int ic = wave_prefix_sum_i32(lc);
    const int ia = wave_prefix_sum_i32(la);
    const int il = wave_prefix_sum_i32(ll);
    int bc = ic - lc, ba = ia - la, bl = il - ll;
    for (int e = e0; e < e1; ++e) {
        base[e] = bc;
        offsets[e] = bc;
        counts[e] = cnt[e];
        if (cnt[e] > m_split)
            large[bl++] = e;
        else if (cnt[e] > 0)
            active[ba++] = e;
        bc += cnt[e];
    }
    if (lane == kWave - 1) {
        offsets[E] = ic;
        meta[0] = ia;
        meta[1] = nbad;
        meta[2] = il;
    }
}

// Per-expert counts of the n slots (all NT threads), then scan_experts.
// Ends with a barrier.
template <int NT, class Ids>
__device__ __forceinline__ void count_and_scan(Ids ids, int n, int E, int m_split, int* cnt,
                                               int* base, int* nbad, int32_t* __restrict__ meta,
                                               int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ active,
                                               int32_t* __restrict__ large) {
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += NT) cnt[e] = 0;
    if (tid == 0) *nbad = 0;
    __syncthreads();
    for (int s = tid; s < n; s += NT) {
        const int e = ids(s);
        if (e >= 0 && e < E)
            atomicAdd(&cnt[e], 1);
        else
            atomicAdd(nbad, 1);
    }
    __syncthreads();
    if (tid < kWave) scan_experts(cnt, E, m_split, *nbad, base, meta, counts, offsets, active, large);
    __syncthreads();
}

// Stable scatter of slots [s0, s1) by one wave, 64 at a time (the next
// chunk's ids are requested before this one is placed): a slot's place is
// run[e] (its expert's offset plus the slots of that expert placed before
// this chunk) plus the lanes below it in this chunk with the same expert.
// Lanes with equal ids are found bit by bit with ballots; the last lane of
// each group advances run[e] (LDS operations of one wave complete in order).
template <class Ids>
__device__ __forceinline__ void scatter_range(Ids ids, int s0, int s1, int E, int* run,
                                              int32_t* __restrict__ sorted_slot) {
    const int lane = threadIdx.x & (kWave - 1);
    int e_next = s0 + lane < s1 ? ids(s0 + lane) : -1;
    for (int c0 = s0; c0 < s1; c0 += kWave) {
        const int s = c0 + lane;
        const int e = e_next;
        const int sn = s + kWave;
        e_next = sn < s1 ? ids(sn) : -1;
        const bool ok = s < s1 && e >= 0 && e < E;
        const int key = ok ? e : kMaxExperts;   // every dropped slot in one group
        unsigned long long eq = ~0ull;
#pragma unroll
        for (int b = 0; b < 11; ++b) {          // ids < 2048
            const bool bit = (key >> b) & 1;
            const unsigned long long m = __ballot(bit);
            eq &= bit ? m : ~m;
        }
        const int below = __builtin_amdgcn_mbcnt_hi(
            (unsigned)(eq >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)eq, 0u));
        const int group = __popcll(eq);
        int pos = 0;
        if (ok) pos = run[e] + below;
        if (ok) sorted_slot[pos] = s;
        if (ok && below == group - 1) run[e] = pos + 1;
    }
}

// ---------------------------------------------------------------------------
// The index built inside a consumer kernel's prologue (decode-sized batches:
// at most kFusedMaxSlots slots over at most kFusedMaxExperts experts, every
// active expert on the small-m list).  Every workgroup builds the same index
// into its own LDS (the algorithm is deterministic), so no workgroup waits for
// another; one of them also publishes it to global memory for the kernels
// that follow (the down product, the status query).
// ---------------------------------------------------------------------------
constexpr int kFusedMaxSlots = 256;
constexpr int kFusedMaxExperts = 256;
// LDS copy of the index, in ints: offsets [E+1], active [E], sorted_slot
// [n], meta [3] (as the global meta)
constexpr int kFxOffsets = 0;
constexpr int kFxActive = kFusedMaxExperts + 4;
constexpr int kFxSorted = kFxActive + kFusedMaxExperts;
constexpr int kFxMeta = kFxSorted + kFusedMaxSlots;
constexpr int kFxInts = kFxMeta + 4;
// LDS scratch of the build, in ints (free again once it returns): per-expert
// counts, the runs of the scatter, the counts' copy, the staged ids, the
// dropped-slot count
constexpr int kFxScratchInts = 3 * kFusedMaxExperts + kFusedMaxSlots + 1;

// Global-memory destination of the published index.
struct IndexOut {
    int32_t* meta;
    int32_t* counts;
    int32_t* offsets;
    int32_t* active;
    int32_t* sorted_slot;
};

// Builds the index of the n slots ids[0..n) into ix (kFxInts ints of LDS)
// with all NT threads of the workgroup; tmp: kFxScratchInts ints of LDS.
// publish: also write it to out.  Returns the active-expert count; ends with
// a barrier, after which tmp is no longer read.
template <int NT>
__device__ __forceinline__ int build_index_lds(const int32_t* __restrict__ ids, int n, int E,
                                               int* tmp, int* ix, bool publish,
                                               const IndexOut& out) {
    int* cnt = tmp;
    int* run = tmp + kFusedMaxExperts;
    int* counts = tmp + 2 * kFusedMaxExperts;
    int* sid = tmp + 3 * kFusedMaxExperts;
    int* nbad = sid + kFusedMaxSlots;
    const int tid = threadIdx.x;
    for (int s = tid; s < n; s += NT) sid[s] = ids[s];
    count_and_scan<NT>(LdsIds{sid}, n, E, INT_MAX, cnt, run, nbad, ix + kFxMeta, counts,
                       ix + kFxOffsets, ix + kFxActive, nullptr);
    if (publish) {
        const int n_act = ix[kFxMeta];
        for (int e = tid; e < E; e += NT) {
            out.counts[e] = counts[e];
            out.offsets[e] = ix[kFxOffsets + e];
        }
        for (int a = tid; a < n_act; a += NT) out.active[a] = ix[kFxActive + a];
        if (tid < 3) out.meta[tid] = ix[kFxMeta + tid];
        if (tid == 0) out.offsets[E] = ix[kFxOffsets + E];
    }
    if (tid < kWave) scatter_range(LdsIds{sid}, 0, n, E, run, ix + kFxSorted);
    __syncthreads();
    if (publish) {
        const int placed = ix[kFxOffsets + E];
        for (int p = tid; p < placed; p += NT) out.sorted_slot[p] = ix[kFxSorted + p];
    }
    return ix[kFxMeta];
}

}  // namespace moe
