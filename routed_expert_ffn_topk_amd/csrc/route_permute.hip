// Routing and gather-index kernels.
//
// route_topk: the top-k gate of HiNa-MoE §2.1 / Fig. 2 (k per Table 3).
// permute:    the per-expert token lists that drive the gather of §4.1
//             (each expert's routed tokens form one small matrix).
#include <climits>
#include <cmath>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kMaxExperts = 1024;          // matches MOE_FFN_MAX_EXPERTS
constexpr int kPerLane = kMaxExperts / kWave;

// (value, expert) ordering of the router: larger logit first, then lower id.
// e == INT_MAX marks "no candidate", which loses to everything.
__device__ __forceinline__ bool route_better(float va, int ea, float vb, int eb) {
    if (ea == INT_MAX) return false;
    if (eb == INT_MAX) return true;
    return va > vb || (va == vb && ea < eb);
}

// One wave per token.  Lane l holds logits l, l+64, l+128, ...; k rounds of
// a wave-wide arg-max pick the experts in descending order.  The weights are
// exp(l_j - l_max) / sum over the chosen of exp(l_i - l_max): the softmax
// over all E experts renormalised over the chosen ones, with the common
// denominator cancelled.
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int T, int E, int k,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    if (t >= T) return;
    const float* l = logits + (size_t)t * E;
    float v[kPerLane];
    unsigned taken = 0;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int e = lane + kWave * i;
        v[i] = e < E ? l[e] : -INFINITY;
        if (e >= E) taken |= 1u << i;
    }
    float my_v = -INFINITY;
    int my_e = -1;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int be = INT_MAX;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            // candidates of one lane come in ascending expert order, so a
            // strict comparison keeps the lower id on ties
            if (!((taken >> i) & 1u) && (be == INT_MAX || v[i] > bv)) {
                bv = v[i];
                be = lane + kWave * i;
            }
        }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, kWave);
            const int oe = __shfl_xor(be, off, kWave);
            if (route_better(ov, oe, bv, be)) {
                bv = ov;
                be = oe;
            }
        }
        if (lane == j) {
            my_v = bv;
            my_e = be;
        }
        if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
    }
    const float mx = __shfl(my_v, 0, kWave);
    const float ex = lane < k ? expf(my_v - mx) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_e;
        w[(size_t)t * k + lane] = ex / sum;
    }
}

// Stable counting sort of the T*k slots by expert, in one workgroup.
// Writes counts, offsets (exclusive prefix), the ascending list of active
// experts, and sorted_slot (expert-major, slot order within an expert).
// Slots with ids outside [0, E) are left out and counted in meta[1].
constexpr int kPermThreads = 256;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ ids, int n_slots, int E, int32_t* __restrict__ meta,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ active, int32_t* __restrict__ sorted_slot) {
    __shared__ int cnt[kMaxExperts];
    __shared__ int base[kMaxExperts];
    __shared__ int run[kMaxExperts];
    __shared__ int scan_c[kPermThreads];
    __shared__ int scan_a[kPermThreads];
    __shared__ int chunk_e[kPermThreads];
    __shared__ int nbad;
    const int tid = threadIdx.x;

    for (int e = tid; e < E; e += kPermThreads) {
        cnt[e] = 0;
        run[e] = 0;
    }
    if (tid == 0) nbad = 0;
    __syncthreads();
    for (int s = tid; s < n_slots; s += kPermThreads) {
        const int e = ids[s];
        if (e >= 0 && e < E)
            atomicAdd(&cnt[e], 1);
        else
            atomicAdd(&nbad, 1);
    }
    __syncthreads();

    // Each thread owns a run of consecutive experts; scan the per-thread
    // totals of slots and of active experts across the workgroup.
    const int per = (E + kPermThreads - 1) / kPermThreads;
    const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
    int lc = 0, la = 0;
    for (int e = e0; e < e1; ++e) {
        lc += cnt[e];
        la += cnt[e] > 0;
    }
    scan_c[tid] = lc;
    scan_a[tid] = la;
    __syncthreads();
    for (int d = 1; d < kPermThreads; d <<= 1) {
        const int vc = tid >= d ? scan_c[tid - d] : 0;
        const int va = tid >= d ? scan_a[tid - d] : 0;
        __syncthreads();
        scan_c[tid] += vc;
        scan_a[tid] += va;
        __syncthreads();
    }
    int bc = scan_c[tid] - lc;
    int ba = scan_a[tid] - la;
    for (int e = e0; e < e1; ++e) {
        base[e] = bc;
        offsets[e] = bc;
        counts[e] = cnt[e];
        if (cnt[e] > 0) active[ba++] = e;
        bc += cnt[e];
    }
    if (tid == kPermThreads - 1) {
        offsets[E] = scan_c[kPermThreads - 1];
        meta[0] = scan_a[kPermThreads - 1];
        meta[1] = nbad;
    }
    __syncthreads();

    // Stable scatter, one chunk of slots at a time: a slot's place is its
    // expert's base, plus the slots of that expert in earlier chunks, plus
    // the earlier slots of that expert in this chunk.
    for (int c0 = 0; c0 < n_slots; c0 += kPermThreads) {
        const int s = c0 + tid;
        const int e = s < n_slots ? ids[s] : -1;
        const bool ok = e >= 0 && e < E;
        chunk_e[tid] = ok ? e : -1;
        __syncthreads();
        if (ok) {
            int rank = 0;
            for (int j = 0; j < tid; ++j) rank += chunk_e[j] == e;
            sorted_slot[base[e] + run[e] + rank] = s;
        }
        __syncthreads();
        if (ok) atomicAdd(&run[e], 1);
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids,
                             float* w, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int tokens_per_block = 256 / kWave;
    const int grid = (T + tokens_per_block - 1) / tokens_per_block;
    hipLaunchKernelGGL(route_topk_kernel, dim3(grid), dim3(256), 0, stream, logits, T, E,
                       k, ids, w);
    return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, const FfnShape& s, const Workspace& ws,
                          hipStream_t stream) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, stream, ids,
                       s.T * s.k, s.E, ws.meta, ws.counts, ws.offsets, ws.active,
                       ws.sorted_slot);
    return hipGetLastError();
}

}  // namespace moe
