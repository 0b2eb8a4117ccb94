// Routing and gather-index kernels.
//
// route_topk:    the top-k gate of HiNa-MoE §2.1 / Fig. 2 (k per Table 3).
// permute:       the per-expert token lists that drive the gather of §4.1
//                (each expert's routed tokens form one small matrix).
// route_permute: both in one workgroup, for decode-sized batches.
// route_grouped: the grouped sigmoid gate (selection bias, group-limited
//                top-k, scaled weights).
#include <cmath>

#include "common.hpp"
#include "gather_index.hpp"
#include "launch.hpp"

namespace moe {

namespace {

// The fused router + gather index: batches of at most this many tokens and
// slots (16 waves route up to four tokens each; one wave places the slots),
// with the logits staged in LDS when the batch's T*E fits.
constexpr int kRoutePermMaxTokens = 64;
constexpr int kRoutePermMaxSlots = 512;
constexpr int kRoutePermMaxLogits = 16384;

// Order-preserving integer key of a float (not NaN): keys compare as the
// values do, and -0 is mapped to +0 so that the two tie.  INT_MIN is the key
// of no float (it would be a NaN pattern) and marks "no candidate".
__device__ __forceinline__ int route_key(float f) {
    const int b = __builtin_bit_cast(int, f + 0.0f);
    return b >= 0 ? b : b ^ 0x7fffffff;
}
__device__ __forceinline__ float route_key_value(int key) {
    return __builtin_bit_cast(float, key >= 0 ? key : key ^ 0x7fffffff);
}

// Routes one token with one wave (all 64 lanes active).  Lane l holds the
// logits of experts l, l+64, ..., l+64(PL-1); k rounds each pick the
// remaining expert with the largest logit (ties: the lower id) with a
// wave-wide max over the keys, then a wave-wide min over the ids holding
// that key.  The weights are exp(l_j - l_max) / sum over the chosen of
// exp(l_i - l_max): the softmax over all E experts renormalised over the
// chosen ones (the common denominator cancels).  Lane j < k returns the
// j-th choice in (*id, *wt); the other lanes return id -1, weight 0.
template <int PL>
__device__ __forceinline__ void route_token(const float* __restrict__ l, int E, int k,
                                            int lane, int* id, float* wt) {
    int key[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int e = lane + kWave * i;
        key[i] = e < E ? route_key(l[e]) : INT_MIN;
    }
    int my_key = INT_MIN;
    int my_e = -1;
    int top_key = INT_MIN;
    for (int j = 0; j < k; ++j) {
        // this lane's best candidate: largest key, then lowest expert id
        int bk = INT_MIN, be = INT_MAX;
#pragma unroll
        for (int i = 0; i < PL; ++i)
            if (key[i] > bk) {
                bk = key[i];
                be = lane + kWave * i;
            }
        const int K = wave_max_i32(bk);
        const int W = wave_min_i32(bk == K ? be : INT_MAX);
        if (j == 0) top_key = K;
        if (lane == j) {
            my_key = K;
            my_e = W;
        }
#pragma unroll
        for (int i = 0; i < PL; ++i)
            if (lane + kWave * i == W) key[i] = INT_MIN;
    }
    const float mx = route_key_value(top_key);
    const float ex = lane < k ? expf(route_key_value(my_key) - mx) : 0.0f;
    const float sum = wave_sum_f32(ex);
    *id = lane < k ? my_e : -1;
    *wt = lane < k ? ex / sum : 0.0f;
}

// route_token for the expert count E (the candidates per lane are a
// compile-time count).
__device__ __forceinline__ void route_token_any(const float* __restrict__ l, int E, int k,
                                                int lane, int* id, float* wt) {
    if (E <= 64)
        route_token<1>(l, E, k, lane, id, wt);
    else if (E <= 128)
        route_token<2>(l, E, k, lane, id, wt);
    else if (E <= 256)
        route_token<4>(l, E, k, lane, id, wt);
    else if (E <= 512)
        route_token<8>(l, E, k, lane, id, wt);
    else
        route_token<16>(l, E, k, lane, id, wt);
}

// One wave per token.
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int T, int E, int k,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    if (t >= T) return;
    int id;
    float wt;
    route_token_any(logits + (size_t)t * E, E, k, lane, &id, &wt);
    if (lane < k) {
        ids[(size_t)t * k + lane] = id;
        w[(size_t)t * k + lane] = wt;
    }
}

// ---------------------------------------------------------------------------
// Grouped sigmoid routing (the gate of DeepSeek-V3, one of the models of the
// pages' evaluation, whose gate they do not spell out): sigmoid scores s,
// selection scores c = s + bias, the experts in n_group groups of G
// consecutive ids scored by the sum of their two largest c, the topk_group
// best groups kept, the k best experts of those by c, and weights
// scale * s_j / sum_j s_j.  Ties go to the lower group and the lower id.
// ---------------------------------------------------------------------------

// One token with one wave.  Lane l holds experts l, l + 64, ...; the
// selection scores also go to this wave's LDS row (cw), where lane g < n_group
// reads its group's G scores.  Lane j < k returns the j-th choice.
template <int PL>
__device__ __forceinline__ void route_token_grouped(const float* __restrict__ l,
                                                    const float* __restrict__ bias, int E,
                                                    int n_group, int topk_group, int k,
                                                    float scale, int lane, float* cw, int* id,
                                                    float* wt) {
    const int G = E / n_group;
    float sv[PL];
    int key[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int e = lane + kWave * i;
        sv[i] = 0.0f;
        key[i] = INT_MIN;
        if (e < E) {
            sv[i] = 1.0f / (1.0f + expf(-l[e]));
            const float c = sv[i] + (bias ? bias[e] : 0.0f);
            key[i] = route_key(c);
            cw[e] = c;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // group scores: the largest selection score of the group plus the second
    int gkey = INT_MIN;
    if (lane < n_group) {
        float b1 = -INFINITY, b2 = -INFINITY;
        for (int e = lane * G; e < (lane + 1) * G; ++e) {
            const float c = cw[e];
            if (c > b1) {
                b2 = b1;
                b1 = c;
            } else if (c > b2) {
                b2 = c;
            }
        }
        gkey = route_key(G > 1 ? b1 + b2 : b1);
    }
    // the topk_group best groups (uniform bit mask)
    uint64_t kept = 0;
    for (int j = 0; j < topk_group; ++j) {
        const int K = wave_max_i32(gkey);
        const int W = wave_min_i32(gkey == K ? lane : INT_MAX);
        kept |= 1ull << W;
        if (lane == W) gkey = INT_MIN;
    }
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int e = lane + kWave * i;
        if (e < E && !((kept >> (e / G)) & 1ull)) key[i] = INT_MIN;
    }
    // k rounds over the kept experts: largest c, then lowest id
    float my_s = 0.0f;
    int my_e = -1;
    for (int j = 0; j < k; ++j) {
        int bk = INT_MIN, be = INT_MAX;
        float bs = 0.0f;
#pragma unroll
        for (int i = 0; i < PL; ++i)
            if (key[i] > bk) {
                bk = key[i];
                be = lane + kWave * i;
                bs = sv[i];
            }
        const int K = wave_max_i32(bk);
        const int W = wave_min_i32(bk == K ? be : INT_MAX);
        const float sW = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bs), W & (kWave - 1)));
        if (lane == j) {
            my_e = W;
            my_s = sW;
        }
#pragma unroll
        for (int i = 0; i < PL; ++i)
            if (lane + kWave * i == W) key[i] = INT_MIN;
    }
    // the sum of the chosen sigmoids in ascending slot order
    float sum = 0.0f;
    for (int j = 0; j < k; ++j)
        sum += __builtin_bit_cast(float,
                                  __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_s), j));
    *id = lane < k ? my_e : -1;
    *wt = lane < k ? my_s / sum * scale : 0.0f;
}

// Four tokens per 256-thread workgroup, one wave each.
__global__ __launch_bounds__(256) void route_grouped_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int n_group,
    int topk_group, int k, float scale, int32_t* __restrict__ ids, float* __restrict__ w) {
    __shared__ float cs[4][kMaxExperts];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;
    const float* l = logits + (size_t)t * E;
    int id;
    float wt;
    if (E <= 64)
        route_token_grouped<1>(l, bias, E, n_group, topk_group, k, scale, lane, cs[wv], &id, &wt);
    else if (E <= 128)
        route_token_grouped<2>(l, bias, E, n_group, topk_group, k, scale, lane, cs[wv], &id, &wt);
    else if (E <= 256)
        route_token_grouped<4>(l, bias, E, n_group, topk_group, k, scale, lane, cs[wv], &id, &wt);
    else if (E <= 512)
        route_token_grouped<8>(l, bias, E, n_group, topk_group, k, scale, lane, cs[wv], &id, &wt);
    else
        route_token_grouped<16>(l, bias, E, n_group, topk_group, k, scale, lane, cs[wv], &id,
                                &wt);
    if (lane < k) {
        ids[(size_t)t * k + lane] = id;
        w[(size_t)t * k + lane] = wt;
    }
}

// Batches up to this many slots: ids staged in LDS, counted by the 256
// threads of permute_kernel, placed by one wave.  Larger batches
// (permute_large_kernel, 16 waves): every wave counts, then places, a
// contiguous range of slots, starting from the slots of each expert in the
// ranges before it.
constexpr int kOneWaveSlots = 512;
constexpr int kPermThreads = 256;
constexpr int kPermLargeThreads = 1024;
constexpr int kPermWaves = kPermLargeThreads / kWave;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ ids, int n, int E, int m_split, int32_t* __restrict__ meta,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ active, int32_t* __restrict__ large,
    int32_t* __restrict__ sorted_slot) {
    __shared__ int cnt[kMaxExperts];
    __shared__ int base[kMaxExperts];
    __shared__ int sid[kOneWaveSlots];
    __shared__ int nbad;
    for (int s = threadIdx.x; s < n; s += kPermThreads) sid[s] = ids[s];
    __syncthreads();
    count_and_scan<kPermThreads>(LdsIds{sid}, n, E, m_split, cnt, base, &nbad, meta, counts,
                                 offsets, active, large);
    if (threadIdx.x < kWave) scatter_range(LdsIds{sid}, 0, n, E, base, sorted_slot);
}

__global__ __launch_bounds__(kPermLargeThreads) void permute_large_kernel(
    const int32_t* __restrict__ ids, int n, int E, int m_split, int32_t* __restrict__ meta,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ active, int32_t* __restrict__ large,
    int32_t* __restrict__ sorted_slot) {
    __shared__ int cnt[kMaxExperts];
    __shared__ int base[kMaxExperts];
    __shared__ int hist[kPermWaves * kMaxExperts];   // per-wave counts, then runs
    __shared__ int nbad_w[kPermWaves];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    int* my = hist + wave * kMaxExperts;
    for (int i = tid; i < kPermWaves * kMaxExperts; i += kPermLargeThreads) hist[i] = 0;
    __syncthreads();
    const int s0 = (int)((long long)n * wave / kPermWaves);
    const int s1 = (int)((long long)n * (wave + 1) / kPermWaves);
    int bad = 0;
    for (int c0 = s0; c0 < s1; c0 += 4 * kWave) {
        int ev[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int s = c0 + u * kWave + lane;
            ev[u] = s < s1 ? ids[s] : 0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int s = c0 + u * kWave + lane;
            if (s >= s1) continue;
            if (ev[u] >= 0 && ev[u] < E)
                atomicAdd(&my[ev[u]], 1);
            else
                ++bad;
        }
    }
    bad = wave_prefix_sum_i32(bad);
    if (lane == kWave - 1) nbad_w[wave] = bad;
    __syncthreads();
    // totals, and each wave's start within its expert's slots
    for (int e = tid; e < E; e += kPermLargeThreads) {
        int c = 0;
        for (int w = 0; w < kPermWaves; ++w) {
            const int h = hist[w * kMaxExperts + e];
            hist[w * kMaxExperts + e] = c;
            c += h;
        }
        cnt[e] = c;
    }
    __syncthreads();
    if (tid < kWave) {
        int nb = 0;
        for (int w = 0; w < kPermWaves; ++w) nb += nbad_w[w];
        scan_experts(cnt, E, m_split, nb, base, meta, counts, offsets, active, large);
    }
    __syncthreads();
    for (int i = tid; i < kPermWaves * E; i += kPermLargeThreads) {
        const int w = i / E, e = i - w * E;
        hist[w * kMaxExperts + e] += base[e];
    }
    __syncthreads();
    scatter_range(GlobalIds{ids}, s0, s1, E, my, sorted_slot);
}

// Router and gather index in one workgroup (decode-sized batches).  The
// batch's logits are first staged in LDS by all threads at once (one memory
// latency instead of one per token and wave) when T*E fits; each wave then
// routes tokens wave, wave + 16, ...; the chosen ids go to the caller's
// topk_ids / topk_w and to LDS, and the gather index reads them from LDS.
// One launch instead of two, with no round trip through memory.
constexpr int kRoutePermThreads = 1024;

__global__ __launch_bounds__(kRoutePermThreads) void route_permute_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ w, int32_t* __restrict__ meta, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ active, int32_t* __restrict__ large,
    int32_t* __restrict__ sorted_slot) {
    __shared__ float slg[kRoutePermMaxLogits];
    __shared__ int sid[kRoutePermMaxSlots];
    __shared__ int cnt[kMaxExperts];
    __shared__ int base[kMaxExperts];
    __shared__ int nbad;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int n_logits = T * E;
    const bool staged = n_logits <= kRoutePermMaxLogits;
    if (staged) {
        for (int i = threadIdx.x; i < n_logits; i += kRoutePermThreads) slg[i] = logits[i];
        __syncthreads();
    }
    const float* src = staged ? slg : logits;
    for (int t = wave; t < T; t += kRoutePermThreads / kWave) {
        int id;
        float wt;
        route_token_any(src + (size_t)t * E, E, k, lane, &id, &wt);
        if (lane < k) {
            ids[(size_t)t * k + lane] = id;
            w[(size_t)t * k + lane] = wt;
            sid[t * k + lane] = id;
        }
    }
    __syncthreads();
    const int n = T * k;
    // decode-sized batches: every expert goes to the small-m product
    count_and_scan<kRoutePermThreads>(LdsIds{sid}, n, E, INT_MAX, cnt, base, &nbad, meta,
                                      counts, offsets, active, large);
    if (threadIdx.x < kWave) scatter_range(LdsIds{sid}, 0, n, E, base, sorted_slot);
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

hipError_t launch_route_grouped(const float* logits, const float* bias, int T, int E,
                               int n_group, int topk_group, int k, float scale, int32_t* ids,
                               float* w, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int grid = (T + 3) / 4;
    hipLaunchKernelGGL(route_grouped_kernel, dim3(grid), dim3(256), 0, stream, logits, bias, T,
                       E, n_group, topk_group, k, scale, ids, w);
    return hipGetLastError();
}

hipError_t launch_route_permute(const float* logits, int32_t* ids, float* w,
                                const FfnShape& s, const Workspace& ws, int m_split,
                                hipStream_t stream) {
    if (s.T > kRoutePermMaxTokens || (int64_t)s.T * s.k > kRoutePermMaxSlots ||
        m_split != INT_MAX) {
        // larger batches: the router on one wave per token, then the sort
        hipError_t err = launch_route_topk(logits, s.T, s.E, s.k, ids, w, stream);
        return err == hipSuccess ? launch_permute(ids, s, ws, m_split, stream) : err;
    }
    hipLaunchKernelGGL(route_permute_kernel, dim3(1), dim3(kRoutePermThreads), 0, stream,
                       logits, s.T, s.E, s.k, ids, w, ws.meta, ws.counts, ws.offsets,
                       ws.active, ws.large, ws.sorted_slot);
    return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, const FfnShape& s, const Workspace& ws,
                          int m_split, hipStream_t stream) {
    const int n = s.T * s.k;
    if (n <= kOneWaveSlots)
        hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, stream, ids, n, s.E,
                           m_split, ws.meta, ws.counts, ws.offsets, ws.active, ws.large,
                           ws.sorted_slot);
    else
        hipLaunchKernelGGL(permute_large_kernel, dim3(1), dim3(kPermLargeThreads), 0, stream,
                           ids, n, s.E, m_split, ws.meta, ws.counts, ws.offsets, ws.active,
                           ws.large, ws.sorted_slot);
    return hipGetLastError();
}

MOE_DEVICE_CHECK_READER(route_permute)

}  // namespace moe
