// C ABI of the routed-expert MoE FFN library: argument checks, workspace
// layout and kernel launches on the caller's stream.  The declarations and
// their contracts are in include/moe_ffn.h.
#include "../../include/moe_ffn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "launch.hpp"

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool shape_ok(int64_t T, int64_t H, int64_t I, int32_t E, int32_t top_k) {
    if (T < 0 || H < 1 || I < 1) return false;
    if (E < 1 || E > MOE_FFN_MAX_EXPERTS) return false;
    if (top_k < 1 || top_k > E) return false;
    if (T * (int64_t)top_k >= ((int64_t)1 << 31)) return false;
    if (H >= ((int64_t)1 << 30) || I >= ((int64_t)1 << 30)) return false;
    return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

std::atomic<int> g_num_cu[kMaxDevices];

// Benchmark hook (moe_ffn_set_stage_events): consumed by the next forward
// call of this thread.
thread_local moe::StageEvents t_stage_events = {{nullptr, nullptr, nullptr, nullptr}, 0};

// Test hook (moe_ffn_set_split): K splits forced on this thread's calls.
thread_local moe::SplitOverride t_split;

moe::StageEvents take_stage_events() {
    const moe::StageEvents ev = t_stage_events;
    t_stage_events.n = 0;
    return ev;
}

// Compute units of the current device (cached; the persistent grids are
// sized from it).
int num_cu(int* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_FFN_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) {
        const int cached = g_num_cu[dev].load(std::memory_order_relaxed);
        if (cached > 0) {
            *out = cached;
            return MOE_FFN_OK;
        }
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        return MOE_FFN_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) g_num_cu[dev].store(n, std::memory_order_relaxed);
    *out = n;
    return MOE_FFN_OK;
}

moe::Workspace carve(void* base, const moe_ffn_ws_layout& L) {
    char* b = static_cast<char*>(base);
    moe::Workspace ws;
    ws.meta = reinterpret_cast<int32_t*>(b + L.meta);
    ws.counts = reinterpret_cast<int32_t*>(b + L.counts);
    ws.offsets = reinterpret_cast<int32_t*>(b + L.offsets);
    ws.active = reinterpret_cast<int32_t*>(b + L.active);
    ws.large = reinterpret_cast<int32_t*>(b + L.large);
    ws.sorted_slot = reinterpret_cast<int32_t*>(b + L.sorted_slot);
    ws.h = reinterpret_cast<uint16_t*>(b + L.h);
    ws.y = reinterpret_cast<float*>(b + L.y);
    return ws;
}

// Checks common to both weight formats.
int check_forward(const void* x, const int32_t* ids, const float* w, const void* out,
                  int64_t T, int64_t H, int64_t I, int32_t E, int32_t top_k,
                  const void* workspace, size_t workspace_bytes, int64_t k_multiple,
                  moe_ffn_ws_layout* L) {
    if (!shape_ok(T, H, I, E, top_k)) return MOE_FFN_ERR_BAD_SHAPE;
    if (H % k_multiple != 0 || I % k_multiple != 0) return MOE_FFN_ERR_BAD_SHAPE;
    if (T == 0) return MOE_FFN_OK;
    if (!x || !ids || !w || !out) return MOE_FFN_ERR_NULL_ARG;
    if (!workspace) return MOE_FFN_ERR_WORKSPACE;
    if (!aligned16(x) || !aligned16(out)) return MOE_FFN_ERR_MISALIGNED;
    if ((reinterpret_cast<uintptr_t>(ids) & 3u) || (reinterpret_cast<uintptr_t>(w) & 3u))
        return MOE_FFN_ERR_MISALIGNED;
    const size_t xb = (size_t)T * (size_t)H * 2;
    if (overlap(x, xb, out, xb)) return MOE_FFN_ERR_ALIAS;
    const size_t sb = (size_t)T * (size_t)top_k * 4;
    if (overlap(ids, sb, out, xb) || overlap(w, sb, out, xb)) return MOE_FFN_ERR_ALIAS;
    if (moe_ffn_workspace_layout(T, H, I, E, top_k, L) != MOE_FFN_OK) return MOE_FFN_ERR_BAD_SHAPE;
    if (workspace_bytes < L->total_bytes) return MOE_FFN_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return MOE_FFN_ERR_MISALIGNED;
    if (overlap(workspace, L->total_bytes, out, xb) || overlap(workspace, L->total_bytes, x, xb))
        return MOE_FFN_ERR_ALIAS;
    return MOE_FFN_OK;
}

// Workspace of moe_ffn_forward_noalloc: a device array the library holds on
// every GPU it runs on, until the process ends.  In host code `scratch` only
// names the symbol; its device address (one per GPU) comes from
// hipGetSymbolAddress, and only that address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_FFN_NOALLOC_WORKSPACE_BYTES];

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and cached.
int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_FFN_ERR_HIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return MOE_FFN_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MOE_FFN_OK;
}

}  // namespace

extern "C" {

int moe_ffn_workspace_layout(int64_t T, int64_t H, int64_t I, int32_t E, int32_t top_k,
                             moe_ffn_ws_layout* layout) {
    if (!layout) return MOE_FFN_ERR_NULL_ARG;
    if (!shape_ok(T, H, I, E, top_k)) return MOE_FFN_ERR_BAD_SHAPE;
    const size_t S = (size_t)T * (size_t)top_k;
    size_t off = 0;
    layout->meta = off;
    off += round_up(8 * sizeof(int32_t));
    layout->counts = off;
    off += round_up((size_t)E * sizeof(int32_t));
    layout->offsets = off;
    off += round_up(((size_t)E + 1) * sizeof(int32_t));
    layout->active = off;
    off += round_up((size_t)E * sizeof(int32_t));
    layout->large = off;
    off += round_up((size_t)E * sizeof(int32_t));
    layout->sorted_slot = off;
    off += round_up((S ? S : 1) * sizeof(int32_t));
    layout->h = off;
    off += round_up(S * (size_t)I * sizeof(uint16_t));
    layout->y = off;
    layout->y_parts = (size_t)moe::tiled_down_parts(T, H, I, E, top_k);
    off += round_up(layout->y_parts * S * (size_t)H * sizeof(float));
    layout->total_bytes = off;
    return MOE_FFN_OK;
}

size_t moe_ffn_workspace_bytes(int64_t T, int64_t H, int64_t I, int32_t E, int32_t top_k) {
    moe_ffn_ws_layout L;
    if (moe_ffn_workspace_layout(T, H, I, E, top_k, &L) != MOE_FFN_OK) return 0;
    return L.total_bytes;
}

int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t top_k,
                   int32_t* topk_ids, float* topk_w, void* stream) {
    if (T < 0 || E < 1 || E > MOE_FFN_MAX_EXPERTS || top_k < 1 || top_k > E || top_k > 64 ||
        T * (int64_t)top_k >= ((int64_t)1 << 31))
        return MOE_FFN_ERR_BAD_SHAPE;
    if (T == 0) return MOE_FFN_OK;
    if (!logits || !topk_ids || !topk_w) return MOE_FFN_ERR_NULL_ARG;
    if ((reinterpret_cast<uintptr_t>(logits) | reinterpret_cast<uintptr_t>(topk_ids) |
         reinterpret_cast<uintptr_t>(topk_w)) & 3u)
        return MOE_FFN_ERR_MISALIGNED;
    const size_t sb = (size_t)T * (size_t)top_k * 4;
    if (overlap(topk_ids, sb, topk_w, sb) || overlap(logits, (size_t)T * E * 4, topk_ids, sb) ||
        overlap(logits, (size_t)T * E * 4, topk_w, sb))
        return MOE_FFN_ERR_ALIAS;
    const hipError_t err = moe::launch_route_topk(logits, (int)T, E, top_k, topk_ids, topk_w,
                                                  static_cast<hipStream_t>(stream));
    return err == hipSuccess ? MOE_FFN_OK : MOE_FFN_ERR_HIP;
}

int moe_route_grouped(const float* logits, const float* bias, int64_t T, int32_t E,
                      int32_t n_group, int32_t topk_group, int32_t top_k, float scale,
                      int32_t* topk_ids, float* topk_w, void* stream) {
    if (T < 0 || E < 1 || E > MOE_FFN_MAX_EXPERTS || n_group < 1 || n_group > 64 ||
        E % n_group != 0 || topk_group < 1 || topk_group > n_group || top_k < 1 ||
        top_k > 64 || top_k > topk_group * (E / n_group) ||
        T * (int64_t)top_k >= ((int64_t)1 << 31) || T >= ((int64_t)1 << 31) / 4)
        return MOE_FFN_ERR_BAD_SHAPE;
    if (T == 0) return MOE_FFN_OK;
    if (!logits || !topk_ids || !topk_w) return MOE_FFN_ERR_NULL_ARG;
    if ((reinterpret_cast<uintptr_t>(logits) | reinterpret_cast<uintptr_t>(bias) |
         reinterpret_cast<uintptr_t>(topk_ids) | reinterpret_cast<uintptr_t>(topk_w)) & 3u)
        return MOE_FFN_ERR_MISALIGNED;
    const size_t sb = (size_t)T * (size_t)top_k * 4;
    const size_t lb = (size_t)T * (size_t)E * 4;
    const size_t bb = (size_t)E * 4;
    if (overlap(topk_ids, sb, topk_w, sb) || overlap(logits, lb, topk_ids, sb) ||
        overlap(logits, lb, topk_w, sb) ||
        (bias && (overlap(bias, bb, topk_ids, sb) || overlap(bias, bb, topk_w, sb))))
        return MOE_FFN_ERR_ALIAS;
    const hipError_t err =
        moe::launch_route_grouped(logits, bias, (int)T, E, n_group, topk_group, top_k, scale,
                                  topk_ids, topk_w, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? MOE_FFN_OK : MOE_FFN_ERR_HIP;
}

int moe_ffn_forward(const void* x, const int32_t* topk_ids, const float* topk_w,
                    const void* W_gate, const void* W_up, const void* W_down, void* out,
                    int64_t T, int64_t H, int64_t I, int32_t E, int32_t top_k,
                    void* workspace, size_t workspace_bytes, void* stream) {
    moe_ffn_ws_layout L;
    int rc = check_forward(x, topk_ids, topk_w, out, T, H, I, E, top_k, workspace,
                           workspace_bytes, 32, &L);
    if (rc != MOE_FFN_OK || T == 0) return rc;
    if (!W_gate || !W_up || !W_down) return MOE_FFN_ERR_NULL_ARG;
    if (!aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_down))
        return MOE_FFN_ERR_MISALIGNED;
    int ncu = 0;
    if ((rc = num_cu(&ncu)) != MOE_FFN_OK) return rc;
    const moe::FfnShape s{(int)T, (int)H, (int)I, E, top_k};
    const moe::FfnWeights W{W_gate, W_up, W_down, nullptr, nullptr, nullptr};
    const moe::Routing route{nullptr, const_cast<int32_t*>(topk_ids), const_cast<float*>(topk_w)};
    const hipError_t err = moe::launch_ffn_bf16(
        static_cast<const uint16_t*>(x), route, W, static_cast<uint16_t*>(out), s,
        carve(workspace, L), ncu, take_stage_events(), t_split, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? MOE_FFN_OK : MOE_FFN_ERR_HIP;
}

int moe_ffn_forward_noalloc(const void* x, const int32_t* topk_ids, const float* topk_w,
                            const void* W_gate, const void* W_up, const void* W_down, void* out,
                            int64_t T, int64_t H, int64_t I, int32_t E, int32_t top_k,
                            void* stream) {
    if (!shape_ok(T, H, I, E, top_k) || H % 32 != 0 || I % 32 != 0) return MOE_FFN_ERR_BAD_SHAPE;
    if (T == 0) return MOE_FFN_OK;
    moe_ffn_ws_layout L;
    if (moe_ffn_workspace_layout(T, H, I, E, top_k, &L) != MOE_FFN_OK) return MOE_FFN_ERR_BAD_SHAPE;
    if (L.total_bytes > MOE_FFN_NOALLOC_WORKSPACE_BYTES) return MOE_FFN_ERR_WORKSPACE;
    // every other check (pointers, alignment, overlaps) is moe_ffn_forward's;
    // the workspace argument is the library's array
    void* ws = nullptr;
    if (!x || !topk_ids || !topk_w || !out || !W_gate || !W_up || !W_down)
        return MOE_FFN_ERR_NULL_ARG;
    if (const int rc = scratch_address(&ws); rc != MOE_FFN_OK) return rc;
    return moe_ffn_forward(x, topk_ids, topk_w, W_gate, W_up, W_down, out, T, H, I, E, top_k, ws,
                           MOE_FFN_NOALLOC_WORKSPACE_BYTES, stream);
}

int moe_ffn_forward_logits(const void* x, const float* logits, int32_t* topk_ids,
                           float* topk_w, const void* W_gate, const void* W_up,
                           const void* W_down, void* out, int64_t T, int64_t H, int64_t I,
                           int32_t E, int32_t top_k, void* workspace, size_t workspace_bytes,
                           void* stream) {
    if (top_k > 64) return MOE_FFN_ERR_BAD_SHAPE;
    moe_ffn_ws_layout L;
    int rc = check_forward(x, topk_ids, topk_w, out, T, H, I, E, top_k, workspace,
                           workspace_bytes, 32, &L);
    if (rc != MOE_FFN_OK || T == 0) return rc;
    if (!logits || !W_gate || !W_up || !W_down) return MOE_FFN_ERR_NULL_ARG;
    if (reinterpret_cast<uintptr_t>(logits) & 3u) return MOE_FFN_ERR_MISALIGNED;
    if (!aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_down))
        return MOE_FFN_ERR_MISALIGNED;
    // the routing outputs are written: they may overlap no input, each
    // other, or the workspace
    const size_t sb = (size_t)T * (size_t)top_k * 4;
    const size_t lb = (size_t)T * (size_t)E * 4;
    const size_t xb = (size_t)T * (size_t)H * 2;
    if (overlap(topk_ids, sb, topk_w, sb) || overlap(logits, lb, topk_ids, sb) ||
        overlap(logits, lb, topk_w, sb) || overlap(x, xb, topk_ids, sb) ||
        overlap(x, xb, topk_w, sb) || overlap(workspace, L.total_bytes, topk_ids, sb) ||
        overlap(workspace, L.total_bytes, topk_w, sb) || overlap(logits, lb, out, xb))
        return MOE_FFN_ERR_ALIAS;
    int ncu = 0;
    if ((rc = num_cu(&ncu)) != MOE_FFN_OK) return rc;
    const moe::FfnShape s{(int)T, (int)H, (int)I, E, top_k};
    const moe::FfnWeights W{W_gate, W_up, W_down, nullptr, nullptr, nullptr};
    const moe::Routing route{logits, topk_ids, topk_w};
    const hipError_t err = moe::launch_ffn_bf16(
        static_cast<const uint16_t*>(x), route, W, static_cast<uint16_t*>(out), s,
        carve(workspace, L), ncu, take_stage_events(), t_split, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? MOE_FFN_OK : MOE_FFN_ERR_HIP;
}

int moe_ffn_forward_int8(const void* x, const int32_t* topk_ids, const float* topk_w,
                         const int8_t* Q_gate, const float* S_gate, const int8_t* Q_up,
                         const float* S_up, const int8_t* Q_down, const float* S_down,
                         int32_t group, void* out, int64_t T, int64_t H, int64_t I,
                         int32_t E, int32_t top_k, void* workspace, size_t workspace_bytes,
                         void* stream) {
    if (group != MOE_FFN_INT8_GROUP) return MOE_FFN_ERR_BAD_SHAPE;
    moe_ffn_ws_layout L;
    int rc = check_forward(x, topk_ids, topk_w, out, T, H, I, E, top_k, workspace,
                           workspace_bytes, MOE_FFN_INT8_GROUP, &L);
    if (rc != MOE_FFN_OK || T == 0) return rc;
    if (!Q_gate || !S_gate || !Q_up || !S_up || !Q_down || !S_down) return MOE_FFN_ERR_NULL_ARG;
    if (!aligned16(Q_gate) || !aligned16(Q_up) || !aligned16(Q_down) || !aligned4(S_gate) ||
        !aligned4(S_up) || !aligned4(S_down))
        return MOE_FFN_ERR_MISALIGNED;
    int ncu = 0;
    if ((rc = num_cu(&ncu)) != MOE_FFN_OK) return rc;
    const moe::FfnShape s{(int)T, (int)H, (int)I, E, top_k};
    const moe::FfnWeights W{Q_gate, Q_up, Q_down, S_gate, S_up, S_down};
    const moe::Routing route{nullptr, const_cast<int32_t*>(topk_ids), const_cast<float*>(topk_w)};
    const hipError_t err = moe::launch_ffn_int8(
        static_cast<const uint16_t*>(x), route, W, static_cast<uint16_t*>(out), s,
        carve(workspace, L), ncu, take_stage_events(), t_split, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? MOE_FFN_OK : MOE_FFN_ERR_HIP;
}

namespace {

bool attn_shape_ok(int32_t B, int32_t h_q, int32_t h_kv, int32_t d, int32_t max_len) {
    if (B < 0 || h_q < 1 || h_kv < 1 || max_len < 0) return false;
    if (h_q % h_kv != 0 || h_q / h_kv > 16) return false;
    if (d != 64 && d != 128 && d != 256) return false;
    // element offsets of the KV cache fit in 64 bits; grid dims in range
    if ((int64_t)B * h_kv * (int64_t)max_len * d >= ((int64_t)1 << 62)) return false;
    if ((int64_t)B * h_kv >= ((int64_t)1 << 31)) return false;
    // the merge grid is (h_q, B); the split grid (B * h_kv, max_len / 128)
    if (B > 65535 || (int64_t)max_len / 128 > 65535) return false;
    return true;
}

}  // namespace

size_t moe_attn_decode_workspace_bytes(int32_t B, int32_t h_q, int32_t h_kv, int32_t d,
                                       int32_t max_len) {
    if (!attn_shape_ok(B, h_q, h_kv, d, max_len)) return 0;
    const size_t n = moe::attn_workspace_bytes(B, h_kv, d, max_len);
    return n == 0 ? kAlign : (n + kAlign - 1) / kAlign * kAlign;
}

int moe_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* seq_lens, void* out, int32_t B, int32_t h_q, int32_t h_kv,
                    int32_t d, int32_t max_len, float scale, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (!attn_shape_ok(B, h_q, h_kv, d, max_len)) return MOE_FFN_ERR_BAD_SHAPE;
    if (B == 0) return MOE_FFN_OK;
    if (!q || !seq_lens || !out) return MOE_FFN_ERR_NULL_ARG;
    if (max_len > 0 && (!k_cache || !v_cache)) return MOE_FFN_ERR_NULL_ARG;
    if (!workspace) return MOE_FFN_ERR_WORKSPACE;
    if (workspace_bytes < moe_attn_decode_workspace_bytes(B, h_q, h_kv, d, max_len))
        return MOE_FFN_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(out) || (max_len > 0 && (!aligned16(k_cache) ||
                                                              !aligned16(v_cache))))
        return MOE_FFN_ERR_MISALIGNED;
    if ((reinterpret_cast<uintptr_t>(seq_lens) & 3u) ||
        reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
        return MOE_FFN_ERR_MISALIGNED;
    const size_t qb = (size_t)B * h_q * d * 2;
    const size_t kvb = (size_t)B * h_kv * (size_t)max_len * d * 2;
    const size_t wb = moe_attn_decode_workspace_bytes(B, h_q, h_kv, d, max_len);
    if (overlap(out, qb, q, qb) || overlap(out, qb, workspace, wb) ||
        overlap(out, qb, seq_lens, (size_t)B * 4) ||
        (max_len > 0 && (overlap(out, qb, k_cache, kvb) || overlap(out, qb, v_cache, kvb) ||
                         overlap(workspace, wb, k_cache, kvb) ||
                         overlap(workspace, wb, v_cache, kvb))) ||
        overlap(workspace, wb, q, qb) || overlap(workspace, wb, seq_lens, (size_t)B * 4))
        return MOE_FFN_ERR_ALIAS;
    // the standard score scale unless the caller gives a positive one
    if (!(scale > 0.f)) scale = (float)(1.0 / std::sqrt((double)d));
    const hipError_t err = moe::launch_attn_decode(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
        static_cast<const uint16_t*>(v_cache), seq_lens, static_cast<uint16_t*>(out), B, h_q,
        h_kv, d, max_len, scale, workspace, take_stage_events(), static_cast<hipStream_t>(stream));
    return err == hipSuccess ? MOE_FFN_OK : MOE_FFN_ERR_HIP;
}

int moe_ffn_forward_int4(const void* x, const int32_t* topk_ids, const float* topk_w,
                         const uint8_t* P_gate, const float* S_gate, const uint8_t* P_up,
                         const float* S_up, const uint8_t* P_down, const float* S_down,
                         int32_t group, void* out, int64_t T, int64_t H, int64_t I,
                         int32_t E, int32_t top_k, void* workspace, size_t workspace_bytes,
                         void* stream) {
    if (group != MOE_FFN_INT8_GROUP) return MOE_FFN_ERR_BAD_SHAPE;
    moe_ffn_ws_layout L;
    int rc = check_forward(x, topk_ids, topk_w, out, T, H, I, E, top_k, workspace,
                           workspace_bytes, MOE_FFN_INT8_GROUP, &L);
    if (rc != MOE_FFN_OK || T == 0) return rc;
    if (!P_gate || !S_gate || !P_up || !S_up || !P_down || !S_down) return MOE_FFN_ERR_NULL_ARG;
    if (!aligned16(P_gate) || !aligned16(P_up) || !aligned16(P_down) || !aligned4(S_gate) ||
        !aligned4(S_up) || !aligned4(S_down))
        return MOE_FFN_ERR_MISALIGNED;
    int ncu = 0;
    if ((rc = num_cu(&ncu)) != MOE_FFN_OK) return rc;
    const moe::FfnShape s{(int)T, (int)H, (int)I, E, top_k};
    const moe::FfnWeights W{P_gate, P_up, P_down, S_gate, S_up, S_down};
    const moe::Routing route{nullptr, const_cast<int32_t*>(topk_ids), const_cast<float*>(topk_w)};
    const hipError_t err = moe::launch_ffn_int4(
        static_cast<const uint16_t*>(x), route, W, static_cast<uint16_t*>(out), s,
        carve(workspace, L), ncu, take_stage_events(), t_split, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? MOE_FFN_OK : MOE_FFN_ERR_HIP;
}

int moe_ffn_forward_resplit(const void* x, const int32_t* topk_ids, const float* topk_w,
                            const uint8_t* P_gate, const float* S_gate, const uint8_t* R_gate,
                            const float* SR_gate, const uint8_t* P_up, const float* S_up,
                            const uint8_t* R_up, const float* SR_up, const uint8_t* P_down_lo,
                            const float* S_down_lo, const int8_t* Q_down_hi,
                            const float* S_down_hi, const uint8_t* critical, int32_t group,
                            void* out, int64_t T, int64_t H, int64_t I, int32_t E,
                            int32_t top_k, void* workspace, size_t workspace_bytes,
                            void* stream) {
    if (group != MOE_FFN_INT8_GROUP) return MOE_FFN_ERR_BAD_SHAPE;
    moe_ffn_ws_layout L;
    int rc = check_forward(x, topk_ids, topk_w, out, T, H, I, E, top_k, workspace,
                           workspace_bytes, MOE_FFN_INT8_GROUP, &L);
    if (rc != MOE_FFN_OK || T == 0) return rc;
    const void* const weights[] = {P_gate, R_gate, P_up, R_up, P_down_lo, Q_down_hi};
    const void* const scales[] = {S_gate, SR_gate, S_up, SR_up, S_down_lo, S_down_hi};
    for (const void* t : weights) {
        if (!t) return MOE_FFN_ERR_NULL_ARG;
        if (!aligned16(t)) return MOE_FFN_ERR_MISALIGNED;
    }
    for (const void* t : scales) {
        if (!t) return MOE_FFN_ERR_NULL_ARG;
        if (!aligned4(t)) return MOE_FFN_ERR_MISALIGNED;
    }
    if (!critical) return MOE_FFN_ERR_NULL_ARG;
    int ncu = 0;
    if ((rc = num_cu(&ncu)) != MOE_FFN_OK) return rc;
    const moe::FfnShape s{(int)T, (int)H, (int)I, E, top_k};
    moe::FfnWeights W{P_gate, P_up, P_down_lo, S_gate, S_up, S_down_lo};
    W.gate2 = R_gate;
    W.up2 = R_up;
    W.down2 = Q_down_hi;
    W.s_gate2 = SR_gate;
    W.s_up2 = SR_up;
    W.s_down2 = S_down_hi;
    W.critical = critical;
    const moe::Routing route{nullptr, const_cast<int32_t*>(topk_ids), const_cast<float*>(topk_w)};
    const hipError_t err = moe::launch_ffn_resplit(
        static_cast<const uint16_t*>(x), route, W, static_cast<uint16_t*>(out), s,
        carve(workspace, L), ncu, take_stage_events(), t_split, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? MOE_FFN_OK : MOE_FFN_ERR_HIP;
}

int moe_ffn_check_status(const void* workspace, void* stream, int64_t* n_dropped) {
    if (!workspace) return MOE_FFN_ERR_NULL_ARG;
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess)
        return MOE_FFN_ERR_HIP;
    int32_t meta[2] = {0, 0};
    if (hipMemcpy(meta, workspace, sizeof meta, hipMemcpyDeviceToHost) != hipSuccess)
        return MOE_FFN_ERR_HIP;
    if (n_dropped) *n_dropped = meta[1];
    return meta[1] > 0 ? MOE_FFN_ERR_BAD_IDS : MOE_FFN_OK;
}

int moe_ffn_read_probe(const void* buf, size_t bytes, void* sink, void* stream) {
    if (!buf || !sink) return MOE_FFN_ERR_NULL_ARG;
    if (bytes == 0 || bytes % 16 != 0) return MOE_FFN_ERR_BAD_SHAPE;
    if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
        return MOE_FFN_ERR_MISALIGNED;
    int ncu = 0;
    if (const int rc = num_cu(&ncu); rc != MOE_FFN_OK) return rc;
    return moe::launch_read_probe(buf, bytes, static_cast<uint32_t*>(sink), ncu,
                                  static_cast<hipStream_t>(stream)) == hipSuccess
               ? MOE_FFN_OK
               : MOE_FFN_ERR_HIP;
}

int moe_ffn_launch_probe(int32_t n, void* stream) {
    if (n < 0 || n > 1000000) return MOE_FFN_ERR_BAD_SHAPE;
    return moe::launch_empty_chain(n, static_cast<hipStream_t>(stream)) == hipSuccess
               ? MOE_FFN_OK
               : MOE_FFN_ERR_HIP;
}

int moe_ffn_set_split(int32_t gate_up_split, int32_t down_split) {
    auto ok = [](int32_t v) { return v == 0 || v == 1 || v == 2 || v == 4; };
    if (!ok(gate_up_split) || !ok(down_split)) return MOE_FFN_ERR_BAD_SHAPE;
    t_split.gate_up = gate_up_split;
    t_split.down = down_split;
    return MOE_FFN_OK;
}

int moe_ffn_set_stage_events(void* const* events, int32_t n_events) {
    if (n_events < 0 || n_events > 4) return MOE_FFN_ERR_BAD_SHAPE;
    if (!events) n_events = 0;
    for (int i = 0; i < n_events; ++i)
        t_stage_events.ev[i] = static_cast<hipEvent_t>(events[i]);
    t_stage_events.n = n_events;
    return MOE_FFN_OK;
}

int moe_ffn_device_check(int32_t* where) {
    if (!where) return MOE_FFN_ERR_NULL_ARG;
    *where = 0;
    if (hipDeviceSynchronize() != hipSuccess) return MOE_FFN_ERR_HIP;
    // translation units in a fixed order; the first that reports wins
    hipError_t (*const readers[])(int*) = {moe::device_check_route_permute, moe::device_check_expert_gemm,
                                           moe::device_check_expert_tile, moe::device_check_combine,
                                           moe::device_check_attn_decode};
    for (int i = 0; i < (int)(sizeof(readers) / sizeof(readers[0])); ++i) {
        int line = 0;
        if (readers[i](&line) != hipSuccess) return MOE_FFN_ERR_HIP;
        if (line != 0 && *where == 0) *where = (i + 1) * 100000 + line;
    }
#ifdef MOE_FFN_DEVICE_CHECKS
    return 1;
#else
    return 0;
#endif
}

const char* moe_ffn_status_string(int status) {
    switch (status) {
        case MOE_FFN_OK: return "ok";
        case MOE_FFN_ERR_NULL_ARG: return "a required pointer is NULL";
        case MOE_FFN_ERR_BAD_SHAPE: return "sizes outside the supported range";
        case MOE_FFN_ERR_MISALIGNED: return "a pointer is not suitably aligned";
        case MOE_FFN_ERR_ALIAS: return "output overlaps an input";
        case MOE_FFN_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_FFN_ERR_HIP: return "HIP runtime error";
        case MOE_FFN_ERR_BAD_IDS: return "expert ids outside [0, E) were dropped";
        default: return "unknown status";
    }
}

}  // extern "C"
