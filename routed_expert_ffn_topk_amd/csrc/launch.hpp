// Host-side launchers of the MoE FFN kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Pointers into the caller's workspace, carved by the C-ABI layer.
struct Workspace {
    int32_t* meta;         // [0] experts of active, [1] dropped slots, [2] experts of large
    int32_t* counts;       // [E]
    int32_t* offsets;      // [E+1]
    int32_t* active;       // [E] experts of the small-m product
    int32_t* large;        // [E] experts of the tiled product
    int32_t* sorted_slot;  // [T*k]
    uint16_t* h;           // [T*k][I] bf16, sorted order
    float* y;              // [T*k][H] f32, slot order
};

// Optional per-kernel timing events (benchmark hook): ev[i] is recorded
// right after kernel i of a forward call is enqueued, for i < n.
struct StageEvents {
    hipEvent_t ev[4];
    int n;
    hipError_t mark(int i, hipStream_t stream) const {
        return i < n ? hipEventRecord(ev[i], stream) : hipSuccess;
    }
};

// K parts per row block forced on the two grouped products (0: chosen on the
// device from the active-expert count); a test hook.
struct SplitOverride {
    int gate_up = 0;
    int down = 0;
};

struct FfnShape {
    int T, H, I, E, k;
};

// Where a forward call's routing comes from: the caller's top-k ids and
// weights (logits == nullptr; ids and w are only read), or router logits,
// routed on the device into ids and w (written) before the gather index.
struct Routing {
    const float* logits;
    int32_t* ids;
    float* w;
};

// Weights of one layer: BF16 (no scales), or INT8 / INT4 (packed nibbles)
// with per-128 group scales.
struct FfnWeights {
    const void* gate;
    const void* up;
    const void* down;
    const float* s_gate;  // INT8 / INT4 only
    const float* s_up;
    const float* s_down;
    // residual split only: W^R of gate and up, the high-precision down copy,
    // their scales, and the per-expert precision flags
    const void* gate2 = nullptr;
    const void* up2 = nullptr;
    const void* down2 = nullptr;
    const float* s_gate2 = nullptr;
    const float* s_up2 = nullptr;
    const float* s_down2 = nullptr;
    const uint8_t* critical = nullptr;
};

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids,
                             float* w, hipStream_t stream);
hipError_t launch_route_grouped(const float* logits, const float* bias, int T, int E,
                               int n_group, int topk_group, int k, float scale, int32_t* ids,
                               float* w, hipStream_t stream);

// Gather index of ids [T][k]; experts with more than m_split slots are listed
// for the tiled product (INT_MAX: none).
hipError_t launch_permute(const int32_t* ids, const FfnShape& s, const Workspace& ws,
                          int m_split, hipStream_t stream);

// Router and gather index from logits [T][E]: writes ids / w [T][k] and the
// workspace's gather index (one launch for decode-sized batches).
hipError_t launch_route_permute(const float* logits, int32_t* ids, float* w,
                                const FfnShape& s, const Workspace& ws, int m_split,
                                hipStream_t stream);

hipError_t launch_ffn_bf16(const uint16_t* x, const Routing& route, const FfnWeights& W,
                           uint16_t* out, const FfnShape& s, const Workspace& ws, int num_cu,
                           const StageEvents& ev, const SplitOverride& split,
                           hipStream_t stream);

hipError_t launch_ffn_int4(const uint16_t* x, const Routing& route, const FfnWeights& W,
                           uint16_t* out, const FfnShape& s, const Workspace& ws, int num_cu,
                           const StageEvents& ev, const SplitOverride& split,
                           hipStream_t stream);

hipError_t launch_ffn_int8(const uint16_t* x, const Routing& route, const FfnWeights& W,
                           uint16_t* out, const FfnShape& s, const Workspace& ws, int num_cu,
                           const StageEvents& ev, const SplitOverride& split,
                           hipStream_t stream);
hipError_t launch_ffn_resplit(const uint16_t* x, const Routing& route, const FfnWeights& W,
                           uint16_t* out, const FfnShape& s, const Workspace& ws, int num_cu,
                           const StageEvents& ev, const SplitOverride& split,
                           hipStream_t stream);

// Tiled products (BF16) over the workspace's large list: gate/up with the
// SiLU*up epilogue into h, and down into y.
hipError_t launch_tiled_gate_up(const uint16_t* x, const FfnWeights& W, const FfnShape& s,
                                const Workspace& ws, int num_cu, hipStream_t stream);
hipError_t launch_tiled_down(const FfnWeights& W, const FfnShape& s, const Workspace& ws,
                             int num_cu, hipStream_t stream);

// The tiled product takes experts with more than kTiledMinTokens tokens in
// batches of more than kTiledMinBatch tokens (BF16 weights).
constexpr int kTiledMinBatch = 64;
constexpr int kTiledMinTokens = 32;

// K parts of the tiled down product for these sizes (1, 2 or 4; a pure host
// function): y holds this many planes of partial sums, [part][slot][H], of
// which the slots of tiled experts fill every plane, the others the first.
int tiled_down_parts(int64_t T, int64_t H, int64_t I, int E, int k);

// Weighted combine shared by every weight format: y plane 0, plus planes 1 ..
// parts - 1 (plane floats apart) for slots whose expert has more than
// large_min tokens (counts).
hipError_t launch_combine(const float* y, const int32_t* ids, const float* w,
                          uint16_t* out, const FfnShape& s, const int32_t* counts,
                          int large_min, int parts, size_t plane, hipStream_t stream);

// Decode attention with grouped-query heads: workspace bytes, and the split
// kernel + merge kernel on the caller's stream (sizes validated by the C ABI).
int attn_chunk(int B, int h_kv, int max_len);
size_t attn_workspace_bytes(int B, int h_kv, int d, int max_len);
hipError_t launch_attn_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* lens, uint16_t* out, int B, int h_q, int h_kv,
                              int d, int max_len, float scale, void* workspace,
                              const StageEvents& ev, hipStream_t stream);

// Streaming-read probe over bytes (a multiple of 16) of buf; sink is one
// device word.
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, int num_cu,
                             hipStream_t stream);

// n launches of an empty one-wave kernel on stream (launch-gap probe).
hipError_t launch_empty_chain(int n, hipStream_t stream);

// Debug build (-DMOE_FFN_DEVICE_CHECKS): the first device bounds check that
// failed in each translation unit since the last read (0: none), cleared by
// the read; release builds report 0.
hipError_t device_check_route_permute(int* line);
hipError_t device_check_expert_gemm(int* line);
hipError_t device_check_expert_tile(int* line);
hipError_t device_check_combine(int* line);
hipError_t device_check_attn_decode(int* line);

}  // namespace moe
