/*
 * moe_ffn.h -- C ABI of the routed-expert MoE FFN library for MI355X (gfx950).
 *
 * The operation is the routed-expert feed-forward layer of Mixture-of-Experts
 * decoding described in "HiNa-MoE: High-Performance, Non-Intrusive MoE
 * Inference on CPUs with Matrix Engines" (arXiv 2610.05123):
 *   - §2.1 / Fig. 2: a gate sends every token to k of E experts (Table 3:
 *     top-2 for Mixtral, top-8 for DeepSeek-V3 and Qwen3);
 *   - §4.1 / Fig. 5: the tokens routed to one expert are gathered into a small
 *     matrix I and the expert computes FFN(I) = SiLU(I*Wgate) (.) (I*Wup) * Wdown
 *     (FFN equation of §4.1);
 *   - §4.1 ("transform I, not W"): expert weights stay in their ordinary
 *     row-major layout; only the small gathered matrix is laid out for the
 *     matrix unit, and the result is written back row-major;
 *   - §4.2.1: BF16 operands with FP32 accumulation; §8.1 / Fig. 11: an INT8
 *     variant with symmetric group-wise weight quantisation.
 *
 * Conventions for every entry point:
 *   - Tensors are plain device pointers in caller-owned memory (e.g. from
 *     PyTorch).  The library never allocates, frees, repacks or copies weights,
 *     and keeps no state between calls besides a cached CU count per device and
 *     the per-thread benchmark hook of moe_ffn_set_stage_events.
 *   - BF16 values are IEEE bfloat16 bit patterns (uint16).  All arrays are
 *     dense row-major with the last index contiguous.
 *   - `stream` is a hipStream_t (NULL = the default stream) of the current HIP
 *     device; all pointers must be memory of that device.  Work is enqueued
 *     asynchronously; no entry point synchronises except
 *     moe_ffn_check_status.
 *   - Return value: MOE_FFN_OK (0) or a negative MOE_FFN_ERR_* code; on an
 *     error nothing has been enqueued.  Shape and pointer checks are done on
 *     the host before any launch.
 *   - Calls that use distinct workspaces may run concurrently; calls that
 *     share a workspace must be ordered (same stream).
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_FFN_OK 0
#define MOE_FFN_ERR_NULL_ARG (-1)    /* a required pointer is NULL */
#define MOE_FFN_ERR_BAD_SHAPE (-2)   /* sizes outside the supported range */
#define MOE_FFN_ERR_MISALIGNED (-3)  /* a tensor pointer is not 16-byte aligned */
#define MOE_FFN_ERR_ALIAS (-4)       /* out overlaps x (or ids/weights overlap) */
#define MOE_FFN_ERR_WORKSPACE (-5)   /* workspace NULL or smaller than required */
#define MOE_FFN_ERR_HIP (-6)         /* a HIP runtime call or launch failed */
#define MOE_FFN_ERR_BAD_IDS (-7)     /* (device-side) expert ids outside [0, E) */

/* Largest supported expert count (per-expert tables live in on-chip memory). */
#define MOE_FFN_MAX_EXPERTS 1024
/* INT8 variant: one FP32 scale per this many consecutive K elements of a row. */
#define MOE_FFN_INT8_GROUP 128

/*
 * Workspace layout.  The workspace is caller-owned device memory, at least
 * total_bytes long and 256-byte aligned; each region starts at the given byte
 * offset.  Regions (T tokens, k = top_k, S = T*k slots, slot s = t*k + j):
 *   meta        int32[8]   [0] number of experts listed in `active`, [1] number
 *                          of slots whose expert id was outside [0, E) (those
 *                          slots contribute nothing to the output), [2] number
 *                          of experts listed in `large`
 *   counts      int32[E]   tokens routed to each expert
 *   offsets     int32[E+1] start of each expert's run in sorted_slot
 *   active      int32[E]   experts with counts > 0 that the small-m product
 *                          handles, ascending
 *   large       int32[E]   experts that the tiled (many-token) product
 *                          handles, ascending: those with more than 32 tokens
 *                          when the batch has T > 64 tokens and BF16 weights
 *                          (moe_ffn_forward, moe_ffn_forward_logits);
 *                          otherwise none, and `active` lists every expert
 *                          with counts > 0
 *   sorted_slot int32[S]   slots grouped by expert (ascending), ascending
 *                          slot order within an expert (the gather order)
 *   h           bf16[S][I] SiLU(gate)*up of each gathered row, in
 *                          sorted_slot order (row p belongs to slot
 *                          sorted_slot[p])
 *   y           f32[P][S][H] down-projection output of each slot, slot
 *                          order, P = y_parts.  With P > 1 (BF16 batches with
 *                          few tiles of many tokens per expert: the K of the
 *                          down product is split into P parts) the slots of
 *                          experts listed in `large` hold partial sums in
 *                          every plane, whose sum is their output; every other
 *                          slot holds its output in plane 0.
 * After a forward call the regions hold these values (tests inspect them).
 * y_parts is a count, not an offset; it depends on the sizes alone.
 */
typedef struct moe_ffn_ws_layout {
    size_t total_bytes;
    size_t meta;
    size_t counts;
    size_t offsets;
    size_t active;
    size_t large;
    size_t sorted_slot;
    size_t h;
    size_t y;
    size_t y_parts;
} moe_ffn_ws_layout;

/* Fill *layout for the given sizes.  Pure host computation (no HIP call).
 * Returns MOE_FFN_ERR_NULL_ARG if layout is NULL, MOE_FFN_ERR_BAD_SHAPE for
 * T < 0, H or I < 1, E outside [1, MOE_FFN_MAX_EXPERTS], top_k outside [1, E]. */
int moe_ffn_workspace_layout(int64_t T, int64_t H, int64_t I, int32_t E,
                             int32_t top_k, moe_ffn_ws_layout* layout);

/* Workspace bytes needed by moe_ffn_forward / moe_ffn_forward_int8 for these
 * sizes, or 0 if the sizes are invalid. */
size_t moe_ffn_workspace_bytes(int64_t T, int64_t H, int64_t I, int32_t E,
                               int32_t top_k);

/*
 * Top-k router (HiNa-MoE §2.1 / Fig. 2; k from Table 3).
 *   logits   [T][E] float32, device.
 *   topk_ids [T][top_k] int32, device, written: for each token the top_k
 *            experts by descending logit (= descending softmax probability),
 *            ties broken toward the lower expert id.
 *   topk_w   [T][top_k] float32, device, written: the softmax probabilities of
 *            the chosen experts renormalised to sum to one (equal to a softmax
 *            over the top_k chosen logits).
 * Each token needs at least top_k finite logits; NaN logits are not supported.
 * Errors: NULL_ARG, BAD_SHAPE (T < 0, E outside [1, MOE_FFN_MAX_EXPERTS],
 * top_k outside [1, min(E, 64)]), ALIAS (outputs overlap), HIP.
 */
int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t top_k,
                   int32_t* topk_ids, float* topk_w, void* stream);

/*
 * Grouped sigmoid router (the gate of DeepSeek-V3, one of the models in the
 * pages' Table 3 and RapidMoE's evaluation; the pages name the model but do
 * not spell out its gate).  For each token t, with l = logits[t]:
 *   s_e = 1 / (1 + exp(-l_e)),  c_e = s_e + bias_e  (bias NULL: 0)   FP32
 *   the E experts form n_group groups of E / n_group consecutive ids; a
 *   group's score is its largest c plus its second largest (the largest
 *   alone for groups of one);
 *   the topk_group groups of highest score are kept (ties: lower group);
 *   the top_k experts of the kept groups by descending c are chosen (ties:
 *   lower id), slot j holding the j-th;
 *   topk_w[t][j] = s_{e_j} / (sum over the chosen s, ascending j) * scale.
 *   logits [T][E] float32, bias [E] float32 or NULL, device;
 *   topk_ids [T][top_k] int32, topk_w [T][top_k] float32, device (written).
 * Sizes: T >= 0 (0 is a no-op), 1 <= E <= MOE_FFN_MAX_EXPERTS, n_group in
 * [1, 64] dividing E, 1 <= topk_group <= n_group, 1 <= top_k <= 64 and
 * top_k <= topk_group * E / n_group.  Pointers 4-byte aligned.
 * Errors: BAD_SHAPE, NULL_ARG, MISALIGNED, ALIAS (an output overlaps an input
 * or the other output), HIP.  Asynchronous on `stream`.
 */
int moe_route_grouped(const float* logits, const float* bias, int64_t T, int32_t E,
                      int32_t n_group, int32_t topk_group, int32_t top_k, float scale,
                      int32_t* topk_ids, float* topk_w, void* stream);

/*
 * Routed-expert FFN layer, BF16 weights (HiNa-MoE §4.1 FFN equation).
 *   x        [T][H] bf16, device: token activations.
 *   topk_ids [T][top_k] int32, device: expert of each slot.  Ids outside
 *            [0, E) drop that slot (it adds nothing) and are counted in the
 *            workspace meta[1]; read them with moe_ffn_check_status.
 *   topk_w   [T][top_k] float32, device: routing weight of each slot (any
 *            values; they need not sum to one).  Duplicate ids in a row each
 *            count.
 *   W_gate, W_up [E][I][H] bf16, device: row i of expert e holds the H
 *            weights producing intermediate feature i (K = H contiguous).
 *   W_down   [E][H][I] bf16, device: row n produces output feature n.
 *            Experts that no slot names are never read.
 *   out      [T][H] bf16, device, fully overwritten:
 *            out[t] = RNE_bf16( sum_j topk_w[t,j] * y_{t,j} ), FP32 sum over
 *            ascending j, where y_{t,j} = W_down[e] * h (FP32 accumulation),
 *            h = RNE_bf16( silu(g) * u ), g = W_gate[e] x_t, u = W_up[e] x_t
 *            (BF16 products, FP32 accumulation), e = topk_ids[t,j].
 *   workspace / workspace_bytes: at least moe_ffn_workspace_bytes(...) bytes,
 *            256-byte aligned, device; contents on entry are ignored.
 * Sizes: T >= 0 (T = 0 is a no-op), H and I multiples of 32,
 * 1 <= E <= MOE_FFN_MAX_EXPERTS, 1 <= top_k <= E, T*top_k < 2^31.
 * Errors: NULL_ARG, BAD_SHAPE, MISALIGNED (x, out, weights not 16-byte
 * aligned), ALIAS (out overlaps x), WORKSPACE, HIP.
 */
int moe_ffn_forward(const void* x, const int32_t* topk_ids, const float* topk_w,
                    const void* W_gate, const void* W_up, const void* W_down,
                    void* out, int64_t T, int64_t H, int64_t I, int32_t E,
                    int32_t top_k, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Workspace bytes the library holds, per GPU, for moe_ffn_forward_noalloc. */
#define MOE_FFN_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)

/*
 * moe_ffn_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a device array of
 * MOE_FFN_NOALLOC_WORKSPACE_BYTES (32 MiB) that the library holds on every GPU
 * it runs on until the process ends; its address is looked up once per
 * device, on the first call made with that device current.  The call itself
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * Arguments and result: as moe_ffn_forward (x, topk_ids, topk_w, W_gate,
 * W_up, W_down, out and the sizes mean the same, the caller owns them).
 * The array's contents on entry are ignored (every region a call reads is
 * written earlier in the same call), so no clearing is needed between calls.
 * All calls on one GPU share the array: calls that may overlap on one GPU
 * (different streams or threads without ordering) race and give undefined
 * results; calls ordered on one stream are safe.  Slots with ids outside
 * [0, E) are dropped as in moe_ffn_forward, but their count is not reported
 * (moe_ffn_check_status needs a caller workspace).
 * Errors: as moe_ffn_forward, and MOE_FFN_ERR_WORKSPACE when these sizes need
 * more than MOE_FFN_NOALLOC_WORKSPACE_BYTES (moe_ffn_workspace_bytes gives the
 * need; decode-sized batches need a few MiB), MOE_FFN_ERR_HIP if the array's
 * address cannot be obtained.
 */
int moe_ffn_forward_noalloc(const void* x, const int32_t* topk_ids, const float* topk_w,
                            const void* W_gate, const void* W_up, const void* W_down,
                            void* out, int64_t T, int64_t H, int64_t I, int32_t E,
                            int32_t top_k, void* stream);

/*
 * Routed-expert FFN layer from router logits, BF16 weights: the top-k gate
 * (HiNa-MoE §2.1 / Fig. 2) followed by the layer of moe_ffn_forward
 * (§4.1 FFN equation), with the router and the per-expert gather index
 * computed by one kernel for batches of up to 64 tokens and 512 slots
 * (T*top_k), and by the router kernel of moe_route_topk followed by the
 * gather-index kernel above that.
 *   logits   [T][E] float32, device: router logits (each token needs at least
 *            top_k finite values; NaN is not supported).
 *   topk_ids [T][top_k] int32, device, written: as moe_route_topk.
 *   topk_w   [T][top_k] float32, device, written: as moe_route_topk.
 *   x, W_gate, W_up, W_down, out, workspace: as moe_ffn_forward; out equals
 *            moe_ffn_forward(x, topk_ids, topk_w, ...) on the ids and weights
 *            written here.
 * Sizes as moe_ffn_forward, and top_k <= 64.  Errors: as moe_ffn_forward,
 * plus MISALIGNED (logits, topk_ids or topk_w not 4-byte aligned) and ALIAS
 * (topk_ids or topk_w overlap each other, logits, x, out or the workspace,
 * or out overlaps logits).
 */
int moe_ffn_forward_logits(const void* x, const float* logits, int32_t* topk_ids,
                           float* topk_w, const void* W_gate, const void* W_up,
                           const void* W_down, void* out, int64_t T, int64_t H,
                           int64_t I, int32_t E, int32_t top_k, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Routed-expert FFN layer, INT8 weights with group scales (HiNa-MoE §8.1,
 * Fig. 11: symmetric group-wise INT8; group = MOE_FFN_INT8_GROUP along K).
 * As moe_ffn_forward, except every weight row r is int8 q[r][K] with one
 * float32 scale s(r, g) per group g of 128 consecutive K, and each dot
 * product is
 *   sum_g s(r, g) * (sum_{c in group g} v_c * q[r][c])   (FP32).
 * Weights and scales are read in the layout a framework keeps them in
 * (HiNa-MoE §3.1 and Table 1: no weight reformatting), row-major with the
 * groups of a row contiguous:
 *   Q_gate, Q_up [E][I][H] int8 with S_gate, S_up [E][I][H/128] float32;
 *   Q_down [E][H][I] int8 with S_down [E][H][I/128] float32.
 * `group` is the scale group length along K; this library implements
 * group = MOE_FFN_INT8_GROUP (128) and returns MOE_FFN_ERR_BAD_SHAPE for any
 * other value.  Sizes: H and I multiples of 128.  Weight pointers 16-byte
 * aligned, scale pointers 4-byte aligned.
 */
int moe_ffn_forward_int8(const void* x, const int32_t* topk_ids,
                         const float* topk_w, const int8_t* Q_gate,
                         const float* S_gate, const int8_t* Q_up,
                         const float* S_up, const int8_t* Q_down,
                         const float* S_down, int32_t group, void* out,
                         int64_t T, int64_t H, int64_t I, int32_t E,
                         int32_t top_k, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Decode attention with grouped-query heads (HiNa-MoE §6.1, decode
 * attention as small matrix products).  With grouped-query attention,
 * g = h_q / h_kv consecutive query heads read the same KV head; during
 * decoding each contributes one query row, so per KV head the scores are a
 * g-row matrix times the head's keys, and the output that g-row softmax
 * matrix times the head's values.
 *   q        [B][h_q][d] bf16, device: one query vector per sequence and
 *            query head.
 *   k_cache, v_cache [B][h_kv][max_len][d] bf16, device: the KV cache;
 *            sequence b uses its first seq_lens[b] positions.
 *   seq_lens [B] int32, device: valid positions per sequence, in
 *            [0, max_len] (values outside are clamped into that range).
 *   out      [B][h_q][d] bf16, device, fully overwritten: for query head h
 *            (KV head j = h / (h_q / h_kv)) and sequence b,
 *              s_t = scale * (q . k_t)   (BF16 products, FP32 accumulation)
 *              out = RNE_bf16( sum_t softmax(s)_t * v_t )
 *            over t < seq_lens[b] (the softmax weights enter the value
 *            product as BF16); an empty sequence gives zeros.
 *   scale    the score scale; a value that is not positive (0, negative or
 *            NaN) selects 1/sqrt(d), the scale of standard attention,
 *            computed in double precision and rounded to float.
 *   workspace / workspace_bytes: at least
 *            moe_attn_decode_workspace_bytes(...) bytes, 256-byte aligned,
 *            device; contents on entry are ignored (per-split partial
 *            results).
 * Sizes: B >= 0 (B = 0 is a no-op), h_kv >= 1, h_q a multiple of h_kv with
 * h_q / h_kv <= 16, d in {64, 128, 256}, max_len >= 0.
 * Errors: NULL_ARG, BAD_SHAPE, MISALIGNED (q, k_cache, v_cache, out not
 * 16-byte aligned, seq_lens not 4-byte aligned, workspace not 256-byte
 * aligned), ALIAS (out or the workspace overlap an input or each other),
 * WORKSPACE, HIP.
 */
int moe_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* seq_lens, void* out, int32_t B, int32_t h_q,
                    int32_t h_kv, int32_t d, int32_t max_len, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes moe_attn_decode needs for these sizes (a positive multiple
 * of 256), or 0 if the sizes are invalid.  Pure host computation. */
size_t moe_attn_decode_workspace_bytes(int32_t B, int32_t h_q, int32_t h_kv,
                                       int32_t d, int32_t max_len);

/*
 * Routed-expert FFN layer, INT4 weights with group scales (the low-bit
 * counterpart of moe_ffn_forward_int8; HiNa-MoE §8.1 / Fig. 11 quantises
 * symmetrically per group, and the summary of the paper notes that low-bit
 * packing changes the weights' layout).  Identical arithmetic to
 * moe_ffn_forward_int8 on integer weights q in [-7, 7] (any value in
 * [-8, 7] is accepted), stored two per byte as offset-binary nibbles
 * u = q + 8: K element 2i of a row in the low nibble of byte i, element
 * 2i + 1 in the high nibble.
 *   P_gate, P_up [E][I][H/2] uint8 with S_gate, S_up [E][I][H/128] float32;
 *   P_down [E][H][I/2] uint8 with S_down [E][H][I/128] float32
 * (scales row-major as for INT8).  `group` must be MOE_FFN_INT8_GROUP
 * (128).  Sizes: H and I multiples of 128.  Weight pointers 16-byte
 * aligned, scale pointers 4-byte aligned.
 * Batches of any size take the small-m product (no tiled INT4 product).
 */
int moe_ffn_forward_int4(const void* x, const int32_t* topk_ids,
                         const float* topk_w, const uint8_t* P_gate,
                         const float* S_gate, const uint8_t* P_up,
                         const float* S_up, const uint8_t* P_down,
                         const float* S_down, int32_t group, void* out,
                         int64_t T, int64_t H, int64_t I, int32_t E,
                         int32_t top_k, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Routed-expert FFN layer with residual-split low-bit weights and a precision
 * chosen per expert (RapidMoE: "Residual-Split Representation", "GLU
 * Architecture Adoption", "Expert-Residual Offloading").  Each weight of gate
 * and up is held as W^Q, its INT4 group quantisation, plus W^R, the INT4
 * group quantisation of the residual W - W^Q; down is held as two separately
 * quantised copies, INT4 (low precision) and INT8 (high).  An expert with
 * critical[e] != 0 runs in high precision:
 *   g = x W^Q_gate + x W^R_gate,  u = x W^Q_up + x W^R_up,  y = h W_down(INT8)
 * every other expert in low precision:
 *   g = x W^Q_gate,  u = x W^Q_up,  y = h W_down(INT4)
 * with h = RNE_bf16(silu(g) * u) and the combine of moe_ffn_forward.  Each
 * term is a grouped product as in moe_ffn_forward_int8 (FP32 group sums
 * times the group scale).  Choosing which experts are critical (the pages
 * derive it from the router scores, averaged over a batch's tokens) is the
 * caller's.
 *   P_gate, R_gate, P_up, R_up [E][I][H/2] uint8 (W^Q and W^R, the INT4
 *            nibble layout of moe_ffn_forward_int4) with S_gate, SR_gate,
 *            S_up, SR_up [E][I][H/128] float32 (row-major, as for INT8);
 *   P_down_lo [E][H][I/2] uint8 with S_down_lo [E][H][I/128] float32;
 *   Q_down_hi [E][H][I] int8 with S_down_hi [E][H][I/128] float32;
 *   critical [E] uint8, device.
 * Only the tensors an expert's precision needs are read: R_*, SR_* and the
 * high down copy of critical experts, the low down copy of the others.
 * `group` must be MOE_FFN_INT8_GROUP (128).  Sizes: H and I multiples of 128.
 * Weight pointers 16-byte aligned, scale pointers 4-byte aligned.  Batches
 * of any size take the small-m product.  Errors as for moe_ffn_forward_int8 (NULL_ARG also for a
 * null critical).
 */
int moe_ffn_forward_resplit(const void* x, const int32_t* topk_ids,
                            const float* topk_w, const uint8_t* P_gate,
                            const float* S_gate, const uint8_t* R_gate,
                            const float* SR_gate, const uint8_t* P_up,
                            const float* S_up, const uint8_t* R_up,
                            const float* SR_up, const uint8_t* P_down_lo,
                            const float* S_down_lo, const int8_t* Q_down_hi,
                            const float* S_down_hi, const uint8_t* critical,
                            int32_t group, void* out, int64_t T, int64_t H,
                            int64_t I, int32_t E, int32_t top_k, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Device bounds checks (debug build).  libmoe_ffn_debug.so is the same
 * library compiled with -DMOE_FFN_DEVICE_CHECKS: before its kernels' global
 * accesses (weight rows, gathered token rows, h and y rows) an index outside
 * its buffer is recorded and the access skipped or redirected to row 0, so a
 * bad index shows up here instead of as a memory fault.  This call waits for
 * the device, then writes to *where the first failed check since the last
 * call, as (source file number) * 100000 + source line (files: 1
 * route_permute, 2 expert_gemm, 3 expert_tile, 4 combine, 5 attn_decode), or
 * 0 if none, and clears the record.  Returns 1 for the debug build, 0 for
 * the release build (whose kernels carry no checks: *where is always 0), or
 * MOE_FFN_ERR_NULL_ARG / MOE_FFN_ERR_HIP.  A debugging aid for the callers
 * and tests of this library, not one of the pages' operations. */
int moe_ffn_device_check(int32_t* where);

/* Wait for `stream`, then read the workspace meta written by the last forward
 * call: MOE_FFN_ERR_BAD_IDS if it dropped slots with out-of-range ids,
 * MOE_FFN_OK otherwise (MOE_FFN_ERR_HIP if the wait or the read fails).  If
 * n_dropped is not NULL it receives the number of dropped slots. */
int moe_ffn_check_status(const void* workspace, void* stream, int64_t* n_dropped);

/* Static description of a status code (never NULL). */
const char* moe_ffn_status_string(int status);

/*
 * Benchmark hook: per-kernel timing with HIP events.  After this call, the
 * next forward call made by the calling host thread (either weight format)
 * records events[i] on its stream right after enqueuing kernel i, for
 * i < n_events: 0 = gather index (permute; for moe_ffn_forward_logits the
 * router and gather index), 1 = gate/up, 2 = down, 3 = combine; for
 * moe_attn_decode, 0 = the split kernel (scores, softmax and values per
 * split of positions) and 1 = the merge of the splits.  The events are hipEvent_t handles owned by the caller.  The
 * setting is consumed by that one call; n_events = 0 (or events = NULL)
 * clears it.  Only the calling thread is affected.  Returns MOE_FFN_OK, or
 * MOE_FFN_ERR_BAD_SHAPE if n_events is outside [0, 4].
 */
int moe_ffn_set_stage_events(void* const* events, int32_t n_events);

/*
 * Test hook: force the number of K parts per row block of the gate/up and of
 * the down product (1, 2 or 4) for the forward calls (either weight format)
 * made by the calling host thread from now on; 0 restores the choice the
 * kernels make on the device from the active-expert count.  The result of a
 * call does not depend on the split beyond FP32 summation order.  Returns
 * MOE_FFN_OK, or MOE_FFN_ERR_BAD_SHAPE for a value outside {0, 1, 2, 4}.
 */
int moe_ffn_set_split(int32_t gate_up_split, int32_t down_split);

/*
 * Measurement helper: the HBM streaming-read ceiling that the expert
 * products are compared against (the GPU counterpart of the STREAM bandwidth
 * the HiNa-MoE evaluation reports for its CPUs, Table 2).  Enqueues on
 * `stream` one kernel that reads each of the `bytes` bytes of device buffer
 * `buf` once, with 16-byte loads, from a grid that fills the device; it
 * writes nothing but, rarely, one 32-bit word at device address `sink`.
 * `bytes` must be a positive multiple of 16, `buf` 16-byte aligned and
 * `sink` 4-byte aligned.  Returns MOE_FFN_OK, MOE_FFN_ERR_NULL_ARG,
 * MOE_FFN_ERR_BAD_SHAPE, MOE_FFN_ERR_MISALIGNED or MOE_FFN_ERR_HIP.
 */
int moe_ffn_read_probe(const void* buf, size_t bytes, void* sink, void* stream);

/*
 * Measurement helper: the dispatch gap between back-to-back kernels.
 * Enqueues n launches of an empty one-wave kernel on `stream`; the GPU time
 * of the chain divided by n is the fixed cost one more kernel adds to a layer
 * (the floor under the four launches of a forward call).  n in [0, 10^6].
 * Returns MOE_FFN_OK, MOE_FFN_ERR_BAD_SHAPE or MOE_FFN_ERR_HIP.
 */
int moe_ffn_launch_probe(int32_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
