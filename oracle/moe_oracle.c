/*
 * moe_oracle.c -- plain CPU oracle for the routed-expert MoE FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library it checks; both sides receive
 * the same seeded inputs and nothing else.
 *
 * Every routine here is the plain definition of one step, written as
 * straight loops in the order the definition states, with no blocking, no
 * fusion and no reordering of sums.  Built with -ffp-contract=off and without
 * -ffast-math so that every "a += b * c" is one IEEE multiply followed by one
 * IEEE add, in the written order.
 *
 * Source of the method: "HiNa-MoE: High-Performance, Non-Intrusive MoE
 * Inference on CPUs with Matrix Engines" (arXiv 2610.05123).
 *   - §2.1 (MoE architecture, Fig. 2): a gating function sends each token to
 *     a small subset of experts; Table 3 gives top-2 (Mixtral) and top-8
 *     (DeepSeek-V3, Qwen3).
 *   - §4.1 (FFN equation): FFN(I) = SiLU(I*Wgate) (.) (I*Wup) * Wdown, applied
 *     to the matrix I of the tokens gathered for one expert.  Gathering and
 *     the layout transforms change only where data sits, never the values, so
 *     the per-token form below is the same function.
 *   - §4.2.1 (Eq. 1 and the text after it): the matrix engine multiplies
 *     BF16 operands and accumulates in FP32.  The intermediate SiLU*up result
 *     is written as the operand of the next (down) product, i.e. as BF16
 *     (§4.1, second transform).
 *   - §8.1 (Fig. 11): an INT8 variant with symmetric group-wise quantisation.
 *   - §6.1 (SDPA in decoding, GQA): each KV head is shared by h_q/h_kv query
 *     heads; per query head, scaled dot-product scores against the l_seq keys,
 *     a softmax over the sequence, and the weighted sum of the values.
 * and, for the residual-split weights, "RapidMoE" (the page on hybrid
 * CPU-GPU MoE inference): "Residual-Split Representation" (W^Q, then the
 * residual W - W^Q quantised as W^R; high precision W^Q + W^R, low W^Q),
 * "GLU Architecture Adoption" (the split for gate/up only, two quantised
 * copies of down) and "Expert-Residual Offloading" (h_gate/up = W^Q x +
 * W^R x).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - router: softmax over all experts, the k largest kept (ties -> lower
 *     expert id), weights renormalised over the k kept; the grouped sigmoid
 *     variant as stated at oracle_route_grouped;
 *   - h = RNE_bf16( silu(g) * u ) with g, u and silu(g) kept in FP32;
 *   - out[t] = RNE_bf16( sum_j w[t,j] * y_j ), summed in FP32 over ascending j,
 *     where y_j is the FP32 down-projection output (not rounded);
 *   - a slot whose expert id is outside [0, E) contributes nothing;
 *   - INT8: w = q * s with one FP32 scale s per 128 consecutive K elements of
 *     a row; g = sum_groups s_g * (sum_{c in group} x_c * q_c), in FP32.
 *   - residual split: W^Q, W^R and the low-precision down copy are INT4
 *     (integers in [-8, 7]), the high-precision down copy INT8, each with one
 *     FP32 scale per 128 K; a per-expert flag chooses the precision;
 *   - attention: query head h reads KV head h / (h_q / h_kv); the score scale
 *     is 1/sqrt(d) unless the caller gives another; scores, softmax and the
 *     weighted sum in FP32 (BF16 inputs); the output rounded once to BF16; an
 *     empty sequence gives a zero output.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_MISSING_EXPERT (-2)
#define ORACLE_ERR_NOMEM (-3)

/* Threads the OpenMP loops below will use (reported with CPU timings). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Set that thread count (n >= 1); used to time a single-thread run.  The
 * results do not depend on it: the loops split only independent outputs. */
void oracle_set_num_threads(int n) {
    if (n >= 1) omp_set_num_threads(n);
}

/* ---------------------------------------------------------------------- */
/* BF16 <-> FP32.  BF16 is the upper half of an IEEE binary32 word.        */
/* ---------------------------------------------------------------------- */

float oracle_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round-to-nearest, ties-to-even, on the bit pattern: add 0x7FFF plus the
 * lowest kept bit, then drop the low 16 bits.  A NaN keeps its sign and is
 * forced quiet so that rounding can never turn it into an infinity. */
uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7fffu + keep_lsb;
    return (uint16_t)(u >> 16);
}

void oracle_f32_to_bf16_array(const float* src, uint16_t* dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_f32_to_bf16(src[i]);
}

/* ---------------------------------------------------------------------- */
/* Routing (§2.1, Fig. 2; Table 3 for k).                                 */
/* ---------------------------------------------------------------------- */

/* For each token t: choose k experts by descending logit (softmax is strictly
 * increasing, so this is the order of the probabilities), ties broken toward
 * the lower expert id; then softmax over all E logits in double precision and
 * renormalise the k chosen probabilities to sum to one.  Slot j of token t
 * holds the j-th largest.  Returns ORACLE_OK. */
int oracle_route_topk(const float* logits, int64_t T, int32_t E, int32_t k,
                      int32_t* topk_ids, float* topk_w) {
    if (T < 0 || E <= 0 || k <= 0 || k > E) return ORACLE_ERR_ARG;
    unsigned char* chosen = (unsigned char*)malloc((size_t)E);
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    if (!chosen || !p) { free(chosen); free(p); return ORACLE_ERR_NOMEM; }
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        memset(chosen, 0, (size_t)E);
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (chosen[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            chosen[best] = 1;
            topk_ids[t * k + j] = best;
        }
        double mx = -INFINITY;
        for (int32_t e = 0; e < E; ++e)
            if ((double)l[e] > mx) mx = (double)l[e];
        double z = 0.0;
        for (int32_t e = 0; e < E; ++e) {
            p[e] = exp((double)l[e] - mx);
            z += p[e];
        }
        for (int32_t e = 0; e < E; ++e) p[e] /= z;
        double kept = 0.0;
        for (int32_t j = 0; j < k; ++j) kept += p[topk_ids[t * k + j]];
        for (int32_t j = 0; j < k; ++j)
            topk_w[t * k + j] = (float)(p[topk_ids[t * k + j]] / kept);
    }
    free(chosen);
    free(p);
    return ORACLE_OK;
}

/* Grouped sigmoid routing, the variant of the gate used by DeepSeek-V3
 * (one of the models of HiNa-MoE's Table 3 and RapidMoE's evaluation; the
 * pages name the model but do not spell out its gate).  For each token t:
 *   s_e = 1 / (1 + exp(-l_e))                 (FP32)
 *   c_e = s_e + bias_e                        (selection score; bias may be NULL = 0)
 *   the E experts form n_group groups of G = E / n_group consecutive ids;
 *   group score = the largest c in the group plus the second largest
 *     (the largest alone when G = 1), added in that order;
 *   keep the topk_group groups of highest score (ties -> lower group id);
 *   choose k experts of the kept groups by descending c (ties -> lower id);
 *   w_j = scale * s_{e_j} / (s_{e_0} + ... + s_{e_{k-1}}), the sum in
 *     ascending j, then the division, then the multiplication (FP32).
 * Slot j of token t holds the j-th choice.  Returns ORACLE_OK, or
 * ORACLE_ERR_ARG for inconsistent sizes. */
int oracle_route_grouped(const float* logits, const float* bias, int64_t T, int32_t E,
                         int32_t n_group, int32_t topk_group, int32_t k, float scale,
                         int32_t* topk_ids, float* topk_w) {
    if (T < 0 || E <= 0 || n_group <= 0 || E % n_group != 0 || topk_group <= 0 ||
        topk_group > n_group || k <= 0 || k > topk_group * (E / n_group))
        return ORACLE_ERR_ARG;
    const int32_t G = E / n_group;
    float* s = (float*)malloc(sizeof(float) * (size_t)E);
    float* c = (float*)malloc(sizeof(float) * (size_t)E);
    float* gs = (float*)malloc(sizeof(float) * (size_t)n_group);
    unsigned char* kept = (unsigned char*)malloc((size_t)n_group);
    unsigned char* chosen = (unsigned char*)malloc((size_t)E);
    if (!s || !c || !gs || !kept || !chosen) {
        free(s); free(c); free(gs); free(kept); free(chosen);
        return ORACLE_ERR_NOMEM;
    }
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        for (int32_t e = 0; e < E; ++e) {
            s[e] = 1.0f / (1.0f + expf(-l[e]));
            c[e] = s[e] + (bias ? bias[e] : 0.0f);
        }
        for (int32_t g = 0; g < n_group; ++g) {
            /* largest, then second largest, of the group's selection scores */
            int32_t b1 = -1, b2 = -1;
            for (int32_t e = g * G; e < (g + 1) * G; ++e)
                if (b1 < 0 || c[e] > c[b1]) b1 = e;
            for (int32_t e = g * G; e < (g + 1) * G; ++e)
                if (e != b1 && (b2 < 0 || c[e] > c[b2])) b2 = e;
            gs[g] = b2 < 0 ? c[b1] : c[b1] + c[b2];
        }
        memset(kept, 0, (size_t)n_group);
        for (int32_t j = 0; j < topk_group; ++j) {
            int32_t best = -1;
            for (int32_t g = 0; g < n_group; ++g)
                if (!kept[g] && (best < 0 || gs[g] > gs[best])) best = g;
            kept[best] = 1;
        }
        memset(chosen, 0, (size_t)E);
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (chosen[e] || !kept[e / G]) continue;
                if (best < 0 || c[e] > c[best]) best = e;
            }
            chosen[best] = 1;
            topk_ids[t * k + j] = best;
        }
        float sum = 0.0f;
        for (int32_t j = 0; j < k; ++j) sum += s[topk_ids[t * k + j]];
        for (int32_t j = 0; j < k; ++j)
            topk_w[t * k + j] = s[topk_ids[t * k + j]] / sum * scale;
    }
    free(s); free(c); free(gs); free(kept); free(chosen);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* Token gathering index (§4.1: the routed tokens of one expert are        */
/* gathered into one matrix I).                                            */
/* ---------------------------------------------------------------------- */

/* Slot s = t*k + j names the j-th expert choice of token t.  For experts in
 * ascending order, list the slots routed to that expert in ascending slot
 * order.  offsets[e] is where expert e's list starts (offsets[E] = number of
 * listed slots); active[] lists the experts with at least one slot, ascending,
 * and *n_active is their number.  Slots whose id is outside [0, E) are left
 * out.  Returns the number of such slots (>= 0). */
int64_t oracle_permute(const int32_t* topk_ids, int64_t n_slots, int32_t E,
                       int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                       int32_t* active, int32_t* n_active) {
    int32_t pos = 0, na = 0;
    for (int32_t e = 0; e < E; ++e) {
        offsets[e] = pos;
        for (int64_t s = 0; s < n_slots; ++s)
            if (topk_ids[s] == e) sorted_slot[pos++] = (int32_t)s;
        counts[e] = pos - offsets[e];
        if (counts[e] > 0) active[na++] = e;
    }
    offsets[E] = pos;
    *n_active = na;
    int64_t invalid = 0;
    for (int64_t s = 0; s < n_slots; ++s)
        if (topk_ids[s] < 0 || topk_ids[s] >= E) ++invalid;
    return invalid;
}

/* ---------------------------------------------------------------------- */
/* One expert applied to one token, BF16 weights (§4.1 FFN equation;       */
/* §4.2.1: BF16 operands, FP32 accumulation).                              */
/* ---------------------------------------------------------------------- */

/* x: [H] bf16.  Wg, Wu: [I][H] bf16 (row i holds the H weights that produce
 * intermediate feature i).  Wd: [H][I] bf16 (row n produces output feature n).
 * h (out): [I] bf16.  y (out): [H] fp32. */
void oracle_expert_ffn_bf16(const uint16_t* x, const uint16_t* Wg,
                            const uint16_t* Wu, const uint16_t* Wd, int64_t H,
                            int64_t I, uint16_t* h, float* y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < I; ++i) {
        float g = 0.0f, u = 0.0f;
        for (int64_t c = 0; c < H; ++c)
            g += oracle_bf16_to_f32(x[c]) * oracle_bf16_to_f32(Wg[i * H + c]);
        for (int64_t c = 0; c < H; ++c)
            u += oracle_bf16_to_f32(x[c]) * oracle_bf16_to_f32(Wu[i * H + c]);
        float silu_g = g / (1.0f + expf(-g));
        h[i] = oracle_f32_to_bf16(silu_g * u);
    }
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < H; ++n) {
        float acc = 0.0f;
        for (int64_t i = 0; i < I; ++i)
            acc += oracle_bf16_to_f32(h[i]) * oracle_bf16_to_f32(Wd[n * I + i]);
        y[n] = acc;
    }
}

/* ---------------------------------------------------------------------- */
/* One expert applied to one token, INT8 group-quantised weights (§8.1,    */
/* Fig. 11: symmetric group-wise INT8; group size read as 128 along K).    */
/* ---------------------------------------------------------------------- */

/* Each weight row r of length K is q[r][0..K) (int8) with one fp32 scale per
 * group of `group` consecutive elements: s[r][0..K/group).  The dot product of
 * a row with a vector v is  sum_g s[r][g] * (sum_{c in group g} v_c * q[r][c]),
 * all in FP32 with ascending c inside a group and ascending g outside. */
static float grouped_dot(const uint16_t* v, const int8_t* q, const float* s,
                         int64_t K, int64_t group) {
    float acc = 0.0f;
    for (int64_t g0 = 0; g0 < K; g0 += group) {
        float part = 0.0f;
        for (int64_t c = g0; c < g0 + group; ++c)
            part += oracle_bf16_to_f32(v[c]) * (float)q[c];
        acc += s[g0 / group] * part;
    }
    return acc;
}

void oracle_expert_ffn_int8(const uint16_t* x, const int8_t* Qg, const float* Sg,
                            const int8_t* Qu, const float* Su, const int8_t* Qd,
                            const float* Sd, int64_t group, int64_t H, int64_t I,
                            uint16_t* h, float* y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < I; ++i) {
        float g = grouped_dot(x, Qg + i * H, Sg + i * (H / group), H, group);
        float u = grouped_dot(x, Qu + i * H, Su + i * (H / group), H, group);
        float silu_g = g / (1.0f + expf(-g));
        h[i] = oracle_f32_to_bf16(silu_g * u);
    }
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < H; ++n)
        y[n] = grouped_dot(h, Qd + n * I, Sd + n * (I / group), I, group);
}

/* ---------------------------------------------------------------------- */
/* The routed-expert FFN layer, per-token definition.                      */
/* ---------------------------------------------------------------------- */

/* out[t] = RNE_bf16( sum_{j<k} w[t,j] * FFN_{ids[t,j]}(x[t]) ), FP32 sum over
 * ascending j.  Weight tables hold one pointer per expert; an expert that no
 * valid slot uses may be NULL.  Optional outputs (may be NULL):
 *   out_f32 [T][H]    the FP32 sum before the final rounding;
 *   h_out   [T*k][I]  the BF16 intermediate of every slot (zero when dropped);
 *   y_out   [T*k][H]  the FP32 down output of every slot (zero when dropped).
 * Returns ORACLE_OK, or ORACLE_ERR_MISSING_EXPERT if a valid slot names an
 * expert whose pointers are NULL. */
static int moe_layer(int int8, const uint16_t* x, const int32_t* ids,
                     const float* w, const void* const* Wg, const float* const* Sg,
                     const void* const* Wu, const float* const* Su,
                     const void* const* Wd, const float* const* Sd, int64_t group,
                     int64_t T, int64_t H, int64_t I, int32_t E, int32_t k,
                     uint16_t* out, float* out_f32, uint16_t* h_out, float* y_out) {
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0) return ORACLE_ERR_ARG;
    float* acc = (float*)malloc(sizeof(float) * (size_t)H);
    float* y = (float*)malloc(sizeof(float) * (size_t)H);
    uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
    if (!acc || !y || !h) { free(acc); free(y); free(h); return ORACLE_ERR_NOMEM; }
    int rc = ORACLE_OK;
    for (int64_t t = 0; t < T && rc == ORACLE_OK; ++t) {
        for (int64_t n = 0; n < H; ++n) acc[n] = 0.0f;
        for (int32_t j = 0; j < k; ++j) {
            int64_t slot = t * k + j;
            int32_t e = ids[slot];
            if (h_out) memset(h_out + slot * I, 0, sizeof(uint16_t) * (size_t)I);
            if (y_out) memset(y_out + slot * H, 0, sizeof(float) * (size_t)H);
            if (e < 0 || e >= E) continue; /* dropped slot */
            if (!Wg[e] || !Wu[e] || !Wd[e] ||
                (int8 && (!Sg[e] || !Su[e] || !Sd[e]))) {
                rc = ORACLE_ERR_MISSING_EXPERT;
                break;
            }
            if (int8)
                oracle_expert_ffn_int8(x + t * H, (const int8_t*)Wg[e], Sg[e],
                                       (const int8_t*)Wu[e], Su[e],
                                       (const int8_t*)Wd[e], Sd[e], group, H, I, h, y);
            else
                oracle_expert_ffn_bf16(x + t * H, (const uint16_t*)Wg[e],
                                       (const uint16_t*)Wu[e],
                                       (const uint16_t*)Wd[e], H, I, h, y);
            for (int64_t n = 0; n < H; ++n) acc[n] += w[slot] * y[n];
            if (h_out) memcpy(h_out + slot * I, h, sizeof(uint16_t) * (size_t)I);
            if (y_out) memcpy(y_out + slot * H, y, sizeof(float) * (size_t)H);
        }
        for (int64_t n = 0; n < H; ++n) {
            out[t * H + n] = oracle_f32_to_bf16(acc[n]);
            if (out_f32) out_f32[t * H + n] = acc[n];
        }
    }
    free(acc);
    free(y);
    free(h);
    return rc;
}

int oracle_moe_ffn_bf16(const uint16_t* x, const int32_t* topk_ids,
                        const float* topk_w, const uint16_t* const* W_gate,
                        const uint16_t* const* W_up, const uint16_t* const* W_down,
                        int64_t T, int64_t H, int64_t I, int32_t E, int32_t k,
                        uint16_t* out, float* out_f32, uint16_t* h_out,
                        float* y_out) {
    return moe_layer(0, x, topk_ids, topk_w, (const void* const*)W_gate, NULL,
                     (const void* const*)W_up, NULL, (const void* const*)W_down,
                     NULL, 0, T, H, I, E, k, out, out_f32, h_out, y_out);
}

int oracle_moe_ffn_int8(const uint16_t* x, const int32_t* topk_ids,
                        const float* topk_w, const int8_t* const* Q_gate,
                        const float* const* S_gate, const int8_t* const* Q_up,
                        const float* const* S_up, const int8_t* const* Q_down,
                        const float* const* S_down, int64_t group, int64_t T,
                        int64_t H, int64_t I, int32_t E, int32_t k, uint16_t* out,
                        float* out_f32, uint16_t* h_out, float* y_out) {
    if (group <= 0 || H % group != 0 || I % group != 0) return ORACLE_ERR_ARG;
    return moe_layer(1, x, topk_ids, topk_w, (const void* const*)Q_gate, S_gate,
                     (const void* const*)Q_up, S_up, (const void* const*)Q_down,
                     S_down, group, T, H, I, E, k, out, out_f32, h_out, y_out);
}

/* ---------------------------------------------------------------------- */
/* Residual-split low-bit weights (RapidMoE: "Residual-Split               */
/* Representation", "GLU Architecture Adoption", "Expert-Residual          */
/* Offloading").                                                           */
/* ---------------------------------------------------------------------- */

/* W^Q is the weight quantised group-wise; W^R is the residual W - W^Q
 * quantised the same way.  The high-precision gate and up projections use
 * W^H = W^Q + W^R through the linear split x W^H = x W^Q + x W^R; the low
 * precision ones use W^Q alone.  down_proj is not split: it is stored as two
 * separately quantised copies, one of high and one of low precision.  An
 * expert flagged critical runs in high precision, every other in low.
 *
 * One expert on one token:
 *   g = gdot(x, Q_gate, S_gate) [+ gdot(x, R_gate, SR_gate) if critical]
 *   u = gdot(x, Q_up,   S_up)   [+ gdot(x, R_up,   SR_up)   if critical]
 *   h = RNE_bf16( silu(g) * u )
 *   y = gdot(h, Q_down, S_down)   (the high or the low copy)
 * with gdot the grouped dot product above, each term in FP32 and the two
 * terms added in the written order.  All q arrays hold integers as int8. */
void oracle_expert_ffn_resplit(const uint16_t* x, const int8_t* Qg, const float* Sg,
                               const int8_t* Rg, const float* SRg, const int8_t* Qu,
                               const float* Su, const int8_t* Ru, const float* SRu,
                               const int8_t* Qd, const float* Sd, int critical,
                               int64_t group, int64_t H, int64_t I, uint16_t* h,
                               float* y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < I; ++i) {
        float g = grouped_dot(x, Qg + i * H, Sg + i * (H / group), H, group);
        float u = grouped_dot(x, Qu + i * H, Su + i * (H / group), H, group);
        if (critical) {
            g = g + grouped_dot(x, Rg + i * H, SRg + i * (H / group), H, group);
            u = u + grouped_dot(x, Ru + i * H, SRu + i * (H / group), H, group);
        }
        float silu_g = g / (1.0f + expf(-g));
        h[i] = oracle_f32_to_bf16(silu_g * u);
    }
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < H; ++n)
        y[n] = grouped_dot(h, Qd + n * I, Sd + n * (I / group), I, group);
}

/* The layer as in moe_layer, with the precision of each slot's expert taken
 * from critical[e] (nonzero: high).  Tables are per expert; those of a
 * precision that no valid slot uses may be NULL (R, SR and the high down copy
 * of non-critical experts, the low down copy of critical ones). */
int oracle_moe_ffn_resplit(const uint16_t* x, const int32_t* ids, const float* w,
                           const int8_t* const* Qg, const float* const* Sg,
                           const int8_t* const* Rg, const float* const* SRg,
                           const int8_t* const* Qu, const float* const* Su,
                           const int8_t* const* Ru, const float* const* SRu,
                           const int8_t* const* Qd_lo, const float* const* Sd_lo,
                           const int8_t* const* Qd_hi, const float* const* Sd_hi,
                           const uint8_t* critical, int64_t group, int64_t T, int64_t H,
                           int64_t I, int32_t E, int32_t k, uint16_t* out,
                           float* out_f32, uint16_t* h_out, float* y_out) {
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0) return ORACLE_ERR_ARG;
    if (group <= 0 || H % group != 0 || I % group != 0) return ORACLE_ERR_ARG;
    float* acc = (float*)malloc(sizeof(float) * (size_t)H);
    float* y = (float*)malloc(sizeof(float) * (size_t)H);
    uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
    if (!acc || !y || !h) { free(acc); free(y); free(h); return ORACLE_ERR_NOMEM; }
    int rc = ORACLE_OK;
    for (int64_t t = 0; t < T && rc == ORACLE_OK; ++t) {
        for (int64_t n = 0; n < H; ++n) acc[n] = 0.0f;
        for (int32_t j = 0; j < k; ++j) {
            int64_t slot = t * (int64_t)k + j;
            int32_t e = ids[slot];
            if (h_out) memset(h_out + slot * I, 0, sizeof(uint16_t) * (size_t)I);
            if (y_out) memset(y_out + slot * H, 0, sizeof(float) * (size_t)H);
            if (e < 0 || e >= E) continue; /* dropped slot */
            int crit = critical[e] != 0;
            const int8_t* qd = crit ? Qd_hi[e] : Qd_lo[e];
            const float* sd = crit ? Sd_hi[e] : Sd_lo[e];
            if (!Qg[e] || !Sg[e] || !Qu[e] || !Su[e] || !qd || !sd ||
                (crit && (!Rg[e] || !SRg[e] || !Ru[e] || !SRu[e]))) {
                rc = ORACLE_ERR_MISSING_EXPERT;
                break;
            }
            oracle_expert_ffn_resplit(x + t * H, Qg[e], Sg[e], crit ? Rg[e] : NULL,
                                      crit ? SRg[e] : NULL, Qu[e], Su[e],
                                      crit ? Ru[e] : NULL, crit ? SRu[e] : NULL, qd, sd,
                                      crit, group, H, I, h, y);
            const float wt = w[slot];
            for (int64_t n = 0; n < H; ++n) acc[n] += wt * y[n];
            if (h_out) memcpy(h_out + slot * I, h, sizeof(uint16_t) * (size_t)I);
            if (y_out) memcpy(y_out + slot * H, y, sizeof(float) * (size_t)H);
        }
        for (int64_t n = 0; n < H; ++n) {
            out[t * H + n] = oracle_f32_to_bf16(acc[n]);
            if (out_f32) out_f32[t * H + n] = acc[n];
        }
    }
    free(acc);
    free(y);
    free(h);
    return rc;
}

/* ---------------------------------------------------------------------- */
/* Decode attention with grouped-query heads (§6.1).                       */
/* ---------------------------------------------------------------------- */

/* q   [B][h_q][d] BF16: one query vector per sequence and query head.
 * k, v [B][h_kv][max_len][d] BF16: the cached keys and values; sequence b
 *     uses its first len[b] positions (0 <= len[b] <= max_len).
 * out [B][h_q][d] BF16.
 * For sequence b and query head h (KV head j = h / (h_q / h_kv)):
 *   s_t = scale * sum_{c < d} q[c] * k[t][c]          (FP32, ascending c)
 *   m = max_t s_t;  e_t = exp(s_t - m);  L = sum_t e_t (FP32, ascending t)
 *   out[c] = RNE_bf16( (sum_t e_t * v[t][c]) / L )    (FP32, ascending t)
 * which is softmax(s) weighted over v; len[b] = 0 gives out = 0.
 * Returns ORACLE_OK, or ORACLE_ERR_ARG for inconsistent sizes. */
int oracle_attn_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const int32_t* len, int32_t B, int32_t h_q, int32_t h_kv,
                       int32_t d, int32_t max_len, float scale, uint16_t* out) {
    if (B < 0 || h_q < 1 || h_kv < 1 || d < 1 || max_len < 0 || h_q % h_kv != 0)
        return ORACLE_ERR_ARG;
    for (int32_t b = 0; b < B; ++b)
        if (len[b] < 0 || len[b] > max_len) return ORACLE_ERR_ARG;
    const int32_t g = h_q / h_kv;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic) collapse(2)
    for (int32_t b = 0; b < B; ++b) {
        for (int32_t h = 0; h < h_q; ++h) {
            const int32_t j = h / g;
            const int32_t n = len[b];
            const uint16_t* qh = q + ((size_t)b * h_q + h) * d;
            const uint16_t* kh = k + ((size_t)b * h_kv + j) * (size_t)max_len * d;
            const uint16_t* vh = v + ((size_t)b * h_kv + j) * (size_t)max_len * d;
            uint16_t* oh = out + ((size_t)b * h_q + h) * d;
            if (n == 0) {
                for (int32_t c = 0; c < d; ++c) oh[c] = 0;
                continue;
            }
            float* s = (float*)malloc(sizeof(float) * (size_t)n);
            float* acc = (float*)malloc(sizeof(float) * (size_t)d);
            if (!s || !acc) {
                free(s);
                free(acc);
#pragma omp atomic write
                status = ORACLE_ERR_NOMEM;
                continue;
            }
            for (int32_t t = 0; t < n; ++t) {
                float dot = 0.0f;
                for (int32_t c = 0; c < d; ++c)
                    dot += oracle_bf16_to_f32(qh[c]) * oracle_bf16_to_f32(kh[(size_t)t * d + c]);
                s[t] = scale * dot;
            }
            float m = s[0];
            for (int32_t t = 1; t < n; ++t)
                if (s[t] > m) m = s[t];
            float L = 0.0f;
            for (int32_t t = 0; t < n; ++t) {
                s[t] = expf(s[t] - m);
                L += s[t];
            }
            for (int32_t c = 0; c < d; ++c) acc[c] = 0.0f;
            for (int32_t t = 0; t < n; ++t)
                for (int32_t c = 0; c < d; ++c)
                    acc[c] += s[t] * oracle_bf16_to_f32(vh[(size_t)t * d + c]);
            for (int32_t c = 0; c < d; ++c) oh[c] = oracle_f32_to_bf16(acc[c] / L);
            free(s);
            free(acc);
        }
    }
    return status;
}
