/*
 * Memory-safety driver for the CPU oracle (oracle/moe_oracle.c), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitizers.py.  It calls every oracle entry point on
 * small seeded inputs whose buffers are allocated at their exact sizes (one
 * allocation per tensor and expert, so that a read or write past any of them
 * is caught), including the edge cases the oracle handles: an empty batch,
 * one expert, top_k = E, out-of-range and duplicate expert ids, experts that
 * no slot names (their weight pointers are NULL and must not be read), and
 * empty and full attention sequences.  Exit status 0: every call returned
 * success and no sanitizer fired (the sanitizers abort on the first error).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_ids,
                      float* topk_w);
int oracle_route_grouped(const float* logits, const float* bias, int64_t T, int32_t E,
                         int32_t n_group, int32_t topk_group, int32_t k, float scale,
                         int32_t* topk_ids, float* topk_w);
int64_t oracle_permute(const int32_t* topk_ids, int64_t n_slots, int32_t E, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_slot, int32_t* active,
                       int32_t* n_active);
int oracle_moe_ffn_bf16(const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                        const uint16_t* const* W_gate, const uint16_t* const* W_up,
                        const uint16_t* const* W_down, int64_t T, int64_t H, int64_t I,
                        int32_t E, int32_t k, uint16_t* out, float* out_f32, uint16_t* h_out,
                        float* y_out);
int oracle_moe_ffn_int8(const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                        const int8_t* const* Q_gate, const float* const* S_gate,
                        const int8_t* const* Q_up, const float* const* S_up,
                        const int8_t* const* Q_down, const float* const* S_down, int64_t group,
                        int64_t T, int64_t H, int64_t I, int32_t E, int32_t k, uint16_t* out,
                        float* out_f32, uint16_t* h_out, float* y_out);
int oracle_moe_ffn_resplit(const uint16_t* x, const int32_t* ids, const float* w,
                           const int8_t* const* Qg, const float* const* Sg,
                           const int8_t* const* Rg, const float* const* SRg,
                           const int8_t* const* Qu, const float* const* Su,
                           const int8_t* const* Ru, const float* const* SRu,
                           const int8_t* const* Qd_lo, const float* const* Sd_lo,
                           const int8_t* const* Qd_hi, const float* const* Sd_hi,
                           const uint8_t* critical, int64_t group, int64_t T, int64_t H,
                           int64_t I, int32_t E, int32_t k, uint16_t* out, float* out_f32,
                           uint16_t* h_out, float* y_out);
int oracle_attn_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const int32_t* len, int32_t B, int32_t h_q, int32_t h_kv, int32_t d,
                       int32_t max_len, float scale, uint16_t* out);

static uint32_t g_rng = 0x9e3779b9u;
static uint32_t next_u32(void) {  /* xorshift32 */
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 17;
    g_rng ^= g_rng << 5;
    return g_rng;
}
static float next_f(void) { return (float)((int32_t)(next_u32() % 2001) - 1000) / 1000.0f; }
static void* xalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}
static uint16_t bf16_bits(float f) {  /* truncation suffices for test inputs */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}
static uint16_t* bf16_array(size_t n, float scale) {
    uint16_t* a = (uint16_t*)xalloc(n * 2);
    for (size_t i = 0; i < n; ++i) a[i] = bf16_bits(next_f() * scale);
    return a;
}
static int8_t* q_array(size_t n, int qmax) {
    int8_t* a = (int8_t*)xalloc(n);
    for (size_t i = 0; i < n; ++i) a[i] = (int8_t)((int)(next_u32() % (2 * qmax + 1)) - qmax);
    return a;
}
static float* f_array(size_t n, float scale) {
    float* a = (float*)xalloc(n * 4);
    for (size_t i = 0; i < n; ++i) a[i] = next_f() * scale;
    return a;
}
static int fails = 0;
static void check(int rc, const char* what) {
    if (rc != 0) { fprintf(stderr, "%s returned %d\n", what, rc); ++fails; }
}

/* One layer case through router, permute and the three FFN variants. */
static void layer_case(int64_t T, int64_t H, int64_t I, int32_t E, int32_t k, int bad_ids) {
    const int64_t S = T * k;
    float* logits = f_array((size_t)(T * E), 2.0f);
    int32_t* ids = (int32_t*)xalloc((size_t)S * 4);
    float* w = (float*)xalloc((size_t)S * 4);
    check(oracle_route_topk(logits, T, E, k, ids, w), "route_topk");
    if (bad_ids && S >= 3) {
        ids[0] = E;          /* out of range: dropped */
        ids[1] = -1;         /* out of range: dropped */
        ids[2] = ids[S - 1]; /* a duplicate */
    }
    int32_t* counts = (int32_t*)xalloc((size_t)E * 4);
    int32_t* offsets = (int32_t*)xalloc(((size_t)E + 1) * 4);
    int32_t* sorted = (int32_t*)xalloc((size_t)S * 4);
    int32_t* active = (int32_t*)xalloc((size_t)E * 4);
    int32_t n_active = 0;
    const int64_t dropped = oracle_permute(ids, S, E, counts, offsets, sorted, active, &n_active);
    if (dropped < 0) check(-1, "permute");
    /* weights of the experts some valid slot names; the others stay NULL */
    uint16_t **Wg = calloc((size_t)E, sizeof(void*)), **Wu = calloc((size_t)E, sizeof(void*)),
             **Wd = calloc((size_t)E, sizeof(void*));
    int8_t **Qg = calloc((size_t)E, sizeof(void*)), **Qu = calloc((size_t)E, sizeof(void*)),
           **Qd = calloc((size_t)E, sizeof(void*)), **Rg = calloc((size_t)E, sizeof(void*)),
           **Ru = calloc((size_t)E, sizeof(void*)), **Qdh = calloc((size_t)E, sizeof(void*));
    float **Sg = calloc((size_t)E, sizeof(void*)), **Su = calloc((size_t)E, sizeof(void*)),
          **Sd = calloc((size_t)E, sizeof(void*)), **SRg = calloc((size_t)E, sizeof(void*)),
          **SRu = calloc((size_t)E, sizeof(void*)), **Sdh = calloc((size_t)E, sizeof(void*));
    uint8_t* critical = (uint8_t*)xalloc((size_t)E);
    const int64_t G = 128;
    const int quant = H % G == 0 && I % G == 0;
    for (int32_t e = 0; e < E; ++e) {
        critical[e] = (uint8_t)(e & 1);
        if (counts[e] == 0) continue;
        Wg[e] = bf16_array((size_t)(I * H), 0.05f);
        Wu[e] = bf16_array((size_t)(I * H), 0.05f);
        Wd[e] = bf16_array((size_t)(H * I), 0.05f);
        if (!quant) continue;
        Qg[e] = q_array((size_t)(I * H), 127);
        Qu[e] = q_array((size_t)(I * H), 127);
        Qd[e] = q_array((size_t)(H * I), 127);
        Rg[e] = q_array((size_t)(I * H), 7);
        Ru[e] = q_array((size_t)(I * H), 7);
        Qdh[e] = q_array((size_t)(H * I), 127);
        Sg[e] = f_array((size_t)(I * H / G), 0.01f);
        Su[e] = f_array((size_t)(I * H / G), 0.01f);
        Sd[e] = f_array((size_t)(H * I / G), 0.01f);
        SRg[e] = f_array((size_t)(I * H / G), 0.001f);
        SRu[e] = f_array((size_t)(I * H / G), 0.001f);
        Sdh[e] = f_array((size_t)(H * I / G), 0.01f);
    }
    uint16_t* x = bf16_array((size_t)(T * H), 1.0f);
    uint16_t* out = (uint16_t*)xalloc((size_t)(T * H) * 2);
    float* out_f32 = (float*)xalloc((size_t)(T * H) * 4);
    uint16_t* h = (uint16_t*)xalloc((size_t)(S * I) * 2);
    float* y = (float*)xalloc((size_t)(S * H) * 4);
    check(oracle_moe_ffn_bf16(x, ids, w, (const uint16_t* const*)Wg, (const uint16_t* const*)Wu,
                              (const uint16_t* const*)Wd, T, H, I, E, k, out, out_f32, h, y),
          "moe_ffn_bf16");
    check(oracle_moe_ffn_bf16(x, ids, w, (const uint16_t* const*)Wg, (const uint16_t* const*)Wu,
                              (const uint16_t* const*)Wd, T, H, I, E, k, out, NULL, NULL, NULL),
          "moe_ffn_bf16 (out only)");
    if (quant) {
        check(oracle_moe_ffn_int8(x, ids, w, (const int8_t* const*)Qg, (const float* const*)Sg,
                                  (const int8_t* const*)Qu, (const float* const*)Su,
                                  (const int8_t* const*)Qd, (const float* const*)Sd, G, T, H, I,
                                  E, k, out, out_f32, h, y),
              "moe_ffn_int8");
        check(oracle_moe_ffn_resplit(
                  x, ids, w, (const int8_t* const*)Qg, (const float* const*)Sg,
                  (const int8_t* const*)Rg, (const float* const*)SRg, (const int8_t* const*)Qu,
                  (const float* const*)Su, (const int8_t* const*)Ru, (const float* const*)SRu,
                  (const int8_t* const*)Qd, (const float* const*)Sd, (const int8_t* const*)Qdh,
                  (const float* const*)Sdh, critical, G, T, H, I, E, k, out, out_f32, h, y),
              "moe_ffn_resplit");
    }
    for (int32_t e = 0; e < E; ++e) {
        free(Wg[e]); free(Wu[e]); free(Wd[e]); free(Qg[e]); free(Qu[e]); free(Qd[e]);
        free(Rg[e]); free(Ru[e]); free(Qdh[e]); free(Sg[e]); free(Su[e]); free(Sd[e]);
        free(SRg[e]); free(SRu[e]); free(Sdh[e]);
    }
    free(Wg); free(Wu); free(Wd); free(Qg); free(Qu); free(Qd); free(Rg); free(Ru); free(Qdh);
    free(Sg); free(Su); free(Sd); free(SRg); free(SRu); free(Sdh); free(critical);
    free(x); free(out); free(out_f32); free(h); free(y); free(logits); free(ids); free(w);
    free(counts); free(offsets); free(sorted); free(active);
}

int main(void) {
    /* T, H, I, E, k, with bad ids */
    layer_case(0, 128, 128, 4, 2, 0);     /* empty batch */
    layer_case(5, 128, 256, 1, 1, 0);     /* one expert */
    layer_case(7, 256, 128, 4, 4, 1);     /* top_k = E, bad and duplicate ids */
    layer_case(16, 256, 512, 8, 2, 1);    /* the Tiny shape */
    layer_case(9, 96, 160, 16, 3, 1);     /* not multiples of 128: BF16 only */
    layer_case(3, 128, 384, 32, 8, 0);    /* most experts unused */

    /* grouped sigmoid router: 64 experts in 8 groups, 4 kept, k = 6 */
    {
        const int64_t T = 5;
        const int32_t E = 64, k = 6;
        float* logits = f_array((size_t)(T * E), 3.0f);
        float* bias = f_array((size_t)E, 0.1f);
        int32_t* ids = (int32_t*)xalloc((size_t)(T * k) * 4);
        float* w = (float*)xalloc((size_t)(T * k) * 4);
        check(oracle_route_grouped(logits, bias, T, E, 8, 4, k, 2.5f, ids, w), "route_grouped");
        check(oracle_route_grouped(logits, NULL, T, E, 1, 1, k, 1.0f, ids, w),
              "route_grouped (one group, no bias)");
        free(logits); free(bias); free(ids); free(w);
    }
    /* decode attention: ragged lengths with an empty and a full sequence */
    {
        const int32_t B = 3, h_q = 8, h_kv = 2, d = 64, L = 70;
        uint16_t* q = bf16_array((size_t)B * h_q * d, 1.0f);
        uint16_t* kc = bf16_array((size_t)B * h_kv * L * d, 1.0f);
        uint16_t* vc = bf16_array((size_t)B * h_kv * L * d, 1.0f);
        int32_t* len = (int32_t*)xalloc((size_t)B * 4);
        len[0] = L; len[1] = 0; len[2] = 33;
        uint16_t* out = (uint16_t*)xalloc((size_t)B * h_q * d * 2);
        check(oracle_attn_decode(q, kc, vc, len, B, h_q, h_kv, d, L, 0.125f, out), "attn_decode");
        free(q); free(kc); free(vc); free(len); free(out);
    }
    if (fails) {
        fprintf(stderr, "%d oracle calls failed\n", fails);
        return 1;
    }
    printf("oracle sanitizer driver: all calls ok\n");
    return 0;
}
