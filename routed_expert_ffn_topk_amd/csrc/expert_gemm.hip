// Routed-expert FFN kernels: the grouped expert product (gate/up with the
// SiLU*up epilogue, and down) for BF16, INT8, INT4 and residual-split INT4
// weights, and the launch sequence of a forward call (the combine kernel is
// in combine.hip).
//
// HiNa-MoE §4.1 (FFN equation, Fig. 5): each expert multiplies the small
// matrix of its gathered tokens by W_gate and W_up, applies SiLU to the gate
// branch, multiplies the branches elementwise and multiplies by W_down.
// §4.1 "transform I, not W": the weights are read in their plain row-major
// layout, which is already the MFMA A-operand layout (one row per lane,
// consecutive K values per lane); only the small gathered token matrix is
// rearranged, into the B-operand fragment order, and results are written back
// row-major.  §4.2.1: BF16 operands, FP32 accumulation; the matrix unit is
// used for every token count (16-column tiles padded with a real token row),
// never a vector fallback.  §4.2.2: weights are streamed once, with no reuse.
// §8.1 / Fig. 11: symmetric group-wise INT8 weights, dequantised in registers;
// INT4 the same way.  RapidMoE ("Residual-Split Representation"): INT4 W^Q
// plus an INT4 residual W^R for the gate/up of critical experts, chosen per
// expert within one launch.
//
// One kernel skeleton serves both projections and all weight formats.  Work
// unit: a row block (16 output rows of one active expert, all its tokens).
// The four waves of a workgroup form R row blocks x S K-parts (R * S = 4); a
// round is R row blocks of one expert.  S is chosen on the device from the
// actual number of active experts, so that the rounds fill the persistent
// grid evenly.  Each XCD owns a contiguous slice of the expert-major round
// list, and its workgroups take the slice's rounds interleaved.
//
// B operand (the gathered tokens, i.e. the pages' matrix I): the workgroup
// stages K-slabs of the 16-token tile in LDS, which all its waves share,
// double-buffered.  Each token's slab row (512 K values) is one direct
// global->LDS load of contiguous memory, and only the chunk's distinct tokens
// are staged; the MFMA reads its B fragments (token column, 8 K values) from
// the token rows, which are padded so the reads are free of bank conflicts.
// Weights stream through registers in batches with the next batch always in
// flight, also across slab barriers.
#include <type_traits>

#include "common.hpp"
#include "gather_index.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kSlabBlocks = 16;      // 32-wide K steps per LDS slab buffer
constexpr int kBlockU4 = 4;          // 16-byte words per LDS block of one token (32 K values)
constexpr int kTokRowU4 = kSlabBlocks * kBlockU4;   // one token's slab row (1 KB)
// LDS start (16-byte words) of token c's slab row in a slab buffer: rows are
// 1 KB apart plus a skew of two words per token.  The B-fragment read of a
// wave (lane: token column col, K group kg) is served eight columns x two K
// groups at a time on gfx950; with the skew those 16 reads fall in distinct
// banks (measured: no LDS bank conflicts).
__device__ __forceinline__ int tok_base(int c) { return c * (kTokRowU4 + 2); }
constexpr int kSlabU4 = 16 * (kTokRowU4 + 2);     // slab buffer of 16 token rows
// Scale tables in LDS (scaled formats), per row block and K part of a round,
// in one of two layouts; either way the four output rows 4kg .. 4kg + 3 of a
// lane form one aligned f32x4 per unit.
//  * rows: [unit][16 rows].  A 64-lane staging load of 4-byte entries reads
//    4 units of 16 rows (16 cache lines of the row-major [N][K/128] table);
//    the four row quads a wave reads at once lie in 64 contiguous bytes.
//  * quads: [row quad][unit][4 rows].  A staging load reads 16 units of 4
//    rows (4 cache lines); the four row quads lie 16 x (units per group)
//    bytes apart, which shares LDS banks from 16 units up.
// Floats between consecutive units of a row quad:
constexpr int kScaleUnitStrideRows = 16;
constexpr int kScaleUnitStrideQuads = 4;

// One grouped expert product: for every active expert e and gathered row p
// of e, out[p][n] = sum_k W[e][n][k] * B[p][k].
struct ExpertGemm {
    const uint16_t* b_src;    // B rows: x (gate/up) or the gathered h rows (down)
    const void* w0;           // W_gate or W_down, [E][N][K] (BF16 or INT8)
    const void* w1;           // W_up (gate/up only)
    const float* s0;          // INT8/INT4: group scales of w0, [E][K/128][N]
    const float* s1;          // INT8/INT4: group scales of w1
    // second weight set: the quantised residuals W^R of w0/w1 (residual-split
    // gate/up) or the high-precision copy of W_down, with their scales
    const void* hw0;
    const void* hw1;
    const float* hs0;
    const float* hs1;
    const uint8_t* critical;  // [E], mixed-precision launches: nonzero = high precision
    const int32_t* meta;      // [0] = active experts
    const int32_t* offsets;
    const int32_t* active;
    const int32_t* sorted_slot;
    uint16_t* h;              // gate/up output, row p at p * N
    float* y;                 // down output, slot s at s * N
    int b_pitch;              // elements between B rows
    int b_rows;               // B rows (x: T; h: T * top_k), for the debug build's checks
    int slots;                // T * top_k: rows of h and y
    int N, K;                 // rows per expert matrix, reduction length
    int top_k;                // gate/up: B row of gathered row p is token sorted_slot[p] / top_k
    int split;                // K parts per row block (1, 2 or 4); 0 = chosen on the device
    // gate/up launched with the gather index built in its prologue: the
    // slots' expert ids [n_slots] (topk_ids), the expert count, and where
    // workgroup 0 publishes the index; meta/offsets/active/sorted_slot above
    // are then not read
    const int32_t* ids;
    int n_slots;
    int E;
    IndexOut ix_out;
};

// Where a launch reads the gather index: the workspace, or the LDS copy its
// prologue built.
struct IndexView {
    const int32_t* offsets;
    const int32_t* active;
    const int32_t* sorted_slot;
};

// ---------------------------------------------------------------------------
// Weight formats.  A "unit" is the K range one batch entry covers:
//   BF16: one 32-wide K step = one MFMA per matrix, one LDS block;
//   INT8: one 128-wide scale group = four MFMAs per matrix, four LDS blocks.
// ---------------------------------------------------------------------------

// Per-lane weight pointers of one round: this lane's weight row at its K
// group; r: the second set (residuals).  Scales are not read per lane: the
// workgroup stages the scales of groups of slabs in LDS (see gemm_rounds).
struct WeightSrc {
    const void* w[2];
    const void* r[2];
};

struct Bf16Weights {
    static constexpr bool kResidual = false;
    static constexpr bool kScaled = false;
    // weight batches double-buffered as pairs with fixed register roles
    // (measured 3-10 % slower for BF16 than the parity-switched loop)
    static constexpr bool kFixedRolePipeline = false;
    static constexpr int kBlocks = 1;
    static constexpr float kBytesPerWeight = 2.0f;
    static constexpr int kUnitBytes = kWave * 16;       // weight bytes a wave loads per unit
    template <int NMAT, int U>
    struct Batch {
        u32x4 w[U][NMAT];
    };
    // vector-memory load instructions issued by load<NMAT, U>
    template <int NMAT, int U>
    static constexpr int loads() { return U * NMAT; }
    // K offset (elements) of LDS block `sub` of a unit, for K group kg
    __device__ static int block_offset(int sub, int kg) { return sub * 32 + kg * 8; }
    __device__ static const void* row_ptr(const void* base, size_t row, int K, int kg) {
        return static_cast<const uint16_t*>(base) + row * K + kg * 8;
    }
    template <int NMAT, int U>
    __device__ static void load(Batch<NMAT, U>& d, const WeightSrc& src, int u) {
#pragma unroll
        for (int i = 0; i < U; ++i)
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
                d.w[i][m] = load16(static_cast<const uint16_t*>(src.w[m]) + (u + i) * 32);
    }
    // bl: this lane's B fragment of the batch's first LDS block; block b of
    // the batch at bl[b * kBlockU4].  sl: scales in LDS (scaled formats):
    // unit i of scale tensor t at sl[t * TS + SU * i], the lane's four output
    // rows 4kg .. 4kg + 3 as one aligned f32x4
    template <int NMAT, int U, int TS, int SU>
    __device__ static void mma(const Batch<NMAT, U>& d, const u32x4* bl, const float*,
                               f32x4* acc) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const u32x4 bq = bl[i * kBlockU4];
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
                acc[m] = mfma16x16x32(as_bf16x8(d.w[i][m]), as_bf16x8(bq), acc[m]);
        }
    }
};

// INT8 -> BF16 is exact (|q| <= 127 has at most 7 significant bits).
__device__ __forceinline__ bf16x8 i8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    bf16x8 r;
    r[0] = static_cast<__bf16>((float)((int32_t)(lo << 24) >> 24));
    r[1] = static_cast<__bf16>((float)((int32_t)(lo << 16) >> 24));
    r[2] = static_cast<__bf16>((float)((int32_t)(lo << 8) >> 24));
    r[3] = static_cast<__bf16>((float)((int32_t)lo >> 24));
    r[4] = static_cast<__bf16>((float)((int32_t)(hi << 24) >> 24));
    r[5] = static_cast<__bf16>((float)((int32_t)(hi << 16) >> 24));
    r[6] = static_cast<__bf16>((float)((int32_t)(hi << 8) >> 24));
    r[7] = static_cast<__bf16>((float)((int32_t)hi >> 24));
    return r;
}

// INT8 with one FP32 scale per 128 consecutive K of a row.  Each lane loads 16
// consecutive int8 of its row per 64-wide half group: bytes 0-7 feed one MFMA
// and bytes 8-15 the next, so within a group LDS block 2c+h holds, for K group
// kg, the token values at K = 64c + 16kg + 8h .. +8 (the same K the weights
// use).  The group's FP32 partial tile is scaled by the per-row scale of each
// of the lane's four output rows (4kg + j) and added to the accumulator:
//   dot(row, v) = sum_g s[row][g] * (sum_{c in g} v_c * q[row][c]).
// The scales come from the scale table of the slab's group in LDS.
__device__ __forceinline__ f32x4 lds_f32x4(const float* p) {
    return *reinterpret_cast<const f32x4*>(p);
}

struct Int8Weights {
    static constexpr bool kResidual = false;
    static constexpr bool kScaled = true;
    static constexpr bool kFixedRolePipeline = true;
    static constexpr int kBlocks = 4;
    static constexpr float kBytesPerWeight = 1.0f;
    static constexpr int kUnitBytes = kWave * 32;       // weight bytes a wave loads per unit
    template <int NMAT, int U>
    struct Batch {
        u32x4 w[U][NMAT][2];
    };
    // two 16-byte weight loads per unit and matrix
    template <int NMAT, int U>
    static constexpr int loads() { return U * NMAT * 2; }
    __device__ static int block_offset(int sub, int kg) {
        return (sub >> 1) * 64 + kg * 16 + (sub & 1) * 8;
    }
    __device__ static const void* row_ptr(const void* base, size_t row, int K, int kg) {
        return static_cast<const int8_t*>(base) + row * K + kg * 16;
    }
    template <int NMAT, int U>
    __device__ static void load(Batch<NMAT, U>& d, const WeightSrc& src, int u) {
#pragma unroll
        for (int i = 0; i < U; ++i)
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const int8_t* p = static_cast<const int8_t*>(src.w[m]) + (size_t)(u + i) * 128;
                d.w[i][m][0] = load16(p);
                d.w[i][m][1] = load16(p + 64);
            }
    }
    template <int NMAT, int U, int TS, int SU>
    __device__ static void mma(const Batch<NMAT, U>& d, const u32x4* bl, const float* sl,
                               f32x4* acc) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const u32x4 w = d.w[i][m][c];
                    part = mfma16x16x32(i8x8_to_bf16x8(w.x, w.y),
                                        as_bf16x8(bl[(4 * i + 2 * c) * kBlockU4]), part);
                    part = mfma16x16x32(i8x8_to_bf16x8(w.z, w.w),
                                        as_bf16x8(bl[(4 * i + 2 * c + 1) * kBlockU4]), part);
                }
                acc[m] += lds_f32x4(sl + m * TS + SU * i) * part;
            }
        }
    }
};

// INT4 with one FP32 scale per 128 consecutive K of a row, stored two per
// byte as offset-binary nibbles u = q + 8 (K element 2i in the low nibble of
// byte i).  A unit is one group: each lane loads the 16 bytes (32 K values)
// of its row at group offset 32 kg, and word t of them (8 K values) feeds
// MFMA t.  The BF16 with bits 0x4300 | u is exactly 128 + u, so one AND-OR
// turns two nibbles into two BF16 operands: (w & 0x000F000F) | 0x43004300
// holds K elements 0 and 4 of the word, and the shifts by 4, 8, 12 give
// (1, 5), (2, 6), (3, 7).  The matrix unit then forms
//   sum_k (128 + u_k) x_k = sum_k q_k x_k + 136 sum_k x_k,
// and one more MFMA against the constant 136 (shared by the matrices)
// forms the second term, subtracted before the group scale.  The token
// values are read in the matching K order: LDS block t of K group kg holds K
// values 32 kg + 8 t .. +8 of the group, and each B fragment's BF16 halves
// are interleaved (0, 4, 1, 5, 2, 6, 3, 7).  About one VALU operation per
// weight.
struct Int4Weights {
    static constexpr bool kResidual = false;
    static constexpr bool kScaled = true;
    static constexpr bool kFixedRolePipeline = true;
    static constexpr int kBlocks = 4;
    static constexpr float kBytesPerWeight = 0.5f;
    static constexpr int kUnitBytes = kWave * 16;       // weight bytes a wave loads per unit
    template <int NMAT, int U>
    struct Batch {
        u32x4 w[U][NMAT];
    };
    // one 16-byte weight load per unit and matrix
    template <int NMAT, int U>
    static constexpr int loads() { return U * NMAT; }
    __device__ static int block_offset(int sub, int kg) { return kg * 32 + sub * 8; }
    __device__ static const void* row_ptr(const void* base, size_t row, int K, int kg) {
        return static_cast<const uint8_t*>(base) + row * (size_t)(K / 2) + kg * 16;
    }
    template <int NMAT, int U>
    __device__ static void load(Batch<NMAT, U>& d, const WeightSrc& src, int u) {
#pragma unroll
        for (int i = 0; i < U; ++i)
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
                d.w[i][m] = load16(static_cast<const uint8_t*>(src.w[m]) + (size_t)(u + i) * 64);
    }
    __device__ static u32x4 nibbles_to_bf16(uint32_t w) {
        constexpr uint32_t kMask = 0x000F000Fu, kBias = 0x43004300u;
        return u32x4{(w & kMask) | kBias, ((w >> 4) & kMask) | kBias,
                     ((w >> 8) & kMask) | kBias, ((w >> 12) & kMask) | kBias};
    }
    // token values (x0..x7) -> (x0, x4, x1, x5, x2, x6, x3, x7)
    __device__ static u32x4 interleave(u32x4 b) {
        return u32x4{(b.x & 0xffffu) | (b.z << 16), (b.x >> 16) | (b.z & 0xffff0000u),
                     (b.y & 0xffffu) | (b.w << 16), (b.y >> 16) | (b.w & 0xffff0000u)};
    }
    template <int NMAT, int U, int TS, int SU>
    __device__ static void mma(const Batch<NMAT, U>& d, const u32x4* bl, const float* sl,
                               f32x4* acc) {
        const u32x4 k136 = {0x43084308u, 0x43084308u, 0x43084308u, 0x43084308u};  // BF16 136
#pragma unroll
        for (int i = 0; i < U; ++i) {
            u32x4 bx[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) bx[t] = interleave(bl[(4 * i + t) * kBlockU4]);
            f32x4 corr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t) corr = mfma16x16x32(as_bf16x8(k136), as_bf16x8(bx[t]), corr);
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const u32x4 w = d.w[i][m];
                const uint32_t words[4] = {w.x, w.y, w.z, w.w};
                f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    part = mfma16x16x32(as_bf16x8(nibbles_to_bf16(words[t])), as_bf16x8(bx[t]),
                                        part);
                acc[m] += lds_f32x4(sl + m * TS + SU * i) * (part - corr);
            }
        }
    }
};

// Residual-split INT4 (RapidMoE, "Residual-Split Representation" and
// "Expert-Residual Offloading"): the high-precision weight is W^Q + W^R, W^Q
// the INT4 weight and W^R its INT4-quantised residual, both in the INT4
// layout with their own group scales, and by linearity
//   x (W^Q + W^R) = x W^Q + x W^R.
// A unit is one group of both: two 16-byte weight loads and two 4-byte scale
// loads per matrix.  The token fragments and the bias product (136 sum x) are
// shared by the two terms and the two matrices:
//   acc += s_Q (sum (128 + u_Q) x - 136 sum x) + s_R (sum (128 + u_R) x - 136 sum x).
struct Int4ResidualWeights {
    static constexpr bool kResidual = true;
    static constexpr bool kScaled = true;
    static constexpr bool kFixedRolePipeline = true;
    static constexpr int kBlocks = 4;
    static constexpr float kBytesPerWeight = 1.0f;
    static constexpr int kUnitBytes = 2 * kWave * 16;
    template <int NMAT, int U>
    struct Batch {
        u32x4 w[U][NMAT];
        u32x4 r[U][NMAT];
    };
    template <int NMAT, int U>
    static constexpr int loads() { return U * NMAT * 2; }
    __device__ static int block_offset(int sub, int kg) {
        return Int4Weights::block_offset(sub, kg);
    }
    __device__ static const void* row_ptr(const void* base, size_t row, int K, int kg) {
        return Int4Weights::row_ptr(base, row, K, kg);
    }
    template <int NMAT, int U>
    __device__ static void load(Batch<NMAT, U>& d, const WeightSrc& src, int u) {
#pragma unroll
        for (int i = 0; i < U; ++i)
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const size_t wo = (size_t)(u + i) * 64;
                d.w[i][m] = load16(static_cast<const uint8_t*>(src.w[m]) + wo);
                d.r[i][m] = load16(static_cast<const uint8_t*>(src.r[m]) + wo);
            }
    }
    // scale tensors: W^Q's of the NMAT matrices first, then W^R's
    template <int NMAT, int U, int TS, int SU>
    __device__ static void mma(const Batch<NMAT, U>& d, const u32x4* bl, const float* sl,
                               f32x4* acc) {
        const u32x4 k136 = {0x43084308u, 0x43084308u, 0x43084308u, 0x43084308u};  // BF16 136
#pragma unroll
        for (int i = 0; i < U; ++i) {
            u32x4 bx[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) bx[t] = Int4Weights::interleave(bl[(4 * i + t) * kBlockU4]);
            f32x4 corr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t) corr = mfma16x16x32(as_bf16x8(k136), as_bf16x8(bx[t]), corr);
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const u32x4 w = d.w[i][m], r = d.r[i][m];
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
                const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
                f32x4 pq = {0.f, 0.f, 0.f, 0.f}, pr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    pq = mfma16x16x32(as_bf16x8(Int4Weights::nibbles_to_bf16(ww[t])),
                                      as_bf16x8(bx[t]), pq);
                    pr = mfma16x16x32(as_bf16x8(Int4Weights::nibbles_to_bf16(rw[t])),
                                      as_bf16x8(bx[t]), pr);
                }
                acc[m] += lds_f32x4(sl + m * TS + SU * i) * (pq - corr) +
                          lds_f32x4(sl + (NMAT + m) * TS + SU * i) * (pr - corr);
            }
        }
    }
};

// A launch whose experts run in one of two formats, chosen per expert (per
// round) by ExpertGemm::critical: Hi where it is nonzero, Lo elsewhere.  With
// kHiSecond, Hi reads its weights and scales from the second set (a separate
// high-precision copy); otherwise Hi is a format that reads both sets.
template <class Lo, class Hi, bool kHiSecond>
struct MixedWeights {
    using LoFmt = Lo;
    using HiFmt = Hi;
    static constexpr bool kHiReadsSecond = kHiSecond;
    static_assert(Lo::kBlocks == Hi::kBlocks, "one LDS unit layout for both formats");
    static constexpr int kBlocks = Lo::kBlocks;
    static constexpr float kBytesPerWeight = Hi::kBytesPerWeight;
    static constexpr int kUnitBytes = Hi::kUnitBytes;
};

// Scale tensors a round of format F reads (each staged in LDS per group of slabs):
// one per matrix, two per matrix for a residual format, none for BF16.
template <class F, int NMAT>
struct ScaleTensors {
    static constexpr int value = F::kScaled ? NMAT * (F::kResidual ? 2 : 1) : 0;
};
template <class Lo, class Hi, bool b, int NMAT>
struct ScaleTensors<MixedWeights<Lo, Hi, b>, NMAT> {
    static constexpr int lo = ScaleTensors<Lo, NMAT>::value;
    static constexpr int hi = ScaleTensors<Hi, NMAT>::value;
    static constexpr int value = lo > hi ? lo : hi;
};
// Floats of one slab's scale table per tensor at K split S: R row blocks x S
// K parts x (units per part and slab) x 16 rows = 256 / S (for 4-block units).
constexpr int kScaleSlabFloats = 256;

template <class F>
struct IsMixed {
    static constexpr bool value = false;
};
template <class Lo, class Hi, bool b>
struct IsMixed<MixedWeights<Lo, Hi, b>> {
    static constexpr bool value = true;
};
// the format of one round, and whether it reads the second weight set as
// its first
template <class F, bool kSecond>
struct RoundFmt {
    using Fmt = F;
    static constexpr bool kFromSecond = kSecond;
};

// Residual-split gate/up: critical experts W^Q + W^R, the others W^Q.
using ResidualGateUp = MixedWeights<Int4Weights, Int4ResidualWeights, false>;
// Two-copy down: critical experts the INT8 copy, the others the INT4 one.
using DualDown = MixedWeights<Int4Weights, Int8Weights, true>;

// Tuning per weight format and projection, measured on MI355X over the
// Mixtral-8x7B, DeepSeek-V3, Qwen3-235B and Mixtral-8x22B expert shapes at
// 1-16 tokens per expert (INT4 and the residual split: the Mixtral-8x7B
// shape): batch length U (units), resident workgroups per CU, and the
// deepest slab (kMaxDepth: a slab row of a chunk with few tokens covers up
// to this many times 512 K; scaled formats hold that many times the slab's
// scale table in LDS, which the workgroups per CU must fit), and the batch
// of the wide chunks (kWideBatch units, 0 = none: chunks of up to 32 tokens
// use two B tiles per weight batch; BF16 only), and kEarlyBatch: the
// quantised pipeline requests a slab's second batch before the slab's
// barrier (measured: INT8 down 3-4 % faster at 4-16 tokens per expert; INT8
// and INT4 gate/up, INT4 down and the two-copy down not faster or slower).
// The three grouped products: down (one matrix), gate/up (W_gate and W_up
// per K step), and down as two half-height matrices (the two halves of
// W_down's rows share each token fragment).
enum GemmProj : int { kDown = 1, kGateUp = 2, kDownPair = 3 };
template <class Fmt, int PROJ>
struct GemmTuning;
template <>
struct GemmTuning<Bf16Weights, 2> {   // gate/up: two matrices per K step
    static constexpr int kBlocksPerCU = 4;
    static constexpr int kBatch = 2;
    static constexpr int kMaxDepth = 16;
    static constexpr int kWideBatch = 1;
    static constexpr bool kEarlyBatch = false;
    static constexpr bool kScaleQuads = false;
};
template <>
struct GemmTuning<Bf16Weights, 1> {   // down
    static constexpr int kBlocksPerCU = 3;
    static constexpr int kBatch = 8;
    static constexpr int kMaxDepth = 16;
    static constexpr int kWideBatch = 4;
    static constexpr bool kEarlyBatch = false;
    static constexpr bool kScaleQuads = false;
};
template <>
struct GemmTuning<Int8Weights, 2> {   // (3, 1, 4) before the scales were staged per group: 2-3 % slower
    static constexpr int kBlocksPerCU = 2;
    static constexpr int kBatch = 2;
    static constexpr int kMaxDepth = 8;
    static constexpr int kWideBatch = 0;
    static constexpr bool kEarlyBatch = false;
    static constexpr bool kScaleQuads = true;
};
template <>
struct GemmTuning<Int8Weights, 1> {
    static constexpr int kBlocksPerCU = 3;
    static constexpr int kBatch = 2;
    static constexpr int kMaxDepth = 8;
    static constexpr int kWideBatch = 0;
    static constexpr bool kEarlyBatch = true;
    static constexpr bool kScaleQuads = true;
};
template <>
struct GemmTuning<Int4Weights, 2> {
    static constexpr int kBlocksPerCU = 3;
    static constexpr int kBatch = 2;
    static constexpr int kMaxDepth = 4;
    static constexpr int kWideBatch = 0;
    static constexpr bool kEarlyBatch = false;
    static constexpr bool kScaleQuads = true;
};
template <>
struct GemmTuning<ResidualGateUp, 2> {
    static constexpr int kBlocksPerCU = 2;
    static constexpr int kBatch = 2;
    static constexpr int kMaxDepth = 4;
    static constexpr int kWideBatch = 0;
    static constexpr bool kEarlyBatch = false;
    static constexpr bool kScaleQuads = true;
};
template <>
struct GemmTuning<DualDown, 1> {
    static constexpr int kBlocksPerCU = 2;
    static constexpr int kBatch = 2;
    static constexpr int kMaxDepth = 16;
    static constexpr int kWideBatch = 0;
    static constexpr bool kEarlyBatch = false;
    static constexpr bool kScaleQuads = true;
};
template <>
struct GemmTuning<Int4Weights, kDownPair> {
    static constexpr int kBlocksPerCU = 2;
    static constexpr int kBatch = 2;
    static constexpr int kMaxDepth = 8;
    static constexpr int kWideBatch = 0;
    static constexpr bool kEarlyBatch = false;
    static constexpr bool kScaleQuads = false;
};

// kScaleQuads picks the scale table's LDS layout (quads or rows, above):
// quads measured 1-2 % faster for INT8, 5 % for INT4 gate/up and 4-9 % for
// the residual split's gate/up, and 10-15 % slower for INT4 down as a pair.
// S: K-parts per row block; U: units per weight batch (divides the units of
// one K part in a slab).
// A round is R row blocks of one expert (R = 4 / S), processed by the four
// waves together: they share the LDS token slabs, and the S K parts of a row
// block are summed in LDS.  Rounds never straddle two experts.  The rounds of
// all active experts (expert-major) are dealt out per XCD: each XCD owns a
// contiguous slice, and its workgroups take the slice's rounds interleaved
// (an equal number each, +-1).
// PAIR (down, NMAT = 2): the two "matrices" are the two halves of W_down's
// rows (g.N = H / 2 rows each, the second half at g.w1 / g.s1), so that one
// token fragment feeds both, as W_gate and W_up share it in gate/up.
template <class Fmt, int NMAT, int S, int U, int FMAX, int UW, bool PAIR, bool EARLY, bool QUADS>
__device__ __forceinline__ void gemm_rounds(const ExpertGemm& g, const IndexView ix, int n_act,
                                            int grid,
                                            u32x4 (*xs)[kSlabU4], f32x4* sc) {
    constexpr int R = kWaves / S;              // row blocks per round
    constexpr bool kIsGateUp = NMAT == 2 && !PAIR;
    static_assert(!PAIR || NMAT == 2, "a pair is two matrices");
    const int erows = PAIR ? 2 * g.N : g.N;    // weight rows per expert, output row pitch
    constexpr int SP = kSlabBlocks / S;        // LDS blocks of each K part per slab (depth 1)
    constexpr int SPU = SP / Fmt::kBlocks;     // units of each K part per slab (depth 1)
    constexpr int NB = SPU / U;                // full batches per slab (depth 1)
    static_assert(SPU >= 1 && SPU % U == 0, "batch must divide the slab part");
    static_assert(FMAX >= 1 && FMAX <= 16 && (FMAX & (FMAX - 1)) == 0, "slab depth");
    // wide (32-token) chunks: UW units per weight batch, 0 = none
    constexpr bool kWide = UW > 0 && Fmt::kBlocks == 1 && SPU % (2 * (UW > 0 ? UW : 1)) == 0;
    constexpr int LOG_SP = SP == 16 ? 4 : SP == 8 ? 3 : 2;
    static_assert((1 << LOG_SP) == SP, "power-of-two slab parts");
    // scale table of a group of slabs (scaled formats): per tensor,
    // [R][S][units][16 rows] floats in a region of TS floats (the units of
    // one slab at depth FMAX); two buffers (groups alternate), SCB floats apart
    constexpr int NSC = ScaleTensors<Fmt, NMAT>::value;
    constexpr int TS = R * S * SPU * FMAX * 16;
    constexpr int SCB = NSC * TS;
    static_assert(NSC == 0 || TS <= kScaleSlabFloats * FMAX, "scale table fits its buffer");
    // the scale table's layout and its floats between consecutive units
    constexpr int SU = QUADS ? kScaleUnitStrideQuads : kScaleUnitStrideRows;
    // after the slab loop the first slab buffer doubles as the K-part
    // reduction area (3 x NMAT x 1 KB <= 16 KB)
    f32x4* red = reinterpret_cast<f32x4*>(&xs[0][0]);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int col = lane & 15;  // A row, B column and D column of this lane
    const int kg = lane >> 4;   // K group of the operands, row quad of D
    const int r = wave % R;     // row block of this wave within a round
    const int kp = wave / R;    // K part of this wave
    const int nrb = g.N / 16;                 // row blocks per expert
    const int rpe = (nrb + R - 1) / R;         // rounds per expert
    const int Q = n_act * rpe;                 // rounds of the launch
    const int nunits = g.K / (32 * Fmt::kBlocks);
    const int kpu = (nunits + S - 1) / S;      // units per K part
    const int u0 = min(nunits, kp * kpu);
    const int u1 = min(nunits, u0 + kpu);

    // this workgroup's rounds: every per-th round of its XCD's slice, from
    // its index li in the XCD.  The XCD's workgroups work on neighbouring
    // rounds at any moment, and each takes a mix of the experts of the slice
    // (rounds of experts with more tokens cost more); measured 1-8 % faster
    // than giving each workgroup a contiguous range.
    const int xcd = blockIdx.x % kXcds;
    const int per = grid / kXcds;
    const int li = blockIdx.x / kXcds;
    const int qb = (int)((long long)xcd * Q / kXcds);
    const int qe = (int)((long long)(xcd + 1) * Q / kXcds);

    for (int q = qb + li; q < qe; q += per) {
        const int a = q / rpe;                   // active expert of the round
        const int rb0 = (q - a * rpe) * R;       // its first row block
        const int e = ix.active[a];
        const int beg = ix.offsets[e];
        const int m = ix.offsets[e + 1] - beg;
        const int my = rb0 + r;
        const bool has = my < nrb;
        const int row0 = (has ? my : 0) * 16;
        // this lane's weight row (debug build: row 0 if the expert or row is
        // out of range)
        const size_t arow = MOE_IN_BOUNDS(e >= 0 && e < g.E && row0 + col < erows)
                                ? (size_t)e * erows + row0 + col
                                : 0;
        const int nfull = has ? (u1 - u0) / U : 0;   // full batches of this wave
        const int tail_u = u0 + nfull * U;           // tail units [tail_u, u1)
        // the round in format F (tag: RoundFmt<F, read the second set>)
        auto round = [&](auto tag) {
            using F = typename decltype(tag)::Fmt;
            constexpr bool kSecond = decltype(tag)::kFromSecond;
            constexpr int NSCF = ScaleTensors<F, NMAT>::value;
            const void* w0 = kSecond ? g.hw0 : g.w0;
            const void* w1 = NMAT == 2 ? (kSecond ? g.hw1 : g.w1) : w0;
            WeightSrc src;
            src.w[0] = F::row_ptr(w0, arow, g.K, kg);
            src.w[1] = F::row_ptr(w1, arow, g.K, kg);
            src.r[0] = src.r[1] = nullptr;
            if constexpr (F::kResidual) {
                src.r[0] = F::row_ptr(g.hw0, arow, g.K, kg);
                src.r[1] = F::row_ptr(NMAT == 2 ? g.hw1 : g.hw0, arow, g.K, kg);
            }
            // the expert's row-major scale tables [N][nunits], in the order
            // the format's mma reads them: the matrices' (first or second
            // set), then a residual format's second set
            const float* stab[4] = {nullptr, nullptr, nullptr, nullptr};
            if constexpr (NSCF > 0) {
                const size_t eoff = (size_t)e * erows * nunits;
                const float* p0 = kSecond ? g.hs0 : g.s0;
                const float* p1 = kSecond ? g.hs1 : g.s1;
                stab[0] = p0 + eoff;
                if (NMAT == 2) stab[1] = p1 + eoff;
                if constexpr (F::kResidual) {
                    stab[NMAT] = g.hs0 + eoff;
                    if (NMAT == 2) stab[NMAT + 1] = g.hs1 + eoff;
                }
            }
            // wide chunk: 17-32 tokens, two 16-column B tiles per weight batch
            auto chunk_wide = [&](int c0) __attribute__((always_inline)) {
              if constexpr (kWide && NSCF == 0 && F::kBlocks == 1) {
                constexpr int NC = 2;
                constexpr int UC = UW > 0 ? UW : 1;          // units per weight batch
                static_assert(NC == 1 || (NSCF == 0 && F::kBlocks == 1 && SPU % (2 * UC) == 0),
                              "wide chunks: BF16 weights, half slabs of whole batches");
                const int ntok = min(16 * NC, m - c0);        // distinct tokens of the chunk
                // Slab depth (NC = 1): a slab buffer holds 16 token rows of
                // 512 K; a chunk of ntok <= 16 / 2^d tokens gives each of its
                // rows 2^d times that K (up to FMAX), so a round crosses 2^d
                // times fewer slab barriers.  NC = 2: 32 rows of 256 K.
                const int dl = NC == 2 ? 0
                                       : min(ntok <= 1 ? 4 : ntok <= 2 ? 3 : ntok <= 4 ? 2
                                                                  : ntok <= 8 ? 1 : 0,
                                             FMAX == 16 ? 4 : FMAX == 8 ? 3 : FMAX == 4 ? 2
                                                                : FMAX == 2 ? 1 : 0);
                const int dep = 1 << dl;
                constexpr int SPUC = NC == 1 ? SPU : SPU / 2;    // units per part and slab (depth 1)
                constexpr int SPC = NC == 1 ? SP : SP / 2;       // blocks per part and slab (depth 1)
                constexpr int LOG_SPC = NC == 1 ? LOG_SP : LOG_SP - 1;
                const int spu = SPUC << dl;              // units of each K part per slab
                const int nb = (SPUC / UC) << dl;        // full batches per full slab
                const int tpitch = (kTokRowU4 / NC) * dep + 2;   // LDS words between token rows
                const int nslab = (kpu + spu - 1) / spu;
                const int nfull = has ? (u1 - u0) / UC : 0;   // full batches of this wave
                const int tail_u = u0 + nfull * UC;           // tail units [tail_u, u1)
                // padding columns (beyond the expert's tokens) read token 0's row:
                // an MFMA output column depends only on its own B column, and
                // padding columns are never stored
                bool valid[NC];
                int bcol[NC];
    #pragma unroll
                for (int hh = 0; hh < NC; ++hh) {
                    valid[hh] = 16 * hh + col < ntok;
                    bcol[hh] = valid[hh] ? 16 * hh + col : 0;
                }
                // the first weight batch needs only the expert and the row:
                // request it before the token rows, whose addresses take two
                // dependent loads (the first slab then waits for everything)
                constexpr int kLoads = F::template loads<NMAT, UC>();
                typename F::template Batch<NMAT, UC> A, B;
                if (nfull > 0) F::template load<NMAT, UC>(A, src, u0);
                // staging loads this wave issues per slab: ii = wave, wave + 4,
                // ...; NC = 1: of the chunk's ntok * dep loads, load ii stages
                // 512 K of token ii >> dl, the (ii & (dep - 1))-th of the
                // token's slab row; NC = 2: load ii stages token ii's 256 K
                constexpr int NL = 4 * NC;
                // the loads' B rows (below 2^31; each load forms the row's
                // 64-bit element offset, since rows x pitch can exceed 2^32
                // in large batches)
                uint32_t tp[NL];
    #pragma unroll
                for (int i = 0; i < NL; ++i) {
                    const int c = (wave + kWaves * i) >> dl;
                    const int qq = beg + c0 + (c < ntok ? c : 0);
                    const bool qin = MOE_IN_BOUNDS(qq >= 0 && qq < g.slots);
                    const int b0 = kIsGateUp ? (qin ? ix.sorted_slot[qq] / g.top_k : 0) : qq;
                    const int brow = MOE_IN_BOUNDS(b0 >= 0 && b0 < g.b_rows) ? b0 : 0;
                    tp[i] = (uint32_t)brow;
                }
                f32x4 acc[NC][NMAT];
    #pragma unroll
                for (int hh = 0; hh < NC; ++hh)
    #pragma unroll
                    for (int mm = 0; mm < NMAT; ++mm) acc[hh][mm] = f32x4{0.f, 0.f, 0.f, 0.f};

                // Slab j holds, for each K part pp, its units [start(pp) + j*spu,
                // +spu) at blocks [pp*SPC*dep, (pp+1)*SPC*dep) of every token row.
                // One load instruction stages 16 blocks (1 KB; NC = 2: 8 blocks
                // from lanes 0-31) of one token's slab row: lane L fills block
                // 16i + L/4 for K group L%4, so the row is read from global
                // memory in contiguous runs.
                auto stage = [&](int j, int bsel) {
                    const int kgl = lane & 3;
    #pragma unroll
                    for (int i = 0; i < NL; ++i) {
                        const int ii = wave + kWaves * i;
                        const int c = ii >> dl;
                        const int blk = ((ii & (dep - 1)) << 4) + (lane >> 2);
                        const int pp = blk >> (LOG_SPC + dl);
                        const int bb = blk - (pp << (LOG_SPC + dl));
                        const int p0 = min(nunits, pp * kpu);
                        const int p1 = min(nunits, p0 + kpu);
                        const int u = p0 + j * spu + bb / F::kBlocks;
                        const int off =
                            u * 32 * F::kBlocks + F::block_offset(bb % F::kBlocks, kgl);
                        if (c < ntok && u < p1 && (NC == 1 || lane < 32))
                            __builtin_amdgcn_global_load_lds(
                                (const void*)(g.b_src + (size_t)tp[i] * (size_t)g.b_pitch + off),
                                (lds_void_ptr)&xs[bsel][c * tpitch + ((ii & (dep - 1)) << 6)], 16,
                                0, 0);
                    }
                };
                stage(0, 0);
                // weight batches ping-pong between two register sets: batch bi
                // lives in A when bi is even, in B when odd; the next batch is
                // always requested before the current one is multiplied
                int bi = 0;
                for (int j = 0; j < nslab; ++j) {
                    // this wave's staging loads are done (only the batch
                    // prefetched for this slab may still be in flight; at slab
                    // 0, whose staging follows the first batch, everything)
                    if (j == 0)
                        wait_vmcnt<0>();
                    else if (bi < nfull)
                        wait_vmcnt<(kLoads < 63 ? kLoads : 63)>();
                    else
                        wait_vmcnt<0>();
                    __syncthreads();
                    if (j + 1 < nslab) stage(j + 1, (j + 1) & 1);
                    const int slab_u0 = u0 + j * spu;
                    // this lane's B fragments: token row bcol, K group kg, from the
                    // first block of this wave's K part
                    const u32x4* buf[NC];
    #pragma unroll
                    for (int hh = 0; hh < NC; ++hh)
                        buf[hh] = &xs[j & 1][bcol[hh] * tpitch + ((kp * SPC * kBlockU4) << dl) + kg];
                    // unscaled weights: the formats' mma takes no scales
                    const float* sb = nullptr;
                    const int bend = min(nfull, (j + 1) * nb);
                    for (; bi < bend; ++bi) {
                        const int ub = u0 + bi * UC - slab_u0;   // batch's first unit in the slab
                        // the B pointers before the next batch's loads (computing
                        // them after those loads made the compiler keep far more
                        // registers live in the quantised gate/up kernels)
                        const u32x4* bb[NC];
    #pragma unroll
                        for (int hh = 0; hh < NC; ++hh) bb[hh] = buf[hh] + ub * F::kBlocks * kBlockU4;
                        if ((bi & 1) == 0) {
                            if (bi + 1 < nfull)
                                F::template load<NMAT, UC>(B, src, u0 + (bi + 1) * UC);
                            F::template mma<NMAT, UC, TS, SU>(A, bb[0], sb, acc[0]);
                            if constexpr (NC == 2) F::template mma<NMAT, UC, TS, SU>(A, bb[1], sb, acc[1]);
                        } else {
                            if (bi + 1 < nfull)
                                F::template load<NMAT, UC>(A, src, u0 + (bi + 1) * UC);
                            F::template mma<NMAT, UC, TS, SU>(B, bb[0], sb, acc[0]);
                            if constexpr (NC == 2) F::template mma<NMAT, UC, TS, SU>(B, bb[1], sb, acc[1]);
                        }
                    }
                    if (has && tail_u < u1 && tail_u >= slab_u0 && tail_u < slab_u0 + spu)
                        for (int u = tail_u; u < u1; ++u) {
                            typename F::template Batch<NMAT, 1> t;
                            F::template load<NMAT, 1>(t, src, u);
    #pragma unroll
                            for (int hh = 0; hh < NC; ++hh)
                                F::template mma<NMAT, 1, TS, SU>(
                                    t, buf[hh] + (u - slab_u0) * F::kBlocks * kBlockU4, sb,
                                    acc[hh]);
                        }
                }
                __syncthreads();
                if constexpr (S > 1) {
                    if (kp > 0) {
    #pragma unroll
                        for (int hh = 0; hh < NC; ++hh)
    #pragma unroll
                            for (int mm = 0; mm < NMAT; ++mm)
                                red[(((wave - R) * NC + hh) * NMAT + mm) * kWave + lane] =
                                    acc[hh][mm];
                    }
                    __syncthreads();
                    if (kp == 0) {
    #pragma unroll
                        for (int pp = 1; pp < S; ++pp)
    #pragma unroll
                            for (int hh = 0; hh < NC; ++hh)
    #pragma unroll
                                for (int mm = 0; mm < NMAT; ++mm)
                                    acc[hh][mm] +=
                                        red[((((pp - 1) * R + r) * NC + hh) * NMAT + mm) * kWave +
                                            lane];
                    }
                }
    #pragma unroll
                for (int hh = 0; hh < NC; ++hh) {
                    const size_t p = (size_t)beg + c0 + 16 * hh + col;
                    if (kp == 0 && has && valid[hh] && MOE_IN_BOUNDS(p < (size_t)g.slots)) {
                        if constexpr (kIsGateUp) {
                            const f32x4 gv = acc[hh][0], uv = acc[hh][1];
                            u32x2 packed;
                            packed.x = (uint32_t)f32_to_bf16_bits(silu(gv.x) * uv.x) |
                                       ((uint32_t)f32_to_bf16_bits(silu(gv.y) * uv.y) << 16);
                            packed.y = (uint32_t)f32_to_bf16_bits(silu(gv.z) * uv.z) |
                                       ((uint32_t)f32_to_bf16_bits(silu(gv.w) * uv.w) << 16);
                            *reinterpret_cast<u32x2*>(g.h + p * g.N + row0 + kg * 4) = packed;
                        } else {
                            const int slot = ix.sorted_slot[p];
                            if (MOE_IN_BOUNDS(slot >= 0 && slot < g.slots))
    #pragma unroll
                            for (int mm = 0; mm < NMAT; ++mm)
                                *reinterpret_cast<f32x4*>(g.y + (size_t)slot * erows + mm * g.N +
                                                          row0 + kg * 4) = acc[hh][mm];
                        }
                    }
                }
                if constexpr (S > 1) __syncthreads();
              }
            };
            // an expert with 17-32 tokens: one wide chunk (BF16 weights at
            // splits whose slab parts hold whole wide batches); otherwise
            // chunks of 16
            bool wide_done = false;
            if constexpr (kWide && NSCF == 0 && F::kBlocks == 1) {
                if (m > 16 && m <= 32) {
                    chunk_wide(0);
                    wide_done = true;
                }
            }
            for (int c0 = 0; c0 < m && !wide_done;) {
                const int ntok = min(16, m - c0);        // distinct tokens of the chunk
                // Slab depth: a slab buffer holds 16 token rows of 512 K; a
                // chunk of ntok <= 16 / 2^d tokens gives each of its rows
                // 2^d times that K (up to FMAX), so a round crosses 2^d times
                // fewer slab barriers.
                const int dl = min(ntok <= 1 ? 4 : ntok <= 2 ? 3 : ntok <= 4 ? 2 : ntok <= 8 ? 1 : 0,
                                   FMAX == 16 ? 4 : FMAX == 8 ? 3 : FMAX == 4 ? 2 : FMAX == 2 ? 1 : 0);
                const int dep = 1 << dl;
                const int spu = SPU << dl;               // units of each K part per slab
                const int nb = NB << dl;                 // full batches per full slab
                // Scaled formats stage the scales of P slabs at a time into
                // the table sized for the deepest slab: a row's scales for
                // those slabs are contiguous, so each of its scale lines is
                // fetched once or twice per round instead of by every slab
                // (a round's slabs are microseconds apart and L2 drops the
                // line in between: +18 % reads for INT8 gate/up at 16 tokens
                // per expert, +23 % INT4).  P = FMAX / 2^d, but at most two
                // for INT4 down as a pair (its two matrices' tables make a
                // full group a burst of up to 16 loads per wave, measured 6 %
                // slower at 8 tokens per expert).
                constexpr int kLogF = FMAX == 16 ? 4 : FMAX == 8 ? 3 : FMAX == 4 ? 2 : FMAX == 2 ? 1 : 0;
                const int logP = PAIR ? min(1, kLogF - dl) : kLogF - dl;
                const int P = 1 << logP;
                const int GU = P * spu;                  // units of each K part per scale group
                const int tpitch = kTokRowU4 * dep + 2;  // LDS words between token rows
                const int nslab = (kpu + spu - 1) / spu;
                // padding columns (beyond the expert's tokens) read token 0's row:
                // an MFMA output column depends only on its own B column, and
                // padding columns are never stored
                const bool valid = col < ntok;
                const int bcol = valid ? col : 0;
                // the first weight batch needs only the expert and the row:
                // request it before the token rows, whose addresses take two
                // dependent loads (the first slab then waits for everything)
                constexpr int kLoads = F::template loads<NMAT, U>();
                typename F::template Batch<NMAT, U> A, B;
                if (nfull > 0) F::template load<NMAT, U>(A, src, u0);
                // staging loads this wave issues per slab: ii = wave, wave + 4,
                // ... of the chunk's ntok * dep loads; load ii stages 512 K of
                // token ii >> dl, the (ii & (dep - 1))-th of the token's slab row
                const uint16_t* tp[4];
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = (wave + kWaves * i) >> dl;
                    const int qq = beg + c0 + (c < ntok ? c : 0);
                    const bool qin = MOE_IN_BOUNDS(qq >= 0 && qq < g.slots);
                    const int b0 = kIsGateUp ? (qin ? ix.sorted_slot[qq] / g.top_k : 0) : qq;
                    const int brow = MOE_IN_BOUNDS(b0 >= 0 && b0 < g.b_rows) ? b0 : 0;
                    tp[i] = g.b_src + (size_t)brow * g.b_pitch;
                }
                f32x4 acc[NMAT];
    #pragma unroll
                for (int mm = 0; mm < NMAT; ++mm) acc[mm] = f32x4{0.f, 0.f, 0.f, 0.f};

                // Slab j holds, for each K part pp, its units [start(pp) + j*spu,
                // +spu) at blocks [pp*SP*dep, (pp+1)*SP*dep) of every token row.
                // One load instruction stages 16 blocks (1 KB) of one token's
                // slab row: lane L fills block 16i + L/4 for K group L%4, so the
                // row is read from global memory in contiguous runs.
                // Scaled formats also stage the scales of a group of slabs:
                // the scale of row 16*(rb0 + rr) + 4*rq + t, unit start(pp) +
                // G*GU + jj in group G is entry ((rr*S + pp)*GU + jj)*16 +
                // 4*rq + t (rows) or (((rr*S + pp)*4 + rq)*GU + jj)*4 + t
                // (quads) of its tensor's table; one 4-byte direct load per
                // lane fills 64 consecutive entries.
                auto stage = [&](int j, int bsel) {
                    const int kgl = lane & 3;
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int ii = wave + kWaves * i;
                        const int c = ii >> dl;
                        const int blk = ((ii & (dep - 1)) << 4) + (lane >> 2);
                        const int pp = blk >> (LOG_SP + dl);
                        const int bb = blk - (pp << (LOG_SP + dl));
                        const int p0 = min(nunits, pp * kpu);
                        const int p1 = min(nunits, p0 + kpu);
                        const int u = p0 + j * spu + bb / F::kBlocks;
                        const int off =
                            u * 32 * F::kBlocks + F::block_offset(bb % F::kBlocks, kgl);
                        if (c < ntok && u < p1)
                            __builtin_amdgcn_global_load_lds(
                                (const void*)(tp[i] + off),
                                (lds_void_ptr)&xs[bsel][c * tpitch + ((ii & (dep - 1)) << 6)], 16,
                                0, 0);
                    }
                    if constexpr (NSCF > 0) {
                        // scale group G (slabs [G*P, (G+1)*P)) goes with the
                        // staging of slab (G-1)*P + 1 (group 0 with slab 0)
                        // into scale buffer G & 1, which group G - 1 is then
                        // done with.  Load k (64 entries of every tensor's
                        // table) by wave k % 4: one offset per lane serves all
                        // tensors (they share the [N][nunits] shape).
                        if (j == 0 || ((j - 1) & (P - 1)) == 0) {
                            const int G = j == 0 ? 0 : ((j - 1) >> logP) + 1;
                            const int nld = (R * S * 16 * GU) / kWave;
                            float* sbuf = reinterpret_cast<float*>(sc) + (G & 1) * SCB;
                            for (int k = wave; k < nld; k += kWaves) {
                                const int f = k * kWave + lane;
                                const int qf = QUADS ? f >> 2 : f >> 4;
                                const int jj = qf % GU;
                                const int rp = QUADS ? (qf / GU) >> 2 : qf / GU;
                                const int row = QUADS ? 4 * ((qf / GU) & 3) + (f & 3) : f & 15;
                                const int spp = rp % S;
                                const int rb = rb0 + rp / S;
                                const int q0 = min(nunits, spp * kpu);
                                const int q1 = min(nunits, q0 + kpu);
                                const int su = q0 + G * GU + jj;
                                const size_t soff = (size_t)(rb * 16 + row) * nunits + su;
                                if (rb < nrb && su < q1) {
    #pragma unroll
                                    for (int t = 0; t < NSCF; ++t)
                                        __builtin_amdgcn_global_load_lds(
                                            (const void*)(stab[t] + soff),
                                            (lds_void_ptr)(sbuf + t * TS + k * kWave), 4, 0, 0);
                                }
                            }
                        }
                    }
                };
                stage(0, 0);
                // weight batches ping-pong between two register sets: batch bi
                // lives in A when bi is even, in B when odd; the next batch is
                // always requested before the current one is multiplied
                int bi = 0;
                for (int j = 0; j < nslab; ++j) {
                    const int bend = min(nfull, (j + 1) * nb);
                    if constexpr (F::kFixedRolePipeline && EARLY) {
                        // The slab's first batch requests the one after it
                        // here, before the barrier: the register set it fills
                        // was multiplied by the previous slab's last batch, so
                        // two batches are in flight while the waves meet at
                        // the barrier instead of one (a quantised slab holds
                        // only a few batches per wave).  Then this wave's
                        // staging loads of slab j are done once no more than
                        // the loads issued after them are outstanding: the
                        // previous slab's batch requests (nb - 1 of them, the
                        // last one this slab's first batch) and the request
                        // here.  At slab 0 the staging follows the first batch
                        // and precedes the request.
                        if (bi < bend) {
                            const int un = u0 + min(bi + 1, nfull - 1) * U;
                            if (bi & 1)
                                F::template load<NMAT, U>(A, src, un);
                            else
                                F::template load<NMAT, U>(B, src, un);
                            if (j == 0 || nb < 2)
                                wait_vmcnt<(kLoads < 63 ? kLoads : 63)>();
                            else
                                wait_vmcnt<(2 * kLoads < 63 ? 2 * kLoads : 63)>();
                        } else {
                            wait_vmcnt<0>();
                        }
                    } else {
                        // this wave's staging loads are done (only the batch
                        // prefetched for this slab may still be in flight; at
                        // slab 0, whose staging follows the first batch,
                        // everything)
                        if (j == 0)
                            wait_vmcnt<0>();
                        else if (bi < nfull)
                            wait_vmcnt<(kLoads < 63 ? kLoads : 63)>();
                        else
                            wait_vmcnt<0>();
                    }
                    __syncthreads();
                    if (j + 1 < nslab) stage(j + 1, (j + 1) & 1);
                    const int slab_u0 = u0 + j * spu;
                    // this lane's B fragments: token row bcol, K group kg, from the
                    // first block of this wave's K part
                    const u32x4* buf =
                        &xs[j & 1][bcol * tpitch + ((kp * SP * kBlockU4) << dl) + kg];
                    // this lane's scales: row block r, K part kp, unit 0 of the
                    // slab (slab j & (P - 1) of its group), output rows 4kg .. 4kg + 3
                    const float* sl =
                        reinterpret_cast<const float*>(sc) + ((j >> logP) & 1) * SCB +
                        (QUADS ? (((r * S + kp) * 4 + kg) * GU + (j & (P - 1)) * spu) * SU
                               : ((r * S + kp) * GU + (j & (P - 1)) * spu) * SU + 4 * kg);
                    if constexpr (F::kFixedRolePipeline) {
                        // one batch: request the next one into nxt (after the
                        // last batch, the last again: an unconditional request
                        // keeps the number of loads in flight fixed, so the
                        // compiler waits for cur only), then multiply cur.
                        // Pairs of batches with fixed roles keep the two
                        // register sets apart (with the parity test below
                        // inside the loop the compiler copies between them,
                        // and the copy waits for the batch just requested).
                        auto mult = [&](auto& cur, int b) __attribute__((always_inline)) {
                            const int ub = u0 + b * U - slab_u0;   // batch's first unit in the slab
                            F::template mma<NMAT, U, TS, SU>(cur, buf + ub * F::kBlocks * kBlockU4,
                                                         sl + SU * ub, acc);
                        };
                        auto step = [&](auto& cur, auto& nxt, int b) __attribute__((always_inline)) {
                            F::template load<NMAT, U>(nxt, src, u0 + min(b + 1, nfull - 1) * U);
                            mult(cur, b);
                        };
                        // the slab's first batch (its request was issued above)
                        if (EARLY && bi < bend) {
                            if (bi & 1)
                                mult(B, bi);
                            else
                                mult(A, bi);
                            ++bi;
                        }
                        if (bi < bend && (bi & 1)) step(B, A, bi++);
                        for (; bi + 1 < bend; bi += 2) {
                            step(A, B, bi);
                            step(B, A, bi + 1);
                        }
                        if (bi < bend) step(A, B, bi++);
                    } else {
                        for (; bi < bend; ++bi) {
                            const int ub = u0 + bi * U - slab_u0;   // batch's first unit in the slab
                            const u32x4* bb = buf + ub * F::kBlocks * kBlockU4;
                            const float* sb = sl + SU * ub;
                            if ((bi & 1) == 0) {
                                if (bi + 1 < nfull)
                                    F::template load<NMAT, U>(B, src, u0 + (bi + 1) * U);
                                F::template mma<NMAT, U, TS, SU>(A, bb, sb, acc);
                            } else {
                                if (bi + 1 < nfull)
                                    F::template load<NMAT, U>(A, src, u0 + (bi + 1) * U);
                                F::template mma<NMAT, U, TS, SU>(B, bb, sb, acc);
                            }
                        }
                    }
                    if (has && tail_u < u1 && tail_u >= slab_u0 && tail_u < slab_u0 + spu)
                        for (int u = tail_u; u < u1; ++u) {
                            typename F::template Batch<NMAT, 1> t;
                            F::template load<NMAT, 1>(t, src, u);
                            F::template mma<NMAT, 1, TS, SU>(
                                t, buf + (u - slab_u0) * F::kBlocks * kBlockU4,
                                sl + SU * (u - slab_u0), acc);
                        }
                }
                __syncthreads();
                if constexpr (S > 1) {
                    if (kp > 0) {
    #pragma unroll
                        for (int mm = 0; mm < NMAT; ++mm)
                            red[((wave - R) * NMAT + mm) * kWave + lane] = acc[mm];
                    }
                    __syncthreads();
                    if (kp == 0) {
    #pragma unroll
                        for (int pp = 1; pp < S; ++pp)
    #pragma unroll
                            for (int mm = 0; mm < NMAT; ++mm)
                                acc[mm] += red[(((pp - 1) * R + r) * NMAT + mm) * kWave + lane];
                    }
                }
                const size_t p = (size_t)beg + c0 + col;
                if (kp == 0 && has && valid && MOE_IN_BOUNDS(p < (size_t)g.slots)) {
                    if constexpr (kIsGateUp) {
                        const f32x4 gv = acc[0], uv = acc[1];
                        u32x2 packed;
                        packed.x = (uint32_t)f32_to_bf16_bits(silu(gv.x) * uv.x) |
                                   ((uint32_t)f32_to_bf16_bits(silu(gv.y) * uv.y) << 16);
                        packed.y = (uint32_t)f32_to_bf16_bits(silu(gv.z) * uv.z) |
                                   ((uint32_t)f32_to_bf16_bits(silu(gv.w) * uv.w) << 16);
                        *reinterpret_cast<u32x2*>(g.h + p * g.N + row0 + kg * 4) = packed;
                    } else {
                        const int slot = ix.sorted_slot[p];
                        if (MOE_IN_BOUNDS(slot >= 0 && slot < g.slots))
    #pragma unroll
                        for (int mm = 0; mm < NMAT; ++mm)
                            *reinterpret_cast<f32x4*>(g.y + (size_t)slot * erows + mm * g.N +
                                                      row0 + kg * 4) = acc[mm];
                    }
                }
                if constexpr (S > 1) __syncthreads();
                            c0 += 16;
            }
        };
        if constexpr (IsMixed<Fmt>::value) {
            if (g.critical[e])
                round(RoundFmt<typename Fmt::HiFmt, Fmt::kHiReadsSecond>{});
            else
                round(RoundFmt<typename Fmt::LoFmt, false>{});
        } else {
            round(RoundFmt<Fmt, false>{});
        }
    }
}

constexpr int cmin(int a, int b) { return a < b ? a : b; }

// Rounds of a launch with K split S.
__device__ __forceinline__ int rounds_for(int n_act, int nrb, int S) {
    const int R = kWaves / S;
    return n_act * ((nrb + R - 1) / R);
}

// Workgroups that take part in a launch of Q rounds: at most one round more
// than the others each, and no idle workgroups between busy ones (idle ones
// would share CUs unevenly with busy ones).  A multiple of the XCD count.
__device__ __forceinline__ int busy_grid(int Q) {
    const int q8 = (Q + kXcds - 1) / kXcds * kXcds;
    return min((int)gridDim.x, q8);
}

// K parts per row block, from a latency/bandwidth model of one launch.  With
// split S there are Q_S rounds on G_S = min(grid, Q_S) workgroups, so the
// makespan is ceil(Q_S / G_S) rounds.  A round streams 16 rows x NMAT
// matrices x K/S weights per wave, at the lower of the wave's own rate (its
// bytes in flight, two weight batches, over the load latency) and its share
// of an effective HBM rate among the 4 * G_S busy waves; each LDS slab adds a
// fixed cost (barrier, staging wait).  Constants fitted to forced-split
// measurements on MI355X of the current kernels over the Mixtral-8x7B/8x22B,
// DeepSeek-V3 and Qwen3-235B expert shapes (BF16, INT8, INT4, residual
// split) at 2..103 active experts and 1..16 tokens per expert: the choice
// costs 0.11 % on average against the fastest split, at most 1.7 % (the
// earlier constants, 4 us and 1 us, cost 0.31 % and up to 4.2 %).
constexpr float kHbmBytesPerUs = 8.0e6f;   // effective HBM rate shared by busy waves
constexpr float kLoadLatencyUs = 5.0f;     // loaded-memory latency of a batch
constexpr float kSlabUs = 4.0f;            // fixed cost per slab
template <class Fmt, int NMAT, int U>
__device__ __forceinline__ int choose_split(const ExpertGemm& g, int n_act) {
    constexpr int units1 = kSlabBlocks / Fmt::kBlocks;
    if (n_act <= 0) return 1;
    const int nrb = g.N / 16;
    const int nslab = (g.K + 32 * kSlabBlocks - 1) / (32 * kSlabBlocks);
    float best = 0.f;
    int best_s = 1;
    for (int S = 1; S <= kWaves; S *= 2) {
        const int Q = rounds_for(n_act, nrb, S);
        const int G = busy_grid(Q);
        const int rounds = (Q + G - 1) / G;
        const int u = min(U, units1 / S);            // batch length used at this split
        const float inflight = 2.f * u * NMAT * Fmt::kUnitBytes;
        const float wave_bytes = 16.f * NMAT * (float)(g.K / S) * Fmt::kBytesPerWeight;
        const float rate = fminf(inflight / kLoadLatencyUs, kHbmBytesPerUs / (4.f * G));
        const float t = rounds * (wave_bytes / rate + nslab * kSlabUs);
        if (S == 1 || t < best) {
            best = t;
            best_s = S;
        }
    }
    return best_s;
}

// NMAT = 2: gate/up, epilogue h[p][row] = bf16(silu(g) * u).
// NMAT = 1: down, epilogue y[slot][row] = acc (FP32, slot = sorted_slot[p]).
// One kernel holds the three K splits; the split is uniform over the launch
// (read from the device-side active-expert count, or forced by g.split).
// WIDE: the kernel also holds the wide (17-32 token) chunk path; launched
// only when an expert can receive more than 16 slots (the extra path costs
// registers, which the narrow path of small batches would otherwise pay for).
// FUSED (gate/up, decode-sized batches): every workgroup first builds the
// gather index from the routing ids into LDS and reads it from there;
// workgroup 0 also publishes it for the down product.  One launch fewer per
// layer, and the rounds' expert and token lookups become LDS reads.
// PROJ: kDown, kGateUp or kDownPair (down as two half-height matrices).
template <class Fmt, int PROJ, bool WIDE, bool FUSED>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(GemmTuning<Fmt, PROJ>::kBlocksPerCU)))
void expert_gemm_kernel(const ExpertGemm g) {
    constexpr int NMAT = PROJ == kDown ? 1 : 2;
    constexpr bool PAIR = PROJ == kDownPair;
    using Tune = GemmTuning<Fmt, PROJ>;
    constexpr int U = Tune::kBatch;
    constexpr int FMAX = Tune::kMaxDepth;
    constexpr int UW = WIDE ? Tune::kWideBatch : 0;
    constexpr bool EARLY = Tune::kEarlyBatch;
    constexpr bool QUADS = Tune::kScaleQuads;
    constexpr int units1 = kSlabBlocks / Fmt::kBlocks;   // units of a part per slab, S = 1
    // K-slab buffers of the token tile, double-buffered, followed (scaled
    // formats) by the slabs' scale tables.  Both are filled by direct
    // global->LDS loads and live in one LDS array: the compiler then leaves
    // the waits for those loads to the kernel's own (vmcnt wait + barrier per
    // slab), whereas with two arrays it waited for every outstanding load
    // before each LDS read, which serialised the weight prefetch.
    constexpr int kScF4 =
        ScaleTensors<Fmt, NMAT>::value * kScaleSlabFloats * Tune::kMaxDepth / 4 * 2;
    // (FUSED: the LDS copy of the gather index at the end, in the same array)
    static_assert(!FUSED || PROJ == kGateUp, "the index is built by the gate/up product");
    static_assert(kFxScratchInts * 4 <= (int)sizeof(u32x4) * kSlabU4, "index scratch fits a slab");
    constexpr int kIxF4 = FUSED ? kFxInts / 4 : 0;
    __shared__ u32x4 lds[2 * kSlabU4 + kScF4 + kIxF4];
    u32x4 (*xs)[kSlabU4] = reinterpret_cast<u32x4 (*)[kSlabU4]>(lds);
    f32x4* sc = reinterpret_cast<f32x4*>(lds + 2 * kSlabU4);
    int n_act;
    IndexView ix;
    if constexpr (FUSED) {
        // scratch in the first slab buffer, free before the first round
        int* ixl = reinterpret_cast<int*>(lds + 2 * kSlabU4 + kScF4);
        n_act = build_index_lds<kThreads>(g.ids, g.n_slots, g.E, reinterpret_cast<int*>(lds),
                                          ixl, blockIdx.x == 0, g.ix_out);
        ix = IndexView{ixl + kFxOffsets, ixl + kFxActive, ixl + kFxSorted};
    } else {
        n_act = g.meta[0];
        ix = IndexView{g.offsets, g.active, g.sorted_slot};
    }
    const int S = g.split ? g.split : choose_split<Fmt, NMAT, U>(g, n_act);
    const int G = busy_grid(rounds_for(n_act, g.N / 16, S));
    if ((int)blockIdx.x >= G) return;
    if (S == 1)
        gemm_rounds<Fmt, NMAT, 1, cmin(U, units1), FMAX, cmin(UW, units1 / 2), PAIR, EARLY, QUADS>(
            g, ix, n_act, G, xs, sc);
    else if (S == 2)
        gemm_rounds<Fmt, NMAT, 2, cmin(U, units1 / 2), FMAX, cmin(UW, units1 / 4), PAIR, EARLY, QUADS>(
            g, ix, n_act, G, xs, sc);
    else
        gemm_rounds<Fmt, NMAT, 4, cmin(U, units1 / 4), FMAX, cmin(UW, units1 / 8), PAIR, EARLY, QUADS>(
            g, ix, n_act, G, xs, sc);
}

// Grid of one grouped product: persistent, the resident workgroup count,
// capped by the most rounds any K split can have (every row block its own
// round, at the most experts the routing can activate), as a multiple of the
// XCD count.  The K split itself is chosen on the device.
int gemm_grid(int64_t max_active, int N, int num_cu, int blocks_per_cu) {
    const int64_t rounds = max_active * (N / 16);
    int64_t grid = (int64_t)num_cu * blocks_per_cu;
    if (grid > rounds) grid = rounds;
    grid = (grid + kXcds - 1) / kXcds * kXcds;
    return (int)grid;
}

template <class Fmt, int PROJ, bool FUSED>
hipError_t launch_gemm_as(const ExpertGemm& g, int grid, bool wide, hipStream_t stream) {
    if constexpr (GemmTuning<Fmt, PROJ>::kWideBatch > 0) {
        if (wide) {
            hipLaunchKernelGGL((expert_gemm_kernel<Fmt, PROJ, true, FUSED>), dim3(grid),
                               dim3(kThreads), 0, stream, g);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((expert_gemm_kernel<Fmt, PROJ, false, FUSED>), dim3(grid), dim3(kThreads),
                       0, stream, g);
    return hipGetLastError();
}

// wide: some expert may receive more than 16 slots (T * k > 16); g.ids set:
// the gate/up launch that builds the gather index itself
template <class Fmt, int PROJ>
hipError_t launch_gemm(const ExpertGemm& g, int64_t max_active, int num_cu, bool wide,
                       hipStream_t stream) {
    const int grid = gemm_grid(max_active, g.N, num_cu, GemmTuning<Fmt, PROJ>::kBlocksPerCU);
    if constexpr (PROJ == kGateUp) {
        if (g.ids) return launch_gemm_as<Fmt, PROJ, true>(g, grid, wide, stream);
    }
    return launch_gemm_as<Fmt, PROJ, false>(g, grid, wide, stream);
}

// INT4 down runs as two half-height matrices: its units move 1 KB of
// weights per 16 rows, so the token fragment reads and staging are a larger
// share than in the other formats, and a pair shares them (measured: INT4
// down -15 % at one token per expert; INT8, BF16 and the two-copy down were
// not faster as pairs).
template <class Fmt>
struct PairedDown : std::false_type {};
template <>
struct PairedDown<Int4Weights> : std::true_type {};


// Fmt: the gate/up weight format; FmtDown: down's (the same but for the
// residual split, whose down copies are not split).
template <class Fmt, class FmtDown = Fmt>
hipError_t launch_ffn(const uint16_t* x, const Routing& route, const FfnWeights& W,
                      uint16_t* out, const FfnShape& s, const Workspace& ws, int num_cu,
                      const StageEvents& ev, const SplitOverride& split, hipStream_t stream) {
    // experts with many tokens go to the tiled product (BF16 weights, batches
    // large enough that an expert can have more than kTiledMinTokens)
    const bool tiled = Fmt::kBytesPerWeight == 2.0f && s.T > kTiledMinBatch;
    const int m_split = tiled ? kTiledMinTokens : INT_MAX;
    // decode-sized batches from given ids: the gate/up product builds the
    // gather index in its prologue (no separate index launch)
    const int64_t n_slots = (int64_t)s.T * s.k;
    const bool fused = !route.logits && !tiled && n_slots >= 1 && n_slots <= kFusedMaxSlots &&
                       s.E <= kFusedMaxExperts;
    hipError_t err = hipSuccess;
    if (route.logits)
        err = launch_route_permute(route.logits, route.ids, route.w, s, ws, m_split, stream);
    else if (!fused)
        err = launch_permute(route.ids, s, ws, m_split, stream);
    if (err == hipSuccess) err = ev.mark(0, stream);
    if (err != hipSuccess) return err;
    // upper bound of active experts: every slot could name a different one
    const int64_t max_active = s.E < (int64_t)s.T * s.k ? s.E : (int64_t)s.T * s.k;

    ExpertGemm gu{};
    gu.b_src = x;
    gu.w0 = W.gate;
    gu.w1 = W.up;
    gu.s0 = W.s_gate;
    gu.s1 = W.s_up;
    gu.hw0 = W.gate2;
    gu.hw1 = W.up2;
    gu.hs0 = W.s_gate2;
    gu.hs1 = W.s_up2;
    gu.critical = W.critical;
    gu.meta = ws.meta;
    gu.offsets = ws.offsets;
    gu.active = ws.active;
    gu.sorted_slot = ws.sorted_slot;
    gu.h = ws.h;
    gu.y = nullptr;
    gu.b_pitch = s.H;
    gu.b_rows = s.T;
    gu.slots = s.T * s.k;
    gu.N = s.I;
    gu.K = s.H;
    gu.top_k = s.k;
    gu.split = split.gate_up;
    gu.E = s.E;
    if (fused) {
        gu.ids = route.ids;
        gu.n_slots = (int)n_slots;
        gu.ix_out = IndexOut{ws.meta, ws.counts, ws.offsets, ws.active, ws.sorted_slot};
    }
    // an expert can receive more than 16 slots only if the batch has more
    const bool wide = (int64_t)s.T * s.k > 16;
    err = launch_gemm<Fmt, kGateUp>(gu, max_active, num_cu, wide, stream);
    if (err == hipSuccess && tiled) err = launch_tiled_gate_up(x, W, s, ws, num_cu, stream);
    if (err == hipSuccess) err = ev.mark(1, stream);
    if (err != hipSuccess) return err;

    ExpertGemm dn = gu;
    dn.b_src = ws.h;
    dn.w0 = W.down;
    dn.w1 = nullptr;
    dn.s0 = W.s_down;
    dn.s1 = nullptr;
    dn.hw0 = W.down2;
    dn.hw1 = nullptr;
    dn.hs0 = W.s_down2;
    dn.hs1 = nullptr;
    dn.h = nullptr;
    dn.y = ws.y;
    dn.b_pitch = s.I;
    dn.b_rows = s.T * s.k;
    dn.N = s.H;
    dn.K = s.I;
    dn.split = split.down;
    dn.ids = nullptr;
    // formats whose down product runs as two half-height matrices (the
    // halves of W_down's rows, each H / 2 rows, a whole number of 16-row
    // blocks: the quantised entry points take H a multiple of 128)
    if constexpr (PairedDown<FmtDown>::value) {
        static_assert(std::is_same_v<FmtDown, Int4Weights>, "paired down: INT4 rows");
        const size_t rows = (size_t)(s.H / 2);
        dn.N = s.H / 2;
        dn.w1 = static_cast<const uint8_t*>(W.down) + rows * (size_t)s.I / 2;   // two per byte
        dn.s1 = W.s_down + rows * (s.I / 128);
        err = launch_gemm<FmtDown, kDownPair>(dn, max_active, num_cu, wide, stream);
    } else {
        err = launch_gemm<FmtDown, kDown>(dn, max_active, num_cu, wide, stream);
    }
    if (err == hipSuccess && tiled) err = launch_tiled_down(W, s, ws, num_cu, stream);
    if (err == hipSuccess) err = ev.mark(2, stream);
    if (err != hipSuccess) return err;
    err = launch_combine(ws.y, route.ids, route.w, out, s, ws.counts, m_split,
                         tiled ? tiled_down_parts(s.T, s.H, s.I, s.E, s.k) : 1,
                         (size_t)s.T * s.k * s.H, stream);
    if (err == hipSuccess) err = ev.mark(3, stream);
    return err;
}

}  // namespace

hipError_t launch_ffn_bf16(const uint16_t* x, const Routing& route, const FfnWeights& W,
                           uint16_t* out, const FfnShape& s, const Workspace& ws, int num_cu,
                           const StageEvents& ev, const SplitOverride& split,
                           hipStream_t stream) {
    return launch_ffn<Bf16Weights>(x, route, W, out, s, ws, num_cu, ev, split, stream);
}

hipError_t launch_ffn_int4(const uint16_t* x, const Routing& route, const FfnWeights& W,
                           uint16_t* out, const FfnShape& s, const Workspace& ws, int num_cu,
                           const StageEvents& ev, const SplitOverride& split,
                           hipStream_t stream) {
    return launch_ffn<Int4Weights>(x, route, W, out, s, ws, num_cu, ev, split, stream);
}

hipError_t launch_ffn_int8(const uint16_t* x, const Routing& route, const FfnWeights& W,
                           uint16_t* out, const FfnShape& s, const Workspace& ws, int num_cu,
                           const StageEvents& ev, const SplitOverride& split,
                           hipStream_t stream) {
    return launch_ffn<Int8Weights>(x, route, W, out, s, ws, num_cu, ev, split, stream);
}

MOE_DEVICE_CHECK_READER(expert_gemm)

hipError_t launch_ffn_resplit(const uint16_t* x, const Routing& route, const FfnWeights& W,
                           uint16_t* out, const FfnShape& s, const Workspace& ws, int num_cu,
                           const StageEvents& ev, const SplitOverride& split,
                           hipStream_t stream) {
    return launch_ffn<ResidualGateUp, DualDown>(x, route, W, out, s, ws, num_cu, ev, split, stream);
}

}  // namespace moe
