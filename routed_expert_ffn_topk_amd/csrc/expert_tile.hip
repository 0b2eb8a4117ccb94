// Tiled grouped expert product for experts with many routed tokens
// (prefill-sized batches).
//
// HiNa-MoE §5.1: with long prompts the gathered token matrix I of an expert
// grows until the FFN is compute-bound (the prefill FFN rates of Table 5);
// the FFN equation of §4.1 and the BF16 operands with FP32 accumulation of
// §4.2.1 are unchanged.  Weights stay in their row-major layout and only the
// gathered rows are rearranged, as in the small-m product; what changes is
// the reuse: a weight tile now serves up to 256 tokens, so both operands go
// through LDS in tiles and the matrix unit, not HBM, sets the pace.
//
// Work unit: a tile of two 128-row weight blocks (gate/up: W_gate and W_up;
// down: two consecutive blocks of W_down) x 256 gathered rows of one
// expert, split among sixteen waves, each computing 32 rows of each block x
// 64 tokens with MFMA 16x16x32 blocks.  Per pipeline stage (K = 64) every
// operand tile (rows x 64 K, 128 bytes a row) goes to LDS, with the gather of
// the token rows folded into the load addresses: each wave loads its share
// of the next stage into registers while the MFMAs consume the current one,
// and writes it to the other of two LDS buffers after the step's barrier;
// token rows past the expert's last are not loaded, and the multiplies of
// 16-token blocks that lie past it are skipped.  Rows are stored 128
// bytes apart with their eight 16-byte chunks XOR-swizzled by bits 1-2 of
// the row, so that the MFMA fragment reads (eight rows x two K chunks at a
// time) hit distinct LDS banks.
//
// Schedule: the tiles of all experts on the large list, ordered (expert, row
// tile, K part, token tile) with token tiles fastest, are dealt out per XCD
// like the small-m product's rounds (a contiguous slice per XCD, interleaved
// over its workgroups): the token tiles that share a weight tile run at the
// same time on one XCD, so the weight tile comes from HBM once and from L2
// after that; an expert's tokens are split evenly over its token tiles (in
// 16-token blocks), so that those tiles take equally long and stay in step.
// Gate/up has one K part; down has 1, 2 or 4 (more when a batch
// has few long tiles), each writing its own plane of FP32 partial sums of y.
#include <cmath>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kTileN = 128;                       // weight rows per block
constexpr int kMaxLarge = 1024;                   // matches MOE_FFN_MAX_EXPERTS

// An operand tile of one stage holds 128 rows of RW 16-byte words (K = 8 RW
// values per row).  The words of a row are XOR-swizzled by bits of the row
// so that a fragment read (eight consecutive rows x two adjacent words)
// touches distinct LDS banks.
template <int RW>
__device__ __forceinline__ int row_swizzle(int r) {
    if constexpr (RW == 4)
        return (r >> 1) & 2;
    else
        return ((r >> 1) & 3) << 1;
}

// LDS word of row r, logical 16-byte chunk c (K values 8c .. 8c+7 of the
// stage) in an operand tile.
template <int RW>
__device__ __forceinline__ int tile_word(int r, int c) {
    return r * RW + (c ^ row_swizzle<RW>(r));
}

struct TiledGemm {
    const uint16_t* b_src;    // gathered rows: x (gate/up) or h (down)
    const uint16_t* w0;       // W_gate or W_down, [E][N][K] BF16
    const uint16_t* w1;       // W_up (gate/up only)
    const int32_t* meta;      // [2] = experts on the large list
    const int32_t* offsets;
    const int32_t* large;
    const int32_t* sorted_slot;
    uint16_t* h;              // gate/up output, row p at p * N
    float* y;                 // down output, slot s at s * N (+ y_plane per K part)
    size_t y_plane;           // floats between the partial sums of two K parts
    int b_pitch;              // elements between B rows
    int b_rows;               // B rows (x: T; h: T * top_k), for the debug build's checks
    int slots;                // T * top_k: rows of h and y
    int N, K;
    int top_k;
    int k_parts;              // K parts per tile (down; 1 for gate/up)
    int part_stages;          // K stages of a part (the last part may have fewer)
};

// Per product (gate/up, down): weight blocks of 128 rows per tile
// (gate/up: the same rows of W_gate and W_up; down: kBlocks consecutive
// 128-row blocks of W_down, so a tile covers 128 kBlocks output rows), waves
// per workgroup arranged kWaveRows (along the weight rows) x kWaves /
// kWaveRows (along the tokens), gathered rows per tile (128 or 256), K per
// pipeline stage (32 or 64) and resident workgroups per CU (LDS: two
// buffers of (128 kBlocks + kTokens) rows x 2 kK bytes, + 4 KB).  Both
// products use tiles of 256 gathered rows over sixteen waves, 4 x 4 of 32
// rows (of each weight block) x 64 tokens, K = 64 per stage (132 KB of
// LDS), one workgroup per CU; down stacks two blocks of W_down, so that its
// tiles have the two weight blocks of the gate/up tiles.
enum TileProduct : int { kGateUp = 0, kDownProd = 1 };
template <int P>
struct TileTuning {
    static constexpr int kBlocks = 2;
    static constexpr int kWaves = 16;
    static constexpr int kWaveRows = 4;
    static constexpr int kTokens = 256;
    static constexpr int kK = 64;
    static constexpr int kBlocksPerCU = 1;
};

template <int P>
__global__ __launch_bounds__(TileTuning<P>::kWaves * kWave)
__attribute__((amdgpu_waves_per_eu(TileTuning<P>::kBlocksPerCU * TileTuning<P>::kWaves / 4)))
void expert_tile_kernel(const TiledGemm g) {
    using Tu = TileTuning<P>;
    constexpr bool kDown = P != kGateUp;
    constexpr int NMAT = Tu::kBlocks;             // weight blocks per tile
    constexpr int W = Tu::kWaves;
    constexpr int WR = Tu::kWaveRows;
    constexpr int KS = Tu::kK;                    // K per stage
    constexpr int S = 2;                          // LDS stage buffers
    constexpr int kRows = kDown ? kTileN * NMAT : kTileN;   // output rows per tile
    static_assert(kDown || NMAT == 2, "gate/up tiles hold W_gate and W_up");
    constexpr int M = Tu::kTokens;                // gathered rows per tile
    static_assert((W == 4 || W == 8 || W == 16) && W % WR == 0, "waves per workgroup");
    static_assert(KS == 32 || KS == 64, "stage shape");
    static_assert(M == 128 || M == 256, "tokens per tile");
    constexpr int RW = KS / 8;                    // 16-byte words of a row per stage
    constexpr int kOperandWords = 128 * RW;       // one 128-row weight block
    constexpr int RPI = kWave / RW;               // rows per staging load instruction
    // a stage's rows (NMAT weight blocks, then the M token rows) are staged
    // by NCH load instructions of RPI rows each, IL per wave
    constexpr int WCH = 128 / RPI;
    constexpr int NCH = NMAT * WCH + M / RPI;
    static_assert(NCH % W == 0, "whole staging loads per wave");
    constexpr int IL = NCH / W;
    constexpr int RPW = kTileN / WR;              // weight rows per wave
    constexpr int TPW = M / (W / WR);             // tokens per wave
    constexpr int RB = RPW / 16;                  // 16-row blocks per wave
    constexpr int TB = TPW / 16;                  // 16-token blocks per wave
    constexpr int kStageWords = (NMAT * 128 + M) * RW;
    __shared__ u32x4 lds[S * kStageWords];
    __shared__ int pre[kMaxLarge + 1];

    const int n_large = g.meta[2];
    if (n_large <= 0) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int rt_n = (g.N + kRows - 1) / kRows;       // row tiles per expert

    // tiles before large expert a: pre[a] (wave 0, one run of experts per lane)
    if (wave == 0) {
        const int per = (n_large + kWave - 1) / kWave;
        const int a0 = min(n_large, lane * per), a1 = min(n_large, a0 + per);
        int cnt = 0;
        for (int a = a0; a < a1; ++a) {
            const int e = g.large[a];
            cnt += rt_n * g.k_parts * ((g.offsets[e + 1] - g.offsets[e] + M - 1) / M);
        }
        const int inc = wave_prefix_sum_i32(cnt);
        int b = inc - cnt;
        for (int a = a0; a < a1; ++a) {
            pre[a] = b;
            const int e = g.large[a];
            b += rt_n * g.k_parts * ((g.offsets[e + 1] - g.offsets[e] + M - 1) / M);
        }
        if (lane == kWave - 1) pre[n_large] = inc;
    }
    __syncthreads();
    const int Q = pre[n_large];
    const int G = min((int)gridDim.x, (Q + kXcds - 1) / kXcds * kXcds);
    if ((int)blockIdx.x >= G) return;

    const int xcd = blockIdx.x % kXcds;
    const int per = G / kXcds;
    const int li = blockIdx.x / kXcds;
    const int qb = (int)((long long)xcd * Q / kXcds);
    const int qe = (int)((long long)(xcd + 1) * Q / kXcds);
    const int wr = wave % WR;         // this wave's share of the weight rows
    const int wm = wave / WR;         // this wave's share of the token tile
    const int col = lane & 15;        // A row, B column and D column of this lane
    const int kg = lane >> 4;         // K chunk of the operands, row quad of D
    // staging: load instruction i of this wave fills rows RPI (wave + W i) ..
    // +RPI of an operand tile; lane L brings row + L / RW, logical chunk cl
    // (the instruction's first row is a multiple of 8, so the swizzle of the
    // row depends on L alone)
    const int cl = (lane % RW) ^ row_swizzle<RW>(lane / RW);
    // stages; K is a multiple of 32, so with 64 per stage the last one may
    // hold only its first half
    const int nk_all = (g.K + KS - 1) / KS;

    for (int q = qb + li; q < qe; q += per) {
        int lo = 0, hi = n_large - 1;                 // last a with pre[a] <= q
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= q)
                lo = mid;
            else
                hi = mid - 1;
        }
        const int e = g.large[lo];
        const int beg = g.offsets[e];
        const int m = g.offsets[e + 1] - beg;
        const int mt_n = (m + M - 1) / M;
        // tiles of an expert: (row tile, K part, token tile), token tiles
        // fastest
        const int r = q - pre[lo];
        const int rt = r / (g.k_parts * mt_n);
        const int r2 = r - rt * g.k_parts * mt_n;
        const int kp = r2 / mt_n;
        const int row0 = rt * kRows;
        // the expert's 16-token blocks are split evenly over its mt_n token
        // tiles (at most M / 16 each, at least one), so the token tiles of
        // one weight tile do the same work and stay in step on the XCD: the
        // weight tile is read from HBM once and from L2 by the others.  (With
        // M tokens per tile but the last, a short last tile finished early
        // and then read its weight tiles alone.)
        const int nbe = (m + 15) >> 4;
        const int mt = r2 - kp * mt_n;                // token tile
        // (the products in 64 bits: mt * nbe grows as m^2 / 4096 and passes
        // 2^31 once an expert has about three million tokens)
        const int p0 = 16 * (int)(((int64_t)mt * nbe) / mt_n);
        const int pend = min(m, 16 * (int)(((int64_t)(mt + 1) * nbe) / mt_n));   // tokens [p0, pend)
        // the tile's 16-token blocks, TB per wave in wave order: wave wm
        // takes blocks [bs, bs + nbw).  (Dealing them evenly to the waves
        // was 2-7 % slower on tiles of 100-160 tokens: every wave with a
        // block reads the weight fragments of each stage from LDS, and the
        // LDS reads set the pace.)
        const int nblk = (pend - p0 + 15) >> 4;
        const int bs = TB * wm;
        const int nbw = min(TB, max(0, nblk - bs));
        // this part's stages, and the K left from its first (the last stage
        // of the last part may be a half stage)
        const int s0 = kp * g.part_stages;
        const int nk = min(nk_all, s0 + g.part_stages) - s0;
        const int kl = g.K - s0 * KS;

        // per-lane source rows of the staging loads (rows past the matrix or
        // past the expert's tokens repeat a valid row; their results are
        // never stored)
        const uint16_t* src[IL];
#pragma unroll
        for (int i = 0; i < IL; ++i) {
            const int q = wave + W * i;               // this load's RPI rows of the stage
            if (q < NMAT * WCH) {
                const int mm = q / WCH;
                const int rr = RPI * (q - mm * WCH) + lane / RW;
                const int row = kDown ? row0 + kTileN * mm + rr : row0 + rr;
                const size_t wrow = (size_t)e * g.N + min(row, g.N - 1);
                src[i] = (kDown || mm == 0 ? g.w0 : g.w1) + wrow * g.K + s0 * KS + cl * 8;
            } else {
                const int rr = RPI * (q - NMAT * WCH) + lane / RW;
                const int pp = beg + min(p0 + rr, pend - 1);
                // (debug build: the gathered row itself is checked too)
                const bool pin = MOE_IN_BOUNDS(pp >= 0 && pp < g.slots);
                const int b0 = kDown ? pp : (pin ? g.sorted_slot[pp] / g.top_k : 0);
                const int brow = MOE_IN_BOUNDS(b0 >= 0 && b0 < g.b_rows) ? b0 : 0;
                src[i] = g.b_src + (size_t)brow * g.b_pitch + s0 * KS + cl * 8;
            }
        }
        // register staging loads no token row past the expert's last (their
        // MFMA columns are never stored)
        bool live[IL];
#pragma unroll
        for (int i = 0; i < IL; ++i) {
            const int q = wave + W * i;
            live[i] = q < NMAT * WCH || p0 + RPI * (q - NMAT * WCH) + lane / RW < pend;
        }
        u32x4 rg[IL];
        auto load_regs = [&](int s) {
            int k0 = s * KS;
            if (KS > 32 && k0 + 8 * cl >= kl) k0 -= 32;
#pragma unroll
            for (int i = 0; i < IL; ++i)
                rg[i] = live[i] ? load16(src[i] + k0) : u32x4{0u, 0u, 0u, 0u};
        };
        auto store_regs = [&](int s) {
            u32x4* buf = lds + (s % S) * kStageWords;
#pragma unroll
            for (int i = 0; i < IL; ++i) buf[(wave + W * i) * kWave + lane] = rg[i];
        };
        f32x4 acc[NMAT][RB][TB];
#pragma unroll
        for (int mm = 0; mm < NMAT; ++mm)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) acc[mm][rb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

        // each wave loads its share of stage s + 1 into registers while the
        // MFMAs consume stage s, and writes it to the other LDS buffer after
        // the step's barrier
        load_regs(0);
        store_regs(0);
        if (nk > 1) load_regs(1);
        for (int s = 0; s < nk; ++s) {
            // stage s is in LDS and every wave is done with the other
            // buffer; fill it with stage s + 1 and request stage s + 2
            __syncthreads();
            if (s + 1 < nk) {
                store_regs(s + 1);
                if (s + 2 < nk) load_regs(s + 2);
            }
            const u32x4* buf = lds + (s % S) * kStageWords;
            for (int j = 0; j < KS / 32; ++j) {
                if (j > 0 && s * KS + 32 * j >= kl) break;       // half stage
                // a wave with no token block of this tile has nothing to
                // multiply
                if (nbw == 0) break;
                u32x4 af[NMAT][RB];
#pragma unroll
                for (int mm = 0; mm < NMAT; ++mm)
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        af[mm][rb] = buf[mm * kOperandWords +
                                         tile_word<RW>(RPW * wr + 16 * rb + col, 4 * j + kg)];
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    // only the wave's own token blocks (a uniform test: nbw
                    // is fixed per tile and wave)
                    if (tb >= nbw) break;
                    const u32x4 bf = buf[NMAT * kOperandWords +
                                         tile_word<RW>(16 * (bs + tb) + col, 4 * j + kg)];
#pragma unroll
                    for (int mm = 0; mm < NMAT; ++mm)
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb)
                            acc[mm][rb][tb] = mfma16x16x32(as_bf16x8(af[mm][rb]), as_bf16x8(bf),
                                                           acc[mm][rb][tb]);
                }
            }
        }
        // every wave is done with the stage buffers before the next tile's
        // first stages overwrite them
        __syncthreads();

        // epilogue: lane holds rows n .. n+3 of token column p for each block
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int p = p0 + 16 * (bs + tb) + col;
            if (tb >= nbw || p >= pend) continue;
            if (!MOE_IN_BOUNDS(beg + p < g.slots)) continue;
            if constexpr (kDown) {
                const int slot = g.sorted_slot[beg + p];
                if (!MOE_IN_BOUNDS(slot >= 0 && slot < g.slots)) continue;
                float* yrow = g.y + kp * g.y_plane + (size_t)slot * g.N;
#pragma unroll
                for (int mm = 0; mm < NMAT; ++mm)
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        const int n = row0 + kTileN * mm + RPW * wr + 16 * rb + 4 * kg;
                        if (n < g.N) *reinterpret_cast<f32x4*>(yrow + n) = acc[mm][rb][tb];
                    }
            } else {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const int n = row0 + RPW * wr + 16 * rb + 4 * kg;
                    if (n >= g.N) continue;
                    const f32x4 gv = acc[0][rb][tb], uv = acc[1][rb][tb];
                    u32x2 packed;
                    packed.x = (uint32_t)f32_to_bf16_bits(silu(gv.x) * uv.x) |
                               ((uint32_t)f32_to_bf16_bits(silu(gv.y) * uv.y) << 16);
                    packed.y = (uint32_t)f32_to_bf16_bits(silu(gv.z) * uv.z) |
                               ((uint32_t)f32_to_bf16_bits(silu(gv.w) * uv.w) << 16);
                    *reinterpret_cast<u32x2*>(g.h + (size_t)(beg + p) * g.N + n) = packed;
                }
            }
        }
    }
}

template <int P>
hipError_t launch_tile(const TiledGemm& g, int num_cu, hipStream_t stream) {
    int grid = num_cu * TileTuning<P>::kBlocksPerCU;
    grid = (grid + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((expert_tile_kernel<P>), dim3(grid), dim3(TileTuning<P>::kWaves * kWave),
                       0, stream, g);
    return hipGetLastError();
}

// Workgroup slots of a full GPU for the down product, for the choice of its
// K parts (a function of the sizes alone, since the workspace is sized from
// them): 256 CUs at the down configuration's residency.
constexpr int kNominalCUs = 256;
constexpr int kMaxDownParts = 4;
// nominal rates for the choice: the down product's (TFLOP/s) and HBM's for
// the partial sums (TB/s, a write and a read)
constexpr double kNominalTflops = 600.0;
constexpr double kNominalTBs = 5.0;

// K parts of the down product in configuration D (see tiled_down_parts).
template <int D>
int down_parts(int64_t T, int64_t H, int64_t I, int E, int k) {
    using Tu = TileTuning<D>;
    const int64_t slots = T * k;
    const int64_t large = slots / (kTiledMinTokens + 1) < E ? slots / (kTiledMinTokens + 1) : E;
    constexpr int kRows = kTileN * Tu::kBlocks;   // output rows per tile
    const double tiles = (double)((H + kRows - 1) / kRows) *
                         ((double)slots / Tu::kTokens + 0.5 * (double)large);
    const double wg = (double)kNominalCUs * Tu::kBlocksPerCU;
    const double round_us = wg * 2.0 * kRows * Tu::kTokens * (double)I / (kNominalTflops * 1e6);
    const double plane_us = (double)slots * (double)H * 8.0 / (kNominalTBs * 1e6);
    const int64_t nk = (I + Tu::kK - 1) / Tu::kK;
    int best = 1;
    double best_cost = 1e300;
    for (int P = 1; P <= kMaxDownParts && P <= nk; P *= 2) {
        if ((P - 1) * ((nk + P - 1) / P) >= nk) break;    // a part would be empty
        const double cost = std::ceil(tiles * P / wg) / P * round_us + (P - 1) * plane_us;
        if (cost < best_cost * (1.0 - 1e-9)) {
            best = P;
            best_cost = cost;
        }
    }
    return best;
}

}  // namespace

hipError_t launch_tiled_gate_up(const uint16_t* x, const FfnWeights& W, const FfnShape& s,
                                const Workspace& ws, int num_cu, hipStream_t stream) {
    TiledGemm g{};
    g.b_src = x;
    g.w0 = static_cast<const uint16_t*>(W.gate);
    g.w1 = static_cast<const uint16_t*>(W.up);
    g.meta = ws.meta;
    g.offsets = ws.offsets;
    g.large = ws.large;
    g.sorted_slot = ws.sorted_slot;
    g.h = ws.h;
    g.b_pitch = s.H;
    g.b_rows = s.T;
    g.slots = s.T * s.k;
    g.N = s.I;
    g.K = s.H;
    g.top_k = s.k;
    g.k_parts = 1;
    g.part_stages = 1 << 30;
    return launch_tile<kGateUp>(g, num_cu, stream);
}

hipError_t launch_tiled_down(const FfnWeights& W, const FfnShape& s, const Workspace& ws,
                             int num_cu, hipStream_t stream) {
    TiledGemm g{};
    g.b_src = ws.h;
    g.w0 = static_cast<const uint16_t*>(W.down);
    g.meta = ws.meta;
    g.offsets = ws.offsets;
    g.large = ws.large;
    g.sorted_slot = ws.sorted_slot;
    g.y = ws.y;
    g.y_plane = (size_t)s.T * s.k * s.H;
    g.b_pitch = s.I;
    g.b_rows = s.T * s.k;
    g.slots = s.T * s.k;
    g.N = s.H;
    g.K = s.I;
    g.top_k = s.k;
    g.k_parts = tiled_down_parts(s.T, s.H, s.I, s.E, s.k);
    const int nk = (s.I + TileTuning<kDownProd>::kK - 1) / TileTuning<kDownProd>::kK;
    g.part_stages = (nk + g.k_parts - 1) / g.k_parts;
    return launch_tile<kDownProd>(g, num_cu, stream);
}

// The down product's tiles are long (K = I) and few when a batch has few
// experts (Mixtral-8x7B: 32 row tiles x ~36 token tiles at 2048 tokens,
// against 768 resident workgroups): the last round of tiles leaves much of
// the GPU idle.  Splitting K into parts multiplies the tiles; each part
// writes its own FP32 partial sums of y, which the combine adds.  The part
// count is chosen from the expected tile count (token tiles: T k over the
// gathered rows per tile of the down configuration the sizes select, plus
// half a tile of padding per expert with more than 32 tokens): the rounds of
// tiles it needs, in units of one round of full-K tiles at the product's
// nominal rate, plus the time to write and read back each extra plane of
// partial sums at a nominal HBM rate.
MOE_DEVICE_CHECK_READER(expert_tile)

int tiled_down_parts(int64_t T, int64_t H, int64_t I, int E, int k) {
    if (T <= kTiledMinBatch) return 1;
    return down_parts<kDownProd>(T, H, I, E, k);
}

}  // namespace moe
