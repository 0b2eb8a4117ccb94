// Routed-expert FFN, BF16 weights: gate/up projection with the SiLU*up
// epilogue, down projection, and the weighted combine.
//
// HiNa-MoE §4.1 (FFN equation, Fig. 5): each expert multiplies the small
// matrix of its gathered tokens by W_gate and W_up, applies SiLU to the gate
// branch, multiplies the branches elementwise and multiplies by W_down.
// §4.1 "transform I, not W": the weights are read in their plain row-major
// layout, which is already the MFMA A-operand layout (one row per lane, eight
// consecutive K values per lane); only the small gathered token matrix is
// rearranged, into the B-operand fragment order, and results are written back
// row-major.  §4.2.1: BF16 operands, FP32 accumulation; the matrix unit is
// used for every token count (16-column tiles padded with zeros), never a
// vector fallback.  §4.2.2: weights are streamed once, with no reuse.
//
// One grouped product kernel serves both projections.  Work unit: a row
// block (16 output rows of one active expert, all its tokens).  The four
// waves of a workgroup form R row blocks x S K-parts (R * S = 4; S chosen by
// the host from the problem size so that there are enough waves to keep HBM
// busy).  Workgroups are persistent: each XCD owns a contiguous slice of the
// expert-major row-block list, and each workgroup a balanced contiguous range
// of that slice, walked in rounds of R row blocks of one expert.
//
// B operand (the gathered tokens, i.e. the pages' matrix I): the workgroup
// stages K-slabs of the 16-token tile in LDS, in MFMA fragment order (one
// 1 KB block per 32-wide K step, direct global->LDS loads, double-buffered),
// which all its waves share.  Weights stream through registers in batches of
// U K-steps with the next batch always in flight, also across slab barriers.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kSlabSteps = 16;       // 32-wide K steps per LDS slab buffer (16 KB)
constexpr int kMinWavesPerCU = 8;    // busy waves per CU that keep HBM streaming

// Tuning per projection, measured on MI355X over the Mixtral-8x7B,
// DeepSeek-V3, Qwen3-235B and Mixtral-8x22B expert shapes at 1-16 tokens per
// expert: gate/up streams two matrices per K step and does best with short
// batches and 4 resident workgroups per CU; down with batches of 8 steps and
// 3 workgroups per CU (LDS: 32 KB per workgroup).
template <int NMAT>
struct GemmTuning;
template <>
struct GemmTuning<2> {
    static constexpr int kBlocksPerCU = 4;
    static constexpr int kBatch = 2;
};
template <>
struct GemmTuning<1> {
    static constexpr int kBlocksPerCU = 3;
    static constexpr int kBatch = 8;
};

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Wait until at most N vector-memory loads of this wave are outstanding
// (loads complete in issue order), leaving LDS and export counters alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One grouped expert product: for every active expert e and gathered row p
// of e, out[p][n] = sum_k W[e][n][k] * B[p][k].
struct ExpertGemm {
    const uint16_t* b_src;    // B rows: x (gate/up) or the gathered h rows (down)
    const uint16_t* w0;       // W_gate or W_down, [E][N][K]
    const uint16_t* w1;       // W_up (gate/up only)
    const int32_t* meta;      // [0] = active experts
    const int32_t* offsets;
    const int32_t* active;
    const int32_t* sorted_slot;
    uint16_t* h;              // gate/up output, row p at p * h_pitch
    float* y;                 // down output, slot s at s * N
    int b_pitch;              // elements between B rows
    int N, K;                 // rows per expert matrix, reduction length
    int top_k;                // gate/up: B row of gathered row p is token sorted_slot[p] / top_k
    int h_pitch;
};

// Weight registers of one batch: U K-steps of NMAT matrices.
template <int NMAT, int U>
struct Batch {
    u32x4 w[U][NMAT];
};

template <int NMAT, int U>
__device__ __forceinline__ void load_batch(Batch<NMAT, U>& dst, const uint16_t* const* a, int s) {
#pragma unroll
    for (int i = 0; i < U; ++i)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) dst.w[i][m] = load_weight16<false>(a[m] + (s + i) * 32);
}

// MFMAs of one batch with the B fragments of LDS blocks buf[0..U).  Padding
// columns (beyond the expert's tokens) hold a copy of a real token row: an
// MFMA output column depends only on its own B column, and padding columns
// are never stored, so they need no zeroing.
template <int NMAT, int U>
__device__ __forceinline__ void mma_batch(const Batch<NMAT, U>& src, const u32x4 (*buf)[kWave],
                                          f32x4* acc) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const u32x4 bq = buf[i][lane];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
            acc[m] = mfma16x16x32(as_bf16x8(src.w[i][m]), as_bf16x8(bq), acc[m]);
    }
}

// Single K step (tails shorter than a batch).
template <int NMAT>
__device__ __forceinline__ void mma_step(const uint16_t* const* a, const u32x4* block, int s,
                                         f32x4* acc) {
    const u32x4 bq = block[threadIdx.x & (kWave - 1)];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        const u32x4 aq = load_weight16<false>(a[m] + s * 32);
        acc[m] = mfma16x16x32(as_bf16x8(aq), as_bf16x8(bq), acc[m]);
    }
}

// NMAT = 2: gate/up, epilogue h[p][row] = bf16(silu(g) * u).
// NMAT = 1: down, epilogue y[slot][row] = acc (FP32, slot = sorted_slot[p]).
// S: K-parts per row block; U: K steps per weight batch (divides 16 / S).
template <int NMAT, int S, int U>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(GemmTuning<NMAT>::kBlocksPerCU)))
void expert_gemm_kernel(const ExpertGemm g) {
    constexpr int R = kWaves / S;           // row blocks per round
    constexpr int SP = kSlabSteps / S;      // steps of each K part per slab
    constexpr int NB = SP / U;              // full batches per full slab
    static_assert(SP % U == 0, "batch must divide the slab part");
    // K-slab buffers; after the slab loop the first buffer doubles as the
    // K-part reduction area (3 x NMAT x 1 KB <= 16 KB).
    __shared__ u32x4 xs[2][kSlabSteps][kWave];
    f32x4* red = reinterpret_cast<f32x4*>(&xs[0][0][0]);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int col = lane & 15;  // A row, B column and D column of this lane
    const int kg = lane >> 4;   // K group of the operands, row quad of D
    const int r = wave % R;     // row block of this wave within a round
    const int kp = wave / R;    // K part of this wave
    const int nrb = g.N / 16;
    const int W = g.meta[0] * nrb;
    const int nsteps = g.K / 32;
    const int kps = (nsteps + S - 1) / S;
    const int ks0 = min(nsteps, kp * kps);
    const int ks1 = min(nsteps, ks0 + kps);
    const int nslab = (kps + SP - 1) / SP;

    // this workgroup's row blocks: a balanced share of its XCD's slice
    const int xcd = blockIdx.x % kXcds;
    const int per = gridDim.x / kXcds;
    const int li = blockIdx.x / kXcds;
    const int sb = (int)((long long)xcd * W / kXcds);
    const int n = (int)((long long)(xcd + 1) * W / kXcds) - sb;
    const int rbeg = sb + (int)((long long)li * n / per);
    const int rend = sb + (int)((long long)(li + 1) * n / per);

    for (int r0 = rbeg; r0 < rend;) {
        const int a = r0 / nrb;
        const int r1 = min(min(r0 + R, rend), (a + 1) * nrb);
        const int e = g.active[a];
        const int beg = g.offsets[e];
        const int m = g.offsets[e + 1] - beg;
        const int my = r0 + r;
        const bool has = my < r1;
        const int row0 = (has ? my - a * nrb : 0) * 16;
        const size_t wrow = ((size_t)e * g.N + row0 + col) * g.K + kg * 8;
        const uint16_t* wp[2] = {g.w0 + wrow, NMAT == 2 ? g.w1 + wrow : g.w0 + wrow};
        const int nfull = has ? (ks1 - ks0) / U : 0;   // full batches of this wave
        const int tail_s = ks0 + nfull * U;            // tail steps [tail_s, ks1)
        for (int c0 = 0; c0 < m; c0 += 16) {
            const bool valid = c0 + col < m;
            const int q = beg + (valid ? c0 + col : 0);
            const int brow = NMAT == 2 ? g.sorted_slot[q] / g.top_k : q;
            const uint16_t* bp = g.b_src + (size_t)brow * g.b_pitch + kg * 8;
            f32x4 acc[NMAT];
#pragma unroll
            for (int mm = 0; mm < NMAT; ++mm) acc[mm] = f32x4{0.f, 0.f, 0.f, 0.f};

            // slab j holds, for each K part pp, its steps
            // [start(pp) + j*SP, +SP) at blocks [pp*SP, pp*SP + SP)
            auto stage = [&](int j, int bsel) {
                for (int blk = wave; blk < kSlabSteps; blk += kWaves) {
                    const int pp = blk / SP;
                    const int p0 = min(nsteps, pp * kps);
                    const int p1 = min(nsteps, p0 + kps);
                    const int s = p0 + j * SP + (blk - pp * SP);
                    if (s < p1)
                        __builtin_amdgcn_global_load_lds((const void*)(bp + s * 32),
                                                         (lds_void_ptr)&xs[bsel][blk][0], 16, 0, 0);
                }
            };
            stage(0, 0);
            // weight batches ping-pong between two register sets: batch bi
            // lives in A when bi is even, in B when odd; the next batch is
            // always requested before the current one is multiplied
            Batch<NMAT, U> A, B;
            if (nfull > 0) load_batch<NMAT, U>(A, wp, ks0);
            int bi = 0;
            for (int j = 0; j < nslab; ++j) {
                // this wave's staging loads are done (only the batch
                // prefetched for this slab may still be in flight)
                if (bi < nfull)
                    wait_vmcnt<NMAT * U>();
                else
                    wait_vmcnt<0>();
                __syncthreads();
                if (j + 1 < nslab) stage(j + 1, (j + 1) & 1);
                const int slab_s0 = ks0 + j * SP;
                const u32x4(*buf)[kWave] = &xs[j & 1][kp * SP];
                const int bend = min(nfull, (j + 1) * NB);
                for (; bi < bend; ++bi) {
                    const u32x4(*bb)[kWave] = buf + (ks0 + bi * U - slab_s0);
                    if ((bi & 1) == 0) {
                        if (bi + 1 < nfull) load_batch<NMAT, U>(B, wp, ks0 + (bi + 1) * U);
                        mma_batch<NMAT, U>(A, bb, acc);
                    } else {
                        if (bi + 1 < nfull) load_batch<NMAT, U>(A, wp, ks0 + (bi + 1) * U);
                        mma_batch<NMAT, U>(B, bb, acc);
                    }
                }
                if (has && tail_s < ks1 && tail_s >= slab_s0 && tail_s < slab_s0 + SP)
                    for (int s = tail_s; s < ks1; ++s)
                        mma_step<NMAT>(wp, &buf[s - slab_s0][0], s, acc);
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
            if (kp == 0 && has && valid) {
                const size_t p = (size_t)beg + c0 + col;
                if constexpr (NMAT == 2) {
                    const f32x4 gv = acc[0], uv = acc[1];
                    u32x2 packed;
                    packed.x = (uint32_t)f32_to_bf16_bits(silu(gv.x) * uv.x) |
                               ((uint32_t)f32_to_bf16_bits(silu(gv.y) * uv.y) << 16);
                    packed.y = (uint32_t)f32_to_bf16_bits(silu(gv.z) * uv.z) |
                               ((uint32_t)f32_to_bf16_bits(silu(gv.w) * uv.w) << 16);
                    *reinterpret_cast<u32x2*>(g.h + p * g.h_pitch + row0 + kg * 4) = packed;
                } else {
                    const int slot = g.sorted_slot[p];
                    *reinterpret_cast<f32x4*>(g.y + (size_t)slot * g.N + row0 + kg * 4) = acc[0];
                }
            }
            if constexpr (S > 1) __syncthreads();
        }
        r0 = r1;
    }
}

// Combine: out[t][c] = bf16( sum_{j ascending} w[t][j] * y[t*k + j][c] ),
// skipping slots whose expert id is out of range.  Eight columns per thread;
// the transposed [row x token] tiles of the down kernel are already stored
// token-major in y, so this writes plain row-major rows.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ ids,
                                                      const float* __restrict__ w,
                                                      uint16_t* __restrict__ out, int T,
                                                      int H, int k, int E) {
    const int chunks = H / 8;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= T * chunks) return;
    const int t = idx / chunks;
    const int c = (idx - t * chunks) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
        const int slot = t * k + j;
        const int e = ids[slot];
        if (e < 0 || e >= E) continue;
        const float wj = w[slot];
        const f32x4 a = *reinterpret_cast<const f32x4*>(y + (size_t)slot * H + c);
        const f32x4 b = *reinterpret_cast<const f32x4*>(y + (size_t)slot * H + c + 4);
        acc[0] += wj * a.x; acc[1] += wj * a.y; acc[2] += wj * a.z; acc[3] += wj * a.w;
        acc[4] += wj * b.x; acc[5] += wj * b.y; acc[6] += wj * b.z; acc[7] += wj * b.w;
    }
    u32x4 o;
    o.x = (uint32_t)f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[1]) << 16);
    o.y = (uint32_t)f32_to_bf16_bits(acc[2]) | ((uint32_t)f32_to_bf16_bits(acc[3]) << 16);
    o.z = (uint32_t)f32_to_bf16_bits(acc[4]) | ((uint32_t)f32_to_bf16_bits(acc[5]) << 16);
    o.w = (uint32_t)f32_to_bf16_bits(acc[6]) | ((uint32_t)f32_to_bf16_bits(acc[7]) << 16);
    *reinterpret_cast<u32x4*>(out + (size_t)t * H + c) = o;
}

// Launch shape of one grouped product: the smallest K split that gives
// kMinWavesPerCU waves per CU a row block (counting the most experts the
// routing can make active), and enough workgroups for the row blocks, up to
// the resident limit, as a multiple of the XCD count.
struct GemmShape {
    int split, grid;
};

GemmShape gemm_shape(int64_t max_active, int N, int num_cu, int blocks_per_cu) {
    const int64_t rows = max_active * (N / 16);
    const int64_t resident = (int64_t)num_cu * blocks_per_cu;
    int split = 1;
    while (split < kWaves && rows * split < (int64_t)num_cu * kMinWavesPerCU) split *= 2;
    const int R = kWaves / split;
    int64_t grid = (rows + R - 1) / R;
    if (grid > resident) grid = resident;
    grid = (grid + kXcds - 1) / kXcds * kXcds;
    return {split, (int)grid};
}

// One launch of the grouped product; the batch never exceeds a slab part.
template <int NMAT>
hipError_t launch_gemm(const ExpertGemm& g, int64_t max_active, int num_cu,
                       hipStream_t stream) {
    constexpr int U = GemmTuning<NMAT>::kBatch;
    const GemmShape sh = gemm_shape(max_active, g.N, num_cu, GemmTuning<NMAT>::kBlocksPerCU);
    const dim3 grid(sh.grid), block(kThreads);
    if (sh.split == 1)
        hipLaunchKernelGGL((expert_gemm_kernel<NMAT, 1, U>), grid, block, 0, stream, g);
    else if (sh.split == 2)
        hipLaunchKernelGGL((expert_gemm_kernel<NMAT, 2, (U < 8 ? U : 8)>), grid, block, 0,
                           stream, g);
    else
        hipLaunchKernelGGL((expert_gemm_kernel<NMAT, 4, (U < 4 ? U : 4)>), grid, block, 0,
                           stream, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const float* y, const int32_t* ids, const float* w,
                          uint16_t* out, const FfnShape& s, hipStream_t stream) {
    const int64_t n = (int64_t)s.T * (s.H / 8);
    const int grid = (int)((n + 255) / 256);
    hipLaunchKernelGGL(combine_kernel, dim3(grid), dim3(256), 0, stream, y, ids, w, out,
                       s.T, s.H, s.k, s.E);
    return hipGetLastError();
}

hipError_t launch_ffn_bf16(const uint16_t* x, const int32_t* ids, const float* w,
                           const FfnWeights& W, uint16_t* out, const FfnShape& s,
                           const Workspace& ws, int num_cu, const StageEvents& ev,
                           hipStream_t stream) {
    hipError_t err = launch_permute(ids, s, ws, stream);
    if (err == hipSuccess) err = ev.mark(0, stream);
    if (err != hipSuccess) return err;
    // upper bound of active experts: every slot could name a different one
    const int64_t max_active = s.E < (int64_t)s.T * s.k ? s.E : (int64_t)s.T * s.k;

    ExpertGemm gu{};
    gu.b_src = x;
    gu.w0 = static_cast<const uint16_t*>(W.gate);
    gu.w1 = static_cast<const uint16_t*>(W.up);
    gu.meta = ws.meta;
    gu.offsets = ws.offsets;
    gu.active = ws.active;
    gu.sorted_slot = ws.sorted_slot;
    gu.h = ws.h;
    gu.y = nullptr;
    gu.b_pitch = s.H;
    gu.N = s.I;
    gu.K = s.H;
    gu.top_k = s.k;
    gu.h_pitch = s.I;
    err = launch_gemm<2>(gu, max_active, num_cu, stream);
    if (err == hipSuccess) err = ev.mark(1, stream);
    if (err != hipSuccess) return err;

    ExpertGemm dn = gu;
    dn.b_src = ws.h;
    dn.w0 = static_cast<const uint16_t*>(W.down);
    dn.w1 = nullptr;
    dn.h = nullptr;
    dn.y = ws.y;
    dn.b_pitch = s.I;
    dn.N = s.H;
    dn.K = s.I;
    err = launch_gemm<1>(dn, max_active, num_cu, stream);
    if (err == hipSuccess) err = ev.mark(2, stream);
    if (err != hipSuccess) return err;
    err = launch_combine(ws.y, ids, w, out, s, stream);
    if (err == hipSuccess) err = ev.mark(3, stream);
    return err;
}

}  // namespace moe
