// Routed-expert FFN, BF16 weights: gate/up projection with the SiLU*up
// epilogue, down projection, and the weighted combine.
//
// HiNa-MoE §4.1 (FFN equation, Fig. 5): each expert multiplies the small
// matrix of its gathered tokens by W_gate and W_up, applies SiLU to the gate
// branch, multiplies the branches elementwise and multiplies by W_down.
// §4.1 "transform I, not W": the weights are read in their plain row-major
// layout, which is already the MFMA A-operand layout (one row per lane, eight
// consecutive K values per lane); only the gathered tokens are arranged as the
// B operand, straight from their rows by index, and the results are written
// back row-major.  §4.2.1: BF16 operands, FP32 accumulation; the matrix unit
// is used for every token count (a 16-column tile padded with zeros), never a
// vector fallback.  §4.2.2: weights are streamed with non-temporal loads.
//
// Work decomposition: a task is (active expert, block of 16*RB output rows);
// the four waves of a workgroup split K into four contiguous ranges and their
// FP32 partial tiles are summed in a fixed order through LDS.  The grid is
// persistent: workgroups stride over the task list the permute kernel built,
// so no host read-back of routing counts is needed.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

// Gate/up: h[p][row] = bf16( silu(W_gate[e][row] . x_t) * (W_up[e][row] . x_t) )
// for gathered row p (token t = sorted_slot[p] / k) of expert e.
template <int RB, int U>
__global__ __launch_bounds__(kThreads) void gateup_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wg,
    const uint16_t* __restrict__ Wu, const int32_t* __restrict__ meta,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ active,
    const int32_t* __restrict__ sorted_slot, uint16_t* __restrict__ h, int H, int I,
    int top_k) {
    __shared__ f32x4 red[kWaves - 1][2 * RB][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int col = lane & 15;  // A row, B column and D column of this lane
    const int kg = lane >> 4;   // K group of the operands, row quad of D
    const int nblk = I / (16 * RB);
    const int ntask = meta[0] * nblk;
    const int nsteps = H / 32;
    const int s_begin = (wave * nsteps) / kWaves;
    const int s_end = ((wave + 1) * nsteps) / kWaves;

    for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
        const int a = task / nblk;
        const int rb = task - a * nblk;
        const int e = active[a];
        const int beg = offsets[e];
        const int m = offsets[e + 1] - beg;
        const int row0 = rb * 16 * RB;
        const size_t wrow = ((size_t)e * I + row0 + col) * H + kg * 8;
        const uint16_t* wg = Wg + wrow;
        const uint16_t* wu = Wu + wrow;
        for (int c0 = 0; c0 < m; c0 += 16) {
            const bool valid = c0 + col < m;
            // gather: the B column of this lane is the token of gathered row
            // beg + c0 + col; padding columns read a real row and are zeroed
            const int tok = sorted_slot[beg + (valid ? c0 + col : 0)] / top_k;
            const uint16_t* xr = x + (size_t)tok * H + kg * 8;
            f32x4 accg[RB], accu[RB];
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                accg[r] = f32x4{0.f, 0.f, 0.f, 0.f};
                accu[r] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            int s = s_begin;
            for (; s + U <= s_end; s += U) {
                u32x4 bq[U], gq[U][RB], uq[U][RB];
#pragma unroll
                for (int i = 0; i < U; ++i) {
#pragma unroll
                    for (int r = 0; r < RB; ++r) {
                        gq[i][r] = load_stream16(wg + (size_t)r * 16 * H + (s + i) * 32);
                        uq[i][r] = load_stream16(wu + (size_t)r * 16 * H + (s + i) * 32);
                    }
                    const u32x4 xv = load_cached16(xr + (s + i) * 32);
                    bq[i] = valid ? xv : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int i = 0; i < U; ++i) {
#pragma unroll
                    for (int r = 0; r < RB; ++r) {
                        accg[r] = mfma16x16x32(as_bf16x8(gq[i][r]), as_bf16x8(bq[i]), accg[r]);
                        accu[r] = mfma16x16x32(as_bf16x8(uq[i][r]), as_bf16x8(bq[i]), accu[r]);
                    }
                }
            }
            for (; s < s_end; ++s) {
                const u32x4 xv = load_cached16(xr + s * 32);
                const u32x4 bq = valid ? xv : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    const u32x4 gq = load_stream16(wg + (size_t)r * 16 * H + s * 32);
                    const u32x4 uq = load_stream16(wu + (size_t)r * 16 * H + s * 32);
                    accg[r] = mfma16x16x32(as_bf16x8(gq), as_bf16x8(bq), accg[r]);
                    accu[r] = mfma16x16x32(as_bf16x8(uq), as_bf16x8(bq), accu[r]);
                }
            }
            if (wave > 0) {
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    red[wave - 1][2 * r][lane] = accg[r];
                    red[wave - 1][2 * r + 1][lane] = accu[r];
                }
            }
            __syncthreads();
            if (wave == 0 && valid) {
                const size_t p = (size_t)beg + c0 + col;
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    f32x4 g = accg[r], u = accu[r];
#pragma unroll
                    for (int w = 0; w < kWaves - 1; ++w) {
                        g += red[w][2 * r][lane];
                        u += red[w][2 * r + 1][lane];
                    }
                    u32x2 packed;
                    packed.x = (uint32_t)f32_to_bf16_bits(silu(g.x) * u.x) |
                               ((uint32_t)f32_to_bf16_bits(silu(g.y) * u.y) << 16);
                    packed.y = (uint32_t)f32_to_bf16_bits(silu(g.z) * u.z) |
                               ((uint32_t)f32_to_bf16_bits(silu(g.w) * u.w) << 16);
                    *reinterpret_cast<u32x2*>(h + p * I + row0 + r * 16 + kg * 4) = packed;
                }
            }
            __syncthreads();
        }
    }
}

// Down: y[slot][row] = W_down[e][row] . h[p] for gathered row p of expert e,
// slot = sorted_slot[p] (FP32, written once per slot).
template <int RB, int U>
__global__ __launch_bounds__(kThreads) void down_bf16_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ Wd,
    const int32_t* __restrict__ meta, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ active, const int32_t* __restrict__ sorted_slot,
    float* __restrict__ y, int H, int I) {
    __shared__ f32x4 red[kWaves - 1][RB][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int col = lane & 15;
    const int kg = lane >> 4;
    const int nblk = H / (16 * RB);
    const int ntask = meta[0] * nblk;
    const int nsteps = I / 32;
    const int s_begin = (wave * nsteps) / kWaves;
    const int s_end = ((wave + 1) * nsteps) / kWaves;

    for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
        const int a = task / nblk;
        const int rb = task - a * nblk;
        const int e = active[a];
        const int beg = offsets[e];
        const int m = offsets[e + 1] - beg;
        const int row0 = rb * 16 * RB;
        const uint16_t* wd = Wd + ((size_t)e * H + row0 + col) * I + kg * 8;
        for (int c0 = 0; c0 < m; c0 += 16) {
            const bool valid = c0 + col < m;
            const size_t p = (size_t)beg + (valid ? c0 + col : 0);
            const uint16_t* hr = h + p * I + kg * 8;
            f32x4 acc[RB];
#pragma unroll
            for (int r = 0; r < RB; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
            int s = s_begin;
            for (; s + U <= s_end; s += U) {
                u32x4 bq[U], aq[U][RB];
#pragma unroll
                for (int i = 0; i < U; ++i) {
#pragma unroll
                    for (int r = 0; r < RB; ++r)
                        aq[i][r] = load_stream16(wd + (size_t)r * 16 * I + (s + i) * 32);
                    const u32x4 hv = load_cached16(hr + (s + i) * 32);
                    bq[i] = valid ? hv : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int i = 0; i < U; ++i) {
#pragma unroll
                    for (int r = 0; r < RB; ++r)
                        acc[r] = mfma16x16x32(as_bf16x8(aq[i][r]), as_bf16x8(bq[i]), acc[r]);
                }
            }
            for (; s < s_end; ++s) {
                const u32x4 hv = load_cached16(hr + s * 32);
                const u32x4 bq = valid ? hv : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    const u32x4 aq = load_stream16(wd + (size_t)r * 16 * I + s * 32);
                    acc[r] = mfma16x16x32(as_bf16x8(aq), as_bf16x8(bq), acc[r]);
                }
            }
            if (wave > 0) {
#pragma unroll
                for (int r = 0; r < RB; ++r) red[wave - 1][r][lane] = acc[r];
            }
            __syncthreads();
            if (wave == 0 && valid) {
                const int slot = sorted_slot[p];
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    f32x4 v = acc[r];
#pragma unroll
                    for (int w = 0; w < kWaves - 1; ++w) v += red[w][r][lane];
                    *reinterpret_cast<f32x4*>(y + (size_t)slot * H + row0 + r * 16 + kg * 4) = v;
                }
            }
            __syncthreads();
        }
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

constexpr int kRB = 1;        // row blocks of 16 per task
constexpr int kUnroll = 8;    // K steps (of 32) loaded before their MFMAs
constexpr int kBlocksPerCU = 4;

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
    const int64_t resident = (int64_t)num_cu * kBlocksPerCU;
    const int64_t gu_tasks = max_active * (s.I / (16 * kRB));
    const int64_t dn_tasks = max_active * (s.H / (16 * kRB));
    const int gu_grid = (int)(gu_tasks < resident ? gu_tasks : resident);
    const int dn_grid = (int)(dn_tasks < resident ? dn_tasks : resident);
    hipLaunchKernelGGL((gateup_bf16_kernel<kRB, kUnroll>), dim3(gu_grid), dim3(kThreads), 0,
                       stream, x, (const uint16_t*)W.gate, (const uint16_t*)W.up, ws.meta,
                       ws.offsets, ws.active, ws.sorted_slot, ws.h, s.H, s.I, s.k);
    err = hipGetLastError();
    if (err == hipSuccess) err = ev.mark(1, stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((down_bf16_kernel<kRB, kUnroll>), dim3(dn_grid), dim3(kThreads), 0,
                       stream, ws.h, (const uint16_t*)W.down, ws.meta, ws.offsets,
                       ws.active, ws.sorted_slot, ws.y, s.H, s.I);
    err = hipGetLastError();
    if (err == hipSuccess) err = ev.mark(2, stream);
    if (err != hipSuccess) return err;
    err = launch_combine(ws.y, ids, w, out, s, stream);
    if (err == hipSuccess) err = ev.mark(3, stream);
    return err;
}

}  // namespace moe
