// Routed-expert FFN with INT8 group-quantised weights (HiNa-MoE §8.1,
// Fig. 11: symmetric group-wise INT8 weights, BF16 activations).
//
// Every weight row is int8 q[K] with one FP32 scale per 128 consecutive K.
// In registers each int8 becomes a BF16 (exact: |q| <= 127 needs 7 bits), the
// MFMA accumulates one 128-wide group into an FP32 partial tile, and the tile
// is scaled by the group's per-row scale and added to the running sum:
//   dot(row r, v) = sum_g s[r][g] * (sum_{c in g} v_c * q[r][c]).
// Task decomposition, K split, LDS reduction and the h / y layouts are those
// of the BF16 kernels.
//
// K mapping inside a 64-wide step: lane (col, kg) loads 16 int8 of its row
// at offset 16*kg; the first 8 feed MFMA #0 and the last 8 MFMA #1.  The B
// operand (token row or h row) uses the same mapping, so both sides pair the
// same K index; each 16-byte weight load covers 64 contiguous bytes per row
// across the four K groups.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kGroup = 128;

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

// One wave's share of NMAT [16*RB x K] x [K x 16] products over groups
// [g_begin, g_end).  q[m] points at row (row0 + col) of matrix m, offset
// 16*kg; sc[m] at the scale row of D row (row0 + 4*kg) of matrix m; b at the
// B column's row, offset 16*kg.
template <int NMAT, int RB>
__device__ __forceinline__ void int8_tiles(const int8_t* const* q, const float* const* sc,
                                           const uint16_t* b, bool valid, int K,
                                           int g_begin, int g_end, f32x4 (*acc)[RB]) {
    const int gs = K / kGroup;  // scales per row
    for (int g = g_begin; g < g_end; ++g) {
        const int k0 = g * kGroup;
        // B operand: two 64-wide steps, 16 values each for this lane
        u32x4 bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 v = load_cached16(b + k0 + (i >> 1) * 64 + (i & 1) * 8);
            bv[i] = valid ? v : u32x4{0u, 0u, 0u, 0u};
        }
        u32x4 wq[NMAT][RB][2];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    wq[m][r][i] = load_stream16(q[m] + (size_t)r * 16 * K + k0 + i * 64);
        float s[NMAT][RB][4];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    s[m][r][j] = sc[m][((size_t)r * 16 + j) * gs + g];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const u32x4 w = wq[m][r][i];
                    part = mfma16x16x32(i8x8_to_bf16x8(w.x, w.y), as_bf16x8(bv[2 * i]), part);
                    part = mfma16x16x32(i8x8_to_bf16x8(w.z, w.w), as_bf16x8(bv[2 * i + 1]), part);
                }
                acc[m][r].x += s[m][r][0] * part.x;
                acc[m][r].y += s[m][r][1] * part.y;
                acc[m][r].z += s[m][r][2] * part.z;
                acc[m][r].w += s[m][r][3] * part.w;
            }
        }
    }
}

template <int RB>
__global__ __launch_bounds__(kThreads) void gateup_int8_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ Qg,
    const float* __restrict__ Sg, const int8_t* __restrict__ Qu,
    const float* __restrict__ Su, const int32_t* __restrict__ meta,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ active,
    const int32_t* __restrict__ sorted_slot, uint16_t* __restrict__ h, int H, int I,
    int top_k) {
    __shared__ f32x4 red[kWaves - 1][2][RB][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int col = lane & 15;
    const int kg = lane >> 4;
    const int nblk = I / (16 * RB);
    const int ntask = meta[0] * nblk;
    const int ng = H / kGroup;
    const int g_begin = (wave * ng) / kWaves;
    const int g_end = ((wave + 1) * ng) / kWaves;

    for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
        const int a = task / nblk;
        const int rb = task - a * nblk;
        const int e = active[a];
        const int beg = offsets[e];
        const int m = offsets[e + 1] - beg;
        const int row0 = rb * 16 * RB;
        const int8_t* q[2] = {Qg + ((size_t)e * I + row0 + col) * H + kg * 16,
                              Qu + ((size_t)e * I + row0 + col) * H + kg * 16};
        const float* sc[2] = {Sg + ((size_t)e * I + row0 + 4 * kg) * ng,
                              Su + ((size_t)e * I + row0 + 4 * kg) * ng};
        for (int c0 = 0; c0 < m; c0 += 16) {
            const bool valid = c0 + col < m;
            const int tok = sorted_slot[beg + (valid ? c0 + col : 0)] / top_k;
            const uint16_t* xr = x + (size_t)tok * H + kg * 16;
            f32x4 acc[2][RB];
#pragma unroll
            for (int mm = 0; mm < 2; ++mm)
#pragma unroll
                for (int r = 0; r < RB; ++r) acc[mm][r] = f32x4{0.f, 0.f, 0.f, 0.f};
            int8_tiles<2, RB>(q, sc, xr, valid, H, g_begin, g_end, acc);
            if (wave > 0) {
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    red[wave - 1][0][r][lane] = acc[0][r];
                    red[wave - 1][1][r][lane] = acc[1][r];
                }
            }
            __syncthreads();
            if (wave == 0 && valid) {
                const size_t p = (size_t)beg + c0 + col;
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    f32x4 g = acc[0][r], u = acc[1][r];
#pragma unroll
                    for (int w = 0; w < kWaves - 1; ++w) {
                        g += red[w][0][r][lane];
                        u += red[w][1][r][lane];
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

template <int RB>
__global__ __launch_bounds__(kThreads) void down_int8_kernel(
    const uint16_t* __restrict__ h, const int8_t* __restrict__ Qd,
    const float* __restrict__ Sd, const int32_t* __restrict__ meta,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ active,
    const int32_t* __restrict__ sorted_slot, float* __restrict__ y, int H, int I) {
    __shared__ f32x4 red[kWaves - 1][RB][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int col = lane & 15;
    const int kg = lane >> 4;
    const int nblk = H / (16 * RB);
    const int ntask = meta[0] * nblk;
    const int ng = I / kGroup;
    const int g_begin = (wave * ng) / kWaves;
    const int g_end = ((wave + 1) * ng) / kWaves;

    for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
        const int a = task / nblk;
        const int rb = task - a * nblk;
        const int e = active[a];
        const int beg = offsets[e];
        const int m = offsets[e + 1] - beg;
        const int row0 = rb * 16 * RB;
        const int8_t* q[1] = {Qd + ((size_t)e * H + row0 + col) * I + kg * 16};
        const float* sc[1] = {Sd + ((size_t)e * H + row0 + 4 * kg) * ng};
        for (int c0 = 0; c0 < m; c0 += 16) {
            const bool valid = c0 + col < m;
            const size_t p = (size_t)beg + (valid ? c0 + col : 0);
            const uint16_t* hr = h + p * I + kg * 16;
            f32x4 acc[1][RB];
#pragma unroll
            for (int r = 0; r < RB; ++r) acc[0][r] = f32x4{0.f, 0.f, 0.f, 0.f};
            int8_tiles<1, RB>(q, sc, hr, valid, I, g_begin, g_end, acc);
            if (wave > 0) {
#pragma unroll
                for (int r = 0; r < RB; ++r) red[wave - 1][r][lane] = acc[0][r];
            }
            __syncthreads();
            if (wave == 0 && valid) {
                const int slot = sorted_slot[p];
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    f32x4 v = acc[0][r];
#pragma unroll
                    for (int w = 0; w < kWaves - 1; ++w) v += red[w][r][lane];
                    *reinterpret_cast<f32x4*>(y + (size_t)slot * H + row0 + r * 16 + kg * 4) = v;
                }
            }
            __syncthreads();
        }
    }
}

constexpr int kRB = 1;
constexpr int kBlocksPerCU = 4;

}  // namespace

hipError_t launch_ffn_int8(const uint16_t* x, const int32_t* ids, const float* w,
                           const FfnWeights& W, uint16_t* out, const FfnShape& s,
                           const Workspace& ws, int num_cu, const StageEvents& ev,
                           hipStream_t stream) {
    hipError_t err = launch_permute(ids, s, ws, stream);
    if (err == hipSuccess) err = ev.mark(0, stream);
    if (err != hipSuccess) return err;
    const int64_t max_active = s.E < (int64_t)s.T * s.k ? s.E : (int64_t)s.T * s.k;
    const int64_t resident = (int64_t)num_cu * kBlocksPerCU;
    const int64_t gu_tasks = max_active * (s.I / (16 * kRB));
    const int64_t dn_tasks = max_active * (s.H / (16 * kRB));
    const int gu_grid = (int)(gu_tasks < resident ? gu_tasks : resident);
    const int dn_grid = (int)(dn_tasks < resident ? dn_tasks : resident);
    hipLaunchKernelGGL((gateup_int8_kernel<kRB>), dim3(gu_grid), dim3(kThreads), 0, stream, x,
                       (const int8_t*)W.gate, W.s_gate, (const int8_t*)W.up, W.s_up,
                       ws.meta, ws.offsets, ws.active, ws.sorted_slot, ws.h, s.H, s.I, s.k);
    err = hipGetLastError();
    if (err == hipSuccess) err = ev.mark(1, stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((down_int8_kernel<kRB>), dim3(dn_grid), dim3(kThreads), 0, stream,
                       ws.h, (const int8_t*)W.down, W.s_down, ws.meta, ws.offsets,
                       ws.active, ws.sorted_slot, ws.y, s.H, s.I);
    err = hipGetLastError();
    if (err == hipSuccess) err = ev.mark(2, stream);
    if (err != hipSuccess) return err;
    err = launch_combine(ws.y, ids, w, out, s, stream);
    if (err == hipSuccess) err = ev.mark(3, stream);
    return err;
}

}  // namespace moe
