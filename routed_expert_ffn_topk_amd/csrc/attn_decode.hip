// Decode attention with grouped-query heads as small matrix products.
//
// HiNa-MoE §6.1 (decode attention as small matrix products): under
// grouped-query attention g = h_q / h_kv consecutive query heads read one KV
// head, and a decoding step has one query row per head, so each KV head's
// scores are a g-row matrix times its l_seq x d keys and its output is the
// g-row softmax matrix times its l_seq x d values: products with one small
// operand.  The small operand (the query block) is laid out once for the
// matrix unit and kept resident; the keys are read in their native row-major
// layout, which is already the MFMA A operand (one key row per lane, 8
// consecutive head-dimension values); the value tiles are converted on the
// way (transposed through LDS), so the framework's KV-cache layout stays as
// it is.
//
//   scores  S^T[t][q] = scale * sum_c K[t][c] * Q[q][c]      (MFMA, K rows = A)
//   softmax over t, online: running max m[q], sum l[q]
//   output  O^T[c][q] = sum_t V^T[c][t] * P^T[t][q]          (MFMA, V^T = A)
//
// Layout: q [B][h_q][d], k / v [B][h_kv][max_len][d] (BF16), lens [B];
// query head h reads KV head h / g, g = h_q / h_kv <= 16 (padded to the
// MFMA's 16 columns), d a multiple of 32 up to 256.
//
// Work: one workgroup per (sequence, KV head, split of `chunk` positions),
// the (sequence, head) index fastest;
// its four waves take 32-position tiles in turn and keep their own softmax
// state, merged in LDS at the end into one partial result per split
// (unnormalised output, max, sum).  A second kernel merges the splits of
// each query head (flash-decoding), so that even one sequence spreads over
// the whole GPU.  The path is bound by reading K and V from HBM.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kAttnWaves = 4;
constexpr int kAttnThreads = kAttnWaves * kWave;
constexpr int kTilePos = 32;          // positions per wave tile (the PV MFMA's K)

// Pitch (bytes) of a position row of the wave's V tile in LDS: 16 bytes of
// padding shift the four position groups that one transposed read touches
// onto disjoint banks.
__device__ __forceinline__ constexpr int v_pitch(int d) { return 2 * d + 16; }

template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ lens, int h_q, int h_kv,
    int max_len, int chunk, int n_split, float scale, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
    constexpr int KS = D / 32;        // 32-wide K steps of the score product
    constexpr int DB = D / 16;        // 16-row blocks of the output product
    constexpr int PITCH = v_pitch(D);
    constexpr int kVChunks = kTilePos * D / 8 / kWave;     // 16-byte V loads per lane
    // V tiles of the four waves; reused for the cross-wave merge (needs
    // 4 x 16 x (D + 2) floats)
    constexpr int kLdsBytes = kAttnWaves * kTilePos * PITCH;
    static_assert(kLdsBytes >= kAttnWaves * 16 * (D + 2) * 4, "merge area");
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];

    // (sequence, KV head) fastest: the workgroups of one split index spread
    // over all heads and so over the XCDs, which receive workgroups
    // round-robin (split-fastest order gave the XCDs that hold the late
    // splits of short sequences little work)
    const int j = blockIdx.x % h_kv;          // KV head
    const int b = blockIdx.x / h_kv;          // sequence
    const int split = blockIdx.y;
    const int g = h_q / h_kv;
    const int len = min(max(lens[b], 0), max_len);
    const int t_beg = split * chunk;
    const int t_end = min(len, t_beg + chunk);
    if (t_beg >= t_end) return;               // the merge skips empty splits

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int col = lane & 15;                // query column; A row of a fragment
    const int kg = lane >> 4;                 // K group; output row quad

    const size_t head = ((size_t)b * h_kv + j) * (size_t)max_len * D;
    const uint16_t* kh = k + head;
    const uint16_t* vh = v + head;

    // the query block as the score product's B operand: lane (col, kg) holds
    // Q[col][32 s + 8 kg .. +8]; columns past the group are zero
    u32x4 qf[KS];
    {
        const bool qv = col < g;
        const uint16_t* qp = q + ((size_t)b * h_q + (size_t)j * g + (qv ? col : 0)) * D + 8 * kg;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const u32x4 w = load16(qp + 32 * s);
            qf[s] = qv ? w : u32x4{0u, 0u, 0u, 0u};
        }
    }

    unsigned char* vt = lds + wave * kTilePos * PITCH;   // this wave's V tile
    float m_run = -INFINITY;                  // running max of column col
    float l_part = 0.0f;                      // this lane's share of the sum
    f32x4 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int t0 = t_beg + wave * kTilePos; t0 < t_end; t0 += kAttnWaves * kTilePos) {
        // keys: rows t0 + 16 blk + col (past the end: the last valid row)
        u32x4 kf[2][KS];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int t = min(t0 + 16 * blk + col, t_end - 1);
            const uint16_t* kp = kh + (size_t)t * D + 8 * kg;
#pragma unroll
            for (int s = 0; s < KS; ++s) kf[blk][s] = load16(kp + 32 * s);
        }
        // values: the tile's 32 rows, 16 bytes per load, into LDS
        u32x4 vr[kVChunks];
#pragma unroll
        for (int u = 0; u < kVChunks; ++u) {
            const int c = lane + kWave * u;
            const int row = c / (D / 8), cc = c % (D / 8);
            const int t = min(t0 + row, t_end - 1);
            vr[u] = load16(vh + (size_t)t * D + 8 * cc);
        }
        // scores S^T[16 blk + 4 kg + i][col]
        f32x4 sc[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) a = mfma16x16x32(as_bf16x8(kf[blk][s]), as_bf16x8(qf[s]), a);
            sc[blk] = a;
        }
        float sv[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 16 * blk + 4 * kg + i;
                const float x = t < t_end ? sc[blk][i] * scale : -INFINITY;
                sv[4 * blk + i] = x;
                tmax = fmaxf(tmax, x);
            }
        // column max over the four K groups (lanes col, col + 16, +32, +48)
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
        const float m_new = fmaxf(m_run, tmax);          // finite: t0 < t_end
        const float alpha = expf(m_run - m_new);         // 0 on the first tile
        m_run = m_new;
        float p[8];
        float psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = expf(sv[i] - m_new);                  // 0 past the end
            psum += p[i];
        }
        l_part = l_part * alpha + psum;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        // P^T fragment: lane (col, kg) holds positions 4 kg .. 4 kg + 3 and
        // 16 + 4 kg .. 16 + 4 kg + 3 of column col (the K order both operands
        // of the output product use)
        u32x4 pf;
        pf.x = (uint32_t)f32_to_bf16_bits(p[0]) | ((uint32_t)f32_to_bf16_bits(p[1]) << 16);
        pf.y = (uint32_t)f32_to_bf16_bits(p[2]) | ((uint32_t)f32_to_bf16_bits(p[3]) << 16);
        pf.z = (uint32_t)f32_to_bf16_bits(p[4]) | ((uint32_t)f32_to_bf16_bits(p[5]) << 16);
        pf.w = (uint32_t)f32_to_bf16_bits(p[6]) | ((uint32_t)f32_to_bf16_bits(p[7]) << 16);

        // V tile into LDS (row-major, padded rows), then read transposed:
        // lane (r, kg) of block db gathers V[pos][16 db + r] over its eight
        // positions
#pragma unroll
        for (int u = 0; u < kVChunks; ++u) {
            const int c = lane + kWave * u;
            const int row = c / (D / 8), cc = c % (D / 8);
            *reinterpret_cast<u32x4*>(vt + row * PITCH + 16 * cc) = vr[u];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const unsigned char* cp = vt + 2 * (16 * db + col);
            uint32_t w[4];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int r0 = 16 * h + 4 * kg + 2 * i;
                    const uint32_t lo = *reinterpret_cast<const uint16_t*>(cp + r0 * PITCH);
                    const uint32_t hi = *reinterpret_cast<const uint16_t*>(cp + (r0 + 1) * PITCH);
                    w[2 * h + i] = lo | (hi << 16);
                }
            const u32x4 vf = {w[0], w[1], w[2], w[3]};
            acc[db] = mfma16x16x32(as_bf16x8(vf), as_bf16x8(pf), acc[db]);
        }
        // the next tile's LDS writes come after every lane's reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // this wave's column sum over the four K groups
    float l_w = l_part;
    l_w += __shfl_xor(l_w, 16, kWave);
    l_w += __shfl_xor(l_w, 32, kWave);

    // merge the four waves: max, rescaled sums and outputs, through LDS
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);          // [wave][16][D + 2]
    float* mine = red + wave * 16 * (D + 2) + col * (D + 2);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[16 * db + 4 * kg + i] = acc[db][i];
    if (kg == 0) {
        mine[D] = m_run;
        mine[D + 1] = l_w;
    }
    __syncthreads();
    const size_t pidx = (((size_t)b * h_kv + j) * n_split + split) * 16;
    for (int e = threadIdx.x; e < g * D; e += kAttnThreads) {
        const int qq = e / D, c = e - qq * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, red[(w * 16 + qq) * (D + 2) + D]);
        float o = 0.0f, L = 0.0f;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) {
            const float* rw = red + (w * 16 + qq) * (D + 2);
            const float f = rw[D] == -INFINITY ? 0.0f : expf(rw[D] - M);
            o += f * rw[c];
            L += f * rw[D + 1];
        }
        part_o[(pidx + qq) * D + c] = o;
        if (c == 0) {
            part_ml[(pidx + qq) * 2] = M;
            part_ml[(pidx + qq) * 2 + 1] = L;
        }
    }
}

// Merge of the splits of one query head: out = sum_s O_s e^(M_s - M) /
// sum_s L_s e^(M_s - M), M = max_s M_s; an empty sequence gives zeros.  A
// block takes `cols` head-dimension elements of one query head (the whole
// head, or 32 of them when there are many splits): its threads take the max
// over the splits together, then each sums one element over a subset of the
// splits (256 / cols subsets), merged through LDS.  Column blocks keep each
// thread's chain of split loads short when a long sequence has many splits;
// with few splits whole heads avoid recomputing the max per block.
constexpr int kMergeThreads = 256;
constexpr int kMergeManySplits = 64;

__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ lens, int h_q, int h_kv, int d, int max_len, int chunk,
    int n_split, int cols, uint16_t* __restrict__ out) {
    __shared__ float red[kMergeThreads];
    __shared__ float red_l[kMergeThreads];
    const int ncb = d / cols;                     // column blocks per head
    const int h = blockIdx.x / ncb;
    const int c0 = (blockIdx.x - h * ncb) * cols;
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int g = h_q / h_kv;
    const int j = h / g, qq = h - j * g;
    const int n_valid = (min(max(lens[b], 0), max_len) + chunk - 1) / chunk;
    uint16_t* o_row = out + ((size_t)b * h_q + h) * d;
    if (n_valid == 0) {
        if (tid < cols) o_row[c0 + tid] = 0;
        return;
    }
    const size_t base = ((size_t)b * h_kv + j) * n_split * 16 + qq;
    float mx = -INFINITY;
    for (int s = tid; s < n_valid; s += kMergeThreads)
        mx = fmaxf(mx, part_ml[(base + (size_t)s * 16) * 2]);
    red[tid] = mx;
    __syncthreads();
    for (int w = kMergeThreads / 2; w > 0; w >>= 1) {
        if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
        __syncthreads();
    }
    const float M = red[0];
    __syncthreads();
    const int nsub = kMergeThreads / cols;
    const int sub = tid / cols, c = c0 + (tid - sub * cols);
    float o = 0.0f, L = 0.0f;
    if (sub < nsub) {
        // eight splits per round, their loads issued together
        constexpr int U = 8;
        int s = sub;
        for (; s + (U - 1) * nsub < n_valid; s += U * nsub) {
            float mv[U], lv[U], ov[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const size_t r = base + (size_t)(s + u * nsub) * 16;
                mv[u] = part_ml[r * 2];
                lv[u] = part_ml[r * 2 + 1];
                ov[u] = part_o[r * d + c];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float f = expf(mv[u] - M);
                o += f * ov[u];
                L += f * lv[u];
            }
        }
        for (; s < n_valid; s += nsub) {
            const size_t r = base + (size_t)s * 16;
            const float f = expf(part_ml[r * 2] - M);
            o += f * part_o[r * d + c];
            L += f * part_ml[r * 2 + 1];
        }
    }
    red[tid] = o;
    red_l[tid] = L;
    __syncthreads();
    if (sub == 0) {
        for (int k2 = 1; k2 < nsub; ++k2) {
            o += red[k2 * cols + tid];
            L += red_l[k2 * cols + tid];
        }
        o_row[c] = f32_to_bf16_bits(o / L);
    }
}

}  // namespace

// Positions per split: a power of two from 256 up, so that a launch has
// about 1024 workgroups (four per CU of a 256-CU MI355X; the partial results
// stay small next to the KV bytes), at most 8192.  (Measured: about 2048
// workgroups from 128 positions up were 1-4 % slower on long batches and
// ragged lengths and 12 % slower on one long sequence, where each workgroup
// then held a single tile per wave; 4096 no better.)
int attn_chunk(int B, int h_kv, int max_len) {
    const long long positions = (long long)B * h_kv * max_len;
    int chunk = 2 * kTilePos * kAttnWaves;
    while (chunk < 8192 && positions / chunk > 1024) chunk *= 2;
    return chunk;
}

size_t attn_workspace_bytes(int B, int h_kv, int d, int max_len) {
    const int chunk = attn_chunk(B, h_kv, max_len);
    const size_t n_split = max_len > 0 ? (size_t)(max_len + chunk - 1) / chunk : 1;
    const size_t rows = (size_t)B * h_kv * n_split * 16;
    return rows * (size_t)d * 4 + rows * 2 * 4;
}

hipError_t launch_attn_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* lens, uint16_t* out, int B, int h_q, int h_kv,
                              int d, int max_len, float scale, void* workspace,
                              const StageEvents& ev, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    const int chunk = attn_chunk(B, h_kv, max_len);
    const int n_split = max_len > 0 ? (max_len + chunk - 1) / chunk : 1;
    const size_t rows = (size_t)B * h_kv * n_split * 16;
    float* part_o = static_cast<float*>(workspace);
    float* part_ml = part_o + rows * d;
    if (max_len > 0) {
        const dim3 grid(B * h_kv, n_split);
        switch (d) {
            case 64:
                hipLaunchKernelGGL(attn_split_kernel<64>, grid, dim3(kAttnThreads), 0, stream, q,
                                   k, v, lens, h_q, h_kv, max_len, chunk, n_split, scale,
                                   part_o, part_ml);
                break;
            case 128:
                hipLaunchKernelGGL(attn_split_kernel<128>, grid, dim3(kAttnThreads), 0, stream,
                                   q, k, v, lens, h_q, h_kv, max_len, chunk, n_split, scale,
                                   part_o, part_ml);
                break;
            case 256:
                hipLaunchKernelGGL(attn_split_kernel<256>, grid, dim3(kAttnThreads), 0, stream,
                                   q, k, v, lens, h_q, h_kv, max_len, chunk, n_split, scale,
                                   part_o, part_ml);
                break;
            default:
                return hipErrorInvalidValue;
        }
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipError_t err = ev.mark(0, stream);
    if (err != hipSuccess) return err;
    const int cols = n_split >= kMergeManySplits ? 32 : d;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(h_q * (d / cols), B), dim3(kMergeThreads), 0,
                       stream, part_o, part_ml, lens, h_q, h_kv, d, max_len, chunk, n_split,
                       cols, out);
    err = hipGetLastError();
    return err == hipSuccess ? ev.mark(1, stream) : err;
}

MOE_DEVICE_CHECK_READER(attn_decode)

}  // namespace moe
