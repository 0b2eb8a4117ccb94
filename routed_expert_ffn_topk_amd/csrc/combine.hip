// Weighted combine of a forward call: each token's output row from the FP32
// per-slot down outputs y.
//
// HiNa-MoE §4.1 (Fig. 5): the experts' outputs for a token are weighted by
// its routing weights and summed, and the result is written back row-major
// (the third transform).  The sum runs over a token's k slots in ascending
// order, with no atomics: each output element is written once, by one
// thread, and the result does not depend on which expert finished first.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

// out[t][c] = bf16( sum_{j ascending} w[t][j] * y[t*k + j][c] ), skipping
// slots whose expert id is out of range.  Eight columns per thread; the
// transposed [row x token] tiles of the down kernels are already stored
// token-major in y, so this writes plain row-major rows.  The slots of
// experts with more than large_min tokens have their y in `parts` planes of
// K-part partial sums (the tiled down product), added first in plane order.
template <int B>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ ids,
                                                      const float* __restrict__ w,
                                                      uint16_t* __restrict__ out, int T,
                                                      int H, int k, int E,
                                                      const int32_t* __restrict__ counts,
                                                      int large_min, int parts,
                                                      size_t plane) {
    // (the thread index in 64 bits: T * H / 8 passes 2^31 for batches of a
    // few million tokens)
    const int chunks = H / 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)T * chunks) return;
    const int t = (int)(idx / chunks);
    const int c = (int)(idx - (int64_t)t * chunks) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // slots in batches of B: every id, weight and y row of a batch is
    // requested before any is used (slots past k re-read the last one; their
    // values are not used), so a batch costs two memory latencies, not two
    // per slot
    for (int j0 = 0; j0 < k; j0 += B) {
        int e[B];
        float wj[B];
        f32x4 a[B], b[B];
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int slot = t * k + min(j0 + u, k - 1);
            e[u] = ids[slot];
            wj[u] = w[slot];
            a[u] = *reinterpret_cast<const f32x4*>(y + (size_t)slot * H + c);
            b[u] = *reinterpret_cast<const f32x4*>(y + (size_t)slot * H + c + 4);
        }
#pragma unroll
        for (int u = 0; u < B; ++u) {
            if (j0 + u >= k || e[u] < 0 || e[u] >= E) continue;
            f32x4 av = a[u], bv = b[u];
            if (parts > 1 && counts[e[u]] > large_min) {
                const float* yp = y + (size_t)(t * k + j0 + u) * H + c;
                for (int pt = 1; pt < parts; ++pt) {
                    av += *reinterpret_cast<const f32x4*>(yp + pt * plane);
                    bv += *reinterpret_cast<const f32x4*>(yp + pt * plane + 4);
                }
            }
            const float ww = wj[u];
            acc[0] += ww * av.x; acc[1] += ww * av.y; acc[2] += ww * av.z; acc[3] += ww * av.w;
            acc[4] += ww * bv.x; acc[5] += ww * bv.y; acc[6] += ww * bv.z; acc[7] += ww * bv.w;
        }
    }
    u32x4 o;
    o.x = (uint32_t)f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[1]) << 16);
    o.y = (uint32_t)f32_to_bf16_bits(acc[2]) | ((uint32_t)f32_to_bf16_bits(acc[3]) << 16);
    o.z = (uint32_t)f32_to_bf16_bits(acc[4]) | ((uint32_t)f32_to_bf16_bits(acc[5]) << 16);
    o.w = (uint32_t)f32_to_bf16_bits(acc[6]) | ((uint32_t)f32_to_bf16_bits(acc[7]) << 16);
    *reinterpret_cast<u32x4*>(out + (size_t)t * H + c) = o;
}

}  // namespace

hipError_t launch_combine(const float* y, const int32_t* ids, const float* w,
                          uint16_t* out, const FfnShape& s, const int32_t* counts,
                          int large_min, int parts, size_t plane, hipStream_t stream) {
    const int64_t n = (int64_t)s.T * (s.H / 8);
    const int grid = (int)((n + 255) / 256);
    // batch of slots per round of loads: k itself up to 8 (no re-read of
    // the last slot for small k), then 8 at a time
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, stream, y, ids, w, out, s.T, s.H, s.k,
                           s.E, counts, large_min, parts, plane);
    };
    if (s.k <= 1)
        go(combine_kernel<1>);
    else if (s.k <= 2)
        go(combine_kernel<2>);
    else if (s.k <= 4)
        go(combine_kernel<4>);
    else
        go(combine_kernel<8>);
    return hipGetLastError();
}

MOE_DEVICE_CHECK_READER(combine)

}  // namespace moe
