// Measurement helpers.  HBM read-bandwidth probe: the streaming-read ceiling the expert products are
// measured against (the GPU analogue of the STREAM bandwidth the HiNa-MoE
// evaluation quotes for its CPUs, Table 2).  Every byte of the buffer is read
// once with 16-byte non-temporal loads, grid-stride, eight loads in flight per
// lane, 16 workgroups per CU: the fastest of the streaming-read designs tried
// on MI355X (grid-stride or per-workgroup contiguous chunks, 4-16 loads in
// flight, 4-16 workgroups per CU, cached or non-temporal).  Nothing is written
// except, in the unlikely case that the XOR of all loaded words hits a fixed
// value, one word of the sink (which keeps the loads from being optimised
// away).
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr int kProbeBlocksPerCU = 16;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ p,
                                                                   size_t n16,
                                                                   uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * kProbeThreads;
    size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) *sink = 1u;
}

// An empty kernel: a chain of launches measures the dispatch gap between
// back-to-back kernels on a stream (the fixed cost each of a layer's kernels
// adds).
__global__ __launch_bounds__(64) void empty_kernel() {}

}  // namespace

hipError_t launch_empty_chain(int n, hipStream_t stream) {
    for (int i = 0; i < n; ++i) {
        hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, int num_cu,
                             hipStream_t stream) {
    const int grid = num_cu * kProbeBlocksPerCU;
    hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(kProbeThreads), 0, stream,
                       static_cast<const u32x4*>(buf), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace moe
