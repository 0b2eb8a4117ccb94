// Device-side helpers shared by the MoE FFN kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Ordinary 16-byte global load.  Weights are read once per call, but on the
// row-tile pattern of the kernels cached loads stream HBM faster than
// non-temporal ones (measured on MI355X), and every weight byte is still
// fetched from HBM exactly once.
__device__ __forceinline__ u32x4 load16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies row
// (l % 16) of A and column (l % 16) of B, each as 8 K values of K-group
// (l / 16) (any K order works as long as A and B use the same one); it
// receives D[4 * (l / 16) + q][l % 16], q = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// FP32 -> BF16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float silu(float g) {
    return g / (1.0f + expf(-g));
}

// Number of XCDs (accelerator dies with private L2) on gfx950; workgroups of
// a launch are handed to them round-robin by workgroup id.
constexpr int kXcds = 8;

}  // namespace moe
