// Device-side helpers shared by the MoE FFN kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

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

// The four values of a lane's quad (lanes 4j .. 4j+3), in quad order: DPP
// quad_perm broadcasts of quad positions 0, 1, 2, 3.
__device__ __forceinline__ f32x4 quad_gather_f32(float v) {
    const int b = __builtin_bit_cast(int, v);
    return f32x4{__builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0x00, 0xf, 0xf, false)),
                 __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0x55, 0xf, 0xf, false)),
                 __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0xaa, 0xf, 0xf, false)),
                 __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0xff, 0xf, 0xf, false))};
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

// LDS address space (destination of the direct global->LDS loads).
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// ---------------------------------------------------------------------------
// Device bounds checks of the debug build (compiled with
// -DMOE_FFN_DEVICE_CHECKS: libmoe_ffn_debug.so).  MOE_IN_BOUNDS(cond) guards
// an index before a global access: in the debug build a false condition
// records the source line in this translation unit's check word (the first
// failing line wins, a vector atomic) and yields false, and the caller then
// skips the access or substitutes a valid index, so a bad index becomes a
// report (moe_ffn_device_check) rather than a memory fault.  Release builds
// compile the guards away (the condition is not even evaluated).
// ---------------------------------------------------------------------------
#ifdef MOE_FFN_DEVICE_CHECKS
namespace {
__device__ int g_check_line;
}
__device__ __forceinline__ bool check_bound(bool ok, int line) {
    if (!ok) atomicCAS(&g_check_line, 0, line);
    return ok;
}
#define MOE_IN_BOUNDS(cond) ::moe::check_bound((cond), __LINE__)
// Host side: the first failing line of this translation unit since the last
// read (0: none), cleared by the read.
#define MOE_DEVICE_CHECK_READER(name)                                               \
    hipError_t device_check_##name(int* line) {                                     \
        hipError_t e = hipMemcpyFromSymbol(line, HIP_SYMBOL(g_check_line), sizeof(int)); \
        const int zero = 0;                                                         \
        if (e == hipSuccess)                                                        \
            e = hipMemcpyToSymbol(HIP_SYMBOL(g_check_line), &zero, sizeof(int));    \
        return e;                                                                   \
    }
#else
#define MOE_IN_BOUNDS(cond) true
#define MOE_DEVICE_CHECK_READER(name)                                               \
    hipError_t device_check_##name(int* line) {                                     \
        *line = 0;                                                                  \
        return hipSuccess;                                                          \
    }
#endif

// Wait until at most N vector-memory loads of this wave are outstanding
// (loads complete in issue order), leaving LDS and export counters alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------------------
// Wave-wide reductions with DPP (data-parallel primitives: a VALU operand
// read from another lane of the same row).  Inclusive scan over the 64
// lanes: shifts by 1, 2, 4 and 8 lanes within each row of 16, then the last
// lane of row 0 / row 2 into rows 1 / 3 (row_bcast:15), then lane 31 into
// rows 2 and 3 (row_bcast:31).  Lane 63 ends with the total.  Lanes whose
// source is outside the row, or rows masked off, take the identity.  All 64
// lanes must be active.
// ---------------------------------------------------------------------------
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114,
              kDppRowShr8 = 0x118, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <class Op>
__device__ __forceinline__ int wave_scan_i32(int v, int identity, Op op) {
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowShr1, 0xf, 0xf, false));
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowShr2, 0xf, 0xf, false));
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowShr4, 0xf, 0xf, false));
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowShr8, 0xf, 0xf, false));
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowBcast15, 0xa, 0xf, false));
    v = op(v, __builtin_amdgcn_update_dpp(identity, v, kDppRowBcast31, 0xc, 0xf, false));
    return v;
}

__device__ __forceinline__ int wave_max_i32(int v) {
    v = wave_scan_i32(v, INT_MIN, [](int a, int b) { return a > b ? a : b; });
    return __builtin_amdgcn_readlane(v, kWave - 1);
}

__device__ __forceinline__ int wave_min_i32(int v) {
    v = wave_scan_i32(v, INT_MAX, [](int a, int b) { return a < b ? a : b; });
    return __builtin_amdgcn_readlane(v, kWave - 1);
}

// Inclusive prefix sum over the lanes.
__device__ __forceinline__ int wave_prefix_sum_i32(int v) {
    return wave_scan_i32(v, 0, [](int a, int b) { return a + b; });
}

// Sum over the lanes, in the fixed order of the scan.
__device__ __forceinline__ float wave_sum_f32(float v) {
    auto add = [](int a, int b) {
        return __builtin_bit_cast(int, __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
    };
    const int r = wave_scan_i32(__builtin_bit_cast(int, v), 0, add);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(r, kWave - 1));
}

}  // namespace moe
