// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// gfx950 converts with v_cvt_pk_bf16_f32: round to nearest even.
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 load16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void store16(void* p, u32x4 v) { *(u32x4*)p = v; }

// 16 consecutive bytes from global memory, or zeros when !valid (no load issued).
__device__ __forceinline__ u32x4 load16_or_zero(const void* p, bool valid) {
    u32x4 z = {0u, 0u, 0u, 0u};
    return valid ? load16(p) : z;
}

// Row of the first GEMM operand for grouped row r: r itself, or the token
// of assignment rowmap[r] (K slots per token; -1 reads token 0).
__device__ __forceinline__ int src_row(const int32_t* rowmap, int topk, int r) {
    if (!rowmap) return r;
    const int a = rowmap[r];
    return a < 0 ? 0 : a / topk;
}

// SiLU(z) = z * sigmoid(z), with the hardware reciprocal (1 ulp) in place of
// an IEEE divide: the result is rounded to bf16 or summed in fp32 next.
// exp(-z) = inf for very negative z gives z * 0 = -0, the limit.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Wave-wide reductions (64 lanes).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// MFMA wrappers (gfx950 bf16 with fp32 accumulation).
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace moe
