// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int BLK = 64;          // tokens per block (query and key side)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(8))) int32_t i32x8;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 pair, packed low = a, high = b
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 r;
    r[0] = static_cast<__bf16>(a);
    r[1] = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float a) {
    return static_cast<uint16_t>(pack_bf16x2(a, 0.0f) & 0xFFFFu);
}

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

// Round-to-nearest-even fp32 -> fp16 pair, packed low = a, high = b
// (v_cvt_pk_f16_f32 on gfx950); magnitudes beyond 65504 become inf.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    f16x2 r;
    r[0] = static_cast<_Float16>(a);
    r[1] = static_cast<_Float16>(b);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t f32_to_f16(float a) {
    return static_cast<uint16_t>(pack_f16x2(a, 0.0f) & 0xFFFFu);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Lanes l and l ^ 32 combined (v_permlane32_swap, no LDS round trip): with
// both operands = x the swap returns (own, other) in the low half of the wave
// and (other, own) in the high half, so a symmetric combination of the two
// results is the same on both lanes.
__device__ __forceinline__ float pair_max(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, static_cast<uint32_t>(r[0])),
                 __builtin_bit_cast(float, static_cast<uint32_t>(r[1])));
}

__device__ __forceinline__ float pair_sum(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, static_cast<uint32_t>(r[0])) +
           __builtin_bit_cast(float, static_cast<uint32_t>(r[1]));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// fp8 e4m3 (OCP) byte pair from two floats, round to nearest even, written
// into the low (HIGH = false) or high 16 bits of `old`.
template <bool HIGH>
__device__ __forceinline__ uint32_t pack_fp8x2(float a, float b, uint32_t old) {
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, static_cast<int>(old), HIGH));
}

}  // namespace sa
