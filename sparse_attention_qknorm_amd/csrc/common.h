// Shared device helpers for the gfx950 kernels of the joint-sequence attention layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace saq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;   // MI355X: 8 accelerator complex dies, workgroups dealt round-robin

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    __bf16 h = (__bf16)x;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Map a hardware workgroup id to a logical work item so that each XCD gets one
// contiguous range of logical items (hardware deals ids round-robin over XCDs).
__device__ __forceinline__ int64_t xcd_contiguous_index(int64_t hw, int64_t n) {
    const int64_t xcd = hw % kNumXcd;
    const int64_t idx = hw / kNumXcd;
    const int64_t q = n / kNumXcd;
    const int64_t r = n % kNumXcd;
    return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

}  // namespace saq
