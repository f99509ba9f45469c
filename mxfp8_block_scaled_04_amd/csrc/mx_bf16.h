// bf16 pairs packed in a dword (element 0 in the low half): unpacking to
// fp32 and packing back with round-to-nearest-even.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// two floats -> two bf16 (nearest even), a in the low half
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

}  // namespace mx
