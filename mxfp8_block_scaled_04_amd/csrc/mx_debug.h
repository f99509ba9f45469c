// Debug build (compiled with MXMOE_DEBUG): the kernels that take group
// offsets check the device-side part of their contract and record each kind
// of violation as a bit of an error word held by their code object; the C
// entry point mx_debug_flags reads and clears those words.  A check only
// records: the kernels clamp malformed offsets either way, so every access
// stays in bounds with or without the debug build.  In the release build the
// checks compile to nothing.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

enum : uint32_t {
    kDbgOffsets = 1u,  // group offsets not 0 <= o[0] <= ... <= o[G] <= M
    kDbgPadded = 2u,   // padded offsets not multiples of 256, not increasing by the
                       // padded group sizes, or past the capacity
    kDbgTile = 4u,     // a work tile with no rows of its group
};

#ifdef MXMOE_DEBUG
// one error word per code object (static: every source file has its own)
static __device__ uint32_t debug_word;

__device__ __forceinline__ void debug_flag(bool cond, uint32_t bit) {
    if (cond) __hip_atomic_fetch_or(&debug_word, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Host: this code object's error word, then cleared (after the caller has
// synchronized the stream its kernels ran on).
static inline hipError_t debug_take_word(uint32_t* out) {
    hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(debug_word), sizeof(uint32_t));
    if (e != hipSuccess) return e;
    const uint32_t zero = 0;
    return hipMemcpyToSymbol(HIP_SYMBOL(debug_word), &zero, sizeof(uint32_t));
}
#else
__device__ __forceinline__ void debug_flag(bool, uint32_t) {}
#endif

// Offsets check shared by the kernels: entry g of a G+1 array against its
// successor and the range [0, M].
__device__ __forceinline__ bool offsets_entry_bad(const int32_t* off, int g, int G, int64_t M) {
    const int64_t v = off[g];
    if (v < 0 || v > M) return true;
    return g < G && off[g + 1] < v;
}

}  // namespace mx
