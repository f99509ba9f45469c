// Device-side check of a group_offsets array (the boundary leaves malformed
// offsets undefined and clamps them; this lets a caller verify them without
// a host read): 0 <= o[0] <= o[1] <= ... <= o[G] <= M.  One workgroup;
// result[0] = 0 if the array is valid, else 1 + the first index that breaks
// the rule.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {
namespace {

__global__ __launch_bounds__(1024) void validate_offsets_kernel(const int32_t* __restrict__ off, int32_t G, int64_t M,
                                                                int32_t* __restrict__ result) {
    __shared__ int32_t first_bad;
    if (threadIdx.x == 0) first_bad = 0x7FFFFFFF;
    __syncthreads();
    for (int i = threadIdx.x; i <= G; i += 1024) {
        const int64_t v = off[i];
        const bool bad = v < 0 || v > M || (i > 0 && v < (int64_t)off[i - 1]);
        if (bad) atomicMin(&first_bad, i);
    }
    __syncthreads();
    if (threadIdx.x == 0) result[0] = first_bad == 0x7FFFFFFF ? 0 : first_bad + 1;
}

}  // namespace

hipError_t launch_validate_offsets(const int32_t* offsets, int32_t G, int64_t M, int32_t* result, hipStream_t stream) {
    hipLaunchKernelGGL(validate_offsets_kernel, dim3(1), dim3(1024), 0, stream, offsets, G, M, result);
    return hipGetLastError();
}

}  // namespace mx
