// HBM calibration stream: the read:write ratio of the quantizers (2 bytes of
// bf16 read per byte of fp8 written) and their access pattern (16 bytes read
// and 8 bytes written per lane, non-temporal), with none of their arithmetic:
// 8-byte granule i of dst = words 0 ^ 1 and 2 ^ 3 of 16-byte granule i of
// src.  Two granules per lane, 256 lanes apart; a one-shot grid.  Its rate is
// the practical streaming ceiling the quantize kernels are compared with,
// next to the 8 TB/s specification.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {
namespace {

constexpr int kPer = 2;  // granules per lane

__global__ __launch_bounds__(256) void stream21_kernel(const u32x4* __restrict__ src, u32x2* __restrict__ dst,
                                                       int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * 256 * kPer + threadIdx.x;
    u32x4 v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int64_t o = base + (int64_t)i * 256;
        if (o < n) v[i] = __builtin_nontemporal_load(src + o);
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int64_t o = base + (int64_t)i * 256;
        if (o < n) __builtin_nontemporal_store(u32x2{v[i].x ^ v[i].y, v[i].z ^ v[i].w}, dst + o);
    }
}

}  // namespace

hipError_t launch_stream21(const void* src, void* dst, int64_t dst_bytes, hipStream_t stream) {
    const int64_t n = dst_bytes / 8;  // granules: 16 bytes in, 8 bytes out
    if (n == 0) return hipSuccess;
    const int64_t blocks = (n + 256 * kPer - 1) / (256 * kPer);
    hipLaunchKernelGGL(stream21_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x2*>(dst), n);
    return hipGetLastError();
}

}  // namespace mx
