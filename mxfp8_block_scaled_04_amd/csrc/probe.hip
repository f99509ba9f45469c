// One scaled matrix instruction per wave on caller-given operands: a
// diagnostic of v_mfma_scale_f32_32x32x64_f8f6f4 itself (how it forms and
// sums the 64 scaled E4M3 products of one K step and adds the accumulator),
// the arithmetic on which the grouped GEMM's accuracy bound rests.  Not a
// step of the method.
//
// Wave t computes, for m, n in [0, 32):
//   D[t][m][n] = C[t][m][n] + sum_k A[t][m][k] B[t][n][k] 2^(SA[t][m][k/32] - 127) 2^(SB[t][n][k/32] - 127)
// with A, B E4M3 codes [32][64] and SA, SB scale bytes [32][2], exactly as
// the instruction rounds it.  Operand order as in the GEMM: lane l carries
// row l % 32 with K bytes [16 h, 16 h + 16) and [32 + 16 h, 48 + 16 h)
// (h = l / 32) and the scale of K block h; lane l holds output column
// l % 32, rows 8 (i / 4) + 4 h + i % 4 of accumulator register i.
#include "mx_device.h"

namespace mx {
namespace {

__global__ __launch_bounds__(64) void mfma_probe_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                        const uint8_t* __restrict__ SA,
                                                        const uint8_t* __restrict__ SB, const float* __restrict__ C,
                                                        float* __restrict__ D) {
    const int64_t t = blockIdx.x;
    const int l = threadIdx.x;
    const int r = l & 31, h = l >> 5;
    const uint32_t* a = reinterpret_cast<const uint32_t*>(A + (t * 32 + r) * 64);
    const uint32_t* b = reinterpret_cast<const uint32_t*>(B + (t * 32 + r) * 64);
    i32x8 fa, fb;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        fa[q] = (int)a[4 * h + q];
        fa[4 + q] = (int)a[8 + 4 * h + q];
        fb[q] = (int)b[4 * h + q];
        fb[4 + q] = (int)b[8 + 4 * h + q];
    }
    const int sa = SA[(t * 32 + r) * 2 + h];
    const int sb = SB[(t * 32 + r) * 2 + h];
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = C[(t * 32 + 8 * (i / 4) + 4 * h + i % 4) * 32 + r];
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc, 0, 0, 0, sa, 0, sb);
#pragma unroll
    for (int i = 0; i < 16; ++i) D[(t * 32 + 8 * (i / 4) + 4 * h + i % 4) * 32 + r] = acc[i];
}

}  // namespace

hipError_t launch_mfma_probe(const uint8_t* A, const uint8_t* B, const uint8_t* SA, const uint8_t* SB, const float* C,
                             float* D, int32_t T, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)T), dim3(64), 0, stream, A, B, SA, SB, C, D);
    return hipGetLastError();
}

}  // namespace mx
