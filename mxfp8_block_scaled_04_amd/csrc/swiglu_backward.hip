// Backward pass of SwiGLU for the MoE layer (the activation between the
// gate+up and down projections; kucoin.com MoK page, section 02, on the
// MXFP8 data path through the SwiGLU step).  With sigma(g) = 1 / (1 + e^-g):
//   h       = silu(g) u = g sigma(g) u
//   d gate  = dh u silu'(g),   silu'(g) = sigma(g) (1 + g (1 - sigma(g)))
//   d up    = dh silu(g)
// in fp32 (hardware exp2 and reciprocal), results rounded to bf16 (nearest
// even).  gate/up (and their gradients) are stored in the interleaved column
// order of the fused forward kernel: columns [64 b, 64 b + 32) are the gate
// values of hidden units [32 b, 32 b + 32), columns [64 b + 32, 64 b + 64)
// their up values.  Bound by HBM: 6 bytes read and 6 written per hidden unit
// (4 written without h).
#include "mx_device.h"
#include "mx_internal.h"
#include "mx_swiglu.h"

namespace mx {
namespace {

__device__ __forceinline__ void store_stream16(void* p, uint4 v) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// One lane: 8 consecutive hidden units c0 .. c0 + 7 of one row (c0 % 8 == 0):
// 16 bytes of gate, of up and of dh in, 16 bytes of d gate, d up (and h) out.
template <bool WRITE_H>
__global__ __launch_bounds__(256) void swiglu_backward_kernel(const uint16_t* __restrict__ pre,
                                                              const uint16_t* __restrict__ dh, int64_t M, int64_t I,
                                                              uint16_t* __restrict__ dpre, uint16_t* __restrict__ hout) {
    const int64_t upr = I / 8;
    const int64_t units = M * upr;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t unit = (int64_t)blockIdx.x * 256 + threadIdx.x; unit < units; unit += stride) {
        const int64_t m = unit / upr;
        const int64_t c0 = (unit - m * upr) * 8;
        const int64_t b = c0 >> 5, j = c0 & 31;
        const int64_t gcol = m * 2 * I + 64 * b + j;  // gate columns; up columns 32 further
        const uint4 gv = load_stream16(pre + gcol);
        const uint4 uv = load_stream16(pre + gcol + 32);
        const uint4 dv = load_stream16(dh + m * I + c0);
        const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
        const uint32_t uw[4] = {uv.x, uv.y, uv.z, uv.w};
        const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w};
        uint32_t og[4], ou[4], oh[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const Grad r0 = swiglu_grad(lo_bf16(gw[k]), lo_bf16(uw[k]), lo_bf16(dw[k]));
            const Grad r1 = swiglu_grad(hi_bf16(gw[k]), hi_bf16(uw[k]), hi_bf16(dw[k]));
            og[k] = pack_bf16(r0.dg, r1.dg);
            ou[k] = pack_bf16(r0.du, r1.du);
            oh[k] = pack_bf16(r0.h, r1.h);
        }
        // d gate and d up fill the two 64-byte halves of each 128-byte line
        // from two store instructions: ordinary stores, so that L2 joins the
        // halves (measured 11 % faster than non-temporal ones)
        *reinterpret_cast<uint4*>(dpre + gcol) = make_uint4(og[0], og[1], og[2], og[3]);
        *reinterpret_cast<uint4*>(dpre + gcol + 32) = make_uint4(ou[0], ou[1], ou[2], ou[3]);
        if (WRITE_H) store_stream16(hout + m * I + c0, make_uint4(oh[0], oh[1], oh[2], oh[3]));
    }
}

}  // namespace

hipError_t launch_swiglu_backward(const uint16_t* preact, const uint16_t* dh, int64_t M, int64_t I, uint16_t* dpre,
                                  uint16_t* h, hipStream_t stream) {
    if (M == 0 || I == 0) return hipSuccess;
    const int64_t units = M * (I / 8);
    int64_t blocks = (units + 255) / 256;
    const int64_t cap = 256 * 32;  // grid-stride beyond 32 workgroups per CU
    if (blocks > cap) blocks = cap;
    if (h) hipLaunchKernelGGL((swiglu_backward_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, stream, preact, dh,
                              M, I, dpre, h);
    else hipLaunchKernelGGL((swiglu_backward_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, stream, preact, dh,
                            M, I, dpre, h);
    return hipGetLastError();
}

}  // namespace mx
