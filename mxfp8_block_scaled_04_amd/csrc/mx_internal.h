// Internal launchers of libmxmoe (host side).  Arguments are validated by
// the C-ABI layer before these are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// Workgroup size of the row-wise quantize kernel (one workgroup per unit of
// 32 rows x 256 columns); the entry point bounds the grid with it.
constexpr int kQuantRowsThreads = 512;

hipError_t launch_quantize_rows(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                                uint8_t* s, hipStream_t stream);

// P[0..G] (padded column offsets of the column-wise layout) from the group
// offsets, one workgroup.
hipError_t launch_cols_prefix(const int32_t* group_offsets, int32_t G, int64_t M, int32_t* padded_offsets,
                              hipStream_t stream);

hipError_t launch_quantize_cols(const uint16_t* x, int64_t M, int64_t N, int64_t ldx,
                                const int32_t* group_offsets, int32_t G, uint8_t* qT, uint8_t* sT,
                                int64_t Mcap, int32_t* padded_offsets, hipStream_t stream);

hipError_t launch_quantize_dual(const uint16_t* x, int64_t M, int64_t N, int64_t ldx,
                                const int32_t* group_offsets, int32_t G, uint8_t* q, uint8_t* s, uint8_t* qT,
                                uint8_t* sT, int64_t Mcap, int32_t* padded_offsets, hipStream_t stream);

hipError_t launch_grouped_gemm(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq,
                               const uint8_t* Ws, const int32_t* group_offsets, int32_t G, int64_t M,
                               int64_t N, int64_t K, uint16_t* out, hipStream_t stream);

hipError_t launch_grouped_gemm_swiglu(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                                      const int32_t* group_offsets, int32_t G, int64_t M, int64_t I, int64_t K,
                                      uint8_t* hq, uint8_t* hs, uint16_t* preact, hipStream_t stream);

hipError_t launch_grouped_gemm_dgrad(const uint8_t* dYq, const uint8_t* dYs, const uint8_t* WTq,
                                     const uint8_t* WTs, const int32_t* group_offsets, int32_t G, int64_t M,
                                     int64_t N, int64_t K, int64_t Wcap, uint16_t* dX, hipStream_t stream);

hipError_t launch_grouped_gemm_wgrad(const uint8_t* A, const uint8_t* As, const uint8_t* B,
                                     const uint8_t* Bs, const int32_t* padded_offsets, int32_t G,
                                     int64_t N, int64_t K, int64_t Mcap, uint16_t* dW,
                                     hipStream_t stream);

hipError_t launch_swiglu_backward(const uint16_t* preact, const uint16_t* dh, int64_t M, int64_t I, uint16_t* dpre,
                                  uint16_t* h, hipStream_t stream);

hipError_t launch_validate_offsets(const int32_t* offsets, int32_t G, int64_t M, int32_t* result,
                                  hipStream_t stream);

hipError_t launch_stream21(const void* src, void* dst, int64_t dst_bytes, hipStream_t stream);

}  // namespace mx
