// C-ABI entry points of libmxmoe: argument validation, then the launchers.
// See include/libmxmoe.h for the contract of each call.
#include "../../include/libmxmoe.h"

#include <hip/hip_runtime.h>

#include "mx_internal.h"

namespace mx {
// probe.hip (diagnostic of the matrix instruction; not a step of the method)
hipError_t launch_mfma_probe(const uint8_t* A, const uint8_t* B, const uint8_t* SA, const uint8_t* SB, const float* C,
                             float* D, int32_t T, hipStream_t stream);
// swiglu_backward_quant.hip
hipError_t launch_swiglu_backward_quant(const uint16_t* preact, const uint16_t* dh, int64_t M, int64_t I,
                                        const int32_t* group_offsets, int32_t G, uint8_t* q, uint8_t* s,
                                        uint8_t* qT, uint8_t* sT, uint8_t* hT, uint8_t* hTs, int64_t Mcap,
                                        int32_t* padded_offsets, hipStream_t stream);
// routing.hip and the gathering dual quantizer (quantize_dual.hip)
hipError_t launch_route_plan(const int32_t* experts, const float* weights, int64_t T, int32_t k, int32_t G,
                             int32_t* offsets, int32_t* src, int32_t* slot_of, float* slot_weight,
                             hipStream_t stream);
hipError_t launch_gather_quantize(const uint16_t* x, int64_t T, int64_t N, int64_t ldx, const int32_t* src,
                                  const float* row_scale, int64_t M, const int32_t* group_offsets, int32_t G,
                                  uint8_t* q, uint8_t* s, uint8_t* qT, uint8_t* sT, int64_t Mcap,
                                  int32_t* padded_offsets, hipStream_t stream);
hipError_t launch_combine(const uint16_t* y, int64_t M, int64_t N, int64_t ldy, const int32_t* slot_of,
                          const float* w, int64_t T, int32_t k, uint16_t* out, hipStream_t stream);
#ifdef MXMOE_DEBUG
// the debug build's error words, one per code object (mx_debug.h)
hipError_t debug_take_quantize(uint32_t* out);
hipError_t debug_take_dual(uint32_t* out);
hipError_t debug_take_gemm(uint32_t* out);
hipError_t debug_take_swiglu_quant(uint32_t* out);
#endif
}  // namespace mx

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

mx_status from_hip(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_HIP; }

constexpr int32_t kMaxGroups = 4096;

}  // namespace

extern "C" {

const char* mx_status_str(int status) {
    switch (status) {
        case MX_OK: return "MX_OK";
        case MX_ERR_NULL: return "MX_ERR_NULL";
        case MX_ERR_SHAPE: return "MX_ERR_SHAPE";
        case MX_ERR_ALIGN: return "MX_ERR_ALIGN";
        case MX_ERR_CAPACITY: return "MX_ERR_CAPACITY";
        case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED";
        case MX_ERR_HIP: return "MX_ERR_HIP";
        default: return "MX_ERR_UNKNOWN";
    }
}

int mx_version(void) { return 100; }

int64_t mx_scale_bytes(int64_t R, int64_t K) {
    if (R < 0 || K < 0) return -1;
    return ((R + 31) / 32) * 32 * (8 * ((K + 255) / 256));
}

int64_t mx_cols_capacity(int64_t M, int32_t G) {
    if (M < 0 || G < 1) return -1;
    return 256 * ((M + 255) / 256 + (int64_t)G - 1);
}

mx_status mx_quantize_rows(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, uint8_t* s,
                           void* stream) {
    if (M < 0 || K < 0 || K % 32 != 0 || ldx < K) return MX_ERR_SHAPE;
    if (M == 0 || K == 0) return MX_OK;
    if (!x || !q || !s) return MX_ERR_NULL;
    if (!aligned16(x) || !aligned16(q) || !aligned16(s) || ldx % 8 != 0) return MX_ERR_ALIGN;
    // one workgroup of kQuantRowsThreads per 32 x 256 unit; total work-items < 2^32
    if (((M + 31) / 32) * ((K + 255) / 256) > (int64_t)(UINT32_MAX / mx::kQuantRowsThreads))
        return MX_ERR_UNSUPPORTED;
    return from_hip(mx::launch_quantize_rows(x, M, K, ldx, q, s, (hipStream_t)stream));
}

mx_status mx_quantize_cols(const uint16_t* x, int64_t M, int64_t N, int64_t ldx, const int32_t* group_offsets,
                           int32_t G, uint8_t* qT, uint8_t* sT, int64_t Mcap, int32_t* padded_offsets,
                           void* stream) {
    if (group_offsets == nullptr) G = 1;
    if (M < 0 || N < 0 || ldx < N || Mcap < 0) return MX_ERR_SHAPE;
    if (G < 1 || G > kMaxGroups) return MX_ERR_SHAPE;
    if (N % 8 != 0) return MX_ERR_UNSUPPORTED;
    if (Mcap % 256 != 0 || Mcap < mx_cols_capacity(M, G)) return MX_ERR_CAPACITY;
    if (group_offsets != nullptr && padded_offsets == nullptr) return MX_ERR_NULL;
    if (N == 0 || Mcap == 0) {
        if (group_offsets == nullptr) return MX_OK;
    } else {
        if (!x && M > 0) return MX_ERR_NULL;
        if (!qT || !sT) return MX_ERR_NULL;
        if ((x && !aligned16(x)) || !aligned16(qT) || !aligned16(sT) || ldx % 8 != 0) return MX_ERR_ALIGN;
    }
    if (Mcap / 256 > (int64_t)UINT32_MAX / 1024 || (N + 63) / 64 > 65535) return MX_ERR_UNSUPPORTED;  // grid
    return from_hip(mx::launch_quantize_cols(x, M, N, ldx, group_offsets, G, qT, sT, Mcap, padded_offsets,
                                             (hipStream_t)stream));
}

mx_status mx_quantize_dual(const uint16_t* x, int64_t M, int64_t N, int64_t ldx, const int32_t* group_offsets,
                           int32_t G, uint8_t* q, uint8_t* s, uint8_t* qT, uint8_t* sT, int64_t Mcap,
                           int32_t* padded_offsets, void* stream) {
    if (group_offsets == nullptr) G = 1;
    if (M < 0 || N < 0 || N % 32 != 0 || ldx < N || Mcap < 0) return MX_ERR_SHAPE;
    if (G < 1 || G > kMaxGroups) return MX_ERR_SHAPE;
    if (Mcap % 256 != 0 || Mcap < mx_cols_capacity(M, G)) return MX_ERR_CAPACITY;
    if (group_offsets != nullptr && padded_offsets == nullptr) return MX_ERR_NULL;
    if (N == 0 || Mcap == 0) {
        if (group_offsets == nullptr) return MX_OK;
    } else {
        if (!x && M > 0) return MX_ERR_NULL;
        if (!qT || !sT || (M > 0 && (!q || !s))) return MX_ERR_NULL;
        if ((x && !aligned16(x)) || !aligned16(qT) || !aligned16(sT) || (q && !aligned16(q)) ||
            (s && !aligned16(s)) || ldx % 8 != 0)
            return MX_ERR_ALIGN;
    }
    if (Mcap / 256 > 65535 || (N + 255) / 256 > (int64_t)UINT32_MAX / 256) return MX_ERR_UNSUPPORTED;  // grid
    return from_hip(mx::launch_quantize_dual(x, M, N, ldx, group_offsets, G, q, s, qT, sT, Mcap, padded_offsets,
                                             (hipStream_t)stream));
}

mx_status mx_grouped_gemm(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                          const int32_t* group_offsets, int32_t G, int64_t M, int64_t N, int64_t K, uint16_t* out,
                          void* stream) {
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return MX_ERR_SHAPE;
    if (G < 1 || G > kMaxGroups) return MX_ERR_SHAPE;
    // the kernels need at least one 256-wide contraction chunk per tile
    if (K % 256 != 0 || K == 0) return MX_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return MX_OK;
    if (!Xq || !Xs || !Wq || !Ws || !group_offsets || !out) return MX_ERR_NULL;
    if (!aligned16(Xq) || !aligned16(Xs) || !aligned16(Wq) || !aligned16(Ws) || !aligned16(out))
        return MX_ERR_ALIGN;
    // 32-bit per-tile offsets inside the kernel: 256 rows of an operand and
    // 256 rows of the output must span < 4 GiB.
    if (K > (1 << 23) || N > (1 << 22)) return MX_ERR_UNSUPPORTED;
    // 32-bit scale offsets: packed scale arrays below 4 GiB
    if (mx_scale_bytes(M, K) >= ((int64_t)1 << 32) || mx_scale_bytes((int64_t)G * N, K) >= ((int64_t)1 << 32))
        return MX_ERR_UNSUPPORTED;
    return from_hip(mx::launch_grouped_gemm(Xq, Xs, Wq, Ws, group_offsets, G, M, N, K, out, (hipStream_t)stream));
}

mx_status mx_grouped_gemm_swiglu(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                                 const int32_t* group_offsets, int32_t G, int64_t M, int64_t I, int64_t K,
                                 uint8_t* hq, uint8_t* hs, uint16_t* preact, void* stream) {
    if (M < 0 || I < 0 || K < 0 || K % 32 != 0) return MX_ERR_SHAPE;
    if (G < 1 || G > kMaxGroups) return MX_ERR_SHAPE;
    if (K % 256 != 0 || K == 0 || I % 128 != 0) return MX_ERR_UNSUPPORTED;
    if (M == 0 || I == 0) return MX_OK;
    if (!Xq || !Xs || !Wq || !Ws || !group_offsets || !hq || !hs) return MX_ERR_NULL;
    if (!aligned16(Xq) || !aligned16(Xs) || !aligned16(Wq) || !aligned16(Ws) || !aligned16(hq) || !aligned16(hs) ||
        (preact && !aligned16(preact)))
        return MX_ERR_ALIGN;
    if (K > (1 << 23) || 2 * I > (1 << 22)) return MX_ERR_UNSUPPORTED;
    if (mx_scale_bytes(M, K) >= ((int64_t)1 << 32) || mx_scale_bytes((int64_t)G * 2 * I, K) >= ((int64_t)1 << 32) ||
        mx_scale_bytes(M, I) >= ((int64_t)1 << 32))
        return MX_ERR_UNSUPPORTED;
    return from_hip(mx::launch_grouped_gemm_swiglu(Xq, Xs, Wq, Ws, group_offsets, G, M, I, K, hq, hs, preact,
                                                   (hipStream_t)stream));
}

mx_status mx_grouped_gemm_dgrad(const uint8_t* dYq, const uint8_t* dYs, const uint8_t* WTq, const uint8_t* WTs,
                                const int32_t* group_offsets, int32_t G, int64_t M, int64_t N, int64_t K,
                                int64_t Wcap, uint16_t* dX, void* stream) {
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || Wcap < 0) return MX_ERR_SHAPE;
    if (G < 1 || G > kMaxGroups) return MX_ERR_SHAPE;
    if (K % 256 != 0 || K == 0) return MX_ERR_UNSUPPORTED;
    if (Wcap % 256 != 0 || Wcap < (int64_t)G * K) return MX_ERR_CAPACITY;
    if (M == 0 || N == 0) return MX_OK;
    if (!dYq || !dYs || !WTq || !WTs || !group_offsets || !dX) return MX_ERR_NULL;
    if (!aligned16(dYq) || !aligned16(dYs) || !aligned16(WTq) || !aligned16(WTs) || !aligned16(dX))
        return MX_ERR_ALIGN;
    if (K > (1 << 23) || N > (1 << 22) || Wcap > (1 << 23)) return MX_ERR_UNSUPPORTED;
    if (mx_scale_bytes(M, K) >= ((int64_t)1 << 32) || mx_scale_bytes(N, Wcap) >= ((int64_t)1 << 32))
        return MX_ERR_UNSUPPORTED;
    return from_hip(mx::launch_grouped_gemm_dgrad(dYq, dYs, WTq, WTs, group_offsets, G, M, N, K, Wcap, dX,
                                                  (hipStream_t)stream));
}

mx_status mx_grouped_gemm_wgrad(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs,
                                const int32_t* padded_offsets, int32_t G, int64_t N, int64_t K, int64_t Mcap,
                                uint16_t* dW, void* stream) {
    if (N < 0 || K < 0 || Mcap < 0) return MX_ERR_SHAPE;
    if (G < 1 || G > kMaxGroups) return MX_ERR_SHAPE;
    if (Mcap % 256 != 0) return MX_ERR_CAPACITY;
    if (N == 0 || K == 0) return MX_OK;
    if (!dW || !padded_offsets) return MX_ERR_NULL;
    if (Mcap > 0 && (!A || !As || !B || !Bs)) return MX_ERR_NULL;
    if ((A && !aligned16(A)) || (As && !aligned16(As)) || (B && !aligned16(B)) || (Bs && !aligned16(Bs)) ||
        !aligned16(dW))
        return MX_ERR_ALIGN;
    if (Mcap > (1 << 23) || K > (1 << 22)) return MX_ERR_UNSUPPORTED;
    if (mx_scale_bytes(N, Mcap) >= ((int64_t)1 << 32) || mx_scale_bytes(K, Mcap) >= ((int64_t)1 << 32))
        return MX_ERR_UNSUPPORTED;
    return from_hip(mx::launch_grouped_gemm_wgrad(A, As, B, Bs, padded_offsets, G, N, K, Mcap, dW,
                                                  (hipStream_t)stream));
}

mx_status mx_swiglu_backward(const uint16_t* preact, const uint16_t* dh, int64_t M, int64_t I, uint16_t* dpre,
                             uint16_t* h, void* stream) {
    if (M < 0 || I < 0 || I % 32 != 0) return MX_ERR_SHAPE;
    if (M == 0 || I == 0) return MX_OK;
    if (!preact || !dh || !dpre) return MX_ERR_NULL;
    if (!aligned16(preact) || !aligned16(dh) || !aligned16(dpre) || (h && !aligned16(h))) return MX_ERR_ALIGN;
    return from_hip(mx::launch_swiglu_backward(preact, dh, M, I, dpre, h, (hipStream_t)stream));
}

mx_status mx_swiglu_backward_quant(const uint16_t* preact, const uint16_t* dh, int64_t M, int64_t I,
                                   const int32_t* group_offsets, int32_t G, uint8_t* q, uint8_t* s, uint8_t* qT,
                                   uint8_t* sT, uint8_t* hT, uint8_t* hTs, int64_t Mcap, int32_t* padded_offsets,
                                   void* stream) {
    if (group_offsets == nullptr) G = 1;
    if (M < 0 || I < 0 || Mcap < 0) return MX_ERR_SHAPE;
    if (G < 1 || G > kMaxGroups) return MX_ERR_SHAPE;
    if (I % 128 != 0) return MX_ERR_UNSUPPORTED;
    if (Mcap % 256 != 0 || Mcap < mx_cols_capacity(M, G)) return MX_ERR_CAPACITY;
    if (group_offsets != nullptr && padded_offsets == nullptr) return MX_ERR_NULL;
    if (I == 0 || Mcap == 0) {
        if (group_offsets == nullptr) return MX_OK;
    } else {
        if (M > 0 && (!preact || !dh || !q || !s)) return MX_ERR_NULL;
        if (!qT || !sT || !hT || !hTs) return MX_ERR_NULL;
        if ((preact && !aligned16(preact)) || (dh && !aligned16(dh)) || (q && !aligned16(q)) ||
            (s && !aligned16(s)) || !aligned16(qT) || !aligned16(sT) || !aligned16(hT) || !aligned16(hTs))
            return MX_ERR_ALIGN;
    }
    if (Mcap / 256 > 65535) return MX_ERR_UNSUPPORTED;  // grid
    return from_hip(mx::launch_swiglu_backward_quant(preact, dh, M, I, group_offsets, G, q, s, qT, sT, hT, hTs, Mcap,
                                                     padded_offsets, (hipStream_t)stream));
}

mx_status mx_route_plan(const int32_t* experts, const float* weights, int64_t T, int32_t k, int32_t G,
                        int32_t* offsets, int32_t* src, int32_t* slot_of, float* slot_weight, void* stream) {
    if (T < 0 || k < 1) return MX_ERR_SHAPE;
    if (G < 1 || G > kMaxGroups) return MX_ERR_SHAPE;
    if (T * (int64_t)k >= ((int64_t)1 << 31)) return MX_ERR_UNSUPPORTED;  // int32 slots
    if (!offsets) return MX_ERR_NULL;
    if (T > 0 && (!experts || !src || !slot_of)) return MX_ERR_NULL;
    if (slot_weight && !weights && T > 0) return MX_ERR_NULL;
    if (!aligned4(offsets) || (experts && !aligned4(experts)) || (src && !aligned4(src)) ||
        (slot_of && !aligned4(slot_of)) || (weights && !aligned4(weights)) || (slot_weight && !aligned4(slot_weight)))
        return MX_ERR_ALIGN;
    return from_hip(mx::launch_route_plan(experts, weights, T, k, G, offsets, src, slot_of, slot_weight,
                                          (hipStream_t)stream));
}

mx_status mx_gather_quantize(const uint16_t* x, int64_t T, int64_t N, int64_t ldx, const int32_t* src,
                             const float* row_scale, int64_t M, const int32_t* group_offsets, int32_t G, uint8_t* q,
                             uint8_t* s, uint8_t* qT, uint8_t* sT, int64_t Mcap, int32_t* padded_offsets,
                             void* stream) {
    if (group_offsets == nullptr) G = 1;
    if (T < 0 || M < 0 || N < 0 || N % 32 != 0 || ldx < N || Mcap < 0) return MX_ERR_SHAPE;
    if (G < 1 || G > kMaxGroups) return MX_ERR_SHAPE;
    if (Mcap % 256 != 0 || Mcap < mx_cols_capacity(M, G)) return MX_ERR_CAPACITY;
    if (group_offsets != nullptr && padded_offsets == nullptr) return MX_ERR_NULL;
    if (N == 0 || Mcap == 0) {
        if (group_offsets == nullptr) return MX_OK;
    } else {
        if ((!x && T > 0) || (!src && M > 0)) return MX_ERR_NULL;
        if (!qT || !sT || (M > 0 && (!q || !s))) return MX_ERR_NULL;
        if ((x && !aligned16(x)) || !aligned16(qT) || !aligned16(sT) || (q && !aligned16(q)) ||
            (s && !aligned16(s)) || ldx % 8 != 0 || (src && !aligned4(src)) || (row_scale && !aligned4(row_scale)))
            return MX_ERR_ALIGN;
    }
    if (Mcap / 256 > 65535 || (N + 255) / 256 > (int64_t)UINT32_MAX / 256) return MX_ERR_UNSUPPORTED;  // grid
    return from_hip(mx::launch_gather_quantize(x, T, N, ldx, src, row_scale, M, group_offsets,
                                               G, q, s, qT, sT, Mcap, padded_offsets, (hipStream_t)stream));
}

mx_status mx_combine(const uint16_t* y, int64_t M, int64_t N, int64_t ldy, const int32_t* slot_of,
                     const float* weights, int64_t T, int32_t k, uint16_t* out, void* stream) {
    if (M < 0 || N < 0 || ldy < N || T < 0 || k < 1) return MX_ERR_SHAPE;
    if (N % 8 != 0) return MX_ERR_UNSUPPORTED;
    if (T == 0 || N == 0) return MX_OK;
    if (!slot_of || !out || (M > 0 && !y)) return MX_ERR_NULL;
    if ((y && !aligned16(y)) || !aligned16(out) || ldy % 8 != 0 || !aligned4(slot_of) ||
        (weights && !aligned4(weights)))
        return MX_ERR_ALIGN;
    // grid: T workgroups of 256 lanes (the combine kernel's size; total
    // work-items < 2^32) by N / 2048
    if (T > (int64_t)(UINT32_MAX / 256) || (N / 8 + 255) / 256 > 65535) return MX_ERR_UNSUPPORTED;
    return from_hip(mx::launch_combine(y, M, N, ldy, slot_of, weights, T, k, out, (hipStream_t)stream));
}

mx_status mx_validate_offsets(const int32_t* group_offsets, int32_t G, int64_t M, int32_t* result, void* stream) {
    if (G < 1 || G > kMaxGroups || M < 0) return MX_ERR_SHAPE;
    if (!group_offsets || !result) return MX_ERR_NULL;
    return from_hip(mx::launch_validate_offsets(group_offsets, G, M, result, (hipStream_t)stream));
}

mx_status mx_stream21(const void* src, void* dst, int64_t dst_bytes, void* stream) {
    if (dst_bytes < 0 || dst_bytes % 16 != 0) return MX_ERR_SHAPE;
    if (dst_bytes == 0) return MX_OK;
    if (!src || !dst) return MX_ERR_NULL;
    if (!aligned16(src) || !aligned16(dst)) return MX_ERR_ALIGN;
    // one lane per 2 granules (16 bytes read, 8 written each): work-items < 2^32
    if (dst_bytes / 16 >= ((int64_t)1 << 32) - 256) return MX_ERR_UNSUPPORTED;
    return from_hip(mx::launch_stream21(src, dst, dst_bytes, (hipStream_t)stream));
}

mx_status mx_probe_mfma_scale(const uint8_t* A, const uint8_t* B, const uint8_t* SA, const uint8_t* SB,
                              const float* C, float* D, int32_t T, void* stream) {
    if (T < 0 || T > 65536) return MX_ERR_SHAPE;
    if (T == 0) return MX_OK;
    if (!A || !B || !SA || !SB || !C || !D) return MX_ERR_NULL;
    if (!aligned16(A) || !aligned16(B) || !aligned16(C) || !aligned16(D)) return MX_ERR_ALIGN;
    return from_hip(mx::launch_mfma_probe(A, B, SA, SB, C, D, T, (hipStream_t)stream));
}

mx_status mx_debug_flags(uint32_t* flags, void* stream) {
    if (!flags) return MX_ERR_NULL;
    *flags = 0;
#ifdef MXMOE_DEBUG
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MX_ERR_HIP;
    uint32_t all = 0;
    for (hipError_t (*take)(uint32_t*) :
         {mx::debug_take_quantize, mx::debug_take_dual, mx::debug_take_gemm, mx::debug_take_swiglu_quant}) {
        uint32_t w = 0;
        if (take(&w) != hipSuccess) return MX_ERR_HIP;
        all |= w;
    }
    *flags = all;
    return MX_OK;
#else
    (void)stream;
    return MX_ERR_UNSUPPORTED;
#endif
}

}  // extern "C"
