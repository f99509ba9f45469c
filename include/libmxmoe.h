/*
 * libmxmoe -- MXFP8 quantization and block-scaled grouped GEMM for AMD
 * Instinct MI355X (gfx950).  C ABI.
 *
 * What it computes follows the public write-ups on Cursor's Blackwell MoE
 * kernels:
 *  - lpnh.cn 2479732, section 1: MX block scaling -- cut the tensor into
 *    blocks of 32 elements, compute one scale per block, divide the block by
 *    it and cast to FP8 E4M3; the forward pass quantizes its input matrix
 *    and writes it back to memory, the backward pass needs a transposed
 *    quantization as well.
 *  - aigc.bar "被忽视的量化税" / "秘密武器": the quantization kernel writes its
 *    scales in the layout the matrix instruction consumes, so no reshape pass
 *    sits between quantization and the GEMM; FP8 E4M3 with block size 32.
 *  - aigc.bar "为MoE量身定制优化": the per-expert grouped GEMM, scheduled with
 *    expert-aware cache reuse.
 * Readings of what the pages leave open (fixed here, identical in every
 * entry point):
 *  - scale byte S is E8M0 (value 2^(S-127)); S = clamp(floor(log2 amax) - 8,
 *    -127, 127) + 127, and S = 0 for an all-zero block;
 *  - element code = OCP E4M3FN of x * 2^(127-S), saturated to +/-448, round to
 *    nearest even, sign kept for zero; bf16 subnormals are exact inputs;
 *  - inputs are finite (non-finite inputs give unspecified codes).
 *
 * Data formats
 *  - bf16 tensors are arrays of uint16 bit patterns, row-major.
 *  - FP8 codes are one byte per element, row-major, same shape as the input
 *    (column-wise results are stored transposed, see mx_quantize_cols).
 *  - Scales are stored in the PACKED order of the gfx950 instruction
 *    v_mfma_scale_f32_32x32x64_f8f6f4, for a matrix of R rows and a
 *    contraction length K (K % 32 == 0):
 *        KB     = 8 * ceil(K / 256)                 bytes per row
 *        size   = ceil(R / 32) * 32 * KB            bytes (mx_scale_bytes)
 *        offset(r, b) = (r / 32) * 32 * KB + (b / 8) * 256
 *                       + 4 * (32 * (b % 2) + r % 32) + (b % 8) / 2
 *    for row r and 32-wide block b.  Each 256-byte unit is the 64 lane
 *    registers of one 32-row x 256-K slice in lane order; byte j of a lane
 *    register serves the j-th 64-wide K step.  Pad bytes are written as 0.
 *
 * Conventions
 *  - Every pointer argument is a DEVICE pointer owned by the caller.  The
 *    library allocates nothing, keeps no state, never synchronizes and never
 *    reads device data on the host (mx_debug_flags of the debug build
 *    excepted).  Every call is asynchronous on `stream`
 *    (a hipStream_t; NULL = the default stream).
 *  - Host-checkable preconditions are validated before any launch; a
 *    failing call returns an error code and launches nothing.  A launch
 *    failure returns MX_ERR_HIP.
 *  - group_offsets is an int32 device array of G+1 exclusive prefix
 *    offsets: [0] = 0, non-decreasing, [G] = M; empty groups are allowed.
 *    Entries are clamped on the device to stay monotone within [0, M], so a
 *    malformed array gives wrong results but no out-of-bounds access.
 *  - M = 0 (and empty groups) are legal and do no work.
 */
#ifndef LIBMXMOE_H
#define LIBMXMOE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MX_OK = 0,
    MX_ERR_NULL = 1,        /* a required pointer is NULL */
    MX_ERR_SHAPE = 2,       /* negative size, K % 32 != 0, ld too small, ... */
    MX_ERR_ALIGN = 3,       /* a pointer or leading dimension is not 16-byte aligned */
    MX_ERR_CAPACITY = 4,    /* Mcap below mx_cols_capacity(M, G) or not a multiple of 256 */
    MX_ERR_UNSUPPORTED = 5, /* valid per the format but not supported by these kernels */
    MX_ERR_HIP = 6          /* the HIP runtime reported an error at launch */
} mx_status;

/* Short human-readable name of a status code (static string). */
const char* mx_status_str(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int mx_version(void);

/* Bytes of the packed scale array for R rows and contraction length K. */
int64_t mx_scale_bytes(int64_t R, int64_t K);

/* Upper bound of the padded column count of mx_quantize_cols for M rows in
 * G groups: 256 * (ceil(M / 256) + G - 1) (G = 1 when offsets are NULL). */
int64_t mx_cols_capacity(int64_t M, int32_t G);

/*
 * Row-wise MXFP8 quantization (scales along K; the forward-pass operand
 * layout -- lpnh.cn 2479732 section 1).
 *   x   bf16 [M][ldx] (first K columns used), 16-byte aligned, ldx % 8 == 0
 *   q   uint8 [M][K] codes, 16-byte aligned
 *   s   packed scales for R = M rows, contraction K (mx_scale_bytes(M, K))
 * Requires K % 32 == 0, ldx >= K.  MX_ERR_UNSUPPORTED when
 * ceil(M / 32) * ceil(K / 256) exceeds 2^23 - 1 (the launch grid would pass
 * 2^32 work-items).
 */
mx_status mx_quantize_rows(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                           uint8_t* s, void* stream);

/*
 * Column-wise (transposed) MXFP8 quantization: blocks of 32 consecutive rows
 * of one column (the backward-pass transpose-quantize -- lpnh.cn 2479732
 * section 1).  Rows are split into groups by group_offsets (NULL = one
 * group of all M rows, G ignored); blocks restart at each group's first row
 * and the group's tail is zero-padded to a multiple of 256 rows.  Group g
 * lands at padded column P[g] = sum_{h<g} 256 * ceil(m_h / 256) of the
 * transposed result.
 *   x        bf16 [M][ldx] (first N columns used), 16-byte aligned, ldx % 8 == 0
 *   qT       uint8 [N][Mcap] codes (row n = column n of x); columns >= P[G] are 0
 *   sT       packed scales for R = N rows, contraction Mcap (mx_scale_bytes(N, Mcap))
 *   padded_offsets  int32 [G+1] device output P (required when group_offsets
 *            is given; may be NULL otherwise)
 * Requires N % 8 == 0, Mcap % 256 == 0, Mcap >= mx_cols_capacity(M, G),
 * 1 <= G <= 4096.
 */
mx_status mx_quantize_cols(const uint16_t* x, int64_t M, int64_t N, int64_t ldx,
                           const int32_t* group_offsets, int32_t G, uint8_t* qT, uint8_t* sT,
                           int64_t Mcap, int32_t* padded_offsets, void* stream);

/*
 * Dual-layout quantization: one read of x, both results.  The backward pass
 * needs a bf16 gradient quantized along both of its axes (lpnh.cn 2479732
 * section 1: the backward pass adds a transposed quantization; aigc.bar
 * "被忽视的量化税": the quantization passes are pure memory traffic), so
 * reading it once moves 4.06 instead of 6.06 bytes per element.
 *   q, s    exactly the outputs of mx_quantize_rows(x, M, N, ldx, q, s)
 *           (codes uint8 [M][N], packed scales R = M, contraction N)
 *   qT, sT, padded_offsets  exactly the outputs of
 *           mx_quantize_cols(x, M, N, ldx, group_offsets, G, qT, sT, Mcap,
 *           padded_offsets)
 * provided the group offsets follow the convention above (first 0, last M):
 * the row-wise result covers the rows that lie in a group.  Requires
 * N % 32 == 0 (MX_ERR_SHAPE otherwise) and the alignment and capacity rules
 * of both calls; all buffers are caller-owned device memory.
 */
mx_status mx_quantize_dual(const uint16_t* x, int64_t M, int64_t N, int64_t ldx,
                           const int32_t* group_offsets, int32_t G, uint8_t* q, uint8_t* s,
                           uint8_t* qT, uint8_t* sT, int64_t Mcap, int32_t* padded_offsets,
                           void* stream);

/*
 * Grouped GEMM (M-grouped; forward and dgrad): rows [o_g, o_{g+1}) of X use
 * expert g's weights (aigc.bar "为MoE量身定制优化"; lpnh.cn 2479732 section 1):
 *   out[m][n] = sum_k deq(Xq[m][k]) * deq(Wq[g][n][k]),   fp32 accumulation,
 * scales applied by the matrix instruction per 32-wide K block, result
 * rounded to bf16 (nearest even).  Every output row in [0, M) that belongs
 * to a group is written exactly once.
 *   Xq  uint8 [M][K], Xs packed scales (R = M, contraction K)
 *   Wq  uint8 [G][N][K], Ws packed scales of the [G*N][K] matrix
 *   out bf16 [M][N]
 * Requires K % 256 == 0 and K > 0 (MX_ERR_UNSUPPORTED otherwise; an empty
 * contraction is not supported), 1 <= G <= 4096, 16-byte aligned pointers.
 * G = 1 with offsets {0, M} is a dense GEMM.
 */
mx_status mx_grouped_gemm(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq,
                          const uint8_t* Ws, const int32_t* group_offsets, int32_t G, int64_t M,
                          int64_t N, int64_t K, uint16_t* out, void* stream);

/*
 * Gate+up grouped GEMM with a quantizing SwiGLU epilogue (the MoE layer's
 * first projection, its activation and the MXFP8 quantization of the
 * activation for the down projection in one pass: kucoin.com MoK page,
 * section 02, MXFP8 fused into the SwiGLU step; aigc.bar "被忽视的量化税" on
 * the cost of separate quantization passes).  With Y = the grouped GEMM of Xq and Wq
 * (fp32 accumulation, as mx_grouped_gemm) over 2I output columns:
 *   h[m][c] = silu(gate[m][c]) * up[m][c],   silu(x) = x / (1 + e^-x),
 * where the rows of each expert's [2I][K] weights alternate 32-row blocks:
 * rows [64 b, 64 b + 32) are the gate rows of hidden units [32 b, 32 b + 32)
 * and rows [64 b + 32, 64 b + 64) their up rows.  h is computed in fp32 and
 * quantized along c like mx_quantize_rows (S = max(expfield(amax) - 8, 0)
 * on the fp32 exponent field; codes E4M3FN of h * 2^(127-S), saturated to
 * +/-448, nearest even):
 *   Xq, Xs  as mx_grouped_gemm (R = M, contraction K)
 *   Wq      uint8 [G][2I][K] in the interleaved row order above, Ws its
 *           packed scales ([G*2I][K])
 *   hq      uint8 [M][I] codes; hs packed scales (R = M, contraction I),
 *           ready as the X operand of the down projection
 *   preact  NULL, or bf16 [M][2I]: also store the gate and up values
 *           themselves (bf16 of the fp32 accumulators, columns in the
 *           interleaved order of Wq's rows), as the backward pass of SwiGLU
 *           needs them; 16-byte aligned
 * Rows of a group are written once; rows outside every group, the scale
 * bytes of the padding rows [M, 32 ceil(M / 32)) and, when I % 256 == 128,
 * those of the padding blocks [I / 32, 8 ceil(I / 256)) of every row are left
 * untouched (no output reads them: as a contraction, I must be a multiple of
 * 256 for the grouped GEMM entry points).  Requires K % 256 == 0, K > 0 and I % 128 == 0
 * (MX_ERR_UNSUPPORTED otherwise), 1 <= G <= 4096, 16-byte aligned pointers.
 */
mx_status mx_grouped_gemm_swiglu(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq,
                                 const uint8_t* Ws, const int32_t* group_offsets, int32_t G,
                                 int64_t M, int64_t I, int64_t K, uint8_t* hq, uint8_t* hs,
                                 uint16_t* preact, void* stream);

/*
 * Data-gradient grouped GEMM (M-grouped, weights read transposed; the
 * backward pass of lpnh.cn 2479732 section 1):
 *   dX[m][n] = sum_k deq(dY[m][k]) * deq(W[g(m)][k][n])
 * with W^T taken straight from mx_quantize_cols of the weights viewed as
 * [G*K][N] with group offsets {0, K, 2K, ..., GK}: that call stores expert
 * g's W^T as the column slice [g K, g K + K) of WT [N][Wcap], which this call
 * reads in place (no re-layout).  Here K is the forward output width (the
 * contraction of dgrad) and N the forward input width.
 *   dYq uint8 [M][K], dYs packed scales (R = M, contraction K)
 *   WTq uint8 [N][Wcap], WTs packed scales (R = N, contraction Wcap)
 *   dX  bf16 [M][N]
 * Requires K % 256 == 0 and K > 0 (so that expert g starts at column g K;
 * MX_ERR_UNSUPPORTED otherwise), Wcap % 256 == 0, Wcap >= G * K,
 * 1 <= G <= 4096.
 */
mx_status mx_grouped_gemm_dgrad(const uint8_t* dYq, const uint8_t* dYs, const uint8_t* WTq,
                                const uint8_t* WTs, const int32_t* group_offsets, int32_t G,
                                int64_t M, int64_t N, int64_t K, int64_t Wcap, uint16_t* dX,
                                void* stream);

/*
 * Weight-gradient grouped GEMM (contraction-grouped): groups partition the
 * contraction axis by the padded offsets P written by mx_quantize_cols
 * (lpnh.cn 2479732 section 1, the backward pass):
 *   dW[g][n][k] = sum_{t in [P[g], P[g+1])} deq(A[n][t]) * deq(B[k][t])
 *   A   uint8 [N][Mcap] (dY^T, column-wise quantized), As packed (R = N, Mcap)
 *   B   uint8 [K][Mcap] (X^T, column-wise quantized),  Bs packed (R = K, Mcap)
 *   dW  bf16 [G][N][K]; an empty group gets an all-zero dW[g]
 * Requires Mcap % 256 == 0, 1 <= G <= 4096.  P entries are rounded down to
 * multiples of 256 and clamped to [0, Mcap] on the device.
 */
mx_status mx_grouped_gemm_wgrad(const uint8_t* A, const uint8_t* As, const uint8_t* B,
                                const uint8_t* Bs, const int32_t* padded_offsets, int32_t G,
                                int64_t N, int64_t K, int64_t Mcap, uint16_t* dW, void* stream);

/*
 * Backward pass of SwiGLU, the activation between the two projections of
 * the MoE layer (kucoin.com MoK page, section 02, on the MXFP8 data path
 * through the SwiGLU step), elementwise over M rows and I hidden units:
 *   h  = silu(g) u,  silu(g) = g sigma(g),  sigma(g) = 1 / (1 + e^-g)
 *   dg = dh u sigma(g) (1 + g (1 - sigma(g))),   du = dh silu(g)
 * computed in fp32, each result rounded to bf16 (nearest even).
 *   preact  bf16 [M][2I] gate and up values in the interleaved column order
 *           of mx_grouped_gemm_swiglu (its preact output): columns
 *           [64 b, 64 b + 32) gate of hidden units [32 b, 32 b + 32),
 *           [64 b + 32, 64 b + 64) their up values
 *   dh      bf16 [M][I] gradient of the activation
 *   dpre    bf16 [M][2I] out: dg and du in the same interleaved order (the
 *           gradient of the gate+up projection's output)
 *   h       NULL, or bf16 [M][I] out: the activation itself (for the weight
 *           gradient of the down projection)
 * Requires I % 32 == 0 (MX_ERR_SHAPE), 16-byte aligned pointers.
 */
mx_status mx_swiglu_backward(const uint16_t* preact, const uint16_t* dh, int64_t M, int64_t I,
                             uint16_t* dpre, uint16_t* h, void* stream);

/*
 * SwiGLU backward fused with the quantizations that the rest of the backward
 * pass reads (kucoin.com MoK page, section 02, MXFP8 on the data path through
 * the SwiGLU step; lpnh.cn 2479732 section 1, the backward pass quantizes
 * along both axes).  Equal, byte for byte, to mx_swiglu_backward(preact, dh)
 * giving dpre and h, followed by mx_quantize_dual(dpre, group_offsets) and
 * mx_quantize_cols(h, group_offsets), but neither dpre nor h is written:
 *   preact, dh   as mx_swiglu_backward (bf16 [M][2I] interleaved gate/up,
 *                bf16 [M][I])
 *   q, s         row-wise MXFP8 of d(gate, up): uint8 [M][2I] + packed scales
 *                (R = M, contraction 2I)
 *   qT, sT       column-wise MXFP8 of d(gate, up): uint8 [2I][Mcap] + packed
 *                scales (R = 2I, contraction Mcap)
 *   hT, hTs      column-wise MXFP8 of h: uint8 [I][Mcap] + packed scales
 *                (R = I, contraction Mcap)
 *   padded_offsets  as mx_quantize_cols (one array serves both column-wise
 *                results)
 * Group offsets, capacity and padding as mx_quantize_dual.  Requires
 * I % 128 == 0 (MX_ERR_UNSUPPORTED), Mcap as mx_quantize_cols
 * (MX_ERR_CAPACITY), 16-byte aligned pointers, 1 <= G <= 4096.
 */
mx_status mx_swiglu_backward_quant(const uint16_t* preact, const uint16_t* dh, int64_t M, int64_t I,
                                   const int32_t* group_offsets, int32_t G, uint8_t* q, uint8_t* s, uint8_t* qT,
                                   uint8_t* sT, uint8_t* hT, uint8_t* hTs, int64_t Mcap, int32_t* padded_offsets,
                                   void* stream);

/*
 * The one-GPU share of expert-parallel dispatch and combine (kucoin.com MoK
 * page, section 02: the expert side pulls each routed token by its source
 * position and lays the rows out in local expert order; each expert output
 * goes back to its token; MXFP8 is applied on the dispatch path).  A routed
 * entry j = t k + c is choice c of token t; experts[j] is its expert.
 *
 * mx_route_plan: a stable counting sort of the entries by expert.
 *   experts      int32 [T][k], device; entries outside [0, G) are dropped
 *   weights      NULL, or float [T][k] routing weights (device)
 *   offsets      int32 [G+1] out: exclusive prefix of the per-expert counts
 *                (offsets[G] = number of routed entries), the group offsets
 *                of the expert-ordered rows
 *   src          int32 [T k] out: src[i] = token of the entry placed in slot
 *                i, for i < offsets[G] (slots grouped by expert, in entry
 *                order inside an expert); later entries untouched
 *   slot_of      int32 [T k] out: the slot of entry j, or -1 when dropped
 *   slot_weight  NULL, or float [T k] out: weights[j] at slot_of[j] (needs
 *                weights; MX_ERR_NULL otherwise)
 * Requires T >= 0, k >= 1, 1 <= G <= 4096 (MX_ERR_SHAPE), T k < 2^31
 * (MX_ERR_UNSUPPORTED), 4-byte aligned pointers.  Three launches (count,
 * scan, place); the first and the last read the expert list once per expert
 * (O(G T k) reads, from L2).
 */
mx_status mx_route_plan(const int32_t* experts, const float* weights, int64_t T, int32_t k, int32_t G,
                        int32_t* offsets, int32_t* src, int32_t* slot_of, float* slot_weight, void* stream);

/*
 * mx_gather_quantize: mx_quantize_dual of the gathered matrix R [M][N] whose
 * row r is row src[r] of x (T rows, row stride ldx): the dispatch pull with
 * its quantization (x = token rows, src from mx_route_plan); with a row
 * scale, R[r][c] = bf16(fp32(row_scale[r] * x[src[r]][c])) (the product in
 * binary32, then rounded to bf16, each to nearest even), the backward of a
 * weighted combine (x = output gradient of the tokens, row_scale =
 * slot_weight).  Rows whose src lies outside [0, T) quantize as zeros.
 *   src        int32 [M], device (may be NULL when M == 0)
 *   row_scale  NULL, or float [M], device
 * Everything else, outputs included, as mx_quantize_dual with M rows
 * (group_offsets over [0, M], Mcap >= mx_cols_capacity(M, G)); x may be NULL
 * when T == 0.  Byte for byte equal to mx_quantize_dual of R.
 */
mx_status mx_gather_quantize(const uint16_t* x, int64_t T, int64_t N, int64_t ldx, const int32_t* src,
                             const float* row_scale, int64_t M, const int32_t* group_offsets, int32_t G, uint8_t* q,
                             uint8_t* s, uint8_t* qT, uint8_t* sT, int64_t Mcap, int32_t* padded_offsets,
                             void* stream);

/*
 * mx_combine: out[t][c] = bf16( sum_{i<k} w[t][i] y[slot_of[t][i]][c] ),
 * the routing-weighted sum of a token's expert outputs (weights == NULL: the
 * plain sum, the backward of the gather).  The sum runs in fp32 in choice
 * order (fused multiply-add, one rounding per step) and is rounded to bf16
 * (nearest even) once; entries whose slot lies outside [0, M) are skipped
 * (a token with none gets zeros).
 *   y        bf16 [M][ldy] expert-ordered rows (device; may be NULL when M == 0)
 *   slot_of  int32 [T][k] (mx_route_plan), weights NULL or float [T][k]
 *   out      bf16 [T][N], written in full
 * Requires N % 8 == 0 (MX_ERR_UNSUPPORTED), ldy >= N, k >= 1 (MX_ERR_SHAPE),
 * y, out 16-byte aligned, ldy % 8 == 0, slot_of and weights 4-byte aligned
 * (MX_ERR_ALIGN); T < 2^24, N / 2048 < 65536 (MX_ERR_UNSUPPORTED).
 */
mx_status mx_combine(const uint16_t* y, int64_t M, int64_t N, int64_t ldy, const int32_t* slot_of,
                     const float* weights, int64_t T, int32_t k, uint16_t* out, void* stream);

/*
 * Device-side check of a group_offsets array, for callers that want to
 * verify it (the kernels clamp malformed offsets instead of reading out of
 * bounds): valid means 0 <= o[0] <= o[1] <= ... <= o[G] <= M (rows outside
 * [o[0], o[G]) belong to no group).  Writes result[0] (int32, device) = 0 if
 * valid, else 1 + the first index that breaks the rule; asynchronous like
 * every call.  1 <= G <= 4096, M >= 0 (MX_ERR_SHAPE).
 */
mx_status mx_validate_offsets(const int32_t* group_offsets, int32_t G, int64_t M, int32_t* result,
                              void* stream);

/*
 * HBM calibration stream (measurement only; not a step of the method):
 * reads 2 * dst_bytes from src and writes dst_bytes to dst, the 2:1
 * read:write ratio of bf16 -> fp8 quantization and its access pattern,
 * with no arithmetic beyond an XOR: 8-byte granule i of dst = 32-bit words
 * 0 ^ 1 and 2 ^ 3 of 16-byte granule i of src.
 * Its rate is the practical streaming ceiling that the quantize kernels are
 * reported against (next to the 8 TB/s specification; the quantize-bandwidth
 * benchmark of lpnh.cn 2479732 section 4 counts bytes the same way).
 * Requires dst_bytes % 16 == 0 (MX_ERR_SHAPE), 16-byte aligned pointers;
 * src holds 2 * dst_bytes bytes.  MX_ERR_UNSUPPORTED from dst_bytes / 16 >=
 * 2^32 - 256 on (one lane per 16 bytes written: the grid limit).
 */
mx_status mx_stream21(const void* src, void* dst, int64_t dst_bytes, void* stream);

/*
 * Matrix-instruction diagnostic (not a step of the method): T independent
 * v_mfma_scale_f32_32x32x64_f8f6f4 operations, one per wave, on
 * caller-given operands, so that tests can pin how the instruction rounds the
 * block-scaled products and sums that every grouped GEMM entry point is built
 * from (the scaled product of aigc.bar "拥抱原生硬件指令": block scales applied
 * by the matrix instruction itself).  For t < T and m, n < 32:
 *   D[t][m][n] = C[t][m][n] + sum_{k<64} e4m3(A[t][m][k]) e4m3(B[t][n][k])
 *                             2^(SA[t][m][k/32] - 127) 2^(SB[t][n][k/32] - 127)
 * as the instruction computes it.  A, B: uint8 E4M3 codes [T][32][64]; SA,
 * SB: uint8 scale bytes [T][32][2]; C, D: float32 [T][32][32], row-major;
 * all device memory.  0 <= T <= 65536 (MX_ERR_SHAPE); A, B, C, D 16-byte
 * aligned (MX_ERR_ALIGN).
 */
mx_status mx_probe_mfma_scale(const uint8_t* A, const uint8_t* B, const uint8_t* SA, const uint8_t* SB,
                              const float* C, float* D, int32_t T, void* stream);

/*
 * Debug build (libmxmoe_debug.so, compiled with MXMOE_DEBUG): the kernels
 * that take group offsets check their device-side contract and record
 * violations; this call synchronizes `stream`, then writes to *flags (a HOST
 * pointer) the OR of the violations recorded since the last call, and clears
 * them.  Bits: 1 = group offsets not 0 <= o[0] <= ... <= o[G] <= M (the
 * rule of mx_validate_offsets); 2 = padded offsets not multiples of 256, not
 * increasing by each group's padded size, or past the capacity; 4 = a work
 * tile with no rows of its group.  The checks only record: the kernels clamp
 * malformed offsets either way.  The release library returns
 * MX_ERR_UNSUPPORTED with *flags = 0 (no checks compiled in).  Unlike every
 * other entry point this one synchronizes.  MX_ERR_NULL for flags == NULL.
 */
mx_status mx_debug_flags(uint32_t* flags, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBMXMOE_H */
