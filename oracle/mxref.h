/*
 * mxref -- CPU oracle for MXFP8 block quantization and the block-scaled
 * grouped GEMM it feeds.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never calls it, and the two share
 * no code, headers, tables or constants.
 *
 * Everything here is written straight from the definitions, one step at a
 * time, in double precision (every operation used is exact: ldexp, frexp,
 * nearbyint under round-to-nearest-even, products of short significands).
 *
 * Sources (the public write-ups on the Cursor Blackwell MoE kernels):
 *  - "Blackwell性能陷阱？Cursor揭秘" (aigc.bar), sections "被忽视的量化税" and
 *    "秘密武器": MX block scaling, E4M3 with block size 32, a scale layout
 *    that feeds the matrix instruction with no reshape pass.
 *  - lpnh.cn news 2479732, section 1: cut the tensor into 32-element blocks,
 *    compute one scale per block, divide the block by it, then cast to FP8;
 *    the backward pass needs a transposed quantization.
 * The pages do not fix the scale rule, the FP8 variant, rounding, saturation
 * or layouts; the readings taken here are listed beside each function.
 */
#ifndef MXREF_H
#define MXREF_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* O1: bf16 bit pattern -> exact value (subnormals kept, never flushed). */
double mxref_bf16_value(uint16_t bits);

/* O5 inverse: value of an OCP E4M3FN code (NaN for 0x7F / 0xFF). */
double mxref_e4m3_value(uint8_t code);

/* O4+O5: saturate |y| to 448, round to nearest-even on the E4M3FN grid,
 * keep the sign (also for zero). y must be finite. */
uint8_t mxref_e4m3_encode(double y);

/* O2: E8M0 scale byte of one block of n bf16 values read with the given
 * stride (n <= 32; missing tail elements count as zero).
 * S = clamp(floor(log2 amax) - 8, -127, 127) + 127, amax = 0 -> S = 0. */
uint8_t mxref_block_scale(const uint16_t* x, int64_t n, int64_t stride);

/* O3-O5 for a whole array under one given scale byte S. */
void mxref_quantize_with_scale(const uint16_t* x, int64_t n, uint8_t S, uint8_t* q);

/* O8: exact value of element code q under scale byte S. */
double mxref_dequant(uint8_t q, uint8_t S);

/* Row-wise quantization of bf16 x[M][K] (row-major, K % 32 == 0).
 * q[M][K] codes; s[M][K/32] scale bytes in canonical (row, block) order. */
void mxref_quantize_rows(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, uint8_t* s);

/* Column-wise (transposed) quantization of bf16 x[M][N] (row-major) with
 * row groups [off[g], off[g+1]) (off == NULL: one group of all M rows).
 * Blocks of 32 rows restart at each group start; the tail of a group is
 * zero-padded to a multiple of 256 rows.  Group g is stored at padded
 * offset P[g] = sum_{h<g} 256*ceil(m_h/256).
 * qT[N][Mcap], sT[N][Mcap/32] (canonical), padded[G+1] = P (may be NULL).
 * Positions of qT / sT beyond P[G] are set to 0.  Returns 0, or -1 if Mcap
 * is too small. */
int mxref_quantize_cols(const uint16_t* x, int64_t M, int64_t N, const int32_t* off, int32_t G,
                        int64_t Mcap, uint8_t* qT, uint8_t* sT, int32_t* padded);

/* Pack canonical scales s[R][NB] (NB = K/32 blocks per row) into the tiled
 * order the scaled matrix instruction consumes; see mxref.c for the map.
 * packed must hold mxref_packed_scale_bytes(R, K) bytes; padding is zero. */
int64_t mxref_packed_scale_bytes(int64_t R, int64_t K);
void mxref_pack_scales(const uint8_t* s, int64_t R, int64_t K, uint8_t* packed);
void mxref_unpack_scales(const uint8_t* packed, int64_t R, int64_t K, uint8_t* s);

/* O9: grouped GEMM reference, fp64.  Rows [off[g], off[g+1]) of X use
 * expert g: out[m][n] = sum_k deq(Xq[m][k]) * deq(Wq[g][n][k]).
 * Xs[M][K/32], Ws[G][N][K/32] canonical scales. out is double[M][N]. */
void mxref_grouped_gemm(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                        const int32_t* off, int32_t G, int64_t M, int64_t N, int64_t K, double* out);

/* Same definition evaluated only at the listed (row, col) points. */
void mxref_grouped_gemm_points(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq,
                               const uint8_t* Ws, const int32_t* off, int32_t G, int64_t M,
                               int64_t N, int64_t K, const int64_t* rows, const int64_t* cols,
                               int64_t npts, double* out);

/* O10: weight-gradient reference, fp64.  A = dY^T codes [N][Mcap], B = X^T
 * codes [K][Mcap] (both column-wise quantized, canonical scales
 * [.][Mcap/32]); groups partition the contraction axis by padded offsets
 * P[0..G]: dW[g][n][k] = sum_{t in [P[g], P[g+1])} deq(A[n][t]) deq(B[k][t]).
 * dW is double[G][N][K]. */
void mxref_wgrad(const uint8_t* Aq, const uint8_t* As, const uint8_t* Bq, const uint8_t* Bs,
                 const int32_t* P, int32_t G, int64_t N, int64_t K, int64_t Mcap, double* dW);

/* Same definition evaluated only at the listed (g, n, k) points. */
void mxref_wgrad_points(const uint8_t* Aq, const uint8_t* As, const uint8_t* Bq, const uint8_t* Bs,
                        const int32_t* P, int32_t G, int64_t N, int64_t K, int64_t Mcap,
                        const int64_t* gs, const int64_t* ns, const int64_t* ks, int64_t npts,
                        double* out);

/* SwiGLU + MXFP8 of its result (readings in mxref.c). */
double mxref_silu(double x);
uint8_t mxref_block_scale_f64(const double* x, int64_t n);
void mxref_quantize_f64_with_scale(const double* x, int64_t n, uint8_t S, uint8_t* q);
/* x double [M][K] (K % 32 == 0) -> codes [M][K], canonical scales [M][K/32] */
void mxref_quantize_rows_f64(const double* x, int64_t M, int64_t K, uint8_t* q, uint8_t* s);
/* gate, up double [M][I] -> h = silu(gate) up [M][I], its codes and scales */
void mxref_swiglu_quantize(const double* gate, const double* up, int64_t M, int64_t I, double* h, uint8_t* q,
                           uint8_t* s);

/* SwiGLU backward (readings in mxref.c); all arrays of n doubles. */
double mxref_dsilu(double x);
uint16_t mxref_bf16_round(double x);
void mxref_bf16_round_n(const double* x, int64_t n, uint16_t* out);
void mxref_swiglu_backward(const double* gate, const double* up, const double* dh, int64_t n, double* dgate,
                           double* dup, double* h);

/* The one-GPU share of expert-parallel dispatch and combine (kucoin.com MoK
 * page, section 02: the expert side pulls each routed token by its source
 * position and lays the rows out in local expert order; results go back to
 * their tokens; MXFP8 is applied on the dispatch path).  The pages give no
 * formulas; readings in mxref.c. */

/* Stable counting sort of routed entries by expert.  experts[n] (n = T k,
 * entry j = token j / k, choice j % k); entries outside [0, G) are dropped.
 * offsets[G+1]: exclusive prefix of the per-expert counts; src[slot] = token
 * of the entry placed there (slots ordered by expert, then by entry index);
 * slot_of[j] = its slot, or -1 when dropped. */
void mxref_route_plan(const int32_t* experts, int64_t n, int32_t k, int32_t G, int32_t* offsets, int32_t* src,
                      int32_t* slot_of);

/* Nearest-even binary32 value of x (subnormal quantum 2^-149, overflow to
 * infinity), as a double. */
double mxref_f32_round(double x);

/* Gathered rows: out[r][:] = x[src[r]][:] (bf16 bit patterns), or, with a
 * row scale, bf16(f32(scale[r] * x[src[r]][c])) (the product rounded to
 * binary32, then to bf16, each to nearest even); rows with src[r] outside
 * [0, T) are zero. */
void mxref_gather_rows(const uint16_t* x, int64_t T, int64_t N, const int32_t* src, const float* scale, int64_t M,
                       uint16_t* out);

/* Combine: out[t][c] = sum_j w[t][j] y[slot_of[t][j]][c] over the entries
 * whose slot lies in [0, M) (w == NULL: weight 1), in double. */
void mxref_combine(const uint16_t* y, int64_t M, int64_t N, const int32_t* slot_of, const float* w, int64_t T,
                   int32_t k, double* out);

#ifdef __cplusplus
}
#endif
#endif
