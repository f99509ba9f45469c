/*
 * mxref.c -- CPU oracle for MXFP8 (1x32 blocks, E4M3FN elements, E8M0
 * scales) and the block-scaled grouped GEMM.  TEST INFRASTRUCTURE ONLY: the
 * product path never links or calls this file.
 *
 * Written from the definitions in the public write-ups on Cursor's
 * Blackwell MoE kernels (aigc.bar, "被忽视的量化税" and "秘密武器";
 * lpnh.cn 2479732, section 1).  The pages say: cut the tensor into blocks of
 * 32, compute one scale per block, divide the block by the scale, cast to
 * FP8 E4M3.  They fix nothing else.  Readings taken here:
 *   - scale byte S (E8M0, value 2^(S-127)) = clamp(floor(log2 amax) - 8,
 *     -127, 127) + 127, amax = 0 counting as floor(log2 0) = -inf (S = 0);
 *     8 is the exponent of the largest power of two in E4M3;
 *   - elements: y = x * 2^(127-S) (exact), |y| saturated to 448, then
 *     round-to-nearest-even on the OCP E4M3FN grid (bias 7, subnormal
 *     quantum 2^-9, no infinities), sign kept also for zero;
 *   - bf16 subnormals are exact inputs (never flushed);
 *   - non-finite inputs are outside the contract.
 * Arithmetic is double precision and every step is exact: ldexp/frexp scale
 * by powers of two, nearbyint rounds to an integer with ties to even (the
 * default FE_TONEAREST mode, asserted on every call that rounds).
 */
#include "mxref.h"
#include <fenv.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

static void require_rne(void) {
    if (fegetround() != FE_TONEAREST) abort();
}

/* bf16 = the upper 16 bits of an IEEE binary32: sign, 8 exponent bits
 * (bias 127), 7 fraction bits.  Decoded field by field, not by type punning,
 * so that no float hardware (and no flush-to-zero) is involved. */
double mxref_bf16_value(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int ef = (bits >> 7) & 0xFF;
    int fr = bits & 0x7F;
    double v;
    if (ef == 0) {
        v = ldexp((double)fr, -126 - 7);              /* subnormal: 0.f * 2^-126 */
    } else if (ef == 0xFF) {
        v = fr ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + fr), ef - 127 - 7);  /* 1.f * 2^(e-127) */
    }
    return sign ? -v : v;
}

/* OCP E4M3FN: sign, 4 exponent bits (bias 7), 3 fraction bits; exponent
 * field 0 is subnormal (0.f * 2^-6); S.1111.111 is NaN; no infinities. */
double mxref_e4m3_value(uint8_t code) {
    int sign = (code >> 7) & 1;
    int ef = (code >> 3) & 0xF;
    int fr = code & 7;
    double v;
    if (ef == 15 && fr == 7) return NAN;
    if (ef == 0) v = ldexp((double)fr, -6 - 3);
    else v = ldexp((double)(8 + fr), ef - 7 - 3);
    return sign ? -v : v;
}

uint8_t mxref_e4m3_encode(double y) {
    require_rne();
    int neg = signbit(y) ? 1 : 0;
    double a = fabs(y);
    int code;
    if (a > 448.0) a = 448.0;                /* saturate; 448 is on the grid */
    if (a < ldexp(1.0, -6)) {
        /* subnormal range (and zero): multiples of 2^-9 */
        code = (int)nearbyint(ldexp(a, 9));  /* 0..8; 8 is the smallest normal */
    } else {
        int e;
        (void)frexp(a, &e);                  /* a = f * 2^e, f in [0.5, 1) */
        int E = e - 1;                       /* floor(log2 a), -6..8 */
        int n = (int)nearbyint(ldexp(a, 3 - E));  /* 8..16; 16 carries into E+1 */
        code = ((E + 7) << 3) + (n - 8);
    }
    return (uint8_t)(code | (neg << 7));
}

/* E8M0 scale byte of a block whose largest magnitude is amax. */
static uint8_t scale_of_amax(double amax) {
    if (amax == 0.0) return 0;               /* floor(log2 0) = -inf, clamped to -127 */
    int e;
    (void)frexp(amax, &e);
    int shared = (e - 1) - 8;                /* floor(log2 amax) - emax(E4M3) */
    if (shared < -127) shared = -127;
    if (shared > 127) shared = 127;
    return (uint8_t)(shared + 127);
}

uint8_t mxref_block_scale(const uint16_t* x, int64_t n, int64_t stride) {
    double amax = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double a = fabs(mxref_bf16_value(x[i * stride]));
        if (a > amax) amax = a;
    }
    return scale_of_amax(amax);
}

void mxref_quantize_with_scale(const uint16_t* x, int64_t n, uint8_t S, uint8_t* q) {
    for (int64_t i = 0; i < n; ++i) {
        double y = ldexp(mxref_bf16_value(x[i]), 127 - (int)S);  /* x / 2^(S-127) */
        q[i] = mxref_e4m3_encode(y);
    }
}

double mxref_dequant(uint8_t q, uint8_t S) {
    return ldexp(mxref_e4m3_value(q), (int)S - 127);
}

void mxref_quantize_rows(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, uint8_t* s) {
    int64_t nb = K / 32;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t* blk = x + m * K + b * 32;
            uint8_t S = mxref_block_scale(blk, 32, 1);
            s[m * nb + b] = S;
            mxref_quantize_with_scale(blk, 32, S, q + m * K + b * 32);
        }
    }
}

int mxref_quantize_cols(const uint16_t* x, int64_t M, int64_t N, const int32_t* off, int32_t G,
                        int64_t Mcap, uint8_t* qT, uint8_t* sT, int32_t* padded) {
    int32_t one_group[2];
    if (off == NULL) {
        one_group[0] = 0;
        one_group[1] = (int32_t)M;
        off = one_group;
        G = 1;
    }
    int64_t* P = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G + 1));
    P[0] = 0;
    for (int32_t g = 0; g < G; ++g) {
        int64_t mg = (int64_t)off[g + 1] - off[g];
        P[g + 1] = P[g] + 256 * ((mg + 255) / 256);
    }
    if (P[G] > Mcap) {
        free(P);
        return -1;
    }
    memset(qT, 0, (size_t)(N * Mcap));
    memset(sT, 0, (size_t)(N * (Mcap / 32)));
    uint16_t col[32];
    for (int32_t g = 0; g < G; ++g) {
        int64_t r0 = off[g], r1 = off[g + 1];
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t j = 0; r0 + 32 * j < r1; ++j) {
                int64_t first = r0 + 32 * j;
                int64_t cnt = r1 - first < 32 ? r1 - first : 32;
                for (int64_t i = 0; i < cnt; ++i) col[i] = x[(first + i) * N + n];
                /* the missing tail of the last block is zero padding: it adds
                   nothing to amax and its codes stay 0x00 (set above) */
                uint8_t S = mxref_block_scale(col, cnt, 1);
                int64_t dst = P[g] + 32 * j;
                sT[n * (Mcap / 32) + dst / 32] = S;
                mxref_quantize_with_scale(col, cnt, S, qT + n * Mcap + dst);
            }
        }
    }
    if (padded)
        for (int32_t g = 0; g <= G; ++g) padded[g] = (int32_t)P[g];
    free(P);
    return 0;
}

/*
 * Packed scale order.  The gfx950 scaled matrix instruction
 * v_mfma_scale_f32_32x32x64_f8f6f4 takes, per lane l (0..63), one 32-bit
 * scale register and a byte selector: lane l scales row (l mod 32) of its
 * 32-row operand for 32-wide K block (l div 32) of the 64-wide K step.  Four
 * consecutive K steps (256 elements of K = 8 blocks) therefore share one
 * register per lane, byte j serving step j.  The packed array is cut into
 * units of 32 rows x 8 blocks = 256 bytes, each laid out as the 64 lane
 * registers in lane order:
 *     unit(r, b)  = (r div 32) * (KB * 32) + (b div 8) * 256
 *     lane(r, b)  = 32 * (b mod 2) + (r mod 32)
 *     byte(r, b)  = (b mod 8) div 2
 *     offset      = unit + 4 * lane + byte
 * with KB = 8 * ceil(K / 256) bytes per row and rows padded to a multiple
 * of 32.  Pad bytes are zero.
 */
static int64_t packed_offset(int64_t r, int64_t b, int64_t KB) {
    int64_t unit = (r / 32) * (KB * 32) + (b / 8) * 256;
    int64_t lane = 32 * (b % 2) + (r % 32);
    int64_t byte = (b % 8) / 2;
    return unit + 4 * lane + byte;
}

int64_t mxref_packed_scale_bytes(int64_t R, int64_t K) {
    int64_t KB = 8 * ((K + 255) / 256);
    return ((R + 31) / 32) * 32 * KB;
}

void mxref_pack_scales(const uint8_t* s, int64_t R, int64_t K, uint8_t* packed) {
    int64_t KB = 8 * ((K + 255) / 256);
    int64_t nb = K / 32;
    memset(packed, 0, (size_t)mxref_packed_scale_bytes(R, K));
    for (int64_t r = 0; r < R; ++r)
        for (int64_t b = 0; b < nb; ++b) packed[packed_offset(r, b, KB)] = s[r * nb + b];
}

void mxref_unpack_scales(const uint8_t* packed, int64_t R, int64_t K, uint8_t* s) {
    int64_t KB = 8 * ((K + 255) / 256);
    int64_t nb = K / 32;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t b = 0; b < nb; ++b) s[r * nb + b] = packed[packed_offset(r, b, KB)];
}

/* One output element of the grouped GEMM: a plain fp64 dot product of the
 * dequantized row of X and the dequantized row n of expert g's weights.
 * Each product is exact in double (two 4-bit significands); the sum runs in
 * order of k. */
static double gemm_point(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                         int32_t g, int64_t m, int64_t n, int64_t N, int64_t K) {
    int64_t nb = K / 32;
    const uint8_t* xr = Xq + m * K;
    const uint8_t* xs = Xs + m * nb;
    const uint8_t* wr = Wq + ((int64_t)g * N + n) * K;
    const uint8_t* ws = Ws + ((int64_t)g * N + n) * nb;
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += mxref_dequant(xr[k], xs[k / 32]) * mxref_dequant(wr[k], ws[k / 32]);
    return acc;
}

void mxref_grouped_gemm(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                        const int32_t* off, int32_t G, int64_t M, int64_t N, int64_t K, double* out) {
    memset(out, 0, sizeof(double) * (size_t)(M * N));
    for (int32_t g = 0; g < G; ++g)
        for (int64_t m = off[g]; m < off[g + 1]; ++m)
            for (int64_t n = 0; n < N; ++n) out[m * N + n] = gemm_point(Xq, Xs, Wq, Ws, g, m, n, N, K);
}

static int32_t group_of_row(const int32_t* off, int32_t G, int64_t m) {
    for (int32_t g = 0; g < G; ++g)
        if (m >= off[g] && m < off[g + 1]) return g;
    return -1;
}

void mxref_grouped_gemm_points(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq,
                               const uint8_t* Ws, const int32_t* off, int32_t G, int64_t M,
                               int64_t N, int64_t K, const int64_t* rows, const int64_t* cols,
                               int64_t npts, double* out) {
    (void)M;
    for (int64_t i = 0; i < npts; ++i) {
        int32_t g = group_of_row(off, G, rows[i]);
        out[i] = g < 0 ? 0.0 : gemm_point(Xq, Xs, Wq, Ws, g, rows[i], cols[i], N, K);
    }
}

static double wgrad_point(const uint8_t* Aq, const uint8_t* As, const uint8_t* Bq, const uint8_t* Bs,
                          const int32_t* P, int32_t g, int64_t n, int64_t k, int64_t Mcap) {
    int64_t nb = Mcap / 32;
    double acc = 0.0;
    for (int64_t t = P[g]; t < P[g + 1]; ++t)
        acc += mxref_dequant(Aq[n * Mcap + t], As[n * nb + t / 32]) *
               mxref_dequant(Bq[k * Mcap + t], Bs[k * nb + t / 32]);
    return acc;
}

void mxref_wgrad(const uint8_t* Aq, const uint8_t* As, const uint8_t* Bq, const uint8_t* Bs,
                 const int32_t* P, int32_t G, int64_t N, int64_t K, int64_t Mcap, double* dW) {
    for (int32_t g = 0; g < G; ++g)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t k = 0; k < K; ++k)
                dW[((int64_t)g * N + n) * K + k] = wgrad_point(Aq, As, Bq, Bs, P, g, n, k, Mcap);
}

void mxref_wgrad_points(const uint8_t* Aq, const uint8_t* As, const uint8_t* Bq, const uint8_t* Bs,
                        const int32_t* P, int32_t G, int64_t N, int64_t K, int64_t Mcap,
                        const int64_t* gs, const int64_t* ns, const int64_t* ks, int64_t npts,
                        double* out) {
    (void)G;
    (void)N;
    (void)K;
    for (int64_t i = 0; i < npts; ++i) out[i] = wgrad_point(Aq, As, Bq, Bs, P, (int32_t)gs[i], ns[i], ks[i], Mcap);
}

/* ---- SwiGLU of the gate and up projections, quantized to MXFP8 ----
 * The pages fuse the MXFP8 quantization of the activation into the SwiGLU
 * step of the MoE layer (kucoin.com MoK page, section 02; aigc.bar "被忽视的量化税" on
 * the cost of a separate quantization pass).  They give no formula.  Readings
 * taken here:
 *   - SwiGLU(gate, up) = silu(gate) * up with silu(x) = x * sigmoid(x) =
 *     x / (1 + e^-x), elementwise (the usual gated-MLP activation);
 *   - the result h is a real number (double here), quantized directly: one
 *     scale per 32 consecutive hidden units of a row by the rule above,
 *     applied to |h| itself, then y = h * 2^(127-S) encoded as E4M3FN with
 *     saturation and nearest-even.  There is no intermediate bf16 rounding
 *     of h.
 */
double mxref_silu(double x) {
    return x / (1.0 + exp(-x));              /* exp(-x) = inf for x < -709: -0 */
}

uint8_t mxref_block_scale_f64(const double* x, int64_t n) {
    double amax = 0.0;
    for (int64_t i = 0; i < n; ++i)
        if (fabs(x[i]) > amax) amax = fabs(x[i]);
    return scale_of_amax(amax);
}

void mxref_quantize_f64_with_scale(const double* x, int64_t n, uint8_t S, uint8_t* q) {
    for (int64_t i = 0; i < n; ++i) q[i] = mxref_e4m3_encode(ldexp(x[i], 127 - (int)S));
}

void mxref_quantize_rows_f64(const double* x, int64_t M, int64_t K, uint8_t* q, uint8_t* s) {
    int64_t nb = K / 32;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < nb; ++b) {
            const double* blk = x + m * K + b * 32;
            uint8_t S = mxref_block_scale_f64(blk, 32);
            s[m * nb + b] = S;
            mxref_quantize_f64_with_scale(blk, 32, S, q + m * K + b * 32);
        }
}

void mxref_swiglu_quantize(const double* gate, const double* up, int64_t M, int64_t I, double* h, uint8_t* q,
                           uint8_t* s) {
    for (int64_t i = 0; i < M * I; ++i) h[i] = mxref_silu(gate[i]) * up[i];
    mxref_quantize_rows_f64(h, M, I, q, s);
}

/* ---- Backward pass of SwiGLU ----
 * Readings (the pages give no formula; this is the derivative of the
 * forward reading above, term by term):
 *   sigma(g) = 1 / (1 + e^-g), silu'(g) = sigma(g) (1 + g (1 - sigma(g)));
 *   d gate = dh * up * silu'(gate), d up = dh * silu(gate), and the
 *   activation h = silu(gate) * up, all in double;
 *   results stored as bf16: round to nearest, ties to even, directly from
 *   the double value (one rounding), overflow to infinity.
 */
double mxref_dsilu(double x) {
    double sig = 1.0 / (1.0 + exp(-x));
    return sig * (1.0 + x * (1.0 - sig));
}

uint16_t mxref_bf16_round(double x) {
    require_rne();
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);
    int E = e - 1;                                    /* floor(log2 a) */
    if (E < -126) {
        /* subnormal range: multiples of 2^-133 (128 of them reach 2^-126) */
        int n = (int)nearbyint(ldexp(a, 133));
        return (uint16_t)(sign | n);                  /* n = 128 is the smallest normal */
    }
    double n = nearbyint(ldexp(a, 7 - E));            /* 128..256 */
    if (n == 256.0) {
        n = 128.0;
        E += 1;
    }
    if (E > 127) return (uint16_t)(sign | 0x7F80);    /* infinity */
    return (uint16_t)(sign | ((E + 127) << 7) | ((int)n - 128));
}

void mxref_bf16_round_n(const double* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = mxref_bf16_round(x[i]);
}

void mxref_swiglu_backward(const double* gate, const double* up, const double* dh, int64_t n, double* dgate,
                           double* dup, double* h) {
    for (int64_t i = 0; i < n; ++i) {
        dgate[i] = dh[i] * up[i] * mxref_dsilu(gate[i]);
        dup[i] = dh[i] * mxref_silu(gate[i]);
        h[i] = mxref_silu(gate[i]) * up[i];
    }
}

/* ---- the one-GPU share of dispatch and combine ----
 * Readings (the MoK page, section 02, describes pull dispatch and push
 * combine without formulas):
 *   - a routed entry is a (token, choice) pair with an expert index; the
 *     expert side lays its entries out grouped by expert and, inside an
 *     expert, in entry order (token-major): a stable sort by expert;
 *   - an entry whose expert index is outside [0, G) is not routed;
 *   - combine is the routing-weighted sum of a token's expert outputs, the
 *     usual top-k mixture; without weights the plain sum (the backward of the
 *     gather);
 *   - the scaled gather (the backward of the weighted combine: the output
 *     gradient of a token times the entry's weight) is formed in binary32
 *     and stored as bf16 before it is quantized. */
void mxref_route_plan(const int32_t* experts, int64_t n, int32_t k, int32_t G, int32_t* offsets, int32_t* src,
                      int32_t* slot_of) {
    int64_t* cursor = calloc((size_t)G + 1, sizeof(int64_t));
    for (int64_t j = 0; j < n; ++j)
        if (experts[j] >= 0 && experts[j] < G) cursor[experts[j] + 1] += 1;
    for (int32_t g = 0; g < G; ++g) cursor[g + 1] += cursor[g];
    for (int32_t g = 0; g <= G; ++g) offsets[g] = (int32_t)cursor[g];
    for (int64_t j = 0; j < n; ++j) {
        const int32_t e = experts[j];
        if (e < 0 || e >= G) {
            slot_of[j] = -1;
            continue;
        }
        const int64_t slot = cursor[e]++;
        src[slot] = (int32_t)(j / k);
        slot_of[j] = (int32_t)slot;
    }
    free(cursor);
}

double mxref_f32_round(double x) {
    require_rne();
    double a = fabs(x);
    if (a == 0.0) return x;
    int e;
    (void)frexp(a, &e);
    int E = e - 1;                                    /* floor(log2 a) */
    if (E < -126) return copysign(ldexp(nearbyint(ldexp(a, 149)), -149), x);
    double n = ldexp(nearbyint(ldexp(a, 23 - E)), E - 23);
    if (n >= ldexp(1.0, 128)) return copysign(INFINITY, x);
    return copysign(n, x);
}

void mxref_gather_rows(const uint16_t* x, int64_t T, int64_t N, const int32_t* src, const float* scale, int64_t M,
                       uint16_t* out) {
    for (int64_t r = 0; r < M; ++r) {
        uint16_t* o = out + r * N;
        if (src[r] < 0 || src[r] >= T) {
            memset(o, 0, (size_t)N * sizeof(uint16_t));
            continue;
        }
        const uint16_t* in = x + (int64_t)src[r] * N;
        for (int64_t c = 0; c < N; ++c) {
            if (scale == NULL) {
                o[c] = in[c];
            } else {
                /* 24 x 8 significant bits: the double product is exact */
                const double p = (double)scale[r] * mxref_bf16_value(in[c]);
                o[c] = mxref_bf16_round(mxref_f32_round(p));
            }
        }
    }
}

void mxref_combine(const uint16_t* y, int64_t M, int64_t N, const int32_t* slot_of, const float* w, int64_t T,
                   int32_t k, double* out) {
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < N; ++c) {
            double acc = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                const int32_t slot = slot_of[t * k + j];
                if (slot < 0 || slot >= M) continue;
                acc += (w ? (double)w[t * k + j] : 1.0) * mxref_bf16_value(y[(int64_t)slot * N + c]);
            }
            out[t * N + c] = acc;
        }
}
