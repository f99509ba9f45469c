// Dual-layout MXFP8 quantization for gfx950: one read of a bf16 matrix, both
// the row-wise result (scales along the row, as quantize_rows_kernel) and the
// column-wise / transposed one (per-group blocks along the column, as
// quantize_cols_kernel), bit-identical to the two separate kernels.
//
// Method (lpnh.cn 2479732 section 1: the backward pass quantizes the same
// gradient along both axes; aigc.bar "被忽视的量化税": the quantization passes
// are pure memory traffic, so reading the input once saves a third of it).
#include "mx_bf16.h"
#include "mx_device.h"
#include "mx_internal.h"
#include "mx_debug.h"

namespace mx {

// ---------------------------------------------------------------------------
// Dual layout: one read of x, the row-wise and the column-wise results.  One
// 256-thread workgroup per padded row tile pt (256 rows of one group, as in
// the column-wise kernel) and 256-column chunk ct, walked as 4 sub-tiles of
// 64 columns:
//  * row-wise: in the load phase, the 4 lanes of a DPP quad hold one
//    32-column block of each of their two rows; quad max, codes exchanged
//    between adjacent lanes so that each lane stores 16 bytes of one row,
//    those of sub-tiles 2p and 2p + 1 together (128 contiguous bytes per
//    row, in two store instructions of 64 bytes per row: ordinary stores, so
//    that L2 joins the halves of each line -- measured 7 % faster than
//    non-temporal stores on [131072, 7168] and 19 % on a 16-group
//    [32768, 7168]), scale bytes collected in LDS in packed dword order (the
//    chunk's 8 blocks of a row are two dwords) and written once per row at
//    the end, 128 contiguous bytes per 32 rows;
//  * column-wise: the rows are paired into the transposed LDS tile; each
//    lane quantizes 16 consecutive rows of a column (a lane pair per 32-row
//    block) with the element map of the column-wise kernel and stores 16
//    code bytes (16-byte stores: 1-4 % faster than 8-byte ones);
//  * the loads of the next sub-tile are issued before the column-wise phase
//    of the current one.
// Every row of a group lies in exactly one row tile; rows in
// [M, 32 ceil(M / 32)) get zero row-wise scale bytes, and blocks past N read
// as zeros, so both packed arrays equal those of the separate kernels.
//
// GATHER: row r of the quantized matrix is row src[r] of x (T rows), the
// pull side of an expert-parallel dispatch (kucoin.com MoK page, section
// 02: MXFP8 applied on the dispatch path); with a row scale, each element is
// first multiplied by rscale[r] in fp32 and rounded to bf16 (nearest even).
// Rows whose source index lies outside [0, T) quantize as zeros.
// ---------------------------------------------------------------------------
template <bool GATHER>
__global__ __launch_bounds__(256) void quantize_dual_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t N,
                                                            int64_t ldx, const int32_t* __restrict__ off,
                                                            const int32_t* __restrict__ P, int32_t G,
                                                            uint8_t* __restrict__ q, uint8_t* __restrict__ s,
                                                            uint8_t* __restrict__ qT, uint8_t* __restrict__ sT,
                                                            int64_t Mcap, const int32_t* __restrict__ src,
                                                            const float* __restrict__ rscale, int64_t T) {
    __shared__ uint4 tile[64 * 32];
    __shared__ uint32_t unit_s[2][64];
    __shared__ uint32_t row_s[256][2];  // per tile row: packed dwords of K halves 0 and 1 of the chunk
    __shared__ int32_t sh_g;
    const int t = threadIdx.x;
    // column chunks vary fastest: the workgroups in flight read whole rows
    // (measured 5 % faster than row tiles fastest)
    const int64_t pt = blockIdx.y;
    const int64_t ct = blockIdx.x;
    const int64_t col0 = pt * 256;

    row_s[t][0] = 0;
    row_s[t][1] = 0;
    if (t == 0) sh_g = -1;
    __syncthreads();
    if (off == nullptr) {
        if (col0 < ((M + 255) / 256) * 256 && t == 0) sh_g = 0;
    } else {
        for (int g = t; g < G; g += 256)
            if (P[g] <= col0 && col0 < P[g + 1]) sh_g = g;
    }
    __syncthreads();
    const int g = sh_g;
    int64_t row_begin = 0, row_end = 0;
    if (g >= 0) {
        if (off == nullptr) {
            row_begin = col0;
            row_end = M;
        } else {
            const int64_t o0 = clamp_off(off, g, M), o1 = clamp_off(off, g + 1, M);
            row_begin = o0 + (col0 - P[g]);
            row_end = o1;
            if (t == 0) {
                const int64_t mg = o1 > o0 ? o1 - o0 : 0;
                debug_flag(P[g] % 256 != 0 || P[g + 1] - P[g] != ((mg + 255) / 256) * 256 || P[g + 1] > Mcap,
                           kDbgPadded);
                debug_flag(row_begin >= row_end, kDbgTile);
            }
        }
    }
    const int c8 = t & 7;  // 16-byte column chunk (8 columns) of a sub-tile
    uint4 da[4], db[4];
    // GATHER: source rows of this lane's row pairs (-1: none) and their scales
    int64_t sra[4], srb[4];
    float fa[4], fb[4];
    if constexpr (GATHER) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pr = i * 32 + (t >> 3);
            const int64_t r0 = row_begin + 2 * pr, r1 = r0 + 1;
            sra[i] = (g >= 0 && r0 < row_end) ? (int64_t)src[r0] : -1;
            srb[i] = (g >= 0 && r1 < row_end) ? (int64_t)src[r1] : -1;
            if (sra[i] >= T) sra[i] = -1;
            if (srb[i] >= T) srb[i] = -1;
            fa[i] = (rscale != nullptr && sra[i] >= 0) ? rscale[r0] : 1.0f;
            fb[i] = (rscale != nullptr && srb[i] >= 0) ? rscale[r1] : 1.0f;
        }
    }
    auto scaled = [&](uint4 v, float f) {
        return make_uint4(pack_bf16(lo_bf16(v.x) * f, hi_bf16(v.x) * f), pack_bf16(lo_bf16(v.y) * f, hi_bf16(v.y) * f),
                          pack_bf16(lo_bf16(v.z) * f, hi_bf16(v.z) * f), pack_bf16(lo_bf16(v.w) * f, hi_bf16(v.w) * f));
    };
    auto load = [&](int st) {
        const int64_t ncol = (ct * 4 + st) * 64 + c8 * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pr = i * 32 + (t >> 3);
            const int64_t r0 = row_begin + 2 * pr, r1 = r0 + 1;
            da[i] = make_uint4(0, 0, 0, 0);
            db[i] = make_uint4(0, 0, 0, 0);
            if (g >= 0 && ncol < N) {
                if constexpr (GATHER) {
                    if (sra[i] >= 0) da[i] = load_stream16(x + sra[i] * ldx + ncol);
                    if (srb[i] >= 0) db[i] = load_stream16(x + srb[i] * ldx + ncol);
                } else {
                    if (r0 < row_end) da[i] = load_stream16(x + r0 * ldx + ncol);
                    if (r1 < row_end) db[i] = load_stream16(x + r1 * ldx + ncol);
                }
            }
        }
        if constexpr (GATHER) {
            if (rscale != nullptr) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    da[i] = scaled(da[i], fa[i]);
                    db[i] = scaled(db[i], fb[i]);
                }
            }
        }
    };
    load(0);
    // row-wise codes of an even sub-tile wait in registers and go out next to
    // the odd sub-tile's, so each row gets 128 contiguous bytes at once
    uint4 pend[4];
    uint8_t* rs = reinterpret_cast<uint8_t*>(row_s);
    uint8_t* us = reinterpret_cast<uint8_t*>(unit_s);
#pragma unroll 1
    for (int st = 0; st < 4; ++st) {
        const int64_t nt = ct * 4 + st;
        const int64_t ncol = nt * 64 + c8 * 8;
        const int b = st * 2 + (c8 >> 2);  // block of the chunk, 0..7
        // ---- row-wise, from the registers
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pr = i * 32 + (t >> 3);
            const int64_t r0 = row_begin + 2 * pr, r1 = r0 + 1;
            const uint32_t Sa = scale_from_maxmag(quad_max_u32(max_mag8(da[i])));
            const uint32_t Sb = scale_from_maxmag(quad_max_u32(max_mag8(db[i])));
            const uint2 ca = quant8(da[i], Sa), cb = quant8(db[i], Sb);
            // adjacent lanes (c8 even / odd) swap halves: the even lane then
            // holds 16 code bytes of row r0 (columns ncol .. ncol + 15), the odd
            // lane those of row r1 (columns ncol - 8 .. ncol + 7)
            const uint2 snd = (c8 & 1) ? ca : cb;
            const uint32_t rx = (uint32_t)__builtin_amdgcn_mov_dpp((int)snd.x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
            const uint32_t ry = (uint32_t)__builtin_amdgcn_mov_dpp((int)snd.y, 0xB1, 0xF, 0xF, false);
            const uint4 o = (c8 & 1) ? make_uint4(rx, ry, cb.x, cb.y) : make_uint4(ca.x, ca.y, rx, ry);
            const int64_t rr = (c8 & 1) ? r1 : r0;
            const int64_t cc = ncol - (c8 & 1) * 8;
            if (st & 1) {
                if (g >= 0 && rr < row_end) {
                    if (cc - 64 < N) store16(q + rr * N + cc - 64, pend[i]);
                    if (cc < N) store16(q + rr * N + cc, o);
                }
            } else {
                pend[i] = o;
            }
            if ((t & 3) == 0) {
                rs[(2 * pr) * 8 + (b & 1) * 4 + (b >> 1)] = (uint8_t)Sa;
                rs[(2 * pr + 1) * 8 + (b & 1) * 4 + (b >> 1)] = (uint8_t)Sb;
            }
        }
        // ---- pair rows into the transposed tile
        uint32_t* tw = reinterpret_cast<uint32_t*>(tile);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pr = i * 32 + (t >> 3);
            const uint32_t aw[4] = {da[i].x, da[i].y, da[i].z, da[i].w};
            const uint32_t bw[4] = {db[i].x, db[i].y, db[i].z, db[i].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t lo = __builtin_amdgcn_perm(bw[k], aw[k], 0x05040100u);
                const uint32_t hi = __builtin_amdgcn_perm(bw[k], aw[k], 0x07060302u);
                const int n0 = c8 * 8 + 2 * k, n1 = n0 + 1;
                tw[n0 * 128 + (((pr >> 2) ^ ((n0 >> 3) & 7)) << 2) + (pr & 3)] = lo;
                tw[n1 * 128 + (((pr >> 2) ^ ((n1 >> 3) & 7)) << 2) + (pr & 3)] = hi;
            }
        }
        __syncthreads();
        if (st < 3) load(st + 1);
        // ---- column-wise from the tile: 16 consecutive rows of one column per
        // task (two 16-byte granules), a 32-row block per lane pair
        const int jj = t & 15;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = i * 16 + (t >> 4);
            const int sw = (n >> 3) & 7;
            const uint4 d0 = tile[n * 32 + ((2 * jj) ^ sw)];
            const uint4 d1 = tile[n * 32 + ((2 * jj + 1) ^ sw)];
            uint32_t m = max_mag8(d0);
            const uint32_t m1 = max_mag8(d1);
            m = m > m1 ? m : m1;
            const uint32_t mo = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false);  // the pair's other lane
            m = m > mo ? m : mo;
            const uint32_t S = scale_from_maxmag(m);
            const uint2 c0 = quant8(d0, S), c1 = quant8(d1, S);
            const int64_t ng = nt * 64 + n;
            if (ng < N) store_stream16(qT + ng * Mcap + col0 + 16 * jj, make_uint4(c0.x, c0.y, c1.x, c1.y));
            if ((t & 1) == 0) us[(n >> 5) * 256 + unit_byte((uint32_t)(n & 31), (uint32_t)(jj >> 1))] = (uint8_t)S;
        }
        __syncthreads();
        if (t < 128) {
            const int u = t >> 6;
            const int64_t rowunit = nt * 2 + u;
            if (rowunit * 32 < N) {
                const int64_t KB = Mcap / 32;
                __builtin_nontemporal_store(unit_s[u][t & 63],
                                            reinterpret_cast<uint32_t*>(sT + rowunit * 32 * KB + pt * 256) + (t & 63));
            }
        }
    }
    __syncthreads();
    // ---- row-wise packed scales: one tile row per thread, two dwords
    const int64_t KBr = 8 * ((N + 255) / 256);
    if (g >= 0 && row_begin + t < row_end) {
        const int64_t r = row_begin + t;
        uint32_t* dst = reinterpret_cast<uint32_t*>(s + (r >> 5) * 32 * KBr + ct * 256) + (r & 31);
        dst[0] = row_s[t][0];
        dst[32] = row_s[t][1];
    }
    // the pad rows [M, 32 ceil(M / 32)) of the packed array get zero scale
    // bytes, written by the first row tile of each column chunk (no group
    // tile's window needs to reach them)
    const int64_t Mpad = ((M + 31) / 32) * 32;
    if (pt == 0 && t < Mpad - M) {
        const int64_t r = M + t;
        uint32_t* dst = reinterpret_cast<uint32_t*>(s + (r >> 5) * 32 * KBr + ct * 256) + (r & 31);
        dst[0] = 0u;
        dst[32] = 0u;
    }
}

#ifdef MXMOE_DEBUG
hipError_t debug_take_dual(uint32_t* out) { return debug_take_word(out); }
#endif

static hipError_t launch_dual(const uint16_t* x, int64_t M, int64_t N, int64_t ldx, const int32_t* group_offsets,
                              int32_t G, uint8_t* q, uint8_t* s, uint8_t* qT, uint8_t* sT, int64_t Mcap,
                              int32_t* padded_offsets, const int32_t* src, const float* rscale, int64_t T,
                              hipStream_t stream) {
    if (group_offsets != nullptr) {
        hipError_t e = launch_cols_prefix(group_offsets, G, M, padded_offsets, stream);
        if (e != hipSuccess) return e;
    } else {
        G = 1;
    }
    if (N == 0 || Mcap == 0) return hipSuccess;
    dim3 grid((unsigned)((N + 255) / 256), (unsigned)(Mcap / 256));
    if (src != nullptr)
        hipLaunchKernelGGL(quantize_dual_kernel<true>, grid, dim3(256), 0, stream, x, M, N, ldx, group_offsets,
                           (const int32_t*)padded_offsets, G, q, s, qT, sT, Mcap, src, rscale, T);
    else
        hipLaunchKernelGGL(quantize_dual_kernel<false>, grid, dim3(256), 0, stream, x, M, N, ldx, group_offsets,
                           (const int32_t*)padded_offsets, G, q, s, qT, sT, Mcap, nullptr, nullptr, M);
    return hipGetLastError();
}

hipError_t launch_quantize_dual(const uint16_t* x, int64_t M, int64_t N, int64_t ldx,
                                const int32_t* group_offsets, int32_t G, uint8_t* q, uint8_t* s, uint8_t* qT,
                                uint8_t* sT, int64_t Mcap, int32_t* padded_offsets, hipStream_t stream) {
    return launch_dual(x, M, N, ldx, group_offsets, G, q, s, qT, sT, Mcap, padded_offsets, nullptr, nullptr, M,
                       stream);
}

hipError_t launch_gather_quantize(const uint16_t* x, int64_t T, int64_t N, int64_t ldx, const int32_t* src,
                                  const float* row_scale, int64_t M, const int32_t* group_offsets, int32_t G,
                                  uint8_t* q, uint8_t* s, uint8_t* qT, uint8_t* sT, int64_t Mcap,
                                  int32_t* padded_offsets, hipStream_t stream) {
    return launch_dual(x, M, N, ldx, group_offsets, G, q, s, qT, sT, Mcap, padded_offsets, src, row_scale, T,
                       stream);
}

}  // namespace mx
