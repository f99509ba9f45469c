// SwiGLU backward fused with the MXFP8 quantizations the rest of the
// backward pass reads (kucoin.com MoK page, section 02: MXFP8 built into the
// SwiGLU step; lpnh.cn 2479732 section 1: the backward pass quantizes its
// gradients along both axes).  From the saved gate/up values and dh it
// computes, per element and with the arithmetic of mx_swiglu_backward,
//   d(gate, up) in bf16 -> row-wise MXFP8 (the gate+up dgrad operand) and
//                          column-wise MXFP8 per group (the gate+up wgrad operand)
//   h in bf16           -> column-wise MXFP8 per group (the down wgrad operand)
// bit-identical to mx_swiglu_backward followed by mx_quantize_dual of d(gate,
// up) and mx_quantize_cols of h, without writing or reading the bf16
// d(gate, up) and h.
//
// Work split as in the dual-layout quantizer: one workgroup per
// padded 256-row group tile x 256 columns of d(gate, up) (= 128 hidden
// units), walked as 4 sub-tiles of 64 columns, i.e. one hidden block of 32
// units each (gate columns [64 b, 64 b + 32), up columns [64 b + 32, 64 b + 64)).
// A lane loads 16 bytes (8 columns) of two rows of gate/up and the matching 16
// bytes of dh; the lanes holding gate and up of the same units (4 apart)
// split the 8 units: each computes the gradients (and h) of 4 of them after
// receiving the other half of their gate/up values, then they trade the
// gradients of the other column by lane swizzles.  The next sub-tile's loads
// are issued before the column-wise pass of the current one.
#include "mx_debug.h"
#include "mx_device.h"
#include "mx_internal.h"
#include "mx_swiglu.h"

namespace mx {

// 512 threads held to 128 VGPRs (two workgroups, 16 waves per CU): measured
// 4 % faster than 256 threads at 218 VGPRs (two workgroups, 8 waves) and 13 %
// faster than 512 threads at 134 VGPRs (one workgroup)
constexpr int kSbqThreads = 512;
constexpr int kSbqPairs = 128 / (kSbqThreads / 8);  // row pairs per lane

__global__ __launch_bounds__(kSbqThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void swiglu_backward_quant_kernel(
    const uint16_t* __restrict__ pre, const uint16_t* __restrict__ dh, int64_t M, int64_t I,
    const int32_t* __restrict__ off, const int32_t* __restrict__ P, int32_t G, uint8_t* __restrict__ q,
    uint8_t* __restrict__ s, uint8_t* __restrict__ qT, uint8_t* __restrict__ sT, uint8_t* __restrict__ hT,
    uint8_t* __restrict__ hTs, int64_t Mcap) {
    __shared__ uint4 tile[64 * 32];   // d(gate, up) sub-tile: 64 columns x 128 row pairs
    __shared__ uint4 htile[32 * 32];  // h sub-tile: 32 hidden columns x 128 row pairs
    __shared__ uint32_t unit_s[2][64];
    __shared__ uint32_t hunit_s[64];
    __shared__ uint32_t row_s[256][2];
    __shared__ int32_t sh_g;
    const int t = threadIdx.x;
    const int64_t N = 2 * I;
    const int64_t pt = blockIdx.y;
    const int64_t ct = blockIdx.x;
    const int64_t col0 = pt * 256;

    if (t == 0) sh_g = -1;
    __syncthreads();
    if (off == nullptr) {
        if (col0 < ((M + 255) / 256) * 256 && t == 0) sh_g = 0;
    } else {
        for (int g = t; g < G; g += kSbqThreads)
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
    const int c8 = t & 7;         // 16-byte column chunk of a sub-tile: gate (c8 < 4) or up
    const bool gate = c8 < 4;
    uint4 pa[kSbqPairs], pb[kSbqPairs], ea[kSbqPairs], eb[kSbqPairs];  // gate or up of rows r0, r1; dh of them
    auto load = [&](int st) {
        const int64_t nt = ct * 4 + st;  // hidden block of the sub-tile
        const int64_t ncol = nt * 64 + c8 * 8;
        const int64_t hcol = nt * 32 + (c8 & 3) * 8;
#pragma unroll
        for (int i = 0; i < kSbqPairs; ++i) {
            const int pr = i * (kSbqThreads / 8) + (t >> 3);
            const int64_t r0 = row_begin + 2 * pr, r1 = r0 + 1;
            pa[i] = pb[i] = ea[i] = eb[i] = make_uint4(0, 0, 0, 0);
            if (g >= 0) {
                if (r0 < row_end) {
                    pa[i] = load_stream16(pre + r0 * N + ncol);
                    ea[i] = load_stream16(dh + r0 * I + hcol);
                }
                if (r1 < row_end) {
                    pb[i] = load_stream16(pre + r1 * N + ncol);
                    eb[i] = load_stream16(dh + r1 * I + hcol);
                }
            }
        }
    };
    // d(gate, up) of this lane's 8 columns (units u0 .. u0 + 7 of one row) and
    // h of 4 of those units: the gate lane (c8 < 4) computes units 0-3, its up
    // partner (lane ^ 4) units 4-7, each after receiving the other half of
    // the gate/up pair, then they trade the gradients of the other column
    auto grad8 = [&](uint4 own, uint4 e, uint4& out, uint2& hv) {
        const uint32_t ow[4] = {own.x, own.y, own.z, own.w};
        const uint32_t dw[4] = {e.x, e.y, e.z, e.w};
        uint32_t dgp[2], dup[2], hp[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            // gate lane sends gate of units 4-7, receives up of units 0-3
            const uint32_t sent = gate ? ow[2 + k] : ow[k];
            const uint32_t got = (uint32_t)__builtin_amdgcn_ds_swizzle((int)sent, 0x101F);  // lane ^ 4
            const uint32_t gw = gate ? ow[k] : got;
            const uint32_t uw = gate ? got : ow[2 + k];
            const uint32_t d = gate ? dw[k] : dw[2 + k];
            const Grad r0 = swiglu_grad(lo_bf16(gw), lo_bf16(uw), lo_bf16(d));
            const Grad r1 = swiglu_grad(hi_bf16(gw), hi_bf16(uw), hi_bf16(d));
            dgp[k] = pack_bf16(r0.dg, r1.dg);
            dup[k] = pack_bf16(r0.du, r1.du);
            hp[k] = pack_bf16(r0.h, r1.h);
        }
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            // gate lane keeps d gate of units 0-3 and receives those of 4-7;
            // the up lane keeps d up of units 4-7 and receives those of 0-3
            const uint32_t got = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(gate ? dup[k] : dgp[k]), 0x101F);
            o[k] = gate ? dgp[k] : got;
            o[2 + k] = gate ? got : dup[k];
        }
        out = make_uint4(o[0], o[1], o[2], o[3]);
        hv = make_uint2(hp[0], hp[1]);
    };
    load(0);
    uint4 pend[kSbqPairs];
    uint8_t* rs = reinterpret_cast<uint8_t*>(row_s);
    uint8_t* us = reinterpret_cast<uint8_t*>(unit_s);
    uint8_t* hus = reinterpret_cast<uint8_t*>(hunit_s);
    const int64_t KB = Mcap / 32;
#pragma unroll 1
    for (int st = 0; st < 4; ++st) {
        const int64_t nt = ct * 4 + st;
        const int64_t ncol = nt * 64 + c8 * 8;
        const int b = st * 2 + (c8 >> 2);  // block of the chunk, 0..7
        uint32_t* tw = reinterpret_cast<uint32_t*>(tile);
        uint32_t* hw = reinterpret_cast<uint32_t*>(htile);
        // ---- per pair of rows: the gradients, d(gate, up) row-wise (as the
        // dual quantizer), then both rows paired into the transposed tiles
#pragma unroll
        for (int i = 0; i < kSbqPairs; ++i) {
            const int pr = i * (kSbqThreads / 8) + (t >> 3);
            const int64_t r0 = row_begin + 2 * pr, r1 = r0 + 1;
            uint4 da, db;
            uint2 ha, hb;
            grad8(pa[i], ea[i], da, ha);
            grad8(pb[i], eb[i], db, hb);
            const uint32_t Sa = scale_from_maxmag(quad_max_u32(max_mag8(da)));
            const uint32_t Sb = scale_from_maxmag(quad_max_u32(max_mag8(db)));
            const uint2 ca = quant8(da, Sa), cb = quant8(db, Sb);
            const uint2 snd = (c8 & 1) ? ca : cb;
            const uint32_t rx = (uint32_t)__builtin_amdgcn_mov_dpp((int)snd.x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
            const uint32_t ry = (uint32_t)__builtin_amdgcn_mov_dpp((int)snd.y, 0xB1, 0xF, 0xF, false);
            const uint4 o = (c8 & 1) ? make_uint4(rx, ry, cb.x, cb.y) : make_uint4(ca.x, ca.y, rx, ry);
            const int64_t rr = (c8 & 1) ? r1 : r0;
            const int64_t cc = ncol - (c8 & 1) * 8;
            if (st & 1) {
                if (g >= 0 && rr < row_end) {
                    store16(q + rr * N + cc - 64, pend[i]);
                    store16(q + rr * N + cc, o);
                }
            } else {
                pend[i] = o;
            }
            if ((t & 3) == 0) {
                rs[(2 * pr) * 8 + (b & 1) * 4 + (b >> 1)] = (uint8_t)Sa;
                rs[(2 * pr + 1) * 8 + (b & 1) * 4 + (b >> 1)] = (uint8_t)Sb;
            }
            const uint32_t aw[4] = {da.x, da.y, da.z, da.w};
            const uint32_t bw[4] = {db.x, db.y, db.z, db.w};
            const uint32_t haw[2] = {ha.x, ha.y};
            const uint32_t hbw[2] = {hb.x, hb.y};
            const int slot = (pr & 3);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int n0 = c8 * 8 + 2 * k, n1 = n0 + 1;
                tw[n0 * 128 + (((pr >> 2) ^ ((n0 >> 3) & 7)) << 2) + slot] = __builtin_amdgcn_perm(bw[k], aw[k], 0x05040100u);
                tw[n1 * 128 + (((pr >> 2) ^ ((n1 >> 3) & 7)) << 2) + slot] = __builtin_amdgcn_perm(bw[k], aw[k], 0x07060302u);
            }
            // h: units 0-3 of the 8 from the gate lane, 4-7 from the up lane
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int n0 = (c8 & 3) * 8 + (gate ? 0 : 4) + 2 * k, n1 = n0 + 1;
                hw[n0 * 128 + (((pr >> 2) ^ ((n0 >> 3) & 7)) << 2) + slot] = __builtin_amdgcn_perm(hbw[k], haw[k], 0x05040100u);
                hw[n1 * 128 + (((pr >> 2) ^ ((n1 >> 3) & 7)) << 2) + slot] = __builtin_amdgcn_perm(hbw[k], haw[k], 0x07060302u);
            }
        }
        __syncthreads();
        if (st < 3) load(st + 1);
        // ---- column-wise: 16 consecutive rows of one column per task, a
        // lane pair per 32-row block; d(gate, up) 64 columns, then h 32
        const int jj = t & 15;
        constexpr int kCols = kSbqThreads / 16;  // columns per pass
#pragma unroll
        for (int i = 0; i < 96 / kCols; ++i) {
            const bool isd = i < 64 / kCols;
            const int n = (isd ? i : i - 64 / kCols) * kCols + (t >> 4);
            const int sw = (n >> 3) & 7;
            const uint4* src = isd ? tile : htile;
            const uint4 d0 = src[n * 32 + ((2 * jj) ^ sw)];
            const uint4 d1 = src[n * 32 + ((2 * jj + 1) ^ sw)];
            uint32_t m = max_mag8(d0);
            const uint32_t m1 = max_mag8(d1);
            m = m > m1 ? m : m1;
            const uint32_t mo = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false);  // the pair's other lane
            m = m > mo ? m : mo;
            const uint32_t S = scale_from_maxmag(m);
            const uint2 c0 = quant8(d0, S), c1 = quant8(d1, S);
            const uint4 cv = make_uint4(c0.x, c0.y, c1.x, c1.y);
            if (isd) {
                store_stream16(qT + (nt * 64 + n) * Mcap + col0 + 16 * jj, cv);
                if ((t & 1) == 0) us[(n >> 5) * 256 + unit_byte((uint32_t)(n & 31), (uint32_t)(jj >> 1))] = (uint8_t)S;
            } else {
                store_stream16(hT + (nt * 32 + n) * Mcap + col0 + 16 * jj, cv);
                if ((t & 1) == 0) hus[unit_byte((uint32_t)n, (uint32_t)(jj >> 1))] = (uint8_t)S;
            }
        }
        __syncthreads();
        if (t < 128) {
            const int u = t >> 6;
            __builtin_nontemporal_store(unit_s[u][t & 63],
                                        reinterpret_cast<uint32_t*>(sT + (nt * 2 + u) * 32 * KB + pt * 256) + (t & 63));
        } else if (t < 192) {
            __builtin_nontemporal_store(hunit_s[t & 63],
                                        reinterpret_cast<uint32_t*>(hTs + nt * 32 * KB + pt * 256) + (t & 63));
        }
    }
    __syncthreads();
    // ---- d(gate, up) row-wise packed scales: one tile row per thread
    const int64_t KBr = 8 * (N / 256);
    if (t < 256 && g >= 0 && row_begin + t < row_end) {
        const int64_t r = row_begin + t;
        uint32_t* dst = reinterpret_cast<uint32_t*>(s + (r >> 5) * 32 * KBr + ct * 256) + (r & 31);
        dst[0] = row_s[t][0];
        dst[32] = row_s[t][1];
    }
    const int64_t Mpad = ((M + 31) / 32) * 32;
    if (pt == 0 && t < Mpad - M) {
        const int64_t r = M + t;
        uint32_t* dst = reinterpret_cast<uint32_t*>(s + (r >> 5) * 32 * KBr + ct * 256) + (r & 31);
        dst[0] = 0u;
        dst[32] = 0u;
    }
}

#ifdef MXMOE_DEBUG
hipError_t debug_take_swiglu_quant(uint32_t* out) { return debug_take_word(out); }
#endif

hipError_t launch_swiglu_backward_quant(const uint16_t* preact, const uint16_t* dh, int64_t M, int64_t I,
                                        const int32_t* group_offsets, int32_t G, uint8_t* q, uint8_t* s,
                                        uint8_t* qT, uint8_t* sT, uint8_t* hT, uint8_t* hTs, int64_t Mcap,
                                        int32_t* padded_offsets, hipStream_t stream) {
    if (group_offsets != nullptr) {
        hipError_t e = launch_cols_prefix(group_offsets, G, M, padded_offsets, stream);
        if (e != hipSuccess) return e;
    } else {
        G = 1;
    }
    if (I == 0 || Mcap == 0) return hipSuccess;
    dim3 grid((unsigned)(2 * I / 256), (unsigned)(Mcap / 256));
    hipLaunchKernelGGL(swiglu_backward_quant_kernel, grid, dim3(kSbqThreads), 0, stream, preact, dh, M, I, group_offsets,
                       (const int32_t*)padded_offsets, G, q, s, qT, sT, hT, hTs, Mcap);
    return hipGetLastError();
}

}  // namespace mx
