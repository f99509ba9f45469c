// MXFP8 quantization kernels for gfx950: row-wise (scales along K) and
// column-wise / transposed (scales along M, per-group block restart).  The
// dual-layout kernel (both results from one read) is in quantize_dual.hip.
//
// Method (lpnh.cn 2479732 section 1; aigc.bar "秘密武器"): one E8M0 scale per
// 32-element block, the block divided by it and cast to FP8 E4M3; the
// scales are written straight into the packed order the scaled matrix
// instruction reads (no reshape pass).  Both kernels are HBM-bound: they read
// 2 B and write 1 + 1/32 B per element once, with 16-byte coalesced loads.
#include "mx_device.h"
#include "mx_internal.h"
#include "mx_debug.h"

namespace mx {

// ---------------------------------------------------------------------------
// Row-wise.  One workgroup of kRowsWaves waves quantizes one unit of 32 rows
// x 256 columns (16 KB of bf16): every load instruction covers two rows
// (lanes 0-31 one row, 32-63 the next; 4 lanes per 32-wide block), so each
// lane issues 16 / kRowsWaves 16-byte loads -- short-lived lanes with one or
// two loads in flight stream HBM best on this part.  The block max is
// reduced over the lane quad with DPP, the codes are stored 8 bytes per lane
// (256 contiguous bytes per row), and the unit's 256 scale bytes are staged
// in LDS in packed order and written as one coalesced 256-byte store.
// Rows >= M and blocks >= K read as zero, which yields scale 0 and keeps the
// pad bytes of the packed scale array at 0.
// ---------------------------------------------------------------------------
constexpr int kRowsWaves = kQuantRowsThreads / 64;
constexpr int kRowsLoads = 16 / kRowsWaves;  // 16-byte loads per lane
static_assert(kRowsWaves == 4 || kRowsWaves == 8 || kRowsWaves == 16, "unit = 32 rows");

__global__ __launch_bounds__(64 * kRowsWaves) void quantize_rows_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                                        int64_t K, int64_t ldx,
                                                                        uint8_t* __restrict__ q,
                                                                        uint8_t* __restrict__ s, int64_t nchunks) {
    __shared__ uint32_t unit_s[64];
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int l = t & 63;
    const int64_t ru = blockIdx.x / nchunks;
    const int64_t ch = blockIdx.x - ru * nchunks;
    const int64_t col = ch * 256 + (l & 31) * 8;
    const bool colok = col < K;  // K % 32 == 0: a lane's 8 columns are all in or all out

    uint4 d[kRowsLoads];
#pragma unroll
    for (int i = 0; i < kRowsLoads; ++i) {
        const int64_t row = ru * 32 + w * (2 * kRowsLoads) + 2 * i + (l >> 5);
        d[i] = make_uint4(0, 0, 0, 0);
        if (colok && row < M) d[i] = load_stream16(x + row * ldx + col);
    }
    uint8_t* us = reinterpret_cast<uint8_t*>(unit_s);
#pragma unroll
    for (int i = 0; i < kRowsLoads; ++i) {
        const int r32 = w * (2 * kRowsLoads) + 2 * i + (l >> 5);
        const int64_t row = ru * 32 + r32;
        const uint32_t S = scale_from_maxmag(quad_max_u32(max_mag8(d[i])));
        const uint2 c = quant8(d[i], S);
        if (colok && row < M) store_stream8(q + row * K + col, c);
        if ((l & 3) == 0) us[unit_byte((uint32_t)r32, (uint32_t)((l & 31) >> 2))] = (uint8_t)S;
    }
    __syncthreads();
    if (t < 64) {
        const int64_t KB = nchunks * 8;
        __builtin_nontemporal_store(unit_s[t], reinterpret_cast<uint32_t*>(s + ru * 32 * KB + ch * 256) + t);
    }
}

hipError_t launch_quantize_rows(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                                uint8_t* s, hipStream_t stream) {
    if (M == 0 || K == 0) return hipSuccess;
    const int64_t nchunks = (K + 255) / 256;
    const int64_t units = ((M + 31) / 32) * nchunks;
    hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)units), dim3(64 * kRowsWaves), 0, stream, x, M, K,
                       ldx, q, s, nchunks);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Column-wise.  Groups: rows [o_g, o_g + m_g) with o_g = clamp(off[g], 0, M)
// and m_g = max(clamp(off[g+1], 0, M) - o_g, 0).  Group g occupies padded
// columns [P[g], P[g+1]) of the transposed result, P[g+1] - P[g] =
// 256 * ceil(m_g / 256).
// ---------------------------------------------------------------------------

// One workgroup of 1024 threads: P[0..G] from the group offsets.
static_assert(kMaxGroups <= 4 * 1024, "prefix kernel covers 4 groups per thread");
__global__ __launch_bounds__(1024) void cols_prefix_kernel(const int32_t* __restrict__ off, int32_t G,
                                                           int64_t M, int32_t* __restrict__ P) {
    __shared__ int32_t part[1024];
    const int t = threadIdx.x;
    int32_t loc[4];
    int32_t sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int g = 4 * t + j;
        int32_t pad = 0;
        if (g <= G) debug_flag(offsets_entry_bad(off, g, G, M), kDbgOffsets);
        if (g < G) {
            const int32_t a = clamp_off(off, g, M), b = clamp_off(off, g + 1, M);
            const int32_t mg = b > a ? b - a : 0;
            pad = ((mg + kColsPad - 1) / kColsPad) * kColsPad;
        }
        loc[j] = pad;
        sum += pad;
    }
    part[t] = sum;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {  // inclusive Hillis-Steele scan
        const int32_t v = t >= d ? part[t - d] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    int32_t run = part[t] - sum;  // exclusive prefix of this thread's slice
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int g = 4 * t + j;
        if (g <= G) P[g] = run;
        run += loc[j];
    }
    if (t == 1023 && G == 4 * 1024) {  // the one entry past every slice
        P[G] = run;
        debug_flag(offsets_entry_bad(off, G, G, M), kDbgOffsets);
    }
}

// One workgroup handles padded column tile pt (256 rows of one group) x 64
// columns of x.  Load: each task reads 16 bytes (8 columns) of two adjacent
// rows and pairs them per column with v_perm into dwords (x[m][n],
// x[m+1][n]), stored transposed in LDS with a 16-byte XOR swizzle (writes
// spread over all banks, reads of 16 contiguous bytes conflict-free).
// Compute: each task reads 16 bytes = 8 consecutive rows of one column,
// 4 lanes per 32-row block, and proceeds as the row-wise kernel; lanes 0-31
// of a wave store 256 contiguous code bytes of one transposed row.
// kColsThreads lanes per workgroup share the tile's tasks: 256 for large
// grids, 512 (twice the waves per CU at the same LDS) for grids below
// kColsSmallGrid workgroups, where it was measured 9 % faster (and 3 % slower
// on large grids).
constexpr int kColsSmallGrid = 32768;
template <int kColsThreads>
__global__ __launch_bounds__(kColsThreads) void quantize_cols_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                                     int64_t N, int64_t ldx,
                                                                     const int32_t* __restrict__ off,
                                                                     const int32_t* __restrict__ P, int32_t G,
                                                                     uint8_t* __restrict__ qT,
                                                                     uint8_t* __restrict__ sT, int64_t Mcap) {
    // tile[n][pair]: 64 columns x 128 row pairs, 16-byte granules swizzled by n/8
    __shared__ uint4 tile[64 * 32];
    __shared__ uint32_t unit_s[2][64];
    __shared__ int32_t sh_g;
    const int t = threadIdx.x;
    // row tiles vary fastest: workgroups dispatched together read far-apart
    // rows (spread over all HBM channels) and write adjacent 256-byte pieces
    // of the same transposed rows
    const int64_t pt = blockIdx.x;
    const int64_t nt = blockIdx.y;
    const int64_t col0 = pt * 256;  // padded column of the transposed result

    if (t == 0) sh_g = -1;
    __syncthreads();
    int64_t row_begin = 0, row_end = 0;
    if (off == nullptr) {
        if (col0 < ((M + 255) / 256) * 256 && t == 0) sh_g = 0;
    } else {
        for (int g = t; g < G; g += kColsThreads)
            if (P[g] <= col0 && col0 < P[g + 1]) sh_g = g;
    }
    __syncthreads();
    const int g = sh_g;
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
    // ---- load + transpose into LDS (1024 pair tasks)
    const int c8 = t & 7;  // 16-byte column chunk (8 columns)
    const int64_t ncol = nt * 64 + c8 * 8;
#pragma unroll
    for (int i = 0; i < 1024 / kColsThreads; ++i) {
        const int pr = i * (kColsThreads / 8) + (t >> 3);  // row pair 0..127
        const int64_t r0 = row_begin + 2 * pr, r1 = r0 + 1;
        uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
        if (g >= 0 && ncol < N) {
            if (r0 < row_end) a = load_stream16(x + r0 * ldx + ncol);
            if (r1 < row_end) b = load_stream16(x + r1 * ldx + ncol);
        }
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
        uint32_t* tw = reinterpret_cast<uint32_t*>(tile);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo = __builtin_amdgcn_perm(bw[k], aw[k], 0x05040100u);  // (x[r0][2k], x[r1][2k])
            const uint32_t hi = __builtin_amdgcn_perm(bw[k], aw[k], 0x07060302u);  // (x[r0][2k+1], x[r1][2k+1])
            const int n0 = c8 * 8 + 2 * k, n1 = n0 + 1;
            tw[n0 * 128 + (((pr >> 2) ^ ((n0 >> 3) & 7)) << 2) + (pr & 3)] = lo;
            tw[n1 * 128 + (((pr >> 2) ^ ((n1 >> 3) & 7)) << 2) + (pr & 3)] = hi;
        }
    }
    __syncthreads();
    // ---- quantize 8 consecutive rows of one column per task (2048 tasks)
    const int j = t & 31;  // granule: rows 8j..8j+7 of the tile, block j/4
    uint8_t* us = reinterpret_cast<uint8_t*>(unit_s);
#pragma unroll
    for (int i = 0; i < 2048 / kColsThreads; ++i) {
        const int n = i * (kColsThreads / 32) + (t >> 5);
        const uint4 d = tile[n * 32 + (j ^ ((n >> 3) & 7))];
        const uint32_t S = scale_from_maxmag(quad_max_u32(max_mag8(d)));
        const uint2 c = quant8(d, S);
        const int64_t ng = nt * 64 + n;
        if (ng < N) {
            // small grids: ordinary stores (measured 4 % faster there, and 5 %
            // slower on large grids, which keep non-temporal ones)
            if (kColsThreads == 512) store8(qT + ng * Mcap + col0 + 8 * j, c);
            else store_stream8(qT + ng * Mcap + col0 + 8 * j, c);
        }
        if ((t & 3) == 0) us[(n >> 5) * 256 + unit_byte((uint32_t)(n & 31), (uint32_t)(j >> 2))] = (uint8_t)S;
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

#ifdef MXMOE_DEBUG
hipError_t debug_take_quantize(uint32_t* out) { return debug_take_word(out); }
#endif

hipError_t launch_cols_prefix(const int32_t* group_offsets, int32_t G, int64_t M, int32_t* padded_offsets,
                              hipStream_t stream) {
    hipLaunchKernelGGL(cols_prefix_kernel, dim3(1), dim3(1024), 0, stream, group_offsets, G, M, padded_offsets);
    return hipGetLastError();
}

hipError_t launch_quantize_cols(const uint16_t* x, int64_t M, int64_t N, int64_t ldx,
                                const int32_t* group_offsets, int32_t G, uint8_t* qT, uint8_t* sT,
                                int64_t Mcap, int32_t* padded_offsets, hipStream_t stream) {
    if (group_offsets != nullptr) {
        hipError_t e = launch_cols_prefix(group_offsets, G, M, padded_offsets, stream);
        if (e != hipSuccess) return e;
    } else {
        G = 1;
    }
    if (N == 0 || Mcap == 0) return hipSuccess;
    dim3 grid((unsigned)(Mcap / 256), (unsigned)((N + 63) / 64));
    const bool small = (int64_t)grid.x * grid.y < kColsSmallGrid;
    if (small)
        hipLaunchKernelGGL(quantize_cols_kernel<512>, grid, dim3(512), 0, stream, x, M, N, ldx, group_offsets,
                           (const int32_t*)padded_offsets, G, qT, sT, Mcap);
    else
        hipLaunchKernelGGL(quantize_cols_kernel<256>, grid, dim3(256), 0, stream, x, M, N, ldx, group_offsets,
                           (const int32_t*)padded_offsets, G, qT, sT, Mcap);
    return hipGetLastError();
}

}  // namespace mx
