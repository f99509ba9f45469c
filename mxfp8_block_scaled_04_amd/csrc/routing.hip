// The one-GPU share of expert-parallel dispatch and combine for gfx950.
//
// Method (kucoin.com MoK page, section 02): the expert side of the dispatch
// pulls each routed token by its source position and lays the rows out
// grouped by local expert, so that the grouped GEMM reads them in place; the
// combine sends every expert output back to its token.  On one GPU the
// source is local memory and the exchange is a gather:
//  * route_count_kernel + route_place_kernel: a stable counting sort of the
//    routed entries (token t, choice j) by expert, giving the group offsets,
//    the source token of every expert-ordered slot and the slot of every
//    entry (the gather itself, with MXFP8 on the way, is the gathering
//    variant of the dual-layout quantizer);
//  * combine_kernel: out[t] = sum_j w[t][j] y[slot(t, j)], the routing-
//    weighted sum of a token's expert outputs (the plain sum without weights:
//    the backward of the gather).
#include "mx_bf16.h"
#include "mx_debug.h"
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

// ---------------------------------------------------------------------------
// Routing plan, pass 1 (one workgroup of 1024 threads): per-expert counts
// of the entries whose expert lies in [0, G) (LDS atomics: counts do not
// depend on the order), their exclusive prefix into offsets[0..G], and
// slot -1 for the entries outside [0, G).
// ---------------------------------------------------------------------------
static_assert(kMaxGroups <= 4 * 1024, "the count kernel covers 4 experts per thread");
__global__ __launch_bounds__(1024) void route_count_kernel(const int32_t* __restrict__ experts, int64_t n, int32_t G,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ slot_of) {
    __shared__ int32_t cnt[kMaxGroups];
    __shared__ int32_t part[1024];
    const int t = threadIdx.x;
    for (int g = t; g < G; g += 1024) cnt[g] = 0;
    __syncthreads();
    for (int64_t j = t; j < n; j += 1024) {
        const int32_t e = experts[j];
        if (e >= 0 && e < G)
            atomicAdd(&cnt[e], 1);
        else
            slot_of[j] = -1;
    }
    __syncthreads();
    int32_t loc[4];
    int32_t sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = 4 * t + i;
        loc[i] = g < G ? cnt[g] : 0;
        sum += loc[i];
    }
    part[t] = sum;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {  // inclusive Hillis-Steele scan
        const int32_t v = t >= d ? part[t - d] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    int32_t run = part[t] - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = 4 * t + i;
        if (g <= G) offsets[g] = run;
        run += loc[i];
    }
    if (t == 1023 && G == 4 * 1024) offsets[G] = run;
}

// ---------------------------------------------------------------------------
// Routing plan, pass 2: workgroup g places the entries of expert g.  It
// walks all entries in index order, 1024 at a time; a wave ballot gives each
// hit its rank among the hits of its wave, a prefix over the 16 waves its
// rank in the chunk, so slots follow the entry order (stable) and the result
// does not depend on scheduling.  Each workgroup reads the whole expert list
// (n ints, from L2): O(G n) reads in all, with an early exit once the
// expert's count is placed.
// ---------------------------------------------------------------------------
constexpr int kPlaceThreads = 1024;
__global__ __launch_bounds__(kPlaceThreads) void route_place_kernel(const int32_t* __restrict__ experts,
                                                                    const float* __restrict__ weights, int64_t n,
                                                                    int32_t k, const int32_t* __restrict__ offsets,
                                                                    int32_t* __restrict__ src,
                                                                    int32_t* __restrict__ slot_of,
                                                                    float* __restrict__ slot_weight) {
    __shared__ int32_t wave_hits[kPlaceThreads / 64];
    const int t = threadIdx.x;
    const int w = t >> 6, l = t & 63;
    const int32_t g = (int32_t)blockIdx.x;
    int32_t base = offsets[g];
    const int32_t end = offsets[g + 1];
    for (int64_t c = 0; c < n && base < end; c += kPlaceThreads) {
        const int64_t j = c + t;
        const bool hit = j < n && experts[j] == g;
        const uint64_t mask = __ballot(hit);
        if (l == 0) wave_hits[w] = __popcll(mask);
        __syncthreads();
        int32_t before = 0, total = 0;
#pragma unroll
        for (int v = 0; v < kPlaceThreads / 64; ++v) {
            const int32_t h = wave_hits[v];
            before += v < w ? h : 0;
            total += h;
        }
        if (hit) {
            const int32_t slot = base + before + (int32_t)__popcll(mask & ((1ull << l) - 1ull));
            src[slot] = (int32_t)(j / k);
            slot_of[j] = slot;
            if (slot_weight != nullptr) slot_weight[slot] = weights[j];
        }
        base += total;
        __syncthreads();  // wave_hits is rewritten by the next chunk
    }
}

hipError_t launch_route_plan(const int32_t* experts, const float* weights, int64_t T, int32_t k, int32_t G,
                             int32_t* offsets, int32_t* src, int32_t* slot_of, float* slot_weight,
                             hipStream_t stream) {
    const int64_t n = T * k;
    hipLaunchKernelGGL(route_count_kernel, dim3(1), dim3(1024), 0, stream, experts, n, G, offsets, slot_of);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n == 0) return e;
    hipLaunchKernelGGL(route_place_kernel, dim3((unsigned)G), dim3(kPlaceThreads), 0, stream, experts, weights, n, k,
                       (const int32_t*)offsets, src, slot_of, slot_weight);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine: one workgroup of 256 lanes per token row and 2048 columns
// (tokens fastest in the grid); a lane holds 8 columns in fp32, adds w y for
// each of the token's k entries in choice order (fused multiply-add, one
// rounding per step), then rounds to bf16 once and stores 16 bytes.  Entries whose slot lies outside [0, M)
// (not routed) are skipped; without weights every entry counts once.
// ---------------------------------------------------------------------------
constexpr int kCombineThreads = 256;
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const uint16_t* __restrict__ y, int64_t M,
                                                                  int64_t N, int64_t ldy,
                                                                  const int32_t* __restrict__ slot_of,
                                                                  const float* __restrict__ w, int32_t k,
                                                                  uint16_t* __restrict__ out) {
    const int64_t tok = blockIdx.x;
    const int64_t c0 = ((int64_t)blockIdx.y * kCombineThreads + threadIdx.x) * 8;
    if (c0 >= N) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int32_t j = 0; j < k; ++j) {
        const int32_t slot = slot_of[tok * k + j];
        if (slot < 0 || slot >= M) continue;
        const float wj = w != nullptr ? w[tok * k + j] : 1.0f;
        const uint4 v = load_stream16(y + (int64_t)slot * ldy + c0);
        const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = __builtin_fmaf(wj, lo_bf16(vw[i]), acc[2 * i]);
            acc[2 * i + 1] = __builtin_fmaf(wj, hi_bf16(vw[i]), acc[2 * i + 1]);
        }
    }
    store16(out + tok * N + c0, make_uint4(pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]),
                                           pack_bf16(acc[4], acc[5]), pack_bf16(acc[6], acc[7])));
}

hipError_t launch_combine(const uint16_t* y, int64_t M, int64_t N, int64_t ldy, const int32_t* slot_of,
                          const float* w, int64_t T, int32_t k, uint16_t* out, hipStream_t stream) {
    if (T == 0 || N == 0) return hipSuccess;
    dim3 grid((unsigned)T, (unsigned)((N / 8 + kCombineThreads - 1) / kCombineThreads));
    hipLaunchKernelGGL(combine_kernel, grid, dim3(kCombineThreads), 0, stream, y, M, N, ldy, slot_of, w, k, out);
    return hipGetLastError();
}

}  // namespace mx
