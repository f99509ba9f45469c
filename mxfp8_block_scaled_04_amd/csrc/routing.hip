// The one-GPU share of expert-parallel dispatch and combine for gfx950.
//
// Method (kucoin.com MoK page, section 02): the expert side of the dispatch
// pulls each routed token by its source position and lays the rows out
// grouped by local expert, so that the grouped GEMM reads them in place; the
// combine sends every expert output back to its token.  On one GPU the
// source is local memory and the exchange is a gather:
//  * route_count_kernel, route_scan_kernel, route_place_kernel: a stable
//    counting sort of the routed entries (token t, choice j) by expert,
//    giving the group offsets, the source token of every expert-ordered slot
//    and the slot of every entry (the gather itself, with MXFP8 on the way,
//    is the gathering variant of the dual-layout quantizer);
//  * combine_kernel: out[t] = sum_j w[t][j] y[slot(t, j)], the routing-
//    weighted sum of a token's expert outputs (the plain sum without weights:
//    the backward of the gather).
#include "mx_bf16.h"
#include "mx_debug.h"
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

// ---------------------------------------------------------------------------
// Routing plan, pass 1 (one workgroup of 1024 threads per expert): workgroup
// g counts the entries of expert g (a ballot per 1024-entry piece, 8 pieces
// loaded together, no atomics) into offsets[g + 1]; workgroup 0 also sets
// slot -1 for the entries outside [0, G).
// ---------------------------------------------------------------------------
constexpr int kPlanBatch = 8;  // entries per thread loaded together (their latencies overlap)
constexpr int kPlanThreads = 1024;
__global__ __launch_bounds__(kPlanThreads) void route_count_kernel(const int32_t* __restrict__ experts, int64_t n,
                                                                   int32_t G, int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ slot_of) {
    __shared__ int32_t wave_sum[kPlanThreads / 64];
    const int t = threadIdx.x;
    const int l = t & 63;
    const int32_t g = (int32_t)blockIdx.x;
    int32_t mine = 0;  // hits of this wave (lane 0)
    for (int64_t c = 0; c < n; c += kPlanBatch * kPlanThreads) {
        int32_t e[kPlanBatch];
#pragma unroll
        for (int b = 0; b < kPlanBatch; ++b) {
            const int64_t j = c + b * kPlanThreads + t;
            e[b] = j < n ? experts[j] : -1;
        }
#pragma unroll
        for (int b = 0; b < kPlanBatch; ++b) {
            mine += __popcll(__ballot(e[b] == g));
            const int64_t j = c + b * kPlanThreads + t;
            if (g == 0 && j < n && (e[b] < 0 || e[b] >= G)) slot_of[j] = -1;
        }
    }
    if (l == 0) wave_sum[t >> 6] = mine;
    __syncthreads();
    if (t == 0) {
        int32_t total = 0;
        for (int w = 0; w < kPlanThreads / 64; ++w) total += wave_sum[w];
        offsets[g + 1] = total;
        if (g == 0) offsets[0] = 0;
    }
}

// Routing plan, pass 2 (one workgroup): offsets[1..G] from counts to their
// inclusive prefix, so offsets becomes the exclusive prefix of the counts.
static_assert(kMaxGroups <= 4 * 1024, "the scan covers 4 experts per thread");
__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t G, int32_t* __restrict__ offsets) {
    __shared__ int32_t part[1024];
    const int t = threadIdx.x;
    int32_t loc[4];
    int32_t sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = 4 * t + i;
        loc[i] = g < G ? offsets[g + 1] : 0;
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
        run += loc[i];
        if (g < G) offsets[g + 1] = run;
    }
}

// ---------------------------------------------------------------------------
// Routing plan, pass 3: workgroup g places the entries of expert g.  It
// walks all entries in index order, 8 x 1024 at a time (8 loads per thread
// in flight); a wave ballot gives each hit its rank among the hits of its
// wave and 1024-entry piece, a prefix over the pieces and waves before it
// its rank in the batch, so slots follow the entry order (stable) and the
// result does not depend on scheduling.  Each workgroup reads the whole
// expert list (n ints, from L2): O(G n) reads in all, with an early exit once
// the expert's count is placed.
// ---------------------------------------------------------------------------
constexpr int kPlaceThreads = kPlanThreads;
__global__ __launch_bounds__(kPlaceThreads) void route_place_kernel(const int32_t* __restrict__ experts,
                                                                    const float* __restrict__ weights, int64_t n,
                                                                    int32_t k, const int32_t* __restrict__ offsets,
                                                                    int32_t* __restrict__ src,
                                                                    int32_t* __restrict__ slot_of,
                                                                    float* __restrict__ slot_weight) {
    constexpr int kWaves = kPlaceThreads / 64;
    constexpr int kPieces = kPlanBatch * kWaves;  // (1024-entry piece, wave) pairs of a batch, entry order
    static_assert(kPieces <= kPlaceThreads, "one thread per pair in the prefix");
    static_assert(kPieces == 128, "the prefix scan below covers two waves of pairs");
    __shared__ int32_t hits[kPieces];
    __shared__ int32_t incl[kPieces];
    __shared__ int32_t prefix[kPieces + 1];
    const int t = threadIdx.x;
    const int w = t >> 6, l = t & 63;
    const int32_t g = (int32_t)blockIdx.x;
    int32_t base = offsets[g];
    const int32_t end = offsets[g + 1];
    for (int64_t c = 0; c < n && base < end; c += kPlanBatch * kPlaceThreads) {
        bool hit[kPlanBatch];
#pragma unroll
        for (int b = 0; b < kPlanBatch; ++b) {
            const int64_t j = c + b * kPlaceThreads + t;
            hit[b] = j < n && experts[j] == g;
        }
#pragma unroll
        for (int b = 0; b < kPlanBatch; ++b) {
            const uint64_t mask = __ballot(hit[b]);
            if (l == 0) hits[b * kWaves + w] = __popcll(mask);
        }
        __syncthreads();
        // exclusive prefix over the pairs (entry order: piece, then wave):
        // an inclusive scan inside each of the first two waves by lane
        // shifts, then wave 1 adds wave 0's total
        if (t < kPieces) {
            int32_t v = hits[t];
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int32_t u = __shfl_up(v, d);
                if (l >= d) v += u;
            }
            incl[t] = v;
        }
        __syncthreads();
        if (t < kPieces) prefix[t] = incl[t] - hits[t] + (t >= 64 ? incl[63] : 0);
        if (t == kPieces) prefix[t] = incl[63] + incl[127];
        __syncthreads();
#pragma unroll
        for (int b = 0; b < kPlanBatch; ++b) {
            const uint64_t mask = __ballot(hit[b]);
            if (!hit[b]) continue;
            const int64_t j = c + b * kPlaceThreads + t;
            const int32_t slot = base + prefix[b * kWaves + w] + (int32_t)__popcll(mask & ((1ull << l) - 1ull));
            src[slot] = (int32_t)(j / k);
            slot_of[j] = slot;
            if (slot_weight != nullptr) slot_weight[slot] = weights[j];
        }
        base += prefix[kPieces];
        __syncthreads();  // hits and prefix are rewritten by the next batch
    }
}

hipError_t launch_route_plan(const int32_t* experts, const float* weights, int64_t T, int32_t k, int32_t G,
                             int32_t* offsets, int32_t* src, int32_t* slot_of, float* slot_weight,
                             hipStream_t stream) {
    const int64_t n = T * k;
    hipLaunchKernelGGL(route_count_kernel, dim3((unsigned)G), dim3(kPlanThreads), 0, stream, experts, n, G, offsets,
                       slot_of);
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, G, offsets);
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
constexpr int kCombineGroup = 8;  // entries whose rows are loaded together
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const uint16_t* __restrict__ y, int64_t M,
                                                                  int64_t N, int64_t ldy,
                                                                  const int32_t* __restrict__ slot_of,
                                                                  const float* __restrict__ w, int32_t k,
                                                                  uint16_t* __restrict__ out) {
    const int64_t tok = blockIdx.x;
    const int64_t c0 = ((int64_t)blockIdx.y * kCombineThreads + threadIdx.x) * 8;
    if (c0 >= N) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // the entries in groups of 8: all their row loads in flight at once,
    // then the sums in choice order
    for (int32_t j0 = 0; j0 < k; j0 += kCombineGroup) {
        uint4 v[kCombineGroup];
        float wv[kCombineGroup];
#pragma unroll
        for (int u = 0; u < kCombineGroup; ++u) {
            const int32_t j = j0 + u;
            const int32_t slot = j < k ? slot_of[tok * k + j] : -1;
            wv[u] = 0.0f;
            v[u] = make_uint4(0, 0, 0, 0);
            if (slot >= 0 && slot < M) {
                wv[u] = w != nullptr ? w[tok * k + j] : 1.0f;
                v[u] = load_stream16(y + (int64_t)slot * ldy + c0);
            }
        }
#pragma unroll
        for (int u = 0; u < kCombineGroup; ++u) {
            if (j0 + u >= k) break;
            const int32_t slot = slot_of[tok * k + j0 + u];
            if (slot < 0 || slot >= M) continue;
            const uint32_t vw[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = __builtin_fmaf(wv[u], lo_bf16(vw[i]), acc[2 * i]);
                acc[2 * i + 1] = __builtin_fmaf(wv[u], hi_bf16(vw[i]), acc[2 * i + 1]);
            }
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
