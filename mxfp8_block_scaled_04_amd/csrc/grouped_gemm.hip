// Block-scaled grouped GEMM for gfx950 (MXFP8 operands, fp32 accumulation,
// bf16 output).
//
// Method (aigc.bar "为MoE量身定制优化" and "拥抱原生硬件指令"; lpnh.cn 2479732
// section 5): per-expert GEMMs over variable row groups, with the block
// scales applied by the matrix instruction itself (no dequantization pass),
// and an expert-aware tile order so an expert's weights are reused from
// cache.  On gfx950 the instruction is v_mfma_scale_f32_32x32x64_f8f6f4,
// which takes one E8M0 byte per lane per operand; the packed scale layout
// written by the quantize kernels hands each lane that byte for four
// consecutive 64-wide K steps in one dword (byte = op_sel).
//
// Kernel: persistent workgroups of 4 waves, tile 256 x 256, K stage 128.
//  * fp8 A/B stages go straight from global memory into LDS with 16-byte
//    global_load_lds (no VGPR staging), two buffers, one stage in flight
//    while the previous one is multiplied.  Rows are stored 128 bytes apart
//    with the 16-byte granule index XORed by (row mod 8), so the fragment
//    reads (32 rows, same K offset) hit distinct banks.
//  * Each wave owns a 128 x 128 sub-tile = 4 x 4 MFMA blocks; per 64-wide K
//    step a lane holds 16 bytes of each 32-wide block for its row.
//  * Scale dwords come straight from global memory into VGPRs, one chunk
//    (256 of K) ahead.
//  * Tile order: expert-major; inside an expert, bands of 4 M-tiles walked
//    M-fastest; workgroups are mapped so that each XCD (workgroups are
//    dealt to the 8 XCDs round-robin) runs a contiguous range of tile ids
//    and so shares operands through its own L2.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

namespace {

constexpr int TM = 256;
constexpr int TN = 256;
constexpr int TK = 64;     // K bytes per pipeline stage (one MFMA K step)
constexpr int NBUF = 4;    // LDS stage buffers; three stages in flight
constexpr int kBand = 4;   // M-tiles per band of the tile order

typedef __attribute__((address_space(3))) void lds_t;

struct GemmArgs {
    const uint8_t* A;
    const uint8_t* As;
    const uint8_t* B;
    const uint8_t* Bs;
    const int32_t* offsets;
    uint16_t* out;
    int64_t M, N, K, Mcap;
    int32_t G;
    int32_t mode;  // 0: rows of X grouped (forward); 1: contraction grouped (wgrad);
                   // 2: rows grouped, weights read transposed (dgrad)
    int64_t ldb;   // mode 2: row stride of the transposed weights (their Mcap)
};

struct Tile {
    const uint8_t* A;   // base of A data (row 0)
    const uint8_t* As;  // base of A packed scales (row 0)
    int64_t lda, a_unit;  // row stride of A data; bytes per 32-row scale unit (32 * KB)
    int64_t a_row0, a_lim;
    const uint8_t* B;
    const uint8_t* Bs;
    int64_t ldb, b_unit;
    int64_t b_row0, b_lim;
    int64_t k0, k1;  // contraction range, multiples of 256
    uint16_t* out;   // element (0, 0) of the tile
    int64_t ldo;
    int32_t rows, cols;  // valid part of the tile
};

__shared__ __attribute__((aligned(16))) uint8_t lds_a[NBUF][TM * TK];
__shared__ __attribute__((aligned(16))) uint8_t lds_b[NBUF][TN * TK];
__shared__ __attribute__((aligned(16))) uint32_t lds_sa[2][TM / 32][64];  // scale dwords, [chunk parity][32-row unit][lane]
__shared__ __attribute__((aligned(16))) uint32_t lds_sb[2][TN / 32][64];
__shared__ int32_t tile_end[kMaxGroups];  // inclusive prefix of tiles per group

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

// Stage rows are 64 bytes (4 granules of 16 B).  Granule c of tile row r is
// stored at position c ^ swz(r).  Measured on gfx950: a 64-lane ds_read_b128
// is served in 4 passes of 16 lanes at 256 bytes per clock, a pass taking
// lanes whose row index varies in bits 0, 1, 3 and in bit 2 tied to bit 4.
// With 64-byte rows the 16-byte bank group of a read is 4 (r mod 4) + granule,
// so XORing the granule with bits 2-3 of the row makes the 16 groups of every
// pass distinct (zero bank-conflict cycles measured for this pattern).
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

// The address base must be wave-uniform (an SGPR pair).
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// 16-byte direct global->LDS load (global_load_lds_dwordx4): lane i of the
// wave writes LDS bytes [lds + 16 i, lds + 16 i + 16).  Issued as inline asm
// so that the compiler's own wait insertion does not stall every later LDS
// read on it; completion is enforced explicitly (wait_vm<N> + barrier)
// before a buffer is read.  M0 is only written here; no other code in these
// kernels reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
                 : "memory", "m0");
}
// Same DMA, ordered against the MFMAs around it: the asm claims to rewrite the
// A fragments `before` (read by the MFMAs that must be issued first) and
// `after` (read by the MFMAs that must follow).  The registers are not
// touched; the claim only fixes the issue order, so that the DMA issue
// happens while the matrix pipe is busy.
__device__ __forceinline__ void dma16_between(const uint8_t* base, uint32_t voff, uint32_t lds, i32x8& before,
                                              i32x8& after) {
    asm volatile("s_mov_b32 m0, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3"
                 : "+v"(before), "+v"(after)
                 : "v"(voff), "s"(base), "s"(lds)
                 : "memory", "m0");
}

// 4-byte variant (global_load_lds_dword): lane i writes [lds + 4 i, lds + 4 i + 4).
__device__ __forceinline__ void dma4(const uint8_t* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N vector-memory operations of this wave are in flight
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Pin the accumulators at this point of the program: the matrix ops that
// produce them cannot be moved past it (in particular not past the next
// barrier, which would leave that wait without work to hide it).
__device__ __forceinline__ void pin_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) asm volatile("" ::"a"(acc[i][j]));
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) { return (uint32_t)(uintptr_t)(lds_t*)p; }

// Direct-to-LDS loads of one 64-wide K stage: this wave's 64 rows of A and
// of B, 4 instructions each (16 rows x 64 bytes per instruction).  abase and
// bbase are the (uniform) addresses of the tile's first rows at column k.
constexpr int kDmaPerStage = 8;  // vector-memory instructions per wave per stage
__device__ __forceinline__ void issue_stage(const uint8_t* abase, const uint8_t* bbase, const uint32_t (&aoffs)[4],
                                            const uint32_t (&boffs)[4], int buf, int w) {
    const uint32_t a0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_a[buf]) + w * 64 * TK);
    const uint32_t b0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_b[buf]) + w * 64 * TK);
    const uint8_t* ab = uniform_ptr(abase);
    const uint8_t* bb = uniform_ptr(bbase);
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(ab, aoffs[j], a0 + j * 16 * TK);
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(bb, boffs[j], b0 + j * 16 * TK);
}

// Scale dwords of one 256-wide chunk into LDS buffer `par`: the tile's 8 A
// and 8 B 32-row units (256 bytes = one dword per lane each); this wave
// loads units 2w and 2w + 1 of both.  sbase/tbase are the packed scale
// arrays at the chunk, soff/toff this lane's offsets for the two units.
constexpr int kScaleDma = 4;  // vector-memory instructions per wave per chunk
__device__ __forceinline__ void issue_scales(const uint8_t* sbase, const uint8_t* tbase, const uint32_t (&soff)[2],
                                             const uint32_t (&toff)[2], int par, int w) {
    const uint8_t* sb = uniform_ptr(sbase);
    const uint8_t* tb = uniform_ptr(tbase);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        dma4(sb, soff[u], __builtin_amdgcn_readfirstlane(lds_addr((const uint8_t*)lds_sa[par][2 * w + u])));
        dma4(tb, toff[u], __builtin_amdgcn_readfirstlane(lds_addr((const uint8_t*)lds_sb[par][2 * w + u])));
    }
}

// Fragments of one 64-wide K step for this wave: 4 A and 4 B blocks, each
// lane holding 32 bytes of its row (granules h and 2 + h: bytes 0-15 of every
// lane are the instruction's first 32-wide K block, bytes 16-31 its second).
struct Frags {
    i32x8 a[4], b[4];
};

__device__ __forceinline__ void read_frags(int buf, const int (&aoff)[4], const int (&boff)[4], const int (&ga0)[4],
                                           const int (&ga1)[4], const int (&gb0)[4], const int (&gb1)[4], Frags& F) {
    const uint8_t* la = lds_a[buf];
    const uint8_t* lb = lds_b[buf];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 lo = *reinterpret_cast<const uint4*>(la + aoff[i] + ga0[i]);
        const uint4 hi = *reinterpret_cast<const uint4*>(la + aoff[i] + ga1[i]);
        F.a[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 lo = *reinterpret_cast<const uint4*>(lb + boff[j] + gb0[j]);
        const uint4 hi = *reinterpret_cast<const uint4*>(lb + boff[j] + gb1[j]);
        F.b[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
}

// Ask the scheduler to interleave the next step's 16 fragment reads with the
// first MFMAs of this step (4 reads, 1 MFMA, ...), so that the reads are in
// flight early and done by the next barrier.
__device__ __forceinline__ void interleave_reads_with_mfma() {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);
}

// 16 scaled MFMAs of one K step, scale byte OPSEL of each lane's dwords, in
// 4 groups (one A block each), with the 8 DMA instructions of a stage (A rows
// of this wave's share, then B) issued two after each group, while the
// matrix pipe works on that group.  The DMA is unconditional (no branch that
// would let the compiler reorder the groups): at the end of the contraction
// the caller points it at a stage that is already resident, reloading it
// into the buffer that stage occupies.
template <int OPSEL>
__device__ __forceinline__ void mfma_step(Frags& F, const uint32_t (&sa)[4], const uint32_t (&sb)[4],
                                          f32x16 (&acc)[4][4], const uint8_t* an, const uint8_t* bn, int nbuf,
                                          const uint32_t (&aoffs)[4], const uint32_t (&boffs)[4], int w) {
    const uint32_t a0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_a[nbuf]) + w * 64 * TK);
    const uint32_t b0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_b[nbuf]) + w * 64 * TK);
    const uint8_t* ab = uniform_ptr(an);
    const uint8_t* bb = uniform_ptr(bn);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            // B (weight) rows as the instruction's rows and A (token) rows as its
            // columns: each lane then holds 4 consecutive output columns of one
            // output row (see the epilogue)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.b[j], F.a[i], acc[i][j], 0, 0, OPSEL,
                                                                       (int)sb[j], OPSEL, (int)sa[i]);
        i32x8& nxt = F.a[i < 3 ? i + 1 : i];
        if (i < 2) {
            dma16_between(ab, aoffs[2 * i], a0 + (2 * i) * 16 * TK, F.a[i], nxt);
            dma16_between(ab, aoffs[2 * i + 1], a0 + (2 * i + 1) * 16 * TK, F.a[i], nxt);
        } else {
            dma16_between(bb, boffs[2 * i - 4], b0 + (2 * i - 4) * 16 * TK, F.a[i], nxt);
            dma16_between(bb, boffs[2 * i - 3], b0 + (2 * i - 3) * 16 * TK, F.a[i], nxt);
        }
    }
}

__device__ __forceinline__ void run_tile_impl(const Tile& T) {
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int l = t & 63;
    const int wm = w >> 1, wn = w & 1;
    const int h = l >> 5, r32 = l & 31;

    // Tile bases (uniform) and per-lane 32-bit row offsets for the DMA.
    // Rows past the operand's limit read its last row instead; their
    // results are dropped by the epilogue.
    const uint8_t* abase = T.A + T.a_row0 * T.lda;
    const uint8_t* bbase = T.B + T.b_row0 * T.ldb;
    uint32_t aoffs[4], boffs[4];
    {
        const int64_t alast = T.a_lim - 1 - T.a_row0, blast = T.b_lim - 1 - T.b_row0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = w * 64 + j * 16 + (l >> 2);        // tile row written by this lane
            const int gran = ((l & 3) ^ swz(rr)) * 16;       // logical granule stored at physical l%4
            aoffs[j] = (uint32_t)((rr < alast ? rr : alast) * T.lda + gran);
            boffs[j] = (uint32_t)((rr < blast ? rr : blast) * T.ldb + gran);
        }
    }
    // fragment rows in LDS and the physical granules of this lane's two
    // 16-byte pieces (logical granules h and 2 + h)
    int aoff[4], boff[4], ga0[4], ga1[4], gb0[4], gb1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ra = wm * 128 + i * 32 + r32, rb = wn * 128 + i * 32 + r32;
        aoff[i] = ra * TK;
        boff[i] = rb * TK;
        ga0[i] = ((0 + h) ^ swz(ra)) * 16;
        ga1[i] = ((2 + h) ^ swz(ra)) * 16;
        gb0[i] = ((0 + h) ^ swz(rb)) * 16;
        gb1[i] = ((2 + h) ^ swz(rb)) * 16;
    }
    // scale offsets (chunk 0) of this lane for the units 2w, 2w + 1 it loads:
    // lane l carries row 32 u + l % 32 and K-block half l / 32
    uint32_t soff[2], toff[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t ra = clamp64(T.a_row0 + (2 * w + u) * 32 + r32, 0, T.a_lim - 1);
        const int64_t rb = clamp64(T.b_row0 + (2 * w + u) * 32 + r32, 0, T.b_lim - 1);
        soff[u] = (uint32_t)((ra >> 5) * T.a_unit + 4 * (32 * h + (ra & 31)));
        toff[u] = (uint32_t)((rb >> 5) * T.b_unit + 4 * (32 * h + (rb & 31)));
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int64_t nchunk = (T.k1 - T.k0) / 256;
    if (nchunk > 0) {
        // Pipeline over stages j (K bytes [k0 + 64 j, k0 + 64 j + 64), LDS
        // buffer j % 4; scales of chunk c in LDS buffer c % 2), with the
        // fragments of the current step already in registers:
        //   prologue: DMA scales(0), stages 0-3; wait for stage 0; read its
        //     fragments and the chunk-0 scales.
        //   step s: wait for stage s + 1; barrier (every wave is done reading
        //     stage s's buffer); DMA stage s + 4 into it (step 4c also DMAs
        //     scales(c + 1) first); read the fragments of stage s + 1 into
        //     the other register set; 16 MFMAs on stage s.
        // vmcnt bounds (operations issued after the stage waited for): 24 in
        // the prologue; 16, 20, 20, 16 at steps 4c .. 4c + 3; in the last
        // chunk (no scales, reload DMAs instead of new stages) 16, 16, 16 and
        // no wait at step 4c + 3.
        const uint8_t* As = T.As + (T.k0 / 256) * 256;
        const uint8_t* Bs = T.Bs + (T.k0 / 256) * 256;
        const uint8_t* ak = abase + T.k0;
        const uint8_t* bk = bbase + T.k0;
        uint32_t sa[4], sb[4], na[4], nb[4];
        Frags F0, F1;
        issue_scales(As, Bs, soff, toff, 0, w);
#pragma unroll
        for (int j = 0; j < 4; ++j) issue_stage(ak + j * TK, bk + j * TK, aoffs, boffs, j, w);
        wait_vm<3 * kDmaPerStage>();
        __syncthreads();
        read_frags(0, aoff, boff, ga0, ga1, gb0, gb1, F0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sa[i] = lds_sa[0][wm * 4 + i][l];
            sb[i] = lds_sb[0][wn * 4 + i][l];
        }
        for (int64_t c = 0; c < nchunk; ++c) {
            const bool last = c + 1 == nchunk;
            const int par = (int)(c & 1);
            const uint8_t* akc = ak + c * 256;
            const uint8_t* bkc = bk + c * 256;
            // stage fetched during step 4c + s: 4c + s + 4, or (last chunk) a
            // reload of stage 4c + s into the buffer it already occupies
            const int64_t ahead = last ? 0 : 4 * TK;
            // step 4c: stage 4c in F0
            wait_vm<2 * kDmaPerStage>();
            __syncthreads();
            read_frags(1, aoff, boff, ga0, ga1, gb0, gb1, F1);
            if (!last) issue_scales(As + (c + 1) * 256, Bs + (c + 1) * 256, soff, toff, par ^ 1, w);
            mfma_step<0>(F0, sa, sb, acc, akc + ahead, bkc + ahead, 0, aoffs, boffs, w);
            pin_acc(acc);
            // step 4c + 1: stage 4c + 1 in F1
            if (!last) wait_vm<2 * kDmaPerStage + kScaleDma>();
            else wait_vm<2 * kDmaPerStage>();
            __syncthreads();
            read_frags(2, aoff, boff, ga0, ga1, gb0, gb1, F0);
            mfma_step<1>(F1, sa, sb, acc, akc + TK + ahead, bkc + TK + ahead, 1, aoffs, boffs, w);
            pin_acc(acc);
            // step 4c + 2: stage 4c + 2 in F0
            if (!last) wait_vm<2 * kDmaPerStage + kScaleDma>();
            else wait_vm<2 * kDmaPerStage>();
            __syncthreads();
            read_frags(3, aoff, boff, ga0, ga1, gb0, gb1, F1);
            mfma_step<2>(F0, sa, sb, acc, akc + 2 * TK + ahead, bkc + 2 * TK + ahead, 2, aoffs, boffs, w);
            pin_acc(acc);
            // step 4c + 3: stage 4c + 3 in F1; fetch chunk c + 1's first
            // fragments and scales
            if (!last) {
                wait_vm<2 * kDmaPerStage>();
                __syncthreads();
                read_frags(0, aoff, boff, ga0, ga1, gb0, gb1, F0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    na[i] = lds_sa[par ^ 1][wm * 4 + i][l];
                    nb[i] = lds_sb[par ^ 1][wn * 4 + i][l];
                }
            }
            mfma_step<3>(F1, sa, sb, acc, akc + 3 * TK + ahead, bkc + 3 * TK + ahead, 3, aoffs, boffs, w);
            pin_acc(acc);
            if (!last) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sa[i] = na[i];
                    sb[i] = nb[i];
                }
            }
        }
    }
    // Epilogue.  acc[i][j] is the 32 x 32 block (A rows 32 i.., B rows 32 j..)
    // of this wave's 128 x 128 share, transposed by the operand order above:
    // lane l holds output row 32 i + l % 32 and, in element 4 q + u, output
    // column 32 j + 8 q + 4 (l / 32) + u -- four consecutive bf16 columns,
    // stored as one 8-byte write when the row pitch allows it.  The lane bases
    // are made opaque here so that the compiler does not hoist all the
    // row/address values out of the persistent tile loop.
    int rb = wm * 128 + r32;
    int cb = wn * 128 + 4 * h;
    uint32_t ldo = (uint32_t)T.ldo;
    asm volatile("" : "+v"(rb), "+v"(cb), "+s"(ldo));
    const bool vec = (ldo & 3) == 0 && (((uintptr_t)T.out) & 7) == 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = rb + i * 32;
        if (row >= T.rows) continue;
        uint16_t* const orow = T.out + (uint32_t)row * ldo;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = cb + j * 32 + q * 8;
                const __bf16 b0 = (__bf16)acc[i][j][4 * q + 0], b1 = (__bf16)acc[i][j][4 * q + 1];
                const __bf16 b2 = (__bf16)acc[i][j][4 * q + 2], b3 = (__bf16)acc[i][j][4 * q + 3];
                if (vec && col + 4 <= T.cols) {
                    const uint2 pk = make_uint2(
                        (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16),
                        (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16));
                    *reinterpret_cast<uint2*>(orow + col) = pk;
                } else {
                    if (col + 0 < T.cols) orow[col + 0] = __builtin_bit_cast(uint16_t, b0);
                    if (col + 1 < T.cols) orow[col + 1] = __builtin_bit_cast(uint16_t, b1);
                    if (col + 2 < T.cols) orow[col + 2] = __builtin_bit_cast(uint16_t, b2);
                    if (col + 3 < T.cols) orow[col + 3] = __builtin_bit_cast(uint16_t, b3);
                }
            }
    }
    // the next tile reuses the LDS buffers
    __syncthreads();
}

__device__ __forceinline__ void run_tile(const Tile& T) { run_tile_impl(T); }

__device__ __forceinline__ int64_t group_lo(const int32_t* off, int g, int64_t M) {
    return clamp64(off[g], 0, M);
}

__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(GemmArgs a) {
    const int t = threadIdx.x;
    const int nwg = gridDim.x;
    const int bid = blockIdx.x;
    // workgroup -> slot so that each XCD (bid % 8) owns a contiguous slot range
    const int slot = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;

    if (a.mode != 1) {
        const int64_t nN = (a.N + TN - 1) / TN;
        // per-group tile counts and their inclusive prefix (16 per thread)
        const int G = a.G;
        int32_t loc[16];
        int32_t sum = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int g = t * 16 + j;
            int32_t cnt = 0;
            if (g < G) {
                const int64_t lo = group_lo(a.offsets, g, a.M), hi = group_lo(a.offsets, g + 1, a.M);
                const int64_t mg = hi > lo ? hi - lo : 0;
                cnt = (int32_t)(((mg + TM - 1) / TM) * nN);
            }
            sum += cnt;
            loc[j] = sum;
        }
        __shared__ int32_t part[256];
        part[t] = sum;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {
            const int32_t v = t >= d ? part[t - d] : 0;
            __syncthreads();
            part[t] += v;
            __syncthreads();
        }
        const int32_t base = part[t] - sum;
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (t * 16 + j < G) tile_end[t * 16 + j] = base + loc[j];
        __syncthreads();
        const int32_t total = G > 0 ? tile_end[G - 1] : 0;

        for (int64_t tile = slot; tile < total; tile += nwg) {
            // group: first g with tile_end[g] > tile
            int lo = 0, hi = G - 1;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (tile_end[mid] > tile) hi = mid;
                else lo = mid + 1;
            }
            const int g = lo;
            const int64_t first = g > 0 ? tile_end[g - 1] : 0;
            const int64_t local = tile - first;
            const int64_t o0 = group_lo(a.offsets, g, a.M);
            const int64_t o1 = group_lo(a.offsets, g + 1, a.M);
            const int64_t mg = o1 - o0;
            const int64_t nM = (mg + TM - 1) / TM;
            const int64_t band = local / (kBand * nN);
            const int64_t gm = (nM - band * kBand) < kBand ? (nM - band * kBand) : kBand;
            const int64_t r = local - band * kBand * nN;
            const int64_t mt = band * kBand + r % gm;
            const int64_t nt = r / gm;

            Tile T;
            T.A = a.A;
            T.As = a.As;
            T.lda = a.K;
            T.a_unit = 32 * (a.K / 32);
            T.a_row0 = o0 + mt * TM;
            T.a_lim = o1;
            if (a.mode == 0) {
                // expert g's weights: rows [g N, g N + N) of the [G N][K] matrix
                T.B = a.B;
                T.Bs = a.Bs;
                T.ldb = a.K;
                T.b_unit = 32 * (a.K / 32);
                T.b_row0 = (int64_t)g * a.N + nt * TN;
                T.b_lim = (int64_t)g * a.N + a.N;
            } else {
                // transposed weights [N][ldb]: expert g is the column slice
                // [g K, g K + K), i.e. its contraction starts g K bytes (g K / 256
                // scale chunks) into every row
                T.B = a.B + (int64_t)g * a.K;
                T.Bs = a.Bs + ((int64_t)g * a.K / 256) * 256;
                T.ldb = a.ldb;
                T.b_unit = 32 * (a.ldb / 32);
                T.b_row0 = nt * TN;
                T.b_lim = a.N;
            }
            T.k0 = 0;
            T.k1 = a.K;
            T.out = a.out + (o0 + mt * TM) * a.N + nt * TN;
            T.ldo = a.N;
            T.rows = (int32_t)((mg - mt * TM) < TM ? (mg - mt * TM) : TM);
            T.cols = (int32_t)((a.N - nt * TN) < TN ? (a.N - nt * TN) : TN);
            run_tile(T);
        }
    } else {
        // wgrad: every group has the same tile grid over [N] x [K]
        const int64_t nMt = (a.N + TM - 1) / TM;
        const int64_t nNt = (a.K + TN - 1) / TN;
        const int64_t per = nMt * nNt;
        const int64_t total = per * a.G;
        for (int64_t tile = slot; tile < total; tile += nwg) {
            const int64_t g = tile / per;
            const int64_t local = tile - g * per;
            const int64_t band = local / (kBand * nNt);
            const int64_t gm = (nMt - band * kBand) < kBand ? (nMt - band * kBand) : kBand;
            const int64_t r = local - band * kBand * nNt;
            const int64_t mt = band * kBand + r % gm;
            const int64_t nt = r / gm;
            int64_t p0 = clamp64(a.offsets[g], 0, a.Mcap) & ~(int64_t)255;
            int64_t p1 = clamp64(a.offsets[g + 1], 0, a.Mcap) & ~(int64_t)255;
            if (p1 < p0) p1 = p0;

            Tile T;
            T.A = a.A;
            T.As = a.As;
            T.lda = a.Mcap;
            T.a_unit = 32 * (a.Mcap / 32);
            T.a_row0 = mt * TM;
            T.a_lim = a.N;
            T.B = a.B;
            T.Bs = a.Bs;
            T.ldb = a.Mcap;
            T.b_unit = 32 * (a.Mcap / 32);
            T.b_row0 = nt * TN;
            T.b_lim = a.K;
            T.k0 = p0;
            T.k1 = p1;
            T.out = a.out + g * a.N * a.K + mt * TM * a.K + nt * TN;
            T.ldo = a.K;
            T.rows = (int32_t)((a.N - mt * TM) < TM ? (a.N - mt * TM) : TM);
            T.cols = (int32_t)((a.K - nt * TN) < TN ? (a.K - nt * TN) : TN);
            run_tile(T);
        }
    }
}

int num_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

}  // namespace

hipError_t launch_grouped_gemm(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq,
                               const uint8_t* Ws, const int32_t* group_offsets, int32_t G, int64_t M,
                               int64_t N, int64_t K, uint16_t* out, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    GemmArgs a;
    a.A = Xq;
    a.As = Xs;
    a.B = Wq;
    a.Bs = Ws;
    a.offsets = group_offsets;
    a.out = out;
    a.M = M;
    a.N = N;
    a.K = K;
    a.Mcap = 0;
    a.G = G;
    a.mode = 0;
    a.ldb = 0;
    const int64_t ub = ((M + TM - 1) / TM + G) * ((N + TN - 1) / TN);
    int64_t nwg = num_cus();
    if (ub < nwg) nwg = ub;
    hipLaunchKernelGGL(grouped_gemm_kernel, dim3((unsigned)nwg), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm_dgrad(const uint8_t* dYq, const uint8_t* dYs, const uint8_t* WTq,
                                     const uint8_t* WTs, const int32_t* group_offsets, int32_t G, int64_t M,
                                     int64_t N, int64_t K, int64_t Wcap, uint16_t* dX, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    GemmArgs a;
    a.A = dYq;
    a.As = dYs;
    a.B = WTq;
    a.Bs = WTs;
    a.offsets = group_offsets;
    a.out = dX;
    a.M = M;
    a.N = N;
    a.K = K;
    a.Mcap = 0;
    a.G = G;
    a.mode = 2;
    a.ldb = Wcap;
    const int64_t ub = ((M + TM - 1) / TM + G) * ((N + TN - 1) / TN);
    int64_t nwg = num_cus();
    if (ub < nwg) nwg = ub;
    hipLaunchKernelGGL(grouped_gemm_kernel, dim3((unsigned)nwg), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm_wgrad(const uint8_t* A, const uint8_t* As, const uint8_t* B,
                                     const uint8_t* Bs, const int32_t* padded_offsets, int32_t G,
                                     int64_t N, int64_t K, int64_t Mcap, uint16_t* dW,
                                     hipStream_t stream) {
    if (N == 0 || K == 0 || G == 0) return hipSuccess;
    GemmArgs a;
    a.A = A;
    a.As = As;
    a.B = B;
    a.Bs = Bs;
    a.offsets = padded_offsets;
    a.out = dW;
    a.M = 0;
    a.N = N;
    a.K = K;
    a.Mcap = Mcap;
    a.G = G;
    a.mode = 1;
    a.ldb = 0;
    const int64_t total = ((N + TM - 1) / TM) * ((K + TN - 1) / TN) * G;
    int64_t nwg = num_cus();
    if (total < nwg) nwg = total;
    hipLaunchKernelGGL(grouped_gemm_kernel, dim3((unsigned)nwg), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mx
