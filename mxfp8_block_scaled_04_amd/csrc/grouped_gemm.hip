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
// Kernel: persistent workgroups of 4 waves, tile 256 x 256.
//  * Each wave owns a 128 x 128 sub-tile = 4 x 4 MFMA blocks; per 64-wide K
//    step a lane holds 16 bytes of each 32-wide K block for its row.
//  * fp8 operands reach LDS by direct buffer-to-LDS loads (no VGPR staging)
//    in stages of 128 K bytes: every load instruction moves 8 whole 128-byte
//    row segments (measured: 64-byte row pieces, 16 rows per instruction,
//    cost ~11% of the matrix throughput; full 128-byte lines cost nothing
//    measurable).  Two stage buffers (2 x 64 KB); the loads of stage s + 1
//    are issued during the second K step of stage s - 1, and one barrier per
//    stage both publishes a landed stage and frees the other buffer.
//  * Loads go through buffer descriptors whose range ends at the tile's
//    last valid row, so rows past a group's end read as zeros without any
//    per-lane clamping, and the per-lane offsets do not depend on the tile.
//  * The pipeline does not restart between tiles: the last chunk of a tile
//    already loads the next tile's first two stages and scales, and the
//    epilogue (bf16 conversion and 16-byte range-checked stores) runs while
//    they are in flight.
//  * Scale dwords go to LDS by the same 16-byte direct loads, 4 packed
//    32-row units per instruction, one 256-wide K chunk ahead, and are read
//    into registers once per chunk (measured: 1-2 % faster than one 4-byte
//    load per lane and unit, which also gathered each lane's dword; without
//    any scale loads the kernel would be 3-5 % faster).
//  * Tile order: expert-major; inside an expert, bands of 4 M-tiles walked
//    M-fastest; workgroups are mapped so that each XCD (workgroups are dealt
//    to the 8 XCDs round-robin) runs a contiguous range of tile ids and so
//    shares operands through its own L2.
#include "mx_device.h"
#include "mx_internal.h"
#include "mx_debug.h"

namespace mx {

namespace {

constexpr int TM = 256;
constexpr int TN = 256;
constexpr int TK = 64;     // K bytes per MFMA step
constexpr int SK = 128;    // K bytes per LDS stage (two MFMA steps)
constexpr int kBand = 4;   // M-tiles per band of the tile order

typedef __attribute__((address_space(3))) void lds_t;
typedef int i32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
    const uint8_t* A;
    const uint8_t* As;
    const uint8_t* B;
    const uint8_t* Bs;
    const int32_t* offsets;
    uint16_t* out;
    int64_t M, N, K, Mcap;
    int64_t a_scale_bytes, b_scale_bytes;  // sizes of the packed scale arrays
    int32_t G;
    int32_t mode;  // 0: rows of X grouped (forward); 1: contraction grouped (wgrad);
                   // 2: rows grouped, weights read transposed (dgrad)
    int64_t ldb;   // mode 2: row stride of the transposed weights (their Wcap)
    // quantizing SwiGLU epilogue (mode 0 only): hidden width I = N / 2, codes
    // hq [M][I] and packed scales hs (R = M, contraction I)
    uint8_t* hq;
    uint8_t* hs;
};

// Launch-wide constants of the operand layouts.
struct Layout {
    uint32_t lda, ldb;        // row strides (bytes) of the A and B data
    uint32_t a_unit, b_unit;  // bytes per 32-row unit of the packed scales
    uint32_t ldo;             // output row stride (elements)
};

// One output tile (all fields wave-uniform).
struct Tile {
    i32x4 ra, rb;    // A / B data descriptors: base at the tile's first row and first contraction byte
    i32x4 rsa, rsb;  // A / B packed-scale descriptors: base at the tile's first unit and chunk
    int32_t asub, bsub;  // first tile row modulo 32 (A, B)
    int32_t nchunk;      // 256-wide contraction chunks (0: no tile)
    int32_t rows, cols;  // valid part of the output tile
    int64_t outoff;      // element offset of the tile's output element (0, 0)
};

__shared__ __attribute__((aligned(16))) uint8_t lds_a[2][TM * SK];
__shared__ __attribute__((aligned(16))) uint8_t lds_b[2][TN * SK];
// Scale dwords of one 256-wide chunk, [chunk parity][packed 32-row unit][dword]:
// the packed units from the one holding the tile's first row on (9 of them
// when that row is not a multiple of 32; loaded 4 at a time, hence 12)
constexpr int kScaleUnits = 12;
__shared__ __attribute__((aligned(16))) uint32_t lds_sa[2][kScaleUnits][64];
__shared__ __attribute__((aligned(16))) uint32_t lds_sb[2][kScaleUnits][64];
__shared__ int32_t tile_end[kMaxGroups];  // inclusive prefix of tiles per group (position order)
// wgrad with at most kLptGroups groups: its tiles cost in proportion to their
// group's contraction length, so groups are taken longest first (lpt_order[k]
// = the group at position k) and workgroups take the tiles of successive
// rounds in alternating directions, which balances the per-workgroup sums
constexpr int kLptGroups = 256;
__shared__ int32_t lpt_order[kLptGroups];

__device__ __forceinline__ bool lpt_mode(const GemmArgs& a) { return a.mode == 1 && a.G <= kLptGroups; }

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

// Stage rows are 128 bytes (8 granules of 16 B).  Granule c of tile row r is
// stored at position c ^ swz(r).  Measured on gfx950: a 64-lane ds_read_b128
// is served in 4 passes of 16 lanes (256 bytes per clock), the lanes of a
// pass having row indices that differ in bits 0, 1, 3 and in bit 2 tied to
// bit 4.  With 128-byte rows the 16-byte bank group of a read is
// 8 (r mod 2) + physical granule; XORing the granule with row bits 1-3 makes
// the 16 groups of every pass distinct.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Raw buffer descriptor over [base, base + bytes): loads past the range
// return zeros, stores past it are dropped (checked on the full offset,
// including the scalar offset).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r[0] = (int)uni((uint32_t)p);
    r[1] = (int)uni((uint32_t)(p >> 32) & 0xFFFFu);  // stride 0, no swizzle
    r[2] = (int)uni(bytes);
    r[3] = (int)uni(0x00020000u);
    return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_t*)p; }

// Direct buffer->LDS loads.  Issued as inline asm so that the compiler's own
// wait insertion does not stall every later LDS read on them; completion is
// enforced explicitly (wait_vm<N> + barrier) before a buffer is read.  M0 is
// only written here; nothing else in these kernels reads it.
//
// bdma16: 16 bytes per lane (lane i writes LDS [lds + 16 i, lds + 16 i + 16)).
// The asm claims to rewrite the fragments `before` (read by the MFMA that
// must be issued first) and `after` (read by the MFMA that must follow); the
// registers are not touched, the claim only fixes the issue order so that
// the load issue happens while the matrix pipe is busy.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// The scalar offset `so` and LDS address `lb` advance by `ld8` (8 rows) and
// 8 * 128 bytes after every load, inside the asm, so that the compiler does
// not precompute and hold the 8 offsets of a stage in scalar registers.
__device__ __forceinline__ void bdma16_run(const i32x4& rs, uint32_t voff, uint32_t& so, uint32_t& lb, uint32_t ld8,
                                           i32x8& before, i32x8& after) {
    asm volatile(
        "s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %4, %5, %2 offen lds\n\t"
        "s_add_u32 %2, %2, %6\n\ts_add_u32 %3, %3, 0x400"
        : "+v"(before), "+v"(after), "+s"(so), "+s"(lb)
        : "v"(voff), "s"(rs), "s"(ld8)
        : "memory", "m0", "scc");
}
__device__ __forceinline__ void bdma16_run_after(const i32x4& rs, uint32_t voff, uint32_t& so, uint32_t& lb,
                                                 uint32_t ld8, i32x8& before) {
    asm volatile(
        "s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %3, %4, %1 offen lds\n\t"
        "s_add_u32 %1, %1, %5\n\ts_add_u32 %2, %2, 0x400"
        : "+v"(before), "+s"(so), "+s"(lb)
        : "v"(voff), "s"(rs), "s"(ld8)
        : "memory", "m0", "scc");
}
__device__ __forceinline__ void bdma16_plain(const i32x4& rs, uint32_t voff, uint32_t soff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rs),
                 "s"(soff), "s"(lds)
                 : "memory", "m0");
}
// Ordering point with no instruction: keeps the LDS reads of an MFMA group
// between its neighbours (memory clobber) and the groups in order (fake
// fragment dependencies, as above).
__device__ __forceinline__ void order_between(i32x8& before, i32x8& after) {
    asm volatile("" : "+v"(before), "+v"(after) : : "memory");
}
#pragma clang diagnostic pop

// Range-checked stores go through the compiler's buffer-store builtins, never
// inline asm: a store of more than 8 bytes reads its data registers after it
// issues, and on gfx950 a vector ALU op may overwrite them only two wait
// states later.  The compiler's hazard recognizer inserts those wait states
// for stores it can see, not for stores hidden in an asm statement (a
// 16-byte asm store whose data registers were rewritten by the next
// instruction stored partly stale data).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t store_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void bstore16(rsrc_t rs, uint32_t voff, i32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)voff, 0, 0);
}

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

// Per-lane constants of the load and read patterns (independent of the tile).
struct Lane {
    uint32_t va[2], vb[2];  // load offsets for instructions of even / odd index j
    int fo[4];              // fragment read offsets (A lo, A hi, B lo, B hi) of K half 0
};

// One stage = 128 K bytes of the tile's 256 A rows and 256 B rows.  Wave w
// loads rows [64 w, 64 w + 64) of both, 8 instructions each; instruction j
// covers rows 64 w + 8 j + l / 8, lane l holding physical granule l % 8.
struct StageDma {
    i32x4 ra, rb;
    uint32_t soff;    // contraction byte of the stage
    uint32_t la, lb;  // LDS addresses of this wave's first row in the target buffer
};

// Packed-scale loads of one 256-wide chunk: the 256-byte chunks of the 8
// packed 32-row units (9 when the tile's first row is not a multiple of 32)
// from the unit holding the tile's first row, by 16-byte direct loads of 4
// units each (lane l: unit l / 16, bytes 16 (l % 16) of its chunk, so the 4
// chunks land contiguously in LDS): waves 0 and 1 load A units 0-3 and 4-7,
// waves 2 and 3 B units 0-3 and 4-7, waves 0 / 1 also A / B units 8-11 when
// needed.  Units past the end of a scale array read as zeros (no valid row
// uses them).
__device__ __forceinline__ void issue_scales(const i32x4& rsa, const i32x4& rsb, int asub, int bsub,
                                             uint32_t choff, int par, int w, int l, const Layout& L) {
    const uint32_t ua = (uint32_t)(l >> 4) * L.a_unit + (uint32_t)(l & 15) * 16u;
    const uint32_t ub = (uint32_t)(l >> 4) * L.b_unit + (uint32_t)(l & 15) * 16u;
    if (w < 2)
        bdma16_plain(rsa, ua + 4u * (uint32_t)w * L.a_unit, choff, uni(lds_addr(lds_sa[par][4 * w])));
    else
        bdma16_plain(rsb, ub + 4u * (uint32_t)(w - 2) * L.b_unit, choff, uni(lds_addr(lds_sb[par][4 * (w - 2)])));
    if (w == 0 && asub != 0) bdma16_plain(rsa, ua + 8u * L.a_unit, choff, uni(lds_addr(lds_sa[par][8])));
    if (w == 1 && bsub != 0) bdma16_plain(rsb, ub + 8u * L.b_unit, choff, uni(lds_addr(lds_sb[par][8])));
}

// Scale dword of MFMA row block `blk` (tile rows 32 blk .. 32 blk + 31) for
// lane (h, r32): tile row 32 blk + r32 is row sub + 32 blk + r32 of the
// loaded units, whose dword for K-block half h is 32 h + (row % 32).
__device__ __forceinline__ uint32_t read_scale(const uint32_t (&s)[kScaleUnits][64], int sub, int blk, int h,
                                               int r32) {
    const int r = sub + r32;
    return s[blk + (r >> 5)][32 * h + (r & 31)];
}
constexpr int kStageDma = 16;  // vector-memory instructions per wave per stage

__device__ __forceinline__ void issue_stage_plain(const StageDma& S, const Lane& Ln, const Layout& L) {
#pragma unroll
    for (int j = 0; j < 8; ++j) bdma16_plain(S.ra, Ln.va[j & 1], S.soff + j * 8 * L.lda, S.la + j * 8 * SK);
#pragma unroll
    for (int j = 0; j < 8; ++j) bdma16_plain(S.rb, Ln.vb[j & 1], S.soff + j * 8 * L.ldb, S.lb + j * 8 * SK);
}

// Fragments of one 64-wide K step: 4 A and 4 B blocks, each lane holding 32
// bytes of its row (granules h and 2 + h of the step: bytes 0-15 of every
// lane are the instruction's first 32-wide K block, bytes 16-31 its second).
struct Frags {
    i32x8 a[4], b[4];
};

__device__ __forceinline__ i32x8 lds_frag(const uint8_t* base, int lo, int hi) {
    const uint4 x = *reinterpret_cast<const uint4*>(base + lo);
    const uint4 y = *reinterpret_cast<const uint4*>(base + hi);
    return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}

// Fragment reads of K half `half` (0: stage bytes 0-63, 1: 64-127) of
// buffer `buf`: granule g of half 1 is granule g + 4 of the row, i.e. the
// physical offset XOR 64.
__device__ __forceinline__ void read_frags(int buf, int half, const Lane& Ln, Frags& F) {
    const int x = half ? 64 : 0;
    const uint8_t* la = lds_a[buf];
    const uint8_t* lb = lds_b[buf];
#pragma unroll
    for (int i = 0; i < 4; ++i) F.a[i] = lds_frag(la + i * 32 * SK, Ln.fo[0] ^ x, Ln.fo[1] ^ x);
#pragma unroll
    for (int j = 0; j < 4; ++j) F.b[j] = lds_frag(lb + j * 32 * SK, Ln.fo[2] ^ x, Ln.fo[3] ^ x);
}

// One 64-wide K step: 16 scaled MFMAs on the fragments F (scale byte OPSEL
// of each lane's scale dwords), in 4 groups of one A block each.  After
// group i the step reads block i of A and of B of the next step (buffer
// rbuf, K half rhalf) into Fn, so that the four waves, which leave a barrier
// together, do not all queue their 16 KB of LDS reads at once while the
// matrix pipe idles.  With DMA, the step also issues the 16 loads of a stage
// (A rows, then B rows), one after each MFMA, so that a load whose issue
// waits for room in the memory pipeline has a whole matrix op to hide
// behind (measured: 2-4% faster than four loads after every fourth MFMA);
// without, an empty ordering point keeps the group shape.  The fake operand
// dependencies of the loads pin each one between two consecutive MFMAs.
template <int OPSEL, bool DMA>
__device__ __forceinline__ void mfma_step(Frags& F, Frags& Fn, int rbuf, int rhalf, const Lane& Ln,
                                          const uint32_t (&sa)[4], const uint32_t (&sb)[4], f32x16 (&acc)[4][4],
                                          const StageDma& S, const Layout& L) {
    const int x = rhalf ? 64 : 0;
    const uint8_t* la = lds_a[rbuf];
    const uint8_t* lb = lds_b[rbuf];
    uint32_t soa = S.soff, sob = S.soff, lba = S.la, lbb = S.lb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // B (weight) rows as the instruction's rows and A (token) rows as its
            // columns: each lane then holds 4 consecutive output columns of one
            // output row (see the epilogue)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.b[j], F.a[i], acc[i][j], 0, 0, OPSEL,
                                                                       (int)sb[j], OPSEL, (int)sa[i]);
            if (DMA) {
                // load 4 i + j: A rows for i < 2, then B rows
                const bool isb = i >= 2;
                const i32x4& rs = isb ? S.rb : S.ra;
                uint32_t& so = isb ? sob : soa;
                uint32_t& lbr = isb ? lbb : lba;
                const uint32_t ld8 = isb ? L.ldb * 8u : L.lda * 8u;
                const uint32_t v = isb ? Ln.vb[j & 1] : Ln.va[j & 1];
                if (j < 3)
                    bdma16_run(rs, v, so, lbr, ld8, F.b[j], F.b[j + 1]);
                else if (i < 3)
                    bdma16_run(rs, v, so, lbr, ld8, F.b[j], F.a[i + 1]);
                else
                    bdma16_run_after(rs, v, so, lbr, ld8, F.b[j]);
            }
        }
        Fn.a[i] = lds_frag(la + i * 32 * SK, Ln.fo[0] ^ x, Ln.fo[1] ^ x);
        Fn.b[i] = lds_frag(lb + i * 32 * SK, Ln.fo[2] ^ x, Ln.fo[3] ^ x);
        if (!DMA && i < 3) order_between(F.a[i], F.a[i + 1]);
    }
}

// Loads issued during a chunk: the scales of the following chunk and the two
// following stages (of this tile, or of the next one in a tile's last chunk).
struct Ahead {
    i32x4 ra, rb, rsa, rsb;
    int32_t asub, bsub;
    uint32_t choff;         // contraction offset (bytes) of the scale chunk
    uint32_t soff2, soff3;  // contraction offsets of the two stages
};

// Pipeline state carried from step to step.
struct Pipe {
    Frags F0, F1;          // fragments of the current / next step
    uint32_t sa[4], sb[4];  // scale dwords of the current chunk
    int gpar;              // scale parity of the current chunk
};

// One 256-wide contraction chunk = K steps 4c .. 4c + 3 = stages 2c (buffer
// 0) and 2c + 1 (buffer 1).  Step s multiplies the fragments read during
// step s - 1 and reads those of step s + 1:
//   4c     F0 x, read F1 <- buffer 0 half 1
//   4c + 1 wait for stage 2c + 1, barrier; F1 x, read F0 <- buffer 1 half 0;
//          load the scales of the next chunk and stage 2c + 2 (buffer 0)
//   4c + 2 F0 x, read F1 <- buffer 1 half 1
//   4c + 3 wait for stage 2c + 2 and the scales, barrier; F1 x, read F0 <-
//          buffer 0 half 0 and the next chunk's scales; load stage 2c + 3
//          (buffer 1)
// The barrier at 4c + 1 also frees buffer 0 (last read at step 4c), the one
// at 4c + 3 buffer 1 (last read at 4c + 2).  vmcnt bounds: at 4c + 1 nothing
// was issued after stage 2c + 1, except the 32 epilogue stores of the
// previous tile (after_epilogue; EPI_STORES of them); at 4c + 3 nothing after
// stage 2c + 2.
template <int EPI_STORES>
__device__ __forceinline__ void run_chunk(Pipe& P, f32x16 (&acc)[4][4], const Ahead& X, bool after_epilogue,
                                          const Lane& Ln, const Layout& L, int w, int l, int wm, int wn,
                                          uint32_t la0, uint32_t la1, uint32_t lb0, uint32_t lb1) {
    const StageDma S2{X.ra, X.rb, X.soff2, la0, lb0};
    const StageDma S3{X.ra, X.rb, X.soff3, la1, lb1};
    // step 4c
    mfma_step<0, false>(P.F0, P.F1, 0, 1, Ln, P.sa, P.sb, acc, S2, L);
    pin_acc(acc);
    // step 4c + 1
    if (after_epilogue) wait_vm<EPI_STORES>();
    else wait_vm<0>();
    __syncthreads();
    issue_scales(X.rsa, X.rsb, X.asub, X.bsub, X.choff, P.gpar ^ 1, w, l, L);
    mfma_step<1, true>(P.F1, P.F0, 1, 0, Ln, P.sa, P.sb, acc, S2, L);
    pin_acc(acc);
    // step 4c + 2
    mfma_step<2, false>(P.F0, P.F1, 1, 1, Ln, P.sa, P.sb, acc, S3, L);
    pin_acc(acc);
    // step 4c + 3
    wait_vm<0>();
    __syncthreads();
    mfma_step<3, true>(P.F1, P.F0, 0, 0, Ln, P.sa, P.sb, acc, S3, L);
    uint32_t na[4], nb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        na[i] = read_scale(lds_sa[P.gpar ^ 1], X.asub, wm * 4 + i, l >> 5, l & 31);
        nb[i] = read_scale(lds_sb[P.gpar ^ 1], X.bsub, wn * 4 + i, l >> 5, l & 31);
    }
    pin_acc(acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        P.sa[i] = na[i];
        P.sb[i] = nb[i];
    }
    P.gpar ^= 1;
}

__device__ __forceinline__ int64_t group_lo(const int32_t* off, int g, int64_t M) {
    return clamp64(off[g], 0, M);
}

// Output tile of tile id `tile` (nchunk = 0 and empty descriptors when
// tile >= total).  `g` is a search cursor: the tile ids a workgroup visits
// increase, so the group of the next tile is found by walking forward from
// the current one.
template <int EPI>
__device__ __forceinline__ Tile decode_tile(const GemmArgs& a, const Layout& L, int64_t tile, int64_t total,
                                            int& g) {
    Tile T;
    if (tile >= total) {
        T.ra = T.rb = T.rsa = T.rsb = make_rsrc(a.A, 0);
        T.asub = T.bsub = 0;
        T.nchunk = 0;
        T.rows = T.cols = 0;
        T.outoff = 0;
        return T;
    }
    while (tile_end[g] <= tile) ++g;
    g = (int)uni((uint32_t)g);
    const int64_t first = g > 0 ? tile_end[g - 1] : 0;
    const int64_t local = tile - first;
    const int grp = (int)uni((uint32_t)(lpt_mode(a) ? lpt_order[g] : g));  // g: position in tile order
    const uint8_t *B0, *Bs0;
    int64_t arows, brows, k0, k1, arow0, brow0;
    if (a.mode != 1) {
        const int64_t nN = (a.N + TN - 1) / TN;
        const int64_t o0 = group_lo(a.offsets, g, a.M);
        const int64_t o1 = group_lo(a.offsets, g + 1, a.M);
        const int64_t mg = o1 - o0;
        const int64_t nM = (mg + TM - 1) / TM;
        const int64_t band = local / (kBand * nN);
        const int64_t gm = (nM - band * kBand) < kBand ? (nM - band * kBand) : kBand;
        const int64_t r = local - band * kBand * nN;
        const int64_t mt = band * kBand + r % gm;
        const int64_t nt = r / gm;
        arow0 = o0 + mt * TM;
        arows = o1 - arow0;
        debug_flag(arows <= 0, kDbgTile);
        k0 = 0;
        k1 = a.K;
        if (a.mode == 0) {
            // expert g's weights: rows [g N, g N + N) of the [G N][K] matrix
            brow0 = (int64_t)g * a.N + nt * TN;
            brows = a.N - nt * TN;
            B0 = a.B;
            Bs0 = a.Bs;
        } else {
            // transposed weights [N][ldb]: expert g is the column slice
            // [g K, g K + K), i.e. its contraction starts g K bytes (g K / 256
            // scale chunks) into every row
            brow0 = nt * TN;
            brows = a.N - brow0;
            B0 = a.B + (int64_t)g * a.K;
            Bs0 = a.Bs + ((int64_t)g * a.K / 256) * 256;
        }
        // the SwiGLU epilogues need the tile's first row and column tile
        // apart (no 64-bit division in the kernel): they get them packed
        T.outoff = EPI != 0 ? (arow0 << 24) + nt : arow0 * a.N + nt * TN;
        T.rows = (int32_t)(arows < TM ? arows : TM);
        T.cols = (int32_t)((a.N - nt * TN) < TN ? (a.N - nt * TN) : TN);
    } else {
        // wgrad: every non-empty group has the same tile grid over [N] x [K]
        const int64_t nMt = (a.N + TM - 1) / TM;
        const int64_t nNt = (a.K + TN - 1) / TN;
        const int64_t band = local / (kBand * nNt);
        const int64_t gm = (nMt - band * kBand) < kBand ? (nMt - band * kBand) : kBand;
        const int64_t r = local - band * kBand * nNt;
        const int64_t mt = band * kBand + r % gm;
        const int64_t nt = r / gm;
        k0 = clamp64(a.offsets[grp], 0, a.Mcap) & ~(int64_t)255;
        k1 = clamp64(a.offsets[grp + 1], 0, a.Mcap) & ~(int64_t)255;
        if (k1 < k0) k1 = k0;
        arow0 = mt * TM;
        arows = a.N - arow0;
        brow0 = nt * TN;
        brows = a.K - brow0;
        B0 = a.B;
        Bs0 = a.Bs;
        T.outoff = (int64_t)grp * a.N * a.K + arow0 * a.K + nt * TN;
        T.rows = (int32_t)(arows < TM ? arows : TM);
        T.cols = (int32_t)(brows < TN ? brows : TN);
    }
    const int64_t aso = (arow0 >> 5) * (int64_t)L.a_unit + (k0 / 256) * 256;
    const int64_t bso = (Bs0 - a.Bs) + (brow0 >> 5) * (int64_t)L.b_unit + (k0 / 256) * 256;
    const int64_t ar = arows < TM ? arows : TM, br = brows < TN ? brows : TN;
    T.ra = make_rsrc(a.A + arow0 * (int64_t)L.lda + k0, (uint32_t)(ar * L.lda));
    T.rb = make_rsrc(B0 + brow0 * (int64_t)L.ldb + k0, (uint32_t)(br * L.ldb));
    T.rsa = make_rsrc(a.As + aso, (uint32_t)(a.a_scale_bytes - aso));
    T.rsb = make_rsrc(a.Bs + bso, (uint32_t)(a.b_scale_bytes - bso));
    T.asub = (int32_t)(arow0 & 31);
    T.bsub = (int32_t)(brow0 & 31);
    T.nchunk = (int32_t)((k1 - k0) / 256);
    return T;
}

// Epilogue.  acc[i][j] is the 32 x 32 block (A rows 32 i.., B rows 32 j..)
// of this wave's 128 x 128 share, transposed by the operand order of the
// MFMAs: lane l holds output row 32 i + l % 32 and, in element 4 q + u,
// output column 32 j + 8 q + 4 (l / 32) + u.  v_permlane32_swap gathers 8
// consecutive columns per lane (lanes 0-31 columns 16 p + 0..7, lanes 32-63
// 16 p + 8..15 for q = 2p, 2p + 1), stored with one 16-byte range-checked
// store: rows past the tile's valid rows fall outside the descriptor and
// columns past its valid columns get an offset outside it, so every wave
// issues exactly 32 stores (the wait accounting of the next tile counts on
// it).  Requires ldo % 8 == 0 (16-byte aligned rows).
__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)y) << 16);
}

// Row blocks [I0, I1) of the wave's share (all four by default).
template <int I0 = 0, int I1 = 4>
__device__ __forceinline__ void epilogue16(uint16_t* out, const Tile& T, const Layout& L, f32x16 (&acc)[4][4], int wm,
                                           int wn, int h, int r32) {
    const rsrc_t ro = store_rsrc(out, (uint32_t)T.rows * L.ldo * 2u);
#pragma unroll
    for (int i = I0; i < I1; ++i) {
        const uint32_t rowoff = (uint32_t)(wm * 128 + i * 32 + r32) * L.ldo * 2u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int q0 = 2 * p, q1 = 2 * p + 1;
                const uint32_t x0 = pack_bf16x2(acc[i][j][4 * q0 + 0], acc[i][j][4 * q0 + 1]);
                const uint32_t y0 = pack_bf16x2(acc[i][j][4 * q0 + 2], acc[i][j][4 * q0 + 3]);
                const uint32_t x1 = pack_bf16x2(acc[i][j][4 * q1 + 0], acc[i][j][4 * q1 + 1]);
                const uint32_t y1 = pack_bf16x2(acc[i][j][4 * q1 + 2], acc[i][j][4 * q1 + 3]);
                const auto sx = __builtin_amdgcn_permlane32_swap(x0, x1, false, false);
                const auto sy = __builtin_amdgcn_permlane32_swap(y0, y1, false, false);
                const int col = wn * 128 + j * 32 + 16 * p + 8 * h;
                const uint32_t off = col < T.cols ? rowoff + (uint32_t)col * 2u : 0xFFFFFFF0u;
                bstore16(ro, off, i32x4{(int)sx[0], (int)sy[0], (int)sx[1], (int)sy[1]});
            }
    }
}

// Quantizing SwiGLU epilogue (gate+up projection followed by SwiGLU and the
// MXFP8 quantization of its result for the down projection: kucoin.com MoK
// page, section 02, on fusing MXFP8 into the SwiGLU step; aigc.bar
// "被忽视的量化税").
// The weight rows of each expert alternate 32-row gate and up blocks, so the
// tile's MFMA blocks 2jj and 2jj + 1 of a wave are the gate and up values of
// the same 32 hidden units and each lane holds both for its row and 16 of
// the 32 columns (the other 16 are in lane l ^ 32):
//   h = silu(gate) * up = gate * rcp(1 + exp(-gate)) * up       (fp32;
//   hardware exp2 and reciprocal, each within about one ulp)
// then per row and 32 hidden units (one block along the contraction of the
// down projection): amax over both lanes, S = max(expfield(amax) - 8, 0)
// (the same rule as the quantize kernels, on the fp32 exponent field),
// codes = E4M3(clamp(h * 2^(127 - S), +-448)), round to nearest even.
// Per wave: 32 four-byte code stores and 8 one-byte scale stores, all
// issued (rows past the tile and the half of the lanes that does not own
// the scale get offsets outside the descriptors).
constexpr int kSwigluStores = 40;

__device__ __forceinline__ float silu(float x) {
    return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.44269504088896341f));
}

__device__ __forceinline__ void bstore4(rsrc_t rs, uint32_t voff, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b32(v, rs, (int)voff, 0, 0);
}
__device__ __forceinline__ void bstore1(rsrc_t rs, uint32_t voff, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, rs, (int)voff, 0, 0);
}

template <int I0 = 0, int I1 = 4>
__device__ __forceinline__ void epilogue_swiglu(const GemmArgs& a, const Tile& T, f32x16 (&acc)[4][4], int wm, int wn,
                                                int h, int r32) {
    const int64_t I = a.N / 2;
    const int64_t KBh = 8 * ((I + 255) / 256);
    // the tile's first row and first hidden column (column tile nt covers
    // hidden columns [128 nt, 128 nt + 128))
    const int64_t row0 = T.outoff >> 24;
    const int64_t hcol0 = (T.outoff & 0xFFFFFF) * (TN / 2);
    const rsrc_t rq = store_rsrc(a.hq + row0 * I + hcol0, (uint32_t)((int64_t)T.rows * I));
    const int64_t hs_bytes = ((a.M + 31) / 32) * 32 * KBh;
    const rsrc_t rsc = store_rsrc(a.hs, (uint32_t)hs_bytes);
#pragma unroll
    for (int i = I0; i < I1; ++i) {
        const int row = wm * 128 + i * 32 + r32;
        const int64_t grow = row0 + row;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            float hv[16];
            float m = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                hv[e] = silu(acc[i][2 * jj][e]) * acc[i][2 * jj + 1][e];
                m = __builtin_fmaxf(m, __builtin_fabsf(hv[e]));
            }
            {
                // amax over the 32 columns: lanes l and l ^ 32 hold the two halves
                const auto pm = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, m),
                                                                  __builtin_bit_cast(uint32_t, m), false, false);
                m = __builtin_fmaxf(__builtin_bit_cast(float, (uint32_t)pm[0]),
                                    __builtin_bit_cast(float, (uint32_t)pm[1]));
            }
            const int E = (int)((__builtin_bit_cast(uint32_t, m) >> 23) & 0xFF);
            const uint32_t S = (uint32_t)(E > 8 ? E - 8 : 0);
            const float sc = __builtin_bit_cast(float, (254u - S) << 23);  // 2^(127 - S)
            const int hcol = wn * 64 + jj * 32 + 4 * h;                       // + 8 q
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float y[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) y[u] = __builtin_fminf(__builtin_fmaxf(hv[4 * q + u] * sc, -448.0f), 448.0f);
                int c = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
                c = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], c, true);
                const uint32_t off = row < T.rows ? (uint32_t)((int64_t)row * I + hcol + 8 * q) : 0xFFFFFFF0u;
                bstore4(rq, off, (uint32_t)c);
            }
            // scale byte of (grow, block (hcol0 + wn 64 + 32 jj) / 32), from lanes 0-31
            const int64_t b = (hcol0 + wn * 64 + jj * 32) / 32;
            const uint32_t soff = (row < T.rows && h == 0)
                                      ? (uint32_t)((grow >> 5) * 32 * KBh + (b >> 3) * 256 +
                                                   unit_byte((uint32_t)(grow & 31), (uint32_t)(b & 7)))
                                      : 0xFFFFFFF0u;
            bstore1(rsc, soff, S);
        }
    }
}

// General epilogue for row strides that are not a multiple of 8 elements:
// per-element stores with explicit bounds; drains its stores before
// returning, so the wait accounting of the next tile needs no store count.
__device__ __forceinline__ void epilogue_any(uint16_t* out, int rows, int cols, uint32_t ldo, f32x16 (&acc)[4][4],
                                          int wm, int wn, int h, int r32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + r32;
        if (row >= rows) continue;
        uint16_t* const orow = out + (uint32_t)row * ldo;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int col = wn * 128 + j * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                if (col < cols) orow[col] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][j][e]);
            }
    }
    wait_vm<0>();
}

// VEC16: output rows are 16-byte aligned (ldo % 8 == 0): 16-byte epilogue.
// EPI 1: quantizing SwiGLU epilogue instead of bf16 output (mode 0);
// EPI 2: both, the bf16 gate/up tile first (32 + 40 stores per wave, more
// than the 6-bit store count can name: the next tile waits down to 63, which
// still covers every load issued before the epilogue).
template <bool VEC16, int EPI>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(GemmArgs a) {
    constexpr int kEpiWait = EPI == 2 ? 63 : EPI == 1 ? kSwigluStores : (VEC16 ? 32 : 0);
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int l = t & 63;
    const int wm = w >> 1, wn = w & 1;
    const int h = l >> 5, r32 = l & 31;
    const int nwg = gridDim.x;
    const int bid = blockIdx.x;
    // workgroup -> slot so that each XCD (bid % 8) owns a contiguous slot range
    const int slot = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;

    Layout L;
    if (a.mode == 1) {
        L.lda = (uint32_t)a.Mcap;
        L.ldb = (uint32_t)a.Mcap;
        L.a_unit = (uint32_t)a.Mcap;
        L.b_unit = (uint32_t)a.Mcap;
        L.ldo = (uint32_t)a.K;
    } else {
        L.lda = (uint32_t)a.K;
        L.ldb = (uint32_t)(a.mode == 0 ? a.K : a.ldb);
        L.a_unit = (uint32_t)a.K;
        L.b_unit = (uint32_t)(a.mode == 0 ? a.K : a.ldb);
        L.ldo = (uint32_t)a.N;
    }

    // Per-group tile counts and their inclusive prefix (16 groups per thread):
    // modes 0/2 tile a group's rows; mode 1 gives every group with a
    // non-empty contraction range the full [N] x [K] grid.
    const int G = a.G;
    const int64_t nN = (a.N + TN - 1) / TN;
    const int64_t per1 = ((a.N + TM - 1) / TM) * ((a.K + TN - 1) / TN);
    const bool lpt = lpt_mode(a);
    if (lpt) {
        // rank the groups by contraction length, longest first (ties by index)
        __shared__ int32_t lpt_len[kLptGroups];
        if (t < G) {
            const int64_t p0 = clamp64(a.offsets[t], 0, a.Mcap) & ~(int64_t)255;
            const int64_t p1 = clamp64(a.offsets[t + 1], 0, a.Mcap) & ~(int64_t)255;
            lpt_len[t] = p1 > p0 ? (int32_t)((p1 - p0) >> 8) : 0;
        }
        __syncthreads();
        if (t < G) {
            const int32_t c = lpt_len[t];
            int rank = 0;
            for (int h = 0; h < G; ++h) rank += (lpt_len[h] > c || (lpt_len[h] == c && h < t)) ? 1 : 0;
            lpt_order[rank] = t;
        }
        __syncthreads();
    }
    {
        int32_t loc[16];
        int32_t sum = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int g = t * 16 + j;
            int32_t cnt = 0;
            if (g <= G) {
                if (a.mode != 1) {
                    debug_flag(offsets_entry_bad(a.offsets, g, G, a.M), kDbgOffsets);
                } else {
                    const int64_t p = a.offsets[g];
                    debug_flag(p % 256 != 0 || p < 0 || p > a.Mcap || (g < G && a.offsets[g + 1] < p), kDbgPadded);
                }
            }
            if (g < G) {
                if (a.mode != 1) {
                    const int64_t lo = group_lo(a.offsets, g, a.M), hi = group_lo(a.offsets, g + 1, a.M);
                    const int64_t mg = hi > lo ? hi - lo : 0;
                    cnt = (int32_t)(((mg + TM - 1) / TM) * nN);
                } else {
                    const int gg = lpt ? lpt_order[g] : g;
                    const int64_t p0 = clamp64(a.offsets[gg], 0, a.Mcap) & ~(int64_t)255;
                    const int64_t p1 = clamp64(a.offsets[gg + 1], 0, a.Mcap) & ~(int64_t)255;
                    cnt = p1 > p0 ? (int32_t)per1 : 0;
                }
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
    }
    // (a count below 2^31 read from LDS, made wave-uniform so that what is
    // derived from it stays in scalar registers)
    const int64_t total = (int64_t)uni((uint32_t)(G > 0 ? tile_end[G - 1] : 0));

    if (a.mode == 1) {
        // groups with an empty contraction range: dW[g] = 0
        for (int64_t g = 0; g < G; ++g) {
            const int64_t p0 = clamp64(a.offsets[g], 0, a.Mcap) & ~(int64_t)255;
            const int64_t p1 = clamp64(a.offsets[g + 1], 0, a.Mcap) & ~(int64_t)255;
            if (p1 > p0) continue;
            uint16_t* const dst = a.out + g * a.N * a.K;
            const int64_t n = a.N * a.K;
            for (int64_t e = (int64_t)slot * 256 + t; e < n; e += (int64_t)nwg * 256) dst[e] = 0;
        }
        wait_vm<0>();
    }

    // round r gives workgroup slot the tile r nwg + slot, or r nwg + nwg - 1 -
    // slot in odd rounds when the groups are taken longest first: from an even
    // round the next tile is 2 (nwg - slot) - 1 further, from an odd one
    // 2 slot + 1
    int64_t tile = slot;
    bool odd = false;
    if (tile >= total) return;

    // per-lane constants
    Lane Ln;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int row = w * 64 + (l >> 3);
        const int gran = (l & 7) ^ (((l >> 4) & 3) | (p << 2));
        Ln.va[p] = (uint32_t)row * L.lda + (uint32_t)gran * 16u;
        Ln.vb[p] = (uint32_t)row * L.ldb + (uint32_t)gran * 16u;
    }
    {
        const int ra = wm * 128 + r32, rb = wn * 128 + r32;
        Ln.fo[0] = ra * SK + ((0 + h) ^ swz(ra)) * 16;
        Ln.fo[1] = ra * SK + ((2 + h) ^ swz(ra)) * 16;
        Ln.fo[2] = rb * SK + ((0 + h) ^ swz(rb)) * 16;
        Ln.fo[3] = rb * SK + ((2 + h) ^ swz(rb)) * 16;
    }
    const uint32_t la0 = uni(lds_addr(lds_a[0]) + w * 64 * SK), la1 = uni(lds_addr(lds_a[1]) + w * 64 * SK);
    const uint32_t lb0 = uni(lds_addr(lds_b[0]) + w * 64 * SK), lb1 = uni(lds_addr(lds_b[1]) + w * 64 * SK);

    int gcur = 0;
    Tile T = decode_tile<EPI>(a, L, tile, total, gcur);

    // Prologue: scales of chunk 0 into parity 0, stages 0 and 1 into buffers
    // 0 and 1; wait for the scales and stage 0.
    issue_scales(T.rsa, T.rsb, T.asub, T.bsub, uni(0u), 0, w, l, L);
    {
        const StageDma S0{T.ra, T.rb, uni(0u), la0, lb0};
        const StageDma S1{T.ra, T.rb, uni((uint32_t)SK), la1, lb1};
        issue_stage_plain(S0, Ln, L);
        issue_stage_plain(S1, Ln, L);
    }
    wait_vm<kStageDma>();
    __syncthreads();

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    Pipe P;
    read_frags(0, 0, Ln, P.F0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        P.sa[i] = read_scale(lds_sa[0], T.asub, wm * 4 + i, h, r32);
        P.sb[i] = read_scale(lds_sb[0], T.bsub, wn * 4 + i, h, r32);
    }
    P.gpar = 0;
    bool first = true;  // no epilogue stores issued yet

    // The chunks of all of this workgroup's tiles form one pipeline: the last
    // chunk of a tile loads the next tile's chunk-0 scales and stages 0 and 1
    // (nothing, through empty descriptors, after the last tile).
    for (;;) {
        int c = 0;
        for (; c + 1 < T.nchunk; ++c) {
            const Ahead X{T.ra, T.rb, T.rsa, T.rsb, T.asub, T.bsub, uni((uint32_t)(c + 1) * 256u),
                          uni((uint32_t)(2 * c + 2) * SK), uni((uint32_t)(2 * c + 3) * SK)};
            run_chunk<kEpiWait>(P, acc, X, c == 0 && !first && kEpiWait > 0, Ln, L, w, l, wm, wn, la0, la1, lb0,
                                lb1);
        }
        const int64_t next = tile + (!lpt ? nwg : odd ? 2 * slot + 1 : 2 * (nwg - slot) - 1);
        const Tile Tn = decode_tile<EPI>(a, L, next, total, gcur);
        {
            const Ahead X{Tn.ra, Tn.rb, Tn.rsa, Tn.rsb, Tn.asub, Tn.bsub, uni(0u), uni(0u), uni((uint32_t)SK)};
            run_chunk<kEpiWait>(P, acc, X, c == 0 && !first && kEpiWait > 0, Ln, L, w, l, wm, wn, la0, la1, lb0,
                                lb1);
        }
        if (EPI == 2) {
            // bf16 gate/up and the quantized activation, one 32-row block at
            // a time (fewer values live at once)
            uint16_t* const pre = a.out + (T.outoff >> 24) * a.N + (T.outoff & 0xFFFFFF) * TN;
            epilogue16<0, 1>(pre, T, L, acc, wm, wn, h, r32);
            epilogue_swiglu<0, 1>(a, T, acc, wm, wn, h, r32);
            epilogue16<1, 2>(pre, T, L, acc, wm, wn, h, r32);
            epilogue_swiglu<1, 2>(a, T, acc, wm, wn, h, r32);
            epilogue16<2, 3>(pre, T, L, acc, wm, wn, h, r32);
            epilogue_swiglu<2, 3>(a, T, acc, wm, wn, h, r32);
            epilogue16<3, 4>(pre, T, L, acc, wm, wn, h, r32);
            epilogue_swiglu<3, 4>(a, T, acc, wm, wn, h, r32);
        } else if (EPI == 1) {
            epilogue_swiglu(a, T, acc, wm, wn, h, r32);
        } else if (VEC16) {
            epilogue16(a.out + T.outoff, T, L, acc, wm, wn, h, r32);
        } else {
            epilogue_any(a.out + T.outoff, T.rows, T.cols, L.ldo, acc, wm, wn, h, r32);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
        if (Tn.nchunk == 0) break;
        T = Tn;
        tile = next;
        odd = !odd;
        first = false;
    }
    // Loads through empty descriptors and the last stores: let them finish
    // before the wave ends and its LDS is handed to another workgroup.
    wait_vm<0>();
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

void launch(const GemmArgs& a, int64_t nwg, hipStream_t stream) {
    const int64_t ldo = a.mode == 1 ? a.K : a.N;
    if (ldo % 8 == 0)
        hipLaunchKernelGGL((grouped_gemm_kernel<true, 0>), dim3((unsigned)nwg), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<false, 0>), dim3((unsigned)nwg), dim3(256), 0, stream, a);
}

int64_t scale_bytes(int64_t R, int64_t K) { return ((R + 31) / 32) * 32 * (8 * ((K + 255) / 256)); }

}  // namespace

#ifdef MXMOE_DEBUG
hipError_t debug_take_gemm(uint32_t* out) { return debug_take_word(out); }
#endif

hipError_t launch_grouped_gemm(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq,
                               const uint8_t* Ws, const int32_t* group_offsets, int32_t G, int64_t M,
                               int64_t N, int64_t K, uint16_t* out, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    GemmArgs a = {};
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
    a.a_scale_bytes = scale_bytes(M, K);
    a.b_scale_bytes = scale_bytes((int64_t)G * N, K);
    a.G = G;
    a.mode = 0;
    a.ldb = 0;
    const int64_t ub = ((M + TM - 1) / TM + G) * ((N + TN - 1) / TN);
    int64_t nwg = num_cus();
    if (ub < nwg) nwg = ub;
    launch(a, nwg, stream);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm_swiglu(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                                      const int32_t* group_offsets, int32_t G, int64_t M, int64_t I, int64_t K,
                                      uint8_t* hq, uint8_t* hs, uint16_t* preact, hipStream_t stream) {
    if (M == 0 || I == 0) return hipSuccess;
    GemmArgs a = {};
    a.A = Xq;
    a.As = Xs;
    a.B = Wq;
    a.Bs = Ws;
    a.offsets = group_offsets;
    a.out = preact;
    a.M = M;
    a.N = 2 * I;
    a.K = K;
    a.Mcap = 0;
    a.a_scale_bytes = scale_bytes(M, K);
    a.b_scale_bytes = scale_bytes((int64_t)G * 2 * I, K);
    a.G = G;
    a.mode = 0;
    a.ldb = 0;
    a.hq = hq;
    a.hs = hs;
    const int64_t ub = ((M + TM - 1) / TM + G) * ((2 * I + TN - 1) / TN);
    int64_t nwg = num_cus();
    if (ub < nwg) nwg = ub;
    if (preact) hipLaunchKernelGGL((grouped_gemm_kernel<true, 2>), dim3((unsigned)nwg), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((grouped_gemm_kernel<true, 1>), dim3((unsigned)nwg), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm_dgrad(const uint8_t* dYq, const uint8_t* dYs, const uint8_t* WTq,
                                     const uint8_t* WTs, const int32_t* group_offsets, int32_t G, int64_t M,
                                     int64_t N, int64_t K, int64_t Wcap, uint16_t* dX, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    GemmArgs a = {};
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
    a.a_scale_bytes = scale_bytes(M, K);
    a.b_scale_bytes = scale_bytes(N, Wcap);
    a.G = G;
    a.mode = 2;
    a.ldb = Wcap;
    const int64_t ub = ((M + TM - 1) / TM + G) * ((N + TN - 1) / TN);
    int64_t nwg = num_cus();
    if (ub < nwg) nwg = ub;
    launch(a, nwg, stream);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm_wgrad(const uint8_t* A, const uint8_t* As, const uint8_t* B,
                                     const uint8_t* Bs, const int32_t* padded_offsets, int32_t G,
                                     int64_t N, int64_t K, int64_t Mcap, uint16_t* dW,
                                     hipStream_t stream) {
    if (N == 0 || K == 0 || G == 0) return hipSuccess;
    GemmArgs a = {};
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
    a.a_scale_bytes = scale_bytes(N, Mcap);
    a.b_scale_bytes = scale_bytes(K, Mcap);
    a.G = G;
    a.mode = 1;
    a.ldb = 0;
    const int64_t total = ((N + TM - 1) / TM) * ((K + TN - 1) / TN) * G;
    int64_t nwg = num_cus();
    if (total < nwg) nwg = total;
    launch(a, nwg, stream);
    return hipGetLastError();
}

}  // namespace mx
