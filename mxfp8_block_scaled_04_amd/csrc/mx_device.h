// Device helpers shared by the libmxmoe kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) 16-byte load / 8-byte store: the quantize
// kernels touch every byte exactly once.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream8(void* p, uint2 v) {
    __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p));
}
// Ordinary (cached) 8- and 16-byte stores: where one store instruction covers
// only part of each 128-byte line it touches, L2 can merge the parts before
// write-back.
__device__ __forceinline__ void store8(void* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }
__device__ __forceinline__ void store16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
// Streaming (non-temporal) 16-byte store.
__device__ __forceinline__ void store_stream16(void* p, uint4 v) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// Largest group count accepted by the grouped entry points.
constexpr int kMaxGroups = 4096;
// Row padding of a group in the column-wise (transposed) layout.
constexpr int kColsPad = 256;

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// Max over the 4 lanes of a DPP quad (lanes 4i..4i+3).
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
    uint32_t t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    v = v > t ? v : t;
    t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    return v > t ? v : t;
}

// Largest bf16 magnitude (bits & 0x7FFF) among 8 packed bf16 values.
__device__ __forceinline__ uint32_t max_mag8(uint4 d) {
    uint32_t m = pk_max_u16(pk_max_u16(d.x & 0x7FFF7FFFu, d.y & 0x7FFF7FFFu),
                            pk_max_u16(d.z & 0x7FFF7FFFu, d.w & 0x7FFF7FFFu));
    uint32_t lo = m & 0xFFFFu, hi = m >> 16;
    return lo > hi ? lo : hi;
}

// E8M0 scale byte of a block from its largest magnitude:
// floor(log2 amax) - 8 clamped at -127, i.e. max(biased exponent - 8, 0).
__device__ __forceinline__ uint32_t scale_from_maxmag(uint32_t maxmag) {
    int e = (int)(maxmag >> 7);
    return (uint32_t)(e > 8 ? e - 8 : 0);
}

// Clamp the magnitude of both bf16 halves of d to lim (a positive bf16 bit
// pattern), keeping signs.  As int16 only non-negative halves can exceed lim;
// as uint16 only negative halves can exceed 0x8000|lim.
__device__ __forceinline__ uint32_t clamp_mag2(uint32_t d, uint32_t lim2, uint32_t nlim2) {
    i16x2 a = __builtin_elementwise_min(__builtin_bit_cast(i16x2, d), __builtin_bit_cast(i16x2, lim2));
    u16x2 b = __builtin_elementwise_min(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, nlim2));
    return __builtin_bit_cast(uint32_t, b);
}

// Quantize 8 bf16 values (packed low-half-first in d) of one block with
// scale byte S to 8 E4M3FN codes (low byte first).
//  S >= 1: the hardware scaled conversion divides by 2^(S-127) and rounds to
//    nearest even; magnitudes are clamped first to 448 * 2^(S-127) (bf16
//    pattern ((S+8) << 7) | 0x60) so that the result saturates at 448.
//  S == 0 (block amax < 2^-118): y = x * 2^127 is formed exactly in fp32
//    (bf16 subnormals included), clamped to 448 and converted.
__device__ __forceinline__ uint2 quant8(uint4 d, uint32_t S) {
    uint2 r;
    if (S != 0) {
        float sc = __builtin_bit_cast(float, S << 23);
        uint32_t lim = ((S + 8u) << 7) | 0x60u;
        uint32_t lim2 = lim | (lim << 16);
        uint32_t nlim2 = lim2 | 0x80008000u;
        i16x2 z = {0, 0};
        i16x2 a = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(z, __builtin_bit_cast(bf16x2, clamp_mag2(d.x, lim2, nlim2)), sc, false);
        a = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(a, __builtin_bit_cast(bf16x2, clamp_mag2(d.y, lim2, nlim2)), sc, true);
        i16x2 b = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(z, __builtin_bit_cast(bf16x2, clamp_mag2(d.z, lim2, nlim2)), sc, false);
        b = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(b, __builtin_bit_cast(bf16x2, clamp_mag2(d.w, lim2, nlim2)), sc, true);
        r.x = __builtin_bit_cast(uint32_t, a);
        r.y = __builtin_bit_cast(uint32_t, b);
    } else {
        const float up = __builtin_bit_cast(float, 254u << 23);  // 2^127
        float f[8];
        const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __builtin_bit_cast(float, w[i] << 16) * up;
            f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u) * up;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = __builtin_fminf(__builtin_fmaxf(f[i], -448.0f), 448.0f);
        int o[2];
        o[0] = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        o[0] = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], o[0], true);
        o[1] = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
        o[1] = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], o[1], true);
        r.x = (uint32_t)o[0];
        r.y = (uint32_t)o[1];
    }
    return r;
}

// Group offset g clamped to [0, M] (malformed offsets cannot index out of
// bounds).
__device__ __forceinline__ int32_t clamp_off(const int32_t* off, int g, int64_t M) {
    int64_t v = off[g];
    return (int32_t)(v < 0 ? 0 : (v > M ? M : v));
}

// Byte position of the scale of (row r mod 32, block b mod 8) inside one
// 256-byte packed unit: lane register 32*(b%2) + r%32, byte (b%8)/2.
__device__ __forceinline__ uint32_t unit_byte(uint32_t r32, uint32_t b8) {
    return 4u * (32u * (b8 & 1u) + r32) + (b8 >> 1);
}

}  // namespace mx
