// kvq_device.h -- device-side helpers of the HIP path (gfx950 only).
//
// FP8 / INT8 encode and decode written from the formats' definitions ("Accelerating Inference with
// FP8 KV Cache", section "FP8 Formats: E4M3 and E5M2": OCP E4M3 = 1/4/3 bits, E5M2 = 1/5/2 bits;
// section "Current Hardware Support": AMD's E4M3FNUZ, the 1/4/3 layout with bias 8, no infinities,
// no negative zero and its one NaN at 0x80; the online INT8 cache of "[Feature] TurboMind support
// W8A8 or FP8 KV Cache"), plus wave-level reductions.  Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 codes, byte i = code i

constexpr int kDim = KVQ_HEAD_DIM;     // 128
constexpr int kBlock = KVQ_BLOCK_SIZE; // 16
constexpr int kTileBytes = kDim * kBlock;  // 2048 bytes per (block, KV head) tile
// K tile: eight 256-byte chunks, chunk c holding dims 16c .. 16c+15 of the 16 tokens (16 B per
// token).  Any 1 KiB half of the tile is four whole chunks, so a wave's 16-byte-per-lane load of
// one half reads whole 128-byte lines whatever lane owns which (chunk, token) piece.
constexpr int kChunk = 16;
constexpr int kChunkBytes = kChunk * kBlock;  // 256
__device__ __forceinline__ uint32_t k_byte(int t, int d) {
    return (uint32_t)(d / kChunk) * kChunkBytes + (uint32_t)t * kChunk + (uint32_t)(d % kChunk);
}
constexpr float kLog2e = 1.4426950408889634f;
// INT8 scales: one 128-byte row per (block, KV head) tile, its 16 K scales and then its 16 V scales
// (the cache's k_scale points at the rows, v_scale = k_scale + 16), so a wave reading a tile's
// scales reads one whole line.  Index of token t's scale from either pointer:
constexpr int kScaleRow8 = 2 * kBlock;
__device__ __forceinline__ size_t int8_scale_index(int blk, int Hkv, int g, int t) {
    return ((size_t)blk * Hkv + g) * kScaleRow8 + t;
}

// ------------------------------------------------------------------------------------------------
// encode (append path).  y is the fp32 quotient x / kv_scale.
//
// Normal range: round the binary32 significand to M mantissa bits, ties to even, directly on the
// bit pattern -- adding (half ulp - 1) plus the kept LSB and truncating rounds half to even, and a
// carry out of the mantissa moves into the exponent field as it should.  The binary32 exponent
// field (bias 127) is then rebased to the FP8 bias.  Subnormal range: the code is the number of
// steps 2^(1-bias-M), rounded to nearest even; the value 2^M steps is the smallest normal code,
// whose bit pattern is exactly 2^M.  Magnitudes at or above the largest finite value saturate:
// every such value either rounds to it or overflows, and overflow saturates.
// E4M3FNUZ differs only in its constants and special codes: NaN is 0x80 and a magnitude that
// rounds to zero is the unsigned zero 0x00.
template <int FMT>
__device__ __forceinline__ uint32_t encode_fp8(float y) {
#pragma clang fp contract(off)
    constexpr bool FNUZ = FMT == KVQ_FP8_E4M3FNUZ;
    constexpr int M = (FMT == KVQ_FP8_E5M2) ? 2 : 3;
    constexpr int BIAS = (FMT == KVQ_FP8_E5M2) ? 15 : (FNUZ ? 8 : 7);
    constexpr uint32_t MAX_BITS = (FMT == KVQ_FP8_E4M3) ? 0x43E00000u     // 448
                                  : (FNUZ ? 0x43700000u                   // 240
                                          : 0x47600000u);                 // 57344
    constexpr uint32_t MAX_CODE = (FMT == KVQ_FP8_E4M3) ? 0x7Eu : (FNUZ ? 0x7Fu : 0x7Bu);
    constexpr uint32_t MIN_NORMAL_BITS = (uint32_t)(127 + 1 - BIAS) << 23;  // 2^(1-bias)
    constexpr int SH = 23 - M;

    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return FNUZ ? 0x80u : (sign | 0x7Fu);  // NaN
    if (a >= MAX_BITS) return sign | MAX_CODE;         // saturation (covers +-inf)
    if (a >= MIN_NORMAL_BITS) {
        const uint32_t r = a + ((1u << (SH - 1)) - 1u) + ((a >> SH) & 1u);
        return sign | ((r >> SH) - ((uint32_t)(127 - BIAS) << M));
    }
    // exact power-of-two scaling, then round half to even (v_rndne_f32)
    const float steps = __uint_as_float(a) * (float)(1u << (BIAS - 1 + M));
    const uint32_t mag = (uint32_t)__builtin_rintf(steps);
    if constexpr (FNUZ) return mag == 0u ? 0u : (sign | mag);
    return sign | mag;
}

// INT8 code of x for a row scale s (s = fl32(amax / 127) > 0): clamp(rne(fl32(x / s)), -127, 127),
// as a byte; a zero row (s == 0) gives 0.
__device__ __forceinline__ uint32_t encode_int8(float x, float s) {
#pragma clang fp contract(off)
    if (s == 0.0f) return 0u;
    const float r = fminf(fmaxf(__builtin_rintf(x / s), -127.0f), 127.0f);
    return (uint32_t)(int32_t)r & 0xFFu;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// ------------------------------------------------------------------------------------------------
// decode to exact fp16 pairs.  `w` holds four codes (byte i = code i); `SEL` picks bytes
// (2*SEL, 2*SEL+1), returned as (lo, hi) halves.

// E4M3 -> fp16 with the gfx950 converter (unit scale): every E4M3 value, subnormals included, is
// a normal binary16 number, so the conversion is exact.
template <int SEL>
__device__ __forceinline__ half2_t e4m3x2_to_f16(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, SEL != 0);
}

// E5M2 -> fp16 by placement: E5M2 is binary16 with its low 8 fraction bits dropped (same sign,
// exponent width and bias), so the code becomes the high byte of the half.
template <int SEL>
__device__ __forceinline__ half2_t e5m2x2_to_f16(uint32_t w) {
    constexpr uint32_t sel = (SEL == 0) ? 0x010C000Cu : 0x030C020Cu;
    return __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0u, w, sel));
}

// E4M3FNUZ -> fp16 at 2^-7 of the value.  The code's exponent and mantissa fields s.eeee.mmm go to
// the fp16 fields s.0eeee.mmm0000000; with fp16's bias 15 against the code's 8 that is the value
// times 2^-7 exactly, the subnormal codes (e = 0, m * 2^-10) included as fp16 subnormals m * 2^-17.
// The callers fold the 2^7 into their scales (code_unit).  The NaN code 0x80 comes out as -0: the
// attention kernels take a cache without NaN codes (only a NaN input writes one); kvq_dequant
// restores the NaN itself.
template <int SEL>
__device__ __forceinline__ half2_t e4m3fnuz_x2_to_f16(uint32_t w) {
    typedef short short2_t __attribute__((ext_vector_type(2)));
    constexpr uint32_t sel = (SEL == 0) ? 0x010C000Cu : 0x030C020Cu;  // codes to the halves' high bytes
    const uint32_t x = __builtin_amdgcn_perm(0u, w, sel);
    // one arithmetic shift per half leaves s.s.eeee.mmm0000000; clear the second sign bit
    const short2_t sh = __builtin_bit_cast(short2_t, x) >> (short2_t){1, 1};
    return __builtin_bit_cast(half2_t, __builtin_bit_cast(uint32_t, sh) & 0xBF80BF80u);
}

// INT8 -> fp16: put each signed byte, its sign bit flipped, in the low byte of a half with high
// byte 0x64, which is the binary16 number 1024 + (q + 128); subtracting 1152 leaves q exactly
// (all integers below 2048 are exact in binary16).  The sign flip is one XOR of the whole dword,
// which the two pairs of a dword share; the byte permute then takes the 0x64 bytes from its other
// operand.
template <int SEL>
__device__ __forceinline__ half2_t int8x2_to_f16(uint32_t w) {
    constexpr uint32_t sel = (SEL == 0) ? 0x04010400u : 0x04030402u;
    const uint32_t x = __builtin_amdgcn_perm(0x64646464u, w ^ 0x80808080u, sel);
    return __builtin_bit_cast(half2_t, x) - half2_t{(_Float16)1152.0f, (_Float16)1152.0f};
}

// Codes (2*SEL, 2*SEL+1) of w as fp16; each code's value is the result times code_unit(DT).
template <int DT, int SEL>
__device__ __forceinline__ half2_t codes_to_f16(uint32_t w) {
    if constexpr (DT == KVQ_FP8_E4M3) return e4m3x2_to_f16<SEL>(w);
    else if constexpr (DT == KVQ_FP8_E5M2) return e5m2x2_to_f16<SEL>(w);
    else if constexpr (DT == KVQ_FP8_E4M3FNUZ) return e4m3fnuz_x2_to_f16<SEL>(w);
    else return int8x2_to_f16<SEL>(w);
}

// The factor between codes_to_f16's result and the code's value: 2^7 for E4M3FNUZ, else 1.
__host__ __device__ constexpr float code_unit(int dtype) {
    return dtype == KVQ_FP8_E4M3FNUZ ? 128.0f : 1.0f;
}

__device__ __forceinline__ float dot2(half2_t a, half2_t b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    half2_t h = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, h);
}

// ------------------------------------------------------------------------------------------------
// cross-lane helpers (wave64)
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, true));
}
// sum over each quad (xor 1, then xor 2).  Floating-point addition is commutative, so the four
// lanes of a quad end with bitwise the same sum.
__device__ __forceinline__ float sum4(float v) {
    v += dpp<0xB1>(v);  // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);  // quad_perm [2,3,0,1]
    return v;
}
// max over the 16 quads (the four quads of a 16-lane row by rotation, then across rows)
__device__ __forceinline__ float max_across_quads(float v) {
    v = fmaxf(v, dpp<0x124>(v));  // row_ror:4
    v = fmaxf(v, dpp<0x128>(v));  // row_ror:8
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}
// reductions across the eight groups of 8 lanes (lanes l, l^8, l^16, ..., l^56)
__device__ __forceinline__ float max_across8(float v) {
    v = fmaxf(v, dpp<0x128>(v));  // row_ror:8 == xor 8 within a 16-lane row
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}
__device__ __forceinline__ float sum_across8(float v) {
    v += dpp<0x128>(v);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    v = sum_across8(v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    return max_across8(v);
}

// Cache codes are read exactly once per step: load them with the non-temporal (streaming) hint,
// which keeps them from displacing reusable lines and measurably raises the achieved HBM bandwidth.
__device__ __forceinline__ u32x4 ldg16(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ uint32_t ldg4(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
template <typename T>
__device__ __forceinline__ T ldg_nt(const T* p) {
    return __builtin_nontemporal_load(p);
}
// Prefill reads each tile once per row tile of its sequence, so its loads keep the ordinary
// caching: the streaming hint would evict the lines the sequence's other row tiles are about to
// read (measured: twice the kernel time).
__device__ __forceinline__ u32x4 ld16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
template <bool NT, typename T>
__device__ __forceinline__ T ld(const T* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

}  // namespace kvq
