// kvq_int4.h -- device helpers of the INT4 cache: the row encoder, the nibble decoder and the tile
// geometry.
//
// The online INT4 KV cache ("[Feature] TurboMind support W8A8 or FP8 KV Cache" names INT4 beside
// the online INT8 cache), read as asymmetric 4-bit codes with one fp32 (scale, zero point) pair per
// (token, KV head): zp = min x, s = fl32(fl32(max x - zp) / 15),
// q = clamp(rne(fl32(fl32(x - zp) / s)), 0, 15), value q s + zp; two codes per byte.  Nothing here
// is shared with the CPU oracle.
#pragma once

#include "kvq_device.h"

namespace kvq {

typedef float f32x2 __attribute__((ext_vector_type(2)));  // a (scale, zero point) pair

// INT4 code of x for a row with zero point zp (its minimum) and scale s = fl32(range / 15) > 0:
// clamp(rne(fl32(fl32(x - zp) / s)), 0, 15); a constant row (s == 0) gives 0.
__device__ __forceinline__ uint32_t encode_int4(float x, float zp, float s) {
#pragma clang fp contract(off)
    if (s == 0.0f) return 0u;
    const float r = fminf(fmaxf(__builtin_rintf((x - zp) / s), 0.0f), 15.0f);
    return (uint32_t)r;
}

// The eight 4-bit codes of w (nibble i = code i) as exact binary16 subnormals, in the pairs
// (i, i + 4): a half whose bits are a nibble n alone is n * 2^-24, and one holding n << 4 is
// n * 2^-20, so masking alone decodes --
//   h[0] = nibbles (0, 4) * 2^-24,  h[1] = nibbles (1, 5) * 2^-20,
//   h[2] = nibbles (2, 6) * 2^-24,  h[3] = nibbles (3, 7) * 2^-20.
// Callers pair their other operand the same way, accumulate the 2^-24 and the 2^-20 pairs apart
// and fold the powers of two back in (kInt4Even, kInt4Odd).  The one-head kernel feeds these to the
// packed dot-product instruction, whose two products with an fp16 operand are exact in fp32; the
// matrix cores do not keep such products whole (int4x8_centred below).
constexpr float kInt4Even = 16777216.0f;  // 2^24
constexpr float kInt4Odd = 1048576.0f;    // 2^20
__device__ __forceinline__ void int4x8_to_f16(uint32_t w, half2_t (&h)[4]) {
    const uint32_t w8 = w >> 8;
    h[0] = __builtin_bit_cast(half2_t, w & 0x000F000Fu);
    h[1] = __builtin_bit_cast(half2_t, w & 0x00F000F0u);
    h[2] = __builtin_bit_cast(half2_t, w8 & 0x000F000Fu);
    h[3] = __builtin_bit_cast(half2_t, w8 & 0x00F000F0u);
}

// The matrix cores align the products of each group of 8 k-slots by the operands' exponent fields,
// and a binary16 subnormal counts as exponent -14 whatever its value, so codes masked into subnormals
// as above keep only about 14 bits of each product there.  The matrix-core kernels therefore give the K codes as
// exact small binary16 integers, centred: in the pairs (i, i + 4) of int4x8_to_f16, the even pairs as
// n - c0 = (1024 + n) - (1024 + c0) and the odd ones as 16 (n - c0) = (1024 + 16 n) - (1024 + 16 c0),
// each the code placed under the exponent of 1024 (one v_and_or_b32, Int4Bits) and one packed fp16
// addition of ne = -(1024 + c0) or no = -(1024 + 16 c0).
//
// Int4Bits holds the two nibble masks (in SGPRs) and the exponent pattern 0x6400 of 1024 (in a
// VGPR).  With literal operands the compiler issues an AND and an OR for every mask-and-insert; with
// the operands in registers, one v_and_or_b32.  The identity DPP move only hides the constants from
// constant folding.
struct Int4Bits {
    uint32_t even, odd, magic;
};
__device__ __forceinline__ uint32_t int4_opaque(uint32_t c) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)c, 0xE4, 0xF, 0xF, false);
}
__device__ __forceinline__ Int4Bits int4_bits() {
    return {(uint32_t)__builtin_amdgcn_readfirstlane(int4_opaque(0x000F000Fu)),
            (uint32_t)__builtin_amdgcn_readfirstlane(int4_opaque(0x00F000F0u)), int4_opaque(0x64006400u)};
}
__device__ __forceinline__ void int4x8_centred(uint32_t w, half2_t ne, half2_t no, const Int4Bits& b,
                                               half2_t (&h)[4]) {
    const uint32_t w8 = w >> 8;
    h[0] = __builtin_bit_cast(half2_t, (w & b.even) | b.magic) + ne;
    h[1] = __builtin_bit_cast(half2_t, (w & b.odd) | b.magic) + no;
    h[2] = __builtin_bit_cast(half2_t, (w8 & b.even) | b.magic) + ne;
    h[3] = __builtin_bit_cast(half2_t, (w8 & b.odd) | b.magic) + no;
}

// The code of a row (scale s, zero point zp) whose value s c + zp is nearest zero, clamped to
// [0, 15]; NaN or zero parameters give 0.  The kernels centre each token's codes there: its logit
// s (q . (c - c0)) + (zp + s c0) sum q is exact for any integer c0, and with c0 the token's own zero
// code it sums terms no larger than q . k^ itself, where s (q . c) + zp sum q cancels two terms up
// to 15 s sum |q| large.  A token's c0 comes from this one function on the token's own pair
// wherever it is needed, so the K operand and zp' = zp + s c0 always agree.
__device__ __forceinline__ float int4_zero_code(float s, float zp) {
    const float c = __builtin_rintf(-zp * __builtin_amdgcn_rcpf(s));
    return fminf(fmaxf(c, 0.0f), 15.0f);
}

// The pair constants ne = -(1024 + c0), no = -(1024 + 16 c0) of int4x8_centred.
__device__ __forceinline__ void int4_centre_pairs(float c0, half2_t& ne, half2_t& no) {
    const _Float16 e = (_Float16)(-1024.0f - c0), o = (_Float16)(-1024.0f - 16.0f * c0);
    ne = half2_t{e, e};
    no = half2_t{o, o};
}

// Eight 4-bit codes as exact binary16 integers through the FP8 converter.  A byte holding one
// nibble n alone is the E4M3 code of n 2^-9: codes 0..7 are the subnormals n 2^-9 and codes 8..15
// the first normal binade, (1 + (n - 8) / 8) 2^-6 = n 2^-9, so the scaled conversion with scale 2^9
// gives n exactly, two codes per instruction:
//   h[0] = nibbles (0, 2),  h[1] = nibbles (4, 6),  h[2] = nibbles (1, 3),  h[3] = nibbles (5, 7).
// The matrix cores keep products of such operands whole (normal binary16 integers of 4 bits).
constexpr float kNibbleScale = 512.0f;  // 2^9
__device__ __forceinline__ void int4x8_exact(uint32_t w, half2_t (&h)[4]) {
    const uint32_t lo = w & 0x0F0F0F0Fu;         // nibbles 0, 2, 4, 6, one per byte
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // nibbles 1, 3, 5, 7
    h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, kNibbleScale, false);
    h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, kNibbleScale, true);
    h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, kNibbleScale, false);
    h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, kNibbleScale, true);
}
// The nibble of a dword that k-slot s of its operand join8(h[0], h[1], h[2], h[3]) holds.
__device__ __forceinline__ constexpr int int4_slot_nibble(int s) { return s < 4 ? 2 * s : 2 * (s - 4) + 1; }

// Tile geometry (1 KiB per tile).
//   K: four 256-byte chunks of 32 dims x 16 tokens; the byte of dim d of token t holds dims
//      d & ~1 (low nibble) and d | 1.
//   V: four 256-byte blocks, one per quad of tokens; in block t / 4, the 16 bytes at (d % 16) * 16
//      hold the dims d % 16 + 16 r (r = 0..7) as 16-bit units of the quad's four tokens (bytes
//      2r and 2r + 1: tokens 0, 1 and 2, 3 of the quad, the even one in the low nibble).  One
//      16-byte load per lane reads a whole tile whether a lane is a (token quad, dim) piece of the
//      MFMA operands or of the VALU kernel.
constexpr int kTileBytes4 = kTileBytes / 2;
__device__ __forceinline__ uint32_t k_byte4(int t, int d) {
    return (uint32_t)(d / 32) * 256u + (uint32_t)t * 16u + (uint32_t)((d % 32) / 2);
}
__device__ __forceinline__ uint32_t v_byte4(int t, int d) {
    return (uint32_t)(t / 4) * 256u + (uint32_t)(d % 16) * 16u + (uint32_t)(d / 16) * 2u +
           (uint32_t)((t % 4) / 2);
}

// One lane's share of one tile in the matrix-core lane layout (the grouped decode kernel and the
// prefill kernel): K of token l % 16 in chunk l / 16 and V of quad l / 16 for the dims l % 16 + 16 r
// (one 16-byte load each), and the K and V (scale, zero point) pairs of the lane's own token
// 4 (l / 16) + l % 4 -- one of the four tokens 4 q4 + u of the lane's accumulator, so each quad of
// lanes holds all four and hands them round with quad broadcasts (quad_bcast), and a tile costs 12
// registers while its loads are in flight.
struct TileQ4 {
    u32x4 k, v;
    f32x2 kp, vp;
};
__device__ __forceinline__ int int4_own_token(int lane) { return 4 * (lane >> 4) + (lane & 3); }

// NT: the streaming hint (decode reads each tile once; prefill re-reads it for every row tile of
// the sequence and keeps the ordinary caching).  ks / vs are the [blocks][Hkv][16][2] pair arrays.
template <bool NT>
__device__ __forceinline__ void load_tile_q4(const uint8_t* kc, const uint8_t* vc, const float* ks,
                                             const float* vs, int Hkv, TileQ4& t, int blk, int g, uint32_t off,
                                             int own) {
    const size_t pair = (size_t)blk * Hkv + g;
    t.k = ld<NT>(reinterpret_cast<const u32x4*>(kc + pair * kTileBytes4 + off));
    t.v = ld<NT>(reinterpret_cast<const u32x4*>(vc + pair * kTileBytes4 + off));
    t.kp = ld<NT>(reinterpret_cast<const f32x2*>(ks) + pair * kBlock + own);
    t.vp = ld<NT>(reinterpret_cast<const f32x2*>(vs) + pair * kBlock + own);
}

// Value of lane 4 (l / 4) + U of the lane's quad (DPP quad_perm [U, U, U, U]).  In the matrix-core
// kernels every group of these broadcasts is fenced off from the scheduler
// (__builtin_amdgcn_sched_barrier on both sides): interleaved with the surrounding matrix and VALU
// instructions, the K-pair broadcasts of the INT4 prefill kernel gave NaN outputs on the
// low-binade codes test, and with the fences (or with LDS shuffles instead) the same kernel is
// correct.  The cause was not established, so the fences stay wherever these broadcasts meet
// matrix-core code.
template <int U>
__device__ __forceinline__ float quad_bcast(float v) {
    return dpp<U * 0x55>(v);
}

// The 16-bit unit of a V dword (SEL 0: bits 0-15, 1: bits 16-31: four tokens of one dim) as two
// binary16 pairs (see int4x8_to_f16): e = tokens (0, 2) * 2^-24, o = tokens (1, 3) * 2^-20.
template <int SEL>
__device__ __forceinline__ void int4_unit_to_f16(uint32_t w, half2_t& e, half2_t& o) {
    constexpr uint32_t sel = (SEL == 0) ? 0x0C010C00u : 0x0C030C02u;  // its bytes to the halves' low bytes
    const uint32_t x = __builtin_amdgcn_perm(0u, w, sel);
    e = __builtin_bit_cast(half2_t, x & 0x000F000Fu);
    o = __builtin_bit_cast(half2_t, x & 0x00F000F0u);
}

__device__ __forceinline__ float wave_min(float v) {
    v = fminf(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
    v = fminf(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fminf(v, dpp<0x141>(v));  // row_half_mirror
    v = fminf(v, dpp<0x128>(v));  // row_ror:8
    v = fminf(v, __shfl_xor(v, 16));
    v = fminf(v, __shfl_xor(v, 32));
    return v;
}


// Partition kernels of the INT4 cache: one query head per KV head (kvq_attn_mha4.hip) and grouped
// query heads (kvq_attn_gqa4.hip).
struct KernelParams;
void launch_partition_mha4(const KernelParams& kp, hipStream_t stream, hipEvent_t start, hipEvent_t stop);
void launch_partition_gqa4(const KernelParams& kp, hipStream_t stream, hipEvent_t start, hipEvent_t stop);

// Prefill attention over the INT4 cache (kvq_prefill4.hip).
struct PrefillArgs;
hipError_t launch_prefill4(const PrefillArgs& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop);

}  // namespace kvq
