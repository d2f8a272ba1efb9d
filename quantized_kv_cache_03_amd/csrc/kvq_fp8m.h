// kvq_fp8m.h -- FP8 math: the query rows quantized to E4M3 for the QK^T product on the FP8 matrix
// cores (v_mfma_scale_f32_16x16x128_f8f6f4, unit scales), the cache's K codes used as stored.
//
// "[Feature] TurboMind support W8A8 or FP8 KV Cache" points beyond FP8 storage to FP8 attention,
// where E4M3 is the format used; it fixes no scale.  Here each 128-wide query row gets its own
// dynamic scale s_q = fl32(amax / 448) (448 = E4M3's largest finite value; s_q = 1 for a zero row)
// and codes c_d = enc_E4M3(fl32(q_d / s_q)), the encoder of the append path (round to nearest even,
// saturating).  s_q joins the logit scale: z_t = sm_scale * log2(e) * kv_scale * s_q * sum_d c_d k_t,d.
// The sum is the matrix instruction's, not an exact fp32 one: within each group of 8 consecutive
// k-slots the products are aligned to the group's largest exponent and cut 13 bits below it, then
// the group sums join the fp32 accumulator.  The logits carry that error, up to 2^-13 of each
// group's largest product, before the fp32 softmax.
#pragma once

#include "kvq_mfma.h"

namespace kvq {

// One lane's 32 FP8 k-slots of a 16x16x128 operand (byte i = k-slot i of the lane's group).  In A
// (16 rows x 128) and B (128 x 16 columns) lane l holds row / column l % 16 and k-slots
// 32 (l / 16) .. +31 alike, so any assignment of the 128 dims to a lane group's 32 bytes works as
// long as K and Q agree: K's two 16-byte loads of the lane (dims 16 q4 .. +15 and 64 + 16 q4 .. +15)
// and the query codes of the same dims, in the same byte order.
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float q_fp8_scale(float amax) {
    return amax > 0.0f ? amax / kE4M3Max : 1.0f;  // one correctly rounded fp32 division
}

// 8 fp16 query values -> their 8 E4M3 codes under scale s, byte i = value i, in two dwords
__device__ __forceinline__ void q_fp8_codes8(half8_v x, float s, uint32_t& lo, uint32_t& hi) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i)
        w[i >> 2] |= encode_fp8<KVQ_FP8_E4M3>((float)x[i] / s) << (8 * (i & 3));
    lo = w[0];
    hi = w[1];
}

__device__ __forceinline__ float abs_max8(half8_v x, float m) {
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf((float)x[i]));
    return m;
}

// One query row held by the four lanes col, col + 16, col + 32, col + 48 (32 values each, in the
// four half8 operands x[0..3], dims 64 (m/2) + 16 q4 + 8 (m%2) .. +7 of x[m]): its scale and this
// lane's 32 codes in that order.  Every lane of the wave calls it.
__device__ __forceinline__ float quantize_q_row_fp8(const half8_v (&x)[4], i32x8& c) {
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) m = abs_max8(x[k], m);
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    const float s = q_fp8_scale(m);
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) q_fp8_codes8(x[k], s, w[2 * k], w[2 * k + 1]);
    c = i32x8{(int)w[0], (int)w[1], (int)w[2], (int)w[3], (int)w[4], (int)w[5], (int)w[6], (int)w[7]};
    return s;
}

// The lane's K codes (its 16-byte loads from the two 1 KiB halves of the tile) as the A operand.
__device__ __forceinline__ i32x8 k_fp8x32(const u32x4& ka, const u32x4& kb) {
    const uint32_t w[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
    return i32x8{(int)w[0], (int)w[1], (int)w[2], (int)w[3], (int)w[4], (int)w[5], (int)w[6], (int)w[7]};
}

// S^T of one tile, all 128 dims in one instruction: A = K codes (format 0 = E4M3, 1 = E5M2),
// B = E4M3 query codes; unit scales (the scale operands 0 select the unscaled form).
template <int DT>
__device__ __forceinline__ float4_t mfma_qk_fp8(const i32x8& k, const i32x8& q, float4_t acc) {
    constexpr int FMT_A = DT == KVQ_FP8_E5M2 ? 1 : 0;
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k, q, acc, FMT_A, 0, 0, 0, 0, 0);
}

struct KernelParams;

// Decode partition kernel with FP8 math (kvq_attn_gqa.hip), any grouping G <= 16; dtype is
// KVQ_FP8_E4M3 or KVQ_FP8_E5M2.
void launch_partition_fp8math(const KernelParams& kp, int dtype, hipStream_t stream, hipEvent_t start,
                              hipEvent_t stop);

}  // namespace kvq
