// kvq_fp8m.h -- FP8 math: the query rows quantized to E4M3 for the QK^T product on the FP8 matrix
// cores (v_mfma_f32_16x16x32_fp8_fp8 / _bf8_fp8), the cache's K codes used as they are stored.
//
// "[Feature] TurboMind support W8A8 or FP8 KV Cache" points beyond FP8 storage to FP8 attention,
// where E4M3 is the format used; it fixes no scale.  Here each 128-wide query row gets its own
// dynamic scale s_q = fl32(amax / 448) (448 = E4M3's largest finite value; s_q = 1 for a zero row)
// and codes c_d = enc_E4M3(fl32(q_d / s_q)), the encoder of the append path (round to nearest even,
// saturating).  Products of E4M3 (or E5M2) codes are exact, the matrix cores accumulate in fp32,
// and s_q joins the logit scale: z_t = sm_scale * log2(e) * kv_scale * s_q * sum_d c_d k_t,d.
#pragma once

#include "kvq_mfma.h"

namespace kvq {

typedef long fp8x8_t;  // one lane's 8 FP8 k-slots of a v_mfma_f32_16x16x32_{fp8,bf8}_fp8 operand

constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float q_fp8_scale(float amax) {
    return amax > 0.0f ? amax / kE4M3Max : 1.0f;  // one correctly rounded fp32 division
}

// 8 fp16 query values -> their 8 E4M3 codes under scale s, byte i = value i
__device__ __forceinline__ fp8x8_t q_fp8_codes8(half8_v x, float s) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i)
        w[i >> 2] |= encode_fp8<KVQ_FP8_E4M3>((float)x[i] / s) << (8 * (i & 3));
    return (fp8x8_t)(((uint64_t)w[1] << 32) | w[0]);
}

__device__ __forceinline__ float abs_max8(half8_v x, float m) {
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf((float)x[i]));
    return m;
}

// One query row held by the four lanes col, col + 16, col + 32, col + 48 (32 values each, in the
// four half8 operands x[0..3]): its scale and this lane's codes.  Every lane of the wave calls it.
__device__ __forceinline__ float quantize_q_row_fp8(const half8_v (&x)[4], fp8x8_t (&c)[4]) {
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) m = abs_max8(x[k], m);
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    const float s = q_fp8_scale(m);
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = q_fp8_codes8(x[k], s);
    return s;
}

// Two dwords of K codes (8 consecutive dims of one token) as an MFMA operand.
__device__ __forceinline__ fp8x8_t k_fp8x8(uint32_t lo, uint32_t hi) {
    return (fp8x8_t)(((uint64_t)hi << 32) | lo);
}

// S^T accumulation of one 32-dim slice: A = K codes (E4M3 or E5M2), B = E4M3 query codes.
template <int DT>
__device__ __forceinline__ float4_t mfma_qk_fp8(fp8x8_t k, fp8x8_t q, float4_t acc) {
    if constexpr (DT == KVQ_FP8_E5M2) return __builtin_amdgcn_mfma_f32_16x16x32_bf8_fp8(k, q, acc, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(k, q, acc, 0, 0, 0);
}

struct KernelParams;

// Decode partition kernel with FP8 math (kvq_attn_gqa.hip), any grouping G <= 16; dtype is
// KVQ_FP8_E4M3 or KVQ_FP8_E5M2.
void launch_partition_fp8math(const KernelParams& kp, int dtype, hipStream_t stream, hipEvent_t start,
                              hipEvent_t stop);

}  // namespace kvq
