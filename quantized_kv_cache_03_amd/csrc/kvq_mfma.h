// kvq_mfma.h -- fp16 operands of v_mfma_f32_16x16x32_f16 built from 8-bit codes, and the
// column-wise helpers of kernels that keep a 16x16 accumulator (lane l: column l % 16, rows
// 4 (l / 16) .. +3).
#pragma once

#include "kvq_device.h"

namespace kvq {

// One lane's 8 k-slots of an MFMA operand.
typedef _Float16 half8_v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ half8_v join8(half2_t a, half2_t b, half2_t c, half2_t d) {
    return half8_v{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// 8 consecutive codes (two dwords) -> their exact fp16 values, in byte order
template <int DT>
__device__ __forceinline__ half8_v codes8(uint32_t w0, uint32_t w1) {
    return join8(codes_to_f16<DT, 0>(w0), codes_to_f16<DT, 1>(w0), codes_to_f16<DT, 0>(w1),
                 codes_to_f16<DT, 1>(w1));
}

// Max and sum over the four lanes of a column (l, l ^ 16, l ^ 32, l ^ 48), every lane getting the
// result.  v_permlane16_swap / v_permlane32_swap of (x, x) leave the two rows (halves) of each pair
// in the two results, so one VALU operation per step replaces an LDS permute; each lane of a pair
// combines the same two values in the same order, so the results agree bitwise.  (No inline
// assembly here or below: the compiler's hazard recognizer does not see the registers an asm
// statement writes, and a matrix instruction reading them too early takes stale values.)
__device__ __forceinline__ float col_max4(float x) {
    uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    u = __float_as_uint(x);
    auto r2 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
}
__device__ __forceinline__ float col_sum4(float x) {
    uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    u = __float_as_uint(x);
    auto r2 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
}

// Two fp32 weights -> packed fp16 hi parts and lo parts f16(w - f32(hi)) (w - hi is exact in fp32):
// one packed round-toward-zero conversion for the hi parts (v_cvt_pkrtz_f16_f32), and the lo parts
// as fused multiply-adds of each hi half with -1, one mixed-precision v_fma_mix per value reading its
// half of the packed register.  Three instructions per pair: with round-to-nearest hi parts the
// compiler converts each weight a second time for the v_fma_mix inputs (five).  hi + lo keeps
// ~21 significant bits of w (|w - hi| < one fp16 ulp, lo rounded to nearest).  The -1 comes from an
// identity DPP move: as a literal the compiler folds the multiply-add back into a subtraction.
__device__ __forceinline__ float opaque_neg_one() {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                         __builtin_amdgcn_mov_dpp((int)0xBF800000u, 0xE4, 0xF, 0xF, false)));
}
__device__ __forceinline__ void split_hi_lo(float w0, float w1, uint32_t& hi, uint32_t& lo) {
    const half2_t h = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(w0, w1));
    const float m1 = opaque_neg_one();
    const half2_t l = {(_Float16)__builtin_fmaf(m1, (float)h.x, w0), (_Float16)__builtin_fmaf(m1, (float)h.y, w1)};
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
}

}  // namespace kvq
