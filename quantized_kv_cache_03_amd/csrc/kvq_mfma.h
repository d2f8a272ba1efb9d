// kvq_mfma.h -- fp16 operands of v_mfma_f32_16x16x32_f16 built from 8-bit codes.
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

}  // namespace kvq
