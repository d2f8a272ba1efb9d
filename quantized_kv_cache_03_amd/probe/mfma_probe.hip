// mfma_probe.hip -- one matrix instruction per 16x16 problem, as the attention kernels issue it,
// so that tests can hold its accumulation against exact products:
//   v_mfma_f32_16x16x32_f16                 (the fp16-math QK^T and PV tiles),
//   v_mfma_scale_f32_16x16x128_f8f6f4       (the FP8-math QK^T tile, unit scales).
// A test aid beside libkvq.so, not part of the cache's ABI.
//
// Problem p: C = C_in + A B with A [16][K] (row i, k), B given by columns (b[p][j][k] = B[k][j]) and
// C [16][16] (row i, column j).  Lane l holds row / column l % 16 of A / B with k-slots
// (K / 4) (l / 16) .. +K/4-1, and rows 4 (l / 16) .. +3 of column l % 16 of C -- the operand layout of
// the kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 half8_v __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(64) void mfma_f16(const uint16_t* a, const uint16_t* b, const float* c_in,
                                               float* c_out) {
    const int p = blockIdx.x, l = threadIdx.x, col = l & 15, kg = l >> 4;
    half8_v x, y;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x[e] = __builtin_bit_cast(_Float16, a[((size_t)p * 16 + col) * 32 + 8 * kg + e]);
        y[e] = __builtin_bit_cast(_Float16, b[((size_t)p * 16 + col) * 32 + 8 * kg + e]);
    }
    float4_t acc;
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = c_in[((size_t)p * 16 + 4 * kg + u) * 16 + col];
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, y, acc, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) c_out[((size_t)p * 16 + 4 * kg + u) * 16 + col] = acc[u];
}

// FMT_A / FMT_B: 0 = E4M3, 1 = E5M2 (the instruction's format codes)
template <int FMT_A, int FMT_B>
__global__ __launch_bounds__(64) void mfma_fp8(const uint8_t* a, const uint8_t* b, const float* c_in,
                                               float* c_out) {
    const int p = blockIdx.x, l = threadIdx.x, col = l & 15, kg = l >> 4;
    const uint32_t* ar = reinterpret_cast<const uint32_t*>(a + ((size_t)p * 16 + col) * 128 + 32 * kg);
    const uint32_t* br = reinterpret_cast<const uint32_t*>(b + ((size_t)p * 16 + col) * 128 + 32 * kg);
    i32x8 x, y;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x[e] = (int)ar[e];
        y[e] = (int)br[e];
    }
    float4_t acc;
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = c_in[((size_t)p * 16 + 4 * kg + u) * 16 + col];
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, acc, FMT_A, FMT_B, 0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) c_out[((size_t)p * 16 + 4 * kg + u) * 16 + col] = acc[u];
}

}  // namespace

// n problems of fp16 a [n][16][32], b [n][16][32] (by column), fp32 c_in, c_out [n][16][16], all
// device memory.  Returns 0, -1 for bad arguments, or the HIP error code at launch.
extern "C" int kvq_probe_mfma_f16(const void* a, const void* b, const float* c_in, float* c_out, int32_t n,
                                  void* stream) {
    if (!a || !b || !c_in || !c_out || n <= 0 || n > 65535) return -1;
    mfma_f16<<<dim3((unsigned)n), dim3(64), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), c_in, c_out);
    return (int)hipGetLastError();
}

// n problems of FP8 codes a [n][16][128], b [n][16][128] (by column); fmt_a, fmt_b: 0 = E4M3,
// 1 = E5M2.  As kvq_probe_mfma_f16 otherwise.
extern "C" int kvq_probe_mfma_fp8(const void* a, const void* b, int32_t fmt_a, int32_t fmt_b,
                                  const float* c_in, float* c_out, int32_t n, void* stream) {
    if (!a || !b || !c_in || !c_out || n <= 0 || n > 65535 || fmt_a < 0 || fmt_a > 1 || fmt_b < 0 ||
        fmt_b > 1)
        return -1;
    const dim3 grid((unsigned)n), block(64);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t* pa = static_cast<const uint8_t*>(a);
    const uint8_t* pb = static_cast<const uint8_t*>(b);
    if (fmt_a == 0 && fmt_b == 0) mfma_fp8<0, 0><<<grid, block, 0, s>>>(pa, pb, c_in, c_out);
    else if (fmt_a == 0) mfma_fp8<0, 1><<<grid, block, 0, s>>>(pa, pb, c_in, c_out);
    else if (fmt_b == 0) mfma_fp8<1, 0><<<grid, block, 0, s>>>(pa, pb, c_in, c_out);
    else mfma_fp8<1, 1><<<grid, block, 0, s>>>(pa, pb, c_in, c_out);
    return (int)hipGetLastError();
}

// The INT4 kernels' K operand path on its own: for problem p, lane l takes the 16 bytes
// codes[p][l] (32 nibbles), decodes them with int4x8_centred around the zero code c0[p] (the even
// pairs as c - c0, the odd ones as 16 (c - c0)), writes the four decoded dwords of each of its
// 4 code dwords to dec[p][l][16], and issues the kernels' four matrix instructions against the
// fp16 query operands qop[p][l][4][8] (the even operands into one accumulator, the odd into
// another), writing S = se + so / 16 to s_out[p][l][4].
#include "kvq_int4.h"
namespace {
__global__ __launch_bounds__(64) void int4_centred(const uint32_t* codes, const float* c0s,
                                                   const uint16_t* qop, uint32_t* dec, float* s_out) {
    const int p = blockIdx.x, l = threadIdx.x;
    const uint32_t* w = codes + ((size_t)p * 64 + l) * 4;
    kvq::half2_t ne, no;
    kvq::int4_centre_pairs(c0s[p], ne, no);
    const kvq::Int4Bits bits = kvq::int4_bits();
    kvq::half2_t h[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        kvq::int4x8_centred(w[j], ne, no, bits, h[j]);
#pragma unroll
        for (int k = 0; k < 4; ++k) dec[((size_t)p * 64 + l) * 16 + 4 * j + k] = __builtin_bit_cast(uint32_t, h[j][k]);
    }
    const half8_v e0 = {h[0][0].x, h[0][0].y, h[0][2].x, h[0][2].y, h[1][0].x, h[1][0].y, h[1][2].x, h[1][2].y};
    const half8_v o0 = {h[0][1].x, h[0][1].y, h[0][3].x, h[0][3].y, h[1][1].x, h[1][1].y, h[1][3].x, h[1][3].y};
    const half8_v e1 = {h[2][0].x, h[2][0].y, h[2][2].x, h[2][2].y, h[3][0].x, h[3][0].y, h[3][2].x, h[3][2].y};
    const half8_v o1 = {h[2][1].x, h[2][1].y, h[2][3].x, h[2][3].y, h[3][1].x, h[3][1].y, h[3][3].x, h[3][3].y};
    half8_v q[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) q[m][e] = __builtin_bit_cast(_Float16, qop[(((size_t)p * 64 + l) * 4 + m) * 8 + e]);
    float4_t se = {0.0f, 0.0f, 0.0f, 0.0f}, so = {0.0f, 0.0f, 0.0f, 0.0f};
    se = __builtin_amdgcn_mfma_f32_16x16x32_f16(e0, q[0], se, 0, 0, 0);
    so = __builtin_amdgcn_mfma_f32_16x16x32_f16(o0, q[1], so, 0, 0, 0);
    se = __builtin_amdgcn_mfma_f32_16x16x32_f16(e1, q[2], se, 0, 0, 0);
    so = __builtin_amdgcn_mfma_f32_16x16x32_f16(o1, q[3], so, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) s_out[((size_t)p * 64 + l) * 4 + u] = se[u] + so[u] * 0.0625f;
}
}  // namespace

// n problems: codes uint32 [n][64][4], c0 float [n], qop fp16 [n][64][4][8], dec uint32 [n][64][16],
// s_out float [n][64][4]; device memory.  Returns 0, -1 for bad arguments, or the HIP error code.
extern "C" int kvq_probe_int4_centred(const uint32_t* codes, const float* c0, const void* qop, uint32_t* dec,
                                      float* s_out, int32_t n, void* stream) {
    if (!codes || !c0 || !qop || !dec || !s_out || n <= 0 || n > 65535) return -1;
    int4_centred<<<dim3((unsigned)n), dim3(64), 0, static_cast<hipStream_t>(stream)>>>(
        codes, c0, static_cast<const uint16_t*>(qop), dec, s_out);
    return (int)hipGetLastError();
}

// The INT4 kernels' V operand decode on its own (int4x8_exact, the FP8 converter with scale 2^9):
// for problem p, lane l decodes its four code dwords codes[p][l][4] and writes each one's four
// binary16 pairs -- nibbles (0, 2), (4, 6), (1, 3), (5, 7) -- to dec[p][l][16].
namespace {
__global__ __launch_bounds__(64) void int4_exact(const uint32_t* codes, uint32_t* dec) {
    const int p = blockIdx.x, l = threadIdx.x;
    const uint32_t* w = codes + ((size_t)p * 64 + l) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        kvq::half2_t h[4];
        kvq::int4x8_exact(w[j], h);
#pragma unroll
        for (int k = 0; k < 4; ++k) dec[((size_t)p * 64 + l) * 16 + 4 * j + k] = __builtin_bit_cast(uint32_t, h[k]);
    }
}
}  // namespace

// n problems: codes uint32 [n][64][4], dec uint32 [n][64][16]; device memory.  Returns 0, -1 for bad
// arguments, or the HIP error code.
extern "C" int kvq_probe_int4_exact(const uint32_t* codes, uint32_t* dec, int32_t n, void* stream) {
    if (!codes || !dec || n <= 0 || n > 65535) return -1;
    int4_exact<<<dim3((unsigned)n), dim3(64), 0, static_cast<hipStream_t>(stream)>>>(codes, dec);
    return (int)hipGetLastError();
}
