// kvq_dequant.hip -- paged 8-bit (or 4-bit) cache -> dense fp32 rows, through the same decoders the
// attention kernels use.  Each element is fl32(dec(code) * kv_scale) for FP8 ("Accelerating
// Inference with FP8 KV Cache", section "FP8 Formats: E4M3 and E5M2": values carry a per-tensor
// FP32 scale), fl32(q * s) for INT8 and fl32(q * s + zp) for INT4: the decoder gives the exact code
// value, the product (or multiply-add) is one fp32 rounding.  A test and inspection aid; not on the
// decode-step path.
#include "kvq_device.h"
#include "kvq_int4.h"
#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {

// The exact value of a code from the decoder's fp16 result f (code = the low byte of `code`): the
// decoders' unit is folded back in (a power of two, exact), and E4M3FNUZ's NaN code, which the
// attention kernels' decoder does not single out, becomes NaN.
template <int DT>
__device__ __forceinline__ float code_value(float f, uint32_t code) {
    if constexpr (DT == KVQ_FP8_E4M3FNUZ) {
        if ((code & 0xFFu) == 0x80u) return __builtin_nanf("");
        return f * code_unit(DT);
    }
    return f;
}

// One wave per (tile of 16 tokens, KV head, sequence).
template <int DT>
__global__ __launch_bounds__(64) void dequant_kernel(
    const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc, const float* __restrict__ ks,
    const float* __restrict__ vs, float kv_scale, const int32_t* __restrict__ block_tables,
    int32_t max_blocks, const int32_t* __restrict__ ctx, int32_t Hkv, int32_t max_ctx,
    float* __restrict__ k_out, float* __restrict__ v_out) {
    const int tile_idx = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int lane = threadIdx.x;
    const int n = ctx[b];
    if (tile_idx * kBlock >= n) return;
    const int blk = block_tables[(size_t)b * max_blocks + tile_idx];
    const size_t tile = ((size_t)blk * Hkv + g) * kTileBytes;
    const size_t sbase = int8_scale_index(blk, Hkv, g, 0);
    const size_t obase = ((size_t)b * Hkv + g) * (size_t)max_ctx * kDim;

    // K: chunked tile; in each 1 KiB half lane l reads the 16 codes of token l % 16 in chunk
    // 4 half + l / 16 (dims 16 (4 half + l / 16) .. +15).
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int tok = lane & 15;
        const int pos = tile_idx * kBlock + tok;
        const int d0 = (half * 4 + (lane >> 4)) * kChunk;
        const u32x4 w = ldg16(kc + tile + k_byte(tok, d0));
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        const float s = (DT == KVQ_INT8) ? ks[sbase + tok] : kv_scale;
        if (pos < n) {
            float* o = k_out + obase + (size_t)pos * kDim + d0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half2_t lo = codes_to_f16<DT, 0>(ws[i]);
                const half2_t hi = codes_to_f16<DT, 1>(ws[i]);
                const float vals[4] = {(float)lo.x, (float)lo.y, (float)hi.x, (float)hi.y};
#pragma unroll
                for (int k = 0; k < 4; ++k) o[4 * i + k] = code_value<DT>(vals[k], ws[i] >> (8 * k)) * s;
            }
        }
    }
    // V: dim-major tile; lane l reads the 16 tokens of dim l and of dim 64 + l.
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int d = half * 64 + lane;
        const u32x4 w = ldg16(vc + tile + (size_t)d * kBlock);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const half2_t lo = codes_to_f16<DT, 0>(ws[i]);
            const half2_t hi = codes_to_f16<DT, 1>(ws[i]);
            const float vals[4] = {(float)lo.x, (float)lo.y, (float)hi.x, (float)hi.y};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int tok = 4 * i + k;
                const int pos = tile_idx * kBlock + tok;
                if (pos < n) {
                    const float s = (DT == KVQ_INT8) ? vs[sbase + tok] : kv_scale;
                    v_out[obase + (size_t)pos * kDim + d] = code_value<DT>(vals[k], ws[i] >> (8 * k)) * s;
                }
            }
        }
    }
}

// INT4: one wave per (tile of 16 tokens, KV head, sequence); each element is fl32(q * s + zp), one
// rounding (a fused multiply-add).
__global__ __launch_bounds__(64) void dequant_kernel4(
    const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc, const float* __restrict__ ks,
    const float* __restrict__ vs, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ ctx, int32_t Hkv, int32_t max_ctx, float* __restrict__ k_out,
    float* __restrict__ v_out) {
    const int tile_idx = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int lane = threadIdx.x;
    const int n = ctx[b];
    if (tile_idx * kBlock >= n) return;
    const int blk = block_tables[(size_t)b * max_blocks + tile_idx];
    const size_t tile = ((size_t)blk * Hkv + g) * kTileBytes4;
    const size_t sbase = ((size_t)blk * Hkv + g) * kBlock;
    const size_t obase = ((size_t)b * Hkv + g) * (size_t)max_ctx * kDim;
    const f32x2* ksz = reinterpret_cast<const f32x2*>(ks) + sbase;
    const f32x2* vsz = reinterpret_cast<const f32x2*>(vs) + sbase;
    // K: lane l reads the 32 codes of token l % 16 in chunk l / 16 (dims 32 (l / 16) .. +31)
    {
        const int tok = lane & 15;
        const int d0 = (lane >> 4) * 32;
        const int pos = tile_idx * kBlock + tok;
        const u32x4 w = ldg16(kc + tile + k_byte4(tok, d0));
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        const f32x2 sz = ksz[tok];
        if (pos < n) {
            float* o = k_out + obase + (size_t)pos * kDim + d0;
#pragma unroll
            for (int i = 0; i < 32; ++i)
                o[i] = __builtin_fmaf((float)((ws[i / 8] >> (4 * (i % 8))) & 0xFu), sz.x, sz.y);
        }
    }
    // V: lane l reads tokens 4 (l / 16) .. +3 of the dims l % 16 + 16 r, r = 0..7 (unit r is bits
    // 16 (r % 2) .. +15 of dword r / 2)
    {
        const int quad = lane >> 4, dlo = lane & 15;
        const u32x4 w = ldg16(vc + tile + v_byte4(4 * quad, dlo));
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int r = i / 4, d = dlo + 16 * r, tok = 4 * quad + i % 4;
            const int pos = tile_idx * kBlock + tok;
            if (pos < n) {
                const f32x2 sz = vsz[tok];
                v_out[obase + (size_t)pos * kDim + d] =
                    __builtin_fmaf((float)((ws[r / 2] >> (16 * (r % 2) + 4 * (i % 4))) & 0xFu), sz.x, sz.y);
            }
        }
    }
}

hipError_t launch_dequant(const kvq_cache& c, const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t batch, int32_t max_context_len,
                          float* k_out, float* v_out, hipStream_t stream) {
    if (batch == 0 || max_context_len == 0) return hipSuccess;
    const dim3 grid((unsigned)((max_context_len + kBlock - 1) / kBlock), (unsigned)c.num_kv_heads,
                    (unsigned)batch);
#define KVQ_DQ(DT)                                                                                 \
    dequant_kernel<DT><<<grid, 64, 0, stream>>>(c.k_cache, c.v_cache, c.k_scale, c.v_scale,       \
                                                c.kv_scale, block_tables, max_blocks_per_seq,     \
                                                context_lens, c.num_kv_heads, max_context_len,    \
                                                k_out, v_out)
    if (c.dtype == KVQ_INT4) {
        dequant_kernel4<<<grid, 64, 0, stream>>>(c.k_cache, c.v_cache, c.k_scale, c.v_scale, block_tables,
                                                 max_blocks_per_seq, context_lens, c.num_kv_heads,
                                                 max_context_len, k_out, v_out);
        return hipGetLastError();
    }
    switch (c.dtype) {
        case KVQ_FP8_E4M3: KVQ_DQ(KVQ_FP8_E4M3); break;
        case KVQ_FP8_E5M2: KVQ_DQ(KVQ_FP8_E5M2); break;
        case KVQ_FP8_E4M3FNUZ: KVQ_DQ(KVQ_FP8_E4M3FNUZ); break;
        default: KVQ_DQ(KVQ_INT8); break;
    }
#undef KVQ_DQ
    return hipGetLastError();
}

}  // namespace kvq
