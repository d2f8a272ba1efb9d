// kvq_append.hip -- quantize new K/V rows into their paged slots.
//
// FP8: code = enc(fl32(x / kv_scale)) per element ("Accelerating Inference with FP8 KV Cache",
// section "FP8 Formats: E4M3 and E5M2": E4M3/E5M2 with a per-tensor FP32 scale; section "Current
// Hardware Support": AMD's E4M3FNUZ).
// INT8: one fp32 scale per (token, KV head) row, s = fl32(amax / 127), q = clamp(rne(x / s))
// (the online INT8 cache of "[Feature] TurboMind support W8A8 or FP8 KV Cache").
// INT4 (named there beside INT8): one fp32 (scale, zero point) pair per row, zp = min x,
// s = fl32(fl32(max x - zp) / 15), q = clamp(rne(fl32(fl32(x - zp) / s)), 0, 15), two codes per byte.
//
// One wave per (new row, KV head): lane l owns dims 2l and 2l+1 of the K row and the V row.
// The append moves one token per sequence per decode step, so its cost is negligible next to the
// attention read; it is written for exactness, not speed: a correctly rounded fp32 division
// (hipcc's default), integer rounding on the binary32 pattern, no contraction.
#include "kvq_device.h"
#include "kvq_int4.h"
#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {

// Sequence of a row from the row offsets: the last b with cu[b] <= row (empty sequences are
// skipped because their successor has the same offset).
__device__ __forceinline__ int seq_of_row(const int32_t* cu, int batch, int row) {
    int lo = 0, hi = batch;  // invariant: cu[lo] <= row < cu[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= row) lo = mid;
        else hi = mid;
    }
    return lo;
}

template <int DT>
__global__ __launch_bounds__(64) void append_kernel(
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, float* __restrict__ ks,
    float* __restrict__ vs, float kv_scale, const uint32_t* __restrict__ k_new,
    const uint32_t* __restrict__ v_new, const int32_t* __restrict__ cu, int32_t batch,
    const int32_t* __restrict__ block_tables, int32_t max_blocks, const int32_t* __restrict__ ctx,
    int32_t Hkv) {
    const int row = blockIdx.x;
    const int g = blockIdx.y;
    const int lane = threadIdx.x;

    int b, n_b, j;
    if (cu == nullptr) {
        b = row; n_b = 1; j = 0;
    } else {
        b = seq_of_row(cu, batch, row);
        n_b = cu[b + 1] - cu[b];
        j = row - cu[b];
    }
    const int p = ctx[b] - n_b + j;
    if (p < 0 || p / kBlock >= max_blocks) return;  // outside the documented contract: write nothing
    const int blk = block_tables[(size_t)b * max_blocks + p / kBlock];
    const int t = p % kBlock;
    const size_t tile = ((size_t)blk * Hkv + g) * kTileBytes;

    // two fp16 values per lane, K and V
    const size_t src = ((size_t)row * Hkv + g) * (kDim / 2) + lane;
    const uint32_t kw = k_new[src];
    const uint32_t vw = v_new[src];
    const float k0 = half_bits_to_float(kw & 0xFFFFu), k1 = half_bits_to_float(kw >> 16);
    const float v0 = half_bits_to_float(vw & 0xFFFFu), v1 = half_bits_to_float(vw >> 16);

    uint32_t kc0, kc1, vc0, vc1;
    if constexpr (DT == KVQ_INT8) {
        const float ka = wave_max(fmaxf(fabsf(k0), fabsf(k1)));
        const float va = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
        const float sk = ka / 127.0f;  // 0 for an all-zero row
        const float sv = va / 127.0f;
        kc0 = encode_int8(k0, sk);
        kc1 = encode_int8(k1, sk);
        vc0 = encode_int8(v0, sv);
        vc1 = encode_int8(v1, sv);
        if (lane == 0) {
            const size_t so = int8_scale_index(blk, Hkv, g, t);
            ks[so] = sk;
            vs[so] = sv;
        }
    } else {
        kc0 = encode_fp8<DT>(k0 / kv_scale);
        kc1 = encode_fp8<DT>(k1 / kv_scale);
        vc0 = encode_fp8<DT>(v0 / kv_scale);
        vc1 = encode_fp8<DT>(v1 / kv_scale);
    }
    // K tile is chunked [8][16 tokens][16 dims]: dims 2l and 2l+1 are adjacent in one chunk
    *reinterpret_cast<uint16_t*>(kc + tile + k_byte(t, 2 * lane)) = (uint16_t)(kc0 | (kc1 << 8));
    // V tile is dim-major [128][16]: the two codes sit 16 bytes apart
    vc[tile + (size_t)(2 * lane) * kBlock + t] = (uint8_t)vc0;
    vc[tile + (size_t)(2 * lane + 1) * kBlock + t] = (uint8_t)vc1;
}

// INT4: one wave per (new row, KV head), lane l owning dims 2l and 2l+1.  The two K codes of a lane
// make one whole byte of the token's K row.  A V byte holds two tokens of one dim, so a lane
// replaces its token's nibble in the two V bytes with a 32-bit atomic AND (clear) and OR (set) of
// the enclosing dword: another wave may be writing the neighbouring token's nibble of the same byte
// in the same launch, and the atomics keep both.
__global__ __launch_bounds__(64) void append_kernel4(
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, float* __restrict__ ks, float* __restrict__ vs,
    const uint32_t* __restrict__ k_new, const uint32_t* __restrict__ v_new,
    const int32_t* __restrict__ cu, int32_t batch, const int32_t* __restrict__ block_tables,
    int32_t max_blocks, const int32_t* __restrict__ ctx, int32_t Hkv) {
    const int row = blockIdx.x;
    const int g = blockIdx.y;
    const int lane = threadIdx.x;

    int b, n_b, j;
    if (cu == nullptr) {
        b = row; n_b = 1; j = 0;
    } else {
        b = seq_of_row(cu, batch, row);
        n_b = cu[b + 1] - cu[b];
        j = row - cu[b];
    }
    const int p = ctx[b] - n_b + j;
    if (p < 0 || p / kBlock >= max_blocks) return;  // outside the documented contract: write nothing
    const int blk = block_tables[(size_t)b * max_blocks + p / kBlock];
    const int t = p % kBlock;
    const size_t tile = ((size_t)blk * Hkv + g) * kTileBytes4;

    const size_t src = ((size_t)row * Hkv + g) * (kDim / 2) + lane;
    const uint32_t kw = k_new[src];
    const uint32_t vw = v_new[src];
    const float k0 = half_bits_to_float(kw & 0xFFFFu), k1 = half_bits_to_float(kw >> 16);
    const float v0 = half_bits_to_float(vw & 0xFFFFu), v1 = half_bits_to_float(vw >> 16);
    const float kz = wave_min(fminf(k0, k1)), vz = wave_min(fminf(v0, v1));
    const float ksc = (wave_max(fmaxf(k0, k1)) - kz) / 15.0f;  // 0 for a constant row
    const float vsc = (wave_max(fmaxf(v0, v1)) - vz) / 15.0f;
    const uint32_t kq = encode_int4(k0, kz, ksc) | (encode_int4(k1, kz, ksc) << 4);
    kc[tile + k_byte4(t, 2 * lane)] = (uint8_t)kq;
    const uint32_t vq[2] = {encode_int4(v0, vz, vsc), encode_int4(v1, vz, vsc)};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t byte = v_byte4(t, 2 * lane + i);
        const uint32_t sh = 8u * (byte & 3u) + 4u * (uint32_t)(t & 1);
        unsigned int* dw = reinterpret_cast<unsigned int*>(vc + tile + (byte & ~3u));
        atomicAnd(dw, ~(0xFu << sh));
        atomicOr(dw, vq[i] << sh);
    }
    if (lane == 0) {
        const size_t so = (((size_t)blk * Hkv + g) * kBlock + t) * 2;
        *reinterpret_cast<f32x2*>(ks + so) = f32x2{ksc, kz};
        *reinterpret_cast<f32x2*>(vs + so) = f32x2{vsc, vz};
    }
}

hipError_t launch_append(const kvq_cache& c, const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* cu_new_lens, int32_t num_rows, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch,
                         hipStream_t stream) {
    if (num_rows == 0 || batch == 0) return hipSuccess;
    const dim3 grid((unsigned)num_rows, (unsigned)c.num_kv_heads);
    const auto* kw = reinterpret_cast<const uint32_t*>(k_new);
    const auto* vw = reinterpret_cast<const uint32_t*>(v_new);
    switch (c.dtype) {
        case KVQ_FP8_E4M3:
            append_kernel<KVQ_FP8_E4M3><<<grid, 64, 0, stream>>>(
                c.k_cache, c.v_cache, c.k_scale, c.v_scale, c.kv_scale, kw, vw, cu_new_lens, batch,
                block_tables, max_blocks_per_seq, context_lens, c.num_kv_heads);
            break;
        case KVQ_FP8_E5M2:
            append_kernel<KVQ_FP8_E5M2><<<grid, 64, 0, stream>>>(
                c.k_cache, c.v_cache, c.k_scale, c.v_scale, c.kv_scale, kw, vw, cu_new_lens, batch,
                block_tables, max_blocks_per_seq, context_lens, c.num_kv_heads);
            break;
        case KVQ_FP8_E4M3FNUZ:
            append_kernel<KVQ_FP8_E4M3FNUZ><<<grid, 64, 0, stream>>>(
                c.k_cache, c.v_cache, c.k_scale, c.v_scale, c.kv_scale, kw, vw, cu_new_lens, batch,
                block_tables, max_blocks_per_seq, context_lens, c.num_kv_heads);
            break;
        case KVQ_INT4:
            append_kernel4<<<grid, 64, 0, stream>>>(c.k_cache, c.v_cache, c.k_scale, c.v_scale, kw, vw,
                                                    cu_new_lens, batch, block_tables,
                                                    max_blocks_per_seq, context_lens, c.num_kv_heads);
            break;
        default:
            append_kernel<KVQ_INT8><<<grid, 64, 0, stream>>>(
                c.k_cache, c.v_cache, c.k_scale, c.v_scale, c.kv_scale, kw, vw, cu_new_lens, batch,
                block_tables, max_blocks_per_seq, context_lens, c.num_kv_heads);
            break;
    }
    return hipGetLastError();
}

}  // namespace kvq
