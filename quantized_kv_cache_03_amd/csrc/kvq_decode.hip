// kvq_decode.hip -- decode-step attention over the paged 8-bit KV cache: the merge of split-K
// partials and the launch sequence.
//
// The work of each (head, sequence) is split into pieces (fixed partitions, or equal shares of the
// whole batch's tiles), each run by one wave of a partition kernel -- kvq_attn_mha.hip for one
// query head per KV head, kvq_attn_gqa.hip for grouped heads -- which writes the final output when
// it holds a whole sequence and otherwise an fp32 (max, sum, unnormalized output) partial.  A
// second kernel merges the partials with the log-sum-exp rule (flash-decoding split-K).  A fused
// decode step appends the new token inside the partition kernel (see the two kernel files).
#include "kvq_attn.h"
#include "kvq_fp8m.h"
#include "kvq_int4.h"

namespace kvq {

// ------------------------------------------------------------------------------------------------
// Merge of the np partials in rows r0 .. r0 + np - 1 of one (sequence, query head), by one wave:
//   M = max_p m_p,  out = v_scale * sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// Lane l sums dims 4 (l % 32) .. +3 over the partials of parity l / 32 (two partial rows per load
// instruction, four loads in flight), and the two halves are added at the end.  The order of the
// sums is fixed, so the result is bitwise deterministic.
__device__ __forceinline__ void merge_rows(const KernelParams& a, int64_t r0, int np, size_t orow,
                                           int lane) {
    float M = kNegInf;
    for (int p0 = 0; p0 < np; p0 += 64)
        M = fmaxf(M, (p0 + lane < np) ? a.part_m[r0 + p0 + lane] : kNegInf);
    M = wave_max(M);
    const int d4 = (lane & 31) * 4;
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float L = 0.0f;
#pragma unroll 4
    for (int p = lane >> 5; p < np; p += 2) {
        const float w = __builtin_amdgcn_exp2f(a.part_m[r0 + p] - M);
        L += w * a.part_l[r0 + p];
        const float4_t o = *reinterpret_cast<const float4_t*>(a.part_o + (r0 + p) * kDim + d4);
        acc += w * o;
    }
    L += __shfl_xor(L, 32);
    acc.x += __shfl_xor(acc.x, 32);
    acc.y += __shfl_xor(acc.y, 32);
    acc.z += __shfl_xor(acc.z, 32);
    acc.w += __shfl_xor(acc.w, 32);
    if (lane < 32) {
        const float inv = a.v_scale / L;
        const half4_t r = {(_Float16)(acc.x * inv), (_Float16)(acc.y * inv), (_Float16)(acc.z * inv),
                           (_Float16)(acc.w * inv)};
        *reinterpret_cast<half4_t*>(a.out + orow + d4) = r;
    }
}

// Merge kernel, one wave per (query head, sequence): combines the partials of a sequence whose work
// was split; with the balanced split it also writes the zeros of empty sequences.
__global__ __launch_bounds__(64) void attn_merge(KernelParams a) {
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x;
    const int n = a.ctx[b];
    const size_t orow = ((size_t)b * a.Hq + h) * kDim;
    if (a.NW > 0) {
        const int nt = tiles_of(n);
        if (nt == 0) {
            a.out[orow + lane] = 0;
            a.out[orow + 64 + lane] = 0;
            return;
        }
        const int T = a.plan[a.B], nw = a.plan[a.B + 1];
        const int c0 = a.plan[b];
        const int wlo = wave_of_tile(c0, T, nw), whi = wave_of_tile(c0 + nt - 1, T, nw);
        if (wlo == whi) return;  // one wave held the whole sequence and wrote the output
        merge_rows(a, (int64_t)h * a.S + wlo + b, whi - wlo + 1, orow, lane);
    } else {
        const int np = min((n + a.PS - 1) / a.PS, a.P);
        if (np <= 1) return;  // written directly by the partition kernel
        merge_rows(a, ((int64_t)b * a.Hq + h) * a.P, np, orow, lane);
    }
}

// ------------------------------------------------------------------------------------------------
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, hipEvent_t main_begin,
                         hipEvent_t main_end) {
    const kvq_cache& c = *a.cache;
    if (a.batch == 0) return hipSuccess;
    KernelParams kp;
    kp.kc = c.k_cache;
    kp.vc = c.v_cache;
    kp.ks = c.k_scale;
    kp.vs = c.v_scale;
    kp.q = a.q;
    kp.out = a.out;
    kp.part_o = a.part_o;
    kp.part_m = a.part_m;
    kp.part_l = a.part_l;
    kp.plan = a.plan;
    kp.block_tables = a.block_tables;
    kp.ctx = a.context_lens;
    kp.max_blocks = a.max_blocks_per_seq;
    kp.B = a.batch;
    kp.Hq = a.num_q_heads;
    kp.Hkv = c.num_kv_heads;
    kp.P = a.num_partitions;
    kp.PS = a.partition_size;
    kp.NW = a.balanced_waves;
    kp.S = a.balanced_waves + a.batch;
    const bool fp8 = is_fp8(c.dtype);
    // the decoders give code values divided by code_unit (a power of two): fold it into the scales
    const float unit_scale = fp8 ? c.kv_scale * code_unit(c.dtype) : 1.0f;
    kp.qk_scale = a.sm_scale * kLog2e * unit_scale;
    kp.v_scale = unit_scale;
    kp.kv_scale = c.kv_scale;
    kp.k_new = a.k_new;
    kp.v_new = a.v_new;

    if (a.fp8_math)
        launch_partition_fp8math(kp, c.dtype, stream, main_begin, main_end);
    else if (c.dtype == KVQ_INT4 && kp.Hq == kp.Hkv)
        launch_partition_mha4(kp, stream, main_begin, main_end);
    else if (c.dtype == KVQ_INT4)
        launch_partition_gqa4(kp, stream, main_begin, main_end);
    else if (kp.Hq == kp.Hkv)
        launch_partition_mha(kp, c.dtype, stream, main_begin, main_end);
    else
        launch_partition_gqa(kp, c.dtype, stream, main_begin, main_end);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (kp.NW > 0 || kp.P > 1) {
        attn_merge<<<dim3((unsigned)a.num_q_heads, (unsigned)a.batch), 64, 0, stream>>>(kp);
        e = hipGetLastError();
    }
    return e;
}

// ------------------------------------------------------------------------------------------------
// FP8 math query quantization, standalone: one wave per row, lane l holding dims 2l, 2l + 1.
__global__ __launch_bounds__(64) void quantize_q_fp8_kernel(const uint16_t* q, uint8_t* codes,
                                                            float* scales) {
    const int lane = threadIdx.x;
    const size_t row = blockIdx.x;
    const half2_t x = *reinterpret_cast<const half2_t*>(q + row * kDim + 2 * lane);
    const float s = q_fp8_scale(wave_max(fmaxf(fabsf((float)x.x), fabsf((float)x.y))));
    const uint32_t c = encode_fp8<KVQ_FP8_E4M3>((float)x.x / s) |
                       (encode_fp8<KVQ_FP8_E4M3>((float)x.y / s) << 8);
    *reinterpret_cast<uint16_t*>(codes + row * kDim + 2 * lane) = (uint16_t)c;
    if (lane == 0) scales[row] = s;
}

hipError_t launch_quantize_q_fp8(const uint16_t* q, int32_t num_rows, uint8_t* codes, float* scales,
                                 hipStream_t stream) {
    if (num_rows == 0) return hipSuccess;
    quantize_q_fp8_kernel<<<dim3((unsigned)num_rows), 64, 0, stream>>>(q, codes, scales);
    return hipGetLastError();
}

}  // namespace kvq
