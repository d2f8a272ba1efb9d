// kvq_decode.hip -- decode-step attention over the paged 8-bit KV cache.
//
// The cache is stored as 8-bit codes and the attention arithmetic runs at higher precision
// ("Accelerating Inference with FP8 KV Cache", opening section): codes are decoded exactly to
// fp16, the dot products use fp16 inputs with fp32 accumulation, softmax statistics are fp32.
// Long contexts are split into partitions whose (max, sum, unnormalized output) partials a second
// kernel merges with the log-sum-exp rule (flash-decoding split-K).
//
// Scales are factored out of the sums: logits are  sm_scale * kv_scale * (q . dec(k))  and the
// output is  kv_scale * sum_t p_t dec(v_t) / sum_t p_t  (FP8);  INT8 applies the per-token K
// scale to each logit and folds the per-token V scale into the weight p_t * s_t.  Softmax runs in
// base 2 with log2(e) folded into the logit scale.
//
// Work decomposition (one wave per work item, no LDS):
//   grid (partition, query head, sequence); a wave streams its partition in chunks of TW tiles of
//   16 tokens, issuing every K and V load of a chunk before using any, and keeps a running max /
//   sum / accumulator across chunks.
//   K tile (token-major 16 x 128 B): lane l holds 16 dims of token l/8 (and of token 8 + l/8),
//     dots them with its slice of q (v_dot2_f32_f16), and 8-lane DPP sums finish each logit.
//   V tile (dim-major 128 x 16 B): lane l holds the 16 tokens of dims l and 64 + l, so each lane
//     accumulates whole output elements; the 16 weights of a tile reach every lane as packed fp16
//     (hi, lo) pairs read with v_readlane.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr float kNegInf = -__builtin_huge_valf();

// Keep the low `nbytes` (0..4) bytes of w.
__device__ __forceinline__ uint32_t keep_bytes(uint32_t w, int nbytes) {
    return nbytes >= 4 ? w : (nbytes <= 0 ? 0u : (w & ((1u << (8 * nbytes)) - 1u)));
}

template <int DT>
__device__ __forceinline__ float dot16(const uint4& k, const half2_t* q8) {
    float s = 0.0f;
    s = dot2(codes_to_f16<DT, 0>(k.x), q8[0], s);
    s = dot2(codes_to_f16<DT, 1>(k.x), q8[1], s);
    s = dot2(codes_to_f16<DT, 0>(k.y), q8[2], s);
    s = dot2(codes_to_f16<DT, 1>(k.y), q8[3], s);
    s = dot2(codes_to_f16<DT, 0>(k.z), q8[4], s);
    s = dot2(codes_to_f16<DT, 1>(k.z), q8[5], s);
    s = dot2(codes_to_f16<DT, 0>(k.w), q8[6], s);
    s = dot2(codes_to_f16<DT, 1>(k.w), q8[7], s);
    return s;
}

// acc += sum over the 16 tokens of a V row (16 codes) weighted by w_t = hi_t + lo_t, where the
// packed pairs hi[i] = (hi_{2i}, hi_{2i+1}) and lo[i] likewise are fp16.  The two-term split keeps
// the weights to ~22 significant bits, so rounding them to fp16 does not move the output.
template <int DT>
__device__ __forceinline__ float pv_pair(uint32_t codes4, const uint32_t* hi, const uint32_t* lo,
                                         float acc) {
    const half2_t c0 = codes_to_f16<DT, 0>(codes4), c1 = codes_to_f16<DT, 1>(codes4);
    acc = dot2(c0, __builtin_bit_cast(half2_t, hi[0]), acc);
    acc = dot2(c0, __builtin_bit_cast(half2_t, lo[0]), acc);
    acc = dot2(c1, __builtin_bit_cast(half2_t, hi[1]), acc);
    acc = dot2(c1, __builtin_bit_cast(half2_t, lo[1]), acc);
    return acc;
}
template <int DT>
__device__ __forceinline__ float pv16(const uint4& v, const uint32_t* hi, const uint32_t* lo, float acc) {
    acc = pv_pair<DT>(v.x, hi + 0, lo + 0, acc);
    acc = pv_pair<DT>(v.y, hi + 2, lo + 2, acc);
    acc = pv_pair<DT>(v.z, hi + 4, lo + 4, acc);
    acc = pv_pair<DT>(v.w, hi + 6, lo + 6, acc);
    return acc;
}

// (w_a, w_b) -> packed fp16 hi parts and lo parts
__device__ __forceinline__ void split_f16x2(float wa, float wb, uint32_t& hi, uint32_t& lo) {
    const _Float16 ha = (_Float16)wa, hb = (_Float16)wb;
    hi = __builtin_bit_cast(uint32_t, half2_t{ha, hb});
    lo = pack_f16x2(wa - (float)ha, wb - (float)hb);
}

// pairs (w_2i, w_2i+1) of a tile's 16 weights from lanes 8j, which hold (w_j, w_{8+j})
__device__ __forceinline__ void gather_pairs(uint32_t mine, uint32_t* pw) {
    uint32_t r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = __builtin_amdgcn_readlane(mine, 8 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        pw[j] = (r[2 * j] & 0xFFFFu) | (r[2 * j + 1] << 16);          // tokens 2j, 2j+1
        pw[4 + j] = (r[2 * j] >> 16) | (r[2 * j + 1] & 0xFFFF0000u);  // tokens 8+2j, 9+2j
    }
}

struct KernelParams {
    const uint8_t* kc;
    const uint8_t* vc;
    const float* ks;
    const float* vs;
    const uint16_t* q;
    uint16_t* out;
    float* part_o;
    float* part_m;
    float* part_l;
    const int32_t* block_tables;
    const int32_t* ctx;
    int32_t max_blocks;
    int32_t Hq;
    int32_t Hkv;
    int32_t P;          // partitions in the grid
    int32_t PS;         // tokens per partition
    float qk_scale;     // sm_scale * log2(e) (* kv_scale for FP8)
    float v_scale;      // kv_scale for FP8, 1 for INT8
};

// ------------------------------------------------------------------------------------------------
// Partition kernel, one wave per (partition, query head, sequence).
template <int DT, int TW>
__global__ __launch_bounds__(64) void attn_partition_valu(KernelParams a) {
    const int p = blockIdx.x;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int lane = threadIdx.x;
    const int G = a.Hq / a.Hkv;
    const int g = h / G;

    const int n = a.ctx[b];
    const int np = (n + a.PS - 1) / a.PS;  // partitions this sequence uses
    const size_t orow = ((size_t)b * a.Hq + h) * kDim;
    if (n <= 0) {
        if (p == 0) {
            a.out[orow + lane] = 0;
            a.out[orow + 64 + lane] = 0;
        }
        return;
    }
    if (p >= np) return;
    const int t_begin = p * a.PS;
    const int t_end = min(n, t_begin + a.PS);
    const int tile_begin = t_begin / kBlock;
    const int tile_end = (t_end + kBlock - 1) / kBlock;

    // q slice of this lane's K dims: 16 (lane % 8) .. +15
    half2_t qv[8];
    {
        const uint4* qp = reinterpret_cast<const uint4*>(a.q + orow + (lane & 7) * 16);
        const uint4 q0 = qp[0], q1 = qp[1];
        const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[i] = __builtin_bit_cast(half2_t, qw[i]);
    }

    const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks;
    const size_t head_off = (size_t)g * kTileBytes;
    const size_t blk_stride = (size_t)a.Hkv * kTileBytes;
    const int tok_in_tile = lane >> 3;  // 0..7, the K row this lane reads (and 8 + it)

    float m_run = kNegInf;  // running max of the base-2 logits (wave-uniform)
    float l_lane = 0.0f;    // running sum of weights of this lane's two tokens per tile
    float acc0 = 0.0f, acc1 = 0.0f;  // unnormalized output, dims lane and 64 + lane

    for (int tb = tile_begin; tb < tile_end; tb += 64) {
        // block ids of up to 64 tiles, one per lane
        const int nt_grp = min(64, tile_end - tb);
        const int blk_lane = (lane < nt_grp) ? bt[tb + lane] : 0;

        for (int c0 = 0; c0 < nt_grp; c0 += TW) {
            uint4 ka[TW], kb[TW], va[TW], vb[TW];
            int blks[TW];
#pragma unroll
            for (int i = 0; i < TW; ++i) {
                if (c0 + i < nt_grp) {
                    blks[i] = __builtin_amdgcn_readlane(blk_lane, c0 + i);
                    const uint8_t* kt = a.kc + (size_t)blks[i] * blk_stride + head_off;
                    const uint8_t* vt = a.vc + (size_t)blks[i] * blk_stride + head_off;
                    ka[i] = ldg16(kt + 16 * lane);
                    kb[i] = ldg16(kt + 1024 + 16 * lane);
                    va[i] = ldg16(vt + 16 * lane);
                    vb[i] = ldg16(vt + 1024 + 16 * lane);
                } else {
                    blks[i] = 0;
                    ka[i] = kb[i] = va[i] = vb[i] = make_uint4(0u, 0u, 0u, 0u);
                }
            }
            // logits of the chunk (base 2); lanes of group j hold tokens j and 8 + j of each tile
            float za[TW], zb[TW];
            float cmax = kNegInf;
#pragma unroll
            for (int i = 0; i < TW; ++i) {
                const float sa = sum8(dot16<DT>(ka[i], qv));
                const float sb = sum8(dot16<DT>(kb[i], qv));
                const int tile = tb + c0 + i;
                const int pa = tile * kBlock + tok_in_tile;
                const int pb = pa + 8;
                float fa = a.qk_scale, fb = a.qk_scale;
                if constexpr (DT == KVQ_INT8) {
                    if (c0 + i < nt_grp) {
                        const float* st = a.ks + ((size_t)blks[i] * a.Hkv + g) * kBlock;
                        fa *= st[tok_in_tile];
                        fb *= st[tok_in_tile + 8];
                    }
                }
                const bool in_a = (c0 + i < nt_grp) && pa < t_end;
                const bool in_b = (c0 + i < nt_grp) && pb < t_end;
                za[i] = in_a ? sa * fa : kNegInf;
                zb[i] = in_b ? sb * fb : kNegInf;
                cmax = fmaxf(cmax, fmaxf(za[i], zb[i]));
            }
            cmax = max_across8(cmax);  // every chunk holds at least one valid token
            const float m_new = fmaxf(m_run, cmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            acc0 *= alpha;
            acc1 *= alpha;
            l_lane *= alpha;

#pragma unroll
            for (int i = 0; i < TW; ++i) {
                const float pa = __builtin_amdgcn_exp2f(za[i] - m_new);
                const float pb = __builtin_amdgcn_exp2f(zb[i] - m_new);
                l_lane += pa + pb;
                float wa = pa, wb = pb;
                if constexpr (DT == KVQ_INT8) {
                    if (c0 + i < nt_grp) {
                        const float* st = a.vs + ((size_t)blks[i] * a.Hkv + g) * kBlock;
                        const float sa = st[tok_in_tile], sb = st[tok_in_tile + 8];
                        wa = (pa > 0.0f) ? pa * sa : 0.0f;   // masked slots may hold NaN scales
                        wb = (pb > 0.0f) ? pb * sb : 0.0f;
                    }
                }
                // lane 8j holds (w_j, w_{8+j}); gather the 16 weights as pairs (w_2i, w_2i+1)
                uint32_t mine_hi, mine_lo, whi[8], wlo[8];
                split_f16x2(wa, wb, mine_hi, mine_lo);
                gather_pairs(mine_hi, whi);
                gather_pairs(mine_lo, wlo);
                uint4 v0 = va[i], v1 = vb[i];
                const int tile = tb + c0 + i;
                const int valid = t_end - tile * kBlock;  // tokens of this tile inside the partition
                if (valid < kBlock) {
                    // slots past the end may hold any code, NaN included: zero them (weight 0 alone
                    // would still give 0 * NaN)
                    v0.x = keep_bytes(v0.x, valid); v0.y = keep_bytes(v0.y, valid - 4);
                    v0.z = keep_bytes(v0.z, valid - 8); v0.w = keep_bytes(v0.w, valid - 12);
                    v1.x = keep_bytes(v1.x, valid); v1.y = keep_bytes(v1.y, valid - 4);
                    v1.z = keep_bytes(v1.z, valid - 8); v1.w = keep_bytes(v1.w, valid - 12);
                }
                acc0 = pv16<DT>(v0, whi, wlo, acc0);
                acc1 = pv16<DT>(v1, whi, wlo, acc1);
            }
        }
    }
    // each token's weight was added by all 8 lanes of its group: count group leaders only
    // (lanes 0, 8, .., 56 end with the total; broadcast it from lane 0)
    const float l_lead = sum_across8((lane & 7) == 0 ? l_lane : 0.0f);
    const float l_sum =
        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_lead), 0));

    if (np == 1) {
        const float inv = a.v_scale / l_sum;
        a.out[orow + lane] = __builtin_bit_cast(uint16_t, (_Float16)(acc0 * inv));
        a.out[orow + 64 + lane] = __builtin_bit_cast(uint16_t, (_Float16)(acc1 * inv));
    } else {
        const size_t prow = ((size_t)b * a.Hq + h) * a.P + p;
        a.part_o[prow * kDim + lane] = acc0;
        a.part_o[prow * kDim + 64 + lane] = acc1;
        if (lane == 0) {
            a.part_m[prow] = m_run;
            a.part_l[prow] = l_sum;
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Merge kernel, one wave per (query head, sequence) whose context spans several partitions:
//   M = max_p m_p,  out = v_scale * sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// Partials are read in partition order, so the result is bitwise deterministic.
__global__ __launch_bounds__(64) void attn_merge(KernelParams a) {
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x;
    const int n = a.ctx[b];
    const int np = min((n + a.PS - 1) / a.PS, a.P);
    if (np <= 1) return;  // written directly by the partition kernel
    const size_t prow0 = ((size_t)b * a.Hq + h) * a.P;
    float M = kNegInf;
    for (int p = 0; p < np; ++p) M = fmaxf(M, a.part_m[prow0 + p]);
    float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int p = 0; p < np; ++p) {
        const float w = __builtin_amdgcn_exp2f(a.part_m[prow0 + p] - M);
        L += w * a.part_l[prow0 + p];
        const float2 op = reinterpret_cast<const float2*>(a.part_o + (prow0 + p) * kDim)[lane];
        o0 += w * op.x;
        o1 += w * op.y;
    }
    const float inv = a.v_scale / L;
    const size_t orow = ((size_t)b * a.Hq + h) * kDim;
    half2_t r = {(_Float16)(o0 * inv), (_Float16)(o1 * inv)};
    reinterpret_cast<half2_t*>(a.out + orow)[lane] = r;
}

// ------------------------------------------------------------------------------------------------
template <int DT>
static void launch_partition(const KernelParams& kp, dim3 grid, hipStream_t stream) {
    attn_partition_valu<DT, 4><<<grid, 64, 0, stream>>>(kp);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, hipEvent_t main_begin,
                         hipEvent_t main_end, hipEvent_t merge_begin, hipEvent_t merge_end) {
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
    kp.block_tables = a.block_tables;
    kp.ctx = a.context_lens;
    kp.max_blocks = a.max_blocks_per_seq;
    kp.Hq = a.num_q_heads;
    kp.Hkv = c.num_kv_heads;
    kp.P = a.num_partitions;
    kp.PS = a.partition_size;
    const bool fp8 = c.dtype != KVQ_INT8;
    kp.qk_scale = a.sm_scale * kLog2e * (fp8 ? c.kv_scale : 1.0f);
    kp.v_scale = fp8 ? c.kv_scale : 1.0f;

    const dim3 grid((unsigned)a.num_partitions, (unsigned)a.num_q_heads, (unsigned)a.batch);
    if (main_begin) (void)hipEventRecord(main_begin, stream);
    switch (c.dtype) {
        case KVQ_FP8_E4M3: launch_partition<KVQ_FP8_E4M3>(kp, grid, stream); break;
        case KVQ_FP8_E5M2: launch_partition<KVQ_FP8_E5M2>(kp, grid, stream); break;
        default: launch_partition<KVQ_INT8>(kp, grid, stream); break;
    }
    if (main_end) (void)hipEventRecord(main_end, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.num_partitions > 1) {
        if (merge_begin) (void)hipEventRecord(merge_begin, stream);
        attn_merge<<<dim3((unsigned)a.num_q_heads, (unsigned)a.batch), 64, 0, stream>>>(kp);
        if (merge_end) (void)hipEventRecord(merge_end, stream);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace kvq
