// kvq_prefill.hip -- prefill / chunked-prefill attention over the paged 8-bit cache.
//
// Sequence b brings n_b new query rows (rows cu_q[b] .. cu_q[b+1]-1), the last n_b of its
// context_lens[b] tokens; row j sits at position p = context_lens[b] - n_b + j and attends to the
// cache tokens at positions 0 .. p (causal).  Decode is the case n_b = 1.  The cache is stored as
// 8-bit codes and the arithmetic runs at higher precision ("Accelerating Inference with FP8 KV
// Cache", opening section), exactly as in the decode kernels: codes decoded exactly to fp16, fp16
// products with fp32 accumulation, base-2 online softmax in fp32, scales factored out of the sums.
//
// One wave per (KV head, tile of query rows, sequence) on the matrix cores
// (v_mfma_f32_16x16x32_f16).  The 16 MFMA columns are (query row, query head) pairs: R = 16 / G
// consecutive rows times the G heads of the group (16 rows of one head without grouping), so each
// K/V code read serves every column.  Per pair of 16-token tiles:
//   S^T = K Q^T   A = K rows (lane: token l%16, 32 of its dims over the four MFMAs, one 16-byte
//                 load per 1 KiB half of the chunked K tile), B = Q^T (lane: column l%16).
//   O^T += V^T P^T  A = V^T from the dim-major V rows, B = P^T as the S^T accumulator left it;
//                 P enters as fp16 hi + lo parts.
// Each column masks the tokens past its own position; the wave reads the tiles up to the position
// of its last row.  The tiles of a head stay in its XCD's L2 for the other row tiles of the head
// (the KV head is the fastest grid dimension, and workgroup ids go round-robin to the 8 XCDs).
#include "kvq_attn.h"
#include "kvq_mfma.h"

namespace kvq {

struct PrefillParams {
    const uint8_t* kc;
    const uint8_t* vc;
    const float* ks;
    const float* vs;
    const uint16_t* q;      // fp16 [num_q_rows][Hq][128]
    uint16_t* out;          // fp16 [num_q_rows][Hq][128]
    const int32_t* block_tables;
    const int32_t* ctx;     // post-append lengths
    const int32_t* cu_q;    // [B + 1] query row offsets
    int32_t max_blocks;
    int32_t Hq;
    int32_t Hkv;
    int32_t G;              // query heads per KV head
    int32_t R;              // query rows per wave (16 / G)
    int32_t row_tiles;      // grid extent over row tiles
    float qk_scale;         // sm_scale * log2(e) (* kv_scale for FP8)
    float v_scale;          // kv_scale for FP8, 1 for INT8
};

template <int DT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4, 8))) void attn_prefill_mfma(
    PrefillParams a) {
    constexpr int TW = 2;  // tiles per chunk, paired for the PV products
    const int g = blockIdx.x;
    // the row tiles of a sequence run last-first: later rows read more tiles (longest work first)
    const int rt = a.row_tiles - 1 - (int)blockIdx.y;
    const int b = blockIdx.z;
    const int lane = threadIdx.x;
    const int col = lane & 15;  // column: (row jr, head hg) of the tile
    const int q4 = lane >> 4;   // MFMA k-group / C row group

    const int r0 = a.cu_q[b];
    const int nq = a.cu_q[b + 1] - r0;
    const int j0 = rt * a.R;
    if (j0 >= nq) return;
    const int n = a.ctx[b];
    const int rows = min(a.R, nq - j0);
    const int jr = col / a.G, hg = col % a.G;
    const bool live = jr < rows;                    // the column holds a real (row, head)
    const size_t orow = ((size_t)(r0 + j0 + jr) * a.Hq + (size_t)g * a.G + hg) * kDim;
    if (n < nq) {  // more query rows than tokens: outside the contract; the rows get zeros
        if (live) {
#pragma unroll
            for (int r = 0; r < 8; ++r)
                *reinterpret_cast<half4_t*>(a.out + orow + 16 * r + 4 * q4) = half4_t{0, 0, 0, 0};
        }
        return;
    }
    const int pos = n - nq + j0 + (live ? jr : 0);  // last visible position of the column
    const int t_end = n - nq + j0 + rows;           // tokens the wave reads: up to its last row
    const int tile_end = (t_end + kBlock - 1) / kBlock;
    const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks;

    // Q^T operands: MFMA m covers dims 64 (m/2) + 16 q4 + 8 (m%2) .. +7 in k-slots 8 q4 .. +7
    half8_v qB[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) qB[m] = half8_v{0, 0, 0, 0, 0, 0, 0, 0};
    if (live) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
            qB[m] = *reinterpret_cast<const half8_v*>(a.q + orow + 64 * (m >> 1) + 16 * q4 + 8 * (m & 1));
    }

    float m_run = kNegInf;  // running max of this lane's column (base-2 logits)
    float l_lane = 0.0f;    // sum of this lane's weights (tokens 4 q4 .. +3 of every tile)
    float4_t acc[8];        // O^T row blocks: dims 16 r + 4 q4 .. +3 of column col
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const uint32_t k_off = 16u * (uint32_t)lane;  // chunk q4 (+4): token col, dims 16 q4 (+64)
    const uint32_t v_off = (uint32_t)col * kBlock + 4u * (uint32_t)q4;  // dim col (+16 r), tokens 4 q4

    for (int tb = 0; tb < tile_end; tb += 64) {
        const int nt_grp = min(64, tile_end - tb);
        const int blk_lane = (lane < nt_grp) ? bt[tb + lane] : 0;
        for (int c0 = 0; c0 < nt_grp; c0 += TW) {
            u32x4 ka[TW], kb[TW];
            uint32_t vd[TW][8];
            float4_t ks4[TW], vs4[TW];
#pragma unroll
            for (int i = 0; i < TW; ++i) {
                if (c0 + i < nt_grp) {
                    const int blk = __builtin_amdgcn_readlane(blk_lane, c0 + i);
                    const size_t tile = ((size_t)blk * a.Hkv + g) * kTileBytes;
                    const uint8_t* kt = a.kc + tile;
                    const uint8_t* vt = a.vc + tile;
                    ka[i] = ldg16(kt + k_off);
                    kb[i] = ldg16(kt + k_off + 1024u);
#pragma unroll
                    for (int r = 0; r < 8; ++r) vd[i][r] = ldg4(vt + v_off + (uint32_t)r * 256u);
                    if constexpr (DT == KVQ_INT8) {
                        const size_t so = ((size_t)blk * a.Hkv + g) * kBlock + 4 * q4;
                        ks4[i] = ldg_nt(reinterpret_cast<const float4_t*>(a.ks + so));
                        vs4[i] = ldg_nt(reinterpret_cast<const float4_t*>(a.vs + so));
                    }
                } else {
                    ka[i] = kb[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int r = 0; r < 8; ++r) vd[i][r] = 0u;
                    ks4[i] = vs4[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
            // logits S^T: lane holds tokens 4 q4 .. +3 of each tile for column col; a token past
            // the column's own position is masked
            float z[TW][4];
            float cmax = kNegInf;
#pragma unroll
            for (int i = 0; i < TW; ++i) {
                float4_t sacc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8<DT>(ka[i].x, ka[i].y), qB[0], sacc, 0, 0, 0);
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8<DT>(ka[i].z, ka[i].w), qB[1], sacc, 0, 0, 0);
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8<DT>(kb[i].x, kb[i].y), qB[2], sacc, 0, 0, 0);
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8<DT>(kb[i].z, kb[i].w), qB[3], sacc, 0, 0, 0);
                const int tok0 = (tb + c0 + i) * kBlock + 4 * q4;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    float f = a.qk_scale;
                    if constexpr (DT == KVQ_INT8) f *= ks4[i][t];
                    z[i][t] = (tok0 + t <= pos) ? sacc[t] * f : kNegInf;
                    cmax = fmaxf(cmax, z[i][t]);
                }
            }
            // max over the column's tokens: the four row groups of the column.  Every column sees
            // token 0, which the first chunk holds, so the running max is finite from then on.
            cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
            cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
            const float m_new = fmaxf(m_run, cmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_lane *= alpha;
#pragma unroll
            for (int r = 0; r < 8; ++r) acc[r] *= alpha;

#pragma unroll
            for (int i = 0; i < TW; i += 2) {
                // weights of the tile pair (i, i+1), hi and lo fp16 parts, in the B layout
                half8_v whi, wlo;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float pw = __builtin_amdgcn_exp2f(z[i + u][t] - m_new);
                        l_lane += pw;
                        float w = pw;
                        if constexpr (DT == KVQ_INT8) w = (pw > 0.0f) ? pw * vs4[i + u][t] : 0.0f;
                        const _Float16 hi = (_Float16)w;
                        whi[4 * u + t] = hi;
                        wlo[4 * u + t] = (_Float16)(w - (float)hi);
                    }
                }
                // V codes of the slots at and past t_end are zeroed (past the context they may hold
                // NaN codes; a zero weight alone would still give 0 * NaN)
                uint32_t v0[8], v1[8];
                const int valid0 = t_end - (tb + c0 + i) * kBlock - 4 * q4;
                const int valid1 = valid0 - kBlock;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    v0[r] = keep_bytes(vd[i][r], valid0);
                    v1[r] = keep_bytes(vd[i + 1][r], valid1);
                }
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const half8_v va8 = join8(codes_to_f16<DT, 0>(v0[r]), codes_to_f16<DT, 1>(v0[r]),
                                              codes_to_f16<DT, 0>(v1[r]), codes_to_f16<DT, 1>(v1[r]));
                    acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va8, whi, acc[r], 0, 0, 0);
                    acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va8, wlo, acc[r], 0, 0, 0);
                }
            }
        }
    }
    // sum of the column's weights over the four row groups
    float l_sum = l_lane + __shfl_xor(l_lane, 16);
    l_sum += __shfl_xor(l_sum, 32);

    if (live) {
        const float inv = a.v_scale / l_sum;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const half4_t o = {(_Float16)(acc[r][0] * inv), (_Float16)(acc[r][1] * inv),
                               (_Float16)(acc[r][2] * inv), (_Float16)(acc[r][3] * inv)};
            *reinterpret_cast<half4_t*>(a.out + orow + 16 * r + 4 * q4) = o;
        }
    }
}

hipError_t launch_prefill(const PrefillArgs& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    const kvq_cache& c = *p.cache;
    if (p.batch == 0 || p.max_q_len == 0 || p.num_q_rows == 0) return hipSuccess;
    PrefillParams a;
    a.kc = c.k_cache;
    a.vc = c.v_cache;
    a.ks = c.k_scale;
    a.vs = c.v_scale;
    a.q = p.q;
    a.out = p.out;
    a.block_tables = p.block_tables;
    a.ctx = p.context_lens;
    a.cu_q = p.cu_q_lens;
    a.max_blocks = p.max_blocks_per_seq;
    a.Hq = p.num_q_heads;
    a.Hkv = c.num_kv_heads;
    a.G = p.num_q_heads / c.num_kv_heads;
    a.R = 16 / a.G;
    a.row_tiles = (p.max_q_len + a.R - 1) / a.R;
    const bool fp8 = c.dtype != KVQ_INT8;
    a.qk_scale = p.sm_scale * kLog2e * (fp8 ? c.kv_scale : 1.0f);
    a.v_scale = fp8 ? c.kv_scale : 1.0f;
    const dim3 grid((unsigned)a.Hkv, (unsigned)a.row_tiles, (unsigned)p.batch);
    auto go = [&](auto kernel) {
        if (start)
            hipExtLaunchKernelGGL(kernel, grid, dim3(64), 0, stream, start, stop, 0, a);
        else
            hipLaunchKernelGGL(kernel, grid, dim3(64), 0, stream, a);
    };
    switch (c.dtype) {
        case KVQ_FP8_E4M3: go(attn_prefill_mfma<KVQ_FP8_E4M3>); break;
        case KVQ_FP8_E5M2: go(attn_prefill_mfma<KVQ_FP8_E5M2>); break;
        default: go(attn_prefill_mfma<KVQ_INT8>); break;
    }
    return hipGetLastError();
}

}  // namespace kvq
