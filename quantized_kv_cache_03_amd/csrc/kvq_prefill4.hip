// kvq_prefill4.hip -- prefill / chunked-prefill attention over the INT4 cache.
//
// The same causal attention as kvq_prefill.hip (sequence b's n_b query rows are its last n_b
// tokens; row j at position p = context_lens[b] - n_b + j sees the tokens 0 .. p) over the INT4
// cache (asymmetric 4-bit codes, an fp32 (scale, zero point) pair per (token, KV head)), with the
// logits and the output factored as in the grouped INT4 decode kernel (kvq_attn_gqa4.hip):
//     z_t = sm_scale * (s_t (q . (c_t - c0_t)) + zp'_t sum_d q_d),   zp'_t = zp_t + s_t c0_t,
//     out = (sum_t p_t s_t c_t + sum_t p_t zp_t) / sum_t p_t,
// c0_t the code of the token's row nearest zero (int4_zero_code).
// One wave per (KV head, tile of query rows, sequence) on v_mfma_f32_16x16x32_f16, serving two
// blocks of 16 columns -- (query row, query head) pairs as in the 8-bit prefill kernel -- with the
// operands of the grouped INT4 decode kernel: one 16-byte load per lane for each of the K and V
// tiles, decoded once for both blocks, P^T left in the lanes by the S^T accumulator, chunks of four
// tiles.  The matrix cores get exact binary16 integers: K codes as c - c0 and 16 (c - c0)
// (int4x8_centred), V codes as c through the FP8 converter (int4x8_exact).
#include "kvq_attn4.h"
#include "kvq_mfma.h"

namespace kvq {

namespace {

constexpr int kTilesP4 = 4;  // tiles per chunk: the P^T operand spans four tiles

struct Prefill4Params {
    const uint8_t* kc;
    const uint8_t* vc;
    const float* ks;          // (scale, zero point) pairs [num_blocks][Hkv][16][2]
    const float* vs;
    const uint16_t* q;        // fp16 [num_q_rows][Hq][128]
    uint16_t* out;            // fp16 [num_q_rows][Hq][128]
    const int32_t* block_tables;
    const int32_t* ctx;       // post-append lengths
    const int32_t* cu_q;      // [B + 1] query row offsets
    int32_t max_blocks;
    int32_t Hq;
    int32_t Hkv;
    int32_t G;                // query heads per KV head
    int32_t R;                // query rows per column block (16 / G)
    int32_t row_tiles;        // grid extent over row tiles
    float qk_scale;           // sm_scale * log2(e)
};


// The K operands of one tile in the k-slot order of kslot_dim: the four MFMAs take the (0, 4),
// (2, 6) nibble pairs and then the (1, 5), (3, 7) pairs of dwords (0, 1) and of dwords (2, 3); every
// code minus its token's zero code (ne, no): c - c0 in operands 0 and 2, 16 (c - c0) in operands 1 and 3.
__device__ __forceinline__ void k_operands_p4(const u32x4& k, half2_t ne, half2_t no, const Int4Bits& b,
                                              half8_v (&op)[4]) {
    const uint32_t w[4] = {k.x, k.y, k.z, k.w};
    half2_t h[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) int4x8_centred(w[j], ne, no, b, h[j]);
    op[0] = join8(h[0][0], h[0][2], h[1][0], h[1][2]);
    op[1] = join8(h[0][1], h[0][3], h[1][1], h[1][3]);
    op[2] = join8(h[2][0], h[2][2], h[3][0], h[3][2]);
    op[3] = join8(h[2][1], h[2][3], h[3][1], h[3][3]);
}

// Chunk-relative dim of k-slot `slot` of K operand m (see k_operands_p4).
__device__ __forceinline__ int kslot_dim(int m, int slot) {
    const int dw = 2 * (m / 2) + slot / 4;
    const int i = 2 * ((slot % 4) / 2) + (m % 2);  // nibble pair (i, i + 4)
    return 8 * dw + i + 4 * (slot % 2);
}

// NB column blocks of 16 per wave (NB R consecutive rows): the K and V operands of a tile are
// decoded once and feed the MFMAs of every block.
template <int NB>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void attn_prefill_mfma4(
    Prefill4Params a) {
    const int g = blockIdx.x;
    const int rt = a.row_tiles - 1 - (int)blockIdx.y;  // later rows read more tiles: run them first
    const int b = blockIdx.z;
    const int lane = threadIdx.x;
    const int col = lane & 15;  // column of each block: (row jr, head hg)
    const int q4 = lane >> 4;   // MFMA k-group / C row group
    const int own = int4_own_token(lane);         // the token of the lane's K and V pairs
    const int src = 16 * (col >> 2) + (col & 3);  // a lane whose pairs are those of token col

    const int r0 = a.cu_q[b];
    const int nq = a.cu_q[b + 1] - r0;
    const int j0 = rt * (NB * a.R);
    if (j0 >= nq) return;
    const int n = a.ctx[b];
    const int jr = col / a.G, hg = col % a.G;
    bool live[NB];  // the column of block nb holds a real (row, head)
    size_t orow[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int j = j0 + nb * a.R + jr;
        live[nb] = jr < a.R && j < nq;
        orow[nb] = ((size_t)(r0 + j) * a.Hq + (size_t)g * a.G + hg) * kDim;
    }
    if (n < nq) {  // more query rows than tokens: outside the contract; the rows get zeros
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            if (live[nb]) {
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    *reinterpret_cast<half4_t*>(a.out + orow[nb] + 16 * r + 4 * q4) = half4_t{0, 0, 0, 0};
            }
        return;
    }
    const int pos_min = n - nq + j0;                       // every column sees tokens 0 .. pos_min
    const int t_end = n - nq + min(nq, j0 + NB * a.R);     // tokens the wave reads
    const int tile_end = (t_end + kBlock - 1) / kBlock;
    int pos[NB];  // last visible token of each block's column (padding columns: pos_min)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) pos[nb] = live[nb] ? n - nq + j0 + nb * a.R + jr : pos_min;
    const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks;

    // Q^T operands of each block's column over chunk q4's dims, and the sum of its 128 q elements.
    // The logit scale f = sm_scale log2(e) is applied in the exponent as |f| (exp2(fma(z, |f|, -m))
    // with the chunk max taken on the unscaled z and scaled once); a negative f negates q instead.
    const bool neg = a.qk_scale < 0.0f;
    const _Float16 qsign = neg ? (_Float16)-1.0f : (_Float16)1.0f;
    const float qf = fmaxf(fabsf(a.qk_scale), 1.17549435e-38f);  // -inf * qf must stay -inf
    half8_v qB[NB][4];
    float qsum[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        qsum[nb] = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; ++m) qB[nb][m] = half8_v{0, 0, 0, 0, 0, 0, 0, 0};
        if (live[nb]) {
            const uint16_t* qrow = a.q + orow[nb] + 32 * q4;
            uint16_t qv[32];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4 w = reinterpret_cast<const u32x4*>(qrow)[c];
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    qv[8 * c + 2 * k] = (uint16_t)(ww[k] & 0xFFFFu);
                    qv[8 * c + 2 * k + 1] = (uint16_t)(ww[k] >> 16);
                }
            }
#pragma unroll
            for (int d = 0; d < 32; ++d) qsum[nb] += (float)__builtin_bit_cast(_Float16, qv[d]);
            // the odd operands (1, 3) take q 16 times smaller, so that all four K products share
            // one accumulator: exact for |q| >= 2^-10, and below that off by at most 2^-25
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int s = 0; s < 8; ++s)
                    qB[nb][m][s] = __builtin_bit_cast(_Float16, qv[kslot_dim(m, s)]) *
                                   (qsign * (_Float16)((m & 1) ? 0.0625f : 1.0f));
        }
        qsum[nb] = col_sum4(qsum[nb]);  // the logit term of the zero points: qsum * zp'
        if (neg) qsum[nb] = -qsum[nb];
    }

    float m_run[NB], l_lane[NB], z_lane[NB];
    float4_t acc[NB][8];  // O^T row blocks, sum of w c: dims 16 r + 4 q4 .. +3 of the column
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        m_run[nb] = kNegInf;
        l_lane[nb] = z_lane[nb] = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[nb][r] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const uint32_t off = 256u * (uint32_t)q4 + 16u * (uint32_t)col;

    for (int tb = 0; tb < tile_end; tb += 64) {
        const int nt_grp = min(64, tile_end - tb);
        // Lanes past the group's tiles repeat its last block, so a chunk's loads are issued together
        // with no branch between them; the extra tiles' tokens lie past every column's causal limit.
        const int blk_lane = bt[tb + min(lane, nt_grp - 1)];
        for (int c0 = 0; c0 < nt_grp; c0 += kTilesP4) {
            TileQ4 t[kTilesP4];  // this lane's share of each tile (kvq_int4.h)
#pragma unroll
            for (int i = 0; i < kTilesP4; ++i)
                load_tile_q4<false>(a.kc, a.vc, a.ks, a.vs, a.Hkv, t[i], __builtin_amdgcn_readlane(blk_lane, c0 + i), g,
                                    off, own);
            const int tok_base = (tb + c0) * kBlock;
            const Int4Bits bits = int4_bits();
            float z[NB][kTilesP4][4];
            // The K operands and S^T products run at raised wave priority, like P V^T below
            // (s_setprio 1; back to 0 for the softmax).
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int i = 0; i < kTilesP4; ++i) {
                // every token centred at its own zero code (int4_zero_code), computed once per token
                // by the lanes holding its pairs; the K operand rows (token col) take it by shuffle,
                // the accumulator's tokens 4 q4 + u take their K scale and zp' = zp + s c0 by quad
                // broadcast.  The V pairs of slots past the context are zeroed first (they may be
                // NaN, and a zero weight alone would still give 0 * NaN); only the chunk reaching
                // past the context has such slots (wave-uniform test).
                const float zo = int4_zero_code(t[i].kp.x, t[i].kp.y);
                const float zpa = __builtin_fmaf(t[i].kp.x, zo, t[i].kp.y);
                if (tok_base + kTilesP4 * kBlock > n && tok_base + i * kBlock + own >= n) t[i].vp = f32x2{0.0f, 0.0f};
                half2_t ne, no;
                int4_centre_pairs(__shfl(zo, src), ne, no);
                half8_v kop[4];
                k_operands_p4(t[i].k, ne, no, bits, kop);
                float ks[4], zp[4];
                __builtin_amdgcn_sched_barrier(0);
                ks[0] = quad_bcast<0>(t[i].kp.x), zp[0] = quad_bcast<0>(zpa);
                ks[1] = quad_bcast<1>(t[i].kp.x), zp[1] = quad_bcast<1>(zpa);
                ks[2] = quad_bcast<2>(t[i].kp.x), zp[2] = quad_bcast<2>(zpa);
                ks[3] = quad_bcast<3>(t[i].kp.x), zp[3] = quad_bcast<3>(zpa);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    float4_t s = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[0], qB[nb][0],
                                                                        float4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                    s = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[1], qB[nb][1], s, 0, 0, 0);
                    s = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[2], qB[nb][2], s, 0, 0, 0);
                    s = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[3], qB[nb][3], s, 0, 0, 0);
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        z[nb][i][u] = __builtin_fmaf(s[u], ks[u], qsum[nb] * zp[u]);  // z / |f|
                }
            }
            __builtin_amdgcn_s_setprio(0);
            // The causal mask, only for the chunks that reach past the wave's first row
            // (wave-uniform test); and the V parameters of slots past the context are zeroed (they
            // may be NaN, and a zero weight alone would still give 0 * NaN), only in the chunk
            // that reaches past it.
            if (tok_base + kTilesP4 * kBlock - 1 > pos_min) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int lim = pos[nb] - (tok_base + 4 * q4);  // last visible offset in the chunk
#pragma unroll
                    for (int i = 0; i < kTilesP4; ++i)
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (i * kBlock + u > lim) z[nb][i][u] = kNegInf;
                }
            }
            // finite: the first chunk holds token 0.  Lazy rescale (kRescaleSlackInt4), a branch
            // every lane takes or skips together.  The column max (over the column's four lanes)
            // is taken only when some lane's own max passes the reference max plus the slack: the
            // column max passes it exactly when one of its lanes' maxima does (scaling by |f| > 0
            // is monotone).
            bool moved = false;
            float lmax[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float m = kNegInf;
#pragma unroll
                for (int i = 0; i < kTilesP4; ++i)
#pragma unroll
                    for (int u = 0; u < 4; ++u) m = fmaxf(m, z[nb][i][u]);
                lmax[nb] = m;
                moved |= m * qf > m_run[nb] + kRescaleSlackInt4;  // m_run = -inf: any finite max
            }
            if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const float cmax = col_max4(lmax[nb]) * qf;  // the max of z |f|
                    const bool up = cmax > m_run[nb] + kRescaleSlackInt4;
                    const float alpha = up ? __builtin_amdgcn_exp2f(m_run[nb] - cmax) : 1.0f;
                    if (up) m_run[nb] = cmax;
                    l_lane[nb] *= alpha;
                    z_lane[nb] *= alpha;
#pragma unroll
                    for (int r = 0; r < 8; ++r) acc[nb][r] *= alpha;
                }
            }
            // P^T operands per block: tokens (0, 2) and (1, 3) of this lane's quad of each tile,
            // w = p s_v (dword i of an operand: tile i's pair)
            half8_v we_hi[NB], we_lo[NB], wo_hi[NB], wo_lo[NB];
            uint32_t ehi[NB][kTilesP4], elo[NB][kTilesP4], ohi[NB][kTilesP4], olo[NB][kTilesP4];
#pragma unroll
            for (int i = 0; i < kTilesP4; ++i) {
                // the V pairs of the tokens 4 q4 + u, shared by both blocks
                __builtin_amdgcn_sched_barrier(0);
                const float vs[4] = {quad_bcast<0>(t[i].vp.x), quad_bcast<1>(t[i].vp.x), quad_bcast<2>(t[i].vp.x),
                                     quad_bcast<3>(t[i].vp.x)};
                const float vz[4] = {quad_bcast<0>(t[i].vp.y), quad_bcast<1>(t[i].vp.y), quad_bcast<2>(t[i].vp.y),
                                     quad_bcast<3>(t[i].vp.y)};
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    float w[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float pw = __builtin_amdgcn_exp2f(__builtin_fmaf(z[nb][i][u], qf, -m_run[nb]));
                        l_lane[nb] += pw;
                        w[u] = pw * vs[u];
                        z_lane[nb] = __builtin_fmaf(pw, vz[u], z_lane[nb]);
                    }
                    split_hi_lo(w[0], w[2], ehi[nb][i], elo[nb][i]);
                    split_hi_lo(w[1], w[3], ohi[nb][i], olo[nb][i]);
                }
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                we_hi[nb] = __builtin_bit_cast(half8_v, u32x4{ehi[nb][0], ehi[nb][1], ehi[nb][2], ehi[nb][3]});
                we_lo[nb] = __builtin_bit_cast(half8_v, u32x4{elo[nb][0], elo[nb][1], elo[nb][2], elo[nb][3]});
                wo_hi[nb] = __builtin_bit_cast(half8_v, u32x4{ohi[nb][0], ohi[nb][1], ohi[nb][2], ohi[nb][3]});
                wo_lo[nb] = __builtin_bit_cast(half8_v, u32x4{olo[nb][0], olo[nb][1], olo[nb][2], olo[nb][3]});
            }
            // O^T += V^T P^T, row blocks r = 2 d, 2 d + 1 from dword d of every tile's V, at raised
            // wave priority (s_setprio 1): when waves of a SIMD compete, the one feeding the matrix
            // cores issues first
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                half2_t hv[kTilesP4][4];
#pragma unroll
                for (int i = 0; i < kTilesP4; ++i) {
                    const uint32_t w[4] = {t[i].v.x, t[i].v.y, t[i].v.z, t[i].v.w};
                    int4x8_exact(w[d], hv[i]);  // unit 0: tokens (0, 2) in hv[0], (1, 3) in hv[2]; unit 1: hv[1], hv[3]
                }
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = 2 * d + e;
                    const half8_v ae = join8(hv[0][e], hv[1][e], hv[2][e], hv[3][e]);
                    const half8_v ao = join8(hv[0][2 + e], hv[1][2 + e], hv[2][2 + e], hv[3][2 + e]);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        acc[nb][r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ae, we_hi[nb], acc[nb][r], 0, 0, 0);
                        acc[nb][r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ae, we_lo[nb], acc[nb][r], 0, 0, 0);
                        acc[nb][r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ao, wo_hi[nb], acc[nb][r], 0, 0, 0);
                        acc[nb][r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ao, wo_lo[nb], acc[nb][r], 0, 0, 0);
                    }
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const float l_sum = col_sum4(l_lane[nb]);
        const float z_sum = col_sum4(z_lane[nb]);
        if (live[nb]) {
            const float inv = 1.0f / l_sum;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float4_t o = acc[nb][r] + z_sum;
                const half4_t v = {(_Float16)(o[0] * inv), (_Float16)(o[1] * inv), (_Float16)(o[2] * inv),
                                   (_Float16)(o[3] * inv)};
                *reinterpret_cast<half4_t*>(a.out + orow[nb] + 16 * r + 4 * q4) = v;
            }
        }
    }
}

#ifndef KVQ_PREFILL4_BLOCKS
#define KVQ_PREFILL4_BLOCKS 2
#endif

}  // namespace

hipError_t launch_prefill4(const PrefillArgs& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    const kvq_cache& c = *p.cache;
    if (p.batch == 0 || p.max_q_len == 0 || p.num_q_rows == 0) return hipSuccess;
    Prefill4Params a;
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
    const int rows_per_wave = KVQ_PREFILL4_BLOCKS * a.R;
    a.row_tiles = (p.max_q_len + rows_per_wave - 1) / rows_per_wave;
    a.qk_scale = p.sm_scale * kLog2e;
    const dim3 grid((unsigned)a.Hkv, (unsigned)a.row_tiles, (unsigned)p.batch);
    if (start)
        hipExtLaunchKernelGGL(attn_prefill_mfma4<KVQ_PREFILL4_BLOCKS>, grid, dim3(64), 0, stream, start,
                              stop, 0, a);
    else
        hipLaunchKernelGGL(attn_prefill_mfma4<KVQ_PREFILL4_BLOCKS>, grid, dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvq
