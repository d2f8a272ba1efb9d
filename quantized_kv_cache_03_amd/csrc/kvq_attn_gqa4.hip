// kvq_attn_gqa4.hip -- decode attention over the INT4 cache for grouped query heads (MFMA).
//
// The INT4 cache (asymmetric 4-bit codes, an fp32 (scale, zero point) pair per (token, KV head);
// the online INT4 cache named beside INT8 in "[Feature] TurboMind support W8A8 or FP8 KV Cache"):
//     z_t   = sm_scale * (s_t (q . (c_t - c0_t)) + zp'_t sum_d q_d),   zp'_t = zp_t + s_t c0_t,
//     out_d = (sum_t p_t s_t c_td + sum_t p_t zp_t) / sum_t p_t,
// c0_t the code of the token's row nearest zero (int4_zero_code): centred, the logit sums terms
// no larger than q . k^ itself.
// One wave per (KV head, share of the work) serves the G <= 16 query heads of the group, as the
// 8-bit grouped kernel (kvq_attn_gqa.hip) does, with both products on v_mfma_f32_16x16x32_f16
// (query heads padded to 16 columns).  The matrix cores get exact binary16 integers (they align a
// group's products by exponent fields, which would cost subnormal codes their low bits): K codes as
// c - c0 and 16 (c - c0) (int4x8_centred), V codes as c through the FP8 converter (int4x8_exact).
//   S^T = K Q^T per tile: A = K (lane: token l % 16, the 32 dims of chunk l / 16 -- one 16-byte
//       load per lane reads the tile), B = Q^T (lane: head l % 16, the same dims); two MFMAs for
//       the even nibble pairs of the chunk's dims, two for the odd ones.  C: lane (head l % 16,
//       tokens 4 (l / 16) .. +3).
//   O^T += V^T P^T per chunk of four tiles and 16-dim row block: A = V^T (lane: dim l % 16 + 16 r,
//       tokens 0 and 2 -- or 1 and 3 -- of quad l / 16 of each of the four tiles, straight from the
//       lane's 16-byte V load), B = P^T with the weights the S^T accumulator left in the lane
//       (tokens 4 (l / 16) .. +3 of each tile), split into fp16 hi + lo parts.
#include "kvq_attn4.h"
#include "kvq_mfma.h"

namespace kvq {

namespace {

constexpr int kTiles4 = 4;  // tiles per chunk: the P^T operand spans four tiles

__device__ __forceinline__ half8_v join4(half2_t a, half2_t b, half2_t c, half2_t d) {
    return join8(a, b, c, d);
}

// The K operands of one tile: (even, odd) nibble pairs of dwords (0, 1) and (2, 3), every code
// minus its token's zero code (ne, no): c - c0 in the even operands, 16 (c - c0) in the odd ones.
__device__ __forceinline__ void k_operands(const u32x4& k, half2_t ne, half2_t no, const Int4Bits& b,
                                           half8_v (&e)[2], half8_v (&o)[2]) {
    const uint32_t w[4] = {k.x, k.y, k.z, k.w};
    half2_t h0[4], h1[4], h2[4], h3[4];
    int4x8_centred(w[0], ne, no, b, h0);
    int4x8_centred(w[1], ne, no, b, h1);
    int4x8_centred(w[2], ne, no, b, h2);
    int4x8_centred(w[3], ne, no, b, h3);
    e[0] = join4(h0[0], h0[2], h1[0], h1[2]);
    o[0] = join4(h0[1], h0[3], h1[1], h1[3]);
    e[1] = join4(h2[0], h2[2], h3[0], h3[2]);
    o[1] = join4(h2[1], h2[3], h3[1], h3[3]);
}

// The dims of the K operands' k-slots, relative to the chunk's first dim: nibble pairs (i, i + 4)
// of two dwords, the even pairs (i = 0, 2) or the odd ones (i = 1, 3).
__device__ __forceinline__ int k_slot_dim(int dw0, int odd, int slot) {
    const int dw = dw0 + slot / 4;               // dword of the slot
    const int pair = (slot % 4) / 2;             // first or second pair of the dword's kind
    const int i = 2 * pair + odd;                // nibble pair (i, i + 4)
    return 8 * dw + i + 4 * (slot % 2);
}

// One chunk of kTiles4 tiles (tiles past the segment's end repeat its last one; their tokens are masked).
template <bool APPEND>
__device__ __forceinline__ void chunk_g4(const KernelParams& a, TileQ4 (&t)[kTiles4], int tile0, int t_end,
                                         const half8_v (&qe)[2], const half8_v (&qo)[2], float qsum, float qf,
                                         int q4, float& m_run, float& l_lane, float& z_lane,
                                         float4_t (&acc)[8]) {
    float z[kTiles4][4];
    const Int4Bits bits = int4_bits();
    const int col = (int)(threadIdx.x & 15u);  // the token of the lane's K operand row
    const int own = 4 * q4 + (col & 3);        // the token of the lane's pairs
    const int src = 16 * (col >> 2) + (col & 3);  // a lane whose pairs are those of token col
    // The K operands and S^T products run at raised wave priority, like P V^T below (s_setprio 1;
    // back to 0 for the softmax): when waves of a SIMD compete, the one feeding the matrix cores
    // issues first.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < kTiles4; ++i) {
        // every token centred at its own zero code c0 (int4_zero_code), computed once per token by
        // the lanes holding its pairs; the K operand rows (token col) take it by shuffle, and the
        // accumulator's tokens 4 q4 + u take their K scale and zp' = zp + s c0 by quad broadcast
        // (fenced: quad_bcast).
        // The V pairs of slots at and past t_end are zeroed first (past the context they may be
        // NaN, and a zero weight alone would still give 0 * NaN); only a tile that reaches past
        // the end has such slots (wave-uniform test).
        const float zo = int4_zero_code(t[i].kp.x, t[i].kp.y);
        const float zpa = __builtin_fmaf(t[i].kp.x, zo, t[i].kp.y);
        if ((tile0 + i + 1) * kBlock > t_end && (tile0 + i) * kBlock + own >= t_end) t[i].vp = f32x2{0.0f, 0.0f};
        const float zc = __shfl(zo, src);
        float ks[4], zps[4];  // K scale and zp' of the tokens 4 q4 + u
        __builtin_amdgcn_sched_barrier(0);
        ks[0] = quad_bcast<0>(t[i].kp.x), zps[0] = quad_bcast<0>(zpa);
        ks[1] = quad_bcast<1>(t[i].kp.x), zps[1] = quad_bcast<1>(zpa);
        ks[2] = quad_bcast<2>(t[i].kp.x), zps[2] = quad_bcast<2>(zpa);
        ks[3] = quad_bcast<3>(t[i].kp.x), zps[3] = quad_bcast<3>(zpa);
        __builtin_amdgcn_sched_barrier(0);
        half2_t ne, no;
        int4_centre_pairs(zc, ne, no);
        half8_v e[2], o[2];
        k_operands(t[i].k, ne, no, bits, e, o);
        // q . (c - c0): the odd operands hold 16 (c - c0) and meet q / 16 (qo), so all four
        // products share one accumulator
        float4_t s = __builtin_amdgcn_mfma_f32_16x16x32_f16(e[0], qe[0], float4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(o[0], qo[0], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(e[1], qe[1], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(o[1], qo[1], s, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) z[i][u] = __builtin_fmaf(s[u], ks[u], qsum * zps[u]);  // z / qf
    }
    __builtin_amdgcn_s_setprio(0);
    // Tokens at and past t_end are masked; only a chunk that reaches past it has such tokens
    // (wave-uniform test).
    if ((tile0 + kTiles4) * kBlock > t_end) {
#pragma unroll
        for (int i = 0; i < kTiles4; ++i) {
            const int pos0 = (tile0 + i) * kBlock + 4 * q4;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (pos0 + u >= t_end) z[i][u] = kNegInf;
        }
    }
    float cmax = kNegInf;
#pragma unroll
    for (int i = 0; i < kTiles4; ++i)
        cmax = fmaxf(cmax, fmaxf(fmaxf(z[i][0], z[i][1]), fmaxf(z[i][2], z[i][3])));
    // Lazy rescale (kRescaleSlackInt4), a branch every lane takes or skips together.  Every chunk
    // holds a valid token, so cmax is finite.
    cmax = col_max4(cmax) * qf;
    const bool up = cmax > m_run + kRescaleSlackInt4;  // m_run = -inf: any finite max
    if (__builtin_amdgcn_ballot_w64(up)) {
        const float alpha = up ? __builtin_amdgcn_exp2f(m_run - cmax) : 1.0f;
        if (up) m_run = cmax;
        l_lane *= alpha;
        z_lane *= alpha;
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r] *= alpha;
    }
    // P^T operands: the even tokens (0, 2) and the odd tokens (1, 3) of this lane's quad of each
    // tile, as fp16 hi and lo parts of w = p s_v (dword i of an operand: tile i's pair)
    uint32_t ehi[kTiles4], elo[kTiles4], ohi[kTiles4], olo[kTiles4];
#pragma unroll
    for (int i = 0; i < kTiles4; ++i) {
        float w[4];
        __builtin_amdgcn_sched_barrier(0);
        const float vs[4] = {quad_bcast<0>(t[i].vp.x), quad_bcast<1>(t[i].vp.x), quad_bcast<2>(t[i].vp.x),
                             quad_bcast<3>(t[i].vp.x)};  // the V pairs of the tokens 4 q4 + u
        const float vz[4] = {quad_bcast<0>(t[i].vp.y), quad_bcast<1>(t[i].vp.y), quad_bcast<2>(t[i].vp.y),
                             quad_bcast<3>(t[i].vp.y)};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float pw = __builtin_amdgcn_exp2f(__builtin_fmaf(z[i][u], qf, -m_run));
            l_lane += pw;
            w[u] = pw * vs[u];
            z_lane = __builtin_fmaf(pw, vz[u], z_lane);
        }
        split_hi_lo(w[0], w[2], ehi[i], elo[i]);
        split_hi_lo(w[1], w[3], ohi[i], olo[i]);
    }
    const half8_v we_hi = __builtin_bit_cast(half8_v, u32x4{ehi[0], ehi[1], ehi[2], ehi[3]});
    const half8_v we_lo = __builtin_bit_cast(half8_v, u32x4{elo[0], elo[1], elo[2], elo[3]});
    const half8_v wo_hi = __builtin_bit_cast(half8_v, u32x4{ohi[0], ohi[1], ohi[2], ohi[3]});
    const half8_v wo_lo = __builtin_bit_cast(half8_v, u32x4{olo[0], olo[1], olo[2], olo[3]});
    // O^T += V^T P^T, row blocks r = 2 d, 2 d + 1 (dims 16 r .. +15) from dword d of every tile's V,
    // at raised wave priority (s_setprio 1): when waves of a SIMD compete, the one feeding the
    // matrix cores issues first
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        half2_t hv[kTiles4][4];
#pragma unroll
        for (int i = 0; i < kTiles4; ++i) {
            const uint32_t w[4] = {t[i].v.x, t[i].v.y, t[i].v.z, t[i].v.w};
            int4x8_exact(w[d], hv[i]);  // unit 0: tokens (0, 2) in hv[0], (1, 3) in hv[2]; unit 1: hv[1], hv[3]
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int r = 2 * d + e;
            const half8_v ae = join4(hv[0][e], hv[1][e], hv[2][e], hv[3][e]);
            const half8_v ao = join4(hv[0][2 + e], hv[1][2 + e], hv[2][2 + e], hv[3][2 + e]);
            acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ae, we_hi, acc[r], 0, 0, 0);
            acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ae, we_lo, acc[r], 0, 0, 0);
            acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ao, wo_hi, acc[r], 0, 0, 0);
            acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ao, wo_lo, acc[r], 0, 0, 0);
        }
    }
    __builtin_amdgcn_s_setprio(0);
}

// Replace the new token's codes and pairs in the registers of its tile: K in the four lanes whose
// operand row is the token, both pairs in the four lanes that own them, V in the 16 lanes of its quad.
__device__ __forceinline__ void patch_tile_g4(TileQ4& t, const NewToken4& nt, const uint8_t* lds_k,
                                              const uint8_t* lds_v, int lane) {
    const int col = lane & 15, q4 = lane >> 4;
    if (col == nt.slot) t.k = reinterpret_cast<const u32x4*>(lds_k)[q4];
    if (4 * q4 + (col & 3) == nt.slot) {
        t.kp = nt.ks;
        t.vp = nt.vs;
    }
    patch_v_quad(t.v, nt.slot, lds_v, lane);
}

// The work of one segment -- tiles [lo, hi) of sequence b (n tokens, nt tiles): the final output
// when the segment is the whole sequence, else a partial in row h * rmul + radd.
template <bool APPEND>
__device__ __forceinline__ void gqa4_segment(const KernelParams& a, int b, int g, int n, int nt, int lo,
                                             int hi, int64_t rmul, int64_t radd, int lane,
                                             uint8_t* lds_knew, uint8_t* lds_vnew, u32x4* lds_vrow,
                                             PendingAppend4& pend) {
    const int col = lane & 15;  // query head within the group (B / C column), or A row
    const int q4 = lane >> 4;   // k-group / C row group
    const int G = a.Hq / a.Hkv;
    const int h = g * G + col;  // this lane's query head (valid when col < G)
    const int t_end = min(n, hi * kBlock);
    const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks;
    const int tile_new = (APPEND && hi == nt) ? nt - 1 : -1;
    // The appended token (the segment holding the sequence's last tile): an earlier sequence's
    // pending token is stored first (its segment is done; the LDS buffers are reused), then the new
    // one is encoded into LDS, before the loop, so that none of its registers are live there.
    [[maybe_unused]] NewToken4 ntok{};
    if constexpr (APPEND) {
        if (tile_new >= 0) {  // (wave-uniform)
            flush_append4(a, pend, lds_knew, lds_vrow, g, lane);
            ntok = new_token4(a, b, g, n, lane, lds_knew, lds_vnew);
        }
    }

    // Q^T operands over chunk q4's dims in the K operands' slot order, and sum(q) of the head
    half8_v qe[2], qo[2];
    float qsum = 0.0f;
#pragma unroll
    for (int m = 0; m < 2; ++m) qe[m] = qo[m] = half8_v{0, 0, 0, 0, 0, 0, 0, 0};
    // The logit scale f = sm_scale log2(e) is applied in the exponent as |f| (exp2(fma(z, |f|, -m))
    // with the chunk max taken on the unscaled z and scaled once); a negative f negates q instead.
    const bool neg = a.qk_scale < 0.0f;
    const _Float16 qsign = neg ? (_Float16)-1.0f : (_Float16)1.0f;
    const float qf = fmaxf(fabsf(a.qk_scale), 1.17549435e-38f);  // -inf * qf must stay -inf
    if (col < G) {
        const uint16_t* qrow = a.q + ((size_t)b * a.Hq + h) * kDim + 32 * q4;
        uint16_t qv[32];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 w = reinterpret_cast<const u32x4*>(qrow)[j];
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                qv[8 * j + 2 * k] = (uint16_t)(ww[k] & 0xFFFFu);
                qv[8 * j + 2 * k + 1] = (uint16_t)(ww[k] >> 16);
            }
        }
#pragma unroll
        for (int d = 0; d < 32; ++d) qsum += (float)__builtin_bit_cast(_Float16, qv[d]);
        // the odd operands take q 16 times smaller: exact for |q| >= 2^-10, and below that off
        // by at most 2^-25 (negligible beside the sums' own rounding)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                qe[m][s] = __builtin_bit_cast(_Float16, qv[k_slot_dim(2 * m, 0, s)]) * qsign;
                qo[m][s] = __builtin_bit_cast(_Float16, qv[k_slot_dim(2 * m, 1, s)]) * (qsign * (_Float16)0.0625f);
            }
    }
    qsum += __shfl_xor(qsum, 16);
    qsum += __shfl_xor(qsum, 32);
    if (neg) qsum = -qsum;  // the logit term of the zero points is qsum * (zp + s c0)

    float m_run = kNegInf;
    float l_lane = 0.0f, z_lane = 0.0f;
    float4_t acc[8];  // O^T row blocks, sum of w c: dims 16 r + 4 q4 .. +3 of head col
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const uint32_t off = 256u * (uint32_t)q4 + 16u * (uint32_t)col;

    for (int tb = lo; tb < hi; tb += 64) {
        const int nt_grp = min(64, hi - tb);
        // Lanes past the group's tiles repeat its last block, so a chunk's loads are issued together
        // with no branch between them; the extra tiles' tokens lie past the segment and are masked.
        const int blk_lane = bt[tb + min(lane, nt_grp - 1)];
        for (int c0 = 0; c0 < nt_grp; c0 += kTiles4) {
            TileQ4 t[kTiles4];
#pragma unroll
            for (int i = 0; i < kTiles4; ++i)
                load_tile_q4<true>(a.kc, a.vc, a.ks, a.vs, a.Hkv, t[i], __builtin_amdgcn_readlane(blk_lane, c0 + i), g,
                                   off, int4_own_token(lane));
            if constexpr (APPEND) {
                const int inew = tile_new - (tb + c0);  // wave-uniform
                if (inew >= 0 && inew < kTiles4) {
#pragma unroll
                    for (int i = 0; i < kTiles4; ++i)
                        if (i == inew) {
                            patch_tile_g4(t[i], ntok, lds_knew, lds_vnew, lane);
                            lds_vrow[lane] = t[i].v;
                            pend = PendingAppend4{__builtin_amdgcn_readlane(blk_lane, c0 + i), ntok.slot, ntok.ks,
                                                  ntok.vs};
                        }
                }
            }
            chunk_g4<APPEND>(a, t, tb + c0, t_end, qe, qo, qsum, qf, q4, m_run, l_lane, z_lane, acc);
        }
    }
    // the head's weight sum and zero-point sum over the four row groups
    const float l_sum = col_sum4(l_lane);
    const float z_sum = col_sum4(z_lane);

    if (col < G) {
        float4_t o[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) o[r] = acc[r] + z_sum;
        if (lo == 0 && hi == nt) {
            const float inv = a.v_scale / l_sum;
            uint16_t* orow = a.out + ((size_t)b * a.Hq + h) * kDim;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const half4_t v = {(_Float16)(o[r][0] * inv), (_Float16)(o[r][1] * inv),
                                   (_Float16)(o[r][2] * inv), (_Float16)(o[r][3] * inv)};
                *reinterpret_cast<half4_t*>(orow + 16 * r + 4 * q4) = v;
            }
        } else {
            const int64_t prow = h * rmul + radd;
#pragma unroll
            for (int r = 0; r < 8; ++r)
                *reinterpret_cast<float4_t*>(a.part_o + prow * kDim + 16 * r + 4 * q4) = o[r];
            if (q4 == 0) {
                a.part_m[prow] = m_run;
                a.part_l[prow] = l_sum;
            }
        }
    }
}

// BAL: grid (KV head, wave of the balanced split), else (KV head, partition, sequence).
template <bool APPEND, bool BAL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) void attn_partition_mfma4(
    KernelParams a) {
    __shared__ u32x4 lds_knew[APPEND ? 4 : 1];
    __shared__ uint8_t lds_vnew[APPEND ? 128 : 1];
    __shared__ u32x4 lds_vrow[APPEND ? 64 : 1];  // the pending token's patched V rows, one per lane
    const int lane = threadIdx.x;
    const int g = blockIdx.x;
    uint8_t* knew = reinterpret_cast<uint8_t*>(lds_knew);
    PendingAppend4 pend{-1, 0, f32x2{0.0f, 0.0f}, f32x2{0.0f, 0.0f}};
    if constexpr (BAL) {
        const int w = blockIdx.y;
        for_each_segment(a, w, g == 0 && w == 0, lane, [&](int b, int n, int nt, int lo, int hi) {
            gqa4_segment<APPEND>(a, b, g, n, nt, lo, hi, a.S, w + b, lane, knew, lds_vnew, lds_vrow, pend);
        });
        if constexpr (APPEND) flush_append4(a, pend, knew, lds_vrow, g, lane);
    } else {
        const int p = blockIdx.y;
        const int b = blockIdx.z;
        const int G = a.Hq / a.Hkv;
        const int n = a.ctx[b];
        if (n <= 0) {
            if (p == 0) {
                for (int jh = 0; jh < G; ++jh) {
                    const size_t orow = ((size_t)b * a.Hq + g * G + jh) * kDim;
                    a.out[orow + lane] = 0;
                    a.out[orow + 64 + lane] = 0;
                }
            }
            return;
        }
        const int nt = tiles_of(n);
        const int lo = p * (a.PS / kBlock);
        if (lo >= nt) return;
        const int hi = min(nt, lo + a.PS / kBlock);
        gqa4_segment<APPEND>(a, b, g, n, nt, lo, hi, a.P, (int64_t)b * a.Hq * a.P + p, lane, knew, lds_vnew,
                             lds_vrow, pend);
        if constexpr (APPEND) flush_append4(a, pend, knew, lds_vrow, g, lane);
    }
}

template <bool BAL>
void launch_gqa4(const KernelParams& kp, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
    const dim3 grid = BAL ? dim3((unsigned)kp.Hkv, (unsigned)kp.NW)
                          : dim3((unsigned)kp.Hkv, (unsigned)kp.P, (unsigned)kp.B);
    if (kp.k_new)
        launch_timed(attn_partition_mfma4<true, BAL>, grid, kp, stream, t0, t1);
    else
        launch_timed(attn_partition_mfma4<false, BAL>, grid, kp, stream, t0, t1);
}

}  // namespace

void launch_partition_gqa4(const KernelParams& kp, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    if (kp.NW > 0)
        launch_gqa4<true>(kp, stream, start, stop);
    else
        launch_gqa4<false>(kp, stream, start, stop);
}

}  // namespace kvq
