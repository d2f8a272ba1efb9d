// kvq_attn_gqa.hip -- decode attention for grouped query heads (the MFMA kernel).
#include "kvq_attn.h"
#include "kvq_fp8m.h"

namespace kvq {

// Grouped-query kernel: one wave per (KV head, share of the work) serves the G <= 16 query heads
// that share the KV head, so each K/V code is read and decoded once for all of them, and the two
// products run on the matrix cores (v_mfma_f32_16x16x32_f16, query heads padded to 16 columns):
//   S^T = K Q^T   per tile: A = K rows (lane: token lane%16, 8 of its dims), B = Q^T (lane: head
//                 lane%16, the same 8 dims), C = 16 tokens x 16 heads (lane: head lane%16, tokens
//                 4 (lane/16) .. +3).  The 128 dims are 4 MFMAs of 32; any fixed assignment of dims
//                 to MFMA k-slots works as long as K and Q agree.
//   O^T += V^T P^T per pair of tiles and 16-dim row block: A = V^T (lane: dim, tokens 4 (lane/16)
//                 .. +3 of both tiles, read as one dword per tile from the dim-major V rows),
//                 B = P^T in exactly the layout the S^T accumulator left it (lane: head, the same
//                 tokens), so no transposition is needed.  P is split into fp16 hi + lo parts.
// The online softmax keeps one running max per head (all lanes of a column agree).
// F8Q (FP8 math, OCP E4M3 / E5M2 caches): the wave quantizes its query rows to E4M3 (one scale per
// head, kvq_fp8m.h) and S^T of a tile is one v_mfma_scale_f32_16x16x128_f8f6f4 with the lane's K
// codes as loaded (32 one-byte k-slots per lane), so K needs no decode; the head's s_q joins its
// logit scale.  P V^T is unchanged.  With F8Q the kernel also serves one query head per KV head.

// Replace the appended token's slot in the MFMA operand registers of its tile by the codes in LDS
// (K: lane (token, k-group) takes chunks q4 and q4 + 4 of the token; V: the lanes of k-group
// slot / 4 hold the slot's byte in each of their dwords).
template <int DT>
__device__ __forceinline__ void gqa_patch(const NewToken& nt, const u32x4* lds_k, const uint8_t* lds_v,
                                          int lane, u32x4& ka, u32x4& kb, uint32_t (&vd)[8],
                                          float4_t& ks4, float4_t& vs4) {
    const int col = lane & 15, q4 = lane >> 4;
    if (col == nt.slot) {
        ka = lds_k[q4];
        kb = lds_k[4 + q4];
    }
    if (q4 == (nt.slot >> 2)) {
        const int sh = 8 * (nt.slot & 3);
#pragma unroll
        for (int r = 0; r < 8; ++r)
            vd[r] = (vd[r] & ~(0xFFu << sh)) | ((uint32_t)lds_v[16 * r + col] << sh);
        if constexpr (DT == KVQ_INT8) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (t == (nt.slot & 3)) {
                    ks4[t] = nt.ks;
                    vs4[t] = nt.vs;
                }
        }
    }
}

// The appended token's stores, held back until the wave has read all its tiles (stored between
// tiles, into the tile just streamed, they stall the wave's later waits for loads: a CDNA wave
// counts vector loads and stores in one counter).  The K codes wait in LDS, this lane's patched V
// dwords in registers.
struct PendingAppendG {
    int blk;          // physical block of the token's tile; -1 when nothing is pending (wave-uniform)
    int slot;         // position inside the tile
    uint32_t vd[8];   // this lane's V dwords (dims col + 16 r, tokens 4 q4 .. +3), patched
    float ks, vs;     // INT8 scales
};

// Store a pending token: its eight K chunks from LDS (lanes 0..7), the whole V tile from the patched
// registers (each store instruction writes 256 contiguous bytes; the other tokens' bytes are
// written back unchanged -- this wave is the only reader and writer of the tile), and the INT8
// scales.
template <int DT>
__device__ __forceinline__ void flush_append_g(const KernelParams& a, PendingAppendG& pa,
                                               const u32x4* lds_k, int g, int lane, uint32_t v_off) {
    if (pa.blk < 0) return;
    const size_t tile = ((size_t)pa.blk * a.Hkv + g) * kTileBytes;
    uint8_t* kt = const_cast<uint8_t*>(a.kc) + tile;
    uint8_t* vt = const_cast<uint8_t*>(a.vc) + tile;
    if (lane < 8)
        __builtin_nontemporal_store(lds_k[lane], reinterpret_cast<u32x4*>(kt + k_byte(pa.slot, kChunk * lane)));
#pragma unroll
    for (int r = 0; r < 8; ++r)
        __builtin_nontemporal_store(pa.vd[r], reinterpret_cast<uint32_t*>(vt + v_off + (uint32_t)r * 256u));
    if constexpr (DT == KVQ_INT8) {
        if (lane == 0) {
            const size_t so = int8_scale_index(pa.blk, a.Hkv, g, pa.slot);
            const_cast<float*>(a.ks)[so] = pa.ks;
            const_cast<float*>(a.vs)[so] = pa.vs;
        }
    }
    pa.blk = -1;
}

// APPEND: the decode step's new token is quantized by the wave whose segment holds the sequence's
// last tile and patched into its registers; its stores are left pending until the wave's end (one
// wave per (KV head, tile) reads it, so the wave is the tile's only reader and writer).
template <int DT, int TW, bool APPEND, bool F8Q>
__device__ __forceinline__ void gqa_segment(const KernelParams& a, int b, int g, int n, int nt, int lo,
                                            int hi, int64_t rmul, int64_t radd, int lane,
                                            u32x4* lds_knew, uint8_t* lds_vnew, PendingAppendG& pend) {
    static_assert(TW % 2 == 0, "tiles are paired for the PV products");
    const int col = lane & 15;  // query head within the group (B / C column), or A row
    const int q4 = lane >> 4;   // MFMA k-group / C row group
    const int G = a.Hq / a.Hkv;
    const int h = g * G + col;  // this lane's query head (valid when col < G)
    const int t_end = min(n, hi * kBlock);
    const int tile_begin = lo;
    const int tile_end = hi;
    const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks;

    // fused append: the new row's loads are issued now, its encode waits for its tile (the last)
    NewRow raw{0u, 0u, 0u};
    int tile_new = -1;
    if constexpr (APPEND) {
        if (hi == nt) {
            raw = load_new_row(a, b, g, lane);
            tile_new = nt - 1;
        }
    }

    // Q^T operands: MFMA m covers dims 64 (m/2) + 16 q4 + 8 (m%2) .. +7 in k-slots 8 q4 .. +7
    half8_v qB[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) qB[m] = half8_v{0, 0, 0, 0, 0, 0, 0, 0};
    if (col < G) {
        const uint16_t* qrow = a.q + ((size_t)b * a.Hq + h) * kDim;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            qB[m] = *reinterpret_cast<const half8_v*>(qrow + 64 * (m >> 1) + 16 * q4 + 8 * (m & 1));
    }
    [[maybe_unused]] i32x8 q8;       // F8Q: the E4M3 codes of qB
    float qk_f = a.qk_scale;         // logit scale of this lane's head
    if constexpr (F8Q) qk_f *= quantize_q_row_fp8(qB, q8);

    float m_run = kNegInf;  // running max of this lane's head (base-2 logits)
    float l_lane = 0.0f;    // sum of this lane's weights (tokens 4 q4 .. +3 of every tile)
    float4_t acc[8];        // O^T row blocks: dims 16 r + 4 q4 .. +3 of head col
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const uint32_t k_off = 16u * (uint32_t)lane;  // chunk q4 (+4): token col, dims 16 q4 (+64)
    const uint32_t v_off = (uint32_t)col * kBlock + 4u * (uint32_t)q4;  // dim col (+16 r), tokens 4 q4

    for (int tb = tile_begin; tb < tile_end; tb += 64) {
        const int nt_grp = min(64, tile_end - tb);
        // Lanes past the group's tiles repeat its last block, so a chunk's loads are issued together
        // with no branch between them; the extra tiles' tokens lie past the segment: their logits
        // are masked and their V codes zeroed below.
        const int blk_lane = bt[tb + min(lane, nt_grp - 1)];
        for (int c0 = 0; c0 < nt_grp; c0 += TW) {
            u32x4 ka[TW], kb[TW];
            uint32_t vd[TW][8];
            float4_t ks4[TW], vs4[TW];
#pragma unroll
            for (int i = 0; i < TW; ++i) {
                const int blk = __builtin_amdgcn_readlane(blk_lane, c0 + i);
                const size_t tile = ((size_t)blk * a.Hkv + g) * kTileBytes;
                const uint8_t* kt = a.kc + tile;
                const uint8_t* vt = a.vc + tile;
                ka[i] = ldg16(kt + k_off);
                kb[i] = ldg16(kt + k_off + 1024u);
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    vd[i][r] = ldg4(vt + v_off + (uint32_t)r * 256u);
                if constexpr (DT == KVQ_INT8) {
                    const size_t so = int8_scale_index(blk, a.Hkv, g, 4 * q4);
                    ks4[i] = ldg_nt(reinterpret_cast<const float4_t*>(a.ks + so));
                    vs4[i] = ldg_nt(reinterpret_cast<const float4_t*>(a.vs + so));
                } else {
                    ks4[i] = vs4[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
            if constexpr (APPEND) {
                const int inew = tile_new - (tb + c0);  // wave-uniform
                if (inew >= 0 && inew < TW) {
                    flush_append_g<DT>(a, pend, lds_knew, g, lane, v_off);  // an earlier token, if any
                    const NewToken ntok = new_token<DT>(a, raw, n, lane, reinterpret_cast<uint16_t*>(lds_knew));
                    lds_vnew[lane] = (uint8_t)ntok.v0;
                    lds_vnew[64 + lane] = (uint8_t)ntok.v1;
                    __builtin_amdgcn_wave_barrier();
#pragma unroll
                    for (int i = 0; i < TW; ++i)
                        if (i == inew) {
                            gqa_patch<DT>(ntok, lds_knew, lds_vnew, lane, ka[i], kb[i], vd[i], ks4[i],
                                          vs4[i]);
                            pend.blk = __builtin_amdgcn_readlane(blk_lane, c0 + i);
                            pend.slot = ntok.slot;
#pragma unroll
                            for (int r = 0; r < 8; ++r) pend.vd[r] = vd[i][r];
                            pend.ks = ntok.ks;
                            pend.vs = ntok.vs;
                        }
                }
            }
            // logits S^T: lane holds tokens 4 q4 .. +3 of each tile for head col
            float z[TW][4];
            float cmax = kNegInf;
#pragma unroll
            for (int i = 0; i < TW; ++i) {
                float4_t sacc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (F8Q) {
                    sacc = mfma_qk_fp8<DT>(k_fp8x32(ka[i], kb[i]), q8, sacc);
                } else {
                    sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8<DT>(ka[i].x, ka[i].y), qB[0], sacc, 0, 0, 0);
                    sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8<DT>(ka[i].z, ka[i].w), qB[1], sacc, 0, 0, 0);
                    sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8<DT>(kb[i].x, kb[i].y), qB[2], sacc, 0, 0, 0);
                    sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8<DT>(kb[i].z, kb[i].w), qB[3], sacc, 0, 0, 0);
                }
                const int pos0 = (tb + c0 + i) * kBlock + 4 * q4;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    float f = qk_f;
                    if constexpr (DT == KVQ_INT8) f *= ks4[i][t];
                    z[i][t] = (pos0 + t < t_end) ? sacc[t] * f : kNegInf;
                    cmax = fmaxf(cmax, z[i][t]);
                }
            }
            // max over the head's tokens (the four row groups of the column); finite: every chunk
            // holds a valid token.  Lazy rescale (kRescaleSlack, kRescaleSlackInt8), a branch every
            // lane takes or skips together.
            cmax = col_max4(cmax);
            constexpr float slack = DT == KVQ_INT8 ? kRescaleSlackInt8 : kRescaleSlack;
            const bool up = cmax > m_run + slack;  // m_run = -inf: any finite max
            if (__builtin_amdgcn_ballot_w64(up)) {
                const float alpha = up ? __builtin_amdgcn_exp2f(m_run - cmax) : 1.0f;
                if (up) m_run = cmax;
                l_lane *= alpha;
#pragma unroll
                for (int r = 0; r < 8; ++r) acc[r] *= alpha;
            }

#pragma unroll
            for (int i = 0; i < TW; i += 2) {
                // weights of the tile pair (i, i+1), hi and lo fp16 parts, in the B layout
                uint32_t h[4], l[4];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    float w[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float pw = __builtin_amdgcn_exp2f(z[i + u][t] - m_run);
                        l_lane += pw;
                        w[t] = pw;
                        if constexpr (DT == KVQ_INT8) w[t] = (pw > 0.0f) ? pw * vs4[i + u][t] : 0.0f;
                    }
                    split_hi_lo(w[0], w[1], h[2 * u], l[2 * u]);
                    split_hi_lo(w[2], w[3], h[2 * u + 1], l[2 * u + 1]);
                }
                const half8_v whi = __builtin_bit_cast(half8_v, u32x4{h[0], h[1], h[2], h[3]});
                const half8_v wlo = __builtin_bit_cast(half8_v, u32x4{l[0], l[1], l[2], l[3]});
                // V codes of the slots past the end are zeroed (they may hold NaN codes)
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
    // sum of the head's weights over the four row groups
    const float l_sum = col_sum4(l_lane);

    if (col < G) {
        if (lo == 0 && hi == nt) {
            const float inv = a.v_scale / l_sum;
            uint16_t* orow = a.out + ((size_t)b * a.Hq + h) * kDim;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const half4_t o = {(_Float16)(acc[r][0] * inv), (_Float16)(acc[r][1] * inv),
                                   (_Float16)(acc[r][2] * inv), (_Float16)(acc[r][3] * inv)};
                *reinterpret_cast<half4_t*>(orow + 16 * r + 4 * q4) = o;
            }
        } else {
            const int64_t prow = h * rmul + radd;
#pragma unroll
            for (int r = 0; r < 8; ++r)
                *reinterpret_cast<float4_t*>(a.part_o + prow * kDim + 16 * r + 4 * q4) = acc[r];
            if (q4 == 0) {
                a.part_m[prow] = m_run;
                a.part_l[prow] = l_sum;
            }
        }
    }
}

// BAL: grid (KV head, wave of the balanced split), else (KV head, partition, sequence).
template <int DT, int TW, bool APPEND, bool BAL, bool F8Q>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(BAL ? 2 : ((DT == KVQ_INT8 || DT == KVQ_FP8_E4M3FNUZ) && APPEND ? 3 : 4), 8))) void attn_partition_mfma(
    KernelParams a) {
    __shared__ u32x4 lds_knew[APPEND ? 8 : 1];
    __shared__ uint8_t lds_vnew[APPEND ? 128 : 1];
    const int lane = threadIdx.x;
    const int g = blockIdx.x;
    // V offset of this lane: dim col (+16 r), tokens 4 q4 (as in gqa_segment)
    const uint32_t v_off = (uint32_t)(lane & 15) * kBlock + 4u * (uint32_t)(lane >> 4);
    PendingAppendG pend{-1, 0, {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u}, 0.0f, 0.0f};
    if constexpr (BAL) {
        const int w = blockIdx.y;
        for_each_segment(a, w, g == 0 && w == 0, lane, [&](int b, int n, int nt, int lo, int hi) {
            gqa_segment<DT, TW, APPEND, F8Q>(a, b, g, n, nt, lo, hi, a.S, w + b, lane, lds_knew, lds_vnew, pend);
        });
        if constexpr (APPEND) flush_append_g<DT>(a, pend, lds_knew, g, lane, v_off);
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
        gqa_segment<DT, TW, APPEND, F8Q>(a, b, g, n, nt, lo, hi, a.P, (int64_t)b * a.Hq * a.P + p, lane,
                                         lds_knew, lds_vnew, pend);
        if constexpr (APPEND) flush_append_g<DT>(a, pend, lds_knew, g, lane, v_off);
    }
}

// Tiles per chunk (even: tiles are paired for the PV products).
#ifndef KVQ_GQA_TILES
#define KVQ_GQA_TILES 2
#endif

template <int DT, bool BAL, bool F8Q>
static void launch_gqa(const KernelParams& kp, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
    // one wave per KV head; the KV head is the fastest grid dimension
    const dim3 grid = BAL ? dim3((unsigned)kp.Hkv, (unsigned)kp.NW)
                          : dim3((unsigned)kp.Hkv, (unsigned)kp.P, (unsigned)kp.B);
    if (kp.k_new)
        launch_timed(attn_partition_mfma<DT, KVQ_GQA_TILES, true, BAL, F8Q>, grid, kp, stream, t0, t1);
    else
        launch_timed(attn_partition_mfma<DT, KVQ_GQA_TILES, false, BAL, F8Q>, grid, kp, stream, t0, t1);
}

template <int DT, bool F8Q = false>
static void launch_gqa(const KernelParams& kp, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
    if (kp.NW > 0)
        launch_gqa<DT, true, F8Q>(kp, stream, t0, t1);
    else
        launch_gqa<DT, false, F8Q>(kp, stream, t0, t1);
}

void launch_partition_gqa(const KernelParams& kp, int dtype, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop) {
    switch (dtype) {
        case KVQ_FP8_E4M3: launch_gqa<KVQ_FP8_E4M3>(kp, stream, start, stop); break;
        case KVQ_FP8_E5M2: launch_gqa<KVQ_FP8_E5M2>(kp, stream, start, stop); break;
        case KVQ_FP8_E4M3FNUZ: launch_gqa<KVQ_FP8_E4M3FNUZ>(kp, stream, start, stop); break;
        default: launch_gqa<KVQ_INT8>(kp, stream, start, stop); break;
    }
}

void launch_partition_fp8math(const KernelParams& kp, int dtype, hipStream_t stream, hipEvent_t start,
                              hipEvent_t stop) {
    if (dtype == KVQ_FP8_E5M2) launch_gqa<KVQ_FP8_E5M2, true>(kp, stream, start, stop);
    else launch_gqa<KVQ_FP8_E4M3, true>(kp, stream, start, stop);
}

}  // namespace kvq
