// kvq_prefill.hip -- prefill / chunked-prefill attention over the paged 8-bit cache.
//
// Sequence b brings n_b new query rows (rows cu_q[b] .. cu_q[b+1]-1), the last n_b of its
// context_lens[b] tokens; row j sits at position p = context_lens[b] - n_b + j and attends to the
// cache tokens at positions 0 .. p (causal).  Decode is the case n_b = 1.  The cache is stored as
// 8-bit codes and the arithmetic runs at higher precision ("Accelerating Inference with FP8 KV
// Cache", opening section), exactly as in the decode kernels: codes decoded exactly to fp16, fp16
// products summed in fp32 on the matrix cores, base-2 online softmax in fp32, scales factored out
// of the sums.
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
// F8Q (FP8 math, OCP E4M3 / E5M2 caches): each column's query row is quantized to E4M3 with its own
// scale (kvq_fp8m.h) and S^T of a tile is one v_mfma_scale_f32_16x16x128_f8f6f4 per block with the
// K codes as loaded.
#include "kvq_attn.h"
#include "kvq_fp8m.h"
#include "kvq_int4.h"

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
    int32_t R;              // query rows per column block (16 / G)
    int32_t row_tiles;      // grid extent over groups of kPfWaves row tiles (NB R rows each)
    float qk_scale;         // sm_scale * log2(e) (* kv_scale * code_unit for FP8)
    float v_scale;          // kv_scale * code_unit for FP8, 1 for INT8
};

// NB column blocks of 16 per wave (NB R consecutive rows): the K and V^T operands of a tile are
// decoded once and feed the MFMAs of every block.  A workgroup is kPfWaves waves holding
// consecutive row tiles of one (KV head, sequence); they read the same K/V tiles (each up to its own
// causal limit), so each chunk of TW tiles is loaded from memory once per workgroup into LDS and
// every wave reads its operands from there.  Loading every chunk once per wave left the kernel
// waiting on memory: a timing copy with the loads removed ran 1.9 times faster.
#ifndef KVQ_PREFILL_WAVES
#define KVQ_PREFILL_WAVES 4
#endif
constexpr int kPfWaves = KVQ_PREFILL_WAVES;
constexpr int kPfTW = 2;  // tiles per chunk, paired for the PV products

// One staged chunk: the tiles' codes as stored (INT8: with their sign bits flipped), and for INT8 the
// tiles' scale rows (K then V; the K scales times the logit scale, the V scales of the slots past
// the context zero).
struct alignas(16) PfStage {
    uint8_t k[kPfTW][kTileBytes];
    uint8_t v[kPfTW][kTileBytes];
    float s[kPfTW][2 * kBlock];
};

// Staged codes as fp16.  INT8 codes are staged with their sign bits flipped (q + 128 as unsigned
// bytes), one XOR per staged dword instead of one per decoded dword in every wave: each byte goes
// to the low byte of a half with high byte 0x64, the binary16 number 1024 + (q + 128), and
// subtracting 1152 leaves q exactly (as int8x2_to_f16, without its XOR).
template <int DT, int SEL>
__device__ __forceinline__ half2_t staged_to_f16(uint32_t w) {
    if constexpr (DT == KVQ_INT8) {
        constexpr uint32_t sel = (SEL == 0) ? 0x04010400u : 0x04030402u;
        const uint32_t x = __builtin_amdgcn_perm(0x64646464u, w, sel);
        return __builtin_bit_cast(half2_t, x) - half2_t{(_Float16)1152.0f, (_Float16)1152.0f};
    } else {
        return codes_to_f16<DT, SEL>(w);
    }
}

template <int DT>
__device__ __forceinline__ half8_v staged8(uint32_t w0, uint32_t w1) {
    return join8(staged_to_f16<DT, 0>(w0), staged_to_f16<DT, 1>(w0), staged_to_f16<DT, 0>(w1),
                 staged_to_f16<DT, 1>(w1));
}

// FOLD (FP8 formats with a positive logit scale): the logit scale f is applied inside the exponent,
// exp2(fma(s, f, -m)) with the raw products s and the chunk max taken on s (f > 0 keeps the order),
// one FMA per weight instead of a multiply and a subtraction.
template <int DT, int NB, bool F8Q, bool FOLD>
__global__ __launch_bounds__(64 * kPfWaves) __attribute__((amdgpu_waves_per_eu(2, 8))) void attn_prefill_mfma(
    PrefillParams a) {
    static_assert(!(FOLD && DT == KVQ_INT8), "the INT8 logit scale is per token");
    constexpr int TW = kPfTW;
    __shared__ PfStage stage[3];  // three chunks: one read by the softmax, one by S^T, one filling
    const int g = blockIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // (wave-uniform: scalar registers)
    const int lane = threadIdx.x & 63;
    // the row-tile groups of a sequence run last-first: later rows read more tiles (longest first)
    const int rt = kPfWaves * (a.row_tiles - 1 - (int)blockIdx.y) + wave;
    const int b = blockIdx.z;
    const int col = lane & 15;  // column of each block: (row jr, head hg)
    const int q4 = lane >> 4;   // MFMA k-group / C row group

    const int r0 = a.cu_q[b];
    const int nq = a.cu_q[b + 1] - r0;
    const int rows_wave = NB * a.R;
    const int j0 = rt * rows_wave;
    const int j0_first = (rt - wave) * rows_wave;  // the workgroup's first row
    if (j0_first >= nq) return;                    // (workgroup-uniform)
    const int n = a.ctx[b];
    const bool rows = j0 < nq;  // this wave holds query rows (the others only help load)
    const int jr = col / a.G, hg = col % a.G;
    bool live[NB];        // the column of block nb holds a real (row, head)
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
        return;  // (workgroup-uniform)
    }
    const int pos_min = n - nq + j0;                    // the wave's first row: every column sees 0..pos_min
    const int t_end = n - nq + min(nq, j0 + rows_wave);  // tokens the wave reads: up to its last row
    const int tile_end = rows ? (t_end + kBlock - 1) / kBlock : 0;
    // the workgroup's tiles: those of its last wave with rows
    const int wg_t_end = n - nq + min(nq, j0_first + kPfWaves * rows_wave);
    const int wg_tile_end = (wg_t_end + kBlock - 1) / kBlock;
    int pos[NB];  // last visible position of each block's column (padding columns: pos_min)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) pos[nb] = live[nb] ? n - nq + j0 + nb * a.R + jr : pos_min;
    const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks;

    // Q^T operands: MFMA m covers dims 64 (m/2) + 16 q4 + 8 (m%2) .. +7 in k-slots 8 q4 .. +7
    half8_v qB[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int m = 0; m < 4; ++m) qB[nb][m] = half8_v{0, 0, 0, 0, 0, 0, 0, 0};
        if (live[nb]) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
                qB[nb][m] = *reinterpret_cast<const half8_v*>(a.q + orow[nb] + 64 * (m >> 1) + 16 * q4 + 8 * (m & 1));
        }
    }
    [[maybe_unused]] i32x8 q8[NB];       // F8Q: the E4M3 codes of qB
    float qk_f[NB];                      // logit scale of each block's column
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        qk_f[nb] = a.qk_scale;
        if constexpr (F8Q) qk_f[nb] *= quantize_q_row_fp8(qB[nb], q8[nb]);
        if constexpr (FOLD) qk_f[nb] = fmaxf(qk_f[nb], 1.17549435e-38f);  // -inf * f must stay -inf
    }

    float m_run[NB], l_lane[NB];  // per block: reference max (base-2 logits) and this lane's weights
    float4_t acc[NB][8];          // O^T row blocks: dims 16 r + 4 q4 .. +3 of the block's column
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        m_run[nb] = kNegInf;
        l_lane[nb] = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[nb][r] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }

    const uint32_t k_off = 16u * (uint32_t)lane;  // chunk q4 (+4): token col, dims 16 q4 (+64)
    const uint32_t v_off = (uint32_t)col * kBlock + 4u * (uint32_t)q4;  // dim col (+16 r), tokens 4 q4

    // Block ids in groups of 64 tiles, one per lane (the same in every wave): ids_cur for group grp,
    // ids_nxt for grp + 1 (loaded a group ahead).  The staging loads run two chunks ahead.
    auto load_ids = [&](int group) {
        const int t = group * 64 + lane;
        return t < wg_tile_end ? bt[t] : 0;
    };
    int grp = 0;
    int ids_cur = load_ids(0), ids_nxt = load_ids(1);
    auto block_of = [&](int t) {
        return (t >> 6) == grp ? __builtin_amdgcn_readlane(ids_cur, t & 63)
                               : __builtin_amdgcn_readlane(ids_nxt, t & 63);
    };
    auto ids_for = [&](int t) {
        if ((t >> 6) > grp + 1) {
            ++grp;
            ids_cur = ids_nxt;
            ids_nxt = load_ids(grp + 1);
        }
    };

    // Staging: wave w loads tile t0 + w / 2 of the chunk, its K codes (w even, with the INT8 scale
    // row in lanes 0..7) or its V codes (w odd): 32 bytes per lane.  Tiles at or past the
    // workgroup's last repeat that tile; their tokens are masked by every wave.
    const int st_tile = (wave >> 1) & 1;
    const bool st_k = (wave & 1) == 0;
    const bool stager = kPfWaves <= 2 * kPfTW || wave < 2 * kPfTW;  // the first four waves stage; any others only compute
    struct Staged { u32x4 x0, x1; float4_t sc; int valid; };
    auto stage_load = [&](int t0) {
        Staged r{};
        if (!stager) return r;
        const int tile = min(t0 + st_tile, wg_tile_end - 1);
        const int blk = block_of(tile);
        r.valid = n - tile * kBlock;  // the tile's tokens inside the context
        const uint8_t* src = (st_k ? a.kc : a.vc) + ((size_t)blk * a.Hkv + g) * kTileBytes;
        r.x0 = ld16(src + 32u * (uint32_t)lane);
        r.x1 = ld16(src + 32u * (uint32_t)lane + 16u);
        r.sc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (DT == KVQ_INT8) {
            if (st_k && lane < 8)
                r.sc = *reinterpret_cast<const float4_t*>(a.ks + int8_scale_index(blk, a.Hkv, g, 0) + 4 * lane);
        }
        return r;
    };
    auto stage_store = [&](PfStage& st, const Staged& r) {
        if (!stager) return;
        uint8_t* dst = (st_k ? st.k[st_tile] : st.v[st_tile]) + 32u * (uint32_t)lane;
        u32x4 x0 = r.x0, x1 = r.x1;
        // V codes of the slots past the context (only in its last tile) are zeroed: they may hold
        // NaN codes, and their zero weights alone would still give 0 * NaN.  The lane's 32 bytes are
        // dims 2 lane and 2 lane + 1, tokens 0..15 each.  (K codes there only reach logits that the
        // causal mask replaces.)
        if (!st_k && r.valid < kBlock) {
            x0 = u32x4{keep_bytes(x0.x, r.valid), keep_bytes(x0.y, r.valid - 4), keep_bytes(x0.z, r.valid - 8),
                       keep_bytes(x0.w, r.valid - 12)};
            x1 = u32x4{keep_bytes(x1.x, r.valid), keep_bytes(x1.y, r.valid - 4), keep_bytes(x1.z, r.valid - 8),
                       keep_bytes(x1.w, r.valid - 12)};
        }
        if constexpr (DT == KVQ_INT8) {  // (after the zeroing: a zeroed code reads as 0)
            x0 ^= 0x80808080u;
            x1 ^= 0x80808080u;
        }
        *reinterpret_cast<u32x4*>(dst) = x0;
        *reinterpret_cast<u32x4*>(dst + 16) = x1;
        if constexpr (DT == KVQ_INT8) {
            // lanes 0..3: K scales of tokens 4 lane .. +3, times the logit scale (the product each
            // logit takes); lanes 4..7: V scales of tokens 4 (lane - 4) .. +3, those past the context
            // zeroed (they may be NaN, and a zero weight times NaN is NaN)
            if (st_k && lane < 8) {
                float4_t sc = r.sc;
                if (lane < 4) {
                    sc *= a.qk_scale;
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (4 * (lane - 4) + j >= r.valid) sc[j] = 0.0f;
                }
                *reinterpret_cast<float4_t*>(&st.s[st_tile][4 * lane]) = sc;
            }
        }
    };

    struct SBuf { float4_t s[NB][TW]; };

    // S^T of a chunk for every block, from the K operands decoded once (FP8 math: used as loaded)
    auto scores = [&](const PfStage& st, SBuf& sb) {
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            const u32x4 ka = *reinterpret_cast<const u32x4*>(st.k[i] + k_off);
            const u32x4 kb = *reinterpret_cast<const u32x4*>(st.k[i] + 1024u + k_off);
            if constexpr (F8Q) {
                const i32x8 k8 = k_fp8x32(ka, kb);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    sb.s[nb][i] = mfma_qk_fp8<DT>(k8, q8[nb], float4_t{0.0f, 0.0f, 0.0f, 0.0f});
            } else {
                const half8_v k0 = staged8<DT>(ka.x, ka.y), k1 = staged8<DT>(ka.z, ka.w);
                const half8_v k2 = staged8<DT>(kb.x, kb.y), k3 = staged8<DT>(kb.z, kb.w);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    float4_t c = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
                    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qB[nb][0], c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, qB[nb][1], c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(k2, qB[nb][2], c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(k3, qB[nb][3], c, 0, 0, 0);
                    sb.s[nb][i] = c;
                }
            }
        }
    };

    // Softmax of a chunk and its P V^T, with the lazy rescale (kRescaleSlack, kRescaleSlackInt8; a
    // branch every lane takes or skips together).
    auto softmax_pv = [&](const PfStage& st, SBuf& sb, int t0, auto&& mid) {
        const int tok_base = t0 * kBlock;  // first token of the chunk
        float4_t ks4[TW], vs4[TW];         // INT8: the (staged) scales of this lane's four tokens of each tile
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            ks4[i] = vs4[i] = float4_t{1.0f, 1.0f, 1.0f, 1.0f};
            if constexpr (DT == KVQ_INT8) {
                ks4[i] = *reinterpret_cast<const float4_t*>(&st.s[i][4 * q4]);
                vs4[i] = *reinterpret_cast<const float4_t*>(&st.s[i][kBlock + 4 * q4]);
            }
        }
        // The causal mask: a token past the column's own position gets -inf.  Only the chunks that
        // reach past the wave's first row need it (wave-uniform test).  FOLD masks the products
        // in place (they are the logits, scaled in the exponent; in place, the registers need no
        // copies where the branch joins); otherwise the scaled logits are masked.
        const bool diag = tok_base + TW * kBlock - 1 > pos_min;
        auto mask = [&](auto& v) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int lim = pos[nb] - (tok_base + 4 * q4);  // last visible offset in the chunk
#pragma unroll
                for (int i = 0; i < TW; ++i)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (i * kBlock + t > lim) v[nb][i][t] = kNegInf;
            }
        };
        if constexpr (FOLD) {
            if (diag) mask(sb.s);
        }
        float z[NB][TW][4];
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if constexpr (FOLD) {
                        z[nb][i][t] = sb.s[nb][i][t];  // scaled inside the exponent below
                    } else if constexpr (DT == KVQ_INT8) {
                        z[nb][i][t] = sb.s[nb][i][t] * ks4[i][t];  // (K scale times the logit scale)
                    } else {
                        z[nb][i][t] = sb.s[nb][i][t] * qk_f[nb];
                    }
                }
        if constexpr (!FOLD) {
            if (diag) mask(z);
        }
        // Every column sees token 0, which the first chunk holds, so the reference max is finite
        // from then on.  The column max (over the column's four lanes) is taken only when some
        // lane's own max passes the reference max plus the slack: the column max passes it exactly
        // when one of its lanes' maxima does (scaling by f > 0 is monotone), so the rescale
        // decisions are those of the column max, without its cross-lane reduction on every chunk.
        constexpr float slack = DT == KVQ_INT8 ? kRescaleSlackInt8 : kRescaleSlack;
        bool moved = false;
        float lmax[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            float m = kNegInf;
#pragma unroll
            for (int i = 0; i < TW; ++i)
#pragma unroll
                for (int t = 0; t < 4; ++t) m = fmaxf(m, z[nb][i][t]);
            lmax[nb] = m;
            if constexpr (FOLD) m *= qk_f[nb];  // the max of s f, as f > 0
            moved |= m > m_run[nb] + slack;     // m_run = -inf: any finite max
        }
        if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float cmax = col_max4(lmax[nb]);
                if constexpr (FOLD) cmax *= qk_f[nb];
                const bool up = cmax > m_run[nb] + slack;
                const float alpha = up ? __builtin_amdgcn_exp2f(m_run[nb] - cmax) : 1.0f;
                l_lane[nb] *= alpha;
#pragma unroll
                for (int r = 0; r < 8; ++r) acc[nb][r] *= alpha;
                if (up) m_run[nb] = cmax;
            }
        }
        // the next chunk's S^T products, in the same basic block as the weights and P V^T below, so
        // that the scheduler can interleave their matrix instructions with this chunk's VALU work.
        // The wave runs this matrix-core block at raised priority (s_setprio 1, back to 0 after
        // P V^T): when both waves of a SIMD have an instruction ready, the one feeding the matrix
        // cores issues first, and the other's softmax front, staging and barrier fill its gaps.
        // (Not under FP8 math, whose S^T is one matrix instruction per block and tile: there it
        // measured slower.)
        if constexpr (!F8Q) __builtin_amdgcn_s_setprio(1);
        mid();

        // weights of the tile pair, hi and lo fp16 parts, in the B layout, per block
        half8_v whi[NB], wlo[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            uint32_t h[4], l[4];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                float w[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float pw = FOLD ? __builtin_amdgcn_exp2f(__builtin_fmaf(z[nb][u][t], qk_f[nb], -m_run[nb]))
                                          : __builtin_amdgcn_exp2f(z[nb][u][t] - m_run[nb]);
                    l_lane[nb] += pw;
                    w[t] = pw;
                    // INT8: the slots past the context have zero weights and (staged) zero scales
                    if constexpr (DT == KVQ_INT8) w[t] = pw * vs4[u][t];
                }
                split_hi_lo(w[0], w[1], h[2 * u], l[2 * u]);
                split_hi_lo(w[2], w[3], h[2 * u + 1], l[2 * u + 1]);
            }
            whi[nb] = __builtin_bit_cast(half8_v, u32x4{h[0], h[1], h[2], h[3]});
            wlo[nb] = __builtin_bit_cast(half8_v, u32x4{l[0], l[1], l[2], l[3]});
        }
        uint32_t vd[TW][8];
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
            for (int r = 0; r < 8; ++r)
                vd[i][r] = *reinterpret_cast<const uint32_t*>(st.v[i] + v_off + (uint32_t)r * 256u);
        // (slots past the context were zeroed when staged; those in it past the column's own
        // position have zero weights)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const half8_v va8 = join8(staged_to_f16<DT, 0>(vd[0][r]), staged_to_f16<DT, 1>(vd[0][r]),
                                      staged_to_f16<DT, 0>(vd[1][r]), staged_to_f16<DT, 1>(vd[1][r]));
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                acc[nb][r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va8, whi[nb], acc[nb][r], 0, 0, 0);
                acc[nb][r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va8, wlo[nb], acc[nb][r], 0, 0, 0);
            }
        }
        if constexpr (!F8Q) __builtin_amdgcn_s_setprio(0);
    };

    // Pipeline over the workgroup's chunks, three LDS buffers: at step c the staging loads of chunk
    // c + 2 are in flight, S^T of chunk c + 1 is computed from its buffer, chunk c's softmax and
    // P V^T read theirs, and then chunk c + 2 is stored into the buffer chunk c - 1 used; one
    // barrier per step.  A wave computes only the chunks up to its own last tile.
    const int nch = (wg_tile_end + TW - 1) / TW;
    {
        ids_for(min(2 * TW - 1, wg_tile_end - 1));
        const Staged s0 = stage_load(0);
        stage_store(stage[0], s0);
        if (nch > 1) {
            const Staged s1 = stage_load(TW);
            stage_store(stage[1], s1);
        }
        __syncthreads();
    }
    SBuf SA, SB;
    if (0 < tile_end) scores(stage[0], SA);
    auto step = [&](SBuf& sc, SBuf& sn, int c) {
        const int t0 = c * TW;
        Staged nx;
        const bool more = c + 2 < nch;  // (workgroup-uniform)
        if (more) {
            ids_for(min(t0 + 3 * TW - 1, wg_tile_end - 1));
            nx = stage_load(t0 + 2 * TW);
        }
        // S^T of chunk c + 1 is computed by every wave that computes chunk c (on a wave's last chunk,
        // or past the workgroup's last, it reads a buffer of no use and its result is never read)
        if (t0 < tile_end) softmax_pv(stage[c % 3], sc, t0, [&] { scores(stage[(c + 1) % 3], sn); });
        if (more) stage_store(stage[(c + 2) % 3], nx);
        __syncthreads();
    };
    for (int c = 0; c < nch; c += 2) {
        step(SA, SB, c);
        if (c + 1 >= nch) break;
        step(SB, SA, c + 1);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        // sum of the column's weights over the four row groups
        const float l_sum = col_sum4(l_lane[nb]);
        if (live[nb]) {
            const float inv = a.v_scale / l_sum;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const half4_t o = {(_Float16)(acc[nb][r][0] * inv), (_Float16)(acc[nb][r][1] * inv),
                                   (_Float16)(acc[nb][r][2] * inv), (_Float16)(acc[nb][r][3] * inv)};
                *reinterpret_cast<half4_t*>(a.out + orow[nb] + 16 * r + 4 * q4) = o;
            }
        }
    }
}

#ifndef KVQ_PREFILL_BLOCKS
#define KVQ_PREFILL_BLOCKS 2
#endif

hipError_t launch_prefill(const PrefillArgs& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    const kvq_cache& c = *p.cache;
    if (c.dtype == KVQ_INT4) return launch_prefill4(p, stream, start, stop);
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
    // row_tiles counts groups of kPfWaves row tiles (one workgroup each)
    const int rows_per_group = kPfWaves * KVQ_PREFILL_BLOCKS * a.R;
    a.row_tiles = (p.max_q_len + rows_per_group - 1) / rows_per_group;
    const bool fp8 = is_fp8(c.dtype);
    // the decoders give code values divided by code_unit (a power of two): fold it into the scales
    const float unit_scale = fp8 ? c.kv_scale * code_unit(c.dtype) : 1.0f;
    a.qk_scale = p.sm_scale * kLog2e * unit_scale;
    a.v_scale = unit_scale;
    const dim3 grid((unsigned)a.Hkv, (unsigned)a.row_tiles, (unsigned)p.batch);
    auto go = [&](auto kernel) {
        if (start)
            hipExtLaunchKernelGGL(kernel, grid, dim3(64 * kPfWaves), 0, stream, start, stop, 0, a);
        else
            hipLaunchKernelGGL(kernel, grid, dim3(64 * kPfWaves), 0, stream, a);
    };
    const bool fold = a.qk_scale > 0.0f;  // FOLD needs a positive logit scale
    if (p.fp8_math) {
        if (c.dtype == KVQ_FP8_E5M2) {
            if (fold) go(attn_prefill_mfma<KVQ_FP8_E5M2, KVQ_PREFILL_BLOCKS, true, true>);
            else go(attn_prefill_mfma<KVQ_FP8_E5M2, KVQ_PREFILL_BLOCKS, true, false>);
        } else {
            if (fold) go(attn_prefill_mfma<KVQ_FP8_E4M3, KVQ_PREFILL_BLOCKS, true, true>);
            else go(attn_prefill_mfma<KVQ_FP8_E4M3, KVQ_PREFILL_BLOCKS, true, false>);
        }
        return hipGetLastError();
    }
    switch (c.dtype) {
        case KVQ_FP8_E4M3:
            if (fold) go(attn_prefill_mfma<KVQ_FP8_E4M3, KVQ_PREFILL_BLOCKS, false, true>);
            else go(attn_prefill_mfma<KVQ_FP8_E4M3, KVQ_PREFILL_BLOCKS, false, false>);
            break;
        case KVQ_FP8_E5M2:
            if (fold) go(attn_prefill_mfma<KVQ_FP8_E5M2, KVQ_PREFILL_BLOCKS, false, true>);
            else go(attn_prefill_mfma<KVQ_FP8_E5M2, KVQ_PREFILL_BLOCKS, false, false>);
            break;
        case KVQ_FP8_E4M3FNUZ:
            if (fold) go(attn_prefill_mfma<KVQ_FP8_E4M3FNUZ, KVQ_PREFILL_BLOCKS, false, true>);
            else go(attn_prefill_mfma<KVQ_FP8_E4M3FNUZ, KVQ_PREFILL_BLOCKS, false, false>);
            break;
        default: go(attn_prefill_mfma<KVQ_INT8, KVQ_PREFILL_BLOCKS, false, false>); break;
    }
    return hipGetLastError();
}

}  // namespace kvq
