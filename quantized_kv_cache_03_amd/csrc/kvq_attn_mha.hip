// kvq_attn_mha.hip -- decode attention, one query head per KV head (the VALU kernel).
//
// One wave per (query head, share of the work); a wave streams its share in chunks of TW tiles of
// 16 tokens, issuing every K and V load of a chunk before using any, and keeps a running max / sum
// / accumulator across chunks.
//   K tile (eight 256-byte chunks of 16 dims x 16 tokens): lane l holds 32 dims of token l/4 --
//     chunks l%4 and l%4 + 4, one whole 1 KiB half of the tile per load instruction -- dots them
//     with its slice of q (v_dot2_f32_f16), and two quad DPP sums finish each logit.
//   V tile (dim-major 128 x 16 B): lane l holds the 16 tokens of dims l and 64 + l, so each lane
//     accumulates whole output elements; the 16 weights of a tile reach every lane as packed fp16
//     (hi, lo) pairs through a 64-byte LDS broadcast.
#include "kvq_attn.h"

namespace kvq {

template <int DT>
__device__ __forceinline__ float dot16(const u32x4& k, const half2_t* q8) {
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
__device__ __forceinline__ float pv16(const u32x4& v, const uint32_t* hi, const uint32_t* lo, float acc) {
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

// ------------------------------------------------------------------------------------------------
// The codes (and INT8 scales) one lane holds for one tile of 16 tokens.  Lane l is the (token
// tk = l / 4, chunk c = l % 4) piece of the K tile; the two K loads of a tile each read one whole
// 1 KiB half of it.
//   ka / kb : K codes of token tk, dims 16 c .. +15 (chunk c) and 64 + 16 c .. +15 (chunk c + 4)
//   va / vb : the 16 tokens' V codes of dims l and 64 + l
//   ks / vs : INT8 scales of token tk
struct Tile {
    u32x4 ka, kb, va, vb;
    float ks, vs;
};

template <int DT>
__device__ __forceinline__ void load_tile(const KernelParams& a, Tile& t, int blk, int g,
                                          uint32_t k_off, uint32_t v_off, int tk) {
    const size_t tile = ((size_t)blk * a.Hkv + g) * kTileBytes;
    const uint8_t* kt = a.kc + tile;
    const uint8_t* vt = a.vc + tile;
    t.ka = ldg16(kt + k_off);
    t.kb = ldg16(kt + 1024u + k_off);
    t.va = ldg16(vt + v_off);
    t.vb = ldg16(vt + 1024u + v_off);
    if constexpr (DT == KVQ_INT8) {
        const size_t so = int8_scale_index(blk, a.Hkv, g, tk);
        t.ks = ldg_nt(a.ks + so);
        t.vs = ldg_nt(a.vs + so);
    }
}

// Zero the V codes of the slots at and past `valid` (they may hold any code, NaN included, and a
// zero weight alone would still give 0 * NaN).
__device__ __forceinline__ void zero_tail(Tile& t, int valid) {
    t.va.x = keep_bytes(t.va.x, valid); t.va.y = keep_bytes(t.va.y, valid - 4);
    t.va.z = keep_bytes(t.va.z, valid - 8); t.va.w = keep_bytes(t.va.w, valid - 12);
    t.vb.x = keep_bytes(t.vb.x, valid); t.vb.y = keep_bytes(t.vb.y, valid - 4);
    t.vb.z = keep_bytes(t.vb.z, valid - 8); t.vb.w = keep_bytes(t.vb.w, valid - 12);
}

// ------------------------------------------------------------------------------------------------
// One chunk of TW tiles of the partition kernel.  Each lane dots its 32 K dims with the matching q
// slice; the four lanes of a quad (one token) then hold identical logits after two DPP sums.  The
// odd token of a pair takes its even neighbour's weight with a row shift, and one lane per pair
// publishes the packed (hi, lo) fp16 pairs in LDS -- the pairing of adjacent tokens in a V row --
// which every lane reads back with broadcast loads.  MASKED handles a chunk that reaches past the
// partition end (logits past the end become -inf; the caller has already zeroed the V codes of the
// partial tile).
template <int DT, int TW, bool MASKED>
__device__ __forceinline__ void chunk_step(const KernelParams& a, const Tile (&t)[TW], int tile0,
                                           int t_end, const half2_t (&qv)[16], int lane,
                                           uint32_t* lds, float& m_run, float& l_lane, float& acc0,
                                           float& acc1) {
    const int tk = lane >> 2;
    float z[TW];
    float cmax = kNegInf;
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        const float s = sum4(dot16<DT>(t[i].ka, qv) + dot16<DT>(t[i].kb, qv + 8));
        float f = a.qk_scale;
        if constexpr (DT == KVQ_INT8) f *= t[i].ks;
        z[i] = s * f;
        if constexpr (MASKED) z[i] = ((tile0 + i) * kBlock + tk < t_end) ? z[i] : kNegInf;
        cmax = fmaxf(cmax, z[i]);
    }
    cmax = max_across_quads(cmax);  // a chunk always holds at least one valid token
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    acc0 *= alpha;
    acc1 *= alpha;
    l_lane *= alpha;

#pragma unroll
    for (int i = 0; i < TW; ++i) {
        const float pw = __builtin_amdgcn_exp2f(z[i] - m_new);
        l_lane += pw;
        float w = pw;
        // masked slots may hold NaN scales: keep their weight exactly 0
        if constexpr (DT == KVQ_INT8) w = (pw > 0.0f) ? pw * t[i].vs : 0.0f;
        const float w_even = dpp<0x114>(w);  // row_shr:4: the weight of token tk - 1
        if ((lane & 7) == 4) {               // odd token of pair lane / 8, chunk 0
            uint32_t hi, lo;
            split_f16x2(w_even, w, hi, lo);
            lds[i * 16 + (lane >> 3)] = hi;
            lds[i * 16 + 8 + (lane >> 3)] = lo;
        }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        const u32x4* l4 = reinterpret_cast<const u32x4*>(lds + i * 16);
        const u32x4 h0 = l4[0], h1 = l4[1], w0 = l4[2], w1 = l4[3];
        const uint32_t whi[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
        const uint32_t wlo[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        acc0 = pv16<DT>(t[i].va, whi, wlo, acc0);
        acc1 = pv16<DT>(t[i].vb, whi, wlo, acc1);
        // keep the next tile's weight reads from being hoisted: they would pin 16 more VGPRs per tile
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_wave_barrier();
}

// Replace the new token's slot in the registers of its tile by the freshly computed codes.
template <int DT>
__device__ __forceinline__ void patch_tile(Tile& t, const NewToken& nt, const uint16_t* lds_k,
                                           int lane) {
    if ((lane >> 2) == nt.slot) {
        const u32x4* rowk = reinterpret_cast<const u32x4*>(lds_k);
        t.ka = rowk[lane & 3];
        t.kb = rowk[4 + (lane & 3)];
        if constexpr (DT == KVQ_INT8) { t.ks = nt.ks; t.vs = nt.vs; }
    }
    t.va = set_byte(t.va, nt.slot, nt.v0);
    t.vb = set_byte(t.vb, nt.slot, nt.v1);
}

// The appended token's stores, held back until the wave has read all its tiles.  Stored between
// tiles, into the tile the wave has just streamed, they cost ~6 us per step on the Llama-2-7B batch
// (a CDNA wave counts its vector loads and stores in one counter, so later waits for tile loads
// also wait for the stores); held to the wave's end they cost ~1.5 us.  (Holding back the partial
// rows likewise measured no gain, so those are written when ready.)  The K codes wait in LDS, this
// lane's two patched V rows in registers.
struct PendingAppend {
    int blk;       // physical block of the token's tile; -1 when nothing is pending (wave-uniform)
    int slot;      // position inside the tile
    u32x4 va, vb;  // this lane's two V rows (dims lane and 64 + lane) with the new code patched in
    float ks, vs;  // INT8 scales
};

// Store a pending token: its K codes (16 bytes in each of the eight chunks, from LDS, written by
// lanes 0..7) and its V codes.  A V tile row holds one dim's 16 tokens, so the token's V codes are
// one byte in each of 128 rows; each lane rewrites its two whole 16-byte rows as loaded with the
// new code patched in -- the other 15 bytes of each row are written back unchanged.  Only valid
// because this wave is the only reader and writer of the tile (one wave per query head = KV head
// and tile).
template <int DT>
__device__ __forceinline__ void flush_append(const KernelParams& a, PendingAppend& pa,
                                             const uint16_t* lds_k, int g, int lane) {
    if (pa.blk < 0) return;
    const size_t tile = ((size_t)pa.blk * a.Hkv + g) * kTileBytes;
    uint8_t* kt = const_cast<uint8_t*>(a.kc) + tile;
    uint8_t* vt = const_cast<uint8_t*>(a.vc) + tile;
    if (lane < 8) {
        const u32x4 kchunk = reinterpret_cast<const u32x4*>(lds_k)[lane];
        __builtin_nontemporal_store(kchunk, reinterpret_cast<u32x4*>(kt + k_byte(pa.slot, kChunk * lane)));
    }
    __builtin_nontemporal_store(pa.va, reinterpret_cast<u32x4*>(vt + 16u * (uint32_t)lane));
    __builtin_nontemporal_store(pa.vb, reinterpret_cast<u32x4*>(vt + 1024u + 16u * (uint32_t)lane));
    if constexpr (DT == KVQ_INT8) {
        if (lane == 0) {
            const size_t so = int8_scale_index(pa.blk, a.Hkv, g, pa.slot);
            const_cast<float*>(a.ks)[so] = pa.ks;
            const_cast<float*>(a.vs)[so] = pa.vs;
        }
    }
    pa.blk = -1;
}

// ------------------------------------------------------------------------------------------------
// MHA partition kernel: one wave per (query head, share of the work).  The work of one segment --
// tiles [lo, hi) of sequence b (n tokens, nt tiles) -- ends with the final output when the segment
// is the whole sequence, else with a partial in row h * rmul + radd.
// APPEND: the decode step's new token (one per sequence, at position context_lens[b] - 1) is
// quantized by the wave whose segment holds the sequence's last tile and patched into its
// registers; its stores are left pending (flush_append) until the wave has no loads left.
template <int DT, int TW, bool APPEND>
__device__ __forceinline__ void mha_segment(const KernelParams& a, int b, int h, int g, int n, int nt,
                                            int lo, int hi, int64_t rmul, int64_t radd, int lane,
                                            uint32_t* lds, u32x4* lds_knew, PendingAppend& pend) {
    const int tk = lane >> 2;
    const size_t orow = ((size_t)b * a.Hq + h) * kDim;
    const bool has_last = hi == nt;
    const int t_end = min(n, hi * kBlock);
    const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks;

    // fused append: the new row's loads are issued now, its encode waits for its tile (the last)
    NewRow raw{0u, 0u, 0u};
    int tile_new = -1;
    if constexpr (APPEND) {
        if (has_last) {
            raw = load_new_row(a, b, g, lane);
            tile_new = nt - 1;
        }
    }

    // q slice of this lane's K dims: 16 c .. +15 and 64 + 16 c .. +15 (c = lane % 4)
    half2_t qv[16];
    {
        const u32x4* qp = reinterpret_cast<const u32x4*>(a.q + orow + (lane & 3) * kChunk);
        const u32x4 q0 = qp[0], q1 = qp[1], q2 = qp[8], q3 = qp[9];
        const uint32_t qw[16] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w,
                                 q2.x, q2.y, q2.z, q2.w, q3.x, q3.y, q3.z, q3.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) qv[i] = __builtin_bit_cast(half2_t, qw[i]);
    }

    const uint32_t k_off = (uint32_t)kChunkBytes * ((uint32_t)lane & 3u) + (uint32_t)kChunk * (uint32_t)tk;
    const uint32_t v_off = 16u * (uint32_t)lane;

    float m_run = kNegInf;  // running max of the base-2 logits (wave-uniform)
    float l_lane = 0.0f;    // running sum of the weights of this lane's token
    float acc0 = 0.0f, acc1 = 0.0f;  // unnormalized output, dims lane and 64 + lane

    for (int tb = lo; tb < hi; tb += 64) {
        // block ids of up to 64 tiles, one per lane
        const int nt_grp = min(64, hi - tb);
        const int blk_lane = (lane < nt_grp) ? bt[tb + lane] : 0;

        // whole chunks: TW tiles, all inside the segment.  The sequence's last tile (which holds
        // the token a fused step appends) is always left to the single-tile loop below, with or
        // without the fused append, so that both give bitwise the same arithmetic.
        int full_tiles = min(nt_grp, (t_end - tb * kBlock) / kBlock);
        if (has_last) full_tiles = min(full_tiles, nt - 1 - tb);
        const int nfull = full_tiles / TW;
        for (int c = 0; c < nfull; ++c) {
            Tile t[TW];
#pragma unroll
            for (int i = 0; i < TW; ++i)
                load_tile<DT>(a, t[i], __builtin_amdgcn_readlane(blk_lane, c * TW + i), g, k_off,
                              v_off, tk);
            chunk_step<DT, TW, false>(a, t, tb + c * TW, t_end, qv, lane, lds, m_run, l_lane, acc0,
                                      acc1);
        }
        // the rest one tile at a time: the last one possibly partial, or holding the new token
        for (int c0 = nfull * TW; c0 < nt_grp; ++c0) {
            Tile t[1];
            load_tile<DT>(a, t[0], __builtin_amdgcn_readlane(blk_lane, c0), g, k_off, v_off, tk);
            if constexpr (APPEND) {
                if (tb + c0 == tile_new) {
                    uint16_t* lds_k = reinterpret_cast<uint16_t*>(lds_knew);
                    flush_append<DT>(a, pend, lds_k, g, lane);  // an earlier sequence's token, if any
                    const NewToken ntok = new_token<DT>(a, raw, n, lane, lds_k);
                    patch_tile<DT>(t[0], ntok, lds_k, lane);
                    pend = PendingAppend{__builtin_amdgcn_readlane(blk_lane, c0), ntok.slot, t[0].va,
                                         t[0].vb, ntok.ks, ntok.vs};
                }
            }
            const int valid = t_end - (tb + c0) * kBlock;
            if (valid < kBlock) zero_tail(t[0], valid);
            chunk_step<DT, 1, true>(a, t, tb + c0, t_end, qv, lane, lds, m_run, l_lane, acc0, acc1);
        }
    }
    // each token's weight was added by the four lanes of its quad: count one lane per quad
    const float l_sum = wave_sum((lane & 3) == 0 ? l_lane : 0.0f);

    if (lo == 0 && has_last) {
        const float inv = a.v_scale / l_sum;
        a.out[orow + lane] = __builtin_bit_cast(uint16_t, (_Float16)(acc0 * inv));
        a.out[orow + 64 + lane] = __builtin_bit_cast(uint16_t, (_Float16)(acc1 * inv));
    } else {
        const int64_t prow = h * rmul + radd;
        a.part_o[prow * kDim + lane] = acc0;
        a.part_o[prow * kDim + 64 + lane] = acc1;
        if (lane == 0) {
            a.part_m[prow] = m_run;
            a.part_l[prow] = l_sum;
        }
    }
}

// BAL: grid (query head, wave of the balanced split).  Otherwise grid (query head, partition,
// sequence) with fixed partitions of PS tokens.  The balanced split runs about two waves per SIMD,
// so its register budget is that of two waves; fixed partitions can have many more waves than fit
// and are held to the occupancy the plain loop reaches (5; 4 with the append).  The head
// is the fastest grid dimension: workgroups are handed to the eight XCDs round-robin by linear id,
// so consecutive ids should carry equal work -- all heads of one (partition or share, sequence) do.
template <int DT, int TW, bool APPEND, bool BAL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(BAL ? 2 : (APPEND ? 4 : 5), 8))) void attn_partition_valu(
    KernelParams a) {
    __shared__ uint32_t lds[TW * 16];
    __shared__ u32x4 lds_knew[APPEND ? 8 : 1];
    const int lane = threadIdx.x;
    const int h = blockIdx.x;
    const int g = h / (a.Hq / a.Hkv);
    PendingAppend pend{-1, 0, u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}, 0.0f, 0.0f};
    if constexpr (BAL) {
        const int w = blockIdx.y;
        for_each_segment(a, w, h == 0 && w == 0, lane, [&](int b, int n, int nt, int lo, int hi) {
            mha_segment<DT, TW, APPEND>(a, b, h, g, n, nt, lo, hi, a.S, w + b, lane, lds, lds_knew, pend);
        });
        if constexpr (APPEND) flush_append<DT>(a, pend, reinterpret_cast<const uint16_t*>(lds_knew), g, lane);
    } else {
        const int p = blockIdx.y;
        const int b = blockIdx.z;
        const int n = a.ctx[b];
        if (n <= 0) {
            if (p == 0) {
                const size_t orow = ((size_t)b * a.Hq + h) * kDim;
                a.out[orow + lane] = 0;
                a.out[orow + 64 + lane] = 0;
            }
            return;
        }
        const int nt = tiles_of(n);
        const int lo = p * (a.PS / kBlock);
        if (lo >= nt) return;
        const int hi = min(nt, lo + a.PS / kBlock);
        mha_segment<DT, TW, APPEND>(a, b, h, g, n, nt, lo, hi, a.P, (int64_t)b * a.Hq * a.P + p, lane,
                                    lds, lds_knew, pend);
        if constexpr (APPEND) flush_append<DT>(a, pend, reinterpret_cast<const uint16_t*>(lds_knew), g, lane);
    }
}

// Tiles per chunk (loads in flight per wave).
#ifndef KVQ_MHA_TILES
#define KVQ_MHA_TILES 4
#endif

template <int DT, bool BAL>
static void launch_mha(const KernelParams& kp, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
    const dim3 grid = BAL ? dim3((unsigned)kp.Hq, (unsigned)kp.NW)
                          : dim3((unsigned)kp.Hq, (unsigned)kp.P, (unsigned)kp.B);
    if (kp.k_new)
        launch_timed(attn_partition_valu<DT, KVQ_MHA_TILES, true, BAL>, grid, kp, stream, t0, t1);
    else
        launch_timed(attn_partition_valu<DT, KVQ_MHA_TILES, false, BAL>, grid, kp, stream, t0, t1);
}

template <int DT>
static void launch_mha(const KernelParams& kp, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
    if (kp.NW > 0)
        launch_mha<DT, true>(kp, stream, t0, t1);
    else
        launch_mha<DT, false>(kp, stream, t0, t1);
}

void launch_partition_mha(const KernelParams& kp, int dtype, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop) {
    switch (dtype) {
        case KVQ_FP8_E4M3: launch_mha<KVQ_FP8_E4M3>(kp, stream, start, stop); break;
        case KVQ_FP8_E5M2: launch_mha<KVQ_FP8_E5M2>(kp, stream, start, stop); break;
        case KVQ_FP8_E4M3FNUZ: launch_mha<KVQ_FP8_E4M3FNUZ>(kp, stream, start, stop); break;
        default: launch_mha<KVQ_INT8>(kp, stream, start, stop); break;
    }
}

}  // namespace kvq
