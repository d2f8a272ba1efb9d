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
//   grid (query head, partition, sequence); a wave streams its partition in chunks of TW tiles of
//   16 tokens, issuing every K and V load of a chunk before using any, and keeps a running max /
//   sum / accumulator across chunks.
//   K tile (eight 256-byte chunks of 16 dims x 16 tokens): lane l holds 32 dims of token l/4 --
//     chunks l%4 and l%4 + 4, one whole 1 KiB half of the tile per load instruction -- dots them
//     with its slice of q (v_dot2_f32_f16), and two quad DPP sums finish each logit.
//   V tile (dim-major 128 x 16 B): lane l holds the 16 tokens of dims l and 64 + l, so each lane
//     accumulates whole output elements; the 16 weights of a tile reach every lane as packed fp16
//     (hi, lo) pairs through a 64-byte LDS broadcast.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr float kNegInf = -__builtin_huge_valf();

// Keep the low `nbytes` (0..4) bytes of w.
__device__ __forceinline__ uint32_t keep_bytes(uint32_t w, int nbytes) {
    return nbytes >= 4 ? w : (nbytes <= 0 ? 0u : (w & ((1u << (8 * nbytes)) - 1u)));
}

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

struct KernelParams {
    const uint8_t* kc;
    const uint8_t* vc;
    const float* ks;
    const float* vs;
    const uint16_t* q;
    uint16_t* out;
    float* part_o;      // partial rows [R][128]: unnormalized outputs
    float* part_m;      // [R] running max (base-2 logits)
    float* part_l;      // [R] sum of weights
    int32_t* plan;      // balanced split: [B + 2] = tiles before each sequence, total tiles, waves used
    const int32_t* block_tables;
    const int32_t* ctx;
    int32_t max_blocks;
    int32_t B;
    int32_t Hq;
    int32_t Hkv;
    int32_t P;          // fixed partitions: partitions in the grid; partial row (b Hq + h) P + p
    int32_t PS;         // fixed partitions: tokens per partition
    int32_t NW;         // balanced split: waves per head row in the grid (0 for fixed partitions)
    int32_t S;          // balanced split: partial rows per query head (NW + B); row h S + w + b
    float qk_scale;     // sm_scale * log2(e) (* kv_scale for FP8)
    float v_scale;      // kv_scale for FP8, 1 for INT8
    float kv_scale;     // per-tensor scale of the FP8 encoder (fused append)
    const uint16_t* k_new;  // fused append: fp16 [B][Hkv][128] new rows (else NULL)
    const uint16_t* v_new;
};

__device__ __forceinline__ int tiles_of(int n) { return n > 0 ? (n + kBlock - 1) / kBlock : 0; }

// ------------------------------------------------------------------------------------------------
// Balanced split.  Per head row, the tiles of all sequences are laid end to end (T in total) and
// wave w of the row takes tiles [floor(w T / nw), floor((w + 1) T / nw)): every wave streams the
// same amount whatever the mix of context lengths, and a wave's share may hold the end of one
// sequence and the start of the next.  Each piece of one sequence ("segment") yields one partial,
// or the final output when the wave holds the whole sequence.  nw <= NW caps the waves so each
// gets at least kMinTiles tiles.
constexpr int kMinTiles = 8;

__device__ __forceinline__ int balanced_waves(int T, int NW) {
    return T == 0 ? 1 : min(NW, (T + kMinTiles - 1) / kMinTiles);
}
// the wave whose share holds flattened tile c
__device__ __forceinline__ int wave_of_tile(int c, int T, int nw) {
    return (int)(((int64_t)(c + 1) * nw + T - 1) / T) - 1;
}
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d);
        if (lane >= d) v += u;
    }
    return v;
}
__device__ __forceinline__ int readlane_i(int v, int i) { return __builtin_amdgcn_readlane(v, i); }

// Calls seg(b, n, nt, lo, hi) for each segment (tiles [lo, hi) of sequence b, which has n tokens
// in nt tiles) of wave w's share, in sequence order.  The writer wave also stores the plan that
// the merge kernel reads.
template <typename F>
__device__ __forceinline__ void for_each_segment(const KernelParams& a, int w, bool writer, int lane,
                                                 F&& seg) {
    int T = 0;
    for (int base = 0; base < a.B; base += 64) {
        const int idx = base + lane;
        const int nt = tiles_of(idx < a.B ? a.ctx[idx] : 0);
        const int incl = wave_incl_scan(nt, lane);
        if (writer && idx < a.B) a.plan[idx] = T + incl - nt;
        T += readlane_i(incl, 63);
    }
    const int nw = balanced_waves(T, a.NW);
    if (writer && lane == 0) {
        a.plan[a.B] = T;
        a.plan[a.B + 1] = nw;
    }
    if (w >= nw) return;
    const int s1 = (int)((int64_t)(w + 1) * T / nw);
    int cur = (int)((int64_t)w * T / nw);
    int running = 0;  // tiles before the current 64-sequence chunk
    for (int base = 0; base < a.B && cur < s1; base += 64) {
        const int idx = base + lane;
        // only the inclusive prefix stays in a register across the segments
        const int incl = running + wave_incl_scan(tiles_of(idx < a.B ? a.ctx[idx] : 0), lane);
        const int chunk_end = readlane_i(incl, 63);
        while (cur < s1 && cur < chunk_end) {
            // the first sequence of the chunk whose tiles reach past cur (it has tiles)
            const int b = base + (int)__builtin_ctzll(__ballot(incl > cur));
            const int n = a.ctx[b];
            const int ntb = tiles_of(n);
            const int c0 = readlane_i(incl, b - base) - ntb;
            const int hi = min(ntb, s1 - c0);
            seg(b, n, ntb, cur - c0, hi);
            cur = c0 + hi;
        }
        running = chunk_end;
    }
}

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
        const size_t so = ((size_t)blk * a.Hkv + g) * kBlock + tk;
        t.ks = ldg_nt(a.ks + so);
        t.vs = ldg_nt(a.vs + so);
    }
}

__device__ __forceinline__ u32x4 set_byte(u32x4 v, int slot, uint32_t code) {
    const int sh = 8 * (slot & 3);
    const uint32_t m = ~(0xFFu << sh), c = code << sh;
    switch (slot >> 2) {  // wave-uniform
        case 0: v.x = (v.x & m) | c; break;
        case 1: v.y = (v.y & m) | c; break;
        case 2: v.z = (v.z & m) | c; break;
        default: v.w = (v.w & m) | c; break;
    }
    return v;
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

// The appended row's fp16 values: K dims 2l and 2l+1 (as the append kernel holds them) and V dims
// l and 64 + l (as a Tile holds them).  Loaded when the wave starts, quantized at its tile.
struct NewRow {
    uint32_t k2;
    uint32_t v0, v1;
};

__device__ __forceinline__ NewRow load_new_row(const KernelParams& a, int b, int g, int lane) {
    const size_t row = ((size_t)b * a.Hkv + g) * kDim;
    NewRow r;
    r.k2 = reinterpret_cast<const uint32_t*>(a.k_new + row)[lane];
    r.v0 = a.v_new[row + lane];
    r.v1 = a.v_new[row + 64 + lane];
    return r;
}

// The appended token's codes: K in LDS as the token's row of 128 codes (16 bytes per chunk), V in
// the lane layout of a Tile.  The same per-element arithmetic as the append kernel, bit for bit.
struct NewToken {
    int slot;          // position inside the tile
    uint32_t v0, v1;   // V codes of dims lane and 64 + lane
    float ks, vs;      // INT8 scales
};

template <int DT>
__device__ __forceinline__ NewToken new_token(const KernelParams& a, const NewRow& raw, int n,
                                              int lane, uint16_t* lds_k) {
    NewToken nt;
    nt.slot = (n - 1) % kBlock;
    const float k0 = half_bits_to_float(raw.k2 & 0xFFFFu), k1 = half_bits_to_float(raw.k2 >> 16);
    const float vx0 = half_bits_to_float(raw.v0);
    const float vx1 = half_bits_to_float(raw.v1);
    uint32_t kc0, kc1;
    if constexpr (DT == KVQ_INT8) {
        const float ka = wave_max(fmaxf(fabsf(k0), fabsf(k1)));
        const float va = wave_max(fmaxf(fabsf(vx0), fabsf(vx1)));
        nt.ks = ka / 127.0f;
        nt.vs = va / 127.0f;
        kc0 = encode_int8(k0, nt.ks);
        kc1 = encode_int8(k1, nt.ks);
        nt.v0 = encode_int8(vx0, nt.vs);
        nt.v1 = encode_int8(vx1, nt.vs);
    } else {
        const float s = a.kv_scale;
        kc0 = encode_fp8<DT>(k0 / s);
        kc1 = encode_fp8<DT>(k1 / s);
        nt.v0 = encode_fp8<DT>(vx0 / s);
        nt.v1 = encode_fp8<DT>(vx1 / s);
        nt.ks = nt.vs = 0.0f;
    }
    lds_k[lane] = (uint16_t)(kc0 | (kc1 << 8));  // codes of dims 2 lane, 2 lane + 1
    __builtin_amdgcn_wave_barrier();
    return nt;
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

// Store the appended token: its K codes (16 bytes in each of the eight chunks, from LDS, written
// by lanes 0..7) and its V codes.  A V tile row holds one dim's 16 tokens, so the token's V codes
// are one byte in each of 128 rows; instead of 128 scattered byte stores (partial-line writes),
// each lane rewrites its two whole 16-byte rows as loaded with the new code patched in -- the
// other 15 bytes of each row are written back unchanged.  Only valid when this wave is the only
// reader and writer of the tile (the MHA kernel: one wave per (query head = KV head, partition,
// sequence)).
template <int DT>
__device__ __forceinline__ void store_new_token(const KernelParams& a, const NewToken& nt,
                                                const Tile& patched, const uint16_t* lds_k, int blk,
                                                int g, int lane, uint32_t v_off) {
    const size_t tile = ((size_t)blk * a.Hkv + g) * kTileBytes;
    uint8_t* kt = const_cast<uint8_t*>(a.kc) + tile;
    uint8_t* vt = const_cast<uint8_t*>(a.vc) + tile;
    if (lane < 8) {
        const u32x4 kchunk = reinterpret_cast<const u32x4*>(lds_k)[lane];
        __builtin_nontemporal_store(kchunk, reinterpret_cast<u32x4*>(kt + k_byte(nt.slot, kChunk * lane)));
    }
    __builtin_nontemporal_store(patched.va, reinterpret_cast<u32x4*>(vt + v_off));
    __builtin_nontemporal_store(patched.vb, reinterpret_cast<u32x4*>(vt + 1024u + v_off));
    if constexpr (DT == KVQ_INT8) {
        if (lane == 0) {
            const size_t so = ((size_t)blk * a.Hkv + g) * kBlock + nt.slot;
            const_cast<float*>(a.ks)[so] = nt.ks;
            const_cast<float*>(a.vs)[so] = nt.vs;
        }
    }
}

// ------------------------------------------------------------------------------------------------
// MHA partition kernel: one wave per (query head, share of the work).  The work of one segment --
// tiles [lo, hi) of sequence b (n tokens, nt tiles) -- ends with the final output when the segment
// is the whole sequence, else with a partial in row h * rmul + radd.
// APPEND: the decode step's new token (one per sequence, at position context_lens[b] - 1) is
// quantized by the wave whose segment holds the sequence's last tile, patched into its registers
// and stored.  Used only with one query head per KV head (grouped heads take the append kernel
// first).
template <int DT, int TW, bool APPEND>
__device__ __forceinline__ void mha_segment(const KernelParams& a, int b, int h, int g, int n, int nt,
                                            int lo, int hi, int64_t rmul, int64_t radd, int lane,
                                            uint32_t* lds, u32x4* lds_knew) {
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
                    const NewToken ntok = new_token<DT>(a, raw, n, lane, lds_k);
                    patch_tile<DT>(t[0], ntok, lds_k, lane);
                    store_new_token<DT>(a, ntok, t[0], lds_k, __builtin_amdgcn_readlane(blk_lane, c0),
                                        g, lane, v_off);
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
// and are held to the occupancy the plain loop reaches (5, 4 for INT8 with the append).  The head is the fastest grid dimension:
// workgroups are handed to the eight XCDs round-robin by linear id, so consecutive ids should
// carry equal work -- all heads of one (partition or share, sequence) do.
template <int DT, int TW, bool APPEND, bool BAL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(BAL ? 2 : ((DT == KVQ_INT8 && APPEND) ? 4 : 5), 8))) void attn_partition_valu(
    KernelParams a) {
    __shared__ uint32_t lds[TW * 16];
    __shared__ u32x4 lds_knew[APPEND ? 8 : 1];
    const int lane = threadIdx.x;
    const int h = blockIdx.x;
    const int g = h / (a.Hq / a.Hkv);
    if constexpr (BAL) {
        const int w = blockIdx.y;
        for_each_segment(a, w, h == 0 && w == 0, lane, [&](int b, int n, int nt, int lo, int hi) {
            mha_segment<DT, TW, APPEND>(a, b, h, g, n, nt, lo, hi, a.S, w + b, lane, lds, lds_knew);
        });
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
                                    lds, lds_knew);
    }
}

// ------------------------------------------------------------------------------------------------
// Grouped-query kernel: one wave per (KV head, partition, sequence) serves the G <= 16 query heads
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
typedef _Float16 half8_v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ half8_v join8(half2_t a, half2_t b, half2_t c, half2_t d) {
    return half8_v{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

template <int DT>
__device__ __forceinline__ half8_v codes8(uint32_t w0, uint32_t w1) {
    return join8(codes_to_f16<DT, 0>(w0), codes_to_f16<DT, 1>(w0), codes_to_f16<DT, 0>(w1),
                 codes_to_f16<DT, 1>(w1));
}

template <int DT, int TW>
__device__ __forceinline__ void gqa_segment(const KernelParams& a, int b, int g, int n, int nt, int lo,
                                            int hi, int64_t rmul, int64_t radd, int lane) {
    static_assert(TW % 2 == 0, "tiles are paired for the PV products");
    const int col = lane & 15;  // query head within the group (B / C column), or A row
    const int q4 = lane >> 4;   // MFMA k-group / C row group
    const int G = a.Hq / a.Hkv;
    const int h = g * G + col;  // this lane's query head (valid when col < G)
    const int t_end = min(n, hi * kBlock);
    const int tile_begin = lo;
    const int tile_end = hi;
    const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks;

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

    float m_run = kNegInf;  // running max of this lane's head (base-2 logits)
    float l_lane = 0.0f;    // sum of this lane's weights (tokens 4 q4 .. +3 of every tile)
    float4_t acc[8];        // O^T row blocks: dims 16 r + 4 q4 .. +3 of head col
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const uint32_t k_off = 16u * (uint32_t)lane;  // chunk q4 (+4): token col, dims 16 q4 (+64)
    const uint32_t v_off = (uint32_t)col * kBlock + 4u * (uint32_t)q4;  // dim col (+16 r), tokens 4 q4

    for (int tb = tile_begin; tb < tile_end; tb += 64) {
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
                    for (int r = 0; r < 8; ++r)
                        vd[i][r] = ldg4(vt + v_off + (uint32_t)r * 256u);
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
            // logits S^T: lane holds tokens 4 q4 .. +3 of each tile for head col
            float z[TW][4];
            float cmax = kNegInf;
#pragma unroll
            for (int i = 0; i < TW; ++i) {
                float4_t sacc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8<DT>(ka[i].x, ka[i].y), qB[0], sacc, 0, 0, 0);
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8<DT>(ka[i].z, ka[i].w), qB[1], sacc, 0, 0, 0);
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8<DT>(kb[i].x, kb[i].y), qB[2], sacc, 0, 0, 0);
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8<DT>(kb[i].z, kb[i].w), qB[3], sacc, 0, 0, 0);
                const int pos0 = (tb + c0 + i) * kBlock + 4 * q4;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    float f = a.qk_scale;
                    if constexpr (DT == KVQ_INT8) f *= ks4[i][t];
                    z[i][t] = (pos0 + t < t_end) ? sacc[t] * f : kNegInf;
                    cmax = fmaxf(cmax, z[i][t]);
                }
            }
            // max over the head's tokens: the four row groups of the column
            cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
            cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
            const float m_new = fmaxf(m_run, cmax);  // finite: every chunk holds a valid token
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
    float l_sum = l_lane + __shfl_xor(l_lane, 16);
    l_sum += __shfl_xor(l_sum, 32);

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
template <int DT, int TW, bool BAL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(BAL ? 2 : 4, 8))) void attn_partition_mfma(
    KernelParams a) {
    const int lane = threadIdx.x;
    const int g = blockIdx.x;
    if constexpr (BAL) {
        const int w = blockIdx.y;
        for_each_segment(a, w, g == 0 && w == 0, lane, [&](int b, int n, int nt, int lo, int hi) {
            gqa_segment<DT, TW>(a, b, g, n, nt, lo, hi, a.S, w + b, lane);
        });
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
        gqa_segment<DT, TW>(a, b, g, n, nt, lo, hi, a.P, (int64_t)b * a.Hq * a.P + p, lane);
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
template <int DT, bool BAL>
static void launch_partition(const KernelParams& kp, hipStream_t stream) {
    const int hw = kp.Hq == kp.Hkv ? kp.Hq : kp.Hkv;  // waves per column of the grid
    const dim3 grid = BAL ? dim3((unsigned)hw, (unsigned)kp.NW) : dim3((unsigned)hw, (unsigned)kp.P, (unsigned)kp.B);
    if (kp.Hq == kp.Hkv) {
        if (kp.k_new)
            attn_partition_valu<DT, 4, true, BAL><<<grid, 64, 0, stream>>>(kp);
        else
            attn_partition_valu<DT, 4, false, BAL><<<grid, 64, 0, stream>>>(kp);
    } else {
        // grouped query heads: one wave per KV head; the KV head is the fastest grid dimension
        attn_partition_mfma<DT, 2, BAL><<<grid, 64, 0, stream>>>(kp);
    }
}

template <int DT>
static void launch_partition(const KernelParams& kp, hipStream_t stream) {
    if (kp.NW > 0)
        launch_partition<DT, true>(kp, stream);
    else
        launch_partition<DT, false>(kp, stream);
}

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
    const bool fp8 = c.dtype != KVQ_INT8;
    kp.qk_scale = a.sm_scale * kLog2e * (fp8 ? c.kv_scale : 1.0f);
    kp.v_scale = fp8 ? c.kv_scale : 1.0f;
    kp.kv_scale = c.kv_scale;
    kp.k_new = a.k_new;
    kp.v_new = a.v_new;

    if (kp.k_new && kp.Hq != kp.Hkv) {
        // grouped heads: the step's append runs as its own kernel before the attention
        const hipError_t e = launch_append(c, kp.k_new, kp.v_new, nullptr, a.batch, a.block_tables,
                                           a.max_blocks_per_seq, a.context_lens, a.batch, stream);
        if (e != hipSuccess) return e;
        kp.k_new = kp.v_new = nullptr;
    }
    if (main_begin) (void)hipEventRecord(main_begin, stream);
    switch (c.dtype) {
        case KVQ_FP8_E4M3: launch_partition<KVQ_FP8_E4M3>(kp, stream); break;
        case KVQ_FP8_E5M2: launch_partition<KVQ_FP8_E5M2>(kp, stream); break;
        default: launch_partition<KVQ_INT8>(kp, stream); break;
    }
    if (main_end) (void)hipEventRecord(main_end, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (kp.NW > 0 || kp.P > 1) {
        attn_merge<<<dim3((unsigned)a.num_q_heads, (unsigned)a.batch), 64, 0, stream>>>(kp);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace kvq
