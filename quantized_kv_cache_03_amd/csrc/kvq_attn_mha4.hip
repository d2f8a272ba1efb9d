// kvq_attn_mha4.hip -- decode attention over the INT4 cache, one query head per KV head (VALU).
//
// The online INT4 cache ("[Feature] TurboMind support W8A8 or FP8 KV Cache" names INT4 beside the
// online INT8 cache): asymmetric 4-bit codes with an fp32 (scale s, zero point zp) pair per
// (token, KV head), two codes per byte, 1 KiB tiles of 16 tokens.  With k^ = s_t c + zp_t the
// logits and the output factor as
//     z_t   = sm_scale * (s_t (q . c_t) + zp_t sum_d q_d)
//     out_d = (sum_t p_t s_t c_td + sum_t p_t zp_t) / sum_t p_t,
// so the codes enter the dot products exactly (as fp16 subnormals, int4x8_to_f16) and the scales
// stay per token.
//
// One wave per (query head, share of the work), the structure of the 8-bit kernel
// (kvq_attn_mha.hip): chunks of TW tiles with every load issued before any use, a running max /
// sum / accumulator per wave.
//   K tile (four 256-byte chunks of 32 dims x 16 tokens): lane l holds the 32 dims of chunk l % 4
//     of token l / 4 -- one 16-byte load per lane reads the whole tile -- and two quad DPP sums
//     finish each logit.
//   V tile (four 256-byte token-quad blocks): lane l holds tokens 4 (l / 16) .. +3 of the eight
//     dims l % 16 + 16 r (16 contiguous bytes; one load per lane again reads the whole tile) and
//     accumulates those dims over its quad's tokens; the four quads' sums are added once per
//     segment.  The weights p_t s_t of a quad reach its lanes as packed fp16 (hi, lo) pairs
//     through LDS.
// K dwords decode to the pairs (i, i + 4) of their eight nibbles (int4x8_to_f16) and the query
// slice is paired the same way; V units decode to the token pairs (0, 2) and (1, 3) of a quad
// (int4_unit_to_f16) and the weights are published in that order.
#include "kvq_attn.h"
#include "kvq_attn4.h"

namespace kvq {

namespace {

// The codes and scales one lane holds for one tile.
//   k  : K codes of token l / 4, dims 32 (l % 4) .. +31
//   v  : V codes of tokens 4 (l / 16) .. +3 of dims l % 16 + 16 r: unit r in bits 16 (r % 2) .. +15
//        of dword r / 2
//   ks : (scale, zero point) of the K row of token l / 4; vs: of its V row
struct Tile4 {
    u32x4 k, v;
    f32x2 ks, vs;
};

__device__ __forceinline__ void load_tile4(const KernelParams& a, Tile4& t, int blk, int g,
                                           uint32_t k_off, uint32_t v_off, int tk) {
    const size_t tile = ((size_t)blk * a.Hkv + g) * kTileBytes4;
    t.k = ldg16(a.kc + tile + k_off);
    t.v = ldg16(a.vc + tile + v_off);
    const size_t so = ((size_t)blk * a.Hkv + g) * kBlock + tk;
    t.ks = ldg_nt(reinterpret_cast<const f32x2*>(a.ks) + so);
    t.vs = ldg_nt(reinterpret_cast<const f32x2*>(a.vs) + so);
}

// q . c over this lane's 32 dims, in units of 2^-24; qv[4 j + i] pairs dims (8 j + i, 8 j + i + 4)
// of the chunk.  The even and odd nibble pairs (2^-24 and 2^-20 units) are summed apart.
__device__ __forceinline__ float dot32_int4(const u32x4& k, const half2_t (&qv)[16]) {
    const uint32_t w[4] = {k.x, k.y, k.z, k.w};
    float se = 0.0f, so = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        half2_t h[4];
        int4x8_to_f16(w[j], h);
        se = dot2(h[0], qv[4 * j + 0], se);
        so = dot2(h[1], qv[4 * j + 1], so);
        se = dot2(h[2], qv[4 * j + 2], se);
        so = dot2(h[3], qv[4 * j + 3], so);
    }
    return se + so * (kInt4Odd / kInt4Even);
}

// Accumulators of one output dim: the even and odd token pairs apart (2^-24 and 2^-20 units).
struct Acc4 {
    float e, o;
};

// acc += sum over the quad's four tokens of w_t c_t for one 16-bit V unit, with the weights as
// fp16 pairs: wq = (hi(t0, t2), hi(t1, t3), lo(t0, t2), lo(t1, t3)).
// (The components are passed as plain words: a bit cast of a vector component such as wq.y reads
// component x with this toolchain.)
template <int SEL>
__device__ __forceinline__ void pv_unit_int4(uint32_t w, const uint32_t (&wq)[4], Acc4& acc) {
    half2_t e, o;
    int4_unit_to_f16<SEL>(w, e, o);
    acc.e = dot2(e, __builtin_bit_cast(half2_t, wq[0]), acc.e);
    acc.e = dot2(e, __builtin_bit_cast(half2_t, wq[2]), acc.e);
    acc.o = dot2(o, __builtin_bit_cast(half2_t, wq[1]), acc.o);
    acc.o = dot2(o, __builtin_bit_cast(half2_t, wq[3]), acc.o);
}

// An accumulator's value in code units.
__device__ __forceinline__ float acc_value(const Acc4& a) {
    return a.e * kInt4Even + a.o * kInt4Odd;
}

// One chunk of TW tiles.  The four lanes of token tk (the K layout) end with identical logits; lane
// 4 tk publishes the token's weight w = p s_v as fp16 hi and lo halves in its quad's 16 bytes of
// LDS, in the order the V units pair the tokens, and adds p zp_v to the lane's zero-point sum.
// MASKED handles a chunk reaching past the segment end (logits there become -inf, weights 0).
template <int TW, bool MASKED>
__device__ __forceinline__ void chunk_step4(const KernelParams& a, const Tile4 (&t)[TW], int tile0,
                                            int t_end, const half2_t (&qv)[16], float qsum, int lane,
                                            uint16_t* lds, float& m_run, float& l_lane, float& z_lane,
                                            Acc4 (&acc)[8]) {
    const int tk = lane >> 2;
    float z[TW];
    float cmax = kNegInf;
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        const float s = sum4(dot32_int4(t[i].k, qv));  // q . c in units of 2^-24
        z[i] = a.qk_scale * (s * (t[i].ks.x * kInt4Even) + t[i].ks.y * qsum);
        if constexpr (MASKED) z[i] = ((tile0 + i) * kBlock + tk < t_end) ? z[i] : kNegInf;
        cmax = fmaxf(cmax, z[i]);
    }
    cmax = max_across_quads(cmax);  // a chunk always holds at least one valid token
    if (cmax > m_run + kRescaleSlackInt4) {  // lazy rescale; one head per wave, so wave-uniform
        const float alpha = __builtin_amdgcn_exp2f(m_run - cmax);
        m_run = cmax;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            acc[r].e *= alpha;
            acc[r].o *= alpha;
        }
        l_lane *= alpha;
        z_lane *= alpha;
    }

    // half index of token tk: quad tk / 4, then (t0, t2, t1, t3) for hi and again for lo
    const int slot = 8 * (tk >> 2) + (((tk & 1) << 1) | ((tk >> 1) & 1));
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        const float pw = __builtin_amdgcn_exp2f(z[i] - m_run);
        l_lane += pw;
        float vs = t[i].vs.x, vz = t[i].vs.y;
        if constexpr (MASKED) {  // slots past the end may hold NaN scales: their weight is exactly 0
            if ((tile0 + i) * kBlock + tk >= t_end) vs = vz = 0.0f;
        }
        const float w = pw * vs;
        z_lane = __builtin_fmaf(pw, vz, z_lane);
        if ((lane & 3) == 0) {
            const _Float16 h = (_Float16)w;
            lds[i * 32 + slot] = __builtin_bit_cast(uint16_t, h);
            lds[i * 32 + 4 + slot] = __builtin_bit_cast(uint16_t, (_Float16)(w - (float)h));
        }
    }
    __builtin_amdgcn_wave_barrier();
    const int quad = lane >> 4;
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        // the halves were stored as 16-bit values: read them back through memcpy, not a vector
        // pointer of another type
        u32x4 wv;
        __builtin_memcpy(&wv, lds + i * 32 + 8 * quad, sizeof(wv));
        const uint32_t wq[4] = {wv.x, wv.y, wv.z, wv.w};
        pv_unit_int4<0>(t[i].v.x, wq, acc[0]);
        pv_unit_int4<1>(t[i].v.x, wq, acc[1]);
        pv_unit_int4<0>(t[i].v.y, wq, acc[2]);
        pv_unit_int4<1>(t[i].v.y, wq, acc[3]);
        pv_unit_int4<0>(t[i].v.z, wq, acc[4]);
        pv_unit_int4<1>(t[i].v.z, wq, acc[5]);
        pv_unit_int4<0>(t[i].v.w, wq, acc[6]);
        pv_unit_int4<1>(t[i].v.w, wq, acc[7]);
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_wave_barrier();
}

// Replace the new token's codes and scales in the registers of its tile: K in the four lanes of
// the token, V in the 16 lanes of its quad.
__device__ __forceinline__ void patch_tile4(Tile4& t, const NewToken4& nt, const uint8_t* lds_k,
                                            const uint8_t* lds_v, int lane) {
    if ((lane >> 2) == nt.slot) {
        t.k = reinterpret_cast<const u32x4*>(lds_k)[lane & 3];
        t.ks = nt.ks;
        t.vs = nt.vs;
    }
    patch_v_quad(t.v, nt.slot, lds_v, lane);
}

// The work of one segment -- tiles [lo, hi) of sequence b (n tokens, nt tiles) -- as in the 8-bit
// kernel: the final output when the segment is the whole sequence, else a partial in row
// h * rmul + radd (the unnormalized output there already includes the zero-point term).
template <int TW, bool APPEND>
__device__ __forceinline__ void mha4_segment(const KernelParams& a, int b, int h, int g, int n, int nt,
                                             int lo, int hi, int64_t rmul, int64_t radd, int lane,
                                             uint16_t* lds, uint8_t* lds_knew, uint8_t* lds_vnew,
                                             u32x4* lds_vrow, PendingAppend4& pend) {
    const int tk = lane >> 2;
    const size_t orow = ((size_t)b * a.Hq + h) * kDim;
    const bool has_last = hi == nt;
    const int t_end = min(n, hi * kBlock);
    const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks;
    const int tile_new = (APPEND && has_last) ? nt - 1 : -1;

    // q slice of chunk c = lane % 4 (dims 32 c .. +31), paired (8 j + i, 8 j + i + 4), and the sum
    // of all 128 q elements
    half2_t qv[16];
    float qsum;
    {
        const u32x4* qp = reinterpret_cast<const u32x4*>(a.q + orow + (lane & 3) * 32);
        const u32x4 q4[4] = {qp[0], qp[1], qp[2], qp[3]};
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w[4] = {q4[j].x, q4[j].y, q4[j].z, q4[j].w};  // dims 8 j .. 8 j + 7
            const half2_t e0 = __builtin_bit_cast(half2_t, w[0]), e1 = __builtin_bit_cast(half2_t, w[1]);
            const half2_t e2 = __builtin_bit_cast(half2_t, w[2]), e3 = __builtin_bit_cast(half2_t, w[3]);
            qv[4 * j + 0] = half2_t{e0.x, e2.x};
            qv[4 * j + 1] = half2_t{e0.y, e2.y};
            qv[4 * j + 2] = half2_t{e1.x, e3.x};
            qv[4 * j + 3] = half2_t{e1.y, e3.y};
            part += ((float)e0.x + (float)e0.y) + ((float)e1.x + (float)e1.y) +
                    ((float)e2.x + (float)e2.y) + ((float)e3.x + (float)e3.y);
        }
        qsum = sum4(part);
    }

    const uint32_t k_off = 256u * ((uint32_t)lane & 3u) + 16u * (uint32_t)tk;
    const uint32_t v_off = 256u * ((uint32_t)lane >> 4) + 16u * ((uint32_t)lane & 15u);

    float m_run = kNegInf;
    float l_lane = 0.0f, z_lane = 0.0f;
    Acc4 acc[8];  // dims lane % 16 + 16 r, over this lane's token quad
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = Acc4{0.0f, 0.0f};

    for (int tb = lo; tb < hi; tb += 64) {
        const int nt_grp = min(64, hi - tb);
        const int blk_lane = (lane < nt_grp) ? bt[tb + lane] : 0;
        int full_tiles = min(nt_grp, (t_end - tb * kBlock) / kBlock);
        if (has_last) full_tiles = min(full_tiles, nt - 1 - tb);
        const int nfull = full_tiles / TW;
        for (int c = 0; c < nfull; ++c) {
            Tile4 t[TW];
#pragma unroll
            for (int i = 0; i < TW; ++i)
                load_tile4(a, t[i], __builtin_amdgcn_readlane(blk_lane, c * TW + i), g, k_off, v_off, tk);
            chunk_step4<TW, false>(a, t, tb + c * TW, t_end, qv, qsum, lane, lds, m_run, l_lane, z_lane,
                                   acc);
        }
        for (int c0 = nfull * TW; c0 < nt_grp; ++c0) {
            Tile4 t[1];
            load_tile4(a, t[0], __builtin_amdgcn_readlane(blk_lane, c0), g, k_off, v_off, tk);
            if constexpr (APPEND) {
                if (tb + c0 == tile_new) {
                    flush_append4(a, pend, lds_knew, lds_vrow, g, lane);  // an earlier sequence's token, if any
                    const NewToken4 ntok = new_token4(a, b, g, n, lane, lds_knew, lds_vnew);
                    patch_tile4(t[0], ntok, lds_knew, lds_vnew, lane);
                    lds_vrow[lane] = t[0].v;
                    pend = PendingAppend4{__builtin_amdgcn_readlane(blk_lane, c0), ntok.slot, ntok.ks, ntok.vs};
                }
            }
            chunk_step4<1, true>(a, t, tb + c0, t_end, qv, qsum, lane, lds, m_run, l_lane, z_lane, acc);
        }
    }
    const float l_sum = wave_sum((lane & 3) == 0 ? l_lane : 0.0f);
    const float z_sum = wave_sum((lane & 3) == 0 ? z_lane : 0.0f);
    // the four quads' sums of each dim (lanes l, l ^ 16, l ^ 32, l ^ 48); lane (dlo, quad) keeps
    // dims dlo + 16 (2 quad) and dlo + 16 (2 quad + 1)
    const int quad = lane >> 4, dlo = lane & 15;
    float o[2];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        float v = acc_value(acc[r]);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if ((r >> 1) == quad) o[r & 1] = v + z_sum;
    }
    const int d0 = dlo + 32 * quad;  // and d0 + 16

    if (lo == 0 && has_last) {
        const float inv = a.v_scale / l_sum;
        a.out[orow + d0] = __builtin_bit_cast(uint16_t, (_Float16)(o[0] * inv));
        a.out[orow + d0 + 16] = __builtin_bit_cast(uint16_t, (_Float16)(o[1] * inv));
    } else {
        const int64_t prow = h * rmul + radd;
        a.part_o[prow * kDim + d0] = o[0];
        a.part_o[prow * kDim + d0 + 16] = o[1];
        if (lane == 0) {
            a.part_m[prow] = m_run;
            a.part_l[prow] = l_sum;
        }
    }
}

// BAL: grid (query head, wave of the balanced split); otherwise (query head, partition, sequence)
// with fixed partitions, as in the 8-bit kernel; three waves per SIMD there keep the eight-tile
// chunks in registers.
template <int TW, bool APPEND, bool BAL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(BAL ? 2 : 3, 8))) void attn_partition_valu4(
    KernelParams a) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[TW * 32];
    __shared__ u32x4 lds_knew[APPEND ? 4 : 1];
    __shared__ uint8_t lds_vnew[APPEND ? 128 : 1];
    __shared__ u32x4 lds_vrow[APPEND ? 64 : 1];  // the pending token's patched V rows, one per lane
    const int lane = threadIdx.x;
    const int h = blockIdx.x;
    const int g = h / (a.Hq / a.Hkv);
    uint8_t* knew = reinterpret_cast<uint8_t*>(lds_knew);
    PendingAppend4 pend{-1, 0, f32x2{0.0f, 0.0f}, f32x2{0.0f, 0.0f}};
    if constexpr (BAL) {
        const int w = blockIdx.y;
        for_each_segment(a, w, h == 0 && w == 0, lane, [&](int b, int n, int nt, int lo, int hi) {
            mha4_segment<TW, APPEND>(a, b, h, g, n, nt, lo, hi, a.S, w + b, lane, lds, knew, lds_vnew, lds_vrow,
                                     pend);
        });
        if constexpr (APPEND) flush_append4(a, pend, knew, lds_vrow, g, lane);
    } else {
        const int p = blockIdx.y;
        const int b = blockIdx.z;
        const int n = a.ctx[b];
        if (n <= 0) {
            if (p == 0) *reinterpret_cast<uint32_t*>(a.out + ((size_t)b * a.Hq + h) * kDim + 2 * lane) = 0u;
            return;
        }
        const int nt = tiles_of(n);
        const int lo = p * (a.PS / kBlock);
        if (lo >= nt) return;
        const int hi = min(nt, lo + a.PS / kBlock);
        mha4_segment<TW, APPEND>(a, b, h, g, n, nt, lo, hi, a.P, (int64_t)b * a.Hq * a.P + p, lane, lds,
                                 knew, lds_vnew, lds_vrow, pend);
        if constexpr (APPEND) flush_append4(a, pend, knew, lds_vrow, g, lane);
    }
}

#ifndef KVQ_MHA4_TILES
#define KVQ_MHA4_TILES 8
#endif

template <bool BAL>
void launch_mha4(const KernelParams& kp, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
    const dim3 grid = BAL ? dim3((unsigned)kp.Hq, (unsigned)kp.NW)
                          : dim3((unsigned)kp.Hq, (unsigned)kp.P, (unsigned)kp.B);
    if (kp.k_new)
        launch_timed(attn_partition_valu4<KVQ_MHA4_TILES, true, BAL>, grid, kp, stream, t0, t1);
    else
        launch_timed(attn_partition_valu4<KVQ_MHA4_TILES, false, BAL>, grid, kp, stream, t0, t1);
}

}  // namespace

void launch_partition_mha4(const KernelParams& kp, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    if (kp.NW > 0)
        launch_mha4<true>(kp, stream, start, stop);
    else
        launch_mha4<false>(kp, stream, start, stop);
}

}  // namespace kvq
