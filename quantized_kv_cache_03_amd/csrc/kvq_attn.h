// kvq_attn.h -- shared pieces of the decode-attention kernels: launch parameters, the balanced
// split of the work, and the quantization of the token a fused decode step appends.
//
// The cache is stored as 8-bit codes and the attention arithmetic runs at higher precision
// ("Accelerating Inference with FP8 KV Cache", opening section): codes are decoded exactly to
// fp16, the dot products take fp16 inputs and sum in fp32 (the matrix instruction aligns each group
// of 8 products to its largest and keeps 24 bits below it), softmax statistics are fp32.
// Scales are factored out of the sums: logits are  sm_scale * kv_scale * (q . dec(k))  and the
// output is  kv_scale * sum_t p_t dec(v_t) / sum_t p_t  (FP8);  INT8 applies the per-token K
// scale to each logit and folds the per-token V scale into the weight p_t * s_t.  Softmax runs in
// base 2 with log2(e) folded into the logit scale.
#pragma once

#include <hip/hip_ext.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr float kNegInf = -__builtin_huge_valf();

// Lazy rescale of the online softmax: a running (reference) max moves only when a logit exceeds it
// by more than this many binades, so the weights exp2(z - m) stay below 2^kRescaleSlack and the
// rescale of the accumulators becomes rare after the first chunks.  Every sum (weights, outputs,
// and the split-K partials with their m) shares the reference, so the result is unchanged up to
// rounding.
constexpr float kRescaleSlack = 8.0f;

// With per-token V scales (INT8, INT4) the P V products take w = p s_v as fp16 hi + lo parts, and
// p may reach 2^slack, so the slack keeps 2^slack times the largest scale a finite fp16 row can
// have inside the fp16 range: INT8 s_v <= 65504 / 127, and 2^6.5 * 515.8 < 46,700; INT4
// s_v <= 131008 / 15, and 2^2.5 * 8733.9 < 49,400.  (Per-tensor formats: w = p <= 2^8.)
constexpr float kRescaleSlackInt8 = 6.5f;
constexpr float kRescaleSlackInt4 = 2.5f;

// Keep the low `nbytes` (0..4) bytes of w.
__device__ __forceinline__ uint32_t keep_bytes(uint32_t w, int nbytes) {
    return nbytes >= 4 ? w : (nbytes <= 0 ? 0u : (w & ((1u << (8 * nbytes)) - 1u)));
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
    float qk_scale;     // sm_scale * log2(e) (* kv_scale * code_unit for FP8)
    float v_scale;      // kv_scale * code_unit for FP8, 1 for INT8
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

// ------------------------------------------------------------------------------------------------
// Partition-kernel launchers, one translation unit each.  dtype is a kvq_dtype.  With start / stop
// events (kernel-timing hook) the kernel is launched through hipExtLaunchKernel, which records the
// events in the kernel's own dispatch: they time the kernel alone, as a profiler's trace does.
void launch_partition_mha(const KernelParams& kp, int dtype, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop);
void launch_partition_gqa(const KernelParams& kp, int dtype, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop);

template <typename K>
inline void launch_timed(K kernel, dim3 grid, const KernelParams& kp, hipStream_t stream,
                         hipEvent_t start, hipEvent_t stop) {
    if (start)
        hipExtLaunchKernelGGL(kernel, grid, dim3(64), 0, stream, start, stop, 0, kp);
    else
        kernel<<<grid, 64, 0, stream>>>(kp);
}

}  // namespace kvq
