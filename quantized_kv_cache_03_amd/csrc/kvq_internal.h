// kvq_internal.h -- host-side launchers shared between the ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// The formats with one per-tensor scale (the FP8 flavours); INT8 and INT4 scale per token.
constexpr bool is_fp8(int dtype) {
    return dtype == KVQ_FP8_E4M3 || dtype == KVQ_FP8_E5M2 || dtype == KVQ_FP8_E4M3FNUZ;
}

// Launch parameters of the decode-attention kernels, resolved by the ABI layer.
struct DecodeArgs {
    const kvq_cache* cache;
    const uint16_t* q;        // fp16 bits [B][Hq][128]
    uint16_t* out;            // fp16 bits [B][Hq][128]
    int32_t num_q_heads;
    float sm_scale;
    const int32_t* block_tables;
    int32_t max_blocks_per_seq;
    const int32_t* context_lens;
    int32_t batch;
    int32_t num_partitions;   // fixed partitions: grid extent over partitions (>= 1)
    int32_t partition_size;   // fixed partitions: tokens per partition (the whole context when
                              // num_partitions == 1)
    int32_t balanced_waves;   // balanced split: waves per head row (NW); 0 for fixed partitions
    int32_t* plan;            // balanced split: int32 [B + 2]
    float* part_o;            // partial rows: fixed [B][Hq][P][128], balanced [Hq][NW + B][128]
    float* part_m;            // one float per partial row
    float* part_l;            // one float per partial row
    const uint16_t* k_new;    // fused decode step: fp16 [B][Hkv][128] rows to append, else NULL
    const uint16_t* v_new;
    bool fp8_math;            // query rows quantized to E4M3, QK^T on the FP8 matrix cores
};

// Launch parameters of the prefill attention, resolved by the ABI layer.
struct PrefillArgs {
    const kvq_cache* cache;
    const uint16_t* q;        // fp16 bits [num_q_rows][Hq][128]
    uint16_t* out;            // fp16 bits [num_q_rows][Hq][128]
    int32_t num_q_heads;
    float sm_scale;
    const int32_t* cu_q_lens; // [B + 1]
    int32_t num_q_rows;
    int32_t max_q_len;
    const int32_t* block_tables;
    int32_t max_blocks_per_seq;
    const int32_t* context_lens;
    int32_t batch;
    bool fp8_math;            // query rows quantized to E4M3, QK^T on the FP8 matrix cores
};

hipError_t launch_append(const kvq_cache& c, const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* cu_new_lens, int32_t num_rows, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch,
                         hipStream_t stream);

hipError_t launch_dequant(const kvq_cache& c, const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t batch, int32_t max_context_len,
                          float* k_out, float* v_out, hipStream_t stream);

// Partition kernel (with the append of the decode step when k_new is set), then, with the balanced
// split or num_partitions > 1, the merge kernel.  The optional events time the partition kernel's
// own dispatch (kernel-timing hook).
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, hipEvent_t main_begin,
                         hipEvent_t main_end);

// Prefill attention kernel; the optional events time its own dispatch (kernel-timing hook).
hipError_t launch_prefill(const PrefillArgs& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop);

// FP8 math: each 128-wide fp16 query row -> E4M3 codes and its fp32 scale (the quantization the
// FP8-math attention kernels apply to their query rows).
hipError_t launch_quantize_q_fp8(const uint16_t* q, int32_t num_rows, uint8_t* codes, float* scales,
                                 hipStream_t stream);

}  // namespace kvq
