/*
 * kvq.h -- C ABI of the 8-bit paged KV cache for AMD MI355X (gfx950).
 *
 * One decode step of one attention layer over a paged KV cache whose K and V are stored as 8-bit
 * codes and dequantized on read, the arithmetic running in fp16/fp32:
 *
 *   "Accelerating Inference with FP8 KV Cache" (text-generation-inference docs):
 *     opening section    -- K/V are stored as FP8, computation runs at FP16;
 *     "FP8 Formats: E4M3 and E5M2" -- the OCP E4M3 (1/4/3 bits) and E5M2 (1/5/2 bits) layouts and a
 *                           per-tensor FP32 scaling factor;
 *     "FP8 E4M3 KV Cache" -- the scale defaults to 1.0; the names fp8 / fp8_e5m2.
 *     "Current Hardware Support", "Checkpoint structure for KV scales" -- AMD's FP8E4M3FNUZ flavour
 *                           (torch dtype float8_e4m3fnuz), read as the 1/4/3 layout with bias 8,
 *                           no infinities, no negative zero and one NaN code, 0x80.
 *   "[Feature] TurboMind support W8A8 or FP8 KV Cache" (lmdeploy issue thread):
 *     the online INT8 KV cache, read here as symmetric INT8 with one fp32 scale per (token, head);
 *     INT4, named beside it, read as asymmetric 4-bit codes with an fp32 (scale, zero point) pair
 *     per (token, head).
 *     FP8 attention (FP8 in the arithmetic, not only in storage), to which the thread points, with
 *     E4M3 as its format: the *_fp8math calls, read as query rows quantized to E4M3 with one
 *     dynamic fp32 scale per row and QK^T on the FP8 matrix cores.
 *   "[QST] Scale factors and benchmarks" (QQQ issue thread):
 *     the cache lives in a paged-attention serving stack: fixed-size blocks of tokens reached
 *     through a per-sequence block table.
 *
 * Numerics (bit-exact contract of the cache bytes):
 *   FP8 code   = enc(fl32(fl32(x) / kv_scale)), x the fp16 input: one correctly rounded fp32
 *                division, then round to nearest with ties to the even code, finite overflow and
 *                +-inf saturating to +-max (E4M3 448, E5M2 57344, E4M3FNUZ 240), NaN -> sign|0x7F
 *                (E4M3FNUZ: 0x80), signed zero (E4M3FNUZ: unsigned zero) and subnormals kept.
 *                Decode: value = dec(code) * kv_scale.  The attention calls take a cache without
 *                E4M3FNUZ NaN codes (only a NaN input writes one); kvq_dequant decodes them as NaN.
 *   INT8 codes = per (token, KV head) row of 128 values: s = fl32(amax / 127),
 *                q = clamp(rne(fl32(x / s)), -127, 127); an all-zero row gives s = 0, q = 0.
 *                Decode: value = q * s.  Inputs are assumed finite.
 *   INT4 codes = per (token, KV head) row: zp = min x, s = fl32(fl32(max x - zp) / 15),
 *                q = clamp(rne(fl32(fl32(x - zp) / s)), 0, 15); a constant row gives s = 0, q = 0.
 *                Decode: value = q * s + zp.  Inputs are assumed finite.
 *
 * Memory layout (all device memory, caller-owned, dense, no padding):
 *   K codes  uint8 [num_blocks][num_kv_heads][8][16 tokens][16 dims] (2 KiB tile of eight 256-byte
 *            chunks: dim d of token t is byte (d / 16) * 256 + t * 16 + d % 16 of the tile)
 *   V codes  uint8 [num_blocks][num_kv_heads][128 dims][16 tokens]   (dim-major tile, 2 KiB)
 *   INT8 scales  float [num_blocks][num_kv_heads][2][16 tokens]: one 128-byte row per tile, its
 *                16 K scales and then its 16 V scales, so that a tile's scales are one whole
 *                line; k_scale points at the array and v_scale must be k_scale + 16
 *   INT4 (two codes per byte, the even element in the low nibble; tiles of 1 KiB):
 *     K codes  uint8 [num_blocks][num_kv_heads][4][16 tokens][16 bytes]: dim d of token t is in
 *              byte (d / 32) * 256 + t * 16 + (d % 32) / 2 of the tile, nibble d % 2
 *     V codes  uint8 [num_blocks][num_kv_heads][4][16][8][2 bytes]: token t of dim d is in byte
 *              (t / 4) * 256 + (d % 16) * 16 + (d / 16) * 2 + (t % 4) / 2, nibble t % 2 (a 16-bit
 *              unit holds four consecutive tokens of one dim)
 *     scales   float [num_blocks][num_kv_heads][16 tokens][2] = (scale, zero point), for K and V
 *   block_tables int32 [batch][max_blocks_per_seq]: logical block i of sequence b is physical block
 *                block_tables[b][i]; entries past a sequence's last block are never read.
 *   context_lens int32 [batch]: the number of tokens of each sequence after the append.
 *   q, out       fp16 [batch][num_q_heads][128];  query head h reads KV head h / (Hq / Hkv).
 *
 * Conventions:
 *   - head_dim must be 128 and block_size 16; Hq must be a multiple of Hkv with Hq / Hkv <= 16.
 *   - Every call validates its host-side arguments, enqueues its kernels on `stream` (a
 *     hipStream_t; NULL is the legacy default stream) and returns without synchronizing.
 *   - The library allocates no device memory; the split-K workspace is passed in by the caller.
 *   - Return value: KVQ_OK (0) or a negative KVQ_ERR_*; kvq_last_error() then gives a message
 *     (per calling thread).  No call aborts or throws.
 *   - Device-side contract, not checked (violations are undefined behaviour): block ids are in
 *     [0, num_blocks); 0 <= context_lens[b] <= min(max_context_len, 16 * max_blocks_per_seq);
 *     every pointer addresses memory of the documented size on the current device.
 *   - Functions hold no state across calls (apart from the calling thread's optional kernel-timing
 *     session) and may be called concurrently on different streams for disjoint outputs.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVQ_FP8_E4M3 = 1, /* OCP E4M3 with per-tensor fp32 kv_scale ("fp8", "fp8_e4m3")        */
    KVQ_FP8_E5M2 = 2, /* OCP E5M2 with per-tensor fp32 kv_scale, usually 1.0 ("fp8_e5m2")  */
    KVQ_INT8 = 3,     /* symmetric INT8, one fp32 scale per (token, KV head) ("int8")      */
    KVQ_FP8_E4M3FNUZ = 4, /* AMD's E4M3FNUZ with per-tensor fp32 kv_scale ("fp8_e4m3fnuz") */
    KVQ_INT4 = 5      /* asymmetric 4-bit codes, fp32 (scale, zero point) per (token, KV head)
                         ("int4"); two codes per byte                                        */
} kvq_dtype;

enum {
    KVQ_OK = 0,
    KVQ_ERR_ARG = -1,       /* NULL pointer, negative size, non-finite scale, ...          */
    KVQ_ERR_DTYPE = -2,     /* unknown kvq_dtype                                            */
    KVQ_ERR_SHAPE = -3,     /* unsupported head_dim / block_size / head grouping            */
    KVQ_ERR_WORKSPACE = -4, /* split-K workspace missing or too small                       */
    KVQ_ERR_HIP = -5        /* the HIP runtime reported an error at launch                  */
};

#define KVQ_HEAD_DIM 128
#define KVQ_BLOCK_SIZE 16
#define KVQ_MAX_GROUP 16
/* Largest max_context_len the attention calls accept (2^30 tokens: 256 GiB of codes per KV head,
 * beyond one GPU's memory); token positions then stay within 32-bit integers everywhere. */
#define KVQ_MAX_CONTEXT_LEN (1 << 30)

/* Cache descriptor: a host struct read at call time; the pointers are device pointers. */
typedef struct {
    kvq_dtype dtype;
    int32_t num_blocks;
    int32_t block_size;   /* must be 16 */
    int32_t num_kv_heads;
    int32_t head_dim;     /* must be 128 */
    uint8_t *k_cache;     /* K codes, layout above */
    uint8_t *v_cache;     /* V codes, layout above */
    float *k_scale;       /* INT8: the [num_blocks][Hkv][2][16] scale rows; INT4: [num_blocks][Hkv][16][2];
                             NULL for FP8 */
    float *v_scale;       /* INT8: k_scale + 16 (else KVQ_ERR_SHAPE); INT4: [num_blocks][Hkv][16][2];
                             NULL for FP8 */
    float kv_scale;       /* FP8 only: per-tensor scale shared by K and V, finite and > 0;
                             1.0 is the default ("FP8 E4M3 KV Cache" section) */
} kvq_cache;

/* Quantize new K/V rows and write them into their paged slots ("FP8 Formats: E4M3 and E5M2";
 * the online INT8 cache of the lmdeploy thread).
 *   k_new, v_new : fp16 [num_new_rows][Hkv][128], device.
 *   cu_new_lens  : int32 [batch + 1] device row offsets (sequence b owns rows cu[b] .. cu[b+1]-1),
 *                  or NULL for exactly one new row per sequence (then num_new_rows == batch).
 *   The j-th of sequence b's n_b new rows goes to position p = context_lens[b] - n_b + j, i.e.
 *   block block_tables[b][p / 16], slot p % 16.  No other byte of the cache is written.
 *   With cu_new_lens, num_new_rows must equal cu[batch] (the caller's host-side copy). */
int kvq_append(const kvq_cache *cache, const void *k_new, const void *v_new,
               const int32_t *cu_new_lens, int32_t num_new_rows, const int32_t *block_tables,
               int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t batch,
               void *stream);

/* partition_size value selecting the balanced split (see kvq_paged_decode_attn). */
#define KVQ_PARTITION_BALANCED (-1)

/* Bytes of split-K workspace kvq_paged_decode_attn needs for these sizes and partition_size
 * (0 when none is needed, and 0 for every combination of these arguments that the attention calls
 * reject: the two share one validator).  Takes num_kv_heads, not head_dim (fixed at 128): the
 * balanced split plans its waves per head row, whose count depends on the grouping Hq / Hkv.
 * Does not change kvq_last_error(). */
size_t kvq_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t max_context_len, int32_t partition_size);

/* Decode-step attention over the paged 8-bit cache (the opening section of "Accelerating
 * Inference with FP8 KV Cache": stored as FP8, computed at higher precision):
 *   out[b][h] = sum_t softmax_t(sm_scale * q[b][h] . k^[t]) v^[t] over t < context_lens[b],
 *   with k^, v^ the dequantized rows of KV head h / (Hq / Hkv).  context_lens[b] == 0 gives zeros.
 *   sm_scale       : finite; 1/sqrt(128) is the usual value.
 *   max_context_len: host-side upper bound of context_lens (sizes the grid without a device read),
 *                    at most KVQ_MAX_CONTEXT_LEN.
 *   partition_size : how the work is split (flash-decoding split-K: each piece writes fp32 (max,
 *                    sum, unnormalized output) partials into `workspace`, and a second kernel merges
 *                    them with the log-sum-exp rule):
 *                      0                      one pass per sequence, no workspace;
 *                      a positive multiple of 16: fixed partitions of that many tokens;
 *                      KVQ_PARTITION_BALANCED the tiles of all sequences, laid end to end, are cut
 *                                             into equal shares, about 2048 waves in all (with one
 *                                             query head per KV head: 4096 for an INT8 cache, 3072
 *                                             for INT4),
 *                                             whatever the mix of context lengths (a share may hold
 *                                             the end of one sequence and the start of the next).
 *                    For given arguments the result is bitwise deterministic.
 *   workspace      : device memory of at least kvq_decode_workspace_size(...) bytes (may be NULL
 *                    when that size is 0); its contents need no initialization. */
int kvq_paged_decode_attn(const kvq_cache *cache, const void *q, void *out, int32_t num_q_heads,
                          float sm_scale, const int32_t *block_tables, int32_t max_blocks_per_seq,
                          const int32_t *context_lens, int32_t batch, int32_t max_context_len,
                          int32_t partition_size, void *workspace, size_t workspace_bytes,
                          void *stream);

/* One whole decode step: kvq_append of one new row per sequence (cu_new_lens == NULL) followed by
 * kvq_paged_decode_attn, fused so that the append costs no launch of its own.  The cache bytes
 * written and the output are bitwise identical to those two calls made in sequence with the same
 * arguments.  k_new, v_new: fp16 [batch][Hkv][128], the token at position context_lens[b] - 1 of
 * each sequence (context_lens are post-append lengths and must be >= 1; a sequence with
 * context_lens[b] == 0 appends nothing and gets zeros).  Other arguments as for
 * kvq_paged_decode_attn. */
int kvq_decode_step(const kvq_cache *cache, const void *k_new, const void *v_new, const void *q,
                    void *out, int32_t num_q_heads, float sm_scale, const int32_t *block_tables,
                    int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t batch,
                    int32_t max_context_len, int32_t partition_size, void *workspace,
                    size_t workspace_bytes, void *stream);

/* Size of the device scratch array kvq_decode_step_noalloc uses as its split-K workspace (64 MiB
 * per GPU the library runs on, held until the process ends). */
#define KVQ_NOALLOC_SCRATCH_BYTES (64u << 20)

/* kvq_decode_step for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same arguments without workspace /
 * workspace_bytes, the same kernels, and bitwise the same cache bytes and output as kvq_decode_step
 * with a workspace.  The split-K workspace is a file-scope device array of
 * KVQ_NOALLOC_SCRATCH_BYTES; sizes whose workspace (kvq_decode_workspace_size) exceeds it return
 * KVQ_ERR_WORKSPACE before any device work.  The array's device address is looked up once per
 * device, on that device's first call (the call then takes a lock; later calls only read the
 * stored address).  The call allocates nothing.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (on different streams, or from different threads) race
 * and may return wrong results; calls ordered on one stream are safe.  The array needs no
 * clearing: each call writes every partial it reads. */
int kvq_decode_step_noalloc(const kvq_cache *cache, const void *k_new, const void *v_new, const void *q,
                            void *out, int32_t num_q_heads, float sm_scale, const int32_t *block_tables,
                            int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t batch,
                            int32_t max_context_len, int32_t partition_size, void *stream);

/* Prefill / chunked-prefill attention over the paged 8-bit cache (the same formats and arithmetic
 * as kvq_paged_decode_attn: stored as FP8 or INT8, computed at higher precision):
 *   sequence b brings n_b = cu_q_lens[b+1] - cu_q_lens[b] query rows, the last n_b of its
 *   context_lens[b] tokens, whose K/V rows are already in the cache (kvq_append with the same
 *   cu_new_lens).  Row j sits at position p = context_lens[b] - n_b + j and attends to the cache
 *   tokens at positions 0 .. p (causal):
 *     out[cu_q_lens[b] + j][h] = sum_{t <= p} softmax_t(sm_scale * q . k^[t]) v^[t].
 *   Decode is the case n_b = 1; a whole prompt is n_b = context_lens[b].
 *   q, out      : fp16 [num_q_rows][num_q_heads][128], device; num_q_rows = cu_q_lens[batch].
 *   cu_q_lens   : int32 [batch + 1] device row offsets.
 *   max_q_len   : host-side upper bound of n_b (sizes the grid), at most max_context_len
 *                 (itself at most KVQ_MAX_CONTEXT_LEN).
 *   Device-side contract: n_b <= context_lens[b] (rows of a sequence breaking it get zeros),
 *   n_b <= max_q_len.  No workspace; the result is bitwise deterministic. */
int kvq_paged_prefill_attn(const kvq_cache *cache, const void *q, void *out, int32_t num_q_heads,
                           float sm_scale, const int32_t *cu_q_lens, int32_t num_q_rows,
                           int32_t max_q_len, const int32_t *block_tables, int32_t max_blocks_per_seq,
                           const int32_t *context_lens, int32_t batch, int32_t max_context_len,
                           void *stream);

/* FP8 math ("[Feature] TurboMind support W8A8 or FP8 KV Cache": the FP8 attention it points to,
 * whose format is E4M3).  Each 128-wide fp16 query row q is quantized to OCP E4M3 with its own
 * scale,
 *   s_q = fl32(max_d |q_d| / 448)  (1 for an all-zero row),   c_d = enc_E4M3(fl32(q_d / s_q))
 * (the cache encoder: nearest, ties to even, saturating), and the attention is that of the row
 * dec(c) * s_q: QK^T multiplies the E4M3 codes with the cache's K codes as stored, on the FP8
 * matrix cores, and everything after the logits is as in the fp16 calls.  The matrix instruction
 * does not sum exactly in fp32: within each group of 8 consecutive products it aligns the products
 * to the group's largest exponent and keeps 13 bits below it, so a logit may be off by up to about
 * 2^-13 of each group's largest product (more than fp32 rounding where one product dominates many
 * small ones).  The result differs from the fp16-query attention by the query's quantization.
 *   kvq_paged_decode_attn_fp8math, kvq_decode_step_fp8math, kvq_paged_prefill_attn_fp8math take the
 *   arguments of kvq_paged_decode_attn, kvq_decode_step and kvq_paged_prefill_attn (the same
 *   workspace sizes) and need an fp8_e4m3 or fp8_e5m2 cache (else KVQ_ERR_DTYPE); every grouping
 *   Hq / Hkv <= 16 runs on the grouped-head matrix-core kernel.  Inputs are assumed finite. */
int kvq_paged_decode_attn_fp8math(const kvq_cache *cache, const void *q, void *out,
                                  int32_t num_q_heads, float sm_scale, const int32_t *block_tables,
                                  int32_t max_blocks_per_seq, const int32_t *context_lens,
                                  int32_t batch, int32_t max_context_len, int32_t partition_size,
                                  void *workspace, size_t workspace_bytes, void *stream);
int kvq_decode_step_fp8math(const kvq_cache *cache, const void *k_new, const void *v_new,
                            const void *q, void *out, int32_t num_q_heads, float sm_scale,
                            const int32_t *block_tables, int32_t max_blocks_per_seq,
                            const int32_t *context_lens, int32_t batch, int32_t max_context_len,
                            int32_t partition_size, void *workspace, size_t workspace_bytes,
                            void *stream);
int kvq_paged_prefill_attn_fp8math(const kvq_cache *cache, const void *q, void *out,
                                   int32_t num_q_heads, float sm_scale, const int32_t *cu_q_lens,
                                   int32_t num_q_rows, int32_t max_q_len, const int32_t *block_tables,
                                   int32_t max_blocks_per_seq, const int32_t *context_lens,
                                   int32_t batch, int32_t max_context_len, void *stream);

/* The query quantization of the FP8-math calls on its own: q fp16 [num_rows][128] (device) ->
 * codes uint8 [num_rows][128] (E4M3) and scales fp32 [num_rows] (device, caller-owned), bit-exact
 * as defined above.  For inspection and tests. */
int kvq_quantize_q_fp8(const void *q, int32_t num_rows, void *codes, float *scales, void *stream);

/* Dequantize the cache into dense fp32 [batch][Hkv][max_context_len][128] arrays for K and V:
 * each element is fl32(dec(code) * kv_scale) (FP8), fl32(q * s) (INT8) or fl32(q * s + zp)
 * (INT4), one rounding.  Slots t >= context_lens[b] are left untouched; max_context_len is at
 * most KVQ_MAX_CONTEXT_LEN.  For inspection and tests; not on the decode path. */
int kvq_dequant(const kvq_cache *cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                const int32_t *context_lens, int32_t batch, int32_t max_context_len, float *k_out,
                float *v_out, void *stream);

/* "fp8" | "fp8_e4m3" -> KVQ_FP8_E4M3, "fp8_e5m2" -> KVQ_FP8_E5M2, "int8" -> KVQ_INT8,
 * "int4" -> KVQ_INT4, "fp8_e4m3fnuz" -> KVQ_FP8_E4M3FNUZ (the --kv-cache-dtype names and the
 * float8_e4m3fnuz kv_cache_torch_dtype of "Accelerating Inference with FP8 KV Cache").
 * Returns KVQ_OK or KVQ_ERR_DTYPE (out untouched). */
int kvq_dtype_from_string(const char *s, kvq_dtype *out);

/* Static text of a status code. */
const char *kvq_status_string(int status);

/* Message of the last failed call on this thread ("" if none). */
const char *kvq_last_error(void);

/* Kernel-timing hook for benchmarks: after kvq_timing_begin(capacity), each kvq_paged_decode_attn,
 * kvq_decode_step or kvq_paged_prefill_attn call (or its FP8-math variant) times its main
 * (attention) kernel with a HIP event pair recorded in that kernel's own dispatch
 * (hipExtLaunchKernel), on the call's stream, for up to `capacity` calls.  kvq_timing_end() waits
 * for the events, returns the summed milliseconds and the number of timed launches, and releases
 * the events.  Events are created in kvq_timing_begin, outside any timed region.  A session belongs
 * to the thread that began it: only that thread's calls are timed, and threads may hold sessions
 * of their own at the same time (a thread that exits with a session open leaks its events).
 * Returns KVQ_OK or KVQ_ERR_ARG / KVQ_ERR_HIP. */
int kvq_timing_begin(int32_t capacity);
int kvq_timing_end(double *main_ms_total, int32_t *main_count);

/* Library version, "major.minor.patch". */
const char *kvq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
