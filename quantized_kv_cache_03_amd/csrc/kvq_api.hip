// kvq_api.hip -- the extern "C" surface declared in include/kvq.h: argument validation, split-K
// planning, launches on the caller's stream, error reporting and the kernel-timing hook.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_err[0] = '\0';
    return KVQ_OK;
}

int hip_fail(hipError_t e, const char* where) {
    return fail(KVQ_ERR_HIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

int check_cache(const kvq_cache* c) {
    if (!c) return fail(KVQ_ERR_ARG, "cache descriptor is NULL");
    if (c->dtype != KVQ_FP8_E4M3 && c->dtype != KVQ_FP8_E5M2 && c->dtype != KVQ_INT8 &&
        c->dtype != KVQ_FP8_E4M3FNUZ && c->dtype != KVQ_INT4)
        return fail(KVQ_ERR_DTYPE, "unknown kv cache dtype %d", (int)c->dtype);
    if (c->head_dim != KVQ_HEAD_DIM)
        return fail(KVQ_ERR_SHAPE, "head_dim %d is not supported (must be %d)", c->head_dim, KVQ_HEAD_DIM);
    if (c->block_size != KVQ_BLOCK_SIZE)
        return fail(KVQ_ERR_SHAPE, "block_size %d is not supported (must be %d)", c->block_size,
                    KVQ_BLOCK_SIZE);
    if (c->num_kv_heads <= 0) return fail(KVQ_ERR_SHAPE, "num_kv_heads %d must be positive", c->num_kv_heads);
    if (c->num_blocks <= 0) return fail(KVQ_ERR_SHAPE, "num_blocks %d must be positive", c->num_blocks);
    if (!c->k_cache || !c->v_cache) return fail(KVQ_ERR_ARG, "k_cache / v_cache pointer is NULL");
    if (c->dtype == KVQ_INT8 || c->dtype == KVQ_INT4) {
        if (!c->k_scale || !c->v_scale)
            return fail(KVQ_ERR_ARG, "%s cache needs k_scale and v_scale arrays",
                        c->dtype == KVQ_INT8 ? "INT8" : "INT4");
        if (c->dtype == KVQ_INT8 && c->v_scale != c->k_scale + KVQ_BLOCK_SIZE)
            return fail(KVQ_ERR_SHAPE, "an INT8 cache keeps each tile's K and V scales in one row "
                        "[num_blocks][Hkv][2][16]: v_scale must be k_scale + 16");
    } else {
        if (!(isfinite(c->kv_scale) && c->kv_scale > 0.0f))
            return fail(KVQ_ERR_ARG, "kv_scale %g must be finite and positive", (double)c->kv_scale);
    }
    return KVQ_OK;
}

int check_common(const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                 int32_t batch) {
    if (batch < 0) return fail(KVQ_ERR_ARG, "batch %d is negative", batch);
    if (batch == 0) return KVQ_OK;
    if (!block_tables || !context_lens) return fail(KVQ_ERR_ARG, "block_tables / context_lens is NULL");
    if (max_blocks_per_seq <= 0)
        return fail(KVQ_ERR_ARG, "max_blocks_per_seq %d must be positive", max_blocks_per_seq);
    return KVQ_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The checks of the decode calls that depend only on the sizes kvq_decode_workspace_size also
// takes (one validator, so that the size query is 0 exactly for sizes the calls reject).
int check_decode_sizes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_context_len,
                       int32_t partition_size) {
    if (batch < 0) return fail(KVQ_ERR_ARG, "batch %d is negative", batch);
    if (num_kv_heads <= 0) return fail(KVQ_ERR_SHAPE, "num_kv_heads %d must be positive", num_kv_heads);
    if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
        return fail(KVQ_ERR_SHAPE, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                    num_q_heads, num_kv_heads);
    if (num_q_heads / num_kv_heads > KVQ_MAX_GROUP)
        return fail(KVQ_ERR_SHAPE, "query heads per KV head (%d) above %d", num_q_heads / num_kv_heads,
                    KVQ_MAX_GROUP);
    if (max_context_len < 0 || max_context_len > KVQ_MAX_CONTEXT_LEN)
        return fail(KVQ_ERR_ARG, "max_context_len %d is outside [0, %d]", max_context_len, KVQ_MAX_CONTEXT_LEN);
    if (partition_size != KVQ_PARTITION_BALANCED &&
        (partition_size < 0 || partition_size % KVQ_BLOCK_SIZE != 0))
        return fail(KVQ_ERR_ARG,
                    "partition_size %d must be KVQ_PARTITION_BALANCED (-1), 0 or a positive multiple of %d",
                    partition_size, KVQ_BLOCK_SIZE);
    if (batch > 65535 || num_q_heads > 65535)
        return fail(KVQ_ERR_SHAPE, "batch and num_q_heads must be at most 65535");
    if (partition_size > 0) {
        const int64_t P = ((int64_t)max_context_len + partition_size - 1) / partition_size;
        if (P > 65535)
            return fail(KVQ_ERR_SHAPE, "%lld partitions of %d tokens exceed the grid limit 65535",
                        (long long)P, partition_size);
    }
    return KVQ_OK;
}

// FP8 math multiplies the E4M3 query codes with the cache's own codes on the OCP FP8 matrix cores.
int check_fp8_math(const kvq_cache* c) {
    if (c->dtype != KVQ_FP8_E4M3 && c->dtype != KVQ_FP8_E5M2)
        return fail(KVQ_ERR_DTYPE, "FP8 math needs an fp8_e4m3 or fp8_e5m2 cache (dtype %d given)",
                    (int)c->dtype);
    return KVQ_OK;
}

// Work split of the decode attention.  Fixed partitions: P partitions of PS tokens (P == 1: one
// pass, no workspace).  Balanced split: NW waves per head row (query heads for MHA, KV heads for
// grouped heads), about kBalancedWaves waves in all -- two per SIMD of the 1024 on the chip, enough
// to keep HBM busy while each wave streams a long, equal share -- four per SIMD for the one-head
// INT8 kernel and three for the one-head INT4 kernel, which hold that many waves per SIMD and
// measured faster with them.  A wave gets at least
// kMinTiles tiles (the device caps the waves it uses by the same rule on the actual tile count).
// The workspace is sized for the largest target of the shape (any cache dtype fits it).
#ifndef KVQ_BALANCED_WAVES
#define KVQ_BALANCED_WAVES 2048
#endif
constexpr int64_t kBalancedWaves = KVQ_BALANCED_WAVES;
constexpr int64_t kBalancedWavesInt8Mha = 2 * kBalancedWaves;
constexpr int64_t kBalancedWavesInt4Mha = 3 * kBalancedWaves / 2;
constexpr int64_t kMinTiles = 8;

// Waves in all for the balanced split of a cache dtype (dtype < 0: the largest over the dtypes).
int64_t balanced_wave_target(int dtype, int32_t Hq, int32_t Hkv) {
    if (Hq != Hkv) return kBalancedWaves;
    if (dtype < 0 || dtype == KVQ_INT8) return kBalancedWavesInt8Mha;
    if (dtype == KVQ_INT4) return kBalancedWavesInt4Mha;
    return kBalancedWaves;
}

struct Plan {
    int32_t P = 1;
    int32_t PS = KVQ_BLOCK_SIZE;
    int32_t NW = 0;          // balanced split: waves per head row (0 for fixed partitions)
    size_t rows = 0;         // partial rows in the workspace
    size_t plan_bytes = 0;   // balanced split: int32 [batch + 2]
};

Plan plan(int32_t batch, int32_t Hq, int32_t Hkv, int32_t max_context_len, int32_t partition_size,
          int64_t waves) {
    Plan p;
    if (partition_size == KVQ_PARTITION_BALANCED) {
        const int64_t hw = Hq == Hkv ? Hq : Hkv;
        const int64_t max_tiles = (int64_t)batch * (((int64_t)max_context_len + KVQ_BLOCK_SIZE - 1) / KVQ_BLOCK_SIZE);
        int64_t nw = (waves + hw - 1) / hw;
        nw = std::min(nw, std::max<int64_t>(1, (max_tiles + kMinTiles - 1) / kMinTiles));
        nw = std::min<int64_t>(nw, 65535);
        p.NW = (int32_t)nw;
        p.rows = (size_t)Hq * (size_t)(nw + batch);
        p.plan_bytes = (size_t)(batch + 2) * sizeof(int32_t);
    } else if (partition_size == 0) {
        const int64_t whole = (((int64_t)max_context_len + KVQ_BLOCK_SIZE - 1) / KVQ_BLOCK_SIZE) * KVQ_BLOCK_SIZE;
        p.PS = whole > 0 ? (int32_t)whole : KVQ_BLOCK_SIZE;  // max_context_len <= KVQ_MAX_CONTEXT_LEN
    } else {
        p.PS = partition_size;
        p.P = max_context_len > 0
                  ? (int32_t)(((int64_t)max_context_len + partition_size - 1) / partition_size)
                  : 1;
        if (p.P > 1) p.rows = (size_t)batch * (size_t)Hq * (size_t)p.P;
    }
    return p;
}

// Workspace layout: [plan][part_o rows x 128 f32][part_m rows f32][part_l rows f32], each 256-byte
// aligned.
size_t plan_workspace_bytes(const Plan& p) {
    if (p.rows == 0 && p.plan_bytes == 0) return 0;
    return align256(p.plan_bytes) + align256(p.rows * KVQ_HEAD_DIM * sizeof(float)) +
           2 * align256(p.rows * sizeof(float));
}

// Kernel-timing hook state: one session per calling thread (only that thread's calls are timed,
// and sessions on different threads never touch each other's events).
struct Timing {
    bool active = false;
    int32_t capacity = 0;
    int32_t used = 0;
    std::vector<hipEvent_t> ev;  // 2 per call: before and after the partition kernel
};
thread_local Timing g_timing;

void timing_release() {
    for (hipEvent_t e : g_timing.ev)
        if (e) (void)hipEventDestroy(e);
    g_timing.ev.clear();
    g_timing.active = false;
    g_timing.capacity = g_timing.used = 0;
}

}  // namespace

extern "C" {

const char* kvq_version(void) { return "0.1.0"; }

const char* kvq_last_error(void) { return g_err; }

const char* kvq_status_string(int status) {
    switch (status) {
        case KVQ_OK: return "ok";
        case KVQ_ERR_ARG: return "invalid argument";
        case KVQ_ERR_DTYPE: return "unknown kv cache dtype";
        case KVQ_ERR_SHAPE: return "unsupported shape";
        case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
        case KVQ_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int kvq_dtype_from_string(const char* s, kvq_dtype* out) {
    if (!s || !out) return fail(KVQ_ERR_ARG, "NULL argument");
    if (!strcmp(s, "fp8") || !strcmp(s, "fp8_e4m3")) *out = KVQ_FP8_E4M3;
    else if (!strcmp(s, "fp8_e5m2")) *out = KVQ_FP8_E5M2;
    else if (!strcmp(s, "int8")) *out = KVQ_INT8;
    else if (!strcmp(s, "fp8_e4m3fnuz")) *out = KVQ_FP8_E4M3FNUZ;
    else if (!strcmp(s, "int4")) *out = KVQ_INT4;
    else return fail(KVQ_ERR_DTYPE, "unknown kv cache dtype name '%s'", s);
    return ok();
}

int kvq_append(const kvq_cache* cache, const void* k_new, const void* v_new,
               const int32_t* cu_new_lens, int32_t num_new_rows, const int32_t* block_tables,
               int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch, void* stream) {
    int st = check_cache(cache);
    if (st) return st;
    st = check_common(block_tables, max_blocks_per_seq, context_lens, batch);
    if (st) return st;
    if (num_new_rows < 0) return fail(KVQ_ERR_ARG, "num_new_rows %d is negative", num_new_rows);
    if (!cu_new_lens && num_new_rows != batch)
        return fail(KVQ_ERR_ARG, "without cu_new_lens, num_new_rows (%d) must equal batch (%d)",
                    num_new_rows, batch);
    if (batch == 0 || num_new_rows == 0) return ok();
    if (!k_new || !v_new) return fail(KVQ_ERR_ARG, "k_new / v_new is NULL");
    if ((size_t)num_new_rows * (size_t)cache->num_kv_heads > 0x7FFFFFFFull)
        return fail(KVQ_ERR_SHAPE, "too many new rows");
    hipError_t e = kvq::launch_append(*cache, static_cast<const uint16_t*>(k_new),
                                      static_cast<const uint16_t*>(v_new), cu_new_lens, num_new_rows,
                                      block_tables, max_blocks_per_seq, context_lens, batch,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kvq_append");
    return ok();
}

size_t kvq_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t max_context_len, int32_t partition_size) {
    if (batch <= 0) return 0;
    // a size query is not a failed call: the thread's last error stays as it was
    char saved[sizeof(g_err)];
    memcpy(saved, g_err, sizeof(g_err));
    const int st = check_decode_sizes(batch, num_q_heads, num_kv_heads, max_context_len, partition_size);
    memcpy(g_err, saved, sizeof(g_err));
    if (st != KVQ_OK) return 0;
    return plan_workspace_bytes(plan(batch, num_q_heads, num_kv_heads, max_context_len, partition_size,
                                     balanced_wave_target(-1, num_q_heads, num_kv_heads)));
}

}  // extern "C"

namespace {

// Shared body of kvq_paged_decode_attn and kvq_decode_step (k_new / v_new set for the latter) and
// of their FP8-math variants.
int decode_common(const char* where, bool fp8_math, const kvq_cache* cache, const void* k_new,
                  const void* v_new, const void* q, void* out, int32_t num_q_heads, float sm_scale,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, int32_t batch, int32_t max_context_len,
                  int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_cache(cache);
    if (st) return st;
    if (fp8_math && (st = check_fp8_math(cache))) return st;
    st = check_common(block_tables, max_blocks_per_seq, context_lens, batch);
    if (st) return st;
    st = check_decode_sizes(batch, num_q_heads, cache->num_kv_heads, max_context_len, partition_size);
    if (st) return st;
    if (!isfinite(sm_scale)) return fail(KVQ_ERR_ARG, "sm_scale must be finite");
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * KVQ_BLOCK_SIZE)
        return fail(KVQ_ERR_ARG, "max_context_len %d exceeds the block table (%d blocks of %d)",
                    max_context_len, max_blocks_per_seq, KVQ_BLOCK_SIZE);
    if (batch == 0) return ok();
    if (!q || !out) return fail(KVQ_ERR_ARG, "q / out is NULL");
    if ((k_new == nullptr) != (v_new == nullptr)) return fail(KVQ_ERR_ARG, "k_new / v_new is NULL");

    const Plan p = plan(batch, num_q_heads, cache->num_kv_heads, max_context_len, partition_size,
                        balanced_wave_target(cache->dtype, num_q_heads, cache->num_kv_heads));
    const size_t need = plan_workspace_bytes(p);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(KVQ_ERR_WORKSPACE, "split-K workspace of %zu bytes needed, %zu given%s", need,
                    workspace_bytes, workspace ? "" : " (NULL)");

    kvq::DecodeArgs a;
    a.cache = cache;
    a.q = static_cast<const uint16_t*>(q);
    a.out = static_cast<uint16_t*>(out);
    a.num_q_heads = num_q_heads;
    a.sm_scale = sm_scale;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.batch = batch;
    a.num_partitions = p.P;
    a.partition_size = p.PS;
    a.balanced_waves = p.NW;
    a.plan = nullptr;
    a.part_o = a.part_m = a.part_l = nullptr;
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.fp8_math = fp8_math;
    if (need > 0) {
        char* w = static_cast<char*>(workspace);
        if (p.plan_bytes) a.plan = reinterpret_cast<int32_t*>(w);
        w += align256(p.plan_bytes);
        a.part_o = reinterpret_cast<float*>(w);
        w += align256(p.rows * KVQ_HEAD_DIM * sizeof(float));
        a.part_m = reinterpret_cast<float*>(w);
        w += align256(p.rows * sizeof(float));
        a.part_l = reinterpret_cast<float*>(w);
    }

    hipEvent_t ev[2] = {nullptr, nullptr};
    if (g_timing.active && g_timing.used < g_timing.capacity) {
        const int slot = g_timing.used++;
        ev[0] = g_timing.ev[2 * slot];
        ev[1] = g_timing.ev[2 * slot + 1];
    }
    hipError_t e = kvq::launch_decode(a, static_cast<hipStream_t>(stream), ev[0], ev[1]);
    if (e != hipSuccess) return hip_fail(e, where);
    return ok();
}

}  // namespace

extern "C" {

int kvq_paged_decode_attn(const kvq_cache* cache, const void* q, void* out, int32_t num_q_heads,
                          float sm_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t batch, int32_t max_context_len,
                          int32_t partition_size, void* workspace, size_t workspace_bytes,
                          void* stream) {
    return decode_common("kvq_paged_decode_attn", false, cache, nullptr, nullptr, q, out, num_q_heads,
                         sm_scale, block_tables, max_blocks_per_seq, context_lens, batch,
                         max_context_len, partition_size, workspace, workspace_bytes, stream);
}

int kvq_paged_decode_attn_fp8math(const kvq_cache* cache, const void* q, void* out,
                                  int32_t num_q_heads, float sm_scale, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t batch, int32_t max_context_len, int32_t partition_size,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    return decode_common("kvq_paged_decode_attn_fp8math", true, cache, nullptr, nullptr, q, out,
                         num_q_heads, sm_scale, block_tables, max_blocks_per_seq, context_lens, batch,
                         max_context_len, partition_size, workspace, workspace_bytes, stream);
}

int kvq_decode_step(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                    void* out, int32_t num_q_heads, float sm_scale, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch,
                    int32_t max_context_len, int32_t partition_size, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (batch > 0 && (!k_new || !v_new)) return fail(KVQ_ERR_ARG, "k_new / v_new is NULL");
    return decode_common("kvq_decode_step", false, cache, k_new, v_new, q, out, num_q_heads, sm_scale,
                         block_tables, max_blocks_per_seq, context_lens, batch, max_context_len,
                         partition_size, workspace, workspace_bytes, stream);
}

int kvq_decode_step_fp8math(const kvq_cache* cache, const void* k_new, const void* v_new,
                            const void* q, void* out, int32_t num_q_heads, float sm_scale,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t batch, int32_t max_context_len,
                            int32_t partition_size, void* workspace, size_t workspace_bytes,
                            void* stream) {
    if (batch > 0 && (!k_new || !v_new)) return fail(KVQ_ERR_ARG, "k_new / v_new is NULL");
    return decode_common("kvq_decode_step_fp8math", true, cache, k_new, v_new, q, out, num_q_heads,
                         sm_scale, block_tables, max_blocks_per_seq, context_lens, batch,
                         max_context_len, partition_size, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The split-K workspace of kvq_decode_step_noalloc: one array per device, held until the process
// ends.  Host code uses only the device address hipGetSymbolAddress gives for it (the array's
// name is a host-side stand-in), taken once per device on that device's first call.
__device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "kvq_decode_step_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(KVQ_ERR_ARG, "kvq_decode_step_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "kvq_decode_step_noalloc: hipGetSymbolAddress");
        if (!p) return fail(KVQ_ERR_HIP, "kvq_decode_step_noalloc: no device address for the scratch array");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KVQ_OK;
}

}  // namespace

extern "C" {

int kvq_decode_step_noalloc(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                            void* out, int32_t num_q_heads, float sm_scale, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch,
                            int32_t max_context_len, int32_t partition_size, void* stream) {
    int st = check_cache(cache);
    if (st) return st;
    if (batch > 0 && (!k_new || !v_new)) return fail(KVQ_ERR_ARG, "k_new / v_new is NULL");
    // 0 for sizes the call rejects: decode_common then reports them
    const size_t need = kvq_decode_workspace_size(batch, num_q_heads, cache->num_kv_heads, max_context_len,
                                                  partition_size);
    if (need > (size_t)KVQ_NOALLOC_SCRATCH_BYTES)
        return fail(KVQ_ERR_WORKSPACE,
                    "kvq_decode_step_noalloc: these sizes need %zu bytes of split-K workspace, more than "
                    "its %zu-byte scratch (pass a workspace to kvq_decode_step instead)",
                    need, (size_t)KVQ_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need > 0 && (st = scratch_address(&ws))) return st;
    return decode_common("kvq_decode_step_noalloc", false, cache, k_new, v_new, q, out, num_q_heads,
                         sm_scale, block_tables, max_blocks_per_seq, context_lens, batch, max_context_len,
                         partition_size, ws, need > 0 ? (size_t)KVQ_NOALLOC_SCRATCH_BYTES : 0, stream);
}

}  // extern "C"

namespace {

int prefill_common(const char* where, bool fp8_math, const kvq_cache* cache, const void* q, void* out,
                   int32_t num_q_heads, float sm_scale, const int32_t* cu_q_lens, int32_t num_q_rows,
                   int32_t max_q_len, const int32_t* block_tables, int32_t max_blocks_per_seq,
                   const int32_t* context_lens, int32_t batch, int32_t max_context_len, void* stream) {
    int st = check_cache(cache);
    if (st) return st;
    if (fp8_math && (st = check_fp8_math(cache))) return st;
    st = check_common(block_tables, max_blocks_per_seq, context_lens, batch);
    if (st) return st;
    if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0)
        return fail(KVQ_ERR_SHAPE, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                    num_q_heads, cache->num_kv_heads);
    if (num_q_heads / cache->num_kv_heads > KVQ_MAX_GROUP)
        return fail(KVQ_ERR_SHAPE, "query heads per KV head (%d) above %d",
                    num_q_heads / cache->num_kv_heads, KVQ_MAX_GROUP);
    if (!isfinite(sm_scale)) return fail(KVQ_ERR_ARG, "sm_scale must be finite");
    if (max_context_len < 0 || max_context_len > KVQ_MAX_CONTEXT_LEN)
        return fail(KVQ_ERR_ARG, "max_context_len %d is outside [0, %d]", max_context_len, KVQ_MAX_CONTEXT_LEN);
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * KVQ_BLOCK_SIZE)
        return fail(KVQ_ERR_ARG, "max_context_len %d exceeds the block table (%d blocks of %d)",
                    max_context_len, max_blocks_per_seq, KVQ_BLOCK_SIZE);
    if (num_q_rows < 0 || max_q_len < 0)
        return fail(KVQ_ERR_ARG, "num_q_rows %d / max_q_len %d is negative", num_q_rows, max_q_len);
    if (max_q_len > max_context_len)
        return fail(KVQ_ERR_ARG, "max_q_len %d exceeds max_context_len %d (query rows are cache tokens)",
                    max_q_len, max_context_len);
    if (batch == 0 || num_q_rows == 0 || max_q_len == 0) return ok();
    if (!q || !out || !cu_q_lens) return fail(KVQ_ERR_ARG, "q / out / cu_q_lens is NULL");
    if (batch > 65535) return fail(KVQ_ERR_SHAPE, "batch must be at most 65535");
    const int32_t G = num_q_heads / cache->num_kv_heads;
    if ((int64_t)(max_q_len + 16 / G - 1) / (16 / G) > 65535)
        return fail(KVQ_ERR_SHAPE, "max_q_len %d needs more than 65535 row tiles", max_q_len);

    kvq::PrefillArgs a;
    a.cache = cache;
    a.q = static_cast<const uint16_t*>(q);
    a.out = static_cast<uint16_t*>(out);
    a.num_q_heads = num_q_heads;
    a.sm_scale = sm_scale;
    a.cu_q_lens = cu_q_lens;
    a.num_q_rows = num_q_rows;
    a.max_q_len = max_q_len;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.batch = batch;
    a.fp8_math = fp8_math;
    hipEvent_t ev[2] = {nullptr, nullptr};
    if (g_timing.active && g_timing.used < g_timing.capacity) {
        const int slot = g_timing.used++;
        ev[0] = g_timing.ev[2 * slot];
        ev[1] = g_timing.ev[2 * slot + 1];
    }
    hipError_t e = kvq::launch_prefill(a, static_cast<hipStream_t>(stream), ev[0], ev[1]);
    if (e != hipSuccess) return hip_fail(e, where);
    return ok();
}

}  // namespace

extern "C" {

int kvq_paged_prefill_attn(const kvq_cache* cache, const void* q, void* out, int32_t num_q_heads,
                           float sm_scale, const int32_t* cu_q_lens, int32_t num_q_rows,
                           int32_t max_q_len, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t batch, int32_t max_context_len,
                           void* stream) {
    return prefill_common("kvq_paged_prefill_attn", false, cache, q, out, num_q_heads, sm_scale,
                          cu_q_lens, num_q_rows, max_q_len, block_tables, max_blocks_per_seq,
                          context_lens, batch, max_context_len, stream);
}

int kvq_paged_prefill_attn_fp8math(const kvq_cache* cache, const void* q, void* out,
                                   int32_t num_q_heads, float sm_scale, const int32_t* cu_q_lens,
                                   int32_t num_q_rows, int32_t max_q_len, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                   int32_t batch, int32_t max_context_len, void* stream) {
    return prefill_common("kvq_paged_prefill_attn_fp8math", true, cache, q, out, num_q_heads, sm_scale,
                          cu_q_lens, num_q_rows, max_q_len, block_tables, max_blocks_per_seq,
                          context_lens, batch, max_context_len, stream);
}

int kvq_quantize_q_fp8(const void* q, int32_t num_rows, void* codes, float* scales, void* stream) {
    if (num_rows < 0) return fail(KVQ_ERR_ARG, "num_rows %d is negative", num_rows);
    if (num_rows == 0) return ok();
    if (!q || !codes || !scales) return fail(KVQ_ERR_ARG, "q / codes / scales is NULL");
    hipError_t e = kvq::launch_quantize_q_fp8(static_cast<const uint16_t*>(q), num_rows,
                                              static_cast<uint8_t*>(codes), scales,
                                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kvq_quantize_q_fp8");
    return ok();
}

int kvq_dequant(const kvq_cache* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                const int32_t* context_lens, int32_t batch, int32_t max_context_len, float* k_out,
                float* v_out, void* stream) {
    int st = check_cache(cache);
    if (st) return st;
    st = check_common(block_tables, max_blocks_per_seq, context_lens, batch);
    if (st) return st;
    if (max_context_len < 0 || max_context_len > KVQ_MAX_CONTEXT_LEN)
        return fail(KVQ_ERR_ARG, "max_context_len %d is outside [0, %d]", max_context_len, KVQ_MAX_CONTEXT_LEN);
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * KVQ_BLOCK_SIZE)
        return fail(KVQ_ERR_ARG, "max_context_len %d exceeds the block table", max_context_len);
    if (batch == 0 || max_context_len == 0) return ok();
    if (!k_out || !v_out) return fail(KVQ_ERR_ARG, "k_out / v_out is NULL");
    if (batch > 65535 || cache->num_kv_heads > 65535)
        return fail(KVQ_ERR_SHAPE, "batch and num_kv_heads must be at most 65535");
    hipError_t e = kvq::launch_dequant(*cache, block_tables, max_blocks_per_seq, context_lens, batch,
                                       max_context_len, k_out, v_out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kvq_dequant");
    return ok();
}

int kvq_timing_begin(int32_t capacity) {
    if (capacity <= 0 || capacity > (1 << 20)) return fail(KVQ_ERR_ARG, "capacity %d out of range", capacity);
    timing_release();
    g_timing.ev.assign((size_t)capacity * 2, nullptr);
    for (auto& e : g_timing.ev) {
        hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) {
            timing_release();
            return hip_fail(r, "kvq_timing_begin");
        }
    }
    g_timing.capacity = capacity;
    g_timing.used = 0;
    g_timing.active = true;
    return ok();
}

int kvq_timing_end(double* main_ms_total, int32_t* main_count) {
    if (!g_timing.active) return fail(KVQ_ERR_ARG, "no timing session is active");
    double mt = 0.0;
    int32_t mc = 0;
    for (int s = 0; s < g_timing.used; ++s) {
        float ms = 0.0f;
        hipError_t r = hipEventSynchronize(g_timing.ev[2 * s + 1]);
        if (r == hipSuccess) r = hipEventElapsedTime(&ms, g_timing.ev[2 * s], g_timing.ev[2 * s + 1]);
        if (r != hipSuccess) {
            timing_release();
            return hip_fail(r, "kvq_timing_end");
        }
        mt += ms;
        ++mc;
    }
    if (main_ms_total) *main_ms_total = mt;
    if (main_count) *main_count = mc;
    timing_release();
    return ok();
}

}  // extern "C"
