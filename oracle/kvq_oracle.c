/*
 * kvq_oracle.c -- CPU oracle for the 8-bit paged KV cache and its decode-step attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark load this file's library.  The product path (the HIP library) never calls it, shares no
 * code, header, table or constant with it, and must fail loudly when its own extension is missing.
 *
 * It is deliberately plain and slow: scalar loops, fp64 arithmetic, one function per step of the
 * method, each step taken from its definition.  Sources, by page title and section:
 *
 *   [TGI-FP8] "Accelerating Inference with FP8 KV Cache" (text-generation-inference docs)
 *       section "FP8 Formats: E4M3 and E5M2": the OCP E4M3 layout (1 sign, 4 biased-exponent,
 *       3 mantissa bits) and E5M2 layout (1 sign, 5 biased-exponent, 2 mantissa bits); a
 *       per-tensor FP32 scaling factor stored alongside the quantized tensor.
 *       section "FP8 E4M3 KV Cache": the scale defaults to 1.0 when none is given.
 *       opening section: the cache is stored as FP8 while the attention arithmetic runs at higher
 *       precision (FP16 there; fp64 here, since this is the reference).
 *   [LMD-1463] "[Feature] TurboMind support W8A8 or FP8 KV Cache" (lmdeploy issue thread):
 *       the online INT8 KV cache variant.  The thread gives no formula; the reading used here is
 *       symmetric INT8 with one fp32 scale per (token, head): s = amax/127, q = rne(x/s) clamped to
 *       [-127, 127].
 *       The same thread names INT4 next to INT8 for the online KV cache.  The reading used here
 *       for INT4 is asymmetric, one (scale, zero point) pair of fp32 per (token, head): the 16 levels
 *       zp + q * s, q = 0..15, span the row from its minimum zp = min x to its maximum,
 *       s = fl32(fl32(max x - min x) / 15), q = rne(fl32(fl32(x - zp) / s)) clamped to [0, 15]; a
 *       constant row gives s = 0 and q = 0 (its value is zp).  [QQQ-2] cites kv4 caches (QServe).
 *   [QQQ-2] "[QST] Scale factors and benchmarks" (QQQ issue thread): the serving stack the
 *       8-bit cache lives in is paged ("armed with paged attention"): fixed-size token blocks
 *       reached through a per-sequence block table.
 *
 * Readings where the pages are silent:
 *   - Exponent biases and special values follow the OCP definitions the page names: E4M3 has bias 7,
 *     no infinities and NaN only at S.1111.111 (largest finite 448); E5M2 has bias 15 with IEEE-style
 *     infinities (exponent 31, mantissa 0) and NaNs (exponent 31, mantissa != 0).
 *   - E4M3FNUZ, the FP8 flavour the page lists for AMD GPUs ("Current Hardware Support") and as a
 *     kv_cache_torch_dtype ("Checkpoint structure for KV scales"): the same 1/4/3 layout read as the
 *     "finite, NaN-as-unsigned-zero" format -- bias 8, no infinities, no negative zero, and the one
 *     NaN at 0x80 (the code -0 would have); the largest finite value is S.1111.111 = 240.  Every
 *     other code means half of what the same bits mean in E4M3.  A NaN encodes as 0x80 and a value
 *     that rounds to zero as 0x00, whatever its sign.
 *   - Encode direction: code = enc(fl32(x / kv_scale)); decode: value = dec(code) * kv_scale.
 *   - The quotient is one correctly rounded fp32 division; the 8-bit rounding is round-to-nearest,
 *     ties to the code with an even mantissa LSB; finite overflow and +-inf saturate to +-max;
 *     NaN encodes as sign | 0x7F; signed zero and subnormals are kept.
 *   - Cache layout (both formats and INT8): K codes [num_blocks][Hkv][8][16 tokens][16 dims], i.e.
 *     dim d of token t sits at byte (d / 16) * 256 + t * 16 + d % 16 of its 2048-byte tile;
 *     V codes [num_blocks][Hkv][128 dims][16 tokens]; INT8 scales [num_blocks][Hkv][2][16 tokens]:
 *     per (block, head) tile one row of the 16 K scales and then the 16 V scales; k_scale points at
 *     the rows and v_scale at k_scale + 16, so both are indexed alike.
 *   - INT4 layout (two 4-bit codes per byte, the even one in the low nibble): K [num_blocks][Hkv]
 *     [4][16 tokens][16 bytes], dim d of token t in byte (d / 32) * 256 + t * 16 + (d % 32) / 2
 *     of its 1024-byte tile, nibble d % 2; V [num_blocks][Hkv][4 token quads][16][8][2 bytes],
 *     token t of dim d in byte (t / 4) * 256 + (d % 16) * 16 + (d / 16) * 2 + (t % 4) / 2, nibble
 *     t % 2 (each 16-bit unit holds four consecutive tokens of one dim); (scale, zero point) pairs
 *     [num_blocks][Hkv][16][2] for K and for V.
 *   - context_lens are post-append lengths; context_lens[b] == 0 gives an all-zero output row.
 *   - Query head h reads KV head h / (Hq / Hkv).
 *
 * Build (see oracle/build.py): gcc -O2 -std=c11 -ffp-contract=off (no -ffast-math); x86-64 SSE
 * arithmetic, so `float` operations are IEEE binary32 with round-to-nearest-even and the default
 * FE_TONEAREST mode makes nearbyint() round half to even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KVQO_E4M3 1
#define KVQO_E5M2 2
#define KVQO_INT8 3
#define KVQO_E4M3FNUZ 4
#define KVQO_INT4 5

#define KVQO_BLOCK 16
#define KVQO_DIM 128

/* ------------------------------------------------------------------------------------------ */
/* IEEE binary16 -> double, from the format's definition: 1 sign bit, 5 exponent bits with bias 15,
 * 10 fraction bits; exponent 0 is subnormal (f * 2^-24), exponent 31 is inf / NaN.  Exact.      */
double kvqo_fp16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* ------------------------------------------------------------------------------------------ */
/* FP8 format parameters [TGI-FP8 "FP8 Formats: E4M3 and E5M2"] with the OCP bias reading.      */
typedef struct {
    int ebits, mbits, bias;
    double max_finite;   /* E4M3 448, E5M2 57344, E4M3FNUZ 240 */
    double min_normal;   /* 2^(1-bias) */
} kvqo_fp8_fmt;

static int kvqo_get_fmt(int fmt, kvqo_fp8_fmt *out)
{
    if (fmt == KVQO_E4M3) {
        out->ebits = 4; out->mbits = 3; out->bias = 7;
        /* largest exponent field 15 with mantissa 110b: 2^(15-7) * (1 + 6/8) = 448 (111b is NaN) */
        out->max_finite = ldexp(1.0 + 6.0 / 8.0, 15 - 7);
    } else if (fmt == KVQO_E4M3FNUZ) {
        out->ebits = 4; out->mbits = 3; out->bias = 8;
        /* every exponent field is finite: 2^(15-8) * (1 + 7/8) = 240 */
        out->max_finite = ldexp(1.0 + 7.0 / 8.0, 15 - 8);
    } else if (fmt == KVQO_E5M2) {
        out->ebits = 5; out->mbits = 2; out->bias = 15;
        /* largest finite exponent field 30 (31 is inf/NaN) with mantissa 11b: 2^15 * 1.75 = 57344 */
        out->max_finite = ldexp(1.0 + 3.0 / 4.0, 30 - 15);
    } else {
        return -1;
    }
    out->min_normal = ldexp(1.0, 1 - out->bias);
    return 0;
}

/* Decode one FP8 code to its exact value.  Normal: (-1)^s 2^(e-bias) (1 + m/2^mbits);
 * subnormal (e == 0): (-1)^s 2^(1-bias) (m/2^mbits); E4M3 S.1111.111 is NaN; E5M2 exponent 31 is
 * inf (m == 0) or NaN; E4M3FNUZ 0x80 (sign set, all else zero) is NaN.  Returns NAN for an unknown
 * format.                                                                                       */
double kvqo_fp8_decode(int fmt, uint8_t code)
{
    kvqo_fp8_fmt F;
    if (kvqo_get_fmt(fmt, &F) != 0)
        return NAN;
    int sign = code >> 7;
    int e = (code >> F.mbits) & ((1 << F.ebits) - 1);
    int m = code & ((1 << F.mbits) - 1);
    double v;
    if (fmt == KVQO_E4M3 && e == 15 && m == 7)
        v = NAN;
    else if (fmt == KVQO_E4M3FNUZ && code == 0x80)
        v = NAN;
    else if (fmt == KVQO_E5M2 && e == 31)
        v = (m == 0) ? INFINITY : NAN;
    else if (e == 0)
        v = ldexp((double)m, 1 - F.bias - F.mbits);
    else
        v = ldexp((double)((1 << F.mbits) + m), e - F.bias - F.mbits);
    return sign ? -v : v;
}

/* The magnitude bits (the code without its sign) of a >= 0 in format F: saturating, round to
 * nearest, ties to even mantissa LSB.  The magnitude is clamped to max_finite first; every value
 * that would round above max_finite lies above it, and values in (max, rounding threshold] round to
 * max anyway, so clamping first is the same as rounding and then saturating.                    */
static uint8_t kvqo_fp8_encode_magnitude(const kvqo_fp8_fmt *Fp, double a)
{
    kvqo_fp8_fmt F = *Fp;
    if (a > F.max_finite)
        a = F.max_finite;                       /* saturation, also for +-inf */
    if (a >= F.min_normal) {
        int k;
        (void)frexp(a, &k);                     /* a = f * 2^k with f in [0.5, 1) */
        int e = k - 1;                          /* a = 2^e * (1 + frac) */
        double M = nearbyint((ldexp(a, -e) - 1.0) * (double)(1 << F.mbits));
        if (M == (double)(1 << F.mbits)) {      /* mantissa rounded up into the next binade */
            e += 1;
            M = 0.0;
        }
        return (uint8_t)(((e + F.bias) << F.mbits) | (int)M);
    }
    /* subnormal range: multiples of the step 2^(1-bias-mbits); M == 2^mbits is the min-normal code,
     * whose bit pattern is exactly (1 << mbits), so the same expression covers it */
    double M = nearbyint(ldexp(a, F.bias - 1 + F.mbits));
    return (uint8_t)(int)M;
}

/* Encode an fp32 value y (already divided by the scale) to FP8: the sign bit, then the magnitude
 * as above.  NaN encodes as sign | 0x7F (E4M3, E5M2); E4M3FNUZ has one NaN code (0x80) and no
 * negative zero.                                                                                 */
uint8_t kvqo_fp8_encode(int fmt, float y)
{
    kvqo_fp8_fmt F;
    if (kvqo_get_fmt(fmt, &F) != 0)
        return 0;
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    if (isnan(y))
        return (uint8_t)(fmt == KVQO_E4M3FNUZ ? 0x80 : (sign | 0x7F));
    uint8_t mag = kvqo_fp8_encode_magnitude(&F, fabs((double)y));
    if (fmt == KVQO_E4M3FNUZ && mag == 0)
        return 0x00;                            /* unsigned zero */
    return (uint8_t)(sign | mag);
}

/* One element of the FP8 append: y = fl32(fl32(x) / kv_scale), then encode. */
uint8_t kvqo_fp8_quantize(int fmt, uint16_t x_fp16, float kv_scale)
{
    float x = (float)kvqo_fp16_to_double(x_fp16); /* exact: every binary16 value is a binary32 */
    float y = x / kv_scale;                        /* one IEEE binary32 division */
    return kvqo_fp8_encode(fmt, y);
}

/* Online INT8 encode of one (token, head) row of n values: a = max |x| (exact), s = fl32(a/127),
 * q = clamp(rne(fl32(x/s)), -127, 127); a zero row gives s = 0 and q = 0.                        */
void kvqo_int8_quantize_row(const uint16_t *x, int n, int8_t *q, float *s_out)
{
    float amax = 0.0f;
    for (int d = 0; d < n; ++d) {
        float v = fabsf((float)kvqo_fp16_to_double(x[d]));
        if (v > amax)
            amax = v;
    }
    if (amax == 0.0f) {
        for (int d = 0; d < n; ++d)
            q[d] = 0;
        *s_out = 0.0f;
        return;
    }
    float s = amax / 127.0f;
    for (int d = 0; d < n; ++d) {
        float y = (float)kvqo_fp16_to_double(x[d]) / s;
        double r = nearbyint((double)y);
        if (r > 127.0)
            r = 127.0;
        if (r < -127.0)
            r = -127.0;
        q[d] = (int8_t)r;
    }
    *s_out = s;
}

/* Online INT4 encode of one (token, head) row of n values (reading in the header): zp = min x,
 * s = fl32(fl32(max x - zp) / 15), q = clamp(rne(fl32(fl32(x - zp) / s)), 0, 15); a constant row
 * gives s = 0 and q = 0.  Inputs are assumed finite.                                            */
void kvqo_int4_quantize_row(const uint16_t *x, int n, uint8_t *q, float *s_out, float *zp_out)
{
    float mn = INFINITY, mx = -INFINITY;
    for (int d = 0; d < n; ++d) {
        float v = (float)kvqo_fp16_to_double(x[d]);
        if (v < mn)
            mn = v;
        if (v > mx)
            mx = v;
    }
    float range = mx - mn;          /* one binary32 subtraction */
    float s = range / 15.0f;        /* one binary32 division */
    *zp_out = mn;
    if (s == 0.0f) {
        for (int d = 0; d < n; ++d)
            q[d] = 0;
        *s_out = 0.0f;
        return;
    }
    for (int d = 0; d < n; ++d) {
        float y = ((float)kvqo_fp16_to_double(x[d]) - mn) / s;
        double r = nearbyint((double)y);
        if (r > 15.0)
            r = 15.0;
        if (r < 0.0)
            r = 0.0;
        q[d] = (uint8_t)r;
    }
    *s_out = s;
}

/* ------------------------------------------------------------------------------------------ */
/* Paged layout offsets (see the header comment).                                               */
static size_t k_off(int Hkv, int blk, int g, int t, int d)
{
    /* [blk][g][d / 16][t][d % 16]: the tile is eight 256-byte chunks of 16 dims x 16 tokens */
    size_t tile = ((size_t)blk * Hkv + g) * KVQO_BLOCK * KVQO_DIM;
    return tile + (size_t)(d / 16) * (16 * KVQO_BLOCK) + (size_t)t * 16 + (size_t)(d % 16);
}
static size_t v_off(int Hkv, int blk, int g, int t, int d)
{
    return (((size_t)blk * Hkv + g) * KVQO_DIM + d) * KVQO_BLOCK + t;
}
static size_t s_off(int Hkv, int blk, int g, int t)
{
    return ((size_t)blk * Hkv + g) * KVQO_BLOCK + t;
}
/* INT8: token t's scale in the tile's row of 2 * 16 scales, from k_scale or from v_scale */
static size_t s_off8(int Hkv, int blk, int g, int t)
{
    return ((size_t)blk * Hkv + g) * (2 * KVQO_BLOCK) + t;
}
/* INT4: byte offsets; the code is nibble (d % 2) of the K byte and nibble (t % 2) of the V byte */
static size_t k_off4(int Hkv, int blk, int g, int t, int d)
{
    size_t tile = ((size_t)blk * Hkv + g) * (KVQO_BLOCK * KVQO_DIM / 2);
    return tile + (size_t)(d / 32) * (16 * KVQO_BLOCK) + (size_t)t * 16 + (size_t)((d % 32) / 2);
}
static size_t v_off4(int Hkv, int blk, int g, int t, int d)
{
    size_t tile = ((size_t)blk * Hkv + g) * (KVQO_BLOCK * KVQO_DIM / 2);
    return tile + (size_t)(t / 4) * 256 + (size_t)(d % 16) * 16 + (size_t)(d / 16) * 2 + (size_t)((t % 4) / 2);
}
static uint8_t get_nibble(const uint8_t *a, size_t off, int hi)
{
    return hi ? (uint8_t)(a[off] >> 4) : (uint8_t)(a[off] & 0x0F);
}
static void put_nibble(uint8_t *a, size_t off, int hi, uint8_t q)
{
    a[off] = hi ? (uint8_t)((a[off] & 0x0F) | (q << 4)) : (uint8_t)((a[off] & 0xF0) | q);
}

/* Append new K/V rows into the paged cache (all arrays in host memory).
 *   k_new, v_new : fp16 bits [T][Hkv][128]
 *   cu_new_lens  : [B+1] row offsets per sequence, or NULL for exactly one row per sequence
 *   context_lens : post-append lengths; sequence b's j-th new row goes to position
 *                  context_lens[b] - n_b + j, i.e. block block_tables[b][p/16], slot p%16.
 * Returns 0, or -1 for an unknown dtype / a position outside the block table.                   */
int kvqo_append(int dtype, int Hkv, uint8_t *k_cache, uint8_t *v_cache, float *k_scale,
                float *v_scale, float kv_scale, const uint16_t *k_new, const uint16_t *v_new,
                const int32_t *cu_new_lens, const int32_t *block_tables, int max_blocks_per_seq,
                const int32_t *context_lens, int batch)
{
    if (dtype != KVQO_E4M3 && dtype != KVQO_E5M2 && dtype != KVQO_INT8 && dtype != KVQO_E4M3FNUZ &&
        dtype != KVQO_INT4)
        return -1;
    int8_t qk[KVQO_DIM], qv[KVQO_DIM];
    uint8_t uk[KVQO_DIM], uv[KVQO_DIM];
    for (int b = 0; b < batch; ++b) {
        int row0 = cu_new_lens ? cu_new_lens[b] : b;
        int n_b = cu_new_lens ? cu_new_lens[b + 1] - cu_new_lens[b] : 1;
        for (int j = 0; j < n_b; ++j) {
            int p = context_lens[b] - n_b + j;
            if (p < 0 || p / KVQO_BLOCK >= max_blocks_per_seq)
                return -1;
            int blk = block_tables[(size_t)b * max_blocks_per_seq + p / KVQO_BLOCK];
            int t = p % KVQO_BLOCK;
            for (int g = 0; g < Hkv; ++g) {
                const uint16_t *xk = k_new + ((size_t)(row0 + j) * Hkv + g) * KVQO_DIM;
                const uint16_t *xv = v_new + ((size_t)(row0 + j) * Hkv + g) * KVQO_DIM;
                if (dtype == KVQO_INT4) {
                    float sk, zk, sv, zv;
                    kvqo_int4_quantize_row(xk, KVQO_DIM, uk, &sk, &zk);
                    kvqo_int4_quantize_row(xv, KVQO_DIM, uv, &sv, &zv);
                    for (int d = 0; d < KVQO_DIM; ++d) {
                        put_nibble(k_cache, k_off4(Hkv, blk, g, t, d), d % 2, uk[d]);
                        put_nibble(v_cache, v_off4(Hkv, blk, g, t, d), t % 2, uv[d]);
                    }
                    k_scale[2 * s_off(Hkv, blk, g, t)] = sk;
                    k_scale[2 * s_off(Hkv, blk, g, t) + 1] = zk;
                    v_scale[2 * s_off(Hkv, blk, g, t)] = sv;
                    v_scale[2 * s_off(Hkv, blk, g, t) + 1] = zv;
                } else if (dtype == KVQO_INT8) {
                    float sk, sv;
                    kvqo_int8_quantize_row(xk, KVQO_DIM, qk, &sk);
                    kvqo_int8_quantize_row(xv, KVQO_DIM, qv, &sv);
                    for (int d = 0; d < KVQO_DIM; ++d) {
                        k_cache[k_off(Hkv, blk, g, t, d)] = (uint8_t)qk[d];
                        v_cache[v_off(Hkv, blk, g, t, d)] = (uint8_t)qv[d];
                    }
                    k_scale[s_off8(Hkv, blk, g, t)] = sk;
                    v_scale[s_off8(Hkv, blk, g, t)] = sv;
                } else {
                    for (int d = 0; d < KVQO_DIM; ++d) {
                        k_cache[k_off(Hkv, blk, g, t, d)] = kvqo_fp8_quantize(dtype, xk[d], kv_scale);
                        v_cache[v_off(Hkv, blk, g, t, d)] = kvqo_fp8_quantize(dtype, xv[d], kv_scale);
                    }
                }
            }
        }
    }
    return 0;
}

/* Exact dequantized value of one cached element, in fp64: FP8 dec(c) * kv_scale, INT8 q * s,
 * INT4 q * s + zp.  All are exact in fp64.  The products have at most 4 + 24 or 8 + 24 significant
 * bits.  For INT4, zp is a binary16 value (the row's minimum) and s is at least 1/30 of a binary16
 * step at the row's extremes (max > min are both binary16), so the bits of q * s + zp span at most
 * about 41 places.                                                                             */
static double dq4(const uint8_t *codes, size_t off, int hi, const float *sz, size_t so)
{
    return (double)get_nibble(codes, off, hi) * (double)sz[2 * so] + (double)sz[2 * so + 1];
}
static double dq_k(int dtype, int Hkv, const uint8_t *kc, const float *ks, float kv_scale, int blk,
                   int g, int t, int d)
{
    if (dtype == KVQO_INT4)
        return dq4(kc, k_off4(Hkv, blk, g, t, d), d % 2, ks, s_off(Hkv, blk, g, t));
    uint8_t c = kc[k_off(Hkv, blk, g, t, d)];
    if (dtype == KVQO_INT8)
        return (double)(int8_t)c * (double)ks[s_off8(Hkv, blk, g, t)];
    return kvqo_fp8_decode(dtype, c) * (double)kv_scale;
}
static double dq_v(int dtype, int Hkv, const uint8_t *vc, const float *vs, float kv_scale, int blk,
                   int g, int t, int d)
{
    if (dtype == KVQO_INT4)
        return dq4(vc, v_off4(Hkv, blk, g, t, d), t % 2, vs, s_off(Hkv, blk, g, t));
    uint8_t c = vc[v_off(Hkv, blk, g, t, d)];
    if (dtype == KVQO_INT8)
        return (double)(int8_t)c * (double)vs[s_off8(Hkv, blk, g, t)];
    return kvqo_fp8_decode(dtype, c) * (double)kv_scale;
}

/* Dequantize the cache into dense fp32 [B][Hkv][max_context_len][128] for K and V:
 * out = fl32(exact dequantized value) -- one rounding.  Slots t >= context_lens[b] are untouched. */
int kvqo_dequant(int dtype, int Hkv, const uint8_t *k_cache, const uint8_t *v_cache,
                 const float *k_scale, const float *v_scale, float kv_scale,
                 const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                 int batch, int max_context_len, float *k_out, float *v_out)
{
    if (dtype != KVQO_E4M3 && dtype != KVQO_E5M2 && dtype != KVQO_INT8 && dtype != KVQO_E4M3FNUZ &&
        dtype != KVQO_INT4)
        return -1;
    for (int b = 0; b < batch; ++b) {
        int n = context_lens[b];
        if (n > max_context_len)
            return -1;
        for (int g = 0; g < Hkv; ++g)
            for (int t = 0; t < n; ++t) {
                int blk = block_tables[(size_t)b * max_blocks_per_seq + t / KVQO_BLOCK];
                for (int d = 0; d < KVQO_DIM; ++d) {
                    size_t o = (((size_t)b * Hkv + g) * max_context_len + t) * KVQO_DIM + d;
                    k_out[o] = (float)dq_k(dtype, Hkv, k_cache, k_scale, kv_scale, blk, g, t % KVQO_BLOCK, d);
                    v_out[o] = (float)dq_v(dtype, Hkv, v_cache, v_scale, kv_scale, blk, g, t % KVQO_BLOCK, d);
                }
            }
    }
    return 0;
}

/* FP8 math (the "FP8 attention" the lmdeploy thread points to, for the QK^T product): one query
 * row of 128 fp16 values quantized to OCP E4M3 with a dynamic scale of its own,
 *   s_q = fl32(max_d |q_d| / 448),  c_d = enc_E4M3(fl32(q_d / s_q))   (s_q = 1 for a zero row),
 * so that the row's dequantized values are dec(c_d) * s_q.  Inputs are assumed finite.          */
void kvqo_quantize_q_fp8_row(const uint16_t *q, uint8_t *codes, float *s_out)
{
    float amax = 0.0f;
    for (int d = 0; d < KVQO_DIM; ++d) {
        float v = fabsf((float)kvqo_fp16_to_double(q[d]));
        if (v > amax)
            amax = v;
    }
    float s = amax > 0.0f ? amax / 448.0f : 1.0f;   /* one binary32 division */
    for (int d = 0; d < KVQO_DIM; ++d)
        codes[d] = kvqo_fp8_encode(KVQO_E4M3, (float)kvqo_fp16_to_double(q[d]) / s);
    *s_out = s;
}

/* Decode-step attention of one query head h of sequence b over the paged cache, in fp64:
 *   g = h / (Hq/Hkv), n = context_lens[b];
 *   z_t = sm_scale * sum_d q[d] * k^[t][d]      for t < n;
 *   out[d] = sum_t exp(z_t - max z) v^[t][d] / sum_t exp(z_t - max z).
 * q is the row's 128 exact values; out is 128 doubles.  n == 0 gives zeros.  Returns 0 or -1.   */
static int decode_attn_row(int dtype, int Hkv, int Hq, const uint8_t *k_cache, const uint8_t *v_cache,
                           const float *k_scale, const float *v_scale, float kv_scale,
                           const double *qd, float sm_scale, const int32_t *block_tables,
                           int max_blocks_per_seq, const int32_t *context_lens, int b, int h,
                           double *out);

/* The same attention for the fp16 query q[b][h] (fp16 bits [B][Hq][128]).                      */
int kvqo_decode_attn_head(int dtype, int Hkv, int Hq, const uint8_t *k_cache, const uint8_t *v_cache,
                          const float *k_scale, const float *v_scale, float kv_scale,
                          const uint16_t *q, float sm_scale, const int32_t *block_tables,
                          int max_blocks_per_seq, const int32_t *context_lens, int b, int h,
                          double *out)
{
    double qd[KVQO_DIM];
    for (int d = 0; d < KVQO_DIM; ++d)
        qd[d] = kvqo_fp16_to_double(q[((size_t)b * Hq + h) * KVQO_DIM + d]);
    return decode_attn_row(dtype, Hkv, Hq, k_cache, v_cache, k_scale, v_scale, kv_scale, qd, sm_scale,
                           block_tables, max_blocks_per_seq, context_lens, b, h, out);
}

/* The same attention with the query quantized to E4M3 first (FP8 math): q[b][h] is replaced by its
 * exact dequantized values dec(c_d) * s_q (kvqo_quantize_q_fp8_row).                          */
int kvqo_decode_attn_head_fp8q(int dtype, int Hkv, int Hq, const uint8_t *k_cache,
                               const uint8_t *v_cache, const float *k_scale, const float *v_scale,
                               float kv_scale, const uint16_t *q, float sm_scale,
                               const int32_t *block_tables, int max_blocks_per_seq,
                               const int32_t *context_lens, int b, int h, double *out)
{
    uint8_t codes[KVQO_DIM];
    float s;
    double qd[KVQO_DIM];
    kvqo_quantize_q_fp8_row(q + ((size_t)b * Hq + h) * KVQO_DIM, codes, &s);
    for (int d = 0; d < KVQO_DIM; ++d)
        qd[d] = kvqo_fp8_decode(KVQO_E4M3, codes[d]) * (double)s;   /* exact: 4 + 24 bits */
    return decode_attn_row(dtype, Hkv, Hq, k_cache, v_cache, k_scale, v_scale, kv_scale, qd, sm_scale,
                           block_tables, max_blocks_per_seq, context_lens, b, h, out);
}

static int decode_attn_row(int dtype, int Hkv, int Hq, const uint8_t *k_cache, const uint8_t *v_cache,
                           const float *k_scale, const float *v_scale, float kv_scale,
                           const double *qd, float sm_scale, const int32_t *block_tables,
                           int max_blocks_per_seq, const int32_t *context_lens, int b, int h,
                           double *out)
{
    if (dtype != KVQO_E4M3 && dtype != KVQO_E5M2 && dtype != KVQO_INT8 && dtype != KVQO_E4M3FNUZ &&
        dtype != KVQO_INT4)
        return -1;
    if (Hkv <= 0 || Hq % Hkv != 0)
        return -1;
    int G = Hq / Hkv;
    int g = h / G;
    int n = context_lens[b];
    for (int d = 0; d < KVQO_DIM; ++d)
        out[d] = 0.0;
    if (n <= 0)
        return 0;
    double *z = (double *)malloc(sizeof(double) * (size_t)n);
    if (!z)
        return -1;
    double zmax = -INFINITY;
    for (int t = 0; t < n; ++t) {
        int blk = block_tables[(size_t)b * max_blocks_per_seq + t / KVQO_BLOCK];
        double acc = 0.0;
        for (int d = 0; d < KVQO_DIM; ++d)
            acc += qd[d] * dq_k(dtype, Hkv, k_cache, k_scale, kv_scale, blk, g, t % KVQO_BLOCK, d);
        z[t] = (double)sm_scale * acc;
        if (z[t] > zmax)
            zmax = z[t];
    }
    double denom = 0.0;
    for (int t = 0; t < n; ++t) {
        double w = exp(z[t] - zmax);
        int blk = block_tables[(size_t)b * max_blocks_per_seq + t / KVQO_BLOCK];
        denom += w;
        for (int d = 0; d < KVQO_DIM; ++d)
            out[d] += w * dq_v(dtype, Hkv, v_cache, v_scale, kv_scale, blk, g, t % KVQO_BLOCK, d);
    }
    for (int d = 0; d < KVQO_DIM; ++d)
        out[d] /= denom;
    free(z);
    return 0;
}

/* The same attention over dense, unquantized fp16 K/V rows of one (sequence, KV head):
 * k, v are fp16 bits [n][128]; q is fp16 bits [128].  Used only to report how far the quantized
 * cache moves the result; it is not a gate.                                                     */
int kvqo_attn_fp16_dense(const uint16_t *q, const uint16_t *k, const uint16_t *v, int n,
                         float sm_scale, double *out)
{
    for (int d = 0; d < KVQO_DIM; ++d)
        out[d] = 0.0;
    if (n <= 0)
        return 0;
    double *z = (double *)malloc(sizeof(double) * (size_t)n);
    if (!z)
        return -1;
    double zmax = -INFINITY;
    for (int t = 0; t < n; ++t) {
        double acc = 0.0;
        for (int d = 0; d < KVQO_DIM; ++d)
            acc += kvqo_fp16_to_double(q[d]) * kvqo_fp16_to_double(k[(size_t)t * KVQO_DIM + d]);
        z[t] = (double)sm_scale * acc;
        if (z[t] > zmax)
            zmax = z[t];
    }
    double denom = 0.0;
    for (int t = 0; t < n; ++t) {
        double w = exp(z[t] - zmax);
        denom += w;
        for (int d = 0; d < KVQO_DIM; ++d)
            out[d] += w * kvqo_fp16_to_double(v[(size_t)t * KVQO_DIM + d]);
    }
    for (int d = 0; d < KVQO_DIM; ++d)
        out[d] /= denom;
    free(z);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Array forms of the element functions above (plain loops), so the tests can sweep inputs.      */
void kvqo_fp8_decode_array(int fmt, const uint8_t *codes, int n, double *out)
{
    for (int i = 0; i < n; ++i)
        out[i] = kvqo_fp8_decode(fmt, codes[i]);
}

void kvqo_fp8_encode_array(int fmt, const float *y, int n, uint8_t *out)
{
    for (int i = 0; i < n; ++i)
        out[i] = kvqo_fp8_encode(fmt, y[i]);
}

void kvqo_fp8_quantize_array(int fmt, const uint16_t *x, int n, float kv_scale, uint8_t *out)
{
    for (int i = 0; i < n; ++i)
        out[i] = kvqo_fp8_quantize(fmt, x[i], kv_scale);
}

void kvqo_fp16_to_double_array(const uint16_t *x, int n, double *out)
{
    for (int i = 0; i < n; ++i)
        out[i] = kvqo_fp16_to_double(x[i]);
}

void kvqo_int8_quantize_rows(const uint16_t *x, int rows, int n, int8_t *q, float *s)
{
    for (int r = 0; r < rows; ++r)
        kvqo_int8_quantize_row(x + (size_t)r * n, n, q + (size_t)r * n, s + r);
}

void kvqo_int4_quantize_rows(const uint16_t *x, int rows, int n, uint8_t *q, float *s, float *zp)
{
    for (int r = 0; r < rows; ++r)
        kvqo_int4_quantize_row(x + (size_t)r * n, n, q + (size_t)r * n, s + r, zp + r);
}

void kvqo_quantize_q_fp8_rows(const uint16_t *q, int rows, uint8_t *codes, float *s)
{
    for (int r = 0; r < rows; ++r)
        kvqo_quantize_q_fp8_row(q + (size_t)r * KVQO_DIM, codes + (size_t)r * KVQO_DIM, s + r);
}
