"""Pins of the oracle's FP8-math query quantization and of its attention on the quantized query.

"[Feature] TurboMind support W8A8 or FP8 KV Cache" points beyond FP8 storage to FP8 attention and
names E4M3 as the format used there; it gives no scale rule.  The reading: each query row of 128
fp16 values is quantized to OCP E4M3 with its own dynamic scale s_q = fl32(amax / 448) (448 being
E4M3's largest finite value), c_d = enc(fl32(q_d / s_q)), and the attention is the exact attention
of the dequantized row dec(c_d) * s_q over the same cache.  The pins: the scale against numpy's IEEE
float32 division; every code against the nearest of E4M3's finite values built from the page's
field widths (tests/golden/fp8_formats.json), in exact rationals, ties to the even code; the
per-element error within E4M3's half-step; a query already on the grid with a power-of-two scale,
where the quantization is the identity and the attention must equal the fp16-query attention; and
the attention against an fp64 softmax written here over the dequantized cache.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import test_oracle_codec as TC

E4M3 = 1


@pytest.fixture(scope="module")
def e4m3_values(golden_dir):
    """The 254 finite E4M3 values (code -> Fraction) from the page's field widths."""
    with open(os.path.join(golden_dir, "fp8_formats.json")) as f:
        w = json.load(f)["formats"]["E4M3"]
    vals = {}
    for c in range(256):
        v = TC.closed_form_value(c, w, TC.E4M3)
        if isinstance(v, Fraction):
            vals[c] = v
    return vals


def _queries(seed, rows, kind):
    r = np.random.default_rng(seed)
    x = r.standard_normal((rows, 128), dtype=np.float32)
    if kind == "outliers":
        for i in range(rows):
            x[i, r.choice(128, 3, replace=False)] *= np.float32(30)
    if kind == "tiny":   # small magnitudes: many codes land in E4M3's subnormal range
        x *= np.float32(1e-3)
    if kind == "wide":   # magnitudes spread over many binades within a row
        x *= np.exp2(r.uniform(-12, 4, (rows, 128))).astype(np.float32)
    q = x.astype(np.float16)
    q[0] = 0                     # a zero row: scale 1, every code +0
    return q


def _nearest_code(y: Fraction, vals: dict) -> int:
    best = None
    for c, v in vals.items():
        d = abs(v - y)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0 and (best[1] & 1) == 1):
            best = (d, c)
    # +0 and -0 tie exactly: the sign of y picks
    if vals[best[1]] == 0:
        return 0x80 if y < 0 or (y == 0 and best[1] == 0x80) else 0x00
    return best[1]


@pytest.mark.parametrize("kind", ["normal", "outliers", "tiny", "wide"])
def test_q_scale_matches_float32(oracle_mod, kind):
    q = _queries(31, 512, kind)
    c, s = oracle_mod.quantize_q_fp8_rows(q)
    amax = np.abs(q.astype(np.float32)).max(axis=1)
    s_ref = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    np.testing.assert_array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    assert c.shape == q.shape and c.dtype == np.uint8
    assert np.all(c[0] == 0)


@pytest.mark.parametrize("kind", ["normal", "outliers", "tiny", "wide"])
def test_q_codes_nearest_e4m3(oracle_mod, e4m3_values, kind):
    q = _queries(32, 24, kind)
    c, s = oracle_mod.quantize_q_fp8_rows(q)
    qf = q.astype(np.float32)
    y = qf / s[:, None]                 # the fp32 quotient the encoder rounds
    # the largest magnitude of each nonzero row encodes to 448 (or just below the saturation)
    for i in range(1, len(q)):
        for d in range(128):
            exp = _nearest_code(Fraction(float(y[i, d])), e4m3_values)
            if exp != c[i, d]:
                # -0 vs +0 for an input that is exactly zero
                assert y[i, d] == 0 and (exp & 0x7F) == 0 == (c[i, d] & 0x7F) and \
                    bool(c[i, d] & 0x80) == bool(np.signbit(qf[i, d])), (kind, i, d, y[i, d], hex(exp), hex(c[i, d]))
        j = int(np.argmax(np.abs(qf[i])))
        assert (c[i, j] & 0x7F) == 0x7E, (kind, i, hex(c[i, j]))


@pytest.mark.parametrize("kind", ["normal", "outliers", "wide"])
def test_q_error_within_half_step(oracle_mod, kind):
    q = _queries(33, 2048, kind)
    c, s = oracle_mod.quantize_q_fp8_rows(q)
    table = oracle_mod.fp8_decode_table(E4M3)
    qh = table[c] * s[:, None].astype(np.float64)
    qd = q.astype(np.float64)
    # E4M3 keeps 3 fraction bits: half a step is 2^-4 of the value's binade for normals and
    # 2^-10 (half the subnormal spacing 2^-9) below; the fp32 quotient adds at most 2^-24 relative
    bound = np.maximum(2.0 ** -4 * np.abs(qd), 2.0 ** -10 * s[:, None].astype(np.float64)) * (1 + 2.0 ** -20)
    assert np.all(np.abs(qh - qd) <= bound)
    assert np.all(np.sign(qh) * np.sign(qd) >= 0)


def _small_cache(oracle_mod, dtype, seed, ctx, Hkv):
    r = np.random.default_rng(seed)
    B = len(ctx)
    nbps = [(n + 15) // 16 for n in ctx]
    num_blocks = sum(nbps) + 2
    perm = r.permutation(num_blocks).astype(np.int32)
    bt = np.zeros((B, max(max(nbps), 1)), np.int32)
    o = 0
    for b, nb in enumerate(nbps):
        bt[b, :nb] = perm[o:o + nb]
        o += nb
    k = r.standard_normal((sum(ctx), Hkv, 128), dtype=np.float32).astype(np.float16)
    v = r.standard_normal((sum(ctx), Hkv, 128), dtype=np.float32).astype(np.float16)
    cache = oracle_mod.Cache(dtype, num_blocks, Hkv, kv_scale=0.02 if dtype != 3 else 1.0)
    ctxa = np.array(ctx, np.int32)
    cu = np.concatenate([[0], np.cumsum(ctxa)]).astype(np.int32)
    oracle_mod.append(cache, k, v, bt, ctxa, cu_new_lens=cu)
    return cache, bt, ctxa


@pytest.mark.parametrize("dtype,Hq,Hkv", [(1, 4, 4), (2, 8, 2), (1, 8, 1)])
def test_fp8_attention_matches_independent_softmax(oracle_mod, dtype, Hq, Hkv):
    ctx = [1, 17, 40]
    cache, bt, ctxa = _small_cache(oracle_mod, dtype, 40 + dtype, ctx, Hkv)
    r = np.random.default_rng(41)
    q = (r.standard_normal((len(ctx), Hq, 128), dtype=np.float32) * 2).astype(np.float16)
    sm = float(np.float32(1 / np.sqrt(128)))
    got = oracle_mod.decode_attn(cache, q, bt, ctxa, sm_scale=sm, fp8_math=True)
    ko, vo = oracle_mod.dequant(cache, bt, ctxa, max(ctx))
    c, s = oracle_mod.quantize_q_fp8_rows(q)
    qh = oracle_mod.fp8_decode_table(E4M3)[c] * s[..., None].astype(np.float64)
    G = Hq // Hkv
    for b, n in enumerate(ctx):
        for h in range(Hq):
            kk = ko[b, h // G, :n].astype(np.float64)
            vv = vo[b, h // G, :n].astype(np.float64)
            z = sm * (kk @ qh[b, h])
            p = np.exp(z - z.max())
            ref = (p @ vv) / p.sum()
            # the dequantized cache comes back in fp32 (one rounding of each value)
            np.testing.assert_allclose(got[b, h], ref, rtol=1e-6, atol=1e-6)
    # and it is not the fp16-query attention (the quantization changed the logits)
    base = oracle_mod.decode_attn(cache, q, bt, ctxa, sm_scale=sm)
    assert np.abs(got - base).max() > 1e-4


def test_fp8_attention_identity_on_grid(oracle_mod):
    """A query whose values are E4M3 values times 2^-6 with one of magnitude 7 has amax 7, scale
    exactly 2^-6 and codes that reproduce it: the FP8-math attention equals the fp16 one exactly."""
    ctx = [5, 33]
    cache, bt, ctxa = _small_cache(oracle_mod, E4M3, 50, ctx, 2)
    table = oracle_mod.fp8_decode_table(E4M3)
    r = np.random.default_rng(51)
    # every E4M3 value times 2^-6 is exact in fp16 (4 significant bits, at least 2^-15)
    finite = np.array([c for c in range(256) if np.isfinite(table[c]) and abs(table[c]) < 448])
    codes = r.choice(finite, (2, 4, 128))
    codes[..., 5] = 0x7E                # +448 -> 7
    codes[1, 2, 5] = 0xFE               # -448 -> -7
    q = (table[codes] * 2.0 ** -6).astype(np.float16)
    assert np.array_equal(q.astype(np.float64), table[codes] * 2.0 ** -6)   # exact in fp16
    c, s = oracle_mod.quantize_q_fp8_rows(q)
    assert np.all(s == np.float32(2.0 ** -6))
    np.testing.assert_array_equal(table[c], table[codes])
    sm = float(np.float32(1 / np.sqrt(128)))
    a = oracle_mod.decode_attn(cache, q, bt, ctxa, sm_scale=sm, fp8_math=True)
    b = oracle_mod.decode_attn(cache, q, bt, ctxa, sm_scale=sm)
    np.testing.assert_array_equal(a, b)


def test_fp8_prefill_rows_are_fp8_decode_rows(oracle_mod):
    ctx = [20, 9]
    cache, bt, ctxa = _small_cache(oracle_mod, E4M3, 60, ctx, 2)
    r = np.random.default_rng(61)
    nq = [4, 9]
    cu = np.array([0, 4, 13], np.int32)
    q = r.standard_normal((13, 4, 128), dtype=np.float32).astype(np.float16)
    got = oracle_mod.prefill_attn(cache, q, bt, ctxa, cu, fp8_math=True)
    for t in range(13):
        b = 0 if t < 4 else 1
        pos = ctx[b] - nq[b] + (t - cu[b])
        one = oracle_mod.decode_attn(cache, q[t:t + 1], bt[b:b + 1], np.array([pos + 1], np.int32),
                                     fp8_math=True)
        np.testing.assert_array_equal(got[t], one[0])
