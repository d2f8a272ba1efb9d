"""Pins of the oracle's FP8 codec against what the pages and the mathematics fix.

Nothing here re-types the oracle's formulas.  The decode tables are checked against (i) values built
from the bit-field widths printed on "Accelerating Inference with FP8 KV Cache", section "FP8
Formats: E4M3 and E5M2" (tests/golden/fp8_formats.json) with exact rationals, (ii) torch's CPU
float8 dtypes, and (iii) the textbook identity that an E5M2 code is the top byte of an IEEE binary16.
E4M3FNUZ (the AMD flavour the page lists under "Current Hardware Support") is pinned the same way
(its torch dtype is float8_e4m3fnuz) and by its relation to the already pinned E4M3 table.
The encoder is checked by brute force: for every one of the 65,536 fp16 inputs and several scales,
the nearest finite code over all 256 codes (ties to the even code), against torch's cast where the
cast does not overflow, and by the round trip enc(dec(c)) == c.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

E4M3, E5M2, E4M3FNUZ = 1, 2, 4
FMT_NAME = {E4M3: "E4M3", E5M2: "E5M2", E4M3FNUZ: "E4M3FNUZ"}
TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2, E4M3FNUZ: torch.float8_e4m3fnuz}
FMTS = [E4M3, E5M2, E4M3FNUZ]
NAN_CODE = {E4M3: 0x7F, E5M2: 0x7F, E4M3FNUZ: 0x80}  # the code a NaN encodes to (sign aside)


@pytest.fixture(scope="module")
def widths(golden_dir):
    with open(os.path.join(golden_dir, "fp8_formats.json")) as f:
        g = json.load(f)
    return {E4M3: g["formats"]["E4M3"], E5M2: g["formats"]["E5M2"],
            E4M3FNUZ: g["formats"]["E4M3FNUZ"]}, g


def closed_form_value(code: int, w: dict, fmt: int):
    """Exact value (Fraction) or 'nan' / 'inf' / '-inf' from the page's field widths and the OCP
    reading: bias 2^(E-1)-1; E4M3 has no infinities and S.1111.111 is NaN; E5M2's all-ones
    exponent is inf (mantissa 0) or NaN.  FNUZ reading: bias 2^(E-1), no infinities, and the
    negative-zero pattern is the only NaN."""
    eb, mb = w["exponent_bits"], w["mantissa_bits"]
    assert w["sign_bits"] + eb + mb == 8
    bias = 2 ** (eb - 1) - 1 if fmt != E4M3FNUZ else 2 ** (eb - 1)
    s = code >> (eb + mb)
    e = (code >> mb) & (2 ** eb - 1)
    m = code & (2 ** mb - 1)
    if fmt == E4M3FNUZ and code == 0x80:
        return "nan"
    if fmt == E4M3 and e == 2 ** eb - 1 and m == 2 ** mb - 1:
        return "nan"
    if fmt == E5M2 and e == 2 ** eb - 1:
        return "nan" if m else ("-inf" if s else "inf")
    if e == 0:
        v = Fraction(m, 2 ** mb) * Fraction(2) ** (1 - bias)
    else:
        v = (1 + Fraction(m, 2 ** mb)) * Fraction(2) ** (e - bias)
    return -v if s else v


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_table_matches_bit_layout(oracle_mod, widths, fmt):
    w = widths[0][fmt]
    table = oracle_mod.fp8_decode_table(fmt)
    for c in range(256):
        exp = closed_form_value(c, w, fmt)
        got = table[c]
        if exp == "nan":
            assert np.isnan(got), (FMT_NAME[fmt], hex(c))
        elif exp in ("inf", "-inf"):
            assert np.isinf(got) and (got > 0) == (exp == "inf"), hex(c)
        else:
            assert np.isfinite(got), (FMT_NAME[fmt], hex(c), got, exp)
            assert Fraction(float(got)) == exp, (FMT_NAME[fmt], hex(c), got, exp)
            if exp == 0:  # signed zero survives
                assert np.signbit(got) == bool(c & 0x80)


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_table_matches_torch(oracle_mod, fmt):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(TORCH_DT[fmt]).to(torch.float64).numpy()
    got = oracle_mod.fp8_decode_table(fmt)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e5m2_is_fp16_top_byte(oracle_mod):
    """Textbook identity: E5M2 shares binary16's sign and 5-bit exponent with bias 15, so code c
    is exactly the binary16 number whose bits are c << 8."""
    codes = np.arange(256, dtype=np.uint16)
    ref = (codes << 8).astype(np.uint16).view(np.float16).astype(np.float64)
    got = oracle_mod.fp8_decode_table(E5M2)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_fnuz_is_half_of_e4m3(oracle_mod):
    """The two E4M3 flavours share the 1/4/3 layout and differ by one in the bias, so every code
    other than the special ones (FN's NaNs 0x7F / 0xFF, FNUZ's NaN 0x80) means exactly half in
    FNUZ of what it means in FN; FNUZ's 0x7F / 0xFF are finite, +-240: the same mantissa one binade
    above 0x77 / 0xF7."""
    fn = oracle_mod.fp8_decode_table(E4M3)
    fz = oracle_mod.fp8_decode_table(E4M3FNUZ)
    special = {0x7F, 0xFF, 0x80}
    for c in range(256):
        if c in special:
            continue
        assert fz[c] == fn[c] / 2, hex(c)
    assert fz[0x7F] == 240.0 and fz[0xFF] == -240.0 and np.isnan(fz[0x80])
    assert fz[0x7F] == 2 * fz[0x77] and fz[0xFF] == 2 * fz[0xF7]


def test_spot_values(oracle_mod):
    t4 = oracle_mod.fp8_decode_table(E4M3)
    t5 = oracle_mod.fp8_decode_table(E5M2)
    assert t4[0x38] == 1.0 and t4[0x7E] == 448.0 and t4[0x08] == 2.0 ** -6 and t4[0x01] == 2.0 ** -9
    assert t4[0x80] == 0.0 and np.signbit(t4[0x80]) and np.isnan(t4[0x7F]) and np.isnan(t4[0xFF])
    assert np.isfinite(t4).sum() == 254  # no infinities, two NaNs
    assert t5[0x3C] == 1.0 and t5[0x7B] == 57344.0 and t5[0x04] == 2.0 ** -14 and t5[0x01] == 2.0 ** -16
    assert t5[0x7C] == np.inf and t5[0xFC] == -np.inf and np.isnan(t5[0x7D])
    tz = oracle_mod.fp8_decode_table(E4M3FNUZ)
    assert tz[0x40] == 1.0 and tz[0x7F] == 240.0 and tz[0x08] == 2.0 ** -7 and tz[0x01] == 2.0 ** -10
    assert tz[0x00] == 0.0 and not np.signbit(tz[0x00]) and np.isnan(tz[0x80])
    assert np.isfinite(tz).sum() == 255 and not np.signbit(tz[np.isfinite(tz) & (tz == 0)]).any()


def test_fp16_to_double_matches_numpy(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle_mod.fp16_to_double(bits)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


# ---------------------------------------------------------------------------------------------
# encoder: brute force over all codes
def _finite_positive_codes(fmt, widths):
    w = widths[0][fmt]
    codes, vals = [], []
    for c in range(128):
        v = closed_form_value(c, w, fmt)
        if isinstance(v, Fraction):
            codes.append(c)
            vals.append(float(v))  # every FP8 value is exact in binary64
    return np.array(codes, np.int64), np.array(vals, np.float64)


def brute_force_encode(fmt, y: np.ndarray, widths) -> np.ndarray:
    """Nearest finite code to each fp32 value y over all codes, ties to the even code (even mantissa
    LSB); NaN -> sign | 0x7F (FNUZ: 0x80); +-inf -> +-max (saturation); FNUZ zero is unsigned.
    Distances are taken in binary64 and every row where that shows a tie is settled again in exact
    rational arithmetic."""
    codes, vals = _finite_positive_codes(fmt, widths)
    y = np.asarray(y, np.float32)
    sign = np.signbit(y).astype(np.int64) << 7
    a = np.abs(y.astype(np.float64))
    out = np.empty(y.shape, np.int64)
    nan = np.isnan(y)
    inf = np.isinf(y)
    fin = ~(nan | inf)
    CH = 8192
    idx_fin = np.nonzero(fin)[0]
    for s in range(0, len(idx_fin), CH):
        ii = idx_fin[s:s + CH]
        d = np.abs(a[ii, None] - vals[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        # rows where binary64 shows several equally near codes are settled in exact rationals
        for r in np.nonzero(cand.sum(axis=1) > 1)[0]:
            ya = Fraction(float(a[ii[r]]))
            dd = [abs(ya - Fraction(float(vv))) for vv in vals]
            best = min(dd)
            cand[r] = [x == best for x in dd]
        # among equally near codes take the even one
        even = cand & ((codes[None, :] & 1) == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        out[ii] = codes[pick]
    out[inf] = codes[np.argmax(vals)]
    if fmt == E4M3FNUZ:
        sign = np.where(out == 0, 0, sign)  # no negative zero
        out[nan] = 0x80
        sign[nan] = 0
    else:
        out[nan] = 0x7F
    return (out | sign).astype(np.uint8)


def _config1_scale():
    from quantized_kv_cache_03_amd import workloads as W
    w = W.WORKLOADS["tiny-e4m3"]
    ctx = W.context_lens(w)
    k, v, _ = W.all_kv_rows(w, ctx)
    return W.kv_scale(w, k, v)


SCALES = [1.0, "tiny", 2.0 ** -7, 3.0, float(np.float32(1.0 / 3.0))]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("scale", SCALES)
def test_encoder_exhaustive_fp16_bruteforce(oracle_mod, widths, fmt, scale):
    s = np.float32(_config1_scale() if scale == "tiny" else scale)
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    with np.errstate(invalid="ignore"):
        y = x.astype(np.float32) / s  # IEEE binary32 division, round to nearest even
    exp = brute_force_encode(fmt, y, widths)
    got = oracle_mod.fp8_quantize(fmt, x, float(s))
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, [(hex(int(x.view(np.uint16)[i])), float(y[i]), hex(got[i]), hex(exp[i]))
                           for i in bad[:8]]


@pytest.mark.parametrize("fmt", FMTS)
def test_encoder_direct_fp32_edges(oracle_mod, widths, fmt):
    """fp32 values next to every rounding midpoint, subnormal boundary and the saturation
    threshold, plus signed zeros, fp32 subnormals, inf and NaN."""
    codes, vals = _finite_positive_codes(fmt, widths)
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids, [vals[-1] * 1.0625, vals[-1] * 1.125, 1e30, 2.0 ** -140,
                                       2.0 ** -149, 0.0]]).astype(np.float32)
    ups = np.nextafter(pts, np.float32(np.inf))
    dns = np.nextafter(pts, np.float32(0))
    y = np.concatenate([pts, ups, dns])
    y = np.concatenate([y, -y, np.array([np.inf, -np.inf, np.nan, -np.nan], np.float32)])
    exp = brute_force_encode(fmt, y, widths)
    got = oracle_mod.fp8_encode(fmt, y)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, [(float(y[i]), hex(got[i]), hex(exp[i])) for i in bad[:8]]


@pytest.mark.parametrize("fmt", FMTS)
def test_encoder_matches_torch_cast_without_overflow(oracle_mod, fmt):
    """torch's CPU cast rounds to nearest even but does not saturate, so compare only where
    |y| stays below the overflow threshold (E4M3 464, E5M2 61440, E4M3FNUZ 248) and y is not NaN."""
    thr = {E4M3: 464.0, E5M2: 61440.0, E4M3FNUZ: 248.0}[fmt]
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    for s in [1.0, 2.0 ** -7, 3.0, float(np.float32(0.1))]:
        y = x.astype(np.float32) / np.float32(s)
        ok = np.abs(y) < thr
        ref = torch.from_numpy(y[ok]).to(TORCH_DT[fmt]).view(torch.uint8).numpy()
        got = oracle_mod.fp8_encode(fmt, y[ok])
        np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_decode_roundtrip(oracle_mod, fmt):
    """Every FP8 value is exact in fp16, so enc(dec(c)) == c at scale 1 for every non-NaN code."""
    table = oracle_mod.fp8_decode_table(fmt)
    codes = np.array([c for c in range(256) if not np.isnan(table[c]) and not np.isinf(table[c])])
    x = table[codes].astype(np.float16)
    assert np.all(x.astype(np.float64) == table[codes])
    got = oracle_mod.fp8_quantize(fmt, x, 1.0)
    np.testing.assert_array_equal(got, codes.astype(np.uint8))


def test_e5m2_unit_scale_closed_form(oracle_mod):
    """At scale 1.0 an fp16 value rounds to E5M2 by rounding its low byte away, ties to even:
    r = (h + 0x7F + ((h >> 8) & 1)) >> 8 on the magnitude bits h, saturated to 0x7B."""
    bits = np.arange(65536, dtype=np.uint32)
    sign = (bits >> 15) & 1
    h = bits & 0x7FFF
    r = (h + 0x7F + ((h >> 8) & 1)) >> 8
    r = np.where(r >= 0x7C, 0x7B, r)
    r = np.where(h > 0x7C00, 0x7F, r)           # NaN inputs
    r = np.where(h == 0x7C00, 0x7B, r)          # +-inf saturates
    exp = (r | (sign << 7)).astype(np.uint8)
    got = oracle_mod.fp8_quantize(E5M2, bits.astype(np.uint16), 1.0)
    np.testing.assert_array_equal(got, exp)


@pytest.mark.parametrize("fmt", FMTS)
def test_default_scale_is_one(oracle_mod, golden_dir, fmt):
    """The page's default scale is 1.0: quantizing with it equals quantizing the raw value."""
    with open(os.path.join(golden_dir, "fp8_formats.json")) as f:
        default = json.load(f)["default_scale"]["value"]
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    a = oracle_mod.fp8_quantize(fmt, x, default)
    b = oracle_mod.fp8_encode(fmt, x.astype(np.float32))
    np.testing.assert_array_equal(a, b)
