"""The oracle's pins catch plausible mistakes.

Each case copies the oracle's C source, plants one mistake (a wrong bias, a dropped term, a
transposed layout, a wrong index, a rounding mode), builds it with gcc into a temporary directory
and runs a set of the pins against it; at least one pin must fail.  Everything here runs on the
CPU; the shipped oracle is never modified.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import build as obuild

import test_oracle_attention as TA
import test_oracle_codec as TC
import test_oracle_fp8q as TQ
import test_oracle_int4 as T4
import test_oracle_int8 as TI

MUTATIONS = {
    "decode-exponent-off-by-one": (
        "v = ldexp((double)((1 << F.mbits) + m), e - F.bias - F.mbits);",
        "v = ldexp((double)((1 << F.mbits) + m), e - F.bias - F.mbits + 1);"),
    "encode-round-half-up": (
        "double M = nearbyint((ldexp(a, -e) - 1.0) * (double)(1 << F.mbits));",
        "double M = floor(0.5 + (ldexp(a, -e) - 1.0) * (double)(1 << F.mbits));"),
    "encode-no-saturation": (
        "        a = F.max_finite;                       /* saturation, also for +-inf */",
        "        a = a;"),
    "encode-subnormal-step": (
        "double M = nearbyint(ldexp(a, F.bias - 1 + F.mbits));",
        "double M = nearbyint(ldexp(a, F.bias + F.mbits));"),
    "encode-drops-sign": (
        "uint8_t sign = signbit(y) ? 0x80 : 0x00;",
        "uint8_t sign = 0x00;"),
    "e4m3-nan-code-finite": (
        "if (fmt == KVQO_E4M3 && e == 15 && m == 7)",
        "if (fmt == KVQO_E4M3 && e == 16)"),
    "fp16-exponent-bias": (
        "v = ldexp((double)(1024 + f), e - 25);",
        "v = ldexp((double)(1024 + f), e - 24);"),
    "int8-scale-128": (
        "float s = amax / 127.0f;",
        "float s = amax / 128.0f;"),
    "int8-v-uses-k-scale": (
        "return (double)(int8_t)c * (double)vs[s_off8(Hkv, blk, g, t)];",
        "return (double)(int8_t)c * (double)vs[s_off8(Hkv, blk, g, 0)];"),
    "int8-scale-rows-of-16": (
        "return ((size_t)blk * Hkv + g) * (2 * KVQO_BLOCK) + t;",
        "return ((size_t)blk * Hkv + g) * KVQO_BLOCK + t;"),
    "attn-drops-sm-scale": (
        "z[t] = (double)sm_scale * acc;\n        if (z[t] > zmax)\n            zmax = z[t];\n    }\n    double denom = 0.0;\n    for (int t = 0; t < n; ++t) {\n        double w = exp(z[t] - zmax);\n        int blk",
        "z[t] = acc;\n        if (z[t] > zmax)\n            zmax = z[t];\n    }\n    double denom = 0.0;\n    for (int t = 0; t < n; ++t) {\n        double w = exp(z[t] - zmax);\n        int blk"),
    "attn-gqa-index": (
        "int g = h / G;",
        "int g = h % Hkv;"),
    "attn-denominator": (
        "        out[d] /= denom;\n    free(z);\n    return 0;\n}\n\n/* The same attention",
        "        out[d] /= (denom + 1.0);\n    free(z);\n    return 0;\n}\n\n/* The same attention"),
    "k-layout-token-major": (
        "return tile + (size_t)(d / 16) * (16 * KVQO_BLOCK) + (size_t)t * 16 + (size_t)(d % 16);",
        "return tile + (size_t)t * KVQO_DIM + (size_t)d;"),
    "v-layout-token-major": (
        "return (((size_t)blk * Hkv + g) * KVQO_DIM + d) * KVQO_BLOCK + t;",
        "return (((size_t)blk * Hkv + g) * KVQO_BLOCK + t) * KVQO_DIM + d;"),
    "fnuz-bias-7": (
        "out->ebits = 4; out->mbits = 3; out->bias = 8;",
        "out->ebits = 4; out->mbits = 3; out->bias = 7;"),
    "fnuz-keeps-negative-zero": (
        "    if (fmt == KVQO_E4M3FNUZ && mag == 0)\n        return 0x00;",
        "    if (fmt == KVQO_E4M3FNUZ && mag == 0 && !sign)\n        return 0x00;"),
    "fnuz-nan-as-fn": (
        "return (uint8_t)(fmt == KVQO_E4M3FNUZ ? 0x80 : (sign | 0x7F));",
        "return (uint8_t)(sign | 0x7F);"),
    "fnuz-top-code-nan": (
        "    else if (fmt == KVQO_E4M3FNUZ && code == 0x80)\n        v = NAN;",
        "    else if (fmt == KVQO_E4M3FNUZ && (code & 0x7F) == 0x7F)\n        v = NAN;"),
    "int4-divide-16": (
        "float s = range / 15.0f;",
        "float s = range / 16.0f;"),
    "int4-zero-point-max": (
        "*zp_out = mn;",
        "*zp_out = mx;"),
    "int4-k-nibble-offset": (
        "return tile + (size_t)(d / 32) * (16 * KVQO_BLOCK) + (size_t)t * 16 + (size_t)((d % 32) / 2);",
        "return tile + (size_t)(d / 32) * (16 * KVQO_BLOCK) + (size_t)t * 16 + (size_t)((d % 32) % 16);"),
    "int4-v-token-major": (
        "return tile + (size_t)(t / 4) * 256 + (size_t)(d % 16) * 16 + (size_t)(d / 16) * 2 + (size_t)((t % 4) / 2);",
        "return tile + (size_t)t * (KVQO_DIM / 2) + (size_t)(d / 2);"),
    "int4-v-dim-blocks-swapped": (
        "return tile + (size_t)(t / 4) * 256 + (size_t)(d % 16) * 16 + (size_t)(d / 16) * 2 + (size_t)((t % 4) / 2);",
        "return tile + (size_t)(t / 4) * 256 + (size_t)(d / 8) * 16 + (size_t)(d % 8) * 2 + (size_t)((t % 4) / 2);"),
    "int4-dequant-drops-zero-point": (
        "return (double)get_nibble(codes, off, hi) * (double)sz[2 * so] + (double)sz[2 * so + 1];",
        "return (double)get_nibble(codes, off, hi) * (double)sz[2 * so];"),
    "fp8q-scale-240": (
        "float s = amax > 0.0f ? amax / 448.0f : 1.0f;",
        "float s = amax > 0.0f ? amax / 240.0f : 1.0f;"),
    "fp8q-encodes-e5m2": (
        "codes[d] = kvqo_fp8_encode(KVQO_E4M3, (float)kvqo_fp16_to_double(q[d]) / s);",
        "codes[d] = kvqo_fp8_encode(KVQO_E5M2, (float)kvqo_fp16_to_double(q[d]) / s);"),
    "fp8q-dequant-drops-scale": (
        "qd[d] = kvqo_fp8_decode(KVQO_E4M3, codes[d]) * (double)s;",
        "qd[d] = kvqo_fp8_decode(KVQO_E4M3, codes[d]);"),
    "fp8q-signed-max": (
        "        float v = fabsf((float)kvqo_fp16_to_double(q[d]));",
        "        float v = (float)kvqo_fp16_to_double(q[d]);"),
    "append-position-reversed": (
        "int p = context_lens[b] - n_b + j;",
        "int p = context_lens[b] - 1 - j;"),
}


def _pins():
    w = None

    def widths():
        nonlocal w
        if w is None:
            import json
            here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fp8_formats.json")
            with open(here) as f:
                g = json.load(f)
            w = ({TC.E4M3: g["formats"]["E4M3"], TC.E5M2: g["formats"]["E5M2"],
                  TC.E4M3FNUZ: g["formats"]["E4M3FNUZ"]}, g)
        return w

    o = oracle
    return [
        lambda: TC.test_decode_table_matches_bit_layout(o, widths(), TC.E4M3),
        lambda: TC.test_decode_table_matches_bit_layout(o, widths(), TC.E5M2),
        lambda: TC.test_fp16_to_double_matches_numpy(o),
        lambda: TC.test_encoder_exhaustive_fp16_bruteforce(o, widths(), TC.E4M3, 3.0),
        lambda: TC.test_encoder_exhaustive_fp16_bruteforce(o, widths(), TC.E5M2, 2.0 ** -7),
        lambda: TC.test_encoder_direct_fp32_edges(o, widths(), TC.E4M3),
        lambda: TC.test_encoder_direct_fp32_edges(o, widths(), TC.E5M2),
        lambda: TC.test_decode_table_matches_bit_layout(o, widths(), TC.E4M3FNUZ),
        lambda: TC.test_encoder_direct_fp32_edges(o, widths(), TC.E4M3FNUZ),
        lambda: TI.test_int8_matches_numpy_rint(o, True),
        lambda: TI.test_int8_zero_row_and_ties(o),
        lambda: TA.test_append_layout_and_poison(o, TA.INT8),
        lambda: TA.test_dequant_matches_independent_decode(o, TA.INT8),
        lambda: TA.test_attention_matches_torch_sdpa_float64(o, TA.E4M3, 8, 2),
        lambda: TA.test_attention_matches_torch_sdpa_float64(o, TA.INT8, 2, 2),
        lambda: T4.test_int4_matches_numpy(o, "normal"),
        lambda: T4.test_int4_append_layout_and_poison(o),
        lambda: TA.test_dequant_matches_independent_decode(o, TA.INT4),
        lambda: TQ.test_q_scale_matches_float32(o, "outliers"),
        lambda: TQ.test_q_error_within_half_step(o, "wide"),
        lambda: TQ.test_fp8_attention_matches_independent_softmax(o, 1, 8, 2),
    ]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    with open(obuild.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found once in the oracle"
    mut = tmp_path / "kvq_oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", *obuild.CFLAGS, "-w", str(mut), "-o", str(lib), "-lm"], check=True)
    saved = oracle._lib
    oracle._lib = oracle.load(str(lib))
    failed = []
    try:
        for i, pin in enumerate(_pins()):
            try:
                with np.errstate(all="ignore"):
                    pin()
            except AssertionError:
                failed.append(i)
                break
    finally:
        oracle._lib = saved
    assert failed, f"no pin caught the planted mistake {name!r}"
