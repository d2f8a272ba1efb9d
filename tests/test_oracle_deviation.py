"""How far each cache format moves attention away from the unquantized fp16 attention: a report,
not a gate.

The pages judge the formats by model accuracy ("Accelerating Inference with FP8 KV Cache": FP8
keeps accuracy; "[Feature] TurboMind support W8A8 or FP8 KV Cache": FP8 more precise than INT8,
its INT8 accuracy table), which needs trained weights and evaluation suites that are not here:
these numbers are parity unpinned.  What is computed: on seeded synthetic rows (N(0,1), and the
same with 4 channels per KV head scaled by 20), the oracle's attention over each format's codes
against the oracle's attention over the original fp16 rows, per output element -- max abs, max
rel (where the reference is at least 0.1) and RMS.  `pytest -s` prints the table.  The asserts are
orderings the formats' resolution makes expected and that hold here with a wide margin: one
mantissa bit fewer (E5M2 against E4M3: about 2x) or sixteen levels instead of 255 (INT4 against
INT8: about 15x) gives a larger RMS deviation; on the N(0,1) rows, quantizing the query as well
(FP8 math) adds to the E4M3 cache's own.  With the outlier channels the logits are large and the
softmax so peaked that the FP8-math deviation is not ordered against the cache's alone.
"""
import numpy as np
import pytest

from quantized_kv_cache_03_amd import workloads as W

E4M3, E5M2, INT8, E4M3FNUZ, INT4 = 1, 2, 3, 4, 5

# (label, format, per-tensor scale rule, FP8 math)
FORMATS = [("fp8_e4m3", E4M3, "amax/448", False), ("fp8_e5m2", E5M2, "one", False),
           ("int8", INT8, "one", False), ("fp8_e4m3fnuz", E4M3FNUZ, "amax/240", False),
           ("int4", INT4, "one", False), ("fp8_e4m3 + FP8 math", E4M3, "amax/448", True)]


def _deviation(oracle_mod, outliers: int):
    w = W.Workload("deviation", 77, 4, 4, 4, "fp8_e4m3", ("list", [40, 300, 517, 1024]),
                   outliers=outliers)
    ctx = W.context_lens(w)
    bt, nb = W.block_tables(w, ctx)
    k, v, cu = W.all_kv_rows(w, ctx)
    q = W.query(w)
    sm = float(np.float32(1.0 / np.sqrt(128.0)))
    dense = np.empty((w.batch, w.num_q_heads, 128))
    for b in range(w.batch):
        for h in range(w.num_q_heads):
            dense[b, h] = oracle_mod.attn_fp16_dense(q[b, h], k[cu[b]:cu[b + 1], h], v[cu[b]:cu[b + 1], h], sm)
    rows = {}
    for label, fmt, rule, fp8_math in FORMATS:
        scale = W.kv_scale(w.scaled(scale_rule=rule), k, v) if rule != "one" else 1.0
        cache = oracle_mod.Cache(fmt, nb, w.num_kv_heads, scale)
        oracle_mod.append(cache, k, v, bt, ctx, cu)
        got = oracle_mod.decode_attn(cache, q, bt, ctx, sm_scale=sm, fp8_math=fp8_math)
        d = np.abs(got - dense)
        big = np.abs(dense) >= 0.1
        rows[label] = {"max_abs": float(d.max()), "max_rel": float((d[big] / np.abs(dense[big])).max()),
                       "rms": float(np.sqrt(np.mean(d ** 2)))}
    return rows


@pytest.mark.parametrize("outliers", [0, 4])
def test_quantization_deviation_report(oracle_mod, outliers):
    rows = _deviation(oracle_mod, outliers)
    print(f"\nattention over the codes vs over fp16 rows ({'N(0,1)' if not outliers else 'N(0,1), 4 channels x20'})")
    print(f"{'format':22s} {'max abs':>10s} {'max rel':>10s} {'rms':>10s}")
    for label, r in rows.items():
        print(f"{label:22s} {r['max_abs']:10.3e} {r['max_rel']:10.3e} {r['rms']:10.3e}")
    for r in rows.values():
        assert all(np.isfinite(x) for x in r.values())
    assert rows["fp8_e5m2"]["rms"] > rows["fp8_e4m3"]["rms"]
    assert rows["int4"]["rms"] > rows["int8"]["rms"]
    if not outliers:
        assert rows["fp8_e4m3 + FP8 math"]["rms"] > rows["fp8_e4m3"]["rms"]
