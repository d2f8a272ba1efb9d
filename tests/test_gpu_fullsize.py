"""The five decode workloads (and the E4M3FNUZ, INT4, FP8-math and 512-token-partition variants)
at full size, in the launch configuration the benchmark times, against the oracle on every output.

Each case fills a fresh device cache through kvq_append with all but each sequence's last token,
runs the fused decode step twice (kvq_decode_step, or its FP8-math twin: append that token, then
split-K attention with the workload's partition size and the merge, as the benchmark times it),
and checks
- the two outputs bitwise equal (the step is deterministic and idempotent);
- every cache byte of every sequence (and every INT8 / INT4 scale) bit for bit against the oracle's
  own append of the same rows;
- every output element of every (sequence, query head) against the oracle's fp64 attention over
  those codes, within the gate |gpu - oracle| <= 1e-3 + 1e-2 |oracle|.

Workloads that share a cache recipe (the same seeds, shapes and format) share one set of host rows
and one oracle cache; each still gets its own device cache.  The worst element's share of the gate
is printed per workload.
"""
import dataclasses

import numpy as np
import pytest

from gpu_common import (ATOL, RTOL, OracleTwin, assert_attn_close, assert_attn_close_slack,
                        assert_cache_bytes_equal, attn_stats, fp8_math_slack, say)

pytestmark = pytest.mark.gpu

# grouped by cache recipe, so that neighbours reuse the rows and the oracle cache
NAMES = ["tiny-e4m3",
         "llama2-7b-mha-e4m3", "llama2-7b-mha-e4m3-fp8math",
         "llama3-8b-gqa-e5m2", "llama3-8b-gqa-e5m2-fp8math",
         "llama2-13b-mha-int8",
         "llama3-70b-gqa-e4m3-32k", "llama3-70b-gqa-e4m3-32k-p512", "llama3-70b-gqa-e4m3-32k-fp8math",
         "llama2-7b-mha-e4m3fnuz", "llama3-70b-gqa-e4m3fnuz-32k",
         "llama2-7b-mha-int4", "llama3-8b-gqa-int4"]
THREADS = 16

_shared = {}  # the one recipe whose rows and oracle cache are held


@pytest.fixture(scope="module", autouse=True)
def _release_shared():
    yield
    _shared.clear()


def _recipe(w):
    return dataclasses.replace(w, name="", partition_size=-1, fp8_math=False)


def _rows_and_twin(w, H, W):
    key = _recipe(w)
    if _shared.get("key") != key:
        _shared.clear()
        ctx = W.context_lens(w)
        rows = W.all_kv_rows(w, ctx, threads=THREADS)
        _shared.update(key=key, rows=rows, twin=None, ref={})
    return _shared


@pytest.mark.parametrize("name", NAMES)
def test_full_size_decode_step(name):
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from quantized_kv_cache_03_amd import harness as H, workloads as W
    w = W.WORKLOADS[name]
    say(f"[full size] {name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} {w.dtype} "
        f"partition={w.partition_size} fp8_math={w.fp8_math}")
    sh = _rows_and_twin(w, H, W)
    case = H.DeviceCase(w, verbose=False, prefill_last=False, rows=sh["rows"])  # the step writes the last token
    say(f"  cache filled: {case.num_blocks} blocks, sum ctx {int(case.ctx.sum())}, kv_scale {case.kv_scale!r}")
    out1 = case.step().clone()
    out2 = case.step().clone()
    torch.cuda.synchronize()
    o1 = out1.cpu().numpy()
    np.testing.assert_array_equal(o1.view(np.uint16), out2.cpu().numpy().view(np.uint16))
    if sh["twin"] is None:
        sh["twin"] = OracleTwin(case, range(case.B), threads=THREADS)
        say("  oracle cache built")
    twin = sh["twin"]
    assert_cache_bytes_equal(case, twin, name)
    say("  every cache byte equal")
    if w.fp8_math not in sh["ref"]:  # one reference per math mode (any work split must meet it)
        sh["ref"][w.fp8_math] = twin.attention(threads=THREADS, fp8_math=w.fp8_math)
    ref = sh["ref"][w.fp8_math]
    empty = case.ctx == 0
    assert np.all(o1[empty] == 0)
    g, r = o1[~empty], ref[~empty]
    if w.fp8_math and np.any(np.abs(g.astype(np.float64) - r) > ATOL + RTOL * np.abs(r)):
        # FP8 math has a tolerance of its own: the gate widened by the FP8 instruction's
        # accumulation error carried through the softmax
        say(f"  FP8 math outside the plain gate ({attn_stats(g, r)}); the widened gate applies")
        slack = fp8_math_slack(twin.cache, twin.q, twin.bt, twin.ctx)
        assert_attn_close_slack(g, r, slack[~empty], name)
        st = attn_stats(g, r)
    else:
        st = assert_attn_close(g, r, name)
    say(f"  every output of {int((~empty).sum()) * w.num_q_heads} (sequence, head) rows within the gate: {st}")
    del case, out1, out2
    torch.cuda.empty_cache()
