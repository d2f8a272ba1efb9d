"""Outlier-heavy rows (a few channels per KV head scaled by 200) on every kernel family, decode and
prefill, against the oracle.

Such rows are the regime the pages name as the reason for better KV quantization ("[Feature]
TurboMind support W8A8 or FP8 KV Cache", last reply: more advanced INT8 / INT4 quantization; "[QST]
Scale factors and benchmarks", the kv4 reply: channel reordering and smoothing).  With gain 200 the
logits are sums of terms in the thousands whose softmax is sharply peaked, and V rows reach +-800:
a logit error as small as fp32 rounding of those sums moves outputs past the plain gate, for any
implementation that sums in fp32 (the data's conditioning, not a kernel defect).  So the gate here
is widened by a derived bound of that rounding carried through the softmax (gpu_common.fp32_slack:
2^-16 sm_scale sum_d |q_d| w_td per logit), and for FP8 math by the FP8 instruction's accumulation
bound (gpu_common.fp8_math_slack) instead.  Every cache byte is compared bit for bit as everywhere.

The INT4 cases are also held to the plain gate.  Their kernels give the matrix cores each token's
codes centred at its own zero code, as exact binary16 integers (kvq_int4.h); with the codes as
fp16 subnormals and the logit factored as s (q . c) + zp sum q, rows like these once missed the
plain gate by up to 29 times while a float32 evaluation of the same codes met it.

Each case prints the worst element's share of the widened gate and of the plain gate.
"""
import numpy as np
import pytest

import oracle
from gpu_common import (ATOL, RTOL, OracleTwin, assert_attn_close, assert_attn_close_slack, assert_cache_bytes_equal,
                        attn_stats, fp32_attention, fp32_slack, fp8_math_slack, say)

pytestmark = pytest.mark.gpu

BASES = {"fp8_e4m3": "llama2-7b-mha-e4m3", "fp8_e5m2": "llama3-8b-gqa-e5m2", "int8": "llama2-13b-mha-int8",
         "fp8_e4m3fnuz": "llama2-7b-mha-e4m3fnuz", "int4": "llama2-7b-mha-int4"}
GAIN = 200.0


@pytest.fixture(scope="module")
def H():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from quantized_kv_cache_03_amd import harness
    return harness


def _workload(dtype, G, Hkv, ctx, outliers, seed, **kw):
    from quantized_kv_cache_03_amd import workloads as W
    base = W.WORKLOADS[BASES[dtype]]
    return base.scaled(name=f"outliers-{dtype}-G{G}x{Hkv}-o{outliers}", seed=seed, batch=len(ctx),
                       context=("list", list(ctx)), num_q_heads=G * Hkv, num_kv_heads=Hkv, outliers=outliers,
                       outlier_gain=GAIN, **kw)


def _plain(x, ref):
    return float((np.abs(x.astype(np.float64) - ref) / (ATOL + RTOL * np.abs(ref))).max(initial=0))


def _report(tag, gpu, ref, slack, f32, plain=False):
    """Assert the widened gate (and the plain one when `plain`); print the plain gate's share for the
    kernel and for a plain float32 evaluation of the same codes (the data's conditioning)."""
    if plain:
        assert_attn_close(gpu, ref, tag)
    share = assert_attn_close_slack(gpu, ref, slack, tag)
    say(f"    widened gate share {share:.3f}; plain gate share: kernel {_plain(gpu, ref):.3f}, float32 "
        f"evaluation {_plain(f32, ref):.3f}; {attn_stats(gpu, ref)}")


# two outlier channels under the balanced split, eight under 64-token partitions
DECODE = [(dt, G, o, -1 if o == 2 else 64, f8) for dt in BASES for G in (1, 4, 10) for o in (2, 8)
          for f8 in ((False, True) if dt in ("fp8_e4m3", "fp8_e5m2") else (False,))]


@pytest.mark.parametrize("dtype,G,outliers,partition,fp8_math", DECODE,
                         ids=[f"{d}-G{g}-o{o}-p{p}{'-fp8math' if f else ''}" for d, g, o, p, f in DECODE])
def test_outlier_decode(H, dtype, G, outliers, partition, fp8_math):
    ctx = [1, 17, 300, 1100, 64]
    seed = 4000 + 10 * G + outliers + (1 if partition > 0 else 0)
    w = _workload(dtype, G, 2, ctx, outliers, seed, partition_size=partition, fp8_math=fp8_math)
    say(f"[outliers] decode {w.name} partition={partition} fp8_math={fp8_math}")
    case = H.DeviceCase(w, keep_host_rows=True, spare_blocks=1, prefill_last=False)
    out = case.step().cpu().numpy()
    twin = OracleTwin(case, range(case.B))
    assert_cache_bytes_equal(case, twin, w.name)
    ref = twin.attention(fp8_math=fp8_math)
    qe = None
    if fp8_math:
        slack = fp8_math_slack(twin.cache, twin.q, twin.bt, twin.ctx)
        codes, sc = oracle.quantize_q_fp8_rows(twin.q)
        qe = oracle.fp8_decode(oracle.E4M3, codes) * sc[..., None]
    else:
        slack = fp32_slack(twin.cache, twin.q, twin.bt, twin.ctx)
    _report(w.name, out, ref, slack, fp32_attention(twin.cache, twin.q, twin.bt, twin.ctx, q_eff=qe),
            plain=dtype == "int4")


PREFILL = [(dt, G, o, f8) for dt in BASES for G in (1, 4, 10) for o in (2, 8)
           for f8 in ((False, True) if dt in ("fp8_e4m3", "fp8_e5m2") else (False,))]


@pytest.mark.parametrize("dtype,G,outliers,fp8_math", PREFILL,
                         ids=[f"{d}-G{g}-o{o}{'-fp8math' if f else ''}" for d, g, o, f in PREFILL])
def test_outlier_prefill(H, dtype, G, outliers, fp8_math):
    import torch
    from quantized_kv_cache_03_amd import kvq as K
    ctx = [700, 45, 160]
    nq = [120, 45, 33]
    seed = 5000 + 10 * G + outliers
    w = _workload(dtype, G, 2, ctx, outliers, seed, fp8_math=fp8_math)
    say(f"[outliers] prefill {w.name} rows={nq} fp8_math={fp8_math}")
    case = H.DeviceCase(w, keep_host_rows=True, spare_blocks=1)
    cu_q = np.zeros(len(nq) + 1, np.int32)
    cu_q[1:] = np.cumsum(nq)
    q = np.random.default_rng(seed).standard_normal((int(cu_q[-1]), w.num_q_heads, 128),
                                                    dtype=np.float32).astype(np.float16)
    fn = K.paged_prefill_attn_fp8math if fp8_math else K.paged_prefill_attn
    out = fn(case.cache, torch.from_numpy(q).cuda(), torch.from_numpy(cu_q).cuda(), case.bt_d, case.ctx_d,
             case.max_ctx, max(nq)).cpu().numpy()
    twin = OracleTwin(case, range(case.B))
    ref = oracle.prefill_attn(twin.cache, q, twin.bt, twin.ctx, cu_q, threads=8, fp8_math=fp8_math)
    qe = None
    if fp8_math:
        slack = fp8_math_slack(twin.cache, q, twin.bt, twin.ctx, cu_q)
        codes, sc = oracle.quantize_q_fp8_rows(q)
        qe = oracle.fp8_decode(oracle.E4M3, codes) * sc[..., None]
    else:
        slack = fp32_slack(twin.cache, q, twin.bt, twin.ctx, cu_q)
    _report(w.name, out, ref, slack, fp32_attention(twin.cache, q, twin.bt, twin.ctx, cu_q, q_eff=qe),
            plain=dtype == "int4")
