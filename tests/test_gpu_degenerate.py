"""GPU parity at the degenerate ends of the attention's arguments: any finite sm_scale is valid
(0 gives a uniform softmax, a negative one reverses the order of the logits, a large one makes the
softmax nearly one-hot), and an all-zero query gives the mean of the value rows.  Every kernel
family is covered: one query head per KV head and grouped heads, the 8-bit and INT4 caches, FP8
math, and prefill.  Each output is compared with the oracle on the same codes, within the gate.
"""
import numpy as np
import pytest

import oracle
from gpu_common import OracleTwin, assert_attn_close, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from quantized_kv_cache_03_amd import harness
    return harness


CASES = [
    ("llama2-7b-mha-e4m3", {"num_q_heads": 4, "num_kv_heads": 4}, False),
    ("llama3-8b-gqa-e5m2", {"num_q_heads": 8, "num_kv_heads": 2}, False),
    ("llama2-13b-mha-int8", {"num_q_heads": 2, "num_kv_heads": 2}, False),
    ("llama2-7b-mha-int4", {"num_q_heads": 2, "num_kv_heads": 2}, False),
    ("llama3-8b-gqa-int4", {"num_q_heads": 8, "num_kv_heads": 2}, False),
    ("llama3-70b-gqa-e4m3-32k", {"num_q_heads": 8, "num_kv_heads": 1}, True),
]
SCALES = [0.0, -0.3, 2.5]


@pytest.mark.parametrize("name,kw,fp8_math", CASES, ids=[f"{c[0]}{'-fp8math' if c[2] else ''}" for c in CASES])
@pytest.mark.parametrize("partition", [-1, 64])
def test_decode_extreme_sm_scale(H, name, kw, fp8_math, partition):
    from quantized_kv_cache_03_amd import kvq as K
    from quantized_kv_cache_03_amd import workloads as W
    base = W.WORKLOADS[name]
    w = base.scaled(name=f"{name}-degenerate", seed=500 + base.seed, batch=3,
                    context=("list", [700, 33, 1]), partition_size=partition, **kw)
    case = H.DeviceCase(w, keep_host_rows=True, spare_blocks=1)
    twin = OracleTwin(case, range(case.B))
    fn = K.paged_decode_attn_fp8math if fp8_math else K.paged_decode_attn
    for sm in SCALES:
        say(f"[degenerate] {w.name} {w.dtype} partition={partition} fp8_math={fp8_math} sm_scale={sm}")
        out = fn(case.cache, case.q_d, case.bt_d, case.ctx_d, case.max_ctx, sm_scale=sm,
                 partition_size=partition).cpu().numpy()
        ref = oracle.decode_attn(twin.cache, twin.q, twin.bt, twin.ctx, sm_scale=sm, threads=8,
                                 fp8_math=fp8_math)
        assert_attn_close(out, ref, f"{w.name} sm_scale={sm}")
    # an all-zero query: the mean of the dequantized value rows
    import torch
    q0 = torch.zeros_like(case.q_d)
    out = fn(case.cache, q0, case.bt_d, case.ctx_d, case.max_ctx, partition_size=partition).cpu().numpy()
    ref = oracle.decode_attn(twin.cache, np.zeros_like(twin.q), twin.bt, twin.ctx, threads=8,
                             fp8_math=fp8_math)
    assert_attn_close(out, ref, f"{w.name} zero query")


@pytest.mark.parametrize("name,kw,fp8_math", [CASES[0], CASES[1], CASES[4], CASES[5]],
                         ids=["7b-mha-e4m3", "8b-gqa-e5m2", "8b-gqa-int4", "70b-gqa-fp8math"])
def test_prefill_extreme_sm_scale(H, name, kw, fp8_math):
    import torch
    from quantized_kv_cache_03_amd import kvq as K
    from quantized_kv_cache_03_amd import workloads as W
    base = W.WORKLOADS[name]
    ctx, nq = [300, 40], [70, 40]
    w = base.scaled(name=f"{name}-degenerate-prefill", seed=600 + base.seed, batch=2,
                    context=("list", ctx), **kw)
    case = H.DeviceCase(w, keep_host_rows=True, spare_blocks=1)
    cu_q = np.array([0, nq[0], nq[0] + nq[1]], np.int32)
    q = np.random.default_rng(3).standard_normal((int(cu_q[-1]), w.num_q_heads, 128),
                                                 dtype=np.float32).astype(np.float16)
    q_d, cu_d = torch.from_numpy(q).cuda(), torch.from_numpy(cu_q).cuda()
    twin = OracleTwin(case, range(case.B))
    fn = K.paged_prefill_attn_fp8math if fp8_math else K.paged_prefill_attn
    for sm in SCALES:
        say(f"[degenerate prefill] {w.name} {w.dtype} fp8_math={fp8_math} sm_scale={sm}")
        out = fn(case.cache, q_d, cu_d, case.bt_d, case.ctx_d, case.max_ctx, max(nq), sm_scale=sm).cpu().numpy()
        ref = oracle.prefill_attn(twin.cache, q, twin.bt, twin.ctx, cu_q, sm_scale=sm, threads=8,
                                  fp8_math=fp8_math)
        assert_attn_close(out, ref, f"{w.name} prefill sm_scale={sm}")
