"""GPU parity for every head grouping G = Hq / Hkv from 1 to 16.

The grouped-head kernels pad the G query heads of a KV head to 16 matrix-core columns, and the
prefill kernels place 16 / G query rows of G heads in each block of 16 columns (R = floor(16 / G),
so G = 5, 6, 7, 9 .. 15 leave padding columns in every block).  Each case runs on a small ragged
batch and compares every output with the oracle: the fused decode step (E4M3 and INT4 caches),
FP8 math, and prefill (E4M3 and INT4).
"""
import numpy as np
import pytest

import oracle
from gpu_common import OracleTwin, assert_attn_close, assert_cache_bytes_equal, say

pytestmark = pytest.mark.gpu

GROUPS = list(range(1, 17))


@pytest.fixture(scope="module")
def H():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from quantized_kv_cache_03_amd import harness
    return harness


def _w(name, G, ctx, **kw):
    from quantized_kv_cache_03_amd import workloads as W
    base = W.WORKLOADS[name]
    Hkv = 2 if G <= 8 else 1
    return base.scaled(name=f"{name}-G{G}", seed=900 + base.seed + G, batch=len(ctx), context=("list", ctx),
                       num_q_heads=G * Hkv, num_kv_heads=Hkv, **kw)


@pytest.mark.parametrize("name", ["llama3-70b-gqa-e4m3-32k", "llama3-8b-gqa-int4"])
@pytest.mark.parametrize("G", GROUPS)
def test_decode_step_every_grouping(H, name, G):
    w = _w(name, G, [300, 37, 1], partition_size=-1)
    say(f"[groups] decode {w.name} {w.dtype} Hq={w.num_q_heads} Hkv={w.num_kv_heads}")
    case = H.DeviceCase(w, keep_host_rows=True, spare_blocks=1, prefill_last=False)
    out = case.step(fused=True).cpu().numpy()
    twin = OracleTwin(case, range(case.B))
    assert_cache_bytes_equal(case, twin, w.name)
    assert_attn_close(out, twin.attention(), w.name)


@pytest.mark.parametrize("G", GROUPS)
def test_fp8math_every_grouping(H, G):
    w = _w("llama3-8b-gqa-e5m2", G, [300, 37, 1], partition_size=64, fp8_math=True)
    say(f"[groups] fp8 math {w.name} Hq={w.num_q_heads} Hkv={w.num_kv_heads}")
    case = H.DeviceCase(w, keep_host_rows=True, spare_blocks=1)
    out = case.attention().cpu().numpy()
    twin = OracleTwin(case, range(case.B))
    assert_attn_close(out, twin.attention(fp8_math=True), w.name)


@pytest.mark.parametrize("name", ["llama2-7b-mha-e4m3", "llama3-8b-gqa-int4"])
@pytest.mark.parametrize("G", GROUPS)
def test_prefill_every_grouping(H, name, G):
    import torch
    from quantized_kv_cache_03_amd import kvq as K
    ctx, nq = [90, 37], [45, 37]
    w = _w(name, G, ctx)
    say(f"[groups] prefill {w.name} {w.dtype} Hq={w.num_q_heads} Hkv={w.num_kv_heads}")
    case = H.DeviceCase(w, keep_host_rows=True, spare_blocks=1)
    cu_q = np.array([0, nq[0], nq[0] + nq[1]], np.int32)
    q = np.random.default_rng(G).standard_normal((int(cu_q[-1]), w.num_q_heads, 128),
                                                 dtype=np.float32).astype(np.float16)
    out = K.paged_prefill_attn(case.cache, torch.from_numpy(q).cuda(), torch.from_numpy(cu_q).cuda(),
                               case.bt_d, case.ctx_d, case.max_ctx, max(nq)).cpu().numpy()
    twin = OracleTwin(case, range(case.B))
    ref = oracle.prefill_attn(twin.cache, q, twin.bt, twin.ctx, cu_q, threads=8)
    assert_attn_close(out, ref, w.name)
