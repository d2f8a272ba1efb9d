"""The kernel-timing hook (kvq_timing_begin / kvq_timing_end) keeps its session per thread: a
session opened on one thread times only that thread's attention calls, another thread sees no
session and its calls run untimed, and the results of the timed and untimed calls are the same."""
import threading

import numpy as np
import pytest

from gpu_common import say

pytestmark = pytest.mark.gpu


def test_timing_session_is_per_thread():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from quantized_kv_cache_03_amd import harness as H
    from quantized_kv_cache_03_amd import kvq as K
    from quantized_kv_cache_03_amd import workloads as W
    w = W.WORKLOADS["llama3-8b-gqa-e5m2"].scaled(name="timing-threads", seed=77, batch=3,
                                                  context=("list", [300, 17, 64]))
    say(f"[timing] {w.name}")
    case = H.DeviceCase(w)
    ref = case.attention().clone()
    torch.cuda.synchronize()

    got = {}

    def other():
        # no session on this thread: kvq_timing_end fails, and its attention call runs untimed
        try:
            K.timing_end()
            got["end"] = "returned"
        except RuntimeError as e:
            got["end"] = str(e)
        got["out"] = case.attention(out=torch.empty_like(ref)).clone()
        torch.cuda.synchronize()

    K.timing_begin(4)
    try:
        t = threading.Thread(target=other)
        t.start()
        t.join()
        out = case.attention(out=torch.empty_like(ref)).clone()
    finally:
        ms, n = K.timing_end()
    say(f"  other thread's kvq_timing_end: {got['end']}; this thread's session: {n} launch, {ms:.4f} ms")
    assert "no timing session" in got["end"]
    assert n == 1 and ms > 0.0
    np.testing.assert_array_equal(got["out"].cpu().numpy(), ref.cpu().numpy())
    np.testing.assert_array_equal(out.cpu().numpy(), ref.cpu().numpy())
