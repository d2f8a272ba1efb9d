"""Host checks of the Python binding (no GPU): tensors that would send a kernel to the wrong
addresses -- host memory, strided views, a cache whose tensors break the documented layout -- are
refused with ValueError before the library is called."""
import pytest
import torch

from quantized_kv_cache_03_amd import kvq as K


def test_host_tensor_is_refused():
    with pytest.raises(ValueError, match="GPU memory"):
        K._ptr(torch.zeros(4, dtype=torch.float16))
    assert K._ptr(None) is None


def test_cache_on_the_host_is_refused():
    c = K.PagedKVCache.allocate("fp8_e4m3", 2, 1, 1.0, device="cpu")
    with pytest.raises(ValueError, match="GPU memory"):
        c.descriptor()
    with pytest.raises(ValueError, match="GPU memory"):
        K.append(c, torch.zeros(1, 1, 128, dtype=torch.float16), torch.zeros(1, 1, 128, dtype=torch.float16),
                 torch.zeros(1, 1, dtype=torch.int32), torch.ones(1, dtype=torch.int32))


def test_int_caches_need_their_scales():
    c = K.PagedKVCache.allocate("int8", 2, 1, 1.0, device="cpu")
    c2 = K.PagedKVCache(c.dtype, c.k_cache, c.v_cache, None, c.v_scale, 1.0)
    with pytest.raises(ValueError, match="k_scale is required"):
        c2.descriptor()
