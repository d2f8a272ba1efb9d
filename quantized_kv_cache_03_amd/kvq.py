"""Python binding of ``libkvq.so`` (the C ABI in ``include/kvq.h``): argument marshalling only.

Torch supplies device memory and the current HIP stream; every step of the decode path runs in
the library's HIP kernels.  Importing this module loads the library and raises ``ImportError``
if it is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

FP8_E4M3, FP8_E5M2, INT8, FP8_E4M3FNUZ, INT4 = 1, 2, 3, 4, 5
HEAD_DIM = 128
BLOCK_SIZE = 16
DTYPE_NAMES = {"fp8": FP8_E4M3, "fp8_e4m3": FP8_E4M3, "fp8_e5m2": FP8_E5M2, "int8": INT8,
               "fp8_e4m3fnuz": FP8_E4M3FNUZ, "int4": INT4}

OK, ERR_ARG, ERR_DTYPE, ERR_SHAPE, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4, -5

# KVQ_LIBRARY may name another build of the same sources (the host-sanitizer build)
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; "
                      f"g.build()' or python quantized_kv_cache_03_amd/build.py)")


class KvqCache(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("kv_scale", ctypes.c_float),
    ]


_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
lib = ctypes.CDLL(LIB_PATH)
lib.kvq_append.argtypes = [ctypes.POINTER(KvqCache), _vp, _vp, _vp, _i32, _vp, _i32, _vp, _i32, _vp]
lib.kvq_append.restype = ctypes.c_int
lib.kvq_decode_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32]
lib.kvq_decode_workspace_size.restype = _sz
lib.kvq_paged_decode_attn.argtypes = [ctypes.POINTER(KvqCache), _vp, _vp, _i32, _f32, _vp, _i32,
                                      _vp, _i32, _i32, _i32, _vp, _sz, _vp]
lib.kvq_paged_decode_attn.restype = ctypes.c_int
lib.kvq_decode_step.argtypes = [ctypes.POINTER(KvqCache), _vp, _vp, _vp, _vp, _i32, _f32, _vp, _i32,
                                _vp, _i32, _i32, _i32, _vp, _sz, _vp]
lib.kvq_decode_step.restype = ctypes.c_int
lib.kvq_decode_step_noalloc.argtypes = [ctypes.POINTER(KvqCache), _vp, _vp, _vp, _vp, _i32, _f32, _vp, _i32,
                                        _vp, _i32, _i32, _i32, _vp]
lib.kvq_decode_step_noalloc.restype = ctypes.c_int
lib.kvq_paged_prefill_attn.argtypes = [ctypes.POINTER(KvqCache), _vp, _vp, _i32, _f32, _vp, _i32, _i32,
                                       _vp, _i32, _vp, _i32, _i32, _vp]
lib.kvq_paged_prefill_attn.restype = ctypes.c_int
lib.kvq_paged_decode_attn_fp8math.argtypes = lib.kvq_paged_decode_attn.argtypes
lib.kvq_paged_decode_attn_fp8math.restype = ctypes.c_int
lib.kvq_decode_step_fp8math.argtypes = lib.kvq_decode_step.argtypes
lib.kvq_decode_step_fp8math.restype = ctypes.c_int
lib.kvq_paged_prefill_attn_fp8math.argtypes = lib.kvq_paged_prefill_attn.argtypes
lib.kvq_paged_prefill_attn_fp8math.restype = ctypes.c_int
lib.kvq_quantize_q_fp8.argtypes = [_vp, _i32, _vp, _vp, _vp]
lib.kvq_quantize_q_fp8.restype = ctypes.c_int
lib.kvq_dequant.argtypes = [ctypes.POINTER(KvqCache), _vp, _i32, _vp, _i32, _i32, _vp, _vp, _vp]
lib.kvq_dequant.restype = ctypes.c_int
lib.kvq_dtype_from_string.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int)]
lib.kvq_dtype_from_string.restype = ctypes.c_int
lib.kvq_status_string.argtypes = [ctypes.c_int]
lib.kvq_status_string.restype = ctypes.c_char_p
lib.kvq_last_error.argtypes = []
lib.kvq_last_error.restype = ctypes.c_char_p
lib.kvq_timing_begin.argtypes = [_i32]
lib.kvq_timing_begin.restype = ctypes.c_int
lib.kvq_timing_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i32)]
lib.kvq_timing_end.restype = ctypes.c_int
lib.kvq_version.argtypes = []
lib.kvq_version.restype = ctypes.c_char_p

EXPORTS = ["kvq_append", "kvq_decode_workspace_size", "kvq_paged_decode_attn", "kvq_decode_step",
           "kvq_paged_prefill_attn", "kvq_dequant", "kvq_paged_decode_attn_fp8math",
           "kvq_decode_step_fp8math", "kvq_paged_prefill_attn_fp8math", "kvq_quantize_q_fp8",
           "kvq_dtype_from_string", "kvq_status_string", "kvq_last_error", "kvq_timing_begin",
           "kvq_timing_end", "kvq_version", "kvq_decode_step_noalloc"]
NOALLOC_SCRATCH_BYTES = 64 << 20  # KVQ_NOALLOC_SCRATCH_BYTES


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.kvq_last_error().decode(errors="replace")
        super().__init__(f"{where}: {lib.kvq_status_string(status).decode()} ({status}): {msg}")


def _check(status: int, where: str):
    if status != OK:
        raise KvqError(status, where)


def _device_memory(t: torch.Tensor, what: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{what} must be in GPU memory (got a tensor on {t.device})")


def _device_tensor(t: torch.Tensor, what: str) -> None:
    """The library reads and writes device memory in the documented layouts: a host tensor, or a
    strided view, would send a kernel to the wrong addresses."""
    _device_memory(t, what)
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _tensor(t: torch.Tensor, what: str, dtype: torch.dtype, shape=None, device=None) -> None:
    """Check a caller tensor against the layout the library will read or write: GPU memory,
    contiguous, the dtype, the shape (None entries match any extent) and the cache's device."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    _device_tensor(t, what)
    if t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype} (got {t.dtype})")
    if shape is not None and (t.dim() != len(shape) or
                              any(e is not None and t.shape[i] != e for i, e in enumerate(shape))):
        want = "[" + ", ".join("*" if e is None else str(e) for e in shape) + "]"
        raise ValueError(f"{what} must have shape {want} (got {list(t.shape)})")
    if device is not None and t.device != device:
        raise ValueError(f"{what} is on {t.device}, the cache on {device}")


def _tables(block_tables, context_lens, device, batch=None):
    """block_tables int32 [batch][max_blocks], context_lens int32 [batch]; returns batch."""
    _tensor(context_lens, "context_lens", torch.int32, (batch,), device)
    b = context_lens.shape[0]
    _tensor(block_tables, "block_tables", torch.int32, (b, None), device)
    if block_tables.shape[1] < 1:
        raise ValueError("block_tables needs at least one column")
    return b


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    _device_tensor(t, "tensors passed to the library")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def dtype_from_string(name: str) -> int:
    out = ctypes.c_int(0)
    _check(lib.kvq_dtype_from_string(name.encode(), ctypes.byref(out)), "kvq_dtype_from_string")
    return out.value


@dataclass
class PagedKVCache:
    """Device tensors of one layer's paged cache (layouts as in kvq.h)."""
    dtype: int
    k_cache: torch.Tensor           # uint8 [num_blocks][Hkv][8][16][16]: 16-dim chunks x 16 tokens
                                    # (INT4: [num_blocks][Hkv][4][16][16], 32-dim chunks)
    v_cache: torch.Tensor           # uint8 [num_blocks][Hkv][128][16] (INT4: [..][128][8])
    k_scale: torch.Tensor | None    # float32 [num_blocks][Hkv][16] (INT8), [..][16][2] (INT4)
    v_scale: torch.Tensor | None    # INT8: k_scale and v_scale are the two halves of one
                                    # [num_blocks][Hkv][2][16] tensor (a tile's scales in one
                                    # 128-byte row), as allocate() makes them
    kv_scale: float = 1.0

    @property
    def num_blocks(self) -> int:
        return self.k_cache.shape[0]

    @property
    def num_kv_heads(self) -> int:
        return self.k_cache.shape[1]

    @staticmethod
    def allocate(dtype, num_blocks: int, num_kv_heads: int, kv_scale: float = 1.0,
                 device="cuda", poison: bool = True) -> "PagedKVCache":
        if isinstance(dtype, str):
            dtype = dtype_from_string(dtype)
        fill = 0x7F if poison else 0
        per = 2 if dtype == INT4 else 1  # codes per byte
        k = torch.full((num_blocks, num_kv_heads, HEAD_DIM // (16 * per), BLOCK_SIZE, 16), fill,
                       dtype=torch.uint8, device=device)
        v = torch.full((num_blocks, num_kv_heads, HEAD_DIM, BLOCK_SIZE // per), fill, dtype=torch.uint8,
                       device=device)
        ks = vs = None
        sfill = float("nan") if poison else 0.0
        if dtype == INT8:
            rows = torch.full((num_blocks, num_kv_heads, 2, BLOCK_SIZE), sfill, dtype=torch.float32, device=device)
            ks, vs = rows[:, :, 0], rows[:, :, 1]
        elif dtype == INT4:
            ks = torch.full((num_blocks, num_kv_heads, BLOCK_SIZE, 2), sfill, dtype=torch.float32, device=device)
            vs = torch.full_like(ks, sfill)
        return PagedKVCache(dtype, k, v, ks, vs, float(kv_scale))

    def clone(self) -> "PagedKVCache":
        """A copy in new device memory, with the same layout (INT8 scales interleaved again)."""
        c = PagedKVCache.allocate(self.dtype, self.num_blocks, self.num_kv_heads, self.kv_scale,
                                  device=self.k_cache.device, poison=False)
        c.k_cache.copy_(self.k_cache)
        c.v_cache.copy_(self.v_cache)
        if self.k_scale is not None:
            c.k_scale.copy_(self.k_scale)
            c.v_scale.copy_(self.v_scale)
        return c

    def descriptor(self) -> KvqCache:
        per = 2 if self.dtype == INT4 else 1
        nb, hkv = self.k_cache.shape[0], self.k_cache.shape[1]
        layout = {"k_cache": (self.k_cache, torch.uint8, (nb, hkv, HEAD_DIM // (16 * per), BLOCK_SIZE, 16)),
                  "v_cache": (self.v_cache, torch.uint8, (nb, hkv, HEAD_DIM, BLOCK_SIZE // per))}
        if self.dtype in (INT8, INT4):
            sshape = (nb, hkv, BLOCK_SIZE) + ((2,) if self.dtype == INT4 else ())
            for name, t in (("k_scale", self.k_scale), ("v_scale", self.v_scale)):
                if t is None:
                    raise ValueError(f"{name} is required for this cache dtype")
                layout[name] = (t, torch.float32, sshape)
        for name, (t, dt, shape) in layout.items():
            if self.dtype == INT8 and name in ("k_scale", "v_scale"):
                # the halves of one [nb][Hkv][2][16] tensor: strided views, checked below
                _device_memory(t, f"cache.{name}")
            else:
                _device_tensor(t, f"cache.{name}")
            if t.dtype != dt or tuple(t.shape) != shape:
                raise ValueError(f"cache.{name} must be {dt} {list(shape)} (got {t.dtype} {list(t.shape)})")
            if t.device != self.k_cache.device:
                raise ValueError("the cache tensors must be on one device")
        if self.dtype == INT8:
            rows = (hkv * 2 * BLOCK_SIZE, 2 * BLOCK_SIZE, 1)
            if (self.k_scale.stride() != rows or self.v_scale.stride() != rows or
                    self.v_scale.data_ptr() != self.k_scale.data_ptr() + 4 * BLOCK_SIZE):
                raise ValueError("INT8 scales must be the two halves of one [num_blocks][Hkv][2][16] float32 "
                                 "tensor (k_scale = rows[:, :, 0], v_scale = rows[:, :, 1]; "
                                 "PagedKVCache.allocate makes them so)")
        return KvqCache(self.dtype, self.k_cache.shape[0], BLOCK_SIZE, self.k_cache.shape[1], HEAD_DIM,
                        self.k_cache.data_ptr(), self.v_cache.data_ptr(),
                        self.k_scale.data_ptr() if self.k_scale is not None else None,
                        self.v_scale.data_ptr() if self.v_scale is not None else None,
                        float(self.kv_scale))


def append(cache: PagedKVCache, k_new: torch.Tensor, v_new: torch.Tensor, block_tables: torch.Tensor,
           context_lens: torch.Tensor, cu_new_lens: torch.Tensor | None = None,
           num_new_rows: int | None = None, stream=None) -> None:
    """kvq_append: fp16 rows [T][Hkv][128] -> their paged slots (post-append context_lens).
    With cu_new_lens (int32 [B+1], device), num_new_rows must equal cu_new_lens[B] (default: all of
    k_new's rows); without it there is one row per sequence."""
    d = cache.descriptor()
    dev = cache.k_cache.device
    batch = _tables(block_tables, context_lens, dev)
    _tensor(k_new, "k_new", torch.float16, (None, cache.num_kv_heads, HEAD_DIM), dev)
    _tensor(v_new, "v_new", torch.float16, tuple(k_new.shape), dev)
    T = k_new.shape[0] if num_new_rows is None else int(num_new_rows)
    if not 0 <= T <= k_new.shape[0]:
        raise ValueError(f"num_new_rows {T} outside [0, {k_new.shape[0]}] (the rows of k_new)")
    if cu_new_lens is not None:
        _tensor(cu_new_lens, "cu_new_lens", torch.int32, (batch + 1,), dev)
    elif T != batch:
        raise ValueError(f"without cu_new_lens there is one new row per sequence ({batch}), not {T}")
    _check(lib.kvq_append(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(cu_new_lens), T,
                          _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), batch,
                          _stream(stream)), "kvq_append")


PARTITION_BALANCED = -1  # KVQ_PARTITION_BALANCED


def workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, max_context_len: int,
                   partition_size: int) -> int:
    return int(lib.kvq_decode_workspace_size(batch, num_q_heads, num_kv_heads, max_context_len,
                                             partition_size))


def alloc_workspace(batch, num_q_heads, num_kv_heads, max_context_len, partition_size, device="cuda"):
    n = workspace_size(batch, num_q_heads, num_kv_heads, max_context_len, partition_size)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device), n


def paged_decode_attn(cache: PagedKVCache, q: torch.Tensor, block_tables: torch.Tensor,
                      context_lens: torch.Tensor, max_context_len: int, sm_scale: float | None = None,
                      partition_size: int = PARTITION_BALANCED, workspace: torch.Tensor | None = None,
                      out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_paged_decode_attn: q fp16 [B][Hq][128] -> out fp16 [B][Hq][128]."""
    return _decode_attn("kvq_paged_decode_attn", cache, q, block_tables, context_lens, max_context_len,
                        sm_scale, partition_size, workspace, out, stream)


def paged_decode_attn_fp8math(cache: PagedKVCache, q: torch.Tensor, block_tables: torch.Tensor,
                              context_lens: torch.Tensor, max_context_len: int,
                              sm_scale: float | None = None, partition_size: int = PARTITION_BALANCED,
                              workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                              stream=None) -> torch.Tensor:
    """kvq_paged_decode_attn_fp8math: as paged_decode_attn, the query rows quantized to E4M3 and
    QK^T on the FP8 matrix cores (E4M3 / E5M2 caches)."""
    return _decode_attn("kvq_paged_decode_attn_fp8math", cache, q, block_tables, context_lens,
                        max_context_len, sm_scale, partition_size, workspace, out, stream)


_NO_WORKSPACE = object()  # _decode_args: the call brings its own workspace


def _decode_args(cache, q, block_tables, context_lens, max_context_len, partition_size, workspace, out):
    """Checks shared by the decode calls -> (descriptor, out, workspace, workspace bytes)."""
    d = cache.descriptor()
    dev = cache.k_cache.device
    B = _tables(block_tables, context_lens, dev)
    _tensor(q, "q", torch.float16, (B, None, HEAD_DIM), dev)
    Hq = q.shape[1]
    if out is None:
        out = torch.empty_like(q)
    _tensor(out, "out", torch.float16, tuple(q.shape), dev)
    if workspace is _NO_WORKSPACE:
        return d, out, None, 0
    need = workspace_size(B, Hq, cache.num_kv_heads, max_context_len, partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _tensor(workspace, "workspace", torch.uint8, (None,), dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    return d, out, workspace, ws_bytes


def _decode_attn(name, cache, q, block_tables, context_lens, max_context_len, sm_scale, partition_size,
                 workspace, out, stream):
    d, out, workspace, ws_bytes = _decode_args(cache, q, block_tables, context_lens, max_context_len,
                                               partition_size, workspace, out)
    B, Hq, _ = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    _check(getattr(lib, name)(ctypes.byref(d), _ptr(q), _ptr(out), Hq, float(sm_scale),
                              _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), B,
                              int(max_context_len), int(partition_size), _ptr(workspace), ws_bytes,
                              _stream(stream)), name)
    return out


def decode_step(cache: PagedKVCache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                sm_scale: float | None = None, partition_size: int = PARTITION_BALANCED,
                workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """kvq_decode_step: append one row per sequence (fp16 [B][Hkv][128]) and attend, fused."""
    return _decode_step("kvq_decode_step", cache, k_new, v_new, q, block_tables, context_lens,
                        max_context_len, sm_scale, partition_size, workspace, out, stream)


def decode_step_fp8math(cache: PagedKVCache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                        block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                        sm_scale: float | None = None, partition_size: int = PARTITION_BALANCED,
                        workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """kvq_decode_step_fp8math: decode_step with FP8 math for QK^T."""
    return _decode_step("kvq_decode_step_fp8math", cache, k_new, v_new, q, block_tables, context_lens,
                        max_context_len, sm_scale, partition_size, workspace, out, stream)


def _decode_step(name, cache, k_new, v_new, q, block_tables, context_lens, max_context_len, sm_scale,
                 partition_size, workspace, out, stream):
    d, out, workspace, ws_bytes = _decode_args(cache, q, block_tables, context_lens, max_context_len,
                                               partition_size, workspace, out)
    B, Hq, _ = q.shape
    dev = cache.k_cache.device
    _tensor(k_new, "k_new", torch.float16, (B, cache.num_kv_heads, HEAD_DIM), dev)
    _tensor(v_new, "v_new", torch.float16, (B, cache.num_kv_heads, HEAD_DIM), dev)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    _check(getattr(lib, name)(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out), Hq,
                              float(sm_scale), _ptr(block_tables), block_tables.shape[1],
                              _ptr(context_lens), B, int(max_context_len), int(partition_size),
                              _ptr(workspace), ws_bytes, _stream(stream)), name)
    return out


class PreparedCall:
    """One library call whose arguments were checked and marshalled once: calling it only invokes
    the entry point again, with the same device buffers, sizes and stream.  For a loop that issues
    the same call step after step (a serving loop, a benchmark), where the binding's per-call
    checks would otherwise cost more host time than a small step's kernels take."""

    def __init__(self, name: str, args: tuple, keep: tuple, result: torch.Tensor):
        self._name = name
        self._fn = getattr(lib, name)
        self._args = args
        self._keep = keep  # the tensors and the descriptor the marshalled pointers refer to
        self.result = result

    def __call__(self) -> torch.Tensor:
        _check(self._fn(*self._args), self._name)
        return self.result


def prepare_decode_step(cache: PagedKVCache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                        block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                        sm_scale: float | None = None, partition_size: int = PARTITION_BALANCED,
                        workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                        stream=None, fp8_math: bool = False) -> PreparedCall:
    """decode_step (decode_step_fp8math with fp8_math) checked and marshalled once; the returned
    PreparedCall launches it on every call.  The caller keeps the tensors' contents current (new
    rows in k_new / v_new, the lengths in context_lens) and must not reallocate them."""
    name = "kvq_decode_step_fp8math" if fp8_math else "kvq_decode_step"
    d, out, workspace, ws_bytes = _decode_args(cache, q, block_tables, context_lens, max_context_len,
                                               partition_size, workspace, out)
    B, Hq, _ = q.shape
    dev = cache.k_cache.device
    _tensor(k_new, "k_new", torch.float16, (B, cache.num_kv_heads, HEAD_DIM), dev)
    _tensor(v_new, "v_new", torch.float16, (B, cache.num_kv_heads, HEAD_DIM), dev)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    args = (ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out), Hq, float(sm_scale),
            _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), B, int(max_context_len),
            int(partition_size), _ptr(workspace), ws_bytes, _stream(stream))
    keep = (d, cache, k_new, v_new, q, out, block_tables, context_lens, workspace)
    return PreparedCall(name, args, keep, out)


def decode_step_noalloc(cache: PagedKVCache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                        block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                        sm_scale: float | None = None, partition_size: int = PARTITION_BALANCED,
                        out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_decode_step_noalloc: decode_step with the library's own device scratch as the split-K
    workspace (no allocation in the call when `out` is given; calls that overlap on one GPU race)."""
    d, out, _, _ = _decode_args(cache, q, block_tables, context_lens, max_context_len, PARTITION_BALANCED
                                if partition_size is None else partition_size, _NO_WORKSPACE, out)
    B, Hq, _ = q.shape
    dev = cache.k_cache.device
    _tensor(k_new, "k_new", torch.float16, (B, cache.num_kv_heads, HEAD_DIM), dev)
    _tensor(v_new, "v_new", torch.float16, (B, cache.num_kv_heads, HEAD_DIM), dev)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    _check(lib.kvq_decode_step_noalloc(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out), Hq,
                                       float(sm_scale), _ptr(block_tables), block_tables.shape[1],
                                       _ptr(context_lens), B, int(max_context_len), int(partition_size),
                                       _stream(stream)), "kvq_decode_step_noalloc")
    return out


def paged_prefill_attn(cache: PagedKVCache, q: torch.Tensor, cu_q_lens: torch.Tensor,
                       block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                       max_q_len: int, sm_scale: float | None = None, out: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """kvq_paged_prefill_attn: q fp16 [T][Hq][128] (rows of sequence b at cu_q_lens[b] ..
    cu_q_lens[b+1]-1, the last rows of its context) -> out fp16 [T][Hq][128], causal."""
    return _prefill("kvq_paged_prefill_attn", cache, q, cu_q_lens, block_tables, context_lens,
                    max_context_len, max_q_len, sm_scale, out, stream)


def paged_prefill_attn_fp8math(cache: PagedKVCache, q: torch.Tensor, cu_q_lens: torch.Tensor,
                               block_tables: torch.Tensor, context_lens: torch.Tensor,
                               max_context_len: int, max_q_len: int, sm_scale: float | None = None,
                               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_paged_prefill_attn_fp8math: paged_prefill_attn with FP8 math for QK^T."""
    return _prefill("kvq_paged_prefill_attn_fp8math", cache, q, cu_q_lens, block_tables, context_lens,
                    max_context_len, max_q_len, sm_scale, out, stream)


def _prefill(name, cache, q, cu_q_lens, block_tables, context_lens, max_context_len, max_q_len,
             sm_scale, out, stream):
    d = cache.descriptor()
    dev = cache.k_cache.device
    B = _tables(block_tables, context_lens, dev)
    _tensor(q, "q", torch.float16, (None, None, HEAD_DIM), dev)
    _tensor(cu_q_lens, "cu_q_lens", torch.int32, (B + 1,), dev)
    T, Hq, _ = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty_like(q)
    _tensor(out, "out", torch.float16, tuple(q.shape), dev)
    _check(getattr(lib, name)(ctypes.byref(d), _ptr(q), _ptr(out), Hq, float(sm_scale),
                              _ptr(cu_q_lens), T, int(max_q_len), _ptr(block_tables),
                              block_tables.shape[1], _ptr(context_lens), B, int(max_context_len),
                              _stream(stream)), name)
    return out


def quantize_q_fp8(q: torch.Tensor, stream=None):
    """kvq_quantize_q_fp8: fp16 rows [..., 128] -> (E4M3 codes uint8 [..., 128], fp32 scales [...])."""
    _tensor(q, "q", torch.float16)
    if q.dim() < 1 or q.shape[-1] != HEAD_DIM:
        raise ValueError(f"q must have rows of {HEAD_DIM} (got {list(q.shape)})")
    codes = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    scales = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    rows = q.numel() // HEAD_DIM
    _check(lib.kvq_quantize_q_fp8(_ptr(q), rows, _ptr(codes), _ptr(scales), _stream(stream)),
           "kvq_quantize_q_fp8")
    return codes, scales


def dequant(cache: PagedKVCache, block_tables: torch.Tensor, context_lens: torch.Tensor,
            max_context_len: int, k_out: torch.Tensor | None = None, v_out: torch.Tensor | None = None,
            stream=None):
    """kvq_dequant -> (k, v) fp32 [B][Hkv][max_context_len][128] (slots past a context untouched)."""
    d = cache.descriptor()
    dev = cache.k_cache.device
    B = _tables(block_tables, context_lens, dev)
    shape = (B, cache.num_kv_heads, max_context_len, HEAD_DIM)
    if k_out is None:
        k_out = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
    if v_out is None:
        v_out = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
    _tensor(k_out, "k_out", torch.float32, shape, dev)
    _tensor(v_out, "v_out", torch.float32, shape, dev)
    _check(lib.kvq_dequant(ctypes.byref(d), _ptr(block_tables), block_tables.shape[1],
                           _ptr(context_lens), B, int(max_context_len), _ptr(k_out), _ptr(v_out),
                           _stream(stream)), "kvq_dequant")
    return k_out, v_out


def timing_begin(capacity: int) -> None:
    _check(lib.kvq_timing_begin(capacity), "kvq_timing_begin")


def timing_end():
    """-> (summed milliseconds of the timed partition kernels, number of timed launches)."""
    mt = ctypes.c_double(0)
    mc = ctypes.c_int32(0)
    _check(lib.kvq_timing_end(ctypes.byref(mt), ctypes.byref(mc)), "kvq_timing_end")
    return mt.value, mc.value


def version() -> str:
    return lib.kvq_version().decode()
