"""CPU oracle for the 8-bit paged KV cache and its decode-step attention (numpy front end).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this package.  The product path (the HIP library in
``quantized_kv_cache_03_amd``) never imports it and shares no code with it.

Every function here marshals numpy arrays into the plain-C oracle (``kvq_oracle.c``), where each
step is written from its definition in fp64:

* FP8 E4M3 / E5M2 codes: "Accelerating Inference with FP8 KV Cache", section "FP8 Formats: E4M3
  and E5M2" (bit layouts, per-tensor FP32 scale) and section "FP8 E4M3 KV Cache" (default scale 1.0).
* FP8 E4M3FNUZ codes: the same page, sections "Current Hardware Support" (AMD's FP8E4M3FNUZ) and
  "Checkpoint structure for KV scales" (float8_e4m3fnuz): bias 8, no infinities, no negative zero,
  NaN at 0x80.
* Online INT8 codes: "[Feature] TurboMind support W8A8 or FP8 KV Cache" (the online INT8 KV cache);
  read as symmetric INT8 with one fp32 scale per (token, head).
* Online INT4 codes: the same thread names INT4 next to INT8; read as asymmetric 4-bit codes with
  one fp32 (scale, zero point) pair per (token, head), two codes per byte.
* Paged cache: "[QST] Scale factors and benchmarks" (paged attention in the serving stack).

Layouts are those the C file documents: K codes ``[num_blocks][Hkv][8][16][16]`` (16-dim chunks),
V codes ``[num_blocks][Hkv][128][16]``, INT8 scales ``[num_blocks][Hkv][2][16]`` (a tile's K scales,
then its V scales; ``Cache.ks`` / ``Cache.vs`` are the two halves as views); INT4 tiles are half
the size (two codes per byte) and its (scale, zero point) pairs are ``[num_blocks][Hkv][16][2]``.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

E4M3, E5M2, INT8, E4M3FNUZ, INT4 = 1, 2, 3, 4, 5
BLOCK = 16
DIM = 128

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_ORACLE_LIBRARY may name another build of the same source (the sanitizer build)
_LIB_PATH = os.environ.get("KVQ_ORACLE_LIBRARY") or os.path.join(_HERE, "libkvq_oracle.so")
_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_i8p = ctypes.POINTER(ctypes.c_int8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_c_int, _c_float = ctypes.c_int, ctypes.c_float


def lib():
    """Load the oracle library, building it with gcc first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        _lib = load(_LIB_PATH)
    return _lib


def load(path: str):
    """Open an oracle library file and declare its signatures."""
    L = ctypes.CDLL(path)
    L.kvqo_fp16_to_double.argtypes = [ctypes.c_uint16]
    L.kvqo_fp16_to_double.restype = ctypes.c_double
    L.kvqo_fp8_decode.argtypes = [_c_int, ctypes.c_uint8]
    L.kvqo_fp8_decode.restype = ctypes.c_double
    L.kvqo_fp8_encode.argtypes = [_c_int, _c_float]
    L.kvqo_fp8_encode.restype = ctypes.c_uint8
    L.kvqo_fp8_quantize.argtypes = [_c_int, ctypes.c_uint16, _c_float]
    L.kvqo_fp8_quantize.restype = ctypes.c_uint8
    L.kvqo_fp8_decode_array.argtypes = [_c_int, _u8p, _c_int, _f64p]
    L.kvqo_fp8_encode_array.argtypes = [_c_int, _f32p, _c_int, _u8p]
    L.kvqo_fp8_quantize_array.argtypes = [_c_int, _u16p, _c_int, _c_float, _u8p]
    L.kvqo_fp16_to_double_array.argtypes = [_u16p, _c_int, _f64p]
    L.kvqo_int8_quantize_rows.argtypes = [_u16p, _c_int, _c_int, _i8p, _f32p]
    L.kvqo_int4_quantize_rows.argtypes = [_u16p, _c_int, _c_int, _u8p, _f32p, _f32p]
    L.kvqo_append.argtypes = [_c_int, _c_int, _u8p, _u8p, _f32p, _f32p, _c_float, _u16p, _u16p,
                              _i32p, _i32p, _c_int, _i32p, _c_int]
    L.kvqo_append.restype = _c_int
    L.kvqo_dequant.argtypes = [_c_int, _c_int, _u8p, _u8p, _f32p, _f32p, _c_float, _i32p,
                               _c_int, _i32p, _c_int, _c_int, _f32p, _f32p]
    L.kvqo_dequant.restype = _c_int
    L.kvqo_decode_attn_head.argtypes = [_c_int, _c_int, _c_int, _u8p, _u8p, _f32p, _f32p,
                                        _c_float, _u16p, _c_float, _i32p, _c_int, _i32p,
                                        _c_int, _c_int, _f64p]
    L.kvqo_decode_attn_head.restype = _c_int
    L.kvqo_decode_attn_head_fp8q.argtypes = L.kvqo_decode_attn_head.argtypes
    L.kvqo_decode_attn_head_fp8q.restype = _c_int
    L.kvqo_quantize_q_fp8_rows.argtypes = [_u16p, _c_int, _u8p, _f32p]
    L.kvqo_quantize_q_fp8_rows.restype = None
    L.kvqo_attn_fp16_dense.argtypes = [_u16p, _u16p, _u16p, _c_int, _c_float, _f64p]
    L.kvqo_attn_fp16_dense.restype = _c_int
    return L


def _ptr(a: np.ndarray | None, ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctype)


def _fp16_bits(x: np.ndarray) -> np.ndarray:
    """fp16 values (or their uint16 bit patterns) as a contiguous uint16 array."""
    x = np.asarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    assert x.dtype == np.uint16, f"expected float16 or uint16 bits, got {x.dtype}"
    return np.ascontiguousarray(x)


# ---------------------------------------------------------------------------------------------
# element codecs
def fp16_to_double(x) -> np.ndarray:
    bits = _fp16_bits(x)
    out = np.empty(bits.shape, np.float64)
    lib().kvqo_fp16_to_double_array(_ptr(bits.reshape(-1), _u16p), bits.size, _ptr(out.reshape(-1), _f64p))
    return out


def fp8_decode(fmt: int, codes) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.empty(c.shape, np.float64)
    lib().kvqo_fp8_decode_array(fmt, _ptr(c.reshape(-1), _u8p), c.size, _ptr(out.reshape(-1), _f64p))
    return out


def fp8_decode_table(fmt: int) -> np.ndarray:
    return fp8_decode(fmt, np.arange(256, dtype=np.uint8))


def fp8_encode(fmt: int, y) -> np.ndarray:
    """Encode fp32 values that are already divided by the scale."""
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float32))
    out = np.empty(y.shape, np.uint8)
    lib().kvqo_fp8_encode_array(fmt, _ptr(y.reshape(-1), _f32p), y.size, _ptr(out.reshape(-1), _u8p))
    return out


def fp8_quantize(fmt: int, x_fp16, kv_scale: float = 1.0) -> np.ndarray:
    """code = enc(fl32(fl32(x) / kv_scale)) for fp16 inputs x."""
    bits = _fp16_bits(x_fp16)
    out = np.empty(bits.shape, np.uint8)
    lib().kvqo_fp8_quantize_array(fmt, _ptr(bits.reshape(-1), _u16p), bits.size,
                                  float(np.float32(kv_scale)), _ptr(out.reshape(-1), _u8p))
    return out


def int8_quantize_rows(x_fp16) -> tuple[np.ndarray, np.ndarray]:
    """Rows of the last axis -> (int8 codes, fp32 scales)."""
    bits = _fp16_bits(x_fp16)
    n = bits.shape[-1]
    rows = bits.size // n
    q = np.empty(bits.shape, np.int8)
    s = np.empty(bits.shape[:-1], np.float32)
    lib().kvqo_int8_quantize_rows(_ptr(bits.reshape(-1), _u16p), rows, n,
                                  _ptr(q.reshape(-1), _i8p), _ptr(s.reshape(-1), _f32p))
    return q, s


def int4_quantize_rows(x_fp16) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Rows of the last axis -> (uint8 codes 0..15, fp32 scales, fp32 zero points)."""
    bits = _fp16_bits(x_fp16)
    n = bits.shape[-1]
    rows = bits.size // n
    q = np.empty(bits.shape, np.uint8)
    s = np.empty(bits.shape[:-1], np.float32)
    z = np.empty(bits.shape[:-1], np.float32)
    lib().kvqo_int4_quantize_rows(_ptr(bits.reshape(-1), _u16p), rows, n, _ptr(q.reshape(-1), _u8p),
                                  _ptr(s.reshape(-1), _f32p), _ptr(z.reshape(-1), _f32p))
    return q, s, z


def quantize_q_fp8_rows(q_fp16) -> tuple[np.ndarray, np.ndarray]:
    """Query rows of 128 (last axis) -> (E4M3 codes, fp32 per-row scales) of the FP8-math path."""
    bits = _fp16_bits(q_fp16)
    assert bits.shape[-1] == DIM
    rows = bits.size // DIM
    c = np.empty(bits.shape, np.uint8)
    s = np.empty(bits.shape[:-1], np.float32)
    lib().kvqo_quantize_q_fp8_rows(_ptr(bits.reshape(-1), _u16p), rows, _ptr(c.reshape(-1), _u8p),
                                   _ptr(s.reshape(-1), _f32p))
    return c, s


def tile_bytes(dtype: int) -> int:
    """Bytes of one (block, KV head) tile of K (or of V) codes."""
    return BLOCK * DIM // 2 if dtype == INT4 else BLOCK * DIM


# ---------------------------------------------------------------------------------------------
# paged cache
class Cache:
    """Host-memory paged cache in the documented layout (test infrastructure)."""

    def __init__(self, dtype: int, num_blocks: int, num_kv_heads: int, kv_scale: float = 1.0,
                 k_codes=None, v_codes=None, k_scale=None, v_scale=None, poison: bool = True):
        self.dtype = dtype
        self.num_blocks = num_blocks
        self.Hkv = num_kv_heads
        self.kv_scale = float(np.float32(kv_scale))
        shape = (num_blocks, num_kv_heads, tile_bytes(dtype))
        fill = 0x7F if poison else 0
        self.k = np.full(shape, fill, np.uint8) if k_codes is None else np.ascontiguousarray(k_codes, np.uint8).reshape(shape)
        self.v = np.full(shape, fill, np.uint8) if v_codes is None else np.ascontiguousarray(v_codes, np.uint8).reshape(shape)
        self.rows = None
        if dtype == INT8:
            # one row per tile: [..][0][t] the K scale of token t, [..][1][t] its V scale
            self.rows = np.full((num_blocks, num_kv_heads, 2, BLOCK), np.nan, np.float32)
            self.ks, self.vs = self.rows[:, :, 0], self.rows[:, :, 1]
            sshape = (num_blocks, num_kv_heads, BLOCK)
            if k_scale is not None:
                self.ks[...] = np.asarray(k_scale, np.float32).reshape(sshape)
            if v_scale is not None:
                self.vs[...] = np.asarray(v_scale, np.float32).reshape(sshape)
        elif dtype == INT4:
            sshape = (num_blocks, num_kv_heads, BLOCK, 2)
            self.ks = np.full(sshape, np.nan, np.float32) if k_scale is None else np.ascontiguousarray(k_scale, np.float32).reshape(sshape)
            self.vs = np.full(sshape, np.nan, np.float32) if v_scale is None else np.ascontiguousarray(v_scale, np.float32).reshape(sshape)
        else:
            self.ks = None
            self.vs = None

    def args(self):
        if self.rows is not None:  # INT8: k_scale at the rows, v_scale 16 floats on
            ks = _ptr(self.rows, _f32p)
            vs = ctypes.cast(ctypes.addressof(ks.contents) + 4 * BLOCK, _f32p)
        else:
            ks, vs = _ptr(self.ks, _f32p), _ptr(self.vs, _f32p)
        return (self.dtype, self.Hkv, _ptr(self.k, _u8p), _ptr(self.v, _u8p), ks, vs, self.kv_scale)


def append(cache: Cache, k_new, v_new, block_tables, context_lens, cu_new_lens=None) -> None:
    """Write new fp16 K/V rows [T][Hkv][128] at positions context_lens[b] - n_b + j."""
    kb = _fp16_bits(k_new)
    vb = _fp16_bits(v_new)
    bt = np.ascontiguousarray(block_tables, np.int32)
    ctx = np.ascontiguousarray(context_lens, np.int32)
    cu = None if cu_new_lens is None else np.ascontiguousarray(cu_new_lens, np.int32)
    B = ctx.shape[0]
    assert kb.shape == vb.shape and kb.shape[-2:] == (cache.Hkv, DIM)
    rc = lib().kvqo_append(*cache.args(), _ptr(kb, _u16p), _ptr(vb, _u16p), _ptr(cu, _i32p),
                           _ptr(bt, _i32p), bt.shape[1], _ptr(ctx, _i32p), B)
    if rc != 0:
        raise ValueError("oracle append rejected its arguments")


def dequant(cache: Cache, block_tables, context_lens, max_context_len: int,
            fill: float = np.nan) -> tuple[np.ndarray, np.ndarray]:
    bt = np.ascontiguousarray(block_tables, np.int32)
    ctx = np.ascontiguousarray(context_lens, np.int32)
    B = ctx.shape[0]
    ko = np.full((B, cache.Hkv, max_context_len, DIM), fill, np.float32)
    vo = np.full((B, cache.Hkv, max_context_len, DIM), fill, np.float32)
    rc = lib().kvqo_dequant(*cache.args(), _ptr(bt, _i32p), bt.shape[1], _ptr(ctx, _i32p), B,
                            max_context_len, _ptr(ko, _f32p), _ptr(vo, _f32p))
    if rc != 0:
        raise ValueError("oracle dequant rejected its arguments")
    return ko, vo


def decode_attn(cache: Cache, q, block_tables, context_lens, sm_scale: float | None = None,
                heads=None, threads: int = 1, fp8_math: bool = False) -> np.ndarray:
    """fp64 decode attention.  q: fp16 [B][Hq][128].  Returns [B][Hq][128] float64 (rows not in
    ``heads``, a list of (b, h) pairs, are left NaN).  fp8_math=True first replaces each query row
    by its E4M3 quantization (quantize_q_fp8_rows), dequantized exactly."""
    qb = _fp16_bits(q)
    B, Hq, D = qb.shape
    assert D == DIM
    bt = np.ascontiguousarray(block_tables, np.int32)
    ctx = np.ascontiguousarray(context_lens, np.int32)
    if sm_scale is None:
        sm_scale = float(np.float32(1.0 / np.sqrt(DIM)))
    out = np.full((B, Hq, DIM), np.nan, np.float64)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    L = lib()
    fn = L.kvqo_decode_attn_head_fp8q if fp8_math else L.kvqo_decode_attn_head
    cargs = cache.args()
    qp, btp, ctxp = _ptr(qb, _u16p), _ptr(bt, _i32p), _ptr(ctx, _i32p)

    def one(bh):
        b, h = bh
        row = np.empty(DIM, np.float64)
        rc = fn(cargs[0], cargs[1], Hq, *cargs[2:], qp, float(sm_scale), btp,
                bt.shape[1], ctxp, b, h, _ptr(row, _f64p))
        if rc != 0:
            raise ValueError("oracle attention rejected its arguments")
        out[b, h] = row

    if threads <= 1:
        for bh in heads:
            one(bh)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, heads))
    return out


def prefill_attn(cache: Cache, q, block_tables, context_lens, cu_q_lens, sm_scale: float | None = None,
                 rows=None, threads: int = 1, fp8_math: bool = False) -> np.ndarray:
    """fp64 prefill (causal) attention.  q: fp16 [T][Hq][128], sequence b's rows cu_q_lens[b] ..
    cu_q_lens[b+1]-1 being the last n_b of its context_lens[b] tokens; row j of b attends to the
    tokens at positions 0 .. context_lens[b] - n_b + j.  That is decode attention over the row's
    visible prefix, so each row is one decode_attn row with its own length and b's block table.
    Returns [T][Hq][128] float64 (rows not in ``rows``, a list of row indices, are left NaN)."""
    q = np.asarray(q)
    T, Hq, _ = q.shape
    cu = np.asarray(cu_q_lens, np.int64)
    ctx = np.asarray(context_lens, np.int64)
    bt = np.asarray(block_tables, np.int32)
    seq = np.searchsorted(cu, np.arange(T), side="right") - 1   # sequence of each row
    pos = ctx[seq] - (cu[seq + 1] - cu[seq]) + (np.arange(T) - cu[seq])
    assert np.all(pos >= 0), "a sequence has more query rows than tokens"
    if rows is None:
        rows = range(T)
    rows = list(rows)
    out = np.full((T, Hq, DIM), np.nan, np.float64)
    if rows:
        sub = decode_attn(cache, q[rows], bt[seq[rows]], (pos[rows] + 1).astype(np.int32),
                          sm_scale=sm_scale, threads=threads, fp8_math=fp8_math)
        out[rows] = sub
    return out


def attn_fp16_dense(q_row, k_rows, v_rows, sm_scale: float | None = None) -> np.ndarray:
    """fp64 attention of one fp16 query row [128] over unquantized fp16 rows [n][128]."""
    qb = _fp16_bits(q_row)
    kb = _fp16_bits(k_rows)
    vb = _fp16_bits(v_rows)
    if sm_scale is None:
        sm_scale = float(np.float32(1.0 / np.sqrt(DIM)))
    out = np.empty(DIM, np.float64)
    rc = lib().kvqo_attn_fp16_dense(_ptr(qb, _u16p), _ptr(kb, _u16p), _ptr(vb, _u16p),
                                    kb.shape[0], float(sm_scale), _ptr(out, _f64p))
    if rc != 0:
        raise ValueError("oracle dense attention failed")
    return out
