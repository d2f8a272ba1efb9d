"""Seeded synthetic inputs for the quantized paged KV cache (shared by tests, bench and smoke).

This module only draws random numbers and lays them out; it holds none of the method's arithmetic
(no encoding, decoding or attention).  Both the HIP path and the CPU oracle take its arrays.

The five workloads mirror the decode shapes the 8-bit KV cache is used on: a tiny one, and layers
shaped like Llama-2-7B (MHA), Llama-3-8B (GQA 4), Llama-2-13B (MHA, online INT8 with outlier
channels) and Llama-3-70B (GQA 8, 32k context).  The pages measure accuracy on evaluation suites
with trained weights; these seeded normal inputs stand in for model activations.

Generation recipe (every stream is ``numpy.random.default_rng([seed, stream, ...])``):
  stream 0 : context lengths (uniform integers or a lognormal draw, see ``Workload.context``)
  stream 1 : permutation of block ids for a shuffled block table
  stream 2 : q ~ N(0,1), drawn as float32 and rounded to float16
  stream 3 : outlier channels, ``outliers`` distinct channel indices per KV head
  stream (4, b) : sequence b's K rows then V rows ~ N(0,1) float32, outlier channels multiplied by
             ``outlier_gain`` in float32, then rounded to float16.  The last row of each sequence is
             the token appended by the decode step.
The per-tensor scale of the E4M3 workloads is the synthetic calibration ``fl32(amax) / 448``
(``/ 240`` for E4M3FNUZ, whose largest finite value is 240), with amax over every K and V value of
the layer (a stand-in for the offline calibration tools).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

HEAD_DIM = 128
BLOCK_SIZE = 16


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    dtype: str                  # "fp8_e4m3" | "fp8_e5m2" | "int8" | "fp8_e4m3fnuz" | "int4"
    context: tuple              # ("fixed", n) | ("uniform", lo, hi) | ("lognormal", median, sigma, cap)
    table: str = "sequential"   # "sequential" | "shuffled"
    scale_rule: str = "one"     # "amax/448" | "amax/240" | "one"
    outliers: int = 0
    outlier_gain: float = 20.0
    partition_size: int = -1  # the balanced split (KVQ_PARTITION_BALANCED)
    fp8_math: bool = False    # query rows quantized to E4M3, QK^T on the FP8 matrix cores

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def scaled(self, name: str | None = None, **changes) -> "Workload":
        """The same recipe at other sizes (tests use these to stay within oracle time)."""
        return dataclasses.replace(self, name=name or (self.name + "-scaled"), **changes)


WORKLOADS = {
    "tiny-e4m3": Workload("tiny-e4m3", 1, 1, 8, 8, "fp8_e4m3", ("fixed", 512),
                          scale_rule="amax/448"),
    "llama2-7b-mha-e4m3": Workload("llama2-7b-mha-e4m3", 2, 32, 32, 32, "fp8_e4m3",
                                   ("uniform", 512, 4096), table="shuffled",
                                   scale_rule="amax/448"),
    "llama3-8b-gqa-e5m2": Workload("llama3-8b-gqa-e5m2", 3, 64, 32, 8, "fp8_e5m2",
                                   ("fixed", 8192), scale_rule="one"),
    "llama2-13b-mha-int8": Workload("llama2-13b-mha-int8", 4, 128, 40, 40, "int8",
                                    ("lognormal", 2048, 1.0, 16384), outliers=4),
    "llama3-70b-gqa-e4m3-32k": Workload("llama3-70b-gqa-e4m3-32k", 5, 16, 64, 8, "fp8_e4m3",
                                        ("fixed", 32768), scale_rule="amax/448"),
    # the 32k GQA-8 batch at its own work split: fixed 512-token partitions, then the merge kernel
    "llama3-70b-gqa-e4m3-32k-p512": Workload("llama3-70b-gqa-e4m3-32k-p512", 5, 16, 64, 8, "fp8_e4m3",
                                             ("fixed", 32768), scale_rule="amax/448", partition_size=512),
    # the AMD E4M3 flavour (FNUZ) on the Llama-2-7B and Llama-3-70B shapes
    "llama2-7b-mha-e4m3fnuz": Workload("llama2-7b-mha-e4m3fnuz", 2, 32, 32, 32, "fp8_e4m3fnuz",
                                       ("uniform", 512, 4096), table="shuffled",
                                       scale_rule="amax/240"),
    "llama3-70b-gqa-e4m3fnuz-32k": Workload("llama3-70b-gqa-e4m3fnuz-32k", 5, 16, 64, 8,
                                            "fp8_e4m3fnuz", ("fixed", 32768), scale_rule="amax/240"),
    # online INT4 (asymmetric, per (token, head) scale and zero point) on the Llama-2-7B and
    # Llama-3-8B shapes
    "llama2-7b-mha-int4": Workload("llama2-7b-mha-int4", 2, 32, 32, 32, "int4",
                                   ("uniform", 512, 4096), table="shuffled"),
    "llama3-8b-gqa-int4": Workload("llama3-8b-gqa-int4", 3, 64, 32, 8, "int4", ("fixed", 8192)),
    # FP8 math (same caches and queries as the fp16-math workloads of the same shapes)
    "llama2-7b-mha-e4m3-fp8math": Workload("llama2-7b-mha-e4m3-fp8math", 2, 32, 32, 32, "fp8_e4m3",
                                           ("uniform", 512, 4096), table="shuffled",
                                           scale_rule="amax/448", fp8_math=True),
    "llama3-8b-gqa-e5m2-fp8math": Workload("llama3-8b-gqa-e5m2-fp8math", 3, 64, 32, 8, "fp8_e5m2",
                                           ("fixed", 8192), scale_rule="one", fp8_math=True),
    "llama3-70b-gqa-e4m3-32k-fp8math": Workload("llama3-70b-gqa-e4m3-32k-fp8math", 5, 16, 64, 8,
                                                "fp8_e4m3", ("fixed", 32768), scale_rule="amax/448",
                                                fp8_math=True),
}
ORDER = list(WORKLOADS)


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def context_lens(w: Workload) -> np.ndarray:
    kind = w.context[0]
    if kind == "fixed":
        return np.full(w.batch, int(w.context[1]), np.int32)
    if kind == "uniform":
        lo, hi = int(w.context[1]), int(w.context[2])
        return _rng(w.seed, 0).integers(lo, hi + 1, size=w.batch).astype(np.int32)
    if kind == "lognormal":
        median, sigma, cap = float(w.context[1]), float(w.context[2]), int(w.context[3])
        z = _rng(w.seed, 0).standard_normal(w.batch)
        return np.clip(np.rint(np.exp(np.log(median) + sigma * z)), 1, cap).astype(np.int32)
    if kind == "list":
        return np.asarray(w.context[1], np.int32)
    raise ValueError(f"unknown context rule {w.context!r}")


def block_tables(w: Workload, ctx: np.ndarray, spare_blocks: int = 0):
    """-> (block_tables int32 [B][max_blocks] padded with -1, num_blocks).  Block ids are handed
    out sequence by sequence; a shuffled table applies one seeded permutation to all ids."""
    nblk = (ctx.astype(np.int64) + BLOCK_SIZE - 1) // BLOCK_SIZE
    max_blocks = max(1, int(nblk.max()) if len(nblk) else 1)
    total = int(nblk.sum())
    num_blocks = total + spare_blocks
    ids = np.arange(num_blocks, dtype=np.int64)
    if w.table == "shuffled":
        ids = _rng(w.seed, 1).permutation(num_blocks)
    bt = np.full((len(ctx), max_blocks), -1, np.int32)
    start = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = ids[start:start + n]
        start += int(n)
    return bt, num_blocks


def query(w: Workload) -> np.ndarray:
    return _rng(w.seed, 2).standard_normal((w.batch, w.num_q_heads, HEAD_DIM),
                                           dtype=np.float32).astype(np.float16)


def outlier_channels(w: Workload) -> np.ndarray:
    if w.outliers <= 0:
        return np.zeros((w.num_kv_heads, 0), np.int64)
    r = _rng(w.seed, 3)
    return np.stack([r.choice(HEAD_DIM, size=w.outliers, replace=False)
                     for _ in range(w.num_kv_heads)])


def kv_rows(w: Workload, b: int, n: int, channels: np.ndarray | None = None):
    """Sequence b's n K and V rows, fp16 [n][Hkv][128] each."""
    r = _rng(w.seed, 4, b)
    k = r.standard_normal((n, w.num_kv_heads, HEAD_DIM), dtype=np.float32)
    v = r.standard_normal((n, w.num_kv_heads, HEAD_DIM), dtype=np.float32)
    if w.outliers > 0:
        ch = outlier_channels(w) if channels is None else channels
        gain = np.float32(w.outlier_gain)
        for g in range(w.num_kv_heads):
            k[:, g, ch[g]] *= gain
            v[:, g, ch[g]] *= gain
    return k.astype(np.float16), v.astype(np.float16)


def all_kv_rows(w: Workload, ctx: np.ndarray, threads: int = 1):
    """All sequences' rows concatenated: (k [T][Hkv][128], v [T][Hkv][128], cu [B+1]).  Each
    sequence has its own stream, so `threads` > 1 draws them concurrently with the same result."""
    ch = outlier_channels(w)
    cu = np.zeros(len(ctx) + 1, np.int32)
    cu[1:] = np.cumsum(ctx)
    T = int(cu[-1])
    k = np.empty((T, w.num_kv_heads, HEAD_DIM), np.float16)
    v = np.empty((T, w.num_kv_heads, HEAD_DIM), np.float16)

    def one(b):
        kb, vb = kv_rows(w, b, int(ctx[b]), ch)
        k[cu[b]:cu[b + 1]] = kb
        v[cu[b]:cu[b + 1]] = vb

    if threads <= 1:
        for b in range(len(ctx)):
            one(b)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(len(ctx))))
    return k, v, cu


def kv_scale(w: Workload, k: np.ndarray | None = None, v: np.ndarray | None = None,
             ctx: np.ndarray | None = None) -> float:
    """Per-tensor scale: 1.0, or fl32(amax over K and V) / 448 or / 240 (synthetic calibration to
    the largest finite E4M3 or E4M3FNUZ value)."""
    if w.scale_rule == "one" or w.dtype in ("int8", "int4"):
        return 1.0
    if w.scale_rule not in ("amax/448", "amax/240"):
        raise ValueError(w.scale_rule)
    top = np.float32(448.0) if w.scale_rule == "amax/448" else np.float32(240.0)
    if k is not None and v is not None:
        amax = max(float(np.abs(k).max(initial=0)), float(np.abs(v).max(initial=0)))
    else:
        assert ctx is not None
        ch = outlier_channels(w)
        amax = 0.0
        for b, n in enumerate(ctx):
            kb, vb = kv_rows(w, b, int(n), ch)
            amax = max(amax, float(np.abs(kb).max(initial=0)), float(np.abs(vb).max(initial=0)))
    if amax == 0.0:  # no values at all (every sequence empty): the default scale
        return 1.0
    return float(np.float32(amax) / top)
