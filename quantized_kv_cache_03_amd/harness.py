"""Device-side set-up of a synthetic decode workload through the library's own entry points.

Allocates one layer's paged cache on the GPU, fills it with kvq_append (a prefill over every
sequence's rows, optionally all but the last), and prepares the decode step: one new token per
sequence (the last row of each sequence, written to its slot; repeated steps rewrite the same bytes,
so they are idempotent) followed by the attention, as one kvq_decode_step call or as kvq_append then
kvq_paged_decode_attn.  Host arrays come from ``workloads``; nothing here computes the method.
"""
from __future__ import annotations

import numpy as np
import torch

from . import kvq as K
from . import workloads as W

# rows generated and uploaded per prefill chunk (bounds host memory for the largest workloads)
_CHUNK_ROWS = 1 << 20


def kv_bytes_per_token(dtype: str) -> int:
    """Bytes one (token, KV head) occupies in the cache: K and V codes plus their per-token scale
    (INT8) or (scale, zero point) pair (INT4)."""
    return {"int8": 2 * W.HEAD_DIM + 8, "int4": W.HEAD_DIM + 16}.get(dtype, 2 * W.HEAD_DIM)


class DeviceCase:
    def __init__(self, w: W.Workload, device: str = "cuda", spare_blocks: int = 0,
                 keep_host_rows: bool = False, poison: bool = True, verbose: bool = False,
                 prefill_last: bool = True, threads: int = 1, rows=None):
        """prefill_last=False leaves each sequence's last slot unwritten (poisoned), so the first
        decode step is the only writer of the appended token.  threads: host threads drawing the
        rows (the same rows for any count).  rows: the (k, v, cu) that W.all_kv_rows gives for
        this workload's recipe, drawn once and shared by several cases (kept as the host rows)."""
        self.w = w
        self.device = device
        self.ctx = W.context_lens(w)
        self.bt, self.num_blocks = W.block_tables(w, self.ctx, spare_blocks=spare_blocks)
        self.B = w.batch
        self.max_ctx = int(self.ctx.max()) if self.B else 0
        self.channels = W.outlier_channels(w)
        total_vals = int(self.ctx.sum()) * w.num_kv_heads * W.HEAD_DIM * 2
        in_memory = keep_host_rows or rows is not None or total_vals <= (1 << 31)
        self.k_host = self.v_host = None
        if rows is not None:
            keep_host_rows = True
        if in_memory:
            k, v, cu = rows if rows is not None else W.all_kv_rows(w, self.ctx, threads=threads)
            assert k.shape[0] == int(self.ctx.sum()) and v.shape == k.shape
            self.kv_scale = W.kv_scale(w, k, v)
            if keep_host_rows:
                self.k_host, self.v_host, self.cu = k, v, cu
        else:
            k = v = None
            self.kv_scale = W.kv_scale(w, ctx=self.ctx)
        self.cache = K.PagedKVCache.allocate(w.dtype, self.num_blocks, w.num_kv_heads, self.kv_scale,
                                             device=device, poison=poison)
        self.bt_d = torch.from_numpy(self.bt).to(device)
        self.ctx_d = torch.from_numpy(self.ctx).to(device)
        self.q = W.query(w)
        self.q_d = torch.from_numpy(self.q).to(device)
        self.out_d = torch.empty_like(self.q_d)
        self._prefill(k, v, verbose, 0 if prefill_last else 1)
        # the decode step's new rows: the last row of each sequence
        # (an empty sequence appends nothing: its row stays zero)
        last_k = np.zeros((self.B, w.num_kv_heads, W.HEAD_DIM), np.float16)
        last_v = np.zeros_like(last_k)
        has = self.ctx > 0
        if k is not None:
            cu = np.concatenate([[0], np.cumsum(self.ctx)])
            last_k[has] = k[cu[1:][has] - 1]
            last_v[has] = v[cu[1:][has] - 1]
        else:
            for b, n in enumerate(self.ctx):
                if n > 0:
                    kb, vb = W.kv_rows(w, b, int(n), self.channels)
                    last_k[b], last_v[b] = kb[-1], vb[-1]
        self.step_k_host, self.step_v_host = last_k, last_v
        self.step_k_d = torch.from_numpy(last_k).to(device)
        self.step_v_d = torch.from_numpy(last_v).to(device)
        self.partition_size = w.partition_size
        self.workspace, self.workspace_bytes = K.alloc_workspace(
            self.B, w.num_q_heads, w.num_kv_heads, self.max_ctx, self.partition_size, device=device)
        torch.cuda.synchronize()

    def _prefill(self, k, v, verbose, skip: int):
        """Append every sequence's rows but the last `skip` ones, in chunks of sequences."""
        w, ctx = self.w, self.ctx
        pre = np.maximum(ctx - skip, 0).astype(np.int32)
        pre_d = torch.from_numpy(pre).to(self.device)
        b0 = 0
        while b0 < self.B:
            b1, rows = b0, 0
            while b1 < self.B and (rows == 0 or rows + int(ctx[b1]) <= _CHUNK_ROWS):
                rows += int(ctx[b1])
                b1 += 1
            if k is not None:
                cu_all = np.concatenate([[0], np.cumsum(ctx)])
                kc = np.concatenate([k[cu_all[b]:cu_all[b] + pre[b]] for b in range(b0, b1)])
                vc = np.concatenate([v[cu_all[b]:cu_all[b] + pre[b]] for b in range(b0, b1)])
            else:
                parts = [W.kv_rows(w, b, int(ctx[b]), self.channels) for b in range(b0, b1)]
                kc = np.concatenate([p[0][:pre[b0 + i]] for i, p in enumerate(parts)])
                vc = np.concatenate([p[1][:pre[b0 + i]] for i, p in enumerate(parts)])
            cu = np.zeros(b1 - b0 + 1, np.int32)
            cu[1:] = np.cumsum(pre[b0:b1])
            if int(cu[-1]) > 0:
                kd = torch.from_numpy(np.ascontiguousarray(kc)).to(self.device)
                vd = torch.from_numpy(np.ascontiguousarray(vc)).to(self.device)
                K.append(self.cache, kd, vd, self.bt_d[b0:b1].contiguous(), pre_d[b0:b1].contiguous(),
                         cu_new_lens=torch.from_numpy(cu).to(self.device), num_new_rows=int(cu[-1]))
            if verbose:
                print(f"  prefill sequences {b0}..{b1 - 1} ({rows} rows)", flush=True)
            b0 = b1
        torch.cuda.synchronize()

    # one decode step of one layer: append one token per sequence, then attention
    def append_step(self, stream=None):
        K.append(self.cache, self.step_k_d, self.step_v_d, self.bt_d, self.ctx_d, stream=stream)

    def attention(self, partition_size: int | None = None, stream=None, out=None):
        """kvq_paged_decode_attn (kvq_paged_decode_attn_fp8math for an FP8-math workload)."""
        ps = self.partition_size if partition_size is None else partition_size
        ws = self.workspace if ps == self.partition_size else None
        fn = K.paged_decode_attn_fp8math if self.w.fp8_math else K.paged_decode_attn
        return fn(self.cache, self.q_d, self.bt_d, self.ctx_d, self.max_ctx, partition_size=ps,
                  workspace=ws, out=self.out_d if out is None else out, stream=stream)

    def step(self, stream=None, fused: bool = True):
        """One decode step: append one token per sequence, then attention (one fused call, or
        kvq_append followed by the attention call); FP8 math for an FP8-math workload."""
        if not fused:
            self.append_step(stream)
            return self.attention(stream=stream)
        fn = K.decode_step_fp8math if self.w.fp8_math else K.decode_step
        return fn(self.cache, self.step_k_d, self.step_v_d, self.q_d, self.bt_d, self.ctx_d,
                  self.max_ctx, partition_size=self.partition_size, workspace=self.workspace,
                  out=self.out_d, stream=stream)

    def prepared_step(self, cache=None, stream=None) -> K.PreparedCall:
        """The fused step of step() on `cache` (default: this case's), checked and marshalled once."""
        return K.prepare_decode_step(self.cache if cache is None else cache, self.step_k_d, self.step_v_d,
                                     self.q_d, self.bt_d, self.ctx_d, self.max_ctx,
                                     partition_size=self.partition_size, workspace=self.workspace,
                                     out=self.out_d, stream=stream, fp8_math=self.w.fp8_math)

    # host views of the sequences' own rows (regenerated from the seeds)
    def rows_of(self, b: int):
        if self.k_host is not None:
            return self.k_host[self.cu[b]:self.cu[b + 1]], self.v_host[self.cu[b]:self.cu[b + 1]]
        return W.kv_rows(self.w, b, int(self.ctx[b]), self.channels)

    def algorithmic_bytes(self) -> int:
        """Bytes the decode step must move at least once (see the measurement notes)."""
        w = self.w
        sctx = int(self.ctx.sum())
        per_tok = kv_bytes_per_token(w.dtype)
        kv = sctx * w.num_kv_heads * per_tok
        qo = 2 * self.B * w.num_q_heads * W.HEAD_DIM * 2
        table = 4 * int(((self.ctx + 15) // 16).sum()) + 4 * self.B
        # append: the fp16 K and V rows in, their codes and scales out
        append = self.B * w.num_kv_heads * (2 * W.HEAD_DIM * 2 + per_tok)
        return kv + qo + table + append

    def attention_bytes(self) -> int:
        """Algorithmic bytes of the attention alone (codes, scales, table, q in, out)."""
        w = self.w
        sctx = int(self.ctx.sum())
        per_tok = kv_bytes_per_token(w.dtype)
        return (sctx * w.num_kv_heads * per_tok + 2 * self.B * w.num_q_heads * W.HEAD_DIM * 2
                + 4 * int(((self.ctx + 15) // 16).sum()) + 4 * self.B)
