"""CPU pin of the FP8-math tolerance (gpu_common.fp8_math_slack): logit errors of at most e_t must
move no softmax output by more than the slack it returns.  Small oracle caches with outlier
channels; the logits of the exact FP8-math attention are perturbed by random and by worst-case
sign patterns of size e_t, and the perturbed outputs are compared with the unperturbed ones, in the
decode form (exact softmax) and the prefill form (range bound)."""
import numpy as np
import pytest

import oracle
from gpu_common import FP8_ACCUMULATION, fp8_math_slack

SM = 1.0 / np.sqrt(128.0)


def _case(seed, B, Hkv, G, lens, gain):
    r = np.random.default_rng(seed)
    T = int(sum(lens))
    k = r.standard_normal((T, Hkv, 128)).astype(np.float32)
    v = r.standard_normal((T, Hkv, 128)).astype(np.float32)
    ch = r.choice(128, size=4, replace=False)
    k[:, :, ch] *= gain
    v[:, :, ch] *= gain
    k, v = k.astype(np.float16), v.astype(np.float16)
    amax = float(max(np.abs(k).max(), np.abs(v).max()))
    ctx = np.asarray(lens, np.int32)
    nblk = (ctx + 15) // 16
    bt = np.full((B, int(nblk.max())), -1, np.int32)
    s = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = np.arange(s, s + n)
        s += int(n)
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(ctx)
    cache = oracle.Cache(oracle.E4M3, s, Hkv, amax / 448.0)
    oracle.append(cache, k, v, bt, ctx, cu)
    return r, cache, bt, ctx


def _perturbed_max_moves(r, qh, kd, vd, n, e_scale, trials):
    """Largest |o' - o| per dim over perturbations delta_t in [-e_t, e_t] of the logits."""
    z = SM * (kd[:n] @ qh)
    e = FP8_ACCUMULATION * SM * (np.abs(kd[:n]) @ np.abs(qh)) * e_scale
    p = np.exp(z - z.max())
    p /= p.sum()
    o = p @ vd[:n]
    worst = np.zeros(128)
    for i in range(trials):
        if i < 2 * 128:  # worst-case signs for one dim: push weight toward the largest / smallest v
            d = i % 128
            sgn = np.sign(vd[:n, d] - o[d]) * (1 if i < 128 else -1)
        else:
            sgn = r.choice([-1.0, 1.0], size=n)
        zz = z + sgn * e
        pp = np.exp(zz - zz.max())
        pp /= pp.sum()
        worst = np.maximum(worst, np.abs(pp @ vd[:n] - o))
    return worst


@pytest.mark.parametrize("gain", [1.0, 20.0])
def test_decode_slack_bounds_logit_errors(gain):
    B, Hkv, G = 3, 2, 2
    r, cache, bt, ctx = _case(11 + int(gain), B, Hkv, G, [40, 150, 7], gain)
    q = r.standard_normal((B, Hkv * G, 128)).astype(np.float16)
    slack = fp8_math_slack(cache, q, bt, ctx)
    codes, scales = oracle.quantize_q_fp8_rows(q)
    qh = oracle.fp8_decode(oracle.E4M3, codes) * scales[..., None].astype(np.float64)
    kd, vd = oracle.dequant(cache, bt, ctx, int(ctx.max()))
    for b in range(B):
        for h in range(Hkv * G):
            g = h // G
            moves = _perturbed_max_moves(r, qh[b, h], kd[b, g].astype(np.float64), vd[b, g].astype(np.float64),
                                         int(ctx[b]), 1.0, 300)
            assert np.all(moves <= slack[b, h] * (1 + 1e-9) + 1e-12), (b, h, float((moves - slack[b, h]).max()))
            assert slack[b, h].max() > 0
            # the bound is not vacuous: twice the logit errors exceed it somewhere
            moves2 = _perturbed_max_moves(r, qh[b, h], kd[b, g].astype(np.float64), vd[b, g].astype(np.float64),
                                          int(ctx[b]), 4.0, 256)
            assert np.any(moves2 > slack[b, h])


def test_prefill_slack_bounds_logit_errors():
    B, Hkv, G = 2, 1, 3
    r, cache, bt, ctx = _case(5, B, Hkv, G, [60, 33], 20.0)
    nq = [20, 33]
    cu_q = np.array([0, 20, 53], np.int32)
    q = r.standard_normal((53, Hkv * G, 128)).astype(np.float16)
    slack = fp8_math_slack(cache, q, bt, ctx, cu_q)
    codes, scales = oracle.quantize_q_fp8_rows(q)
    qh = oracle.fp8_decode(oracle.E4M3, codes) * scales[..., None].astype(np.float64)
    kd, vd = oracle.dequant(cache, bt, ctx, int(ctx.max()))
    for b in range(B):
        for j in range(0, nq[b], 3):
            row = int(cu_q[b]) + j
            m = int(ctx[b]) - nq[b] + j + 1
            for h in range(Hkv * G):
                moves = _perturbed_max_moves(r, qh[row, h], kd[b, 0].astype(np.float64),
                                             vd[b, 0].astype(np.float64), m, 1.0, 300)
                assert np.all(moves <= slack[row, h] * (1 + 1e-9) + 1e-12), (row, h)
