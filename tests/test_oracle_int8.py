"""Pins of the oracle's online INT8 row encoder.

The online INT8 cache of "[Feature] TurboMind support W8A8 or FP8 KV Cache" comes with no formula;
the reading is symmetric INT8 with one fp32 scale per (token, head): s = fl32(amax / 127),
q = clamp(rne(fl32(x / s)), -127, 127), a zero row giving s = 0 and q = 0.  The pins: numpy's
rint (round half to even) and clip on numpy's IEEE float32 arithmetic, and invariants that hold
for any correct encoder.
"""
import numpy as np
import pytest


def _rows(seed, rows, n=128, outliers=False):
    r = np.random.default_rng(seed)
    x = r.standard_normal((rows, n), dtype=np.float32)
    if outliers:
        for i in range(rows):
            x[i, r.choice(n, 4, replace=False)] *= np.float32(20)
    return x.astype(np.float16)


@pytest.mark.parametrize("outliers", [False, True])
def test_int8_matches_numpy_rint(oracle_mod, outliers):
    x = _rows(7, 4096, outliers=outliers)
    q, s = oracle_mod.int8_quantize_rows(x)
    xf = x.astype(np.float32)
    amax = np.abs(xf).max(axis=1)
    s_ref = amax / np.float32(127.0)
    np.testing.assert_array_equal(s, s_ref)
    q_ref = np.clip(np.rint(xf / s_ref[:, None]), -127, 127).astype(np.int8)
    np.testing.assert_array_equal(q, q_ref)


def test_int8_invariants(oracle_mod):
    x = _rows(8, 2048, outliers=True)
    q, s = oracle_mod.int8_quantize_rows(x)
    xf = x.astype(np.float64)
    # the largest-magnitude element of every row gets |q| = 127, with its sign
    i = np.abs(xf).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(len(q)), i]) == 127)
    assert np.all(np.sign(q[np.arange(len(q)), i]) == np.sign(xf[np.arange(len(q)), i]))
    # codes stay in [-127, 127]; -128 is never produced
    assert q.min() >= -127 and q.max() <= 127
    # reconstruction error: |x - q s| <= s (1/2 + 2^-16): half a step plus the fp32 quotient's error
    err = np.abs(xf - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 2.0 ** -16))
    # sign symmetry: encoding -x negates the codes and keeps the scale
    q2, s2 = oracle_mod.int8_quantize_rows(-x)
    np.testing.assert_array_equal(q2, -q)
    np.testing.assert_array_equal(s2, s)


def test_int8_zero_row_and_ties(oracle_mod):
    x = np.zeros((3, 128), np.float16)
    # row 1: amax 127 so s = 1 and the quotients are the values themselves; x.5 ties go to even
    x[1, :8] = np.array([127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5], np.float16)
    # row 2: a single nonzero element
    x[2, 5] = np.float16(-3.0)
    q, s = oracle_mod.int8_quantize_rows(x)
    assert s[0] == 0.0 and np.all(q[0] == 0)
    assert s[1] == 1.0
    np.testing.assert_array_equal(q[1, :8], [127, 0, 2, 2, 0, -2, -2, 126])
    assert s[2] == np.float32(3.0) / np.float32(127.0)
    assert q[2, 5] == -127 and np.count_nonzero(q[2]) == 1
