"""CPU model of the balanced split's index arithmetic (no GPU): the walk each wave makes over the
sequences' tiles laid end to end, and the writer ranges the merge rebuilds from the prefix table.
The formulas are the kernels' own, restated:
  T tiles in all; nw = 1 if T == 0 else min(NW, ceil(T / 8)); wave w takes [floor(w T / nw),
  floor((w + 1) T / nw)); a segment is the piece of one sequence inside a share; a sequence whose
  tiles fall in more than one share gets partial rows w + b (per head), merged over the waves
  wave_of_tile(c0) .. wave_of_tile(c0 + nt - 1), wave_of_tile(c) = ceil((c + 1) nw / T) - 1.
On 3000 seeded batches (ragged, with empty sequences, one huge sequence, thousands of short ones)
the model checks that every tile is covered exactly once and in order, that the partial rows are
unique and inside the workspace's NW + B rows per head, and that the merge's ranges are exactly the
waves that wrote partials -- the properties the GPU tests check end to end."""
import numpy as np

MIN_TILES = 8
BALANCED_WAVES = 2048


def host_nw(batch, hq, hkv, max_ctx, waves=None):
    """NW of the host plan.  The workspace is sized for the largest wave target of the shape: twice
    BALANCED_WAVES with one query head per KV head (the INT8 one-head kernel's target)."""
    if waves is None:
        waves = 2 * BALANCED_WAVES if hq == hkv else BALANCED_WAVES
    hw = hq if hq == hkv else hkv
    max_tiles = batch * ((max_ctx + 15) // 16)
    nw = (waves + hw - 1) // hw
    nw = min(nw, max(1, (max_tiles + MIN_TILES - 1) // MIN_TILES))
    return min(nw, 65535)


def walk(ctx, NW):
    nt = (ctx + 15) // 16
    incl = np.cumsum(nt)
    T = int(incl[-1]) if len(nt) else 0
    nw = 1 if T == 0 else min(NW, -(-T // MIN_TILES))
    segs = []
    for w in range(nw):
        s0, s1 = w * T // nw, (w + 1) * T // nw
        cur = s0
        while cur < s1:
            b = int(np.searchsorted(incl, cur, side="right"))  # first sequence whose tiles pass cur
            c0 = int(incl[b] - nt[b])
            hi = min(int(nt[b]), s1 - c0)
            segs.append((w, b, cur - c0, hi))
            cur = c0 + hi
    return T, nw, nt, incl - nt, segs


def wave_of_tile(c, T, nw):
    return ((c + 1) * nw + T - 1) // T - 1


def check(ctx, NW):
    T, nw, nt, c0, segs = walk(ctx, NW)
    B = len(ctx)
    covered = [[] for _ in range(B)]
    last = {}
    for w, b, lo, hi in segs:
        assert 0 <= lo < hi <= nt[b]
        # a wave's segments follow one another in tile order
        if w in last:
            assert c0[b] + lo == last[w]
        last[w] = c0[b] + hi
        covered[b].append((lo, hi, w))
    rows = set()
    for b in range(B):
        pieces = sorted(covered[b])
        if nt[b] == 0:
            assert not pieces
            continue
        # every tile exactly once
        assert pieces[0][0] == 0 and pieces[-1][1] == nt[b]
        assert all(pieces[i][1] == pieces[i + 1][0] for i in range(len(pieces) - 1))
        writers = [w for _, _, w in pieces]
        wlo, whi = wave_of_tile(int(c0[b]), T, nw), wave_of_tile(int(c0[b] + nt[b] - 1), T, nw)
        assert writers == list(range(wlo, whi + 1))
        if wlo == whi:
            assert pieces == [(0, int(nt[b]), wlo)]  # one wave, final output written directly
        else:
            for w in writers:
                r = w + b
                assert r not in rows and 0 <= r < NW + B
                rows.add(r)


def test_balanced_split_model_on_random_batches():
    r = np.random.default_rng(4242)
    for i in range(3000):
        kind = i % 4
        B = int(r.integers(1, 300))
        if kind == 0:    # ragged lognormal mix with empty sequences
            ctx = np.where(r.random(B) < 0.2, 0, np.rint(np.exp(r.normal(6.5, 1.5, B)))).clip(0, 40000)
        elif kind == 1:  # many short sequences
            ctx = r.integers(0, 41, B)
        elif kind == 2:  # one huge sequence among short ones
            ctx = r.integers(0, 100, B)
            ctx[int(r.integers(0, B))] = int(r.integers(20000, 140000))
        else:            # uniform
            ctx = r.integers(0, 5000, B)
        ctx = np.asarray(ctx, np.int64)
        hkv = int(r.choice([1, 2, 8, 32]))
        hq = hkv * int(r.choice([1, 4, 8]))
        NW = host_nw(B, hq, hkv, int(ctx.max()))
        if i % 7 == 0:
            NW = int(r.integers(1, 4000))  # any NW the device may receive
        check(ctx, NW)


def test_edge_batches():
    check(np.array([0, 0, 0]), 5)             # nothing to do: one wave, no segments
    check(np.array([1]), 2048)                 # one tile
    check(np.array([16 * 9000]), 2048)         # one sequence over every wave
    check(np.array([17, 0, 33, 1]), 1)         # one wave holds everything
    check(np.full(5000, 16), 2048)             # more sequences than waves


def test_model_nw_is_the_library_plan():
    """The workspace size the library reports for the balanced split encodes its NW (rows =
    Hq (NW + B)); it must equal the size the model's NW gives."""
    from quantized_kv_cache_03_amd import kvq as K

    def align(x):
        return (x + 255) // 256 * 256

    r = np.random.default_rng(7)
    for _ in range(500):
        B = int(r.integers(1, 2000))
        hkv = int(r.choice([1, 2, 4, 8, 32, 64]))
        hq = hkv * int(r.choice([1, 2, 4, 8, 16]))
        L = int(r.choice([0, 1, 16, 17, int(r.integers(1, 200000))]))
        rows = hq * (host_nw(B, hq, hkv, L) + B)
        want = align((B + 2) * 4) + align(rows * 128 * 4) + 2 * align(rows * 4)
        assert K.workspace_size(B, hq, hkv, L, K.PARTITION_BALANCED) == want, (B, hq, hkv, L)
