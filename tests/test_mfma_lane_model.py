"""CPU model of the 8-bit matrix-core kernels' operand mapping (no GPU): the grouped decode kernel
and the prefill kernel read a K tile with two 16-byte loads per lane (bytes 16 l and 1024 + 16 l)
and a V tile with one dword per lane and row block (byte 16 col + 4 q4 + 256 r), and build the
operands of v_mfma_f32_16x16x32_f16 from them.  The kernels' formulas, restated:
  lane l, q4 = l / 16, col = l % 16;
  S^T = K Q^T, MFMA m = 0..3: A k-slots 8 q4 .. +7 of lane l = bytes 8 (m % 2) .. +7 of the load
  at 1024 (m / 2) + 16 l; B k-slots of lane l = query dims 64 (m / 2) + 16 q4 + 8 (m % 2) .. +7;
  O^T += V^T P^T, row block r: A k-slots of lane l = the dword at 16 col + 4 q4 + 256 r of tile 0
  (slots 0..3) and of tile 1 (slots 4..7); B k-slots = the weights of the accumulator rows of S^T
  (tokens 4 q4 + t of tiles 0 and 1) in the same order.
The instruction's documented layout: in A and B lane l holds row (column) l % 16 and k-slots
8 (l / 16) .. +7; in C it holds rows 4 (l / 16) .. +3 of column l % 16.  The codes come from the
oracle's append into its own implementation of the documented cache layout.  The model checks that
every product the instruction forms pairs a K code (V code) with the query value (weight) of the
same dim (token), and that each output sums over every dim (token) exactly once."""
import numpy as np
import pytest

import oracle

LANES = 64
BLOCK = 16
DIM = 128


def k_slot(l, m, s):
    """(tile byte offset) of A k-slot s of lane l in S^T MFMA m."""
    return 1024 * (m // 2) + 16 * l + 8 * (m % 2) + s


def q_dim(l, m, s):
    return 64 * (m // 2) + 16 * (l // 16) + 8 * (m % 2) + s


def k_byte_to(off):
    """The oracle's K layout, inverted: byte (d / 16) 256 + t 16 + d % 16 -> (token, dim)."""
    return (off % 256) // 16, (off // 256) * 16 + off % 16


def v_slot(l, r, s):
    """(tile, byte offset) of A k-slot s of lane l in P V^T row block r."""
    q4, col = l // 16, l % 16
    return s // 4, 16 * col + 4 * q4 + 256 * r + s % 4


def v_byte_to(off):
    """The oracle's V layout, dim-major: byte d 16 + t -> (token, dim)."""
    return off % 16, off // 16


def weight_slot(l, s):
    """(tile, token) of the weight in B k-slot s of lane l: the S^T accumulator row 4 q4 + s % 4 of
    tile s / 4 (the hi / lo dwords are joined in that order)."""
    return s // 4, 4 * (l // 16) + s % 4


@pytest.fixture(scope="module")
def cache():
    rng = np.random.default_rng(1202)
    k = (rng.standard_normal((2 * BLOCK, 1, DIM)) * 3).astype(np.float16)
    v = (rng.standard_normal((2 * BLOCK, 1, DIM)) * 3).astype(np.float16)
    c = oracle.Cache(oracle.E4M3, num_blocks=4, num_kv_heads=1)
    oracle.append(c, k, v, np.array([[3, 1]], np.int32), np.array([2 * BLOCK], np.int32),
                  np.array([0, 2 * BLOCK], np.int32))
    kq = oracle.fp8_quantize(oracle.E4M3, k[:, 0])
    vq = oracle.fp8_quantize(oracle.E4M3, v[:, 0])
    return c, kq, vq


def test_k_operand_bytes_hold_the_lane_row(cache):
    c, kq, _ = cache
    tile = c.k[3, 0]  # the sequence's first block
    for l in range(LANES):
        for m in range(4):
            for s in range(8):
                t, d = k_byte_to(k_slot(l, m, s))
                assert t == l % 16  # A row of lane l
                assert tile[k_slot(l, m, s)] == kq[t, d]


def test_s_products_pair_equal_dims():
    """C[i][j] = sum over MFMAs m and k-slots k = 8 g + s of A[i][k] (lane i + 16 g) times
    B[k][j] (lane j + 16 g): the K dim and the query dim of each product agree, and every dim
    appears once per output."""
    for i in range(16):
        for j in range(16):
            dims = []
            for m in range(4):
                for g in range(4):
                    for s in range(8):
                        _, dk = k_byte_to(k_slot(i + 16 * g, m, s))
                        assert dk == q_dim(j + 16 * g, m, s)
                        dims.append(dk)
            assert sorted(dims) == list(range(DIM))


def test_v_operand_bytes_hold_the_lane_dim(cache):
    c, _, vq = cache
    tiles = (c.v[3, 0], c.v[1, 0])  # blocks of tokens 0..15 and 16..31
    for l in range(LANES):
        for r in range(8):
            for s in range(8):
                tile, off = v_slot(l, r, s)
                t, d = v_byte_to(off)
                assert d == l % 16 + 16 * r  # A row of lane l in row block r
                assert tiles[tile][off] == vq[16 * tile + t, d]


def test_pv_products_pair_equal_tokens():
    for i in range(16):
        for j in range(16):
            toks = []
            for g in range(4):
                for s in range(8):
                    tile, off = v_slot(i + 16 * g, 0, s)
                    tv, _ = v_byte_to(off)
                    tw_tile, tw = weight_slot(j + 16 * g, s)
                    assert (tile, tv) == (tw_tile, tw)
                    toks.append(16 * tile + tv)
            assert sorted(toks) == list(range(2 * BLOCK))


def test_weights_come_from_the_lane_accumulator_rows():
    """The weight in B k-slot s of lane l is one the lane itself holds: S^T's accumulator gives
    lane l the rows (tokens) 4 (l / 16) .. +3 of column l % 16."""
    for l in range(LANES):
        rows = {4 * (l // 16) + u for u in range(4)}
        for s in range(8):
            _, t = weight_slot(l, s)
            assert t in rows


def test_output_rows_cover_every_dim_once():
    """O^T's accumulator gives lane l the rows 16 r + 4 (l / 16) .. +3 of column l % 16, stored at
    those dims of the column's output row: over the four row groups and eight row blocks every
    dim is written exactly once."""
    covered = sorted(16 * r + 4 * q4 + e for q4 in range(4) for r in range(8) for e in range(4))
    assert covered == list(range(DIM))


def perm_b32(hi_src, lo_src, sel):
    """v_perm_b32: byte i of the result is byte sel_i of the 8-byte value (hi_src:lo_src), for the
    selector values 0..7 used here."""
    pool = list(int(lo_src).to_bytes(4, "little")) + list(int(hi_src).to_bytes(4, "little"))
    return int.from_bytes(bytes(pool[(sel >> (8 * i)) & 0xFF] for i in range(4)), "little")


def test_staged_int8_decode_is_exact():
    """The prefill kernel stages INT8 codes with their sign bits flipped and decodes a pair by
    placing each byte under a 0x64 high byte (the binary16 number 1024 + byte) and subtracting
    1152 in binary16: every signed code comes back exactly, in its slot."""
    rng = np.random.default_rng(5)
    codes = np.arange(-128, 128, dtype=np.int64)
    for _ in range(4):
        quads = np.stack([codes, rng.permutation(codes), rng.permutation(codes), rng.permutation(codes)], 1)
        for c in quads:
            w = sum((int(c[i]) & 0xFF) << (8 * i) for i in range(4)) ^ 0x80808080  # the staging flip
            for pair, sel in ((0, 0x04010400), (1, 0x04030402)):
                x = perm_b32(0x64646464, w, sel)
                halves = np.array([x & 0xFFFF, x >> 16], np.uint16).view(np.float16)
                got = (halves - np.float16(1152)).astype(np.float64)
                assert list(got) == [c[2 * pair], c[2 * pair + 1]]


def test_int8_scale_row_lanes():
    """INT8 staging: lanes 0..7 of the K-staging wave carry a tile's scale row as four floats each
    (the oracle's row: the 16 K scales, then the 16 V scales of the tile's tokens), and the softmax
    of lane l reads the K and V scales of its accumulator rows 4 (l / 16) + t at 4 q4 + t and
    16 + 4 q4 + t of the staged row."""
    rng = np.random.default_rng(11)
    k = (rng.standard_normal((BLOCK, 1, DIM)) * np.arange(1, BLOCK + 1)[:, None, None]).astype(np.float16)
    v = (rng.standard_normal((BLOCK, 1, DIM)) * np.arange(BLOCK, 0, -1)[:, None, None]).astype(np.float16)
    c = oracle.Cache(oracle.INT8, num_blocks=2, num_kv_heads=1)
    oracle.append(c, k, v, np.array([[1]], np.int32), np.array([BLOCK], np.int32), np.array([0, BLOCK], np.int32))
    _, ks = oracle.int8_quantize_rows(k[:, 0])
    _, vs = oracle.int8_quantize_rows(v[:, 0])
    flat = c.rows[1, 0].reshape(-1)  # the 128-byte row as stored
    staged = np.empty(2 * BLOCK, np.float32)
    for lane in range(8):  # lane's float4 at 4 lane
        staged[4 * lane:4 * lane + 4] = flat[4 * lane:4 * lane + 4]
    for l in range(LANES):
        q4 = l // 16
        for t in range(4):
            assert staged[4 * q4 + t] == ks[4 * q4 + t]
            assert staged[BLOCK + 4 * q4 + t] == vs[4 * q4 + t]
