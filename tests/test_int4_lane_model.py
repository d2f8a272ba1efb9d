"""CPU model of the INT4 matrix-core kernels' lane mapping (no GPU): which bytes of a (block, KV
head) tile each lane loads, which codes it reads out of them, and where the per-token (scale, zero
point) pairs it needs come from.  The kernels' own formulas, restated:
  lane l, q4 = l / 16, col = l % 16; both 16-byte loads at byte 256 q4 + 16 col of the K and the V
  tile;
  K: token col, dims 32 q4 .. +31, dim 32 q4 + 2 j + h in nibble h of byte j;
  V: the four tokens 4 q4 + u of the dims col + 16 r, unit r = bits 16 (r % 2) .. +15 of dword r / 2,
     token 4 q4 + u in nibble u % 2 of byte u / 2 of the unit;
  own token (the lane's loaded pairs) = 4 q4 + l % 4; quad_bcast<U> reads lane (l & ~3) + U; the
  K operand row's zero code comes by shuffle from lane 16 (col / 4) + col % 4.
The codes come from the oracle's append into its own implementation of the documented layout and
from its row quantizer; the accumulator layout of v_mfma_f32_16x16x32_f16 (lane l holds rows
4 (l / 16) .. +3 of column l % 16) is the instruction's documented one.  A wrong offset, nibble
order or broadcast source fails here before any GPU run."""
import numpy as np
import pytest

import oracle

LANES = 64
BLOCK = 16
DIM = 128


def lane_parts(l):
    return l // 16, l % 16


def own_token(l):
    q4, _ = lane_parts(l)
    return 4 * q4 + (l & 3)


def load_offset(l):
    q4, col = lane_parts(l)
    return 256 * q4 + 16 * col


def k_codes_of_lane(tile, l):
    """{(token, dim): code} the lane reads from its 16 K bytes."""
    q4, col = lane_parts(l)
    b = tile[load_offset(l):load_offset(l) + 16]
    out = {}
    for j in range(16):
        for h in range(2):
            out[(col, 32 * q4 + 2 * j + h)] = (int(b[j]) >> (4 * h)) & 0xF
    return out


def v_codes_of_lane(tile, l):
    """{(token, dim): code} the lane reads from its 16 V bytes, unit by unit."""
    q4, col = lane_parts(l)
    b = tile[load_offset(l):load_offset(l) + 16]
    dwords = b.view("<u4")
    out = {}
    for r in range(8):
        unit = (int(dwords[r // 2]) >> (16 * (r % 2))) & 0xFFFF
        for u in range(4):
            byte = (unit >> (8 * (u // 2))) & 0xFF
            out[(4 * q4 + u, col + 16 * r)] = (byte >> (4 * (u % 2))) & 0xF
    return out


@pytest.fixture(scope="module")
def tiles():
    """One full INT4 tile of K and of V written by the oracle's append, and the codes its row
    quantizer gives for the same rows."""
    rng = np.random.default_rng(20261202)
    hkv, head = 2, 1
    k = (rng.standard_normal((BLOCK, hkv, DIM)) * 1.5).astype(np.float16)
    v = (rng.standard_normal((BLOCK, hkv, DIM)) * 0.7).astype(np.float16)
    cache = oracle.Cache(oracle.INT4, num_blocks=3, num_kv_heads=hkv)
    oracle.append(cache, k, v, np.array([[0, 0, 2]], np.int32), np.array([3 * BLOCK], np.int32),
                  np.array([0, BLOCK], np.int32))  # the sequence's last 16 positions: its third block
    kq, _, _ = oracle.int4_quantize_rows(k[:, head])
    vq, _, _ = oracle.int4_quantize_rows(v[:, head])
    return cache.k[2, head], cache.v[2, head], kq, vq


def test_k_loads_cover_the_tile_once(tiles):
    kt, _, kq, _ = tiles
    seen = {}
    for l in range(LANES):
        for key, code in k_codes_of_lane(kt, l).items():
            assert key not in seen, f"K (token, dim) {key} read by two lanes"
            seen[key] = code
    assert len(seen) == BLOCK * DIM
    for (t, d), code in seen.items():
        assert code == kq[t, d], (t, d)


def test_k_lane_is_one_token_of_one_chunk(tiles):
    kt = tiles[0]
    for l in range(LANES):
        q4, col = lane_parts(l)
        keys = k_codes_of_lane(kt, l).keys()
        assert {t for t, _ in keys} == {col}
        assert sorted(d for _, d in keys) == list(range(32 * q4, 32 * q4 + 32))


def test_v_loads_cover_the_tile_once(tiles):
    _, vt, _, vq = tiles
    seen = {}
    for l in range(LANES):
        for key, code in v_codes_of_lane(vt, l).items():
            assert key not in seen, f"V (token, dim) {key} read by two lanes"
            seen[key] = code
    assert len(seen) == BLOCK * DIM
    for (t, d), code in seen.items():
        assert code == vq[t, d], (t, d)


def test_v_lane_tokens_are_its_accumulator_rows(tiles):
    """The P V^T products pair a lane's V units with the weights of the tokens its accumulator rows
    hold: both must be the tokens 4 (l / 16) .. +3."""
    vt = tiles[1]
    for l in range(LANES):
        q4, col = lane_parts(l)
        keys = v_codes_of_lane(vt, l).keys()
        acc_rows = {4 * q4 + u for u in range(4)}  # accumulator rows of v_mfma_f32_16x16x32_f16
        assert {t for t, _ in keys} == acc_rows
        assert {d for _, d in keys} == {col + 16 * r for r in range(8)}


def test_quad_broadcasts_bring_every_accumulator_token():
    for l in range(LANES):
        q4 = l // 16
        for u in range(4):
            src = (l & ~3) + u
            assert src // 4 == l // 4  # inside the lane's quad (DPP quad_perm)
            assert own_token(src) == 4 * q4 + u  # the lane's accumulator row u


def test_shuffle_source_owns_the_operand_row():
    for l in range(LANES):
        col = l % 16
        src = 16 * (col >> 2) + (col & 3)
        assert own_token(src) == col


def test_every_token_owned_by_four_lanes_of_one_row():
    owners = {}
    for l in range(LANES):
        owners.setdefault(own_token(l), []).append(l)
    assert sorted(owners) == list(range(BLOCK))
    for t, ls in owners.items():
        assert len(ls) == 4
        assert {l // 16 for l in ls} == {t // 4}


def test_pending_token_stores_go_where_the_lanes_loaded():
    """The fused step's held-back stores: lanes 0..3 write the new token's K bytes of chunk lane (16
    bytes at 256 lane + 16 slot), and the 16 lanes of the token's quad write back the 16 V bytes
    each of them loaded.  Every byte the oracle's append of that one token changes lies inside
    those stores."""
    rng = np.random.default_rng(7)
    for slot in range(BLOCK):
        cache = oracle.Cache(oracle.INT4, num_blocks=1, num_kv_heads=1, poison=False)
        row = (rng.standard_normal((1, 1, DIM)) * 2.0).astype(np.float16)
        oracle.append(cache, row, row, np.array([[0]], np.int32), np.array([slot + 1], np.int32))
        k_changed = set(np.flatnonzero(cache.k[0, 0]))
        v_changed = set(np.flatnonzero(cache.v[0, 0]))
        assert k_changed and v_changed
        k_stores = {256 * c + 16 * slot + j for c in range(4) for j in range(16)}
        writers = [l for l in range(LANES) if l // 16 == slot // 4]
        v_stores = {load_offset(l) + j for l in writers for j in range(16)}
        assert k_changed <= k_stores, slot
        assert v_changed <= v_stores, slot
