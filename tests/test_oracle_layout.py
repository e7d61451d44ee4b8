"""Pins for the oracle's byte layouts against hand-derived bytes (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import layout

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "layout_examples.json")))


def test_segment_4bit_nibble_order():
    for ex in GOLD["segment_4bit"]:
        c = np.zeros(32, dtype=np.int64)
        c[:len(ex["codes_first"])] = ex["codes_first"]
        b = layout.pack_segment(c, 4)
        assert b[:len(ex["bytes_first"])].tolist() == ex["bytes_first"]


def test_segment_3bit_examples():
    for ex in GOLD["segment_3bit"]:
        c = np.zeros(32, dtype=np.int64)
        c[ex["code_index"]] = ex["code"]
        assert layout.pack_segment(c, 3).tolist() == ex["bytes"], ex["why"]


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_segment_round_trip(bits):
    rng = np.random.default_rng(bits)
    c = rng.integers(0, 2 ** bits, size=(100, 32))
    b = layout.pack_segment(c, bits)
    assert b.shape == (100, 4 * bits)
    assert np.array_equal(layout.unpack_segment(b, bits), c)
    # every bit of the segment is used by exactly one code: all-ones codes give all-ones bytes
    full = layout.pack_segment(np.full(32, 2 ** bits - 1), bits)
    assert np.all(full == 255)


def test_k_row_is_a_permutation_and_examples():
    chans = sorted(layout.k_row_channel(q, u) for q in range(4) for u in range(32))
    assert chans == list(range(128))
    for ex in GOLD["k_row_4bit"]:
        codes = np.zeros((1, 128), dtype=np.int64)
        codes[0, ex["channel"]] = ex["code"]
        row = layout.pack_k_rows(codes, 4)[0]
        nz = np.nonzero(row)[0].tolist()
        assert nz == [ex["byte_index"]] and row[ex["byte_index"]] == ex["byte"], ex["why"]
    for ex in GOLD["k_row_8bit"]:
        codes = np.zeros((1, 128), dtype=np.int64)
        codes[0, ex["channel"]] = ex["code"]
        row = layout.pack_k_rows(codes, 8)[0]
        assert np.nonzero(row)[0].tolist() == [ex["byte_index"]]
        assert row[ex["byte_index"]] == ex["byte"], ex["why"]


def test_v_tile_is_a_bijection_and_examples():
    pos = sorted(layout.v_tile_position(L, s, u) for L in range(64) for s in range(2)
                 for u in range(32))
    assert pos == [(t, c) for t in range(32) for c in range(128)]
    for ex in GOLD["v_tile_4bit"]:
        codes = np.zeros((32, 128), dtype=np.int64)
        codes[ex["token_in_tile"], ex["channel"]] = ex["code"]
        tile = layout.pack_v_tiles(codes, 4)[0]
        assert tile.shape == (2048,)
        assert np.nonzero(tile)[0].tolist() == [ex["byte_index"]], ex["why"]
        assert tile[ex["byte_index"]] == ex["byte"], ex["why"]


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_v_tile_unpacks_back(bits):
    rng = np.random.default_rng(10 + bits)
    codes = rng.integers(0, 2 ** bits, size=(64, 128))
    tiles = layout.pack_v_tiles(codes, bits)              # [2, 64 * 8 * bits]
    assert tiles.shape == (2, 64 * 8 * bits)
    lb = 8 * bits
    for tix in range(2):
        for L in range(64):
            for s in range(2):
                seg = tiles[tix, L * lb + s * 4 * bits: L * lb + (s + 1) * 4 * bits]
                got = layout.unpack_segment(seg, bits)
                for u in range(32):
                    t, c = layout.v_tile_position(L, s, u)
                    assert got[u] == codes[32 * tix + t, c]


def test_v_pair_tile_is_a_bijection_and_examples():
    pos = sorted(layout.v_pair_position(byte, half) for byte in range(2048) for half in range(2))
    assert pos == [(t, c) for t in range(32) for c in range(128)]
    for ex in GOLD["v_pair_tile_4bit"]:
        codes = np.zeros((32, 128), dtype=np.int64)
        codes[ex["token_in_tile"], ex["channel"]] = ex["code"]
        tile = layout.pack_v_pair_tiles(codes)[0]
        assert tile.shape == (2048,)
        assert np.nonzero(tile)[0].tolist() == [ex["byte_index"]], ex["why"]
        assert tile[ex["byte_index"]] == ex["byte"], ex["why"]


def test_v_pair_tile_unpacks_back():
    rng = np.random.default_rng(44)
    codes = rng.integers(0, 16, size=(64, 128))
    tiles = layout.pack_v_pair_tiles(codes)
    assert tiles.shape == (2, 2048)
    for tix in range(2):
        for byte in range(2048):
            for half in range(2):
                t, c = layout.v_pair_position(byte, half)
                assert (int(tiles[tix, byte]) >> (4 * half)) & 15 == codes[32 * tix + t, c]


def test_bits_round_trip():
    x = np.array([1.5, -2.25, 0.0, 65504.0], dtype=np.float32)
    assert np.array_equal(layout.from_bits(layout.to_bits(x, "f16"), "f16"), x)
    y = np.array([1.5, -3.0, 2.0 ** 100, -1.0 / 1024], dtype=np.float32)
    assert np.array_equal(layout.from_bits(layout.to_bits(y, "bf16"), "bf16"), y)


def test_outlier_column_carries_the_dense_index():
    # one token, one head: the outlier at channel 5 replaced dense index 9,
    # so its column entry is 5 | 9 << 12 = 36869 (hand-derived)
    codes = np.zeros((1, 1, 1, 128), dtype=np.int64)
    codes[0, 0, 0, 5] = 9
    codes[0, 0, 0, 77] = 3
    enc = {"codes": codes, "cols": np.array([[[5, 77]]]),
           "vals": np.array([[[7.5, -6.0]]], dtype=np.float32)}
    fmt = {"quantizer": "codebook", "bits": 4, "outlier_frac": 2 / 128}
    reg = layout.expected_regions(fmt, enc, batch=1, n_kv_heads=1, n_ctx=1, max_ctx=32,
                                  kv_dtype="f16", is_key=True)
    assert reg["col"][:2].tolist() == [36869, 77 | 3 << 12]
    assert reg["val"][:2].tolist() == [7.5, -6.0]
    assert reg["row_ptr"][:3].tolist() == [0, 2, 0]


def test_outlier_tile_index():
    # three heads, three outliers per token, two tokens in tile 0:
    # token 0 at columns 5 (head 0, channel 5), 130 (head 1, channel 2) and
    # 200 (head 1, channel 72); token 1 at columns 0, 1 (head 0) and 300
    # (head 2, channel 44).  Head lists in token order: head 0 = (t0 c5,
    # t1 c0, t1 c1), head 1 = (t0 c2, t0 c72), head 2 = (t1 c44) -> offsets
    # 0, 3, 5 and the count 6.  An entry is c | token << 7 | code << 12 |
    # fp16 bits << 16: values 1.0 (0x3c00) except -2.0 (0xc000) at column
    # 200, whose dense index is 9.
    codes = np.zeros((1, 3, 2, 128), dtype=np.int64)
    codes[0, 1, 0, 72] = 9
    vals = np.ones((1, 2, 3), dtype=np.float32)
    vals[0, 0, 2] = -2.0
    enc = {"codes": codes, "cols": np.array([[[5, 130, 200], [0, 1, 300]]]), "vals": vals}
    fmt = {"quantizer": "codebook", "bits": 4, "outlier_frac": 3 / 384}
    reg = layout.expected_regions(fmt, enc, batch=1, n_kv_heads=3, n_ctx=2, max_ctx=32,
                                  kv_dtype="f16", is_key=True)
    off, ent = reg["tile_off"], reg["tile_ent"]
    assert off.shape == (32, 8) and off.dtype == np.uint16        # 1024 tokens / 32
    assert ent.shape == (32, 96) and ent.dtype == np.uint32       # 32 tokens x 3 entries
    assert off[0].tolist() == [0, 3, 5, 6, 0, 0, 0, 0]
    assert [hex(int(x)) for x in ent[0, :6]] == [
        "0x3c000005", "0x3c000080", "0x3c000081", "0x3c000002", "0xc0009048", "0x3c0000ac"]
    assert not ent[0, 6:].any() and not off[1:].any() and not ent[1:].any()
