"""Pins for the oracle's paged-cache mapping (CPU only): hand-derived row
positions (tests/golden/layout_examples.json), the identity table of one
sequence reproducing the contiguous layout, and the CSR rows."""
import json
import os

import numpy as np

from oracle import layout, paging, quant

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "layout_examples.json")))


def _marker(b, h, t):
    return 1 + ((b * 2 + h) * 64 + t) % 251


def test_token_rows_match_the_hand_derived_positions():
    g = GOLD["paged_rows"]
    table = np.array(g["table"])
    for rec in g["rows"]:
        assert paging.token_row(table, 2, rec["b"], rec["h"], rec["t"]) == rec["row"], rec["why"]
        assert rec["row"] * g["row_bytes"] == rec["byte_offset"]
    for rec in g["csr_rows"]:
        assert paging.csr_row(table, rec["b"], rec["t"]) == rec["row"], rec["why"]


def test_key_row_bytes_land_on_their_page():
    g = GOLD["paged_rows"]
    table = np.array(g["table"])
    B, H, cap, rb = 2, 2, 1024, g["row_bytes"]
    img = np.zeros((B, H, cap, rb), dtype=np.uint8)
    for b in range(B):
        for h in range(H):
            for t in range(64):
                img[b, h, t] = _marker(b, h, t)
    out = paging.paged_regions({"codes": img.reshape(B, H, cap * rb)}, table, n_pages=g["n_pages"],
                               n_ctx=64, capacity=cap, per_channel=False)
    flat = out["codes"].reshape(-1)
    assert flat.size == g["n_pages"] * H * 32 * rb
    for rec in g["rows"]:
        o = rec["byte_offset"]
        assert np.all(flat[o:o + rb] == _marker(rec["b"], rec["h"], rec["t"])), rec["why"]
    # page 2 is in no table entry: zero
    assert not out["codes"][2].any()
    # every written row appears once
    assert np.count_nonzero(flat) == B * H * 64 * rb


def test_identity_table_of_one_sequence_is_the_contiguous_layout():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 96, 3, 128)).astype(np.float16).astype(np.float32)
    for fmt, is_key in (({"quantizer": "asym_minmax", "bits": 4, "group_size": 32,
                          "layout": "per_token"}, True),
                        ({"quantizer": "asym_minmax", "bits": 3, "group_size": 64,
                          "layout": "per_token"}, False)):
        enc = quant.encode_tensor(x, fmt)
        reg = layout.expected_regions(fmt, enc, batch=1, n_kv_heads=3, n_ctx=96, max_ctx=96,
                                      kv_dtype="f16", is_key=is_key)
        table = np.arange(32)[None, :]                  # logical page i -> physical i
        pg = paging.paged_regions(reg, table, n_pages=3, n_ctx=96, capacity=1024,
                                  per_channel=False)
        # [page][head][32 tokens] read back in (head, token) order: the
        # first 96 tokens of each head's contiguous stream
        codes = pg["codes"].transpose(1, 0, 2).reshape(3, -1)
        n = codes.shape[1]
        assert np.array_equal(codes, reg["codes"][0, :, :n])
        prm = pg["params"].transpose(1, 0, 2, 3, 4).reshape(3, 96, -1, 2)
        assert np.array_equal(prm, reg["params"][0, :, :96])


def test_csr_rows_and_pointers():
    # codebook outliers of 2 sequences x 48 tokens, k = 3 per token
    k = 3
    cap = 1024
    col = np.zeros(2 * cap * k, dtype=np.uint16)
    val = np.zeros(2 * cap * k, dtype=np.float16)
    for b in range(2):
        for t in range(48):
            col[(b * cap + t) * k:(b * cap + t + 1) * k] = 1000 * b + t
            val[(b * cap + t) * k:(b * cap + t + 1) * k] = b + t / 64
    table = np.array(GOLD["paged_rows"]["table"])
    pg = paging.paged_regions({"row_ptr": np.zeros(2 * cap + 1, np.int32), "col": col, "val": val},
                              table, n_pages=5, n_ctx=48, capacity=cap, per_channel=False,
                              k_out=k)
    rp = pg["row_ptr"]
    assert rp.shape == (5 * 32 + 1,)
    for rec in GOLD["paged_rows"]["csr_rows"]:
        r = rec["row"]
        assert rp[r] == k * r and rp[r + 1] == k * (r + 1), rec["why"]
        assert np.all(pg["col"][k * r:k * (r + 1)] == 1000 * rec["b"] + rec["t"])
    # rows of page 2 (unused) and of tokens past 48 stay empty
    assert not rp[2 * 32 + 1:3 * 32].any()
    assert not pg["col"][k * (32 + 16):k * (32 + 32)].any()   # sequence 1, tokens 48..63
