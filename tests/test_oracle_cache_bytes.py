"""Pins for the oracle's cache-size closed forms against the values the pages
print (tests/golden/page_values.json), CPU only."""
import json
import os

import pytest

from oracle import cache_bytes as cb
from synth import make_workload

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
NONE = {"quantizer": "none", "bits": 16}


def test_70b_bytes_per_token():
    g = GOLD["kv_bytes_per_token_70b"]
    s = g["shape"]
    v = cb.payload_bytes(NONE, NONE, batch=1, n_kv_heads=s["n_kv_heads"], head_dim=s["head_dim"],
                         n_ctx=1, n_layers=s["n_layers"])
    assert v == g["value"]
    gb = cb.payload_bytes(NONE, NONE, batch=1, n_kv_heads=8, head_dim=128, n_ctx=32000,
                          n_layers=80) / 1e9
    assert round(gb, 1) == GOLD["kv_gb_70b_32k"]["value_gb"]


def test_8b_128k_elements():
    g = GOLD["kv_elements_8b_128k"]
    s = g["shape"]
    nbytes = cb.payload_bytes(NONE, NONE, batch=s["batch"], n_kv_heads=s["n_heads"],
                              head_dim=s["head_dim"], n_ctx=s["seq"], n_layers=s["n_layers"])
    assert nbytes // 2 == g["exact_from_formula"]
    assert abs(nbytes / 2 / 1e9 - g["value_approx"] / 1e9) < 0.1
    assert abs(nbytes / 1e9 - g["fp16_gb_approx"]) < 1.0


def test_one_head_4k():
    g = GOLD["one_head_4k_bytes"]
    assert cb.tensor_payload(NONE, batch=1, n_kv_heads=1, head_dim=128, n_ctx=4096) == g["value"]


def test_groups_2048_by_64():
    g = GOLD["groups_2048_by_64"]
    fmt = {"quantizer": "asym_minmax", "bits": 4, "group_size": 64, "layout": "per_channel"}
    # per-channel params: 4 bytes (scale + zero) per channel per group
    tot = cb.tensor_payload(fmt, batch=1, n_kv_heads=1, head_dim=128, n_ctx=2048)
    assert tot == 2048 * 64 + g["value"] * 128 * 4


# Config 4 by hand: per tensor, 131,072 tokens x 32 heads x 64 code bytes =
# 268,435,456; the per-tile outlier index: 131,072 x 41 entries x 4 bytes =
# 21,495,808 and 4,096 tiles x 40 offsets x 2 bytes = 327,680; codebooks
# 32 x 128 x 16 x 2 = 131,072 -> x 2 tensors = 580,780,032.
@pytest.mark.parametrize("cfg_id,ctx,expected", [
    (1, None, 155_648), (2, 4096, 2_228_224), (2, 8192, 4_456_448), (2, 16384, 8_912_896),
    (3, None, 117_440_512), (4, None, 580_780_032), (5, None, 1_140_850_688)])
def test_workload_payloads(cfg_id, ctx, expected):
    w = make_workload(cfg_id, ctx=ctx)
    v = cb.payload_bytes(w.k, w.v, batch=w.batch, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                         n_ctx=w.ctx, kv_dtype=w.kv_dtype)
    assert v == expected


def test_per_channel_tail_counts_raw_tokens():
    fmt = {"quantizer": "asym_minmax", "bits": 4, "group_size": 128, "layout": "per_channel"}
    a = cb.tensor_payload(fmt, batch=1, n_kv_heads=1, head_dim=128, n_ctx=128)
    b = cb.tensor_payload(fmt, batch=1, n_kv_heads=1, head_dim=128, n_ctx=130)
    assert b - a == 2 * 128 * 2
