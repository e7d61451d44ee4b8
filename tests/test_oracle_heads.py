"""Pins for per-token groups with a group size per KV head (CPU only).

Memory-killer page, section 2.3: finer groups for the attention heads that
quantize badly, coarser ones for stable heads; section 5.3: heads differ in
their sensitivity.  Reading: a per-token format takes one group size per
KV head; each head is quantized as its own per-token tensor.  The inputs are
on hand-chosen grids, and the parameter byte images (contiguous and paged)
are derived by hand in tests/golden/layout_examples.json.
"""
import json
import os

import numpy as np

from oracle import cache_bytes, layout, paging, quant

F32 = np.float32
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "layout_examples.json")))


def _fmt(sizes, q="asym_minmax", bits=4):
    return {"quantizer": q, "bits": bits, "group_size": 0, "layout": "per_token",
            "head_group_size": list(sizes)}


def test_each_head_takes_its_own_group_size():
    # head 0: groups of 32 with ranges [0, 15 s_g]; head 1: one group of 128
    # whose range spans all channels.  Grid values dequantize exactly.
    x = np.zeros((1, 3, 2, 128), dtype=F32)
    k = (np.arange(128) * 7) % 16
    for t in range(3):
        for g in range(4):
            s = F32(2.0 ** (g - t))
            x[0, t, 0, 32 * g:32 * g + 32] = k[32 * g:32 * g + 32] * s + F32(g)
        x[0, t, 1] = k * F32(0.25) - F32(t)
    enc = quant.encode_tensor(x, _fmt([32, 128]))
    assert [a.shape for a in enc["scale"]] == [(1, 3, 4), (1, 3, 1)]
    for t in range(3):
        assert enc["scale"][0][0, t].astype(F32).tolist() == [2.0 ** (g - t) for g in range(4)]
        assert enc["zero"][0][0, t].astype(F32).tolist() == [0.0, 1.0, 2.0, 3.0]
        assert float(enc["scale"][1][0, t, 0]) == 0.25 and float(enc["zero"][1][0, t, 0]) == -t
    assert np.array_equal(enc["codes"][0, 0, :, :], np.tile(k, (3, 1)))
    assert np.array_equal(enc["codes"][0, 1, :, :], np.tile(k, (3, 1)))
    assert np.array_equal(enc["deq"], np.transpose(x, (0, 2, 1, 3)).astype(np.float64))
    # with one group of 128 for head 0 its range would span the four groups
    one = quant.encode_tensor(x, _fmt([128, 128]))
    assert float(one["zero"][0][0, 0, 0]) == 0.0 and float(one["scale"][0][0, 0, 0]) != 1.0


def _gold_input(entry):
    x = np.zeros((1, 2, 2, 128), dtype=F32)
    for rec in entry["groups"]:
        h, t, g = rec["h"], rec["t"], rec["g"]
        G = entry["head_group_size"][h]
        kk = (np.arange(G) + 7 * t + 3 * g) % 16
        x[0, t, h, g * G:(g + 1) * G] = F32(rec["zero"]) + kk.astype(F32) * F32(rec["scale"])
    return x


def test_params_byte_image_per_head():
    e = GOLD["params_per_head"]
    fmt = _fmt(e["head_group_size"])
    x = _gold_input(e)
    enc = quant.encode_tensor(x, fmt)
    reg = layout.expected_regions(fmt, enc, batch=1, n_kv_heads=2, n_ctx=2, max_ctx=2,
                                  kv_dtype="f16", is_key=False)
    raw = np.ascontiguousarray(reg["params"]).view(np.uint8).reshape(-1)
    assert raw.size == e["region_bytes"], e["region_why"]
    for rec in e["groups"]:
        o = rec["offset"]
        assert raw[o:o + 4].tolist() == rec["bytes"], rec["why"]


def test_paged_records_per_head():
    e = GOLD["params_per_head"]
    pg = e["paged"]
    fmt = _fmt(e["head_group_size"])
    # 40 tokens whose parameters are unique per (head, token, group)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 40, 2, 128)).astype(np.float16).astype(F32)
    enc = quant.encode_tensor(x, fmt)
    reg = layout.expected_regions(fmt, enc, batch=1, n_kv_heads=2, n_ctx=40, max_ctx=64,
                                  kv_dtype="f16", is_key=False)
    out = paging.paged_regions(reg, np.array(pg["table"]), n_pages=pg["n_pages"], n_ctx=40,
                               capacity=1024, per_channel=False, head_ng=[2, 1], rec_halves=2)
    recs = out["params"].reshape(-1, 2)
    for r in pg["records"]:
        h, t, g = r["h"], r["t"], r["g"]
        assert recs[r["record"], 0] == enc["scale"][h][0, t, g], r["why"]
        assert recs[r["record"], 1] == enc["zero"][h][0, t, g], r["why"]


def test_payload_by_hand():
    # 4-bit, heads with groups of 32 and 128: per token 2 x 64 code bytes and
    # (4 + 1) records of 4 bytes = 148 bytes; 10 tokens -> 1480 per tensor
    fmt = _fmt([32, 128])
    kw = dict(batch=1, n_kv_heads=2, head_dim=128, n_ctx=10)
    assert cache_bytes.tensor_payload(fmt, **kw) == 1480
    q8 = _fmt([32, 64], q="sym_q8_0", bits=8)
    # 8-bit: 2 x 128 code bytes and (4 + 2) fp16 scales = 268 bytes per token
    assert cache_bytes.tensor_payload(q8, **kw) == 2680
