"""Pins for the per-token branch of the oracle's tensor encoder (CPU only).

``oracle.quant.encode_tensor`` reshapes a [B, T, H, d] tensor into groups
of G consecutive channels of one token (Survey page, section 2.4: every
group of a head and position has its own scale and zero point;
Memory-killer page, section 2.3: each group measures its own range) and
assembles the codes, the per-group parameters and the dequantized values.
These tests build inputs whose every group lies on a grid chosen by hand
(zero + k * scale with exact fp16 scale and zero, or k * scale for q8_0),
different in every (sequence, token, head, group), so the expected codes
and parameters are known without running any quantizer: a group taken
along tokens, a strided channel group or swapped parameter axes changes
them.  ``expected_regions`` is pinned on hand-derived byte images of the
parameter arrays (tests/golden/layout_examples.json).
"""
import json
import os

import numpy as np
import pytest

from oracle import layout, quant

F32 = np.float32
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "layout_examples.json")))

# scales: exact fp16 numbers with at most 2 significant bits, so that every
# grid value below stays exact in fp16 (and in bf16 for bits <= 4)
SCALES = [2.0 ** e * m for e in range(-5, 2) for m in (1.0, 1.5)]


def _grid_tensor(rng, B, T, H, G, quantizer, bits):
    """x [B, T, H, 128] float32 and the hand-known codes [B, H, T, 128],
    scale and zero [B, H, T, 128 // G] of a per-token group encoding."""
    d = 128
    ng = d // G
    codes = np.zeros((B, H, T, d), dtype=np.int64)
    scale = np.zeros((B, H, T, ng), dtype=F32)
    zero = np.zeros((B, H, T, ng), dtype=F32)
    x = np.zeros((B, T, H, d), dtype=F32)
    seen = set()
    for b in range(B):
        for t in range(T):
            for h in range(H):
                in_token = set()
                for g in range(ng):
                    # a (scale, zero) pair new to the tensor when the pool
                    # allows it (absmax + offset and q8_0 have one pair per
                    # scale), and always new within the token
                    for attempt in range(200):
                        s = F32(SCALES[rng.integers(len(SCALES))])
                        if quantizer == "asym_minmax":
                            kmax = 2 ** bits - 1
                            z = F32(int(rng.integers(-2 * kmax, kmax))) * s
                        elif quantizer == "asym_absmax_offset":
                            # absmax / (2^(b-1) - 1) = s needs the range
                            # [-(2^(b-1) - 1) s, (2^(b-1) - 1) s]: codes 0 .. 2^b - 2
                            kmax = 2 ** bits - 2
                            z = -F32(2 ** (bits - 1) - 1) * s
                        else:   # q8_0: codes -127 .. 127, zero point 0
                            kmax = 127
                            z = F32(0)
                        key = (float(s), float(z))
                        if key in in_token:
                            continue
                        if key not in seen or attempt >= 50:
                            break
                    seen.add(key)
                    in_token.add(key)
                    if quantizer == "sym_q8_0":
                        k = rng.integers(-127, 128, size=G)
                        k[rng.integers(G)] = 127 if rng.integers(2) else -127   # absmax = 127 s
                    else:
                        k = rng.integers(0, kmax + 1, size=G)
                        i0, i1 = rng.choice(G, size=2, replace=False)
                        k[i0], k[i1] = 0, kmax       # the group's min and max
                    vals = z + k.astype(F32) * s
                    assert np.all(vals.astype(np.float16).astype(F32) == vals)
                    sl = slice(g * G, (g + 1) * G)
                    x[b, t, h, sl] = vals
                    codes[b, h, t, sl] = k
                    scale[b, h, t, g] = s
                    zero[b, h, t, g] = z
    return x, codes, scale, zero


@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("quantizer,bits", [("asym_minmax", 3), ("asym_minmax", 4),
                                            ("asym_minmax", 8), ("asym_absmax_offset", 3),
                                            ("asym_absmax_offset", 4), ("sym_q8_0", 8)])
def test_per_token_groups_on_hand_built_grids(G, quantizer, bits):
    rng = np.random.default_rng(1000 * G + 10 * bits + len(quantizer))
    B, T, H = 2, 5, 3
    x, codes, scale, zero = _grid_tensor(rng, B, T, H, G, quantizer, bits)
    fmt = {"quantizer": quantizer, "bits": bits, "group_size": G, "layout": "per_token"}
    enc = quant.encode_tensor(x, fmt)
    assert enc["codes"].shape == (B, H, T, 128)
    assert np.array_equal(enc["codes"], codes)
    assert enc["scale"].shape == (B, H, T, 128 // G)
    assert np.array_equal(enc["scale"].astype(F32), scale)
    if quantizer == "sym_q8_0":
        assert "zero" not in enc
    else:
        assert np.array_equal(enc["zero"].astype(F32), zero)
    # every grid value dequantizes to itself, in [B, H, T, d] order
    assert np.array_equal(enc["deq"], np.transpose(x, (0, 2, 1, 3)).astype(np.float64))


def test_per_token_groups_bf16_inputs():
    # config 3's path: bf16 values, 3-bit absmax + offset, G = 64
    rng = np.random.default_rng(77)
    x, codes, scale, zero = _grid_tensor(rng, 1, 4, 2, 64, "asym_absmax_offset", 3)
    u = x.view(np.uint32)
    assert np.all(u & 0xFFFF == 0)          # the grid values are bf16 numbers
    enc = quant.encode_tensor(x, {"quantizer": "asym_absmax_offset", "bits": 3,
                                  "group_size": 64, "layout": "per_token"})
    assert np.array_equal(enc["codes"], codes)
    assert np.array_equal(enc["scale"].astype(F32), scale)
    assert np.array_equal(enc["zero"].astype(F32), zero)


def test_one_group_per_token_is_the_whole_row():
    # G = 128: each token's one group spans all channels -- the min and max
    # of a token decide its parameters even when another token or head has
    # a wider range
    x = np.zeros((1, 2, 2, 128), dtype=F32)
    x[0, 0, 0] = np.arange(128) % 16 * F32(0.5) - F32(1.5)     # range [-1.5, 6.0]
    x[0, 1, 0] = np.arange(128) % 16 * F32(4.0) + F32(8.0)     # range [8, 68]
    x[0, 0, 1] = np.arange(128) % 16 * F32(0.125)              # range [0, 1.875]
    x[0, 1, 1] = np.full(128, F32(-2.0))                       # degenerate
    enc = quant.encode_tensor(x, {"quantizer": "asym_minmax", "bits": 4, "group_size": 128,
                                  "layout": "per_token"})
    assert enc["scale"][0, :, :, 0].astype(F32).tolist() == [[0.5, 4.0], [0.125, 0.0]]
    assert enc["zero"][0, :, :, 0].astype(F32).tolist() == [[-1.5, 8.0], [0.0, -2.0]]
    assert enc["codes"][0, 0, 0].tolist() == (np.arange(128) % 16).tolist()
    assert np.all(enc["codes"][0, 1, 1] == 0)


def _build_from_gold(entry, G, q8):
    """Tensor whose listed groups hold the golden (scale, zero) on a grid;
    every other group of the two tokens is all zero."""
    H = 1 + max(g["h"] for g in entry["groups"])
    x = np.zeros((1, 2, H, 128), dtype=F32)
    for rec in entry["groups"]:
        h, t, g = rec["h"], rec["t"], rec["g"]
        c = np.arange(G)
        s = F32(rec["scale"])
        if q8:
            k = (5 * c + t + g) % 255 - 127
            k[0], k[1] = 127, -127
            x[0, t, h, g * G:(g + 1) * G] = k.astype(F32) * s
        else:
            k = (c + 7 * t + 3 * g) % 16
            x[0, t, h, g * G:(g + 1) * G] = F32(rec["zero"]) + k.astype(F32) * s
    return x, H


def test_params_byte_image_per_token_asym():
    entry = GOLD["params_per_token_asym"]
    x, H = _build_from_gold(entry, 64, False)
    fmt = {"quantizer": "asym_minmax", "bits": 4, "group_size": 64, "layout": "per_token"}
    enc = quant.encode_tensor(x, fmt)
    reg = layout.expected_regions(fmt, enc, batch=1, n_kv_heads=H, n_ctx=2, max_ctx=2,
                                  kv_dtype="f16", is_key=False)
    raw = np.ascontiguousarray(reg["params"]).view(np.uint8).reshape(-1)
    assert raw.size == entry["region_bytes"], entry["region_why"]
    listed = np.zeros(raw.size, dtype=bool)
    for rec in entry["groups"]:
        o = rec["offset"]
        assert raw[o:o + 4].tolist() == rec["bytes"], rec["why"]
        listed[o:o + 4] = True
    assert not raw[~listed].any()     # capacity beyond the two tokens stays zero


def test_params_byte_image_q8_0():
    entry = GOLD["params_q8_0"]
    x, H = _build_from_gold(entry, 32, True)
    fmt = {"quantizer": "sym_q8_0", "bits": 8, "group_size": 32, "layout": "per_token"}
    enc = quant.encode_tensor(x, fmt)
    reg = layout.expected_regions(fmt, enc, batch=1, n_kv_heads=H, n_ctx=2, max_ctx=2,
                                  kv_dtype="f16", is_key=True)
    raw = np.ascontiguousarray(reg["params"]).view(np.uint8).reshape(-1)
    assert raw.size == entry["region_bytes"], entry["region_why"]
    listed = np.zeros(raw.size, dtype=bool)
    for rec in entry["groups"]:
        o = rec["offset"]
        assert raw[o:o + 2].tolist() == rec["bytes"], rec["why"]
        listed[o:o + 2] = True
    assert not raw[~listed].any()     # all-zero blocks store scale 0
