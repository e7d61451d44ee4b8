"""Pins for the oracle's overlapping window statistics of per-channel key
groups and for the tail ring (CPU only).

TurboQuant page, section 3.1: the scale and offset come from a sliding
window's extrema; section 6, problem 1: windows overlapping by 64 tokens
against edge effects.  Reading: window g of a group of G tokens spans
[g G - overlap, g G + G), clipped at token 0.  The cases below are built by
hand so that the window reaching back changes the parameters.
"""
import numpy as np
import pytest

from oracle import layout, quant

F32 = np.float32


def _fmt(q="asym_minmax", bits=4, G=32, overlap=32):
    return {"quantizer": q, "bits": bits, "group_size": G, "layout": "per_channel",
            "window_overlap": overlap}


def test_window_reaches_into_the_previous_group():
    # channel 3: group 0 (tokens 0-31) is 2.0 except 15.0 at token 10;
    # group 1 (tokens 32-63) holds 0, 0.25, 0.5, 0.75, 1 in turn.  Window 1
    # spans tokens 0-63: min 0, max 15 -> 4-bit scale 15/15 = 1, zero 0, and
    # group 1's codes are its values rounded half to even: 0, 0, 0, 1, 1.
    x = np.zeros((1, 64, 1, 128), dtype=F32)
    x[0, :32, 0, 3] = 2.0
    x[0, 10, 0, 3] = 15.0
    g1 = np.array([0.0, 0.25, 0.5, 0.75, 1.0], dtype=F32)
    x[0, 32:, 0, 3] = np.resize(g1, 32)
    enc = quant.encode_tensor(x, _fmt())
    assert float(enc["scale"][0, 0, 1, 3]) == 1.0 and float(enc["zero"][0, 0, 1, 3]) == 0.0
    assert enc["codes"][0, 0, 32:37, 3].tolist() == [0, 0, 0, 1, 1]
    # group 0's window is clipped at token 0: its own range [2, 15]
    assert float(enc["scale"][0, 0, 0, 3]) == float(np.float16(13.0 / 15.0))
    assert float(enc["zero"][0, 0, 0, 3]) == 2.0
    # without the overlap group 1 would use its own range [0, 1]
    plain = quant.encode_tensor(x, _fmt(overlap=0))
    assert float(plain["scale"][0, 0, 1, 3]) == float(np.float16(1.0 / 15.0))


def test_overlap_longer_than_a_group_and_absmax_offset():
    # G = 32, overlap 64: window 2 spans tokens 0-95.  3-bit absmax + offset:
    # a -6 at token 5 and values in [-1, 1] later -> absmax 6, scale
    # 6 / 3 = 2, offset -6; value 1.0 -> (1 + 6) / 2 = 3.5 -> 4 (half to even)
    x = np.zeros((1, 96, 1, 128), dtype=F32)
    x[0, 5, 0, 0] = -6.0
    x[0, 64:, 0, 0] = 1.0
    enc = quant.encode_tensor(x, _fmt("asym_absmax_offset", 3, 32, 64))
    assert float(enc["scale"][0, 0, 2, 0]) == 2.0 and float(enc["zero"][0, 0, 2, 0]) == -6.0
    assert np.all(enc["codes"][0, 0, 64:96, 0] == 4)
    # window 1 (tokens 0-63) sees the -6 as well; window 2 with overlap 32
    # (tokens 32-95) would not
    assert float(enc["zero"][0, 0, 1, 0]) == -6.0
    short = quant.encode_tensor(x, _fmt("asym_absmax_offset", 3, 32, 32))
    assert float(short["zero"][0, 0, 2, 0]) == 0.0
    assert float(short["scale"][0, 0, 2, 0]) == float(np.float16(1.0 / 3.0))


@pytest.mark.parametrize("q,bits", [("asym_minmax", 4), ("asym_minmax", 3),
                                    ("asym_absmax_offset", 3)])
def test_core_tokens_stay_in_range_within_half_a_step(q, bits):
    rng = np.random.default_rng(11)
    G, O = 64, 64
    x = rng.standard_normal((2, 300, 2, 128)).astype(np.float16).astype(F32)
    x[:, ::37, :, 7] *= 20
    enc = quant.encode_tensor(x, _fmt(q, bits, G, O))
    c = enc["codes"]
    assert c.min() >= 0 and c.max() <= 2 ** bits - 1
    xt = np.transpose(x, (0, 2, 1, 3)).astype(np.float64)          # [B, H, T, d]
    for g in range(300 // G):
        core = xt[:, :, g * G:(g + 1) * G]
        lo = xt[:, :, max(0, g * G - O):(g + 1) * G].min(axis=2, keepdims=True)
        s = enc["scale"][:, :, g:g + 1].astype(np.float64)
        z = enc["zero"][:, :, g:g + 1].astype(np.float64)
        # every core token lies inside its window's range, so no code is
        # clamped: half a step, plus the fp16 rounding of the zero point and
        # of the float32 quotient
        err = np.abs(enc["deq"][:, :, g * G:(g + 1) * G] - core)
        assert np.all(err <= 0.5 * s + np.abs(z - lo) + 1e-6 * (np.abs(core) + np.abs(z)))


def test_tail_ring_rows():
    # G = 32, overlap 32, 70 tokens: groups 0 and 1 are quantized, the ring
    # of 64 rows keeps tokens 32-69 (the next window's 32 tokens back and
    # the unfinished group) at row p mod 64: tokens 32-63 in rows 32-63,
    # tokens 64-69 in rows 0-5; rows 6-31 are zero
    raw = np.zeros((1, 1, 70, 128), dtype=F32)
    for p in range(70):
        raw[0, 0, p, :] = p + 1
    ring = layout.tail_ring(raw, 32, 32, 70, "f16")
    vals = ring.view(np.float16).astype(np.float32)[0, 0, :, 0]
    assert vals[32:64].tolist() == [float(p + 1) for p in range(32, 64)]
    assert vals[:6].tolist() == [float(p + 1) for p in range(64, 70)]
    assert not vals[6:32].any()
    # without overlap: row i holds token 64 + i (the unfinished group only)
    ring0 = layout.tail_ring(raw, 32, 0, 70, "f16").view(np.float16).astype(np.float32)[0, 0, :, 0]
    assert ring0[:6].tolist() == [float(p + 1) for p in range(64, 70)]
    assert not ring0[6:].any()
