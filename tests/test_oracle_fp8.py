"""Pins for the oracle's FP8 E5M2 format (CPU only).

The Survey page (section 3.4) names vLLM's fp8 KV cache with 5 exponent and
2 mantissa bits and a scale per head.  The oracle's conversion (torch's
float8_e5m2 cast after saturating at the largest finite value) is pinned to
a brute-force nearest-value search over the 256 codes with ties to the even
code, to the closed form "round the fp16 bit pattern to its high byte" for
fp16 inputs, and to exact round trips; the tensor encode is pinned to the
per-head scale definition.
"""
import numpy as np
import pytest

from oracle import cache_bytes as ocb
from oracle import layout as olay
from oracle import quant as oq

FP8 = dict(quantizer="fp8_e5m2", bits=8, group_size=0, layout="per_token")


def _table():
    """All finite E5M2 values by code, from the bit fields."""
    codes = np.arange(256)
    sign = np.where(codes & 0x80, -1.0, 1.0)
    e = (codes >> 2) & 0x1f
    m = codes & 3
    val = np.where(e == 0, m / 4.0 * 2.0 ** -14, (1 + m / 4.0) * 2.0 ** (e.astype(np.float64) - 15))
    finite = e != 31
    return codes[finite], (sign * val)[finite]


def _brute(x):
    codes, vals = _table()
    out = []
    for v in np.asarray(x, dtype=np.float64):
        v = min(max(v, -57344.0), 57344.0)
        d = np.abs(vals - v)
        best = np.flatnonzero(d == d.min())
        # ties: the code with the even last mantissa bit; zero keeps the sign
        if len(best) > 1:
            even = [c for c in best if codes[c] % 2 == 0 and vals[c] != 0]
            zeros = [c for c in best if vals[c] == 0]
            if zeros:
                best = [c for c in zeros if (codes[c] >= 128) == (np.signbit(v))]
            elif even:
                best = even
        out.append(codes[best[0]])
    return np.array(out, dtype=np.uint8)


def test_table_round_trips():
    codes, vals = _table()
    assert np.array_equal(oq.fp8_e5m2_values(codes.astype(np.uint8)), vals)
    got = oq.fp8_e5m2_codes(vals.astype(np.float32))
    # +0 and -0 both decode to 0; every other code maps back to itself
    assert np.array_equal(got, codes.astype(np.uint8))


def test_every_fp16_value_rounds_its_bit_pattern_to_the_high_byte():
    bits = np.arange(65536, dtype=np.uint32)
    x = bits.astype(np.uint16).view(np.float16)
    finite = np.isfinite(x)
    bits, x = bits[finite], x[finite]
    got = oq.fp8_e5m2_codes(x.astype(np.float32)).astype(np.uint32)
    # closed form: E5M2 is the top byte of fp16; round the low byte to
    # nearest even, saturating at 0x7b (57344)
    mag = bits & 0x7fff
    r = (mag + 0x7f + ((mag >> 8) & 1)) >> 8
    r = np.minimum(r, 0x7b)
    want = r | ((bits >> 8) & 0x80)
    assert np.array_equal(got, want)


def test_against_brute_force_including_ties_and_saturation():
    rng = np.random.default_rng(0)
    codes, vals = _table()
    pos = np.sort(vals[vals > 0])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)       # exact ties in float32
    x = np.concatenate([rng.standard_normal(2000).astype(np.float32) * 10.0 ** rng.integers(-6, 5, 2000),
                        mids, -mids, np.float32([6e4, -7e4, 1e9, 57344, 61439, 61440, 0.0, -0.0, 1e-9])])
    assert np.array_equal(oq.fp8_e5m2_codes(x), _brute(x))


def test_tensor_encode_uses_the_per_head_scale():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((2, 9, 3, 128)) * 3).astype(np.float16).astype(np.float32)
    sc = np.float32([0.5, 1.7, 0.031])
    enc = oq.encode_tensor(x, FP8, head_scale=sc)
    xt = np.transpose(x, (0, 2, 1, 3))
    for h in range(3):
        c = oq.fp8_e5m2_codes(xt[:, h] / sc[h])
        assert np.array_equal(enc["codes"][:, h], c)
        assert np.array_equal(enc["deq"][:, h], oq.fp8_e5m2_values(c) * np.float64(sc[h]))
    # unit scales: the dequantized cache is the fp16 input with its mantissa
    # rounded to two bits, within half a step (2^-3 relative) of it
    e1 = oq.encode_tensor(x, FP8)
    rel = np.abs(e1["deq"] - xt) / np.maximum(np.abs(xt), 2.0 ** -14)
    assert rel.max() <= 2.0 ** -3 + 1e-12


def test_regions_and_payload():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 40, 2, 128)).astype(np.float16).astype(np.float32)
    enc = oq.encode_tensor(x, FP8)
    for is_key in (True, False):
        reg = olay.expected_regions(FP8, enc, batch=1, n_kv_heads=2, n_ctx=40, max_ctx=64,
                                    kv_dtype="f16", is_key=is_key)
        assert set(reg) == {"codes"}
        assert reg["codes"].shape == (1, 2, olay.capacity(64) * 128)
        # 8-bit packing: every code byte appears exactly once in the two
        # 32-token rows / tiles the 40 tokens touch, the rest is zero
        c = enc["codes"].astype(np.uint8)
        want = np.concatenate([c[0, 0].reshape(-1), np.zeros(24 * 128, np.uint8)])
        assert np.array_equal(np.sort(reg["codes"][0, 0, :64 * 128]), np.sort(want))
    kw = dict(batch=3, n_kv_heads=2, head_dim=128, kv_dtype="f16")
    # by hand: each tensor holds 3 sequences x 2 heads x 100 tokens x 128
    # one-byte codes = 76,800 bytes plus 2 float32 head scales = 8 bytes;
    # keys and values together 2 x 76,808 = 153,616 bytes
    assert ocb.payload_bytes(FP8, FP8, n_ctx=100, **kw) == 153_616
    # half the raw fp16 cache (2 * L * h * d * 2 bytes per token, TurboQuant
    # page 2.1: 2 * 2 * 128 * 2 = 1,024 bytes per token and sequence, 307,200
    # for 300 token-sequences) plus the scales
    raw = {"quantizer": "none", "bits": 16}
    assert ocb.payload_bytes(raw, raw, n_ctx=100, **kw) == 307_200
    assert ocb.payload_bytes(FP8, FP8, n_ctx=100, **kw) == 307_200 // 2 + 16
