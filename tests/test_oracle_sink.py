"""Pins for the oracle's attention-sink prefix (CPU only).

The KVQuant page ("Attention Sink") keeps the keys and values of the first
few tokens in full precision.  The oracle's reading: tokens [0, S) keep their
fp16/bf16 values, and tokens [S, T) form an ordinary quantized cache that
starts at token S.  These tests pin that reading against what it must reduce
to: the unquantized cache when S covers every token, the plain encoding when
S = 0, the textbook min-max group of the first per-channel group after the
sink, and the raw byte counts.
"""
import numpy as np
import pytest

from oracle import attention as oatt
from oracle import cache_bytes as ocb
from oracle import layout as olay
from oracle import quant as oq

F4 = dict(quantizer="asym_minmax", bits=4, group_size=32, layout="per_token")
KCH = dict(quantizer="asym_minmax", bits=4, group_size=64, layout="per_channel")


def _x(shape, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape).astype(np.float16).astype(np.float32)


@pytest.mark.parametrize("extra", [0, 5])
def test_sink_covering_every_token_is_the_unquantized_cache(extra):
    x = _x((2, 20, 3, 128), 1)
    enc = oq.encode_with_sink(x, F4, sink=20 + extra)
    raw = oq.encode_tensor(x, dict(quantizer="none", bits=16))["deq"]
    assert enc["rest"] is None
    assert np.array_equal(enc["deq"], raw)
    q = _x((2, 3, 128), 2)
    a = oatt.decode_attention(q, enc["deq"], enc["deq"], n_ctx=20)
    b = oatt.decode_attention(q, raw, raw, n_ctx=20)
    assert np.array_equal(a, b)


def test_sink_zero_is_the_plain_encoding():
    x = _x((1, 40, 2, 128), 3)
    enc = oq.encode_with_sink(x, F4, sink=0)
    ref = oq.encode_tensor(x, F4)
    assert enc["sink"].shape[2] == 0
    assert np.array_equal(enc["deq"], ref["deq"])
    assert np.array_equal(enc["rest"]["codes"], ref["codes"])


def test_prefix_is_exact_and_the_rest_is_the_suffix_encoding():
    x = _x((2, 50, 2, 128), 4)
    enc = oq.encode_with_sink(x, F4, sink=7)
    assert np.array_equal(enc["deq"][:, :, :7], np.transpose(x[:, :7], (0, 2, 1, 3)))
    suffix = oq.encode_tensor(x[:, 7:], F4)
    assert np.array_equal(enc["deq"][:, :, 7:], suffix["deq"])
    # the prefix is exact, the rest is not: quantization changed something
    assert not np.array_equal(enc["deq"][:, :, 7:], np.transpose(x[:, 7:], (0, 2, 1, 3)))


def test_per_channel_groups_start_after_the_sink():
    S, G = 5, 64
    x = _x((1, S + G + 10, 2, 128), 5)
    rest = oq.encode_with_sink(x, KCH, sink=S)["rest"]
    # group 0 of the quantized tokens is absolute tokens [S, S + G): the
    # textbook min-max scale and zero of that window, channel by channel
    win = x[0, S:S + G]                                  # [G, H, d]
    lo, hi = win.min(axis=0), win.max(axis=0)
    s16 = ((hi - lo).astype(np.float32) / np.float32(15)).astype(np.float16)
    assert np.array_equal(rest["scale"][0, :, 0, :], s16)
    assert np.array_equal(rest["zero"][0, :, 0, :], lo.astype(np.float16))
    # the last 10 tokens are the unfinished group, kept as they are
    assert np.array_equal(rest["tail"][0], np.transpose(x[0, S + G:], (1, 0, 2)))


def test_sink_region_bytes():
    x = _x((2, 6, 3, 128), 6)
    img = olay.sink_region(x, 8, kv_dtype="f16")
    assert img.shape == (2, 3, 8, 128)
    assert np.array_equal(img[:, :, :6], np.transpose(x, (0, 2, 1, 3)).astype(np.float16).view(np.uint16))
    assert not img[:, :, 6:].any()


@pytest.mark.parametrize("n", [0, 3, 8, 100])
def test_payload_bytes_with_a_sink(n):
    kw = dict(batch=2, n_kv_heads=3, head_dim=128, kv_dtype="f16")
    raw = dict(quantizer="none", bits=16)
    # raw formats cost the same with or without a sink
    assert (ocb.payload_bytes(raw, raw, n_ctx=n, sink=8, **kw)
            == ocb.payload_bytes(raw, raw, n_ctx=n, **kw) == 2 * 2 * 3 * n * 128 * 2)
    s = min(8, n)
    with_sink = ocb.payload_bytes(F4, KCH, n_ctx=n, sink=8, **kw)
    assert with_sink == ocb.payload_bytes(F4, KCH, n_ctx=n - s, **kw) + 2 * 2 * 3 * s * 128 * 2
