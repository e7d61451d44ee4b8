"""Pins for the oracle's float64 attention (CPU only): a library routine
(torch's scaled_dot_product_attention in float64), textbook special cases,
RoPE identities and a pure-Python brute force on tiny inputs."""
import math

import numpy as np
import pytest
import torch

from oracle import attention


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("g", [1, 2, 8])
def test_matches_torch_sdpa_float64(g):
    rng = np.random.default_rng(g)
    B, Hkv, T, d = 2, 3, 37, 128
    q = _rand(rng, B, Hkv * g, d)
    K = _rand(rng, B, Hkv, T, d)
    V = _rand(rng, B, Hkv, T, d)
    out = attention.decode_attention(q, K, V)
    qt = torch.from_numpy(q)[:, :, None, :]                       # [B, Hq, 1, d]
    Kt = torch.from_numpy(K).repeat_interleave(g, dim=1)
    Vt = torch.from_numpy(V).repeat_interleave(g, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt)[:, :, 0, :].numpy()
    assert np.max(np.abs(out - ref)) < 1e-12


def test_single_token_returns_its_value():
    rng = np.random.default_rng(0)
    q = _rand(rng, 1, 4, 128)
    K = _rand(rng, 1, 2, 1, 128)
    V = _rand(rng, 1, 2, 1, 128)
    out = attention.decode_attention(q, K, V)
    assert np.array_equal(out[0, 0], V[0, 0, 0]) and np.array_equal(out[0, 3], V[0, 1, 0])


def test_zero_query_is_mean_of_values():
    rng = np.random.default_rng(1)
    K = _rand(rng, 1, 1, 50, 128)
    V = _rand(rng, 1, 1, 50, 128)
    out = attention.decode_attention(np.zeros((1, 1, 128)), K, V)
    assert np.allclose(out[0, 0], V[0, 0].mean(axis=0), rtol=0, atol=1e-14)


def test_n_ctx_limits_the_context():
    rng = np.random.default_rng(2)
    q = _rand(rng, 1, 2, 128)
    K = _rand(rng, 1, 1, 40, 128)
    V = _rand(rng, 1, 1, 40, 128)
    a = attention.decode_attention(q, K, V, n_ctx=25)
    b = attention.decode_attention(q, K[:, :, :25], V[:, :, :25])
    assert np.array_equal(a, b)


def test_rope_hand_example():
    # d = 4: pairs (0, 2) and (1, 3); theta_0 = 1, theta_1 = 10000^(-1/2) = 0.01
    x = np.array([1.0, 0.0, 0.0, 0.0])
    r = attention.rope_rotate(x[None], np.array([math.pi / 2]), 10000.0)[0]
    assert np.allclose(r, [0, 0, 1, 0], atol=1e-15)
    y = np.array([0.0, 1.0, 0.0, 0.0])
    r = attention.rope_rotate(y[None], np.array([100.0]), 10000.0)[0]  # angle 1 rad on pair 1
    assert np.allclose(r, [0, math.cos(1.0), 0, math.sin(1.0)], atol=1e-14)


def test_rope_identities():
    rng = np.random.default_rng(3)
    d = 128
    q, k = _rand(rng, d), _rand(rng, d)
    R = lambda x, p: attention.rope_rotate(x[None], np.array([p]), 10000.0)[0]
    assert np.array_equal(R(q, 0.0), q)
    # composition and relative-position invariance of the dot product
    assert np.allclose(R(R(q, 17.0), 40.0), R(q, 57.0), atol=1e-12)
    a = R(q, 1000.0) @ R(k, 977.0)
    b = R(q, 23.0) @ R(k, 0.0)
    assert abs(a - b) < 1e-10
    # norms of every pair are preserved
    r = R(q, 131071.0)
    assert np.allclose(r[:64] ** 2 + r[64:] ** 2, q[:64] ** 2 + q[64:] ** 2, atol=1e-12)


def test_rope_attention_equals_relative_rotation_of_keys():
    rng = np.random.default_rng(4)
    T, d = 30, 128
    q = _rand(rng, 1, 1, d)
    K = _rand(rng, 1, 1, T, d)
    V = _rand(rng, 1, 1, T, d)
    p = 29
    out = attention.decode_attention(q, K, V, rope=True, q_pos=np.array([p]))
    # q . R(t - p) k computed through the shift-invariance with positions t - p
    Kr = attention.rope_rotate(K[0, 0], np.arange(T) - p, 10000.0)
    s = (Kr @ q[0, 0]) / math.sqrt(d)
    w = np.exp(s - s.max())
    w /= w.sum()
    assert np.allclose(out[0, 0], w @ V[0, 0], atol=1e-12)


def test_brute_force_python_loops_tiny():
    rng = np.random.default_rng(5)
    B, Hkv, g, T, d = 1, 2, 2, 6, 8
    q = _rand(rng, B, Hkv * g, d)
    K = _rand(rng, B, Hkv, T, d)
    V = _rand(rng, B, Hkv, T, d)
    out = attention.decode_attention(q, K, V, rope=True, rope_base=100.0, q_pos=np.array([9]))
    for j in range(Hkv * g):
        h = j // g
        def rot(x, pos):
            y = list(x)
            for i in range(d // 2):
                th = 100.0 ** (-2.0 * i / d)
                c, s = math.cos(pos * th), math.sin(pos * th)
                y[i] = x[i] * c - x[i + d // 2] * s
                y[i + d // 2] = x[i] * s + x[i + d // 2] * c
            return y
        qr = rot(list(q[0, j]), 9)
        scores = []
        for t in range(T):
            kr = rot(list(K[0, h, t]), t)
            scores.append(sum(a * b for a, b in zip(qr, kr)) / math.sqrt(d))
        mx = max(scores)
        ws = [math.exp(s - mx) for s in scores]
        tot = sum(ws)
        ref = [sum(ws[t] * V[0, h, t, c] for t in range(T)) / tot for c in range(d)]
        assert np.allclose(out[0, j], ref, atol=1e-13)
