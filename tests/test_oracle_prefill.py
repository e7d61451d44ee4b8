"""Pins for the oracle's causal multi-query (chunked prefill) attention, CPU
only: torch's scaled_dot_product_attention in float64 with a causal mask, the
decode definition on single rows, causality by perturbation, and a
pure-Python brute force with RoPE on tiny inputs."""
import math

import numpy as np
import pytest
import torch

from oracle import attention


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("g,n_q", [(1, 37), (2, 37), (4, 5), (8, 1)])
def test_matches_torch_sdpa_with_a_bottom_right_causal_mask(g, n_q):
    rng = np.random.default_rng(10 + g)
    B, Hkv, T, d = 2, 3, 37, 128
    q = _rand(rng, B, n_q, Hkv * g, d)
    K = _rand(rng, B, Hkv, T, d)
    V = _rand(rng, B, Hkv, T, d)
    out = attention.prefill_attention(q, K, V)
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)                 # [B, Hq, n_q, d]
    Kt = torch.from_numpy(K).repeat_interleave(g, dim=1)
    Vt = torch.from_numpy(V).repeat_interleave(g, dim=1)
    # query i sits at position T - n_q + i and sees keys 0 .. T - n_q + i
    mask = torch.arange(T)[None, :] <= (T - n_q + torch.arange(n_q))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask)
    ref = ref.permute(0, 2, 1, 3).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12
    if n_q == T:   # the whole sequence: torch's own causal flag
        ref2 = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, is_causal=True)
        assert np.max(np.abs(out - ref2.permute(0, 2, 1, 3).numpy())) < 1e-12


def test_rows_are_decode_steps():
    rng = np.random.default_rng(20)
    B, Hkv, g, T, d, n_q = 1, 2, 2, 50, 128, 7
    q = _rand(rng, B, n_q, Hkv * g, d)
    K = _rand(rng, B, Hkv, T, d)
    V = _rand(rng, B, Hkv, T, d)
    out = attention.prefill_attention(q, K, V, rope=True)
    for i in range(n_q):
        p = T - n_q + i
        row = attention.decode_attention(q[:, i], K, V, n_ctx=p + 1, rope=True, q_pos=np.array([p]))
        assert np.allclose(out[:, i], row, rtol=0, atol=1e-13)


def test_first_token_sees_only_itself():
    rng = np.random.default_rng(21)
    T = 9
    q = _rand(rng, 1, T, 2, 128)
    K = _rand(rng, 1, 1, T, 128)
    V = _rand(rng, 1, 1, T, 128)
    out = attention.prefill_attention(q, K, V)
    assert np.array_equal(out[0, 0, 0], V[0, 0, 0]) and np.array_equal(out[0, 0, 1], V[0, 0, 0])


def test_future_tokens_do_not_matter():
    rng = np.random.default_rng(22)
    T, n_q = 40, 12
    q = _rand(rng, 1, n_q, 4, 128)
    K = _rand(rng, 1, 2, T, 128)
    V = _rand(rng, 1, 2, T, 128)
    a = attention.prefill_attention(q, K, V, rope=True)
    K2, V2 = K.copy(), V.copy()
    K2[:, :, 35:] += 5.0
    V2[:, :, 35:] -= 3.0
    b = attention.prefill_attention(q, K2, V2, rope=True)
    # rows 0..6 sit at positions 28..34 and never see tokens 35 and later
    assert np.array_equal(a[:, :7], b[:, :7])
    assert not np.allclose(a[:, 7:], b[:, 7:])


def test_n_ctx_and_argument_checks():
    rng = np.random.default_rng(23)
    q = _rand(rng, 1, 3, 2, 128)
    K = _rand(rng, 1, 1, 30, 128)
    V = _rand(rng, 1, 1, 30, 128)
    a = attention.prefill_attention(q, K, V, n_ctx=20)
    b = attention.prefill_attention(q, K[:, :, :20], V[:, :, :20])
    assert np.array_equal(a, b)
    with pytest.raises(ValueError):
        attention.prefill_attention(q, K, V, n_ctx=2)


def test_brute_force_python_loops_tiny():
    rng = np.random.default_rng(24)
    Hkv, g, T, d, n_q, base = 2, 2, 6, 8, 3, 100.0
    q = _rand(rng, 1, n_q, Hkv * g, d)
    K = _rand(rng, 1, Hkv, T, d)
    V = _rand(rng, 1, Hkv, T, d)
    out = attention.prefill_attention(q, K, V, rope=True, rope_base=base)

    def rot(x, pos):
        y = list(x)
        for i in range(d // 2):
            c, s = math.cos(pos * base ** (-2.0 * i / d)), math.sin(pos * base ** (-2.0 * i / d))
            y[i] = x[i] * c - x[i + d // 2] * s
            y[i + d // 2] = x[i] * s + x[i + d // 2] * c
        return y

    for i in range(n_q):
        p = T - n_q + i
        for j in range(Hkv * g):
            h = j // g
            qr = rot(list(q[0, i, j]), p)
            scores = []
            for t in range(p + 1):
                kr = rot(list(K[0, h, t]), t)
                scores.append(sum(a * b for a, b in zip(qr, kr)) / math.sqrt(d))
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            z = sum(w)
            for c in range(d):
                want = sum(w[t] * V[0, h, t, c] for t in range(p + 1)) / z
                assert abs(out[0, i, j, c] - want) < 1e-12
