"""Float64 decode attention over a dequantized cache.

Test infrastructure: see the package docstring.

This is the plain definition that a fused, split-K kernel reaches faster:
every decode step scores the query against every cached key and takes the
softmax-weighted sum of the cached values (Memory-killer page, section 1.3:
each generated token reads the whole cache; Survey page, section 2.3:
scores, softmax and the value product).  Grouped heads: query head j reads
KV head floor(j / g) (TurboQuant page, section 2.1 counts h = 8 KV heads for
a 64-head 70B model).  Softmax scale 1/sqrt(d) unless given.

RoPE (KVQuant page, sections 2.1-2.2: keys are quantized before the rotary
embedding, which is applied afterwards): rotate-half pairs (i, i + d/2),
theta_i = base^(-2i/d), key t at position t, query at ``q_pos``; angles are
formed in float64.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def rope_rotate(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate the last axis of ``x`` [..., d] at positions ``pos`` (broadcast
    against x[..., 0]) by the rotate-half RoPE with the given base."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    i = np.arange(h, dtype=np.float64)
    theta = np.power(np.float64(base), -2.0 * i / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def decode_attention(q: np.ndarray, k_deq: np.ndarray, v_deq: np.ndarray, *,
                     n_ctx: Optional[int] = None, sm_scale: Optional[float] = None,
                     rope: bool = False, rope_base: float = 10000.0,
                     q_pos: Optional[np.ndarray] = None) -> np.ndarray:
    """q [B, Hq, d]; k_deq, v_deq [B, Hkv, T, d] (float64 dequantized cache).
    Attends over tokens [0, n_ctx).  Returns float64 [B, Hq, d]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k_deq.shape[1]
    T = k_deq.shape[2] if n_ctx is None else n_ctx
    g = Hq // Hkv
    sm = 1.0 / np.sqrt(d) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    out = np.empty((B, Hq, d), dtype=np.float64)
    for b in range(B):
        p = (T - 1) if q_pos is None else int(q_pos[b])
        for h in range(Hkv):
            K = np.asarray(k_deq[b, h, :T], dtype=np.float64)
            V = np.asarray(v_deq[b, h, :T], dtype=np.float64)
            if rope:
                K = rope_rotate(K, np.arange(T), rope_base)
            for jj in range(g):
                j = h * g + jj
                qj = q[b, j]
                if rope:
                    qj = rope_rotate(qj[None, :], np.array([p]), rope_base)[0]
                s = sm * (K @ qj)
                s = s - s.max()
                w = np.exp(s)
                w = w / w.sum()
                out[b, j] = w @ V
    return out


def prefill_attention(q: np.ndarray, k_deq: np.ndarray, v_deq: np.ndarray, *,
                      n_ctx: Optional[int] = None, sm_scale: Optional[float] = None,
                      rope: bool = False, rope_base: float = 10000.0) -> np.ndarray:
    """Causal attention of the last n_q tokens of the cache (chunked prefill).

    The prefill step builds the cache and scores every new token's query
    against the keys before it (NIAH page, section 4.2: first-token latency
    comes from the prefill pass; Survey page, sections 2.3 and 5.3: QK^T,
    softmax and the value product of prefill kept on chip).  Here the new
    tokens have already been appended, so they are the last n_q tokens of a
    cache of n_ctx: query i (position n_ctx - n_q + i) attends tokens
    [0, n_ctx - n_q + i], each row exactly as ``decode_attention`` with that
    context and query position.

    q [B, n_q, Hq, d]; k_deq, v_deq [B, Hkv, T, d] (float64 dequantized
    cache).  Returns float64 [B, n_q, Hq, d].
    """
    q = np.asarray(q, dtype=np.float64)
    B, n_q, Hq, d = q.shape
    Hkv = k_deq.shape[1]
    T = k_deq.shape[2] if n_ctx is None else n_ctx
    if not 1 <= n_q <= T:
        raise ValueError("need 1 <= n_q <= n_ctx")
    g = Hq // Hkv
    sm = 1.0 / np.sqrt(d) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    base = T - n_q
    out = np.empty((B, n_q, Hq, d), dtype=np.float64)
    for b in range(B):
        for h in range(Hkv):
            K = np.asarray(k_deq[b, h, :T], dtype=np.float64)
            V = np.asarray(v_deq[b, h, :T], dtype=np.float64)
            if rope:
                K = rope_rotate(K, np.arange(T), rope_base)
            for i in range(n_q):
                p = base + i                      # query position; keys 0..p
                for jj in range(g):
                    j = h * g + jj
                    qj = q[b, i, j]
                    if rope:
                        qj = rope_rotate(qj[None, :], np.array([p]), rope_base)[0]
                    s = sm * (K[:p + 1] @ qj)
                    s = s - s.max()
                    w = np.exp(s)
                    w = w / w.sum()
                    out[b, i, j] = w @ V[:p + 1]
    return out
