"""Closed-form byte counts of the cache (the bytes a decode step must read).

Test infrastructure: see the package docstring.

Unquantized, a token costs 2 * L * h * d * bytes (K and V, L layers, h KV
heads of dimension d), the TurboQuant page's section 2.1 formula; element
counts follow the Memory-killer page's section 1.2 (2 * L * H * D * S).
Quantized formats count packed codes, fp16 scale (+ zero) per group, the
fp16 tail of an unfinished per-channel group, the CSR outliers (4-byte row
pointer + 2-byte column + 2-byte value per kept entry + a one-byte count
of the row's entries per KV head) and the fp16 codebooks.  With an attention sink of S tokens (KVQuant page, "Attention
Sink"), the first min(S, n) tokens cost their raw fp16/bf16 bytes and the
format applies to the remaining n - min(S, n) tokens.
"""
from __future__ import annotations

from typing import Dict

from .quant import outlier_count

ESIZE = {"f16": 2, "bf16": 2}


def tensor_payload(fmt: Dict, *, batch: int, n_kv_heads: int, head_dim: int, n_ctx: int,
                   kv_dtype: str = "f16") -> int:
    B, H, d, n = batch, n_kv_heads, head_dim, n_ctx
    q = fmt["quantizer"]
    if q == "none":
        return B * H * n * d * ESIZE[kv_dtype]
    bits = fmt["bits"]
    rb = d * bits // 8
    G = fmt.get("group_size", 0)
    if q == "fp8_e5m2":
        # one byte per element and the per-head float32 scales decode reads
        return B * H * n * d + H * 4
    if q == "codebook":
        total = B * H * n * rb + H * d * 16 * 2
        k = outlier_count(fmt.get("outlier_frac", 0.0), H * d)
        if k:
            # the per-tile index decode streams: 4 bytes per entry, and the
            # head offsets of each tile the n tokens touch (rows of whole
            # 16-byte units)
            total += B * (n * 4 * k + (n + 31) // 32 * ((H + 8) // 8 * 16))
        return total
    if fmt.get("layout", "per_token") == "per_channel":
        nf = (n // G) * G
        return B * H * (nf * rb + (nf // G) * d * 4 + (n - nf) * d * ESIZE[kv_dtype])
    psize = 2 if q == "sym_q8_0" else 4
    if fmt.get("head_group_size"):
        # a group size per KV head: each head's own groups per token
        return B * n * (H * rb + sum(d // int(g) for g in fmt["head_group_size"]) * psize)
    return B * H * n * (rb + (d // G) * psize)


def payload_bytes(k_fmt: Dict, v_fmt: Dict, *, batch: int, n_kv_heads: int, head_dim: int,
                  n_ctx: int, n_layers: int = 1, kv_dtype: str = "f16", sink: int = 0) -> int:
    s = min(int(sink), n_ctx)
    kw = dict(batch=batch, n_kv_heads=n_kv_heads, head_dim=head_dim, n_ctx=n_ctx - s,
              kv_dtype=kv_dtype)
    raw = batch * n_kv_heads * s * head_dim * ESIZE[kv_dtype]
    return n_layers * (tensor_payload(k_fmt, **kw) + tensor_payload(v_fmt, **kw) + 2 * raw)
