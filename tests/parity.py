"""Shared helpers for GPU parity tests and the smoke check: run a workload
through the HIP library (via the C ABI binding) and through the CPU oracle,
then compare packed bytes exactly and attention to tolerance.

Tolerance (attention output vs the oracle's float64 attention over the same
dequantized cache): max-abs <= 2e-3 and relative L2 <= 1e-3.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from oracle import attention as oatt
from oracle import layout as olay
from oracle import paging as opag
from oracle import quant as oq
from quantized_kv_cache_04_amd import kvq

MAX_ABS = 2e-3
REL_L2 = 1e-3


def to_np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def oracle_encode(w, inputs: Dict[str, Optional[torch.Tensor]], n_ctx: int, max_ctx: int,
                  sink: int = 0, page_table=None, n_pages: int = 0):
    """Oracle encode of the first n_ctx tokens -> (expected regions per tensor, deq K, deq V).

    With an attention sink of ``sink`` tokens the first min(sink, n_ctx)
    tokens are expected raw in the "sink" region and the rest as a quantized
    cache of their own.  With a page table (paged cache of ``n_pages``
    pages) the per-token regions are expected on the pages."""
    res = {}
    deq = {}
    for name in ("k", "v"):
        fmt = w.k if name == "k" else w.v
        x = to_np32(inputs[name][:, :n_ctx])
        cb = inputs[f"{name}_codebook"]
        cbn = cb.cpu().numpy() if cb is not None else None
        sc = inputs.get(f"{name}_scale")
        scn = sc.cpu().numpy() if sc is not None else None
        if sink:
            both = oq.encode_with_sink(x, fmt, cbn, sink, scn)
            enc, n_q = both["rest"], n_ctx - min(sink, n_ctx)
            deq[name] = both["deq"]
        else:
            enc, n_q = oq.encode_tensor(x, fmt, cbn, scn), n_ctx
            deq[name] = enc["deq"]
        exp = {}
        if fmt["quantizer"] != "none" and enc is not None:
            exp = olay.expected_regions(fmt, enc, batch=w.batch, n_kv_heads=w.n_kv_heads,
                                        n_ctx=n_q, max_ctx=max_ctx, kv_dtype=w.kv_dtype,
                                        is_key=(name == "k"))
            if page_table is not None:
                exp = opag.paged_regions(exp, np.asarray(page_table), n_pages=n_pages,
                                         n_ctx=n_q, capacity=olay.capacity(max_ctx),
                                         per_channel=fmt.get("layout") == "per_channel",
                                         k_out=oq.outlier_count(fmt.get("outlier_frac", 0.0),
                                                                w.n_kv_heads * w.head_dim),
                                         head_ng=([w.head_dim // g for g in fmt["head_group_size"]]
                                                  if fmt.get("head_group_size") else None),
                                         rec_halves=1 if fmt["quantizer"] == "sym_q8_0" else 2)
        if sink:
            exp["sink"] = olay.sink_region(x, sink, kv_dtype=w.kv_dtype)
        res[name] = exp or None
    return res, deq["k"], deq["v"]


def gpu_cache(w, inputs, chunks: Sequence[int], max_ctx: int, decode_splits: int = 0,
              decode_path: str = "auto", device: str = "cuda", sink: int = 0,
              page_table=None, n_pages: int = 0) -> kvq.Cache:
    """Build the cache on the GPU by appending the inputs in ``chunks`` token
    counts (a paged cache of ``n_pages`` pages when ``page_table`` is given)."""
    cfg = kvq.config_from_workload(w, max_ctx=max_ctx, decode_splits=decode_splits,
                                   decode_path=decode_path, sink_tokens=sink,
                                   page_pool=n_pages if page_table is not None else 0)
    dev = lambda t: t.to(device) if t is not None else None  # noqa: E731
    cache = kvq.Cache(cfg, device=device, k_codebook=dev(inputs["k_codebook"]),
                      v_codebook=dev(inputs["v_codebook"]), k_scale=dev(inputs.get("k_scale")),
                      v_scale=dev(inputs.get("v_scale")), page_table=dev(page_table))
    kd = inputs["k"].to(device)
    vd = inputs["v"].to(device)
    t = 0
    for n in chunks:
        cache.append(kd[:, t:t + n].contiguous(), vd[:, t:t + n].contiguous())
        t += n
    torch.cuda.synchronize()
    assert cache.n_ctx == t
    return cache


def _as_bytes(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint8).reshape(-1)


def compare_regions(cache: kvq.Cache, expected) -> List[str]:
    """Byte-exact comparison of every quantized region; returns mismatch descriptions."""
    bad = []
    for name in ("k", "v"):
        exp = expected[name]
        if exp is None:
            continue
        for reg in ("codes", "params", "tail", "row_ptr", "col", "val", "sink", "tile_off", "tile_ent"):
            if reg not in exp:
                continue
            got = cache.region(name, reg).cpu().numpy()
            want = _as_bytes(exp[reg])
            if got.shape != want.shape:
                bad.append(f"{name}.{reg}: size {got.shape} != {want.shape}")
                continue
            diff = np.nonzero(got != want)[0]
            if diff.size:
                bad.append(f"{name}.{reg}: {diff.size} bytes differ, first at {diff[0]} "
                           f"(got {got[diff[0]]}, want {want[diff[0]]})")
    return bad


def attention_errors(out: np.ndarray, ref: np.ndarray):
    d = out.astype(np.float64) - ref
    max_abs = float(np.max(np.abs(d)))
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    return max_abs, rel


def oracle_attention(w, q: torch.Tensor, kdeq, vdeq, n_ctx: int, q_pos=None):
    return oatt.decode_attention(to_np32(q), kdeq, vdeq, n_ctx=n_ctx, rope=w.rope,
                                 rope_base=w.rope_base,
                                 q_pos=None if q_pos is None else np.asarray(q_pos))


def oracle_prefill(w, q: torch.Tensor, kdeq, vdeq, n_ctx: int):
    """Oracle causal attention of the last q.shape[1] tokens of an n_ctx cache."""
    return oatt.prefill_attention(to_np32(q), kdeq, vdeq, n_ctx=n_ctx, rope=w.rope,
                                  rope_base=w.rope_base)
