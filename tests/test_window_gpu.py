"""GPU parity of per-channel key groups whose scale and zero come from
overlapping sliding windows (TurboQuant page, section 3.1: parameters from a
sliding window's extrema; section 6, problem 1: windows overlapping by 64
tokens).  Group g of G tokens takes its statistics from tokens
[g G - overlap, g G + G); the key tail is a ring of G + overlap rows.

Checked: every cache byte against the oracle (codes, per-group parameters,
the tail ring), and decode and prefill attention against the oracle's
float64 attention (max-abs <= 2e-3, rel-L2 <= 1e-3), with bulk, ragged and
one-token appends, on the matrix-core and the general kernel, with a sink
and on a paged cache.
"""
import numpy as np
import pytest
import torch

from synth import make_inputs, make_page_table, make_prefill_queries, make_workload

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

from parity import (MAX_ABS, REL_L2, attention_errors, compare_regions, gpu_cache,  # noqa: E402
                    oracle_attention, oracle_encode, oracle_prefill)


def _kfmt(q, bits, G, overlap):
    return dict(quantizer=q, bits=bits, group_size=G, layout="per_channel", outlier_frac=0.0,
                window_overlap=overlap)


# (name, config, sizes + key format, chunks, sink, path, paged)
CASES = [
    # the TurboQuant page's windows: 256 tokens overlapping by 64 (G = 192)
    ("turboquant_256_64", 5, dict(batch=2, n_kv_heads=2, ctx=900,
                                  k=_kfmt("asym_absmax_offset", 4, 192, 64)),
     [500, 1, 1, 398], 0, "auto", False),
    ("minmax_g128_o32", 5, dict(batch=2, n_kv_heads=2, ctx=700,
                                k=_kfmt("asym_minmax", 4, 128, 32)),
     [1, 127, 1, 300, 271], 0, "auto", False),
    # the window reaches back over several groups
    ("g32_o256_3bit", 1, dict(ctx=600, k=_kfmt("asym_minmax", 3, 32, 256)),
     [100, 33, 1, 466], 0, "auto", False),
    ("general_kernel", 5, dict(batch=1, n_kv_heads=2, ctx=650,
                               k=_kfmt("asym_absmax_offset", 4, 96, 64)),
     [650], 0, "valu", False),
    ("bf16_8bit", 3, dict(batch=1, n_kv_heads=2, ctx=500,
                          k=_kfmt("asym_minmax", 8, 64, 64)),
     [250, 250], 0, "auto", False),
    ("sink", 5, dict(batch=2, n_kv_heads=2, ctx=800, k=_kfmt("asym_minmax", 4, 128, 64)),
     [700, 100], 24, "auto", False),
    ("paged", 5, dict(batch=2, n_kv_heads=2, ctx=700, k=_kfmt("asym_minmax", 4, 128, 64)),
     [300, 400], 0, "auto", True),
]


@pytest.mark.parametrize("name,cfg_id,over,chunks,sink,path,paged", CASES,
                         ids=[c[0] for c in CASES])
def test_window_bytes_and_attention(name, cfg_id, over, chunks, sink, path, paged):
    print(f"[window] case={name} cfg={cfg_id} sink={sink} path={path} paged={paged}", flush=True)
    w = make_workload(cfg_id, **over)
    inputs = make_inputs(w, "cpu")
    assert sum(chunks) == w.ctx
    max_ctx = w.ctx + 40
    table, n_pages = None, 0
    if paged:
        n_pages = w.batch * ((max_ctx + 31) // 32) + 5
        table = make_page_table(w, max_ctx, n_pages)
    cache = gpu_cache(w, inputs, chunks, max_ctx, sink=sink, decode_path=path,
                      page_table=table, n_pages=n_pages)
    exp, kdeq, vdeq = oracle_encode(w, inputs, w.ctx, max_ctx, sink=sink,
                                    page_table=None if table is None else table.numpy(),
                                    n_pages=n_pages)
    bad = compare_regions(cache, exp)
    assert not bad, "; ".join(bad)
    out = cache.decode(inputs["q"].cuda()).cpu().numpy()
    ma, rel = attention_errors(out, oracle_attention(w, inputs["q"], kdeq, vdeq, w.ctx))
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)
    n_q = chunks[-1]
    q = make_prefill_queries(w, n_q)
    outp = cache.prefill(q.cuda()).cpu().numpy()
    ma, rel = attention_errors(outp, oracle_prefill(w, q, kdeq, vdeq, w.ctx))
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)


def test_one_token_steps_through_window_boundaries():
    # the serving step, one token at a time over two group boundaries; the
    # whole cache (ring included) is compared at every step that ends a group
    w = make_workload(5, batch=2, n_kv_heads=1, ctx=290, k=_kfmt("asym_minmax", 4, 64, 64))
    inputs = make_inputs(w, "cpu")
    max_ctx = 300
    cache = gpu_cache(w, inputs, [100], max_ctx)
    kd, vd = inputs["k"].cuda(), inputs["v"].cuda()
    for t in range(100, 290):
        cache.append(kd[:, t:t + 1].contiguous(), vd[:, t:t + 1].contiguous())
        n = t + 1
        if n % 64 in (0, 1, 63):
            torch.cuda.synchronize()
            exp, kdeq, vdeq = oracle_encode(w, inputs, n, max_ctx)
            bad = compare_regions(cache, exp)
            assert not bad, f"n={n}: " + "; ".join(bad)
    out = cache.decode(inputs["q"].cuda()).cpu().numpy()
    _, kdeq, vdeq = oracle_encode(w, inputs, 290, max_ctx)
    ma, rel = attention_errors(out, oracle_attention(w, inputs["q"], kdeq, vdeq, 290))
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)
