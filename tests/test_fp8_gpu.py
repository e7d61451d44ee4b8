"""GPU parity of the FP8 E5M2 cache format (Survey page, section 3.4: vLLM's
fp8 KV cache, 5 exponent and 2 mantissa bits, a scale per head).

Encoded bytes must match the oracle byte for byte (every E5M2 code, in the
8-bit key-row and value-tile layouts); decode and prefill attention must
match the oracle's float64 attention over the same dequantized cache to
max-abs <= 2e-3 and relative L2 <= 1e-3.  Per-head scales are seeded
log-uniform in [1/4, 4]; one case runs with unit scales (null pointers).
"""
import pytest
import torch

from synth import make_inputs, make_prefill_queries, make_workload

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

from parity import (MAX_ABS, REL_L2, attention_errors, compare_regions,  # noqa: E402
                    gpu_cache, oracle_attention, oracle_encode, oracle_prefill)

FP8 = dict(quantizer="fp8_e5m2", bits=8, group_size=0, layout="per_token", outlier_frac=0.0)
Q8 = dict(quantizer="sym_q8_0", bits=8, group_size=32, layout="per_token", outlier_frac=0.0)

# (name, config id, workload overrides, append chunks, sink, unit scales)
CASES = [
    ("serving_fp8", 5, dict(batch=2, n_kv_heads=2, ctx=500, k=FP8, v=FP8), [1, 30, 33, 436], 0, False),
    ("serving_fp8_unit_scales", 5, dict(batch=2, n_kv_heads=2, ctx=300, k=FP8, v=FP8), [300], 0, True),
    ("bf16_fp8_g8", 3, dict(batch=2, n_kv_heads=2, ctx=333, k=FP8, v=FP8), [7, 326], 0, False),
    ("rope_mha_fp8", 4, dict(n_kv_heads=4, ctx=400, k=FP8, v=FP8), [400], 0, False),
    ("fp8_keys_q8_values", 2, dict(ctx=1000, k=FP8, v=Q8), [999, 1], 0, False),
    ("fp8_sink", 5, dict(batch=2, n_kv_heads=2, ctx=700, k=FP8, v=FP8), [600, 100], 16, False),
]


def _build(name, cfg_id, over, chunks, sink, unit, max_extra=37, path="auto"):
    print(f"[fp8] case={name} cfg={cfg_id} sink={sink} unit_scales={unit} path={path}", flush=True)
    w = make_workload(cfg_id, **over)
    inputs = make_inputs(w, "cpu")
    if unit:
        inputs["k_scale"] = inputs["v_scale"] = None
    assert sum(chunks) == w.ctx
    max_ctx = w.ctx + max_extra
    cache = gpu_cache(w, inputs, chunks, max_ctx, sink=sink, decode_path=path)
    exp, kdeq, vdeq = oracle_encode(w, inputs, w.ctx, max_ctx, sink=sink)
    return w, inputs, cache, exp, kdeq, vdeq


@pytest.mark.parametrize("name,cfg_id,over,chunks,sink,unit", CASES, ids=[c[0] for c in CASES])
def test_fp8_bytes_decode_and_prefill(name, cfg_id, over, chunks, sink, unit):
    w, inputs, cache, exp, kdeq, vdeq = _build(name, cfg_id, over, chunks, sink, unit)
    bad = compare_regions(cache, exp)
    assert not bad, "\n".join(bad)
    q = inputs["q"]
    out = cache.decode(q.cuda()).cpu().numpy()
    ma, rel = attention_errors(out, oracle_attention(w, q, kdeq, vdeq, w.ctx))
    print(f"[fp8] {name} decode: max_abs={ma:.3e} rel_l2={rel:.3e}", flush=True)
    assert ma <= MAX_ABS and rel <= REL_L2, ("decode", ma, rel)
    n_q = min(w.ctx, 96)
    qp = make_prefill_queries(w, n_q)
    outp = cache.prefill(qp.cuda()).cpu().numpy()
    ma, rel = attention_errors(outp, oracle_prefill(w, qp, kdeq, vdeq, w.ctx))
    print(f"[fp8] {name} prefill: max_abs={ma:.3e} rel_l2={rel:.3e}", flush=True)
    assert ma <= MAX_ABS and rel <= REL_L2, ("prefill", ma, rel)


# FP8 keys and values without RoPE (config 4 carries RoPE): the matrix-core cases
MFMA_CASES = [c for c in CASES if c[2]["v"] is FP8 and c[1] != 4]


@pytest.mark.parametrize("name,cfg_id,over,chunks,sink,unit", MFMA_CASES,
                         ids=[c[0] for c in MFMA_CASES])
def test_fp8_decode_on_the_general_kernel(name, cfg_id, over, chunks, sink, unit):
    """FP8 keys and values decode on the matrix cores by default; the general
    kernel must agree with the oracle too."""
    w, inputs, cache, exp, kdeq, vdeq = _build(name, cfg_id, over, chunks, sink, unit, path="valu")
    q = inputs["q"]
    out = cache.decode(q.cuda()).cpu().numpy()
    ma, rel = attention_errors(out, oracle_attention(w, q, kdeq, vdeq, w.ctx))
    print(f"[fp8] {name} valu decode: max_abs={ma:.3e} rel_l2={rel:.3e}", flush=True)
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)


@pytest.mark.parametrize("splits", [1, 3])
def test_fp8_mfma_long_context_and_splits(splits):
    over = dict(batch=2, n_kv_heads=2, ctx=3000, k=FP8, v=FP8)
    w, inputs, cache, exp, kdeq, vdeq = _build(f"fp8_splits{splits}", 5, over, [3000], 0, False)
    cache.cfg.decode_splits = splits
    q = inputs["q"]
    out = cache.decode(q.cuda()).cpu().numpy()
    ma, rel = attention_errors(out, oracle_attention(w, q, kdeq, vdeq, w.ctx))
    print(f"[fp8] splits={splits}: max_abs={ma:.3e} rel_l2={rel:.3e}", flush=True)
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)
