"""GPU parity of the attention-sink prefix (KVQuant page, "Attention Sink").

The first S tokens of each sequence stay raw in the sink region and are
attended exactly (S up to 4096, which also covers a position threshold such
as quantizing only past the first 1000 tokens); the tokens after them form a quantized cache of their own
that starts at token S (per-channel key groups start there too), with
absolute positions for RoPE.  Each case checks the sink and the quantized
regions byte for byte against the oracle's encode_with_sink and the decode
output against the oracle's float64 attention (max-abs <= 2e-3, relative
L2 <= 1e-3), on every decode kernel that serves the format.
"""
import numpy as np
import pytest
import torch

from synth import make_inputs, make_workload

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

from parity import (MAX_ABS, REL_L2, attention_errors, compare_regions,  # noqa: E402
                    gpu_cache, oracle_attention, oracle_encode)

# (name, config id, workload overrides, append chunks, sink, decode paths, decode_splits)
CASES = [
    # per-channel 4-bit keys (groups of 64 from token 4 on); the second
    # append straddles the sink boundary (3 raw tokens, 27 quantized)
    ("u4_perchannel_straddle", 1, dict(ctx=500), [1, 30, 33, 64, 100, 272], 4,
     ("auto", "valu"), 0),
    # q8_0 with the largest sink and several splits of the quantized cache
    ("q8_0_sink64", 2, dict(ctx=4096), [4096], 64, ("auto", "valu"), 0),
    # 3-bit bf16, one raw token
    ("u3_sink1", 3, dict(batch=2, n_kv_heads=2, ctx=333), [7, 100, 226], 1, ("auto", "valu"), 0),
    # codebooks with outliers and RoPE: positions of the quantized tokens
    # start at the sink length
    ("nuq_rope_lut", 4, dict(n_kv_heads=4, ctx=300), [2, 1, 297], 4, ("lut", "valu"), 0),
    ("nuq_rope_lut_one_range", 4, dict(n_kv_heads=4, ctx=700), [700], 8, ("lut",), 1),
    # serving shape: single-token appends across the boundary, then a block
    ("serving_single_tokens", 5, dict(batch=2, n_kv_heads=2, ctx=400), [1] * 6 + [394], 4,
     ("auto", "valu"), 0),
    # one split of the quantized cache: the streaming kernel leaves a
    # partial state instead of the output, and the merge adds the sink's
    ("serving_one_split", 5, dict(batch=2, n_kv_heads=2, ctx=2000), [2000], 16,
     ("auto", "valu"), 1),
    # every token in the sink: only the sink kernel and the merge run
    ("all_sink_partial", 1, dict(ctx=3), [3], 8, ("auto",), 0),
    ("all_sink_exact", 5, dict(batch=2, n_kv_heads=2, ctx=8), [8], 8, ("auto",), 0),
    ("all_sink_one_token", 4, dict(n_kv_heads=4, ctx=1), [1], 1, ("lut",), 0),
    # one quantized token after the sink
    ("one_after_sink", 3, dict(batch=1, n_kv_heads=2, ctx=5), [5], 4, ("auto", "valu"), 0),
    # position thresholds: the first 1000 tokens raw, streamed in four
    # splits of their own; appends that end exactly at the threshold
    ("threshold_1000_serving", 5, dict(batch=2, n_kv_heads=2, ctx=1500), [600, 1, 399, 500],
     1000, ("auto", "valu"), 0),
    ("threshold_1000_lut_rope", 4, dict(n_kv_heads=4, ctx=1300), [1300], 1000, ("lut", "valu"), 0),
    # a ragged 300-token sink in one split beside one split of the rest
    ("sink_300_one_split", 3, dict(batch=1, n_kv_heads=2, ctx=700), [700], 300,
     ("auto", "valu"), 1),
    # the largest sink: 16 splits of raw tokens, alone or with a quantized rest
    ("sink_4096_all", 2, dict(ctx=4096), [4096], 4096, ("auto",), 0),
    ("sink_4096_plus", 2, dict(ctx=4200), [4000, 200], 4096, ("auto", "valu"), 0),
    # every token in one split of the sink: the general kernel writes the output
    ("all_sink_direct", 1, dict(ctx=100), [100], 200, ("auto",), 0),
]


def _build(name, cfg_id, over, chunks, sink, path, splits, max_extra=37):
    print(f"[sink] case={name} cfg={cfg_id} over={over} sink={sink} path={path} "
          f"splits={splits}", flush=True)
    w = make_workload(cfg_id, **over)
    inputs = make_inputs(w, "cpu")
    assert sum(chunks) == w.ctx
    max_ctx = w.ctx + max_extra
    cache = gpu_cache(w, inputs, chunks, max_ctx, decode_splits=splits, decode_path=path,
                      sink=sink)
    exp, kdeq, vdeq = oracle_encode(w, inputs, w.ctx, max_ctx, sink=sink)
    return w, inputs, cache, exp, kdeq, vdeq


@pytest.mark.parametrize("name,cfg_id,over,chunks,sink,paths,splits", CASES,
                         ids=[c[0] for c in CASES])
def test_sink_encode_and_attention(name, cfg_id, over, chunks, sink, paths, splits):
    for i, path in enumerate(paths):
        w, inputs, cache, exp, kdeq, vdeq = _build(name, cfg_id, over, chunks, sink, path, splits)
        if i == 0:
            bad = compare_regions(cache, exp)
            assert not bad, "\n".join(bad)
        q = inputs["q"]
        out = cache.decode(q.cuda()).cpu().numpy()
        ref = oracle_attention(w, q, kdeq, vdeq, w.ctx)
        ma, rel = attention_errors(out, ref)
        print(f"[sink] {name} path={path}: max_abs={ma:.3e} rel_l2={rel:.3e}", flush=True)
        assert ma <= MAX_ABS and rel <= REL_L2, (path, ma, rel)


@pytest.mark.parametrize("path", ["lut", "valu"])
def test_sink_with_explicit_query_position(path):
    w, inputs, cache, exp, kdeq, vdeq = _build("sink_qpos", 4, dict(n_kv_heads=2, ctx=257), [257],
                                               4, path, 0)
    q = inputs["q"]
    q_pos = np.array([1000], dtype=np.int32)
    out = cache.decode(q.cuda(), q_pos=torch.from_numpy(q_pos).cuda()).cpu().numpy()
    ref = oracle_attention(w, q, kdeq, vdeq, w.ctx, q_pos=q_pos)
    ma, rel = attention_errors(out, ref)
    print(f"[sink] qpos path={path}: max_abs={ma:.3e} rel_l2={rel:.3e}", flush=True)
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)


def test_sink_of_raw_cache_is_the_plain_raw_cache():
    """With raw fp16 storage a sink changes where the first tokens live, not
    what attention sees: the outputs agree with the sink-free cache to float
    rounding."""
    none = {"quantizer": "none", "bits": 16, "layout": "per_token"}
    over = dict(batch=2, n_kv_heads=2, ctx=300, k=none, v=none)
    w, inputs, with_sink, _, kdeq, vdeq = _build("raw_sink", 5, over, [300], 16, "auto", 0)
    _, _, plain, _, _, _ = _build("raw_plain", 5, over, [300], 0, "auto", 0)
    q = inputs["q"].cuda()
    a, b = with_sink.decode(q).cpu().numpy(), plain.decode(q).cpu().numpy()
    ref = oracle_attention(w, inputs["q"], kdeq, vdeq, w.ctx)
    for out in (a, b):
        ma, rel = attention_errors(out, ref)
        assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)
    assert np.max(np.abs(a - b)) <= 1e-5
