"""GPU parity of chunked-prefill attention (kvq_prefill_attention) against
the oracle's causal multi-query attention over the same dequantized cache.

The chunk's keys and values are appended first; query i of the last n_q
tokens then attends tokens 0 .. n_ctx - n_q + i.  Every format runs on the
matrix-core prefill kernel; outputs must match the oracle's float64 result to
max-abs <= 2e-3 and relative L2 <= 1e-3, the bar of the decode path.
Sizes span several 64-row query tiles, ragged last tiles, several 32-token
blocks and a causal boundary inside a block.
"""
import numpy as np
import pytest
import torch

from synth import make_inputs, make_prefill_queries, make_workload

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

from parity import (MAX_ABS, REL_L2, attention_errors, gpu_cache,  # noqa: E402
                    oracle_attention, oracle_encode, oracle_prefill)

# (name, config id, workload overrides, append chunks, n_q, sink)
CASES = [
    # per-channel 4-bit keys with their fp16 tail, g = 2 (32 tokens a tile)
    ("u4_pc_last_chunk", 1, dict(ctx=500), [1, 30, 33, 64, 100, 272], 272, 0),
    ("u4_pc_whole_sequence", 1, dict(ctx=500), [500], 500, 0),
    ("u4_pc_one_query", 1, dict(ctx=500), [499, 1], 1, 0),
    # q8_0, g = 8 (8 tokens a tile)
    ("q8_0_g8", 2, dict(ctx=1000), [700, 300], 300, 0),
    # 3-bit bf16, g = 8, two sequences
    ("u3_bf16_b2", 3, dict(batch=2, n_kv_heads=2, ctx=333), [233, 100], 100, 0),
    # codebooks with 1% outliers and RoPE, MHA (64 tokens a tile)
    ("nuq_rope_mha", 4, dict(n_kv_heads=4, ctx=300), [200, 100], 100, 0),
    ("nuq_rope_gqa2", 4, dict(n_kv_heads=2, gqa=2, ctx=260), [260], 130, 0),
    # serving formats (per-channel groups of 128), g = 4
    ("serving_chunk", 5, dict(batch=2, n_kv_heads=2, ctx=1000), [872, 128], 128, 0),
    ("serving_whole", 5, dict(batch=1, n_kv_heads=2, ctx=300), [300], 300, 0),
    # attention sink and a position threshold before the quantized tokens
    ("serving_sink4", 5, dict(batch=2, n_kv_heads=2, ctx=700), [600, 100], 100, 4),
    ("nuq_rope_threshold", 4, dict(n_kv_heads=4, ctx=1300), [1000, 300], 300, 1000),
    ("u4_pc_all_sink", 1, dict(ctx=40), [40], 40, 64),
    # the largest group: one query token a tile
    ("u3_g64", 3, dict(batch=1, n_kv_heads=1, gqa=64, ctx=200), [200], 50, 0),
    ("q8_0_g16", 2, dict(n_kv_heads=1, gqa=16, ctx=129), [129], 129, 0),
    # a single token
    ("single_token", 5, dict(batch=1, n_kv_heads=2, ctx=1), [1], 1, 0),
]


def _build(name, cfg_id, over, chunks, sink, max_extra=37):
    print(f"[prefill] case={name} cfg={cfg_id} over={over} sink={sink}", flush=True)
    w = make_workload(cfg_id, **over)
    inputs = make_inputs(w, "cpu")
    assert sum(chunks) == w.ctx
    max_ctx = w.ctx + max_extra
    cache = gpu_cache(w, inputs, chunks, max_ctx, sink=sink)
    _, kdeq, vdeq = oracle_encode(w, inputs, w.ctx, max_ctx, sink=sink)
    return w, cache, kdeq, vdeq


@pytest.mark.parametrize("name,cfg_id,over,chunks,n_q,sink", CASES, ids=[c[0] for c in CASES])
def test_prefill_matches_oracle(name, cfg_id, over, chunks, n_q, sink):
    w, cache, kdeq, vdeq = _build(name, cfg_id, over, chunks, sink)
    q = make_prefill_queries(w, n_q)
    out = cache.prefill(q.cuda()).cpu().numpy()
    ref = oracle_prefill(w, q, kdeq, vdeq, w.ctx)
    ma, rel = attention_errors(out, ref)
    print(f"[prefill] {name}: max_abs={ma:.3e} rel_l2={rel:.3e}", flush=True)
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)


def test_last_prefill_row_is_the_decode_step():
    """The last query row of a chunk sees the whole cache: its output is what
    decode attention gives for that query (both to the oracle's bar)."""
    w, cache, kdeq, vdeq = _build("last_row", 5, dict(batch=2, n_kv_heads=2, ctx=900), [900], 0)
    q = make_prefill_queries(w, 70)
    out = cache.prefill(q.cuda()).cpu().numpy()
    dec = cache.decode(q[:, -1].contiguous().cuda()).cpu().numpy()
    ref = oracle_attention(w, q[:, -1], kdeq, vdeq, w.ctx)
    for got in (out[:, -1], dec):
        ma, rel = attention_errors(got, ref)
        assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)
    assert np.max(np.abs(out[:, -1] - dec)) <= 2 * MAX_ABS


@pytest.mark.parametrize("odt,tdt", [("f16", torch.float16), ("bf16", torch.bfloat16)])
def test_half_outputs_are_rounded_f32_outputs(odt, tdt):
    w, cache, _, _ = _build("prefill_out", 1, dict(ctx=200), [200], 0)
    q = make_prefill_queries(w, 77).cuda()
    o32 = cache.prefill(q)
    oh = cache.prefill(q, out_dtype=odt)
    assert oh.dtype == tdt
    assert torch.equal(oh, o32.to(tdt))


def test_prefill_is_deterministic_and_leaves_the_cache_alone():
    w, cache, _, _ = _build("prefill_repeat", 3, dict(batch=2, n_kv_heads=2, ctx=400), [400], 0)
    before = cache.buffer.clone()
    q = make_prefill_queries(w, 150).cuda()
    a = cache.prefill(q)
    for _ in range(2):
        assert torch.equal(cache.prefill(q), a)
    torch.cuda.synchronize()
    assert torch.equal(cache.buffer, before)


SPLIT_CASES = [
    # the staging kernel (codebooks with RoPE; a sink)
    ("split_nuq_rope", 4, dict(n_kv_heads=2, ctx=2000), [1900, 100], 100, 0),
    ("split_serving_sink", 5, dict(batch=1, n_kv_heads=2, ctx=3000), [3000], 64, 40),
    # the code-operand kernel: per-channel keys with their tail, and q8_0
    # (whose waves share the unpacking)
    ("split_serving", 5, dict(batch=1, n_kv_heads=2, ctx=3001), [2900, 101], 101, 0),
    ("split_q8_0", 2, dict(ctx=4000), [4000], 70, 0),
]


@pytest.mark.parametrize("name,cfg_id,over,chunks,n_q,sink", SPLIT_CASES,
                         ids=[c[0] for c in SPLIT_CASES])
def test_token_axis_split_matches_the_unsplit_kernel(name, cfg_id, over, chunks, n_q, sink):
    """With a workspace the token axis is split over several workgroups and
    their partial states are merged; without one it is not.  Both match the
    oracle."""
    from quantized_kv_cache_04_amd import kvq as K
    w, cache, kdeq, vdeq = _build(name, cfg_id, over, chunks, sink)
    assert K.prefill_workspace_bytes(cache.cfg, n_q, w.ctx) > 0
    q = make_prefill_queries(w, n_q).cuda()
    split = cache.prefill(q).cpu().numpy()
    whole = cache.prefill(q, workspace=torch.empty(0, dtype=torch.uint8, device="cuda")).cpu().numpy()
    ref = oracle_prefill(w, q.cpu(), kdeq, vdeq, w.ctx)
    for out in (split, whole):
        ma, rel = attention_errors(out, ref)
        print(f"[prefill] {name}: max_abs={ma:.3e} rel_l2={rel:.3e}", flush=True)
        assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)
