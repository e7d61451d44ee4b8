"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Packed codes, scales, zero points, tails and CSR outliers must match the
oracle byte for byte (including the untouched zero bytes of the capacity);
decode attention must match the oracle's float64 attention over the same
dequantized cache to max-abs <= 2e-3 and relative L2 <= 1e-3.

Sizes here are small enough for the oracle to finish in seconds, yet span
several 32-token tiles, several quantization groups and a ragged tail.
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

# (name, config id, workload overrides, append chunks)
CASES = [
    ("tiny_full", 1, {}, [512]),
    ("tiny_ragged_chunks", 1, dict(ctx=500), [1, 30, 33, 64, 100, 272]),
    ("tiny_single_token", 1, dict(ctx=1), [1]),
    ("q8_0_4k", 2, dict(ctx=4096), [4096]),
    ("q8_0_16k_chunks", 2, dict(ctx=16384), [8000, 1, 8383]),
    ("q8_0_ragged", 2, dict(ctx=77), [77]),
    ("u3_b2", 3, dict(batch=2, n_kv_heads=2, ctx=1000), [1000]),
    ("u3_chunks", 3, dict(batch=2, n_kv_heads=2, ctx=333), [7, 100, 226]),
    ("nuq_4heads", 4, dict(n_kv_heads=4, ctx=700), [700]),
    ("nuq_32heads_chunks", 4, dict(ctx=300), [100, 1, 199]),
    ("serving_small", 5, dict(batch=3, n_kv_heads=2, ctx=1000), [900] + [1] * 100),
    ("serving_group_edge", 5, dict(batch=2, n_kv_heads=2, ctx=384), [127, 1, 128, 128]),
]


def _run(name, cfg_id, over, chunks, decode_path="auto", decode_splits=0, max_extra=37):
    print(f"[parity] case={name} cfg={cfg_id} over={over} path={decode_path}", flush=True)
    w = make_workload(cfg_id, **over)
    inputs = make_inputs(w, "cpu")
    n = w.ctx
    assert sum(chunks) == n
    max_ctx = n + max_extra
    cache = gpu_cache(w, inputs, chunks, max_ctx, decode_splits=decode_splits,
                      decode_path=decode_path)
    exp, kdeq, vdeq = oracle_encode(w, inputs, n, max_ctx)
    return w, inputs, cache, exp, kdeq, vdeq


@pytest.mark.parametrize("name,cfg_id,over,chunks", CASES, ids=[c[0] for c in CASES])
def test_encode_bytes_and_attention(name, cfg_id, over, chunks):
    w, inputs, cache, exp, kdeq, vdeq = _run(name, cfg_id, over, chunks)
    bad = compare_regions(cache, exp)
    assert not bad, "\n".join(bad)
    q = inputs["q"]
    out = cache.decode(q.cuda()).cpu().numpy()
    ref = oracle_attention(w, q, kdeq, vdeq, w.ctx)
    ma, rel = attention_errors(out, ref)
    print(f"[parity] {name}: max_abs={ma:.3e} rel_l2={rel:.3e}", flush=True)
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)


@pytest.mark.parametrize("name,cfg_id,over,chunks", [c for c in CASES if c[1] in (1, 2, 3, 5)],
                         ids=[c[0] for c in CASES if c[1] in (1, 2, 3, 5)])
def test_both_decode_kernels_agree_with_oracle(name, cfg_id, over, chunks):
    w, inputs, cache, exp, kdeq, vdeq = _run(name, cfg_id, over, chunks, decode_path="valu")
    q = inputs["q"]
    ref = oracle_attention(w, q, kdeq, vdeq, w.ctx)
    out_valu = cache.decode(q.cuda()).cpu().numpy()
    ma, rel = attention_errors(out_valu, ref)
    assert ma <= MAX_ABS and rel <= REL_L2, ("valu", ma, rel)


# lookup-table kernel (codebook keys and values, one query head per KV head):
# (name, workload overrides of config 4, append chunks, decode_splits)
LUT_CASES = [
    ("lut_nuq_4heads", dict(n_kv_heads=4, ctx=700), [700], 0),
    ("lut_nuq_32heads_chunks", dict(ctx=300), [100, 1, 199], 0),
    # 41 outliers per token over 47 chunks of 32 tokens, about 41 entries of
    # each head per chunk
    ("lut_32heads_multichunk", dict(ctx=1500), [1500], 0),
    # one range of 129 chunks: the query rotation is evaluated exactly at
    # chunks 32, 64, 96 and 128, and the last chunk holds a single token
    ("lut_one_range_resync", dict(n_kv_heads=4, ctx=4097), [4097], 1),
    # 6 KV heads with outliers and RoPE: the two empty waves of the second
    # group list no entries
    ("lut_6heads_outliers_rope", dict(n_kv_heads=6, ctx=400), [400], 2),
    # lists longer than a wave: 13 outliers per token over 2 heads (about
    # 200 entries of a head per chunk, taken 64 at a time)
    ("lut_long_outlier_lists", dict(n_kv_heads=2, ctx=500, k=dict(outlier_frac=0.05),
                                    v=dict(outlier_frac=0.05)), [500], 2),
    # one head, a quarter of its values outliers: 1024 entries per chunk
    ("lut_one_head_quarter_outliers", dict(n_kv_heads=1, ctx=300, k=dict(outlier_frac=0.25),
                                           v=dict(outlier_frac=0.25)), [250, 50], 0),
    # 6 KV heads: the second group of 4 has two empty waves
    ("lut_no_outliers_no_rope", dict(n_kv_heads=6, ctx=333, rope=False,
                                     k=dict(outlier_frac=0.0), v=dict(outlier_frac=0.0)), [333], 0),
    ("lut_key_outliers_only", dict(n_kv_heads=4, ctx=200, v=dict(outlier_frac=0.0)), [200], 0),
    ("lut_value_outliers_rope", dict(n_kv_heads=4, ctx=260, k=dict(outlier_frac=0.0)), [260], 0),
    ("lut_bf16_batch2", dict(batch=2, n_kv_heads=4, ctx=500, kv_dtype="bf16"), [500], 3),
]


@pytest.mark.parametrize("name,over,chunks,splits", LUT_CASES, ids=[c[0] for c in LUT_CASES])
def test_lookup_table_kernel(name, over, chunks, splits):
    w, inputs, cache, exp, kdeq, vdeq = _run(name, 4, over, chunks, decode_path="lut",
                                             decode_splits=splits)
    bad = compare_regions(cache, exp)
    assert not bad, "\n".join(bad)
    q = inputs["q"]
    out = cache.decode(q.cuda()).cpu().numpy()
    ref = oracle_attention(w, q, kdeq, vdeq, w.ctx)
    ma, rel = attention_errors(out, ref)
    print(f"[parity] {name}: max_abs={ma:.3e} rel_l2={rel:.3e}", flush=True)
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)


def test_codebook_on_the_general_kernel():
    w, inputs, cache, exp, kdeq, vdeq = _run("nuq_valu", 4, dict(n_kv_heads=4, ctx=700), [700],
                                             decode_path="valu")
    q = inputs["q"]
    out = cache.decode(q.cuda()).cpu().numpy()
    ref = oracle_attention(w, q, kdeq, vdeq, w.ctx)
    ma, rel = attention_errors(out, ref)
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)


@pytest.mark.parametrize("splits", [1, 2, 7])
def test_split_count_invariance(splits):
    w, inputs, cache, exp, kdeq, vdeq = _run(f"splits{splits}", 5,
                                             dict(batch=2, n_kv_heads=2, ctx=2000), [2000],
                                             decode_splits=splits)
    q = inputs["q"]
    out = cache.decode(q.cuda()).cpu().numpy()
    ref = oracle_attention(w, q, kdeq, vdeq, w.ctx)
    ma, rel = attention_errors(out, ref)
    assert ma <= MAX_ABS and rel <= REL_L2, (splits, ma, rel)


def test_rope_explicit_query_position():
    w, inputs, cache, exp, kdeq, vdeq = _run("nuq_qpos", 4, dict(n_kv_heads=2, ctx=257), [257])
    q = inputs["q"]
    q_pos = np.array([1000], dtype=np.int32)
    out = cache.decode(q.cuda(), q_pos=torch.from_numpy(q_pos).cuda()).cpu().numpy()
    ref = oracle_attention(w, q, kdeq, vdeq, w.ctx, q_pos=q_pos)
    ma, rel = attention_errors(out, ref)
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)


@pytest.mark.parametrize("odt,tdt", [("f16", torch.float16), ("bf16", torch.bfloat16)])
def test_half_outputs_are_rounded_f32_outputs(odt, tdt):
    w, inputs, cache, exp, kdeq, vdeq = _run("tiny_out", 1, {}, [512])
    q = inputs["q"].cuda()
    o32 = cache.decode(q)
    oh = cache.decode(q, out_dtype=odt)
    assert oh.dtype == tdt
    assert torch.equal(oh, o32.to(tdt))


def test_repeated_decode_is_deterministic():
    w, inputs, cache, exp, kdeq, vdeq = _run("repeat", 2, dict(ctx=4096), [4096])
    q = inputs["q"].cuda()
    a = cache.decode(q)
    for _ in range(3):
        b = cache.decode(q)
    assert torch.equal(a, b)


def test_bf16_raw_cache_matches_oracle():
    none = {"quantizer": "none", "bits": 16}
    w, inputs, cache, exp, kdeq, vdeq = _run("raw_bf16", 3, dict(batch=1, n_kv_heads=2, ctx=300,
                                                                 k=none, v=none), [300])
    q = inputs["q"]
    out = cache.decode(q.cuda()).cpu().numpy()
    ref = oracle_attention(w, q, kdeq, vdeq, w.ctx)
    ma, rel = attention_errors(out, ref)
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)


def test_decode_events_bracket_the_streaming_kernel():
    """kvq_set_decode_events: the recorded interval lies inside the decode
    call and the output is the same as without the events."""
    from quantized_kv_cache_04_amd import kvq as K
    w, inputs, cache, exp, kdeq, vdeq = _run("events", 5, dict(batch=2, n_kv_heads=2, ctx=4000),
                                             [4000])
    q = inputs["q"].cuda()
    ref = cache.decode(q)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    s = torch.cuda.current_stream()
    for e in ev:
        e.record(s)
    ev[0].record(s)
    K.set_decode_events(ev[1], ev[2])
    out = cache.decode(q)
    ev[3].record(s)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    k_ms, call_ms = ev[1].elapsed_time(ev[2]), ev[0].elapsed_time(ev[3])
    assert 0.0 < k_ms <= call_ms, (k_ms, call_ms)


# Per-channel key groups of 1, 3 and 8 blocks on the matrix-core kernel: the
# waves of a workgroup take a split's blocks one key group at a time and the
# host starts every split on a group boundary.  Splits are chosen so that
# some waves get no group, some get a partial one, and the unquantized tail
# is shared out over the waves; one-token appends cross group boundaries.
# (name, key group size, context, append chunks, decode_splits)
KCH_CASES = [
    ("kch_g32_splits3", 32, 700, [300, 1, 1, 398], 3),
    ("kch_g96_splits5", 96, 1000, [500] + [1] * 97 + [403], 5),
    ("kch_g256_splits2", 256, 2100, [2000] + [1] * 100, 2),
    ("kch_g256_one_group", 256, 300, [300], 0),
    ("kch_g128_splits9", 128, 3000, [2999, 1], 9),
]


@pytest.mark.parametrize("name,G,ctx,chunks,splits", KCH_CASES, ids=[c[0] for c in KCH_CASES])
def test_per_channel_key_groups_on_matrix_cores(name, G, ctx, chunks, splits):
    w, inputs, cache, exp, kdeq, vdeq = _run(name, 5, dict(batch=2, n_kv_heads=2, ctx=ctx,
                                                           k=dict(group_size=G)),
                                             chunks, decode_path="mfma", decode_splits=splits)
    bad = compare_regions(cache, exp)
    assert not bad, "\n".join(bad)
    q = inputs["q"]
    out = cache.decode(q.cuda()).cpu().numpy()
    ref = oracle_attention(w, q, kdeq, vdeq, w.ctx)
    ma, rel = attention_errors(out, ref)
    print(f"[parity] {name}: max_abs={ma:.3e} rel_l2={rel:.3e}", flush=True)
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)


# Many splits: the merge kernel folds the partial states sixteen at a time,
# so well over a hundred splits take it through many rounds; the long
# context also gives every wave many key groups (its LDS parameter ring is
# refilled).  (name, config, workload overrides, decode_splits)
MANY_SPLIT_CASES = [
    ("serving_171_splits", 5, dict(batch=1, n_kv_heads=1, ctx=65536), 250),
    ("u3_70_splits", 3, dict(batch=1, n_kv_heads=1, ctx=20000), 200),
]


@pytest.mark.parametrize("name,cfg_id,over,splits", MANY_SPLIT_CASES,
                         ids=[c[0] for c in MANY_SPLIT_CASES])
def test_many_splits(name, cfg_id, over, splits):
    w, inputs, cache, exp, kdeq, vdeq = _run(name, cfg_id, over, [over["ctx"]],
                                             decode_splits=splits)
    q = inputs["q"]
    out = cache.decode(q.cuda()).cpu().numpy()
    ref = oracle_attention(w, q, kdeq, vdeq, w.ctx)
    ma, rel = attention_errors(out, ref)
    print(f"[parity] {name}: max_abs={ma:.3e} rel_l2={rel:.3e}", flush=True)
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)


# Degenerate groups: constant values make a group's range zero (scale 0,
# every code 0, dequantized value = the zero point), all-zero rows make
# q8_0's absmax zero, and equal magnitudes make every outlier a tie (the
# lower flat index wins).  Bytes and attention must still match the oracle.
@pytest.mark.parametrize("path", ["auto", "valu"])
@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_degenerate_groups(cfg_id, path):
    over = dict(batch=1, n_kv_heads=2, ctx=300)
    w = make_workload(cfg_id, **over)
    inputs = make_inputs(w, "cpu")
    k, v = inputs["k"].clone(), inputs["v"].clone()
    v[:, :64] = 1.5                 # per-token value groups of constant rows
    v[:, 64:96] = 0.0               # all-zero rows
    k[:, :, :, :32] = -0.25         # channels constant over every token
    k[:, 100:140] = 0.0             # all-zero key rows (a per-channel group mixes them)
    k[:, 200:230] = 2.0             # equal magnitudes in whole rows
    inputs = dict(inputs, k=k, v=v)
    n = w.ctx
    chunks = [150, 1, 149]
    print(f"[parity] case=degenerate cfg={cfg_id} path={path}", flush=True)
    cache = gpu_cache(w, inputs, chunks, n + 37, decode_path=path)
    exp, kdeq, vdeq = oracle_encode(w, inputs, n, n + 37)
    bad = compare_regions(cache, exp)
    assert not bad, "\n".join(bad)
    q = inputs["q"]
    out = cache.decode(q.cuda()).cpu().numpy()
    ref = oracle_attention(w, q, kdeq, vdeq, n)
    ma, rel = attention_errors(out, ref)
    print(f"[parity] degenerate cfg{cfg_id} {path}: max_abs={ma:.3e} rel_l2={rel:.3e}", flush=True)
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)
