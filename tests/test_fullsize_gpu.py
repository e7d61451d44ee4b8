"""GPU parity at the workloads' full sizes, in the launch configuration that
bench.py times: the whole context appended in one call, the library's own
split count and decode kernel.

The oracle cannot attend over a whole 16 x 65536-token batch in seconds, so
the check samples outputs: every query head of a few (sequence, KV head)
slices.  Per-token and per-channel groups never cross slices, so the oracle
encodes each sampled slice on its own; its encoded bytes must match the
slice's bytes in the GPU cache exactly.  The codebook workload chooses its
outliers per token across all heads, so there the oracle finds them over all
heads (outlier_mask, in chunks of tokens) and checks the CSR rows of a
sample of tokens.
"""
import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import layout as olay
from oracle import quant as oq
from synth import make_workload
from synth.workloads import make_inputs

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

from quantized_kv_cache_04_amd import kvq  # noqa: E402
from parity import MAX_ABS, REL_L2, _as_bytes, attention_errors, to_np32  # noqa: E402

# (config, context or None for the config's own, sampled (sequence, KV head) slices)
FULL = [
    (1, None, [(0, 0), (0, 1)]),
    (2, 4096, [(0, 1)]),
    (2, 8192, [(0, 0)]),
    (2, 16384, [(0, 0), (0, 1)]),
    (3, None, [(0, 0), (3, 7)]),
    (5, None, [(0, 0), (9, 3), (15, 7)]),
]


def _full_cache(w, max_extra=0):
    inputs = make_inputs(w, "cuda")
    cfg = kvq.config_from_workload(w, max_ctx=w.ctx + max_extra)
    cache = kvq.Cache(cfg, device="cuda", k_codebook=inputs["k_codebook"],
                      v_codebook=inputs["v_codebook"], k_scale=inputs["k_scale"],
                      v_scale=inputs["v_scale"])
    cache.append(inputs["k"], inputs["v"])
    out = cache.decode(inputs["q"])
    torch.cuda.synchronize()
    return inputs, cache, out


def _slice_bytes(cache, w, name, reg, b, h):
    return cache.region(name, reg).view(w.batch, w.n_kv_heads, -1)[b, h].cpu().numpy()


@pytest.mark.parametrize("cfg_id,ctx,slices", FULL,
                         ids=[f"cfg{c}_t{t or 'full'}" for c, t, _ in FULL])
def test_full_size_sampled_slices(cfg_id, ctx, slices):
    w = make_workload(cfg_id, ctx=ctx)
    print(f"[fullsize] cfg={cfg_id} B={w.batch} Hkv={w.n_kv_heads} T={w.ctx} "
          f"path={kvq.decode_path(kvq.config_from_workload(w))}", flush=True)
    extra = 518 if cfg_id == 5 else 0   # bench.py default serving headroom: 5 + 2 x 256 + 1
    inputs, cache, out = _full_cache(w, extra)
    g = w.gqa
    for b, h in slices:
        enc = {}
        for name, fmt in (("k", w.k), ("v", w.v)):
            x = to_np32(inputs[name][b:b + 1, :, h:h + 1, :])
            enc[name] = oq.encode_tensor(x, fmt, None)
            exp = olay.expected_regions(fmt, enc[name], batch=1, n_kv_heads=1, n_ctx=w.ctx,
                                        max_ctx=w.ctx + extra, kv_dtype=w.kv_dtype,
                                        is_key=(name == "k"))
            for reg, arr in exp.items():
                got = _slice_bytes(cache, w, name, reg, b, h)
                want = _as_bytes(arr)
                diff = np.nonzero(got != want)[0]
                assert got.shape == want.shape and diff.size == 0, \
                    f"{name}.{reg} of slice ({b}, {h}): {diff.size} bytes differ"
        q = to_np32(inputs["q"][b:b + 1, h * g:(h + 1) * g])
        ref = oatt.decode_attention(q, enc["k"]["deq"], enc["v"]["deq"], n_ctx=w.ctx,
                                    rope=w.rope, rope_base=w.rope_base)
        got = out[b:b + 1, h * g:(h + 1) * g].cpu().numpy()
        ma, rel = attention_errors(got, ref)
        print(f"[fullsize] cfg={cfg_id} slice=({b},{h}) max_abs={ma:.2e} rel_l2={rel:.2e}",
              flush=True)
        assert ma <= MAX_ABS and rel <= REL_L2, (b, h, ma, rel)


def test_full_size_serving_steps():
    """The step bench.py times, at the serving workload's full size: a cache
    of 65,535 tokens, then two kvq_append_decode steps -- the first closes a
    per-channel key group (append, then decode), the second fuses.  Sampled
    slices' bytes and the second step's attention against the oracle."""
    w = make_workload(5, ctx=65537)
    print(f"[fullsize] serving steps B={w.batch} Hkv={w.n_kv_heads} T={w.ctx}", flush=True)
    extra = 7
    inputs = make_inputs(w, "cuda")
    cfg = kvq.config_from_workload(w, max_ctx=w.ctx + extra)
    cache = kvq.Cache(cfg, device="cuda")
    n0 = w.ctx - 2
    cache.append(inputs["k"][:, :n0].contiguous(), inputs["v"][:, :n0].contiguous())
    assert [kvq.append_decode_fused(cfg, n) for n in (n0, n0 + 1)] == [False, True]
    for t in (n0, n0 + 1):
        out = cache.append_decode(inputs["k"][:, t:t + 1].contiguous(),
                                  inputs["v"][:, t:t + 1].contiguous(), inputs["q"])
    torch.cuda.synchronize()
    assert cache.n_ctx == w.ctx
    g = w.gqa
    for b, h in [(0, 0), (9, 3), (15, 7)]:
        enc = {}
        for name, fmt in (("k", w.k), ("v", w.v)):
            x = to_np32(inputs[name][b:b + 1, :, h:h + 1, :])
            enc[name] = oq.encode_tensor(x, fmt, None)
            exp = olay.expected_regions(fmt, enc[name], batch=1, n_kv_heads=1, n_ctx=w.ctx,
                                        max_ctx=w.ctx + extra, kv_dtype=w.kv_dtype,
                                        is_key=(name == "k"))
            for reg, arr in exp.items():
                got = _slice_bytes(cache, w, name, reg, b, h)
                want = _as_bytes(arr)
                diff = np.nonzero(got != want)[0]
                assert got.shape == want.shape and diff.size == 0, \
                    f"{name}.{reg} of slice ({b}, {h}): {diff.size} bytes differ"
        q = to_np32(inputs["q"][b:b + 1, h * g:(h + 1) * g])
        ref = oatt.decode_attention(q, enc["k"]["deq"], enc["v"]["deq"], n_ctx=w.ctx)
        got = out[b:b + 1, h * g:(h + 1) * g].cpu().numpy()
        ma, rel = attention_errors(got, ref)
        print(f"[fullsize] serving step slice=({b},{h}) max_abs={ma:.2e} rel_l2={rel:.2e}",
              flush=True)
        assert ma <= MAX_ABS and rel <= REL_L2, (b, h, ma, rel)


def test_full_size_codebook_workload():
    """KVQuant-shaped layer: 32 heads, 131072 tokens, codebooks, 1% outliers, RoPE."""
    w = make_workload(4)
    print(f"[fullsize] cfg=4 T={w.ctx} path={kvq.decode_path(kvq.config_from_workload(w))}",
          flush=True)
    inputs, cache, out = _full_cache(w)
    heads = [0, 17]
    H, d, T = w.n_kv_heads, w.head_dim, w.ctx
    deq = {}
    for name, fmt in (("k", w.k), ("v", w.v)):
        cb = inputs[f"{name}_codebook"].cpu().numpy()
        cbf = cb.astype(np.float64)
        k = oq.outlier_count(fmt["outlier_frac"], H * d)
        parts = []
        for t0 in range(0, T, 8192):
            x = to_np32(inputs[name][0, t0:t0 + 8192])               # [n, H, d] all heads
            mask = oq.outlier_mask(x.reshape(x.shape[0], H * d), k).reshape(x.shape)
            xs = x[:, heads, :]                                      # sampled heads
            codes = oq.codebook_codes(xs, cb[heads])                 # [n, 2, d]
            dense = cbf[np.array(heads)[None, :, None], np.arange(d)[None, None, :], codes]
            parts.append(np.where(mask[:, heads, :], oq.f16(xs).astype(np.float64), dense))
        deq[name] = np.transpose(np.concatenate(parts, axis=0), (1, 0, 2))[None]   # [1, 2, T, d]
        # CSR rows of sampled tokens, whole rows (all heads)
        toks = [0, 1, T // 2, T - 1]
        x = to_np32(inputs[name][0, toks]).reshape(len(toks), H * d)
        enc = oq.encode_tensor(x.reshape(1, len(toks), H, d), fmt, cb)
        dense_at = enc["codes"][0].transpose(1, 0, 2).reshape(len(toks), H * d)
        cols = enc["cols"][0]
        want_col = (cols | (np.take_along_axis(dense_at, cols, axis=1) << 12)).astype(np.uint16)
        want_val = oq.f16(enc["vals"][0])
        col_r = cache.region(name, "col").view(torch.int16)
        val_r = cache.region(name, "val").view(torch.int16)
        for i, t in enumerate(toks):
            got_c = col_r[t * k:(t + 1) * k].cpu().numpy().view(np.uint16)
            got_v = val_r[t * k:(t + 1) * k].cpu().numpy().view(np.float16)
            assert np.array_equal(got_c, want_col[i]), (name, t)
            assert np.array_equal(got_v, want_val[i]), (name, t)
        print(f"[fullsize] cfg=4 {name}: oracle slices and CSR rows done", flush=True)
    q = to_np32(inputs["q"][0:1, heads])
    ref = oatt.decode_attention(q, deq["k"], deq["v"], n_ctx=T, rope=True, rope_base=w.rope_base)
    got = out[0:1, heads].cpu().numpy()
    ma, rel = attention_errors(got, ref)
    print(f"[fullsize] cfg=4 heads={heads} max_abs={ma:.2e} rel_l2={rel:.2e}", flush=True)
    assert ma <= MAX_ABS and rel <= REL_L2, (ma, rel)


FP8 = dict(quantizer="fp8_e5m2", bits=8, group_size=0, layout="per_token", outlier_frac=0.0)


def test_full_size_fp8_serving():
    """The serving shape (16 x 65536 tokens, 8 KV heads, g = 4) stored as FP8
    E5M2 with per-head scales, in bench.py's launch configuration (the
    matrix-core kernel, 518 tokens of serving headroom)."""
    w = make_workload(5, k=FP8, v=FP8)
    extra = 518
    print(f"[fullsize] fp8 serving T={w.ctx} path={kvq.decode_path(kvq.config_from_workload(w))}",
          flush=True)
    inputs, cache, out = _full_cache(w, extra)
    g = w.gqa
    for b, h in [(0, 0), (7, 5), (15, 7)]:
        enc = {}
        for name in ("k", "v"):
            x = to_np32(inputs[name][b:b + 1, :, h:h + 1, :])
            sc = inputs[f"{name}_scale"][h:h + 1].cpu().numpy()
            enc[name] = oq.encode_tensor(x, FP8, None, sc)
            exp = olay.expected_regions(FP8, enc[name], batch=1, n_kv_heads=1, n_ctx=w.ctx,
                                        max_ctx=w.ctx + extra, kv_dtype=w.kv_dtype,
                                        is_key=(name == "k"))
            got = _slice_bytes(cache, w, name, "codes", b, h)
            assert np.array_equal(got, _as_bytes(exp["codes"])), (name, b, h)
        q = to_np32(inputs["q"][b:b + 1, h * g:(h + 1) * g])
        ref = oatt.decode_attention(q, enc["k"]["deq"], enc["v"]["deq"], n_ctx=w.ctx)
        ma, rel = attention_errors(out[b:b + 1, h * g:(h + 1) * g].cpu().numpy(), ref)
        print(f"[fullsize] fp8 slice=({b},{h}) max_abs={ma:.2e} rel_l2={rel:.2e}", flush=True)
        assert ma <= MAX_ABS and rel <= REL_L2, (b, h, ma, rel)


def test_full_size_chunked_prefill():
    """bench.py --prefill 512: the serving workload's last 512 tokens appended
    as a chunk to 65,024 cached tokens, then causal attention for the chunk's
    queries; sampled rows of sampled slices against the oracle's decode
    definition at each row's position."""
    from synth import make_prefill_queries
    w = make_workload(5)
    N, T = 512, w.ctx
    inputs = make_inputs(w, "cuda")
    cfg = kvq.config_from_workload(w, max_ctx=T)
    cache = kvq.Cache(cfg, device="cuda")
    cache.append(inputs["k"][:, :T - N].contiguous(), inputs["v"][:, :T - N].contiguous())
    cache.append(inputs["k"][:, T - N:].contiguous(), inputs["v"][:, T - N:].contiguous())
    q = make_prefill_queries(w, N, "cuda")
    out = cache.prefill(q)
    torch.cuda.synchronize()
    g = w.gqa
    for b, h in [(0, 0), (11, 6)]:
        deq = {}
        for name, fmt in (("k", w.k), ("v", w.v)):
            x = to_np32(inputs[name][b:b + 1, :, h:h + 1, :])
            deq[name] = oq.encode_tensor(x, fmt, None)["deq"]
        for i in (0, 1, 255, N - 1):
            p = T - N + i
            qi = to_np32(q[b:b + 1, i, h * g:(h + 1) * g])
            ref = oatt.decode_attention(qi, deq["k"], deq["v"], n_ctx=p + 1, q_pos=np.array([p]))
            got = out[b:b + 1, i, h * g:(h + 1) * g].cpu().numpy()
            ma, rel = attention_errors(got, ref)
            print(f"[fullsize] prefill slice=({b},{h}) row={i} max_abs={ma:.2e} rel_l2={rel:.2e}",
                  flush=True)
            assert ma <= MAX_ABS and rel <= REL_L2, (b, h, i, ma, rel)
