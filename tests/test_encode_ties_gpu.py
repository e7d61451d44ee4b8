"""GPU pins of the encoders' rounding on inputs whose quotients (x - zero) /
scale fall exactly on half-integers, where round-half-even decides the code.

Every value is a multiple of 2^k / 2: each group's minimum is 0 and its
maximum qmax * 2^k (symmetric q8_0: 127 * 2^k at the largest magnitude), so
the group's fp16 scale is exactly 2^k and about half of the quotients are
ties.  The others are whole numbers.  Min and max sit where (t + c) mod 32
is 0 and 1, so every per-token group of channels and every per-channel
group of tokens holds both.  The packed bytes of every encoder (key rows,
value tiles, per-channel key groups, the serving step's own encode) must
match the oracle's byte for byte.
"""
import numpy as np
import pytest
import torch

from synth import make_inputs, make_workload

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

from parity import compare_regions, gpu_cache, oracle_encode  # noqa: E402

K_EXP = -2   # scale 2^-2


def _ties(shape, qmax, symmetric, seed):
    """[B, T, H, 128] fp16 values on the half-integer grid of scale 2^K_EXP."""
    B, T, H, D = shape
    rng = np.random.default_rng(seed)
    s = 2.0 ** K_EXP
    if symmetric:
        j = rng.integers(-qmax, qmax, size=shape)                 # j + 0.5 in (-qmax, qmax)
        top = qmax * s
    else:
        j = rng.integers(0, qmax, size=shape)
        top = qmax * s
    half = rng.random(size=shape) < 0.5
    x = (j + np.where(half, 0.5, 0.0)) * s
    pos = (np.arange(T)[None, :, None, None] + np.arange(D)[None, None, None, :]) % 32
    x = np.where(pos == 0, -top if symmetric else 0.0, x)
    x = np.where(pos == 1, top, x)
    return torch.from_numpy(x.astype(np.float16))


U4_TOK = dict(quantizer="asym_minmax", bits=4, group_size=32, layout="per_token", outlier_frac=0.0)
U4_CH = dict(quantizer="asym_minmax", bits=4, group_size=64, layout="per_channel", outlier_frac=0.0)
U3_TOK = dict(quantizer="asym_minmax", bits=3, group_size=64, layout="per_token", outlier_frac=0.0)
Q8 = dict(quantizer="sym_q8_0", bits=8, group_size=32, layout="per_token", outlier_frac=0.0)

# (name, config, k format, v format, qmax of the grid, symmetric, chunks)
CASES = [
    ("u4_channel_keys_token_values", 5, U4_CH, U4_TOK, 15, False, [200, 1, 55]),
    ("u3_rows_and_tiles", 3, U3_TOK, U3_TOK, 7, False, [129, 127]),
    ("q8_0", 2, Q8, Q8, 127, True, [256]),
]


@pytest.mark.parametrize("name,cfg_id,kf,vf,qmax,sym,chunks", CASES, ids=[c[0] for c in CASES])
def test_half_integer_quotients(name, cfg_id, kf, vf, qmax, sym, chunks):
    print(f"[ties] case={name}", flush=True)
    T = sum(chunks)
    w = make_workload(cfg_id, batch=2, n_kv_heads=2, ctx=T, k=kf, v=vf, kv_dtype="f16")
    inputs = make_inputs(w, "cpu")
    shape = (w.batch, T, w.n_kv_heads, w.head_dim)
    inputs["k"] = _ties(shape, qmax, sym, 1)
    inputs["v"] = _ties(shape, qmax, sym, 2)
    max_ctx = T + 5
    cache = gpu_cache(w, inputs, chunks, max_ctx)
    exp, _, _ = oracle_encode(w, inputs, T, max_ctx)
    bad = compare_regions(cache, exp)
    assert not bad, "\n".join(bad)


def test_half_integer_quotients_in_the_serving_step():
    """The one-token step encodes its token in the merge launch."""
    T = 100
    w = make_workload(5, batch=2, n_kv_heads=2, ctx=T, k=U4_CH, v=U4_TOK)
    inputs = make_inputs(w, "cpu")
    shape = (w.batch, T, w.n_kv_heads, w.head_dim)
    inputs["k"] = _ties(shape, 15, False, 3)
    inputs["v"] = _ties(shape, 15, False, 4)
    cache = gpu_cache(w, inputs, [60], T + 5)
    kd, vd, q = inputs["k"].cuda(), inputs["v"].cuda(), inputs["q"].cuda()
    for t in range(60, T):
        cache.append_decode(kd[:, t:t + 1].contiguous(), vd[:, t:t + 1].contiguous(), q)
    exp, _, _ = oracle_encode(w, inputs, T, T + 5)
    bad = compare_regions(cache, exp)
    assert not bad, "\n".join(bad)
