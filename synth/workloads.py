"""The five synthetic decode workloads and their seeded input generators.

Shapes and value distributions follow the workloads the pages measure:
a tiny 4-bit correctness case, llama.cpp's q8_0 cache at 4K/8K/16K
(TurboQuant NIAH page, section 1.2), a Llama-2-70B-shaped layer with the
3-bit TurboQuant scheme (TurboQuant page, sections 2.1 and 3.1), a
LLaMA-7B-shaped KVQuant layer at 128K (KVQuant page, section 2.2) and an
8B-shaped serving batch.  No public dataset is used: the pages' corpora are
stood in for by seeded normal draws with the outlier structure each workload
names.

Every array is drawn in float32 from its own seeded ``torch.Generator``
stream, then rounded once to the cache dtype.  The same bytes are handed to
the HIP library and to the CPU oracle.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Any, Dict, Optional

import torch

BASE_SEED = 20261202


def _fmt(quantizer: str, bits: int, group_size: int = 0, layout: str = "per_token",
         outlier_frac: float = 0.0) -> Dict[str, Any]:
    return {"quantizer": quantizer, "bits": bits, "group_size": group_size,
            "layout": layout, "outlier_frac": outlier_frac}


# name -> description.  ``ctx`` is the context length of the workload (config 2
# lists three).  ``values`` names the recipe used by ``make_inputs``.
CONFIGS: Dict[int, Dict[str, Any]] = {
    1: dict(name="tiny_u4", batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128, ctx=512,
            kv_dtype="f16", rope=False, rope_base=10000.0,
            k=_fmt("asym_minmax", 4, 64, "per_channel"),
            v=_fmt("asym_minmax", 4, 32, "per_token"),
            values=dict(kind="outlier_channels", channels=(5, 77), scale=20.0)),
    2: dict(name="q8_0_gqa8", batch=1, n_q_heads=16, n_kv_heads=2, head_dim=128,
            ctx=(4096, 8192, 16384),
            kv_dtype="f16", rope=False, rope_base=10000.0,
            k=_fmt("sym_q8_0", 8, 32, "per_token"),
            v=_fmt("sym_q8_0", 8, 32, "per_token"),
            values=dict(kind="clipped_normal", sigma=1.5, clip=6.0)),
    3: dict(name="u3_70b_layer", batch=4, n_q_heads=64, n_kv_heads=8, head_dim=128, ctx=32768,
            kv_dtype="bf16", rope=False, rope_base=10000.0,
            k=_fmt("asym_absmax_offset", 3, 64, "per_token"),
            v=_fmt("asym_absmax_offset", 3, 64, "per_token"),
            values=dict(kind="bernoulli_outliers", p=0.005, scale=15.0)),
    4: dict(name="kvquant_nuq_7b_128k", batch=1, n_q_heads=32, n_kv_heads=32, head_dim=128,
            ctx=131072, kv_dtype="f16", rope=True, rope_base=10000.0,
            k=_fmt("codebook", 4, 0, "per_token", 0.01),
            v=_fmt("codebook", 4, 0, "per_token", 0.01),
            values=dict(kind="normal")),
    5: dict(name="serving_u4_8b_b16", batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128,
            ctx=65536, kv_dtype="f16", rope=False, rope_base=10000.0,
            k=_fmt("asym_minmax", 4, 128, "per_channel"),
            v=_fmt("asym_minmax", 4, 128, "per_token"),
            values=dict(kind="outlier_channels", channels=(11, 42, 73, 104), scale=20.0)),
}

_STREAMS = {"k": 0, "v": 1, "q": 2, "mask": 3, "kcb": 4, "vcb": 5, "step_k": 6, "step_v": 7,
            "step_q": 8, "prefill_q": 9, "kscale": 10, "vscale": 11, "pages": 12}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One concrete instance of a workload: the config with sizes fixed."""
    cfg_id: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx: int
    kv_dtype: str
    rope: bool
    rope_base: float
    k: Dict[str, Any]
    v: Dict[str, Any]
    values: Dict[str, Any]
    seed: int = 0
    sink_tokens: int = 0    # attention-sink tokens kept raw (0 = none)

    @property
    def gqa(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float16 if self.kv_dtype == "f16" else torch.bfloat16


def config_for(cfg_id: int) -> Dict[str, Any]:
    return CONFIGS[cfg_id]


def make_workload(cfg_id: int, *, batch: Optional[int] = None, ctx: Optional[int] = None,
                  n_kv_heads: Optional[int] = None, gqa: Optional[int] = None,
                  seed: int = 0, **fmt_overrides: Any) -> Workload:
    """Fix the sizes of config ``cfg_id`` (defaults: the config's own sizes;
    config 2 defaults to its longest context).  ``k=``/``v=`` overrides patch
    the tensor formats."""
    c = CONFIGS[cfg_id]
    T = ctx if ctx is not None else (max(c["ctx"]) if isinstance(c["ctx"], tuple) else c["ctx"])
    hkv = n_kv_heads if n_kv_heads is not None else c["n_kv_heads"]
    g = gqa if gqa is not None else c["n_q_heads"] // c["n_kv_heads"]
    k = dict(c["k"])
    v = dict(c["v"])
    k.update(fmt_overrides.pop("k", {}))
    v.update(fmt_overrides.pop("v", {}))
    kw = dict(rope=c["rope"], rope_base=c["rope_base"], kv_dtype=c["kv_dtype"],
              values=c["values"])
    kw.update(fmt_overrides)
    return Workload(cfg_id=cfg_id, batch=batch if batch is not None else c["batch"],
                    n_q_heads=hkv * g, n_kv_heads=hkv, head_dim=c["head_dim"], ctx=T,
                    k=k, v=v, seed=seed, **kw)


def _gen(w: Workload, stream: str, device: str, extra: int = 0) -> torch.Generator:
    h = hashlib.sha256(f"{BASE_SEED}/{w.cfg_id}/{w.seed}/{_STREAMS[stream]}/{extra}".encode())
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h.digest()[:8], "little") & ((1 << 63) - 1))
    return g


def _values(w: Workload, shape, stream: str, device: str, extra: int = 0) -> torch.Tensor:
    """Draw one K or V array (float32) following the workload's value recipe."""
    rec = w.values
    g = _gen(w, stream, device, extra)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    kind = rec["kind"]
    if kind == "normal":
        pass
    elif kind == "outlier_channels":
        # fixed channels of every head carry values scaled up by ``scale``
        ch = torch.tensor(rec["channels"], device=device, dtype=torch.long)
        ch = ch[ch < shape[-1]]
        x[..., ch] *= rec["scale"]
    elif kind == "clipped_normal":
        x = (x * rec["sigma"]).clamp_(-rec["clip"], rec["clip"])
    elif kind == "bernoulli_outliers":
        gm = _gen(w, "mask", device, extra * 2 + (0 if stream.endswith("k") else 1))
        m = torch.rand(shape, generator=gm, device=device, dtype=torch.float32) < rec["p"]
        x = torch.where(m, x * rec["scale"], x)
    else:
        raise ValueError(f"unknown value recipe {kind}")
    return x


def _codebook(w: Workload, stream: str, device: str) -> torch.Tensor:
    """16 ascending fp16 centroids per (kv head, channel): the quantiles at
    (i + 0.5) / 16 of 4096 seeded N(0, 1) draws for that channel."""
    g = _gen(w, stream, device)
    n = 4096
    draws = torch.randn((w.n_kv_heads, w.head_dim, n), generator=g, device=device,
                        dtype=torch.float32)
    s = torch.sort(draws, dim=-1).values
    probs = (torch.arange(16, device=device, dtype=torch.float64) + 0.5) / 16.0
    pos = probs * (n - 1)
    lo = pos.floor().long()
    frac = (pos - lo.double()).float()
    hi = torch.clamp(lo + 1, max=n - 1)
    c = s[..., lo] * (1 - frac) + s[..., hi] * frac
    return torch.sort(c.half(), dim=-1).values.contiguous()


def _head_scales(w: Workload, stream: str, device: str) -> torch.Tensor:
    """float32 [Hkv] scales of an FP8 tensor: seeded log-uniform in [1/4, 4]
    (arbitrary, not powers of two, so that the division x / s rounds)."""
    g = _gen(w, stream, device)
    u = torch.rand((w.n_kv_heads,), generator=g, device=device, dtype=torch.float32)
    return torch.exp2(u * 4.0 - 2.0).contiguous()


def make_inputs(w: Workload, device: str = "cpu") -> Dict[str, Optional[torch.Tensor]]:
    """K and V of shape [B, T, Hkv, d] and q of shape [B, Hq, d] in the cache
    dtype, plus fp16 codebooks [Hkv, d, 16] for codebook formats."""
    B, T, H, d = w.batch, w.ctx, w.n_kv_heads, w.head_dim
    dt = w.torch_dtype
    k = _values(w, (B, T, H, d), "k", device).to(dt)
    v = _values(w, (B, T, H, d), "v", device).to(dt)
    q = torch.randn((B, w.n_q_heads, d), generator=_gen(w, "q", device), device=device,
                    dtype=torch.float32).to(dt)
    kcb = _codebook(w, "kcb", device) if w.k["quantizer"] == "codebook" else None
    vcb = _codebook(w, "vcb", device) if w.v["quantizer"] == "codebook" else None
    ksc = _head_scales(w, "kscale", device) if w.k["quantizer"] == "fp8_e5m2" else None
    vsc = _head_scales(w, "vscale", device) if w.v["quantizer"] == "fp8_e5m2" else None
    return {"k": k.contiguous(), "v": v.contiguous(), "q": q.contiguous(),
            "k_codebook": kcb, "v_codebook": vcb, "k_scale": ksc, "v_scale": vsc}


def make_step_tokens(w: Workload, step: int, n_new: int = 1, device: str = "cpu"):
    """New K/V rows [B, n_new, Hkv, d] and a new query for decode step ``step``
    of a serving run, drawn with the workload's recipe."""
    B, H, d = w.batch, w.n_kv_heads, w.head_dim
    dt = w.torch_dtype
    k = _values(w, (B, n_new, H, d), "step_k", device, extra=step).to(dt)
    v = _values(w, (B, n_new, H, d), "step_v", device, extra=step).to(dt)
    q = torch.randn((B, w.n_q_heads, d), generator=_gen(w, "step_q", device, step),
                    device=device, dtype=torch.float32).to(dt)
    return k.contiguous(), v.contiguous(), q.contiguous()


def make_prefill_queries(w: Workload, n_q: int, device: str = "cpu") -> torch.Tensor:
    """Queries [B, n_q, Hq, d] of the last n_q cached tokens for chunked
    prefill: N(0, 1) in the cache dtype, like the decode query."""
    q = torch.randn((w.batch, n_q, w.n_q_heads, w.head_dim), generator=_gen(w, "prefill_q", device),
                    device=device, dtype=torch.float32)
    return q.to(w.torch_dtype).contiguous()


def make_page_table(w: Workload, max_ctx: int, n_pages: int, device: str = "cpu") -> torch.Tensor:
    """Page table of a paged cache: int32 [B, ceil(max_ctx / 32)], a seeded
    shuffle of the physical pages [0, n_pages) dealt out to the sequences'
    logical pages, so that neighbouring logical pages land on scattered,
    non-contiguous physical pages (with unused pages in between when
    n_pages exceeds what the sequences need)."""
    per_seq = (max_ctx + 31) // 32
    if n_pages < w.batch * per_seq:
        raise ValueError(f"{n_pages} pages cannot hold {w.batch} x {per_seq}")
    g = _gen(w, "pages", "cpu")
    perm = torch.randperm(n_pages, generator=g)
    return perm[:w.batch * per_seq].reshape(w.batch, per_seq).to(torch.int32).to(device)
