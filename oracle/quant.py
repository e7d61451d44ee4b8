"""Quantizers of the oracle (float32 encode, round-half-even, float64 decode).

Test infrastructure: see the package docstring.

Common rules (readings where the pages are silent):

* Inputs are fp16 or bf16 and enter as their exact float32 values.
* ``f16(.)`` rounds float32 to fp16 to nearest-even; scales and zero points
  are rounded to fp16 *before* codes are computed, so the stored parameters
  reproduce the dequantized values.
* ``rint`` is round-half-even, the rounding of the TurboQuant page's Python
  ``round`` (section 3.1).
* Each step is one IEEE float32 operation: ``(x - z)`` then ``/ s``, never a
  multiply by a reciprocal, never a fused multiply-add.
* A degenerate group whose fp16 scale is 0 gets code 0 everywhere, so it
  dequantizes to its zero point.
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

F32 = np.float32


def f16(x: np.ndarray) -> np.ndarray:
    """Round float32 to fp16, nearest-even."""
    return np.asarray(x, dtype=F32).astype(np.float16)


def _div_codes(num: np.ndarray, s16: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """code = clamp(rint(num / s), lo, hi) in float32, 0 where s == 0."""
    s32 = s16.astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = num / s32
    r = np.rint(qf)
    r = np.where(s32 == 0, F32(0), r)
    r = np.clip(r, lo, hi)
    return r.astype(np.int32)


def asym_minmax(x: np.ndarray, bits: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Group-wise asymmetric min/max quantization over the last axis.

    Each group gets its own range and scale (Survey page, section 2.4: a
    scale and a zero point per group; Memory-killer page, section 2.3: every
    group measures its own value range).  scale = f16((max - min) / (2^b - 1)),
    zero = f16(min), code = clamp(rint((x - zero) / scale), 0, 2^b - 1).
    Returns (codes int32, scale fp16, zero fp16); parameters drop the last axis.
    """
    x = np.asarray(x, dtype=F32)
    lo = x.min(axis=-1)
    hi = x.max(axis=-1)
    qmax = F32(2 ** bits - 1)
    s = f16((hi - lo) / qmax)
    z = f16(lo)
    codes = _div_codes(x - z.astype(F32)[..., None], s[..., None], 0, 2 ** bits - 1)
    return codes, s, z


def asym_absmax_offset(x: np.ndarray, bits: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """TurboQuant's dynamic asymmetric quantizer (TurboQuant page, section 3.1),
    with fixed non-overlapping groups in place of sliding windows:
    scale = f16(max|x| / (2^(b-1) - 1)), offset = f16(min),
    code = clamp(rint((x - offset) / scale), 0, 2^b - 1).
    """
    x = np.asarray(x, dtype=F32)
    lo = x.min(axis=-1)
    amax = np.abs(x).max(axis=-1)
    s = f16(amax / F32(2 ** (bits - 1) - 1))
    z = f16(lo)
    codes = _div_codes(x - z.astype(F32)[..., None], s[..., None], 0, 2 ** bits - 1)
    return codes, s, z


def sym_q8_0(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """q8_0: symmetric int8, zero point fixed at 0, range [-128, 127] (NIAH
    page, section 1.2), one fp16 scale per block: scale = f16(max|x| / 127),
    code = clamp(rint(x / scale), -128, 127).  Returns (codes int32, scale fp16).
    """
    x = np.asarray(x, dtype=F32)
    amax = np.abs(x).max(axis=-1)
    s = f16(amax / F32(127))
    codes = _div_codes(x, s[..., None], -128, 127)
    return codes, s


E5M2_MAX = 57344.0


def fp8_e5m2_codes(v: np.ndarray) -> np.ndarray:
    """float32 -> FP8 E5M2 bytes (sign, 5 exponent bits, 2 mantissa bits; the
    format of the Survey page, section 3.4, for vLLM's fp8 KV cache), round
    to nearest even; magnitudes past the largest finite value (57344)
    saturate to it.  The rounding is torch's float8_e5m2 conversion."""
    import torch
    v = np.clip(np.asarray(v, dtype=F32), -E5M2_MAX, E5M2_MAX)
    return torch.from_numpy(np.ascontiguousarray(v)).to(torch.float8_e5m2).view(torch.uint8).numpy()


def fp8_e5m2_values(codes: np.ndarray) -> np.ndarray:
    """FP8 E5M2 bytes -> float64 values."""
    import torch
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    return torch.from_numpy(c).view(torch.float8_e5m2).to(torch.float64).numpy()


def codebook_midpoints(cb: np.ndarray) -> np.ndarray:
    """Decision thresholds between neighbouring centroids: m_i = f32(C_i + C_{i+1}) * 0.5
    for i = 0..14 (float32).  ``cb`` is fp16 [..., 16] ascending."""
    c = np.asarray(cb, dtype=np.float16).astype(F32)
    return (c[..., :-1] + c[..., 1:]) * F32(0.5)


def codebook_codes(x: np.ndarray, cb: np.ndarray) -> np.ndarray:
    """Non-uniform quantization (KVQuant page, section 2.2): each value maps to
    the nearest of 16 per-channel centroids, ties to the lower index, computed
    as the number of midpoints strictly below x.  ``x`` [..., H, d] float32,
    ``cb`` fp16 [H, d, 16]."""
    m = codebook_midpoints(cb)                       # [H, d, 15]
    x = np.asarray(x, dtype=F32)
    return (x[..., None] > m).sum(axis=-1).astype(np.int32)


def outlier_count(frac: float, n: int) -> int:
    """Number of outliers kept per token: ceil(frac * n), frac taken as float32."""
    if frac <= 0:
        return 0
    return int(math.ceil(float(np.float32(frac)) * n))


def select_outliers(x: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Dense-and-sparse split (KVQuant page, section 2.2; section 3.3's
    outlier_threshold_ratio): per token (row of ``x``, all heads flattened,
    float32) keep the ``k`` entries of largest |x|, ties to the lower flat
    index.  Returns (cols [N, k] ascending, int64; vals [N, k] float32)."""
    x = np.asarray(x, dtype=F32)
    order = np.argsort(-np.abs(x), axis=1, kind="stable")   # stable: ties keep index order
    cols = np.sort(order[:, :k], axis=1).astype(np.int64)
    vals = np.take_along_axis(x, cols, axis=1)
    return cols, vals


def outlier_mask(x: np.ndarray, k: int) -> np.ndarray:
    """The set select_outliers keeps, as a boolean mask [N, n], found through
    the k-th largest magnitude of each row instead of a full sort: every
    entry above it, then the entries equal to it in index order until k are
    taken (ties to the lower index).  For long contexts."""
    a = np.abs(np.asarray(x, dtype=F32))
    n = a.shape[1]
    kth = np.partition(a, n - k, axis=1)[:, n - k][:, None]
    above = a > kth
    need = k - above.sum(axis=1, keepdims=True)
    ties = a == kth
    return above | (ties & (np.cumsum(ties, axis=1) <= need))


# --------------------------------------------------------------------------
# Whole-tensor encoding (logical codes; byte layouts live in layout.py)
# --------------------------------------------------------------------------

def encode_tensor(x: np.ndarray, fmt: Dict, codebook: np.ndarray = None,
                  head_scale: np.ndarray = None) -> Dict[str, np.ndarray]:
    """Bulk-encode one cache tensor.

    ``x`` is float32 [B, T, H, d] holding fp16/bf16 values.  ``fmt`` has
    quantizer, bits, group_size, layout, outlier_frac.  Returns logical arrays:

    * ``codes`` int32 [B, H, Tq, d] for the Tq quantized tokens
      (Tq = T, except per-channel layout: Tq = floor(T / G) * G),
    * ``scale``/``zero`` fp16: per-token [B, H, T, d/G]; per-channel
      [B, H, T/G, d]; q8_0 has no zero,
    * ``tail`` float32 [B, H, T - Tq, d]: per-channel keys of the unfinished
      group stay unquantized (reading: the pages quantize only complete
      groups of appended rows -- NIAH page section 1.1, KVQuant page
      section 3.4 -- and say nothing of partial groups); ``tail_rows`` is
      every token's raw value, from which the tail's byte image is drawn,
    * per-channel groups with ``window_overlap`` > 0 take their scale and
      zero from a window reaching that many tokens back (``_windowed_groups``),
    * ``cols``/``vals`` for codebook outliers ([B, T, k]),
    * ``deq`` float64 [B, H, T, d]: the values attention sees.

    ``fp8_e5m2`` stores code = E5M2(x / s_h) with one float32 scale s_h per
    KV head (``head_scale``, default 1; reading of the Survey page, section
    3.4: fp8 KV cache "with scale computation per head") and dequantizes to
    E5M2 value * s_h.
    """
    x = np.asarray(x, dtype=F32)
    B, T, H, d = x.shape
    q = fmt["quantizer"]
    bits = fmt["bits"]
    G = fmt.get("group_size", 0)
    layout = fmt.get("layout", "per_token")
    xt = np.transpose(x, (0, 2, 1, 3))                  # [B, H, T, d]
    out: Dict[str, np.ndarray] = {}
    if q == "none":
        out["deq"] = xt.astype(np.float64)
        return out
    if q == "fp8_e5m2":
        sc = np.ones(H, dtype=F32) if head_scale is None else np.asarray(head_scale, dtype=F32)
        codes = fp8_e5m2_codes(xt / sc[None, :, None, None])      # float32 division
        out["codes"] = codes.astype(np.int32)
        out["deq"] = fp8_e5m2_values(codes) * sc.astype(np.float64)[None, :, None, None]
        return out
    if q == "codebook":
        if codebook is None:
            raise ValueError("codebook format needs a codebook")
        codes = codebook_codes(x, codebook)             # [B, T, H, d]
        cbf = np.asarray(codebook, dtype=np.float16).astype(np.float64)
        hh = np.arange(H)[None, None, :, None]
        cc = np.arange(d)[None, None, None, :]
        deq = cbf[hh, cc, codes]                        # [B, T, H, d]
        k = outlier_count(fmt.get("outlier_frac", 0.0), H * d)
        if k > 0:
            flat = x.reshape(B * T, H * d)
            cols, vals = select_outliers(flat, k)
            dflat = deq.reshape(B * T, H * d)
            rows = np.arange(B * T)[:, None]
            # replacement semantics with the stored fp16 value (KVQuant page,
            # section 3.3: outliers are kept in fp16; exact for fp16 inputs,
            # the nearest-even fp16 of a bf16 input)
            dflat[rows, cols] = f16(vals).astype(np.float64)
            deq = dflat.reshape(B, T, H, d)
            out["cols"] = cols.reshape(B, T, k)
            out["vals"] = vals.reshape(B, T, k)
        out["codes"] = np.transpose(codes, (0, 2, 1, 3))
        out["deq"] = np.transpose(deq, (0, 2, 1, 3))
        return out

    if layout == "per_token" and fmt.get("head_group_size"):
        # a group size per KV head (Memory-killer page, sections 2.3 and
        # 5.3: finer groups for the heads that are sensitive to quantization)
        # -- each head is its own per-token tensor; scale and zero become
        # per-head lists of [B, T, d / G_h] arrays
        parts = [encode_tensor(x[:, :, h:h + 1, :], dict(fmt, group_size=int(gh),
                                                           head_group_size=None))
                 for h, gh in enumerate(fmt["head_group_size"])]
        out["codes"] = np.concatenate([p["codes"] for p in parts], axis=1)
        out["deq"] = np.concatenate([p["deq"] for p in parts], axis=1)
        out["scale"] = [p["scale"][:, 0] for p in parts]
        if "zero" in parts[0]:
            out["zero"] = [p["zero"][:, 0] for p in parts]
        return out

    if layout == "per_token":
        if d % G:
            raise ValueError("group size must divide head_dim")
        g = xt.reshape(B, H, T, d // G, G)
        if q == "asym_minmax":
            c, s, z = asym_minmax(g, bits)
        elif q == "asym_absmax_offset":
            c, s, z = asym_absmax_offset(g, bits)
        elif q == "sym_q8_0":
            c, s = sym_q8_0(g)
            z = None
        else:
            raise ValueError(q)
        out["codes"] = c.reshape(B, H, T, d)
        out["scale"] = s
        if z is not None:
            out["zero"] = z
        deq = c.astype(np.float64) * s.astype(np.float64)[..., None]
        if z is not None:
            deq = deq + z.astype(np.float64)[..., None]
        out["deq"] = deq.reshape(B, H, T, d)
        return out

    if layout == "per_channel":
        # Per-channel keys, groups of G consecutive tokens (KVQuant page,
        # section 2.2; Survey page, section 2.4's per-position groups).
        nq = (T // G) * G
        overlap = int(fmt.get("window_overlap", 0))
        if overlap:
            c, s, z = _windowed_groups(xt[:, :, :nq, :], q, bits, G, overlap)
        else:
            g = xt[:, :, :nq, :].reshape(B, H, T // G, G, d)
            g = np.swapaxes(g, -1, -2)                      # [B, H, ng, d, G]
            if q == "asym_minmax":
                c, s, z = asym_minmax(g, bits)
            elif q == "asym_absmax_offset":
                c, s, z = asym_absmax_offset(g, bits)
            else:
                raise ValueError(f"{q} has no per-channel form")
        deq_q = c.astype(np.float64) * s.astype(np.float64)[..., None] + z.astype(np.float64)[..., None]
        out["codes"] = np.swapaxes(c, -1, -2).reshape(B, H, nq, d)
        out["scale"] = s                                  # [B, H, ng, d]
        out["zero"] = z
        out["tail"] = xt[:, :, nq:, :].copy()
        out["tail_rows"] = xt.copy()     # the raw tokens the tail ring draws from
        deq = np.concatenate([np.swapaxes(deq_q, -1, -2).reshape(B, H, nq, d),
                              xt[:, :, nq:, :].astype(np.float64)], axis=2)
        out["deq"] = deq
        return out
    raise ValueError(layout)


def window_params(win: np.ndarray, quantizer: str, bits: int) -> Tuple[np.ndarray, np.ndarray]:
    """(scale, zero) fp16 from the statistics of a window (last axis), by the
    rule of ``quantizer``: min-max (asym_minmax) or the TurboQuant page's
    absmax / (2^(b-1) - 1) with a min offset (asym_absmax_offset)."""
    win = np.asarray(win, dtype=F32)
    lo = win.min(axis=-1)
    if quantizer == "asym_minmax":
        s = f16((win.max(axis=-1) - lo) / F32(2 ** bits - 1))
    elif quantizer == "asym_absmax_offset":
        s = f16(np.abs(win).max(axis=-1) / F32(2 ** (bits - 1) - 1))
    else:
        raise ValueError(f"{quantizer} has no window form")
    return s, f16(lo)


def _windowed_groups(xq: np.ndarray, quantizer: str, bits: int, G: int, overlap: int):
    """Per-channel token groups whose statistics come from overlapping
    sliding windows (TurboQuant page, section 3.1: quantization parameters
    from a sliding window's extrema; section 6, problem 1: a window overlap
    of 64 tokens against edge effects).

    Reading: the windows advance by G tokens and overlap by ``overlap``:
    window g spans tokens [g G - overlap, g G + G) (clipped at token 0), and
    token t is quantized with the parameters of the window whose last G
    tokens hold it, g = t // G.  Looking back rather than ahead lets a group
    be encoded as soon as its own tokens are in, as an append-only cache
    needs.  ``xq`` [B, H, ng * G, d]; returns codes [B, H, ng, d, G] and
    scale, zero [B, H, ng, d]."""
    B, H, nq, d = xq.shape
    ng = nq // G
    codes = np.zeros((B, H, ng, d, G), dtype=np.int32)
    scale = np.zeros((B, H, ng, d), dtype=np.float16)
    zero = np.zeros((B, H, ng, d), dtype=np.float16)
    for g in range(ng):
        win = np.swapaxes(xq[:, :, max(0, g * G - overlap):(g + 1) * G, :], -1, -2)  # [B, H, d, W]
        core = np.swapaxes(xq[:, :, g * G:(g + 1) * G, :], -1, -2)                   # [B, H, d, G]
        s, z = window_params(win, quantizer, bits)
        codes[:, :, g] = _div_codes(core - z.astype(F32)[..., None], s[..., None], 0, 2 ** bits - 1)
        scale[:, :, g] = s
        zero[:, :, g] = z
    return codes, scale, zero


def encode_with_sink(x: np.ndarray, fmt: Dict, codebook: np.ndarray = None,
                     sink: int = 0, head_scale: np.ndarray = None) -> Dict:
    """Bulk-encode one cache tensor whose first ``sink`` tokens are an
    attention sink (KVQuant page, "Attention Sink": the keys and values of
    the first few tokens, which draw very high attention, are kept in full
    precision at quantization and inference time; ``num_sink_tokens``).

    Reading: tokens [0, s), s = min(sink, T), keep their fp16/bf16 values and
    are attended exactly; tokens [s, T) form an ordinary quantized cache of
    their own, encoded by ``encode_tensor`` as a sequence that starts at
    token s (so per-channel key groups start at token s).  Positions (RoPE)
    stay absolute.  Returns ``sink`` float64 [B, H, s, d] (the raw prefix),
    ``rest`` (the encoding of the quantized tokens, or None when every token
    is in the sink) and ``deq`` float64 [B, H, T, d] (what attention sees).
    """
    x = np.asarray(x, dtype=F32)
    B, T, H, d = x.shape
    s = min(int(sink), T)
    pre = np.transpose(x[:, :s], (0, 2, 1, 3)).astype(np.float64)
    rest = encode_tensor(x[:, s:], fmt, codebook, head_scale) if T > s else None
    deq = pre if rest is None else np.concatenate([pre, rest["deq"]], axis=2)
    return {"sink": pre, "rest": rest, "deq": deq}
