"""ctypes binding of libkvq (include/kvq.h): argument marshalling only.

Every step of the quantized-cache path runs in the HIP library; this module
converts Python/torch arguments into the C structs and device pointers the
C ABI expects, and raises ``KvqError`` on a non-OK status.  torch is used
for device memory and the current HIP stream.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Any, Dict, Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvq.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "kvq.h")
# interface version the structures below follow (major * 100 + minor)
ABI_VERSION = 112

# ---- constants mirrored from kvq.h -------------------------------------------
OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_DEVICE = 0, -1, -2, -3, -4
F16, BF16, F32 = 0, 1, 2
QUANT = {"none": 0, "asym_minmax": 1, "asym_absmax_offset": 2, "sym_q8_0": 3, "codebook": 4,
         "fp8_e5m2": 5}
LAYOUT = {"per_token": 0, "per_channel": 1}
BYTES_PAYLOAD, BYTES_ALLOC = 0, 1
PATHS = {"auto": 0, "valu": 1, "mfma": 2, "lut": 3}
PREFILL_CODES, PREFILL_STAGED = 1, 2   # kvq_prefill_kernel results
DTYPES = {"f16": F16, "bf16": BF16, "f32": F32}


class TensorFormat(ctypes.Structure):
    _fields_ = [("quantizer", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("outlier_frac", ctypes.c_float), ("window_overlap", ctypes.c_int32),
                ("head_group_size", ctypes.POINTER(ctypes.c_int32))]


class Config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_ctx", ctypes.c_int64), ("kv_dtype", ctypes.c_int32),
                ("rope", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("decode_splits", ctypes.c_int32), ("decode_path", ctypes.c_int32),
                ("k", TensorFormat), ("v", TensorFormat), ("sink_tokens", ctypes.c_int32),
                ("page_pool", ctypes.c_int32)]


class CacheStruct(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("k_codebook", ctypes.c_void_p),
                ("v_codebook", ctypes.c_void_p), ("n_ctx", ctypes.c_int64),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p)]


class Region(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_uint64), ("bytes", ctypes.c_uint64)]


class TensorRegions(ctypes.Structure):
    _fields_ = [("codes", Region), ("params", Region), ("tail", Region), ("row_ptr", Region),
                ("col", Region), ("val", Region), ("sink", Region), ("tile_off", Region), ("tile_ent", Region)]


class LayoutInfo(ctypes.Structure):
    _fields_ = [("k", TensorRegions), ("v", TensorRegions), ("workspace", Region),
                ("total_bytes", ctypes.c_uint64), ("capacity", ctypes.c_int64),
                ("max_splits", ctypes.c_int32), ("pages_per_seq", ctypes.c_int32)]


class KvqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"kvq status {status}: {msg}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load the in-tree libkvq.so (built by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.kvq_cache_bytes.argtypes = [ctypes.POINTER(Config), ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int32, ctypes.POINTER(ctypes.c_uint64)]
        L.kvq_cache_layout.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(LayoutInfo)]
        L.kvq_quantize_append.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(CacheStruct),
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_void_p]
        L.kvq_decode_attention.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(CacheStruct),
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                           ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
        L.kvq_decode_attention_scratch.argtypes = L.kvq_decode_attention.argtypes
        L.kvq_append_decode.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(CacheStruct),
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_void_p]
        L.kvq_append_decode_fused.restype = ctypes.c_int32
        L.kvq_append_decode_fused.argtypes = [ctypes.POINTER(Config), ctypes.c_int64]
        L.kvq_prefill_attention.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(CacheStruct),
                                            ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
                                            ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_uint64, ctypes.c_void_p]
        L.kvq_prefill_workspace_bytes.argtypes = [ctypes.POINTER(Config), ctypes.c_int32,
                                                  ctypes.c_int64, ctypes.POINTER(ctypes.c_uint64)]
        for fn in ("kvq_cache_bytes", "kvq_cache_layout", "kvq_quantize_append",
                   "kvq_decode_attention", "kvq_decode_attention_scratch", "kvq_append_decode",
                   "kvq_prefill_attention", "kvq_prefill_workspace_bytes"):
            getattr(L, fn).restype = ctypes.c_int32
        L.kvq_last_error.restype = ctypes.c_char_p
        L.kvq_last_error.argtypes = []
        L.kvq_abi_version.restype = ctypes.c_int32
        if L.kvq_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH}: interface version {L.kvq_abi_version()}, "
                               f"this binding expects {ABI_VERSION}; rebuild the library")
        L.kvq_set_decode_events.restype = ctypes.c_int32
        L.kvq_set_decode_events.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.kvq_decode_path.restype = ctypes.c_int32
        L.kvq_decode_path.argtypes = [ctypes.POINTER(Config)]
        L.kvq_prefill_kernel.restype = ctypes.c_int32
        L.kvq_prefill_kernel.argtypes = [ctypes.POINTER(Config)]
        _lib = L
    return _lib


def declared_symbols() -> list:
    """Names of the functions include/kvq.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:kvq_status|const char\*|int32_t)\s+(kvq_\w+)\s*\(",
                                 text, flags=re.M)))


def _check(st: int) -> None:
    if st != OK:
        raise KvqError(st, lib().kvq_last_error().decode())


def fmt_struct(f: Dict[str, Any]) -> TensorFormat:
    """The C struct of a format dict.  Per-head group sizes
    (``head_group_size``, a list) go to a host int32 array that the struct
    keeps alive."""
    hg = f.get("head_group_size")
    arr = (ctypes.c_int32 * len(hg))(*[int(v) for v in hg]) if hg else None
    t = TensorFormat(QUANT[f["quantizer"]], int(f["bits"]), int(f.get("group_size", 0)),
                     LAYOUT[f.get("layout", "per_token")], float(f.get("outlier_frac", 0.0)),
                     int(f.get("window_overlap", 0)),
                     ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)) if arr is not None else None)
    t._keep = arr
    return t


def make_config(*, batch: int, n_q_heads: int, n_kv_heads: int, max_ctx: int,
                kv_dtype: str, k: Dict[str, Any], v: Dict[str, Any], head_dim: int = 128,
                rope: bool = False, rope_base: float = 10000.0, decode_splits: int = 0,
                decode_path: str = "auto", sink_tokens: int = 0, page_pool: int = 0) -> Config:
    kf, vf = fmt_struct(k), fmt_struct(v)
    cfg = Config(batch, n_q_heads, n_kv_heads, head_dim, max_ctx, DTYPES[kv_dtype],
                 int(bool(rope)), float(rope_base), int(decode_splits), PATHS[decode_path],
                 kf, vf, int(sink_tokens), int(page_pool))
    cfg._keep = (kf._keep, vf._keep)   # per-head group-size arrays the struct points to
    return cfg


def config_from_workload(w, max_ctx: Optional[int] = None, decode_splits: int = 0,
                         decode_path: str = "auto", sink_tokens: Optional[int] = None,
                         page_pool: int = 0) -> Config:
    return make_config(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                       max_ctx=max_ctx if max_ctx is not None else w.ctx, kv_dtype=w.kv_dtype,
                       k=w.k, v=w.v, head_dim=w.head_dim, rope=w.rope, rope_base=w.rope_base,
                       decode_splits=decode_splits, decode_path=decode_path,
                       sink_tokens=(sink_tokens if sink_tokens is not None
                                    else getattr(w, "sink_tokens", 0)),
                       page_pool=page_pool)


def cache_bytes(cfg: Config, n_ctx: int = 0, n_layers: int = 1, what: int = BYTES_PAYLOAD) -> int:
    out = ctypes.c_uint64(0)
    _check(lib().kvq_cache_bytes(ctypes.byref(cfg), int(n_ctx), int(n_layers), int(what),
                                 ctypes.byref(out)))
    return int(out.value)


def decode_path(cfg: Config) -> str:
    """"valu", "mfma" or "lut": the decode kernel the library runs for ``cfg``."""
    r = lib().kvq_decode_path(ctypes.byref(cfg))
    if r < 0:
        _check(r)
    return {PATHS["valu"]: "valu", PATHS["mfma"]: "mfma", PATHS["lut"]: "lut"}[r]


def prefill_kernel(cfg: Config) -> str:
    """"codes" or "staged": the prefill kernel the library runs for ``cfg``."""
    r = lib().kvq_prefill_kernel(ctypes.byref(cfg))
    if r < 0:
        _check(r)
    return {PREFILL_CODES: "codes", PREFILL_STAGED: "staged"}[r]


def cache_layout(cfg: Config) -> LayoutInfo:
    info = LayoutInfo()
    _check(lib().kvq_cache_layout(ctypes.byref(cfg), ctypes.byref(info)))
    return info


_TORCH_DTYPES = {"f16": "float16", "bf16": "bfloat16", "f32": "float32"}


def _torch_dtype(name: str):
    import torch
    return getattr(torch, _TORCH_DTYPES[name])


def _dtype_name(t) -> str:
    import torch
    names = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}
    if t.dtype not in names:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return names[t.dtype]


def _check_tensor(name: str, t, shape, dtype=None, device: bool = True) -> None:
    """Raise before any device call unless ``t`` is a contiguous device
    tensor of ``shape`` (and ``dtype``): the C ABI takes raw pointers and
    would read or write past a smaller or differently laid out buffer."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device and not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor (got {t.device})")


def _check_devices(**tensors) -> None:
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name}: must be a device tensor (got {t.device})")


def _resolve_out(out, out_dtype: Optional[str], shape, device):
    """The output tensor and its dtype name: ``out`` decides the dtype when
    given (a conflicting ``out_dtype`` is an error); otherwise a new tensor
    of ``out_dtype`` (default f32)."""
    import torch
    if out is None:
        name = out_dtype or "f32"
        if name not in DTYPES:
            raise ValueError(f"out_dtype must be one of {sorted(DTYPES)}")
        return torch.empty(shape, dtype=_torch_dtype(name), device=device), name
    name = _dtype_name(out)
    if out_dtype is not None and out_dtype != name:
        raise TypeError(f"out has dtype {out.dtype} but out_dtype={out_dtype!r}")
    _check_tensor("out", out, shape, device=False)
    return out, name


def _stream_ptr(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class Cache:
    """A cache allocation (zero-filled torch uint8 device buffer) plus the
    host-side token count.  Codebooks, when used, are fp16 [Hkv, d, 16]
    device tensors, FP8 scales float32 [Hkv] device tensors, the page table
    of a paged cache an int32 [B, pages_per_seq] device tensor; all must
    outlive the cache."""

    def __init__(self, cfg: Config, device="cuda", k_codebook=None, v_codebook=None,
                 k_scale=None, v_scale=None, page_table=None):
        import torch
        self.cfg = cfg
        self.layout = cache_layout(cfg)
        self.buffer = torch.zeros(int(self.layout.total_bytes), dtype=torch.uint8, device=device)
        self.k_codebook = k_codebook.contiguous() if k_codebook is not None else None
        self.v_codebook = v_codebook.contiguous() if v_codebook is not None else None
        self.k_scale = k_scale.contiguous() if k_scale is not None else None
        self.v_scale = v_scale.contiguous() if v_scale is not None else None
        self.page_table = None
        if cfg.page_pool:
            import torch
            if page_table is None:
                raise ValueError("a paged cache (page_pool > 0) needs a page_table")
            _check_tensor("page_table", page_table, (cfg.batch, self.layout.pages_per_seq),
                          torch.int32, device=False)
            self.page_table = page_table
        elif page_table is not None:
            raise ValueError("page_table given for a contiguous cache (page_pool = 0)")
        self.n_ctx = 0

    def struct(self) -> CacheStruct:
        ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        return CacheStruct(self.buffer.data_ptr(), ptr(self.k_codebook), ptr(self.v_codebook),
                           self.n_ctx, ptr(self.k_scale), ptr(self.v_scale),
                           ptr(self.page_table))

    def region(self, tensor: str, name: str):
        """uint8 view of one array of the allocation (e.g. ("k", "codes"))."""
        r = getattr(getattr(self.layout, tensor), name)
        return self.buffer[r.offset:r.offset + r.bytes]

    def append(self, k_new, v_new, stream=None) -> None:
        quantize_append(self, k_new, v_new, stream)

    def decode(self, q, q_pos=None, sm_scale: float = 0.0, out=None,
               out_dtype: Optional[str] = None, stream=None):
        return decode_attention(self, q, q_pos=q_pos, sm_scale=sm_scale, out=out,
                                out_dtype=out_dtype, stream=stream)

    def append_decode(self, k_new, v_new, q, q_pos=None, sm_scale: float = 0.0, out=None,
                      out_dtype: Optional[str] = None, stream=None):
        return append_decode(self, k_new, v_new, q, q_pos=q_pos, sm_scale=sm_scale, out=out,
                             out_dtype=out_dtype, stream=stream)

    def prefill(self, q, sm_scale: float = 0.0, out=None, out_dtype: Optional[str] = None,
                stream=None, workspace=None):
        return prefill_attention(self, q, sm_scale=sm_scale, out=out, out_dtype=out_dtype,
                                 stream=stream, workspace=workspace)


def set_decode_events(start=None, stop=None) -> None:
    """Have the next decode call on this thread record ``start`` and ``stop``
    (torch.cuda.Event objects or raw hipEvent_t handles) right around its
    token-streaming kernel.  A torch event exists only once it has been
    recorded, so record each one once before passing it here."""
    def handle(e):
        if e is None:
            return None
        h = int(e.cuda_event) if hasattr(e, "cuda_event") else int(e)
        if not h:
            raise ValueError("the event has not been created yet: record it once first")
        return h
    _check(lib().kvq_set_decode_events(handle(start), handle(stop)))


def quantize_append(cache: Cache, k_new, v_new, stream=None) -> None:
    """Append k_new/v_new ([B, n_new, Hkv, d], cache dtype, contiguous, on the device)."""
    c = cache.cfg
    if k_new.dim() != 4:
        raise ValueError(f"k_new: expected [B, n_new, Hkv, d], got shape {tuple(k_new.shape)}")
    n_new = int(k_new.shape[1])
    kdt = _torch_dtype({F16: "f16", BF16: "bf16"}[c.kv_dtype])
    shape = (c.batch, n_new, c.n_kv_heads, c.head_dim)
    _check_tensor("k_new", k_new, shape, kdt, device=False)
    _check_tensor("v_new", v_new, shape, kdt, device=False)
    _check_devices(k_new=k_new, v_new=v_new)
    cs = cache.struct()
    _check(lib().kvq_quantize_append(ctypes.byref(cache.cfg), ctypes.byref(cs),
                                     k_new.data_ptr(), v_new.data_ptr(), n_new,
                                     _stream_ptr(stream)))
    cache.n_ctx = int(cs.n_ctx)


def decode_attention(cache: Cache, q, q_pos=None, sm_scale: float = 0.0, out=None,
                     out_dtype: Optional[str] = None, stream=None):
    """One decode step: q [B, Hq, d] -> out [B, Hq, d].  The output dtype is
    that of ``out`` when given, else ``out_dtype`` (default f32).  ``q_pos``:
    int32 [B] device tensor or None."""
    import torch
    c = cache.cfg
    shape = (c.batch, c.n_q_heads, c.head_dim)
    _check_tensor("q", q, shape, _torch_dtype({F16: "f16", BF16: "bf16"}[c.kv_dtype]),
                  device=False)
    if q_pos is not None:
        _check_tensor("q_pos", q_pos, (c.batch,), torch.int32, device=False)
    out, out_dtype = _resolve_out(out, out_dtype, shape, q.device)
    _check_devices(q=q, q_pos=q_pos, out=out)
    cs = cache.struct()
    _check(lib().kvq_decode_attention(ctypes.byref(cache.cfg), ctypes.byref(cs), q.data_ptr(),
                                      q_pos.data_ptr() if q_pos is not None else None,
                                      float(sm_scale), out.data_ptr(), DTYPES[out_dtype],
                                      _stream_ptr(stream)))
    return out


def append_decode_fused(cfg: Config, n_ctx: int) -> bool:
    """Whether append_decode on a cache of n_ctx tokens runs the fused step."""
    r = lib().kvq_append_decode_fused(ctypes.byref(cfg), int(n_ctx))
    if r < 0:
        _check(r)
    return bool(r)


def append_decode(cache: Cache, k_new, v_new, q, q_pos=None, sm_scale: float = 0.0, out=None,
                  out_dtype: Optional[str] = None, stream=None):
    """One serving step: append k_new/v_new ([B, 1, Hkv, d]) and decode q
    ([B, Hq, d]) over the cache that holds them (kvq_append_decode)."""
    import torch
    c = cache.cfg
    kdt = _torch_dtype({F16: "f16", BF16: "bf16"}[c.kv_dtype])
    tok_shape = (c.batch, 1, c.n_kv_heads, c.head_dim)
    _check_tensor("k_new", k_new, tok_shape, kdt, device=False)
    _check_tensor("v_new", v_new, tok_shape, kdt, device=False)
    shape = (c.batch, c.n_q_heads, c.head_dim)
    _check_tensor("q", q, shape, kdt, device=False)
    if q_pos is not None:
        _check_tensor("q_pos", q_pos, (c.batch,), torch.int32, device=False)
    out, out_dtype = _resolve_out(out, out_dtype, shape, q.device)
    _check_devices(k_new=k_new, v_new=v_new, q=q, q_pos=q_pos, out=out)
    cs = cache.struct()
    _check(lib().kvq_append_decode(ctypes.byref(cache.cfg), ctypes.byref(cs), k_new.data_ptr(),
                                   v_new.data_ptr(), q.data_ptr(),
                                   q_pos.data_ptr() if q_pos is not None else None,
                                   float(sm_scale), out.data_ptr(), DTYPES[out_dtype],
                                   _stream_ptr(stream)))
    cache.n_ctx = int(cs.n_ctx)
    return out


def decode_attention_scratch(cache: Cache, q, q_pos=None, sm_scale: float = 0.0, out=None,
                             out_dtype: Optional[str] = None, stream=None):
    """decode_attention through kvq_decode_attention_scratch: the split-K
    partial states live in the library's static device array (calls on one
    GPU must not overlap).  The caller that cannot allocate passes ``out``."""
    import torch
    c = cache.cfg
    shape = (c.batch, c.n_q_heads, c.head_dim)
    _check_tensor("q", q, shape, _torch_dtype({F16: "f16", BF16: "bf16"}[c.kv_dtype]),
                  device=False)
    if q_pos is not None:
        _check_tensor("q_pos", q_pos, (c.batch,), torch.int32, device=False)
    out, out_dtype = _resolve_out(out, out_dtype, shape, q.device)
    _check_devices(q=q, q_pos=q_pos, out=out)
    cs = cache.struct()
    _check(lib().kvq_decode_attention_scratch(ctypes.byref(cache.cfg), ctypes.byref(cs),
                                              q.data_ptr(),
                                              q_pos.data_ptr() if q_pos is not None else None,
                                              float(sm_scale), out.data_ptr(), DTYPES[out_dtype],
                                              _stream_ptr(stream)))
    return out


def prefill_workspace_bytes(cfg: Config, n_q: int, n_ctx: int) -> int:
    out = ctypes.c_uint64(0)
    _check(lib().kvq_prefill_workspace_bytes(ctypes.byref(cfg), int(n_q), int(n_ctx),
                                             ctypes.byref(out)))
    return int(out.value)


def prefill_attention(cache: Cache, q, sm_scale: float = 0.0, out=None,
                      out_dtype: Optional[str] = None, stream=None, workspace=None):
    """Causal attention of the last n_q cached tokens: q [B, n_q, Hq, d] ->
    out [B, n_q, Hq, d] of ``out_dtype``.  ``workspace``: a uint8 device
    tensor for the token-axis split; by default one of the size the library
    asks for is kept on the cache object (grown when needed); pass an empty
    tensor for no split."""
    import torch
    c = cache.cfg
    if q.dim() != 4:
        raise ValueError(f"q: expected [B, n_q, Hq, d], got shape {tuple(q.shape)}")
    n_q = int(q.shape[1])
    shape = (c.batch, n_q, c.n_q_heads, c.head_dim)
    _check_tensor("q", q, shape, _torch_dtype({F16: "f16", BF16: "bf16"}[c.kv_dtype]),
                  device=False)
    out, out_dtype = _resolve_out(out, out_dtype, shape, q.device)
    if workspace is not None:
        _check_tensor("workspace", workspace, (workspace.numel(),), torch.uint8, device=False)
    _check_devices(q=q, out=out, workspace=workspace)
    if workspace is None:
        need = prefill_workspace_bytes(cache.cfg, n_q, cache.n_ctx)
        ws = getattr(cache, "_prefill_ws", None)
        if need and (ws is None or ws.numel() < need):
            ws = torch.empty(need, dtype=torch.uint8, device=q.device)
            cache._prefill_ws = ws
        workspace = ws if need else None
    ws_ptr = workspace.data_ptr() if workspace is not None and workspace.numel() else None
    ws_len = int(workspace.numel()) if ws_ptr else 0
    cs = cache.struct()
    _check(lib().kvq_prefill_attention(ctypes.byref(cache.cfg), ctypes.byref(cs), q.data_ptr(),
                                       n_q, float(sm_scale), out.data_ptr(), DTYPES[out_dtype],
                                       ws_ptr, ws_len, _stream_ptr(stream)))
    return out
