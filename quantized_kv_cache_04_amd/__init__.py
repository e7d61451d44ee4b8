"""Low-bit KV-cache quantization fused into decode (and chunked-prefill)
attention, for MI355X.

The work is done by libkvq.so (hand-written HIP kernels for gfx950 behind
the C ABI in include/kvq.h); this package only exposes that ABI to Python.
"""
from .kvq import (Cache, Config, KvqError, cache_bytes, cache_layout,  # noqa: F401
                  config_from_workload, decode_attention, decode_path, lib, make_config,
                  prefill_attention, prefill_workspace_bytes, quantize_append,
                  set_decode_events)
