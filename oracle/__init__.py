"""CPU oracle for low-bit KV-cache quantization fused into decode attention.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
reference that the HIP library is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the library itself never does, and shares no code with it.

Sources (web pages, cited by page and section):

* "NIAH" page -- TurboQuant NIAH single-needle retrieval, Qwen3.5-35B-A3B
  q8_0 KV cache at 4K/8K/16K (www.cf-1.com/news/5482713).
* "TurboQuant" page -- 3-bit dynamic asymmetric KV-cache quantization for a
  70B model (www.dpshk.com/news/6341316).
* "KVQuant" page -- KVQuant: per-channel pre-RoPE keys, non-uniform
  quantization, dense-and-sparse outliers (www.cf-1.com/news/2306543).
* "Survey" page -- W8A8/W4A8, sparse quantization, FlashAttention-3 and
  KV-cache quantization (www.discosf.com/news/4854722).
* "Memory-killer" page -- the KV cache as memory killer and TurboQuant's
  group-wise scaling and fused dequantization (www.demingchina.com/news/57821).

Precision: encoding is done in IEEE float32 with round-half-even, exactly as
specified in ``quant.py``; dequantization and attention are float64.

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, printed values, invariants and brute force.  Readings of the pages
where they are silent are listed in ``quant.py`` and ``layout.py``.
"""
from . import quant, layout, attention, cache_bytes, paging  # noqa: F401
