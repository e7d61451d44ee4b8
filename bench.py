#!/usr/bin/env python3
"""Benchmark of fused quantized decode attention on one MI355X.

Default workload (``--config 5``): an 8B-shaped serving layer, batch 16,
32 query / 8 KV heads, head_dim 128, 65536 cached tokens per sequence,
4-bit asymmetric keys (per-channel groups of 128 tokens) and values
(per-token groups of 128 channels).  One step = quantize-append one new
token per sequence, then one decode-attention step over the whole cache.

Other configs (``--config 1..4``) time the decode step over a prefilled
cache; caches smaller than 1 GB are replicated and rotated so that every
step streams from HBM rather than the 256 MB last-level cache.

Prints ONE JSON line on stdout.  ``value`` is the effective HBM bandwidth
of the step: the bytes the step must read (packed codes, scales and zeros,
outliers, tail; ``kvq_cache_bytes``) divided by the step time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused quantized decode attention: effective HBM GB/s (% of peak), µs/step"
PEAK_HBM_GBS = 8000.0
DECODE_KERNELS = {"valu": "dec_generic_kernel", "mfma": "dec_mfma_kernel", "lut": "dec_lut_kernel"}
PREFILL_METRIC = "chunked prefill attention over the quantized cache: TFLOP/s (QK^T + PV, causal)"
PEAK_MFMA_F16_TFLOPS = 2500.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


KERNEL_SOURCES = {"dec_mfma_kernel": "decode_mfma.hip", "dec_lut_kernel": "decode_lut.hip",
                  "dec_generic_kernel": "decode_generic.hip", "pre_mfma_kernel": "prefill_mfma.hip",
                  "pre_codes_kernel": "prefill_codes.hip"}


def kernel_source_sha(kernel: str) -> str:
    """Hash of the sources a decode kernel is compiled from: its own .hip
    file and every header of the library."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_kv_cache_04_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name == KERNEL_SOURCES[kernel] or name.endswith(".h"):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def counter_traffic(workload: str, kernel: str):
    """Per-launch HBM bytes of the decode kernel recorded from rocprofv3
    counter runs (profiles/traffic.json), if they were taken on the current
    kernel sources; None otherwise.  Not measured in this run: the record
    says which runs it comes from."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(f"{workload}/{kernel}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_source_sha") != kernel_source_sha(kernel):
        return None
    return {"bytes_per_launch": rec.get("bytes_per_launch"),
            "source": f"recorded in profiles/traffic.json (kernel source sha "
                      f"{rec['kernel_source_sha']}): {rec.get('note', '')}"}


def settle(ms: float, call, stream) -> int:
    """Run ``call(i)`` (a decode that leaves the cache unchanged) on ``stream``
    until ``ms`` milliseconds of wall time have passed; returns the number of
    calls.  A GPU that has just gone from idle to streaming runs the decode
    kernel up to a third slower for tens of launches before its clocks
    settle; a serving GPU runs continuously."""
    import torch
    n = 0
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(20):
                call(n)
                n += 1
            torch.cuda.synchronize()
    return n


def cpu_baseline(w, seconds: float = 12.0):
    """Time the CPU oracle (float32 encode + float64 decode attention) on a
    bounded sample of the workload: whole (sequence, KV head) slices at the
    full context, as many as fit in half of ``seconds``, once with the
    BLAS / OpenMP pools at their default size and once limited to one
    thread.  Encode and attention are timed separately."""
    from oracle import attention as oatt
    from oracle import cache_bytes as ocb
    from oracle import quant as oq
    from synth import make_workload
    from synth.workloads import make_inputs
    from threadpoolctl import threadpool_info, threadpool_limits
    w1 = make_workload(w.cfg_id, batch=1, n_kv_heads=1, ctx=w.ctx, gqa=w.gqa, seed=7, k=w.k, v=w.v)
    inputs = make_inputs(w1, "cpu")
    x_k = inputs["k"].float().numpy()
    x_v = inputs["v"].float().numpy()
    kcb = inputs["k_codebook"].numpy() if inputs["k_codebook"] is not None else None
    vcb = inputs["v_codebook"].numpy() if inputs["v_codebook"] is not None else None
    q = inputs["q"].float().numpy()
    slice_bytes = ocb.payload_bytes(w1.k, w1.v, batch=1, n_kv_heads=1, head_dim=128,
                                    n_ctx=w1.ctx, kv_dtype=w1.kv_dtype)

    def run(budget):
        done, t_enc, t_att = 0, 0.0, 0.0
        while True:
            t0 = time.perf_counter()
            ek = oq.encode_tensor(x_k, w1.k, kcb)
            ev = oq.encode_tensor(x_v, w1.v, vcb)
            t1 = time.perf_counter()
            oatt.decode_attention(q, ek["deq"], ev["deq"], rope=w1.rope, rope_base=w1.rope_base)
            t2 = time.perf_counter()
            done, t_enc, t_att = done + 1, t_enc + (t1 - t0), t_att + (t2 - t1)
            if t_enc + t_att >= budget or done >= 64:
                return done, t_enc, t_att

    cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    n_all, enc_all, att_all = run(seconds / 2)
    with threadpool_limits(limits=1):
        n_one, enc_one, att_one = run(seconds / 2)
    per = lambda n, t: round(t / n, 3)  # noqa: E731
    return {"value": round(n_all * slice_bytes / (enc_all + att_all) / 1e9, 4), "unit": "GB/s",
            "cores": int(cores), "kind": "oracle",
            "sample": f"{n_all} x (1 sequence, 1 KV head, {w1.gqa} query heads, T={w1.ctx}) slices: "
                      f"float32 encode + float64 dequant and attention, {enc_all + att_all:.1f} s "
                      f"(host reports {os.cpu_count()} CPUs)",
            "encode_s_per_slice": per(n_all, enc_all), "attention_s_per_slice": per(n_all, att_all),
            "single_thread": {"value": round(n_one * slice_bytes / (enc_one + att_one) / 1e9, 4),
                              "slices": n_one, "encode_s_per_slice": per(n_one, enc_one),
                              "attention_s_per_slice": per(n_one, att_one)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256,
                    help="timed steps (the serving workload flushes a key group every 128)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--ctx", type=int, default=None, help="context (config 2: 4096/8192/16384)")
    ap.add_argument("--path", choices=["auto", "valu", "mfma", "lut"], default="auto")
    ap.add_argument("--splits", type=int, default=0,
                    help="upper bound on split-K partitions of the token axis (0 = library default)")
    ap.add_argument("--settle-ms", type=float, default=500.0,
                    help="before the warm-up steps, run decode calls (which leave the cache "
                         "unchanged) for this long, so that the GPU's clocks settle into the "
                         "state a continuously serving GPU runs in")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--kv-format", choices=["workload", "fp8_e5m2"], default="workload",
                    help="fp8_e5m2: store keys and values of the workload's shape as FP8 E5M2 "
                         "with per-head scales instead of its own formats")
    ap.add_argument("--paged", nargs="?", const="shuffled", choices=["shuffled", "sequential"],
                    default=None,
                    help="store the cache as a paged cache: a pool of 32-token pages that a "
                         "seeded, shuffled page table (or the identity order) deals out to the "
                         "sequences")
    ap.add_argument("--prefill", type=int, default=0, metavar="N",
                    help="measure chunked prefill instead: each step appends an N-token chunk to "
                         "a cache of ctx - N tokens and runs causal attention for its N queries")
    ap.add_argument("--encode", type=int, default=0, metavar="N",
                    help="measure bulk encode instead: each step appends N tokens per sequence "
                         "to an empty cache")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 launches), the reference "
                         "point for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the decode step of one GPU's share runs on a "
              f"single MI355X (asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_kv_cache_04_amd as kvq_pkg
    from quantized_kv_cache_04_amd import kvq
    from synth import make_workload
    from synth.workloads import make_inputs, make_page_table, make_step_tokens

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kvq_pkg.lib()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        # an elementwise kernel (dst = src * 1 in float32): it reads and
        # writes n bytes once each (a same-type copy_ would go to a DMA copy,
        # not a kernel dispatch)
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "elementwise copy", "bytes_read": n, "bytes_written": n,
                          "launches": 3}), flush=True)
        return
    over = {}
    if args.kv_format == "fp8_e5m2":
        fp8 = dict(quantizer="fp8_e5m2", bits=8, group_size=0, layout="per_token", outlier_frac=0.0)
        over = dict(k=fp8, v=fp8)
    w = make_workload(args.config, ctx=args.ctx, **over)
    if args.prefill:
        bench_prefill(args, w, dev)
        return
    if args.encode:
        bench_encode(args, w, dev)
        return
    serving = args.config == 5
    K, W = args.steps, args.warmup
    # warm-up, the timed steps, then as many instrumented steps (serving: one
    # token per sequence appended at each)
    max_ctx = w.ctx + (W + 2 * K + 1 if serving else 0)
    n_pages = w.batch * ((max_ctx + 31) // 32) if args.paged else 0
    cfg = kvq.config_from_workload(w, max_ctx=max_ctx, decode_path=args.path,
                                   decode_splits=args.splits, page_pool=n_pages)
    stream = torch.cuda.Stream()
    log(f"workload cfg{w.cfg_id} {CONFIG_NAME(w)}: B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} "
        f"T={w.ctx}; generating inputs on the GPU")

    with torch.cuda.stream(stream):
        inputs = make_inputs(w, dev)
        payload0 = kvq.cache_bytes(cfg, w.ctx)
        copies = 1 if serving else max(1, math.ceil(1.0e9 / payload0))
        caches = []
        for i in range(copies):
            table = None
            if args.paged == "shuffled":
                table = make_page_table(w, max_ctx, n_pages, dev)
            elif args.paged == "sequential":
                table = torch.arange(n_pages, dtype=torch.int32, device=dev).reshape(w.batch, -1)
            c = kvq.Cache(cfg, device=dev, k_codebook=inputs["k_codebook"],
                          v_codebook=inputs["v_codebook"], k_scale=inputs["k_scale"],
                          v_scale=inputs["v_scale"], page_table=table)
            c.append(inputs["k"], inputs["v"], stream=stream)
            caches.append(c)
        q = inputs["q"]
        del inputs["k"], inputs["v"]
        if serving:
            steps_tok = [make_step_tokens(w, s, 1, dev) for s in range(W + 2 * K)]
    torch.cuda.synchronize()
    log(f"cache built: {copies} cop{'y' if copies == 1 else 'ies'} x {payload0 / 1e9:.3f} GB payload")

    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    dec_s = [ev() for _ in range(K)]
    dec_e = [ev() for _ in range(K)]
    st_s = [ev() for _ in range(K)]    # whole step (append + decode)
    st_e = [ev() for _ in range(K)]
    flush_step = []                    # the append filled a per-channel key group
    # events around the token-streaming kernel alone (recorded once here so
    # that they exist before their handles go to the library)
    ker_s = [ev() for _ in range(K)]
    ker_e = [ev() for _ in range(K)]
    for e in ker_s + ker_e:
        e.record(stream)
    step_bytes = []

    k_group = w.k.get("group_size", 0) if w.k.get("layout") == "per_channel" else 0

    inst_bytes = []

    def step(i, inst=None):
        """One step; ``inst`` = index of an instrumented step, which records
        HIP events around the whole step, the decode call and the streaming
        kernel."""
        c = caches[i % copies]
        if inst is not None:
            st_s[inst].record(stream)
            dec_s[inst].record(stream)
            kvq.set_decode_events(ker_s[inst], ker_e[inst])
        streamed = c.n_ctx          # tokens the streaming kernel reads (serving: fused steps)
        if serving:
            # one call appends the token and decodes over the cache that holds
            # it; the streaming kernel reads the tokens cached before the step
            # unless the append closes a key group (then append, then decode)
            kn, vn, qn = steps_tok[i]
            fused = kvq.append_decode_fused(cfg, c.n_ctx)
            c.append_decode(kn, vn, qn, out=out, stream=stream)
            if not fused:
                streamed = c.n_ctx
            if inst is not None:
                flush_step.append(bool(k_group) and c.n_ctx % k_group == 0)
        else:
            c.decode(q, out=out, stream=stream)
        if inst is not None:
            dec_e[inst].record(stream)
            st_e[inst].record(stream)
            inst_bytes.append(kvq.cache_bytes(cfg, streamed))
        else:
            step_bytes.append(kvq.cache_bytes(cfg, c.n_ctx))

    settle_calls = settle(args.settle_ms, lambda i: caches[i % copies].decode(q, out=out,
                                                                            stream=stream),
                          stream)
    with torch.cuda.stream(stream):
        for i in range(W):
            step(i)
    torch.cuda.synchronize()
    step_bytes.clear()
    # the timed region: K plain steps
    t_start, t_end = ev(), ev()
    with torch.cuda.stream(stream):
        t_start.record(stream)
        for k in range(K):
            step(W + k)
        t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / K
    bytes_avg = sum(step_bytes) / K
    value = bytes_avg / (ms_step * 1e-3) / 1e9
    # then K instrumented steps for the kernel-level figures (their events
    # would lengthen the timed steps)
    with torch.cuda.stream(stream):
        for k in range(K):
            step(W + K + k, k)
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) for a, b in zip(dec_s, dec_e)]
    ker_ms = sorted(a.elapsed_time(b) for a, b in zip(ker_s, ker_e))
    dec_avg = sum(dec_ms) / K
    ker_avg = sum(ker_ms) / K
    achieved = (sum(inst_bytes) / K) / (ker_avg * 1e-3) / 1e9
    path = kvq.decode_path(cfg)
    kernel = DECODE_KERNELS[path]
    wl = CONFIG_NAME(w)
    traffic = counter_traffic(wl, kernel)
    log(f"{kernel} per instrumented step (us): " + " ".join(f"{a.elapsed_time(b) * 1e3:.0f}"
                                                          for a, b in zip(ker_s, ker_e)))
    log(f"step {ms_step * 1e3:.1f} us, decode call {dec_avg * 1e3:.1f} us, {kernel} avg "
        f"{ker_avg * 1e3:.1f} us (p10 {ker_ms[K // 10] * 1e3:.1f}, p90 {ker_ms[(9 * K) // 10] * 1e3:.1f}), "
        f"{bytes_avg / 1e6:.1f} MB/step -> {achieved:.0f} GB/s ({achieved / PEAK_HBM_GBS:.1%} of peak)")

    cycle = None
    if serving:
        st_ms = [a.elapsed_time(b) for a, b in zip(st_s, st_e)]
        fl = [t for t, f in zip(st_ms, flush_step) if f]
        other = sorted(t for t, f in zip(st_ms, flush_step) if not f)
        cycle = {"key_group_tokens": k_group, "timed_steps": K, "flush_steps": len(fl),
                 "flush_step_us": round(sum(fl) / len(fl) * 1e3, 2) if fl else None,
                 "other_step_us_mean": round(sum(other) / len(other) * 1e3, 2),
                 "other_step_us_p10": round(other[len(other) // 10] * 1e3, 2),
                 "other_step_us_p90": round(other[(9 * len(other)) // 10] * 1e3, 2)}
        log(f"serving cycle: {len(fl)} flush step(s) of {K}: "
            f"{cycle['flush_step_us']} us; other steps {cycle['other_step_us_mean']} us mean")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(w, args.cpu_seconds)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "pct_of_peak_hbm": round(100.0 * value / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-mfma/f32" if path == "mfma" else "f32",
        "data": "synthetic (seeded normal K/V with the workload's outlier structure)",
        "config": {"workload": wl, "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "ctx": w.ctx,
                   "k_format": _fmt(w.k), "v_format": _fmt(w.v),
                   "step": ("append 1 token/sequence + decode (one kvq_append_decode call)"
                            if serving else "decode"),
                   "decode_kernel": kernel, "cache_copies": copies,
                   "paged": ({"pages": n_pages, "page_tokens": 32, "table": args.paged}
                             if args.paged else None),
                   "settle": {"ms": args.settle_ms, "decode_calls": settle_calls}},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic["bytes_per_launch"] if traffic else None,
                     "traffic_source": traffic["source"] if traffic else None,
                     "kernel": kernel, "avg_launch_us": round(ker_avg * 1e3, 2),
                     "decode_call_us": round(dec_avg * 1e3, 2),
                     "algorithmic_bytes_per_launch": int(sum(inst_bytes) / K)},
        "cpu_baseline": cpu,
    }
    if cycle is not None:
        res["serving_cycle"] = cycle
    print(json.dumps(res), flush=True)


def prefill_flops(batch: int, n_q_heads: int, head_dim: int, n_ctx: int, n_q: int) -> int:
    """Algorithmic flops of causal prefill attention: query i of the last n_q
    tokens scores n_ctx - n_q + i + 1 keys (2 d flops each) and sums as many
    values (2 d flops each)."""
    keys = n_q * (n_ctx - n_q + 1) + n_q * (n_q - 1) // 2
    return 4 * head_dim * batch * n_q_heads * keys


def bench_prefill(args, w, dev):
    """Chunked prefill: a step appends one chunk of N tokens (keys and values)
    to a cache of ctx - N tokens and runs causal attention for the chunk's N
    queries over all ctx tokens; the cache is then cut back to ctx - N so
    that every step does the same work (the next append rewrites the same
    rows)."""
    import torch
    from quantized_kv_cache_04_amd import kvq
    from synth import make_prefill_queries
    from synth.workloads import make_inputs

    N, K, W = args.prefill, args.steps, args.warmup
    T = w.ctx
    T0 = T - N
    if not 0 < N <= T:
        print("--prefill N needs 0 < N <= ctx", file=sys.stderr)
        sys.exit(2)
    cfg = kvq.config_from_workload(w, max_ctx=T)
    stream = torch.cuda.Stream()
    wl = f"{CONFIG_NAME(w)}_prefill{N}"
    log(f"workload {wl}: B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} T={T} chunk={N}")
    with torch.cuda.stream(stream):
        inputs = make_inputs(w, dev)
        c = kvq.Cache(cfg, device=dev, k_codebook=inputs["k_codebook"],
                      v_codebook=inputs["v_codebook"], k_scale=inputs["k_scale"],
                      v_scale=inputs["v_scale"])
        if T0:
            c.append(inputs["k"][:, :T0].contiguous(), inputs["v"][:, :T0].contiguous(),
                     stream=stream)
        kc = inputs["k"][:, T0:].contiguous()
        vc = inputs["v"][:, T0:].contiguous()
        del inputs
        q = make_prefill_queries(w, N, dev)
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        c.append(kc, vc, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        c.prefill(q, out=out, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        c.n_ctx = T0

    with torch.cuda.stream(stream):
        for _ in range(W):
            step()
    torch.cuda.synchronize()
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    t_start, t_end = mk(), mk()
    with torch.cuda.stream(stream):
        t_start.record(stream)
        for _ in range(K):
            step()
        t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / K
    evs = [[mk(), mk(), mk()] for _ in range(K)]
    with torch.cuda.stream(stream):
        for k in range(K):
            step(evs[k])
    torch.cuda.synchronize()
    app_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    pre_ms = sorted(e[1].elapsed_time(e[2]) for e in evs)
    app_avg, pre_avg = sum(app_ms) / K, sum(pre_ms) / K
    flops = prefill_flops(w.batch, w.n_q_heads, w.head_dim, T, N)
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (pre_avg * 1e-3) / 1e12
    log(f"step {ms_step * 1e3:.1f} us: append {app_avg * 1e3:.1f} us, prefill attention "
        f"{pre_avg * 1e3:.1f} us (p10 {pre_ms[K // 10] * 1e3:.1f}, p90 {pre_ms[(9 * K) // 10] * 1e3:.1f})"
        f" -> {achieved:.1f} TFLOP/s ({achieved / PEAK_MFMA_F16_TFLOPS:.1%} of the fp16 MFMA peak)")
    res = {
        "metric": PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-mfma/f32",
        "data": "synthetic (seeded normal K/V with the workload's outlier structure)",
        "config": {"workload": wl, "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "ctx": T, "chunk": N,
                   "k_format": _fmt(w.k), "v_format": _fmt(w.v),
                   "step": "append an N-token chunk + causal prefill attention for it"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_MFMA_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_MFMA_F16_TFLOPS, 4),
                     "traffic": None,
                     "kernel": ("pre_codes_kernel" if kvq.prefill_kernel(cfg) == "codes"
                                else "pre_mfma_kernel"),
                     "avg_launch_us": round(pre_avg * 1e3, 2),
                     "append_us": round(app_avg * 1e3, 2),
                     "algorithmic_flops_per_launch": flops},
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def bench_encode(args, w, dev):
    """Bulk encode (the prefill append): a step appends N tokens per sequence
    to an empty cache (the cache is cut back to 0 tokens after each step).
    Bytes per step: the fp16/bf16 keys and values read plus the payload
    written."""
    import torch
    from quantized_kv_cache_04_amd import kvq
    from synth import make_workload
    from synth.workloads import make_inputs

    N, K, W = args.encode, args.steps, args.warmup
    wn = make_workload(w.cfg_id, ctx=N, batch=w.batch, n_kv_heads=w.n_kv_heads, k=w.k, v=w.v)
    cfg = kvq.config_from_workload(wn, max_ctx=N)
    stream = torch.cuda.Stream()
    wl = f"{CONFIG_NAME(w)}_encode{N}"
    with torch.cuda.stream(stream):
        inputs = make_inputs(wn, dev)
        c = kvq.Cache(cfg, device=dev, k_codebook=inputs["k_codebook"],
                      v_codebook=inputs["v_codebook"], k_scale=inputs["k_scale"],
                      v_scale=inputs["v_scale"])
        kin, vin = inputs["k"], inputs["v"]
    torch.cuda.synchronize()

    def step():
        c.n_ctx = 0
        c.append(kin, vin, stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(W):
            step()
    torch.cuda.synchronize()
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    evs = [[mk(), mk()] for _ in range(K)]
    with torch.cuda.stream(stream):
        for e in evs:
            e[0].record(stream)
            step()
            e[1].record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    ms_avg = sum(ms) / K
    in_bytes = 2 * kin.numel() * kin.element_size()
    out_bytes = kvq.cache_bytes(cfg, N)
    gbs = (in_bytes + out_bytes) / (ms_avg * 1e-3) / 1e9
    log(f"{wl}: append of {N} tokens x {wn.batch} sequences: {ms_avg * 1e3:.1f} us "
        f"(p10 {ms[K // 10] * 1e3:.1f}, p90 {ms[(9 * K) // 10] * 1e3:.1f}); "
        f"{in_bytes / 1e6:.1f} MB in + {out_bytes / 1e6:.1f} MB out -> {gbs:.0f} GB/s "
        f"({gbs / PEAK_HBM_GBS:.1%} of peak)")
    print(json.dumps({
        "metric": "bulk encode (append) GB/s: K/V read + payload written", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms_avg, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded normal K/V with the workload's outlier structure)",
        "config": {"workload": wl, "batch": wn.batch, "n_kv_heads": wn.n_kv_heads, "tokens": N,
                   "k_format": _fmt(wn.k), "v_format": _fmt(wn.v)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "encode launches of one append", "bytes_per_step": in_bytes + out_bytes},
        "cpu_baseline": None}), flush=True)


def CONFIG_NAME(w) -> str:
    from synth.workloads import CONFIGS
    name = CONFIGS[w.cfg_id]["name"] + (f"_t{w.ctx}" if w.cfg_id == 2 else "")
    if w.k["quantizer"] == "fp8_e5m2" and CONFIGS[w.cfg_id]["k"]["quantizer"] != "fp8_e5m2":
        name += "_fp8e5m2"
    if PAGED:
        name += "_paged"
    return name


PAGED = any(a.startswith("--paged") for a in sys.argv)


def _fmt(f) -> str:
    s = f"{f['quantizer']}-{f['bits']}bit"
    if f.get("group_size"):
        s += f"-{f.get('layout', 'per_token')}-g{f['group_size']}"
    if f.get("outlier_frac"):
        s += f"-outliers{f['outlier_frac']}"
    return s


if __name__ == "__main__":
    main()
