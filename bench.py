"""Benchmark: GQA decode (headline) and causal GQA prefill on one MI355X.

Prints ONE JSON line. A step is one gqa_decode call (the split kernel and the
log-sum-exp merge kernel) on the ragged Llama-2-70B-shaped decode batch
(B=64, H=64, G=8, d_h=128, lengths uniform in [1024, 8192], bf16), the
largest decode workload that fits one GPU; `value` is its whole-job
throughput in GB/s of algorithmic bytes (the K/V cache positions read, q
read, out written, seqlens) over the wall-clock time of the timed steps.

Every other decode workload is measured in the same run under "decode":
the same batch at G=1 (multi-query) and G=64 (multi-head) with the same
seqlens and q (bytes scale with G), the 131072-token single sequence that
exercises the split and merge, and the Llama-3-8B layer (B=16, H=32, G=8,
context 4096). Causal prefill (B=4, T=8192, H=32, G=8, d_h=128) is reported
under "prefill" in TFLOP/s (2*B*H*T^2*d_h per call) against the dense bf16
MFMA peak, and "next" times the adjacent rows (fused append, sliding
windows, fp16, weighted pooling). "copy_ceiling" measures plain streaming
read and copy kernels over 1 GiB as the practical bandwidth ceiling next to
the 8 TB/s peak, and each decode workload's roofline carries "plain_read",
the same plain read over that workload's bytes and input rotation.
"gemm_ceiling" is its matrix-core counterpart: a plain library bf16 GEMM
(torch.matmul, 8192^3) timed like the prefill, whose rate the prefill
roofline's "of_gemm_ceiling" compares against.

Inputs are synthetic (seeded N(0,1), no datasets or weights) and resident in
HBM before timing starts. A workload whose cache is below 1 GiB rotates
through input copies that together exceed 1 GiB (same seqlens in every copy),
so no call finds its cache in the 256 MB MALL left warm by the call before.

roofline: mean launch time from one HIP event pair recorded on the stream the
kernels run on (torch's current stream, which the library is handed) around
the timed calls, after W warmup calls and a time-based settle of at least
--settle-ms of the same calls (the GPU runs a short burst of work slower than
sustained work); the spread of single calls comes from a separate pass that
brackets every 4th call with its own events. traffic: HBM bytes per call from
the committed rocprofv3 counter summaries in profiles/, reported only while
they were taken on the current kernel source.
cpu_baseline: the fp64 CPU oracle timed on the host cores on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, published (256 CU x 2.4 GHz x 4096 FLOP/clk)
METRIC = "GQA decode HBM GB/s (% of peak) + causal prefill TFLOP/s (% MFMA peak), bf16"
HEADLINE = "decode_llama2_70b_ragged"
PREFILL_WORKLOAD = "prefill_llama3_8b_causal"
ROTATE_BYTES = 1 << 30  # rotate input copies until the cache working set exceeds this

# (key, workload in inputs.WORKLOADS, G override or None)
DECODE_CONFIGS = [
    ("decode_llama2_70b_ragged", "decode_llama2_70b_ragged", None),
    ("decode_llama2_70b_ragged_G1", "decode_llama2_70b_ragged", 1),
    ("decode_llama2_70b_ragged_G64", "decode_llama2_70b_ragged", 64),
    ("decode_long_128k", "decode_long_128k", None),
    ("decode_llama3_8b", "decode_llama3_8b", None),
]

# rocprofv3 FETCH_SIZE / WRITE_SIZE summaries, one per timed workload
TRAFFIC_PROFILES = {key: f"{key}_hbm_counters.md" for key, _, _ in DECODE_CONFIGS}
TRAFFIC_PROFILES[PREFILL_WORKLOAD] = "prefill_b4_t8192_hbm_counters.md"
DECODE_SOURCES = ["grouped_query_kv_gqa_amd/csrc/decode.hip", "grouped_query_kv_gqa_amd/csrc/device_common.h",
                  "grouped_query_kv_gqa_amd/csrc/plan.h", "grouped_query_kv_gqa_amd/csrc/plan.cpp"]
PREFILL_SOURCES = ["grouped_query_kv_gqa_amd/csrc/prefill.hip", "grouped_query_kv_gqa_amd/csrc/device_common.h"]


def source_hash(paths) -> str:
    """Hash of kernel sources without comments and blank lines, so that a
    comment edit does not mark the committed counters as taken on other code."""
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(line.rstrip() for line in text.splitlines() if line.strip()).encode())
    return h.hexdigest()[:16]


def measured_traffic(key: str):
    """HBM bytes per call from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on other kernel source."""
    path = os.path.join(ROOT, "profiles", TRAFFIC_PROFILES[key])
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    srcs = PREFILL_SOURCES if key == PREFILL_WORKLOAD else DECODE_SOURCES
    if d.get("source_hash") != source_hash(srcs):
        return None
    return d.get("hbm_bytes_per_launch")


def decode_bytes(w, seqlens) -> int:
    """Algorithmic bytes of one decode call: the K/V positions read, q, out
    and seqlens (split workspace traffic excluded)."""
    e = 4 if str(w.dtype).endswith("float32") else 2
    L = [min(max(int(x), 0), w.Tmax) for x in seqlens]
    return sum(L) * w.G * w.D * 2 * e + 2 * w.B * w.H * w.D * e + 4 * w.B


def prefill_flops(w) -> int:
    return 2 * w.B * w.H * w.T * w.T * w.D


def pct(xs, q):
    return xs[min(len(xs) - 1, int(q * len(xs)))]


def timed_calls(fn, steps, warmup, settle_ms, stream, every=4):
    """W warmup calls, then further calls until at least `settle_ms` of
    back-to-back work has run, then `steps` timed calls: wall-clock around
    all of them (synchronised on both sides) and one HIP event pair on
    `stream` around the same region, whose elapsed time divided by `steps` is
    the mean call duration. A second, separate pass brackets every `every`-th
    call with its own event pair for the spread of single calls (an event
    pair costs a short call a microsecond or two, so it never sits inside the
    timed region). Returns (wall_s, mean_ms, sampled_ms, settle_calls)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    settle = 0
    t_end = time.perf_counter() + settle_ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn(settle)
            settle += 1
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_ms = e0.elapsed_time(e1) / steps
    sampled = [i for i in range(steps) if i % every == every // 2] or [0]
    ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in sampled}
    for i in range(steps):
        e = ev.get(i)
        if e:
            e[0].record(stream)
        fn(i)
        if e:
            e[1].record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev.values())
    return wall, mean_ms, per, settle


def decode_workload(name, G):
    from grouped_query_kv_gqa_amd import inputs as I
    base = I.WORKLOADS[name]
    return base if G is None or G == base.G else base.with_G(G)


def make_decode_inputs(w, seed):
    """Input copies for rotation: copy 0 from `seed`; further copies keep its
    seqlens (so every call reads the same bytes) and redraw q, K and V."""
    from grouped_query_kv_gqa_amd import inputs as I
    x0 = I.decode_inputs(w, seed=seed, device="cuda")
    lens = x0["seqlens"].cpu().tolist()
    cache_bytes = decode_bytes(w, lens)
    ncopy = 1
    while cache_bytes * ncopy <= ROTATE_BYTES:
        ncopy += 1
    xs = [x0] + [I.decode_inputs(w, seed=seed + 1000 * c, device="cuda", seqlens=lens) for c in range(1, ncopy)]
    return xs, lens


def run_decode(key, w, args, steps, warmup):
    import torch
    import grouped_query_kv_gqa_amd as gq

    xs, lens = make_decode_inputs(w, args.seed)
    ncopy = len(xs)
    outs = [torch.empty_like(x["q"]) for x in xs]
    stream = torch.cuda.current_stream()
    byts = decode_bytes(w, lens)

    def step(i):
        x = xs[i % ncopy]
        gq.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=w.scale, out=outs[i % ncopy])

    wall, mean_ms, per, settle = timed_calls(step, steps, warmup, args.settle_ms, stream)
    gbs = byts / (mean_ms * 1e-3) / 1e9
    plan = gq.decode_plan(w.B, w.H, w.G, w.D, w.Tmax)
    entry = {
        "workload": key, "B": w.B, "H": w.H, "G": w.G, "d_h": w.D, "Tmax": w.Tmax, "dtype": "bf16",
        "sum_L": int(sum(min(max(int(L), 0), w.Tmax) for L in lens)), "seed": args.seed,
        "input_copies": ncopy, "steps": steps, "warmup": warmup, "settle_calls": settle,
        "value": round(byts * steps / wall / 1e9, 2), "unit": "GB/s",
        "ms_per_step": round(wall / steps * 1e3, 5),
        "split_plan": {"chunk_tokens": plan[0], "workgroups": plan[1]},
        "roofline": {
            "kernel": "decode_split_kernel+decode_merge_kernel", "bound": "hbm", "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(key), "algorithmic_bytes_per_launch": byts,
            "launch_ms": {"mean": round(mean_ms, 5), "of_steps": steps,
                          "single_launches": {"sampled": len(per), "median": round(pct(per, 0.5), 5),
                                              "p10": round(pct(per, 0.1), 5), "p90": round(pct(per, 0.9), 5)}},
        },
    }
    if not args.no_plain_read:
        rc = plain_read(byts, ncopy, args)
        rc["decode_over_plain_read"] = round(gbs / rc["GBs"], 4)
        entry["roofline"]["plain_read"] = rc
    return entry, xs[0], wall


def run_prefill(args):
    import torch
    import grouped_query_kv_gqa_amd as gq
    from grouped_query_kv_gqa_amd import inputs as I

    w = I.PREFILL_WORKLOADS[PREFILL_WORKLOAD]
    x = I.prefill_inputs(w, seed=args.seed, device="cuda")
    out = torch.empty_like(x["q"])
    stream = torch.cuda.current_stream()

    def step(i):
        gq.prefill(x["q"], x["k"], x["v"], causal=True, out=out)

    steps = args.prefill_steps
    wall, mean_ms, per, settle = timed_calls(step, steps, args.prefill_warmup, args.settle_ms, stream, every=1)
    flops = prefill_flops(w)
    tf = flops / (mean_ms * 1e-3) / 1e12
    entry = {
        "workload": w.name, "B": w.B, "T": w.T, "H": w.H, "G": w.G, "d_h": w.D, "causal": True, "dtype": "bf16",
        "value": round(flops * steps / wall / 1e12, 3), "unit": "TFLOP/s", "steps": steps,
        "warmup": args.prefill_warmup, "settle_calls": settle, "ms_per_step": round(wall / steps * 1e3, 4),
        "roofline": {"kernel": "prefill_mfma_kernel", "bound": "mfma", "achieved": round(tf, 3),
                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 5),
                     "traffic": measured_traffic(PREFILL_WORKLOAD), "flops_per_launch": flops,
                     "launch_ms": {"mean": round(mean_ms, 4), "median": round(pct(per, 0.5), 4),
                                   "p10": round(pct(per, 0.1), 4), "p90": round(pct(per, 0.9), 4)}},
    }
    return entry, x


_PROBE = None


def _probe_lib():
    global _PROBE
    if _PROBE is None:
        import ctypes
        from grouped_query_kv_gqa_amd import build as gbuild
        lib = ctypes.CDLL(gbuild.PROBE_LIB)
        lib.gqa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.gqa_probe_read_wide.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        lib.gqa_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.gqa_probe_read.restype = lib.gqa_probe_read_wide.restype = lib.gqa_probe_copy.restype = ctypes.c_int
        lib.gqa_probe_threads.restype = ctypes.c_int
        _PROBE = lib
    return _PROBE


def plain_read(nbytes: int, copies: int, args, steps: int = 200):
    """A reference at one workload's size: the probe's plain nontemporal
    streaming read of the same byte count (rounded up to 32 KiB), rotating
    through as many buffers as the workload has input copies, timed like the
    workload (warmup, settle, one event pair around `steps` reads). The read
    is the probe's faster one (one 8-wave workgroup per compute unit, 128 KiB
    per workgroup in flight); a reference, not a bound."""
    import torch
    lib = _probe_lib()
    n = (nbytes + 32767) // 32768 * 32768
    bufs = [torch.ones(n // 4, dtype=torch.int32, device="cuda") for _ in range(copies)]
    sink = torch.empty(lib.gqa_probe_threads(), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def read(i):
        if lib.gqa_probe_read_wide(bufs[i % copies].data_ptr(), n, sink.data_ptr(), stream.cuda_stream) != 0:
            raise RuntimeError("bandwidth probe failed")

    _, mean_ms, _, _ = timed_calls(read, steps, 10, args.settle_ms, stream)
    del bufs, sink
    torch.cuda.empty_cache()
    gbs = nbytes / (mean_ms * 1e-3) / 1e9
    return {"kernel": "plain nontemporal streaming read of the same bytes, same rotation "
                      "(256 workgroups x 512 threads, 16 loads of 16 bytes in flight per thread)",
            "us": round(mean_ms * 1e3, 2), "GBs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def copy_ceiling(args):
    """Practical HBM ceiling: plain streaming kernels (libgqa_probe.so) over a
    1 GiB buffer: 2048 workgroups of 256 threads with four 16-byte loads in
    flight per thread, reading with the default and the nontemporal cache
    policy, and copying (2 GiB moved); and the wide read, 256 workgroups of
    512 threads with sixteen nontemporal loads in flight per thread. Best and
    median of 10 event-timed calls after 3 warmup calls."""
    import torch

    lib = _probe_lib()
    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    sink = torch.empty(lib.gqa_probe_threads(), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def call(rc):
        if rc != 0:
            raise RuntimeError(f"bandwidth probe failed ({rc})")

    def timed(fn, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        return ts[0], ts[len(ts) // 2]

    res = {"bytes": n, "peak_GBs": HBM_PEAK_GBS,
           "kernel": "plain streaming read / copy, 2048 workgroups x 256 threads, 16-byte loads; "
                     "read_wide: 256 workgroups x 512 threads, 16 nontemporal loads in flight per thread"}
    for name, fn, moved in [
        ("read", lambda: call(lib.gqa_probe_read(a.data_ptr(), n, 0, sink.data_ptr(), stream.cuda_stream)), n),
        ("read_nt", lambda: call(lib.gqa_probe_read(a.data_ptr(), n, 1, sink.data_ptr(), stream.cuda_stream)), n),
        ("read_wide", lambda: call(lib.gqa_probe_read_wide(a.data_ptr(), n, sink.data_ptr(), stream.cuda_stream)), n),
        ("copy", lambda: call(lib.gqa_probe_copy(b.data_ptr(), a.data_ptr(), n, stream.cuda_stream)), 2 * n),
    ]:
        best, med = timed(fn)
        res[f"{name}_GBs"] = round(moved / (best * 1e-3) / 1e9, 1)
        res[f"{name}_GBs_median"] = round(moved / (med * 1e-3) / 1e9, 1)
    del a, b, sink
    torch.cuda.empty_cache()
    return res


def gemm_ceiling(args):
    """Practical matrix-core ceiling, the counterpart of the copy ceiling: a
    plain library GEMM (torch.matmul on bf16, served by hipBLASLt), C = A B
    with M = N = K = 8192 (1.1 TFLOP per call), both operands contiguous.
    Timed like the prefill: warmup, the settle period (the clock falls under
    sustained matrix-core load), then event-timed calls. A reference for
    what the chip sustains on a dense bf16 contraction, not a bound."""
    import torch

    n = 8192
    g = torch.Generator(device="cuda").manual_seed(args.seed + 7)
    a = torch.randn(n, n, device="cuda", dtype=torch.float32, generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.float32, generator=g).to(torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)

    def step(i):
        torch.matmul(a, b, out=c)

    steps = 20
    _, mean_ms, per, settle = timed_calls(step, steps, 3, args.settle_ms, torch.cuda.current_stream(), every=2)
    flops = 2 * n ** 3
    tf = flops / (mean_ms * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"kernel": "torch.matmul bf16 (hipBLASLt), M = N = K = 8192, contiguous operands",
            "flops_per_call": flops, "steps": steps, "settle_calls": settle, "ms_per_call": round(mean_ms, 4),
            "TFLOPs": round(tf, 1), "peak_TFLOPs": BF16_MFMA_PEAK_TFLOPS,
            "frac_of_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4)}


def _time_calls(fn, steps, warmup, settle_ms=0.0):
    """Mean milliseconds per call: HIP events on the current stream around
    `steps` back-to-back calls after `warmup` untimed ones and a settle."""
    import torch
    _, mean_ms, _, _ = timed_calls(fn, steps, warmup, settle_ms, torch.cuda.current_stream(), every=steps + 1)
    return mean_ms


def _hbm_entry(byts, ms, cfg):
    gbs = byts / (ms * 1e-3) / 1e9
    return {"value": round(gbs, 2), "unit": "GB/s", "ms_per_call": round(ms, 5), "config": cfg,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": int(byts)}}


def _mfma_entry(flops, ms, cfg):
    tf = flops / (ms * 1e-3) / 1e12
    return {"value": round(tf, 3), "unit": "TFLOP/s", "ms_per_call": round(ms, 4), "config": cfg,
            "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": BF16_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 5),
                         "flops_per_launch": int(flops)}}


NEXT_KEYS = ["decode_append", "decode_window", "decode_fp16", "prefill_window", "prefill_fp16", "weighted_pool"]


def run_next(args, only=None):
    """The adjacent rows built after the hot path, each timed on its own
    workload: fused append + decode, sliding-window decode and prefill, fp16
    storage, weighted group pooling (all of them, or the one named `only`).
    Every input is resident before timing."""
    import torch
    import grouped_query_kv_gqa_amd as gq
    from grouped_query_kv_gqa_amd import inputs as I

    res = {}
    settle = args.settle_ms / 2
    ncopy = 4
    if only in (None, "decode_append"):
        res.update(_next_decode_append(args, gq, I, torch, settle, ncopy))
    if only in (None, "decode_window"):
        res.update(_next_decode_window(args, gq, I, torch, settle))
    if only in (None, "decode_fp16"):
        res.update(_next_decode_fp16(args, gq, I, torch, settle, ncopy))
    if only in (None, "prefill_window"):
        res.update(_next_prefill_window(args, gq, I, torch, settle))
    if only in (None, "prefill_fp16"):
        res.update(_next_prefill_fp16(args, gq, I, torch, settle))
    if only in (None, "weighted_pool"):
        res.update(_next_weighted_pool(args, gq, I, torch, settle, ncopy))
    return res


def _next_decode_append(args, gq, I, torch, settle, ncopy):
    """Fused cache append + decode: the Llama-3-8B layer, every cache one
    short of full, so each call writes position 4095 and attends over 4096."""
    res = {}
    w = I.WORKLOADS["decode_llama3_8b"]
    xs = [I.decode_inputs(w, seed=args.seed + c, device="cuda", seqlens=[w.Tmax - 1] * w.B) for c in range(ncopy)]
    kn = I.random_tensor((w.B, w.G, w.D), seed=args.seed + 50, dtype=w.dtype, device="cuda")
    vn = I.random_tensor((w.B, w.G, w.D), seed=args.seed + 51, dtype=w.dtype, device="cuda")
    outs = [torch.empty_like(x["q"]) for x in xs]

    def app(i):
        x = xs[i % ncopy]
        gq.decode_step(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=w.scale, k_new=kn, v_new=vn,
                       out=outs[i % ncopy])
    ms = _time_calls(app, args.next_steps, 5, settle)
    e = 2
    row = w.G * w.D * e
    byts = w.B * (w.Tmax - 1) * row * 2 + w.B * row * 2 * 2 + 2 * w.B * w.H * w.D * e + 4 * w.B
    res["decode_append"] = _hbm_entry(byts, ms, {
        "workload": "decode_llama3_8b, caches at 4095 of 4096, append + attend over 4096", "B": w.B, "H": w.H,
        "G": w.G, "d_h": w.D, "dtype": "bf16", "input_copies": ncopy})
    del xs, outs
    return res


def _next_decode_window(args, gq, I, torch, settle):
    """Sliding-window decode: the ragged Llama-2-70B batch (B=64, lengths
    1024..8192) with a 4096-position window (0.88 GB read: not rotated)."""
    res = {}
    w = I.WORKLOADS["decode_llama2_70b_ragged"]
    W = 4096
    x = I.decode_inputs(w, seed=args.seed, device="cuda")
    out = torch.empty_like(x["q"])
    ms = _time_calls(lambda i: gq.decode_step(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=w.scale,
                                              window=W, out=out), args.next_steps, 5, settle)
    seen = sum(min(min(max(int(L), 0), w.Tmax), W) for L in x["seqlens"].cpu().tolist())
    byts = seen * w.G * w.D * 2 * 2 + 2 * w.B * w.H * w.D * 2 + 4 * w.B
    res["decode_window"] = _hbm_entry(byts, ms, {
        "workload": "decode_llama2_70b_ragged with a 4096-position window", "B": w.B, "H": w.H, "G": w.G,
        "d_h": w.D, "context": w.Tmax, "window": W, "dtype": "bf16"})
    del x
    return res


def _next_decode_fp16(args, gq, I, torch, settle, ncopy):
    """fp16 decode on the Llama-3-8B layer."""
    res = {}
    base = I.WORKLOADS["decode_llama3_8b"]
    w = I.DecodeWorkload(base.name + "_fp16", base.B, base.H, base.G, base.D, base.Tmax, torch.float16)
    xs = [I.decode_inputs(w, seed=args.seed + c, device="cuda") for c in range(ncopy)]
    outs = [torch.empty_like(x["q"]) for x in xs]

    def dec16(i):
        x = xs[i % ncopy]
        gq.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=w.scale, out=outs[i % ncopy])
    ms = _time_calls(dec16, args.next_steps, 5, settle)
    res["decode_fp16"] = _hbm_entry(decode_bytes(w, [w.Tmax] * w.B), ms, {
        "workload": "decode_llama3_8b with fp16 storage", "B": w.B, "H": w.H, "G": w.G, "d_h": w.D,
        "context": w.Tmax, "dtype": "fp16", "input_copies": ncopy})
    del xs, outs
    return res


def _next_prefill_window(args, gq, I, torch, settle):
    """Causal prefill with a 4096-position sliding window (bf16)."""
    res = {}
    pw = I.PREFILL_WORKLOADS[PREFILL_WORKLOAD]
    x = I.prefill_inputs(pw, seed=args.seed, device="cuda")
    out = torch.empty_like(x["q"])
    W = 4096
    ms = _time_calls(lambda i: gq.prefill(x["q"], x["k"], x["v"], causal=True, window=W, out=out),
                     max(2, args.prefill_steps // 2), 1, settle)
    pairs = sum(min(t + 1, W) for t in range(pw.T))
    res["prefill_window"] = _mfma_entry(4 * pw.B * pw.H * pw.D * pairs, ms, {
        "workload": "prefill_llama3_8b_causal with a 4096-position window", "B": pw.B, "T": pw.T, "H": pw.H,
        "G": pw.G, "d_h": pw.D, "window": W, "dtype": "bf16",
        "flops": "4*B*H*d_h*sum_t min(t+1, window)"})
    del x, out
    return res


def _next_prefill_fp16(args, gq, I, torch, settle):
    """Plain causal prefill with fp16 storage."""
    res = {}
    pw = I.PREFILL_WORKLOADS[PREFILL_WORKLOAD]
    w16 = I.PrefillWorkload(pw.name + "_fp16", pw.B, pw.T, pw.H, pw.G, pw.D, torch.float16, True)
    x = I.prefill_inputs(w16, seed=args.seed, device="cuda")
    out = torch.empty_like(x["q"])
    ms = _time_calls(lambda i: gq.prefill(x["q"], x["k"], x["v"], causal=True, out=out),
                     max(2, args.prefill_steps // 2), 1, settle)
    res["prefill_fp16"] = _mfma_entry(prefill_flops(w16), ms, {
        "workload": "prefill_llama3_8b_causal with fp16 storage", "B": pw.B, "T": pw.T, "H": pw.H, "G": pw.G,
        "d_h": pw.D, "dtype": "fp16", "peak": "fp16 dense MFMA peak equals bf16"})
    del x, out
    return res


def _next_weighted_pool(args, gq, I, torch, settle, ncopy):
    """Weighted group pooling of a Llama-2-70B key projection viewed as
    [d, H, d_h]; 4 input copies (537 MB) rotate so that no call reads its
    input from the MALL."""
    res = {}
    N, H, G, D = 8192, 64, 8, 128
    xins = [I.mean_pool_inputs(N, H, D, dtype=torch.bfloat16, seed=args.seed + c, device="cuda")
            for c in range(ncopy)]
    wts = I.random_tensor((H,), seed=args.seed + 3, dtype=torch.float32, device="cuda")
    out = torch.empty((N, G, D), dtype=torch.bfloat16, device="cuda")
    ms = _time_calls(lambda i: gq.weighted_pool_kv(xins[i % ncopy], wts, G, out=out), args.next_steps, 5, settle)
    res["weighted_pool"] = _hbm_entry(N * H * D * 2 + N * G * D * 2 + 4 * H, ms, {
        "workload": "Llama-2-70B W_K as [8192, 64, 128] -> [8192, 8, 128], 4 input copies rotated",
        "dtype": "bf16"})
    del xins
    return res


def cpu_baseline_decode(w, x, budget_s, max_seqs=None):
    """The fp64 oracle over whole sequences of the decode workload (all of
    them, or the first `max_seqs`), repeated until about `budget_s` seconds;
    GB/s of algorithmic bytes."""
    import numpy as np
    import oracle as O

    cores = len(os.sched_getaffinity(0))
    O.set_threads(cores)
    sl = x["seqlens"].cpu()
    n = w.B if max_seqs is None else min(w.B, max_seqs)
    lens = [min(max(int(L), 0), w.Tmax) for L in sl.tolist()[:n]]
    Lmax = max(max(lens), 1)
    q = x["q"][:n].cpu()
    k = x["k_cache"][:n, :Lmax].cpu()
    v = x["v_cache"][:n, :Lmax].cpu()
    sln = np.array(lens, dtype=np.int32)
    byts = sum(lens) * w.G * w.D * 2 * 2 + 2 * n * w.H * w.D * 2 + 4 * n
    t0 = time.perf_counter()
    reps = 0
    while True:
        O.decode(q, k, v, sln, w.scale)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    what = "whole workload" if n == w.B else f"first {n} of {w.B} sequences"
    return {"value": round(byts * reps / dt / 1e9, 3), "unit": "GB/s", "cores": O.max_threads(), "kind": "oracle",
            "sample": f"{what} of {w.name} (B={w.B}, H={w.H}, G={w.G}, d_h={w.D}, sum_L={sum(lens)}) "
                      f"x{reps} in {dt:.1f} s, fp64"}


def cpu_baseline_prefill(w, x, budget_s):
    """The oracle on random late rows of the prefill workload (the most
    expensive rows), until about `budget_s` seconds; TFLOP/s counting
    4*(t+1)*d_h per row."""
    import numpy as np
    import oracle as O

    q, k, v = (x[n].cpu() for n in ("q", "k", "v"))
    rng = np.random.default_rng(0)
    done_flops, t0, rows = 0, time.perf_counter(), 0
    while time.perf_counter() - t0 < budget_s:
        n = 256
        rb = rng.integers(0, w.B, n)
        rt = rng.integers(w.T // 2, w.T, n)
        rh = rng.integers(0, w.H, n)
        O.prefill(q, k, v, causal=True, rows=(rb, rt, rh))
        done_flops += int(sum(4 * (int(t) + 1) * w.D for t in rt))
        rows += n
    dt = time.perf_counter() - t0
    return {"value": round(done_flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": O.max_threads(),
            "kind": "oracle",
            "sample": f"{rows} random causal rows with t in [T/2, T) of {w.name} in {dt:.1f} s, fp64"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed calls of the headline workload")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="after the warmup calls, keep calling for at least this long before timing")
    # 200 calls: the host's latency in launching the first call of the timed
    # region (the GPU idles until it arrives) stays under 1% of a 38 us call
    ap.add_argument("--no-plain-read", action="store_true",
                    help="skip the plain read of each decode workload's bytes (a reference at its size)")
    ap.add_argument("--config-steps", type=int, default=200, help="timed calls of every other decode workload")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--prefill-warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--only", default=None,
                    help="run one workload only (a decode key, 'prefill', or next:<key> for an adjacent "
                         "row), e.g. under a profiler")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds for the headline CPU baseline")
    ap.add_argument("--cpu-budget-other", type=float, default=2.0, help="seconds per other CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-next", action="store_true", help="skip the adjacent rows (append, windows, fp16, pooling)")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--next-steps", type=int, default=50)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device-to-device copy (for HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the decode and prefill kernels run on one GPU's share and no multi-GPU path exists",
              file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)

    if args.copy_calibration:
        a = torch.empty(1 << 29, dtype=torch.int16, device="cuda")  # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if args.only:
        keys = {k for k, _, _ in DECODE_CONFIGS}
        if args.only == "prefill":
            entry, _ = run_prefill(args)
        elif args.only in keys:
            key, name, G = next(c for c in DECODE_CONFIGS if c[0] == args.only)
            entry, _, _ = run_decode(key, decode_workload(name, G), args, args.steps, args.warmup)
        elif args.only.startswith("next:") and args.only[5:] in NEXT_KEYS:
            entry = run_next(args, only=args.only[5:])[args.only[5:]]
        else:
            sys.exit(f"--only: one of {sorted(keys) + ['prefill'] + ['next:' + k for k in NEXT_KEYS]}")
        print(json.dumps({"only": args.only, **entry}), flush=True)
        return

    decode = {}
    head_inputs = None
    for key, name, G in DECODE_CONFIGS:
        w = decode_workload(name, G)
        headline = key == HEADLINE
        steps, warmup = (args.steps, args.warmup) if headline else (args.config_steps, args.warmup)
        entry, x0, wall = run_decode(key, w, args, steps, warmup)
        if not args.no_cpu_baseline:
            if headline:
                head_inputs = (w, x0)  # timed last, after every GPU measurement
            else:
                entry["cpu_baseline"] = cpu_baseline_decode(w, x0, args.cpu_budget_other,
                                                            max_seqs=8 if w.G >= 64 else None)
        decode[key] = entry
        del x0
        torch.cuda.empty_cache()

    head = decode[HEADLINE]
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "B": head["B"], "H": head["H"], "G": head["G"], "d_h": head["d_h"],
                   "context": "ragged, lengths uniform in [1024, 8192]", "Tmax": head["Tmax"],
                   "sum_L": head["sum_L"], "seed": args.seed, "input_copies": head["input_copies"],
                   "settle_calls": head["settle_calls"], "split_plan": head["split_plan"]},
        "roofline": head["roofline"],
        "decode": {k: v for k, v in decode.items() if k != HEADLINE},
    }
    if not args.no_ceiling:
        line["copy_ceiling"] = copy_ceiling(args)
    pf = None
    if not args.no_prefill:
        pentry, px = run_prefill(args)
        line["prefill"] = pentry
        pf = (pentry, px)
        if not args.no_ceiling:
            gc = gemm_ceiling(args)
            line["gemm_ceiling"] = gc
            pentry["roofline"]["of_gemm_ceiling"] = round(pentry["roofline"]["achieved"] / gc["TFLOPs"], 4)
    if not args.no_next:
        line["next"] = run_next(args)
    if not args.no_cpu_baseline:
        w, x0 = head_inputs
        line["cpu_baseline"] = cpu_baseline_decode(w, x0, args.cpu_budget)
        if pf is not None:
            from grouped_query_kv_gqa_amd import inputs as I
            line["prefill"]["cpu_baseline"] = cpu_baseline_prefill(I.PREFILL_WORKLOADS[PREFILL_WORKLOAD], pf[1],
                                                                   args.cpu_budget_other * 2)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
