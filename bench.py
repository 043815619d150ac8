"""Benchmark: GQA decode (headline) and causal GQA prefill on one MI355X.

Prints ONE JSON line. A decode step is one gqa_decode call on the
Llama-3-8B-shaped decode layer (B=16, H=32, G=8, d_h=128, every sequence at
context 4096, bf16); `value` is whole-job decode throughput in GB/s of
algorithmic bytes (K/V cache read + q read + out write + seqlens) over the
wall-clock time of the timed steps. Prefill (B=4, T=8192, H=32, G=8,
d_h=128, causal, bf16) is timed the same way and reported under "prefill"
in TFLOP/s (2*B*H*T^2*d_h per call).

Inputs are synthetic (seeded N(0,1), no datasets or weights) and resident in
HBM before timing starts. Decode rotates through 4 input copies (1 GiB of
K/V) so that no step can be served from the 256 MB MALL left warm by the
step before it.

roofline: mean launch time from one HIP event pair recorded on the stream the
kernels run on (torch's current stream, which the library is handed) around
the timed launches; the spread of single launches comes from a separate pass
that brackets every 4th launch (decode) or every launch (prefill).
cpu_baseline: the fp64 CPU oracle timed on the host cores on a bounded
sample of the same workload.
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
DECODE_WORKLOAD = "decode_llama3_8b"
PREFILL_WORKLOAD = "prefill_llama3_8b_causal"
TRAFFIC_PROFILES = {  # rocprofv3 FETCH_SIZE / WRITE_SIZE summaries, one per timed kernel and workload
    "decode": "decode_llama3_8b_hbm_counters.md",
    "prefill": "prefill_b4_t8192_hbm_counters.md",
}
KERNEL_SOURCES = {
    "decode": ["grouped_query_kv_gqa_amd/csrc/decode.hip", "grouped_query_kv_gqa_amd/csrc/device_common.h"],
    "prefill": ["grouped_query_kv_gqa_amd/csrc/prefill.hip", "grouped_query_kv_gqa_amd/csrc/device_common.h"],
}


def source_hash(kind: str) -> str:
    """Hash of the kernel sources without comments and blank lines, so that a
    comment edit does not mark the committed counters as taken on other code."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(line.rstrip() for line in text.splitlines() if line.strip()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kind: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on other kernel source."""
    path = os.path.join(ROOT, "profiles", TRAFFIC_PROFILES[kind])
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("source_hash") != source_hash(kind):
        return None
    return d.get("hbm_bytes_per_launch")


def decode_bytes(w, seqlens) -> int:
    e = 4 if str(w.dtype).endswith("float32") else 2
    L = [min(max(int(x), 0), w.Tmax) for x in seqlens]
    return sum(L) * w.G * w.D * 2 * e + 2 * w.B * w.H * w.D * e + 4 * w.B


def prefill_flops(w) -> int:
    return 2 * w.B * w.H * w.T * w.T * w.D


def timed_launches(fn, steps, warmup, stream, every=1):
    """Warm up, then time `steps` back-to-back launches: wall-clock around
    all of them (synchronised on both sides) and one HIP event pair on
    `stream` around the same region, whose elapsed time divided by `steps` is
    the mean launch duration. A second, separate pass brackets every
    `every`-th launch with its own event pair for the spread of single
    launches (an event pair costs a short launch a microsecond or two, so it
    never sits inside the timed region)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = e0.elapsed_time(e1) / steps
    # every `every`-th launch, and at least one (short runs, e.g. under a profiler)
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
    per = sorted(a.elapsed_time(b) for a, b in ev.values())  # ms
    return wall, region_ms, per


def pct(xs, q):
    return xs[min(len(xs) - 1, int(q * len(xs)))]


def run_decode(args):
    import torch
    import grouped_query_kv_gqa_amd as gq
    from grouped_query_kv_gqa_amd import inputs as I

    w = I.WORKLOADS[DECODE_WORKLOAD]
    ncopy = 4
    xs = [I.decode_inputs(w, seed=args.seed + c, device="cuda") for c in range(ncopy)]
    outs = [torch.empty_like(x["q"]) for x in xs]
    stream = torch.cuda.current_stream()
    byts = decode_bytes(w, xs[0]["seqlens"].cpu().tolist())

    def step(i):
        x = xs[i % ncopy]
        gq.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=w.scale, out=outs[i % ncopy])

    wall, region_ms, per = timed_launches(step, args.steps, args.warmup, stream, every=4)
    med = pct(per, 0.5)
    res = {
        "w": w, "bytes": byts, "wall": wall, "per_ms": per, "median_ms": med, "mean_ms": region_ms,
        "plan": gq.decode_plan(w.B, w.H, w.G, w.D, w.Tmax),
        "inputs": xs[0],
    }
    return res


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

    wall, region_ms, per = timed_launches(step, args.prefill_steps, args.prefill_warmup, stream)
    return {"w": w, "flops": prefill_flops(w), "wall": wall, "per_ms": per, "median_ms": pct(per, 0.5),
            "mean_ms": region_ms, "inputs": x}


def _time_calls(fn, steps, warmup):
    """Mean milliseconds per call: HIP events on the current stream around
    `steps` back-to-back calls after `warmup` untimed ones."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _hbm_entry(name, byts, ms, cfg):
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


def run_next(args):
    """The adjacent rows built after the hot path, each timed on its own
    workload: fused append + decode, sliding-window decode and prefill, fp16
    storage, weighted group pooling. Every input is resident before timing."""
    import torch
    import grouped_query_kv_gqa_amd as gq
    from grouped_query_kv_gqa_amd import inputs as I

    res = {}
    # fused cache append + decode: the Llama-3-8B layer, every cache one short
    # of full, so each call writes position 4095 and attends over 4096
    w = I.WORKLOADS[DECODE_WORKLOAD]
    ncopy = 4
    xs = [I.decode_inputs(w, seed=args.seed + c, device="cuda", seqlens=[w.Tmax - 1] * w.B) for c in range(ncopy)]
    kn = I.random_tensor((w.B, w.G, w.D), seed=args.seed + 50, dtype=w.dtype, device="cuda")
    vn = I.random_tensor((w.B, w.G, w.D), seed=args.seed + 51, dtype=w.dtype, device="cuda")
    outs = [torch.empty_like(x["q"]) for x in xs]

    def app(i):
        x = xs[i % ncopy]
        gq.decode_step(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=w.scale, k_new=kn, v_new=vn,
                       out=outs[i % ncopy])
    ms = _time_calls(app, args.next_steps, 5)
    e = 2
    row = w.G * w.D * e
    byts = w.B * (w.Tmax - 1) * row * 2 + w.B * row * 2 * 2 + 2 * w.B * w.H * w.D * e + 4 * w.B
    res["decode_append"] = _hbm_entry("decode_append", byts, ms, {
        "workload": "decode_llama3_8b, caches at 4095 of 4096, append + attend over 4096", "B": w.B, "H": w.H,
        "G": w.G, "d_h": w.D, "dtype": "bf16"})
    del xs, outs

    # sliding-window decode: the ragged Llama-2-70B batch (B=64, lengths
    # 1024..8192) with a 4096-position window
    w = I.WORKLOADS["decode_llama2_70b_ragged"]
    W = 4096
    x = I.decode_inputs(w, seed=args.seed, device="cuda")
    out = torch.empty_like(x["q"])
    ms = _time_calls(lambda i: gq.decode_step(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=w.scale,
                                              window=W, out=out), args.next_steps, 5)
    seen = sum(min(min(max(int(L), 0), w.Tmax), W) for L in x["seqlens"].cpu().tolist())
    byts = seen * w.G * w.D * 2 * 2 + 2 * w.B * w.H * w.D * 2 + 4 * w.B
    res["decode_window"] = _hbm_entry("decode_window", byts, ms, {
        "workload": "decode_llama2_70b_ragged with a 4096-position window", "B": w.B, "H": w.H, "G": w.G,
        "d_h": w.D, "context": w.Tmax, "window": W, "dtype": "bf16"})
    del x

    # fp16 decode on the Llama-3-8B layer
    base = I.WORKLOADS[DECODE_WORKLOAD]
    w = I.DecodeWorkload(base.name + "_fp16", base.B, base.H, base.G, base.D, base.Tmax, torch.float16)
    xs = [I.decode_inputs(w, seed=args.seed + c, device="cuda") for c in range(ncopy)]
    outs = [torch.empty_like(x["q"]) for x in xs]

    def dec16(i):
        x = xs[i % ncopy]
        gq.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=w.scale, out=outs[i % ncopy])
    ms = _time_calls(dec16, args.next_steps, 5)
    res["decode_fp16"] = _hbm_entry("decode_fp16", decode_bytes(w, [w.Tmax] * w.B), ms, {
        "workload": "decode_llama3_8b with fp16 storage", "B": w.B, "H": w.H, "G": w.G, "d_h": w.D,
        "context": w.Tmax, "dtype": "fp16"})
    del xs, outs

    # prefill: sliding window 4096 (bf16) and plain causal with fp16 storage
    pw = I.PREFILL_WORKLOADS[PREFILL_WORKLOAD]
    x = I.prefill_inputs(pw, seed=args.seed, device="cuda")
    out = torch.empty_like(x["q"])
    W = 4096
    ms = _time_calls(lambda i: gq.prefill(x["q"], x["k"], x["v"], causal=True, window=W, out=out),
                     max(2, args.prefill_steps // 2), 1)
    pairs = sum(min(t + 1, W) for t in range(pw.T))
    res["prefill_window"] = _mfma_entry(4 * pw.B * pw.H * pw.D * pairs, ms, {
        "workload": "prefill_llama3_8b_causal with a 4096-position window", "B": pw.B, "T": pw.T, "H": pw.H,
        "G": pw.G, "d_h": pw.D, "window": W, "dtype": "bf16",
        "flops": "4*B*H*d_h*sum_t min(t+1, window)"})
    del x, out
    w16 = I.PrefillWorkload(pw.name + "_fp16", pw.B, pw.T, pw.H, pw.G, pw.D, torch.float16, True)
    x = I.prefill_inputs(w16, seed=args.seed, device="cuda")
    out = torch.empty_like(x["q"])
    ms = _time_calls(lambda i: gq.prefill(x["q"], x["k"], x["v"], causal=True, out=out),
                     max(2, args.prefill_steps // 2), 1)
    res["prefill_fp16"] = _mfma_entry(prefill_flops(w16), ms, {
        "workload": "prefill_llama3_8b_causal with fp16 storage", "B": pw.B, "T": pw.T, "H": pw.H, "G": pw.G,
        "d_h": pw.D, "dtype": "fp16", "peak": "fp16 dense MFMA peak equals bf16"})
    del x, out

    # weighted group pooling of a Llama-2-70B key projection viewed as [d, H, d_h];
    # 4 input copies (537 MB) rotate so that no call reads its input from the MALL
    N, H, G, D = 8192, 64, 8, 128
    xins = [I.mean_pool_inputs(N, H, D, dtype=torch.bfloat16, seed=args.seed + c, device="cuda")
            for c in range(ncopy)]
    wts = I.random_tensor((H,), seed=args.seed + 3, dtype=torch.float32, device="cuda")
    out = torch.empty((N, G, D), dtype=torch.bfloat16, device="cuda")
    ms = _time_calls(lambda i: gq.weighted_pool_kv(xins[i % ncopy], wts, G, out=out), args.next_steps, 5)
    res["weighted_pool"] = _hbm_entry("weighted_pool", N * H * D * 2 + N * G * D * 2 + 4 * H, ms, {
        "workload": "Llama-2-70B W_K as [8192, 64, 128] -> [8192, 8, 128], 4 input copies rotated",
        "dtype": "bf16"})
    del xins
    return res


def cpu_baseline_decode(res, budget_s):
    """Oracle over whole sequences of the decode workload, repeated until
    about `budget_s` seconds; GB/s of algorithmic bytes."""
    import numpy as np
    import oracle as O

    w = res["w"]
    x = res["inputs"]
    cores = len(os.sched_getaffinity(0))
    O.set_threads(cores)
    q, k, v, sl = (x[n].cpu() for n in ("q", "k_cache", "v_cache", "seqlens"))
    byts = decode_bytes(w, sl.tolist())
    t0 = time.perf_counter()
    reps = 0
    while True:
        O.decode(q, k, v, sl.numpy(), w.scale)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(byts * reps / dt / 1e9, 3), "unit": "GB/s", "cores": O.max_threads(), "kind": "oracle",
            "sample": f"whole {w.name} workload (B={w.B}, H={w.H}, G={w.G}, d_h={w.D}, L={w.Tmax}) "
                      f"x{reps} in {dt:.1f} s, fp64"}


def cpu_baseline_prefill(res, budget_s):
    """Oracle on late rows of the prefill workload (the most expensive rows),
    until about `budget_s` seconds; TFLOP/s counting 4*(t+1)*d_h per row."""
    import numpy as np
    import oracle as O

    w = res["w"]
    x = res["inputs"]
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
    ap.add_argument("--steps", type=int, default=200)
    # 500 untimed decode calls (about 25 ms): over the first milliseconds of
    # sustained work the GPU is still settling and a call takes about 1 us more
    # (measured: 48.4-48.8 us per call after 20 warmup calls, 47.8 after 500)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--prefill-warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds per CPU-baseline leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-next", action="store_true", help="skip the adjacent rows (append, windows, fp16, pooling)")
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

    dec = run_decode(args)
    w = dec["w"]
    value = dec["bytes"] * args.steps / dec["wall"] / 1e9
    kernel_gbs = dec["bytes"] / (dec["mean_ms"] * 1e-3) / 1e9
    traffic = measured_traffic("decode")
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["wall"] / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "G": w.G, "d_h": w.D, "context": w.Tmax,
                   "seed": args.seed, "input_copies": 4, "split_plan": list(dec["plan"][:2])},
        "roofline": {
            # one gqa_decode call = the split kernel + the merge kernel; the
            # HIP events bracket the timed calls (both kernels and the gaps)
            "kernel": "decode_split_kernel+decode_merge_kernel",
            "bound": "hbm",
            "achieved": round(kernel_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(kernel_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dec["bytes"],
            "launch_ms": {"mean": round(dec["mean_ms"], 5), "of_steps": args.steps,
                          "single_launches": {"sampled": len(dec["per_ms"]), "median": round(dec["median_ms"], 5),
                                              "p10": round(pct(dec["per_ms"], 0.1), 5),
                                              "p90": round(pct(dec["per_ms"], 0.9), 5)}},
        },
    }
    if not args.no_prefill:
        pf = run_prefill(args)
        pw = pf["w"]
        tflops = pf["flops"] / (pf["mean_ms"] * 1e-3) / 1e12
        line["prefill"] = {
            "workload": pw.name, "B": pw.B, "T": pw.T, "H": pw.H, "G": pw.G, "d_h": pw.D, "causal": True,
            "value": round(pf["flops"] * args.prefill_steps / pf["wall"] / 1e12, 3), "unit": "TFLOP/s",
            "steps": args.prefill_steps, "warmup": args.prefill_warmup,
            "ms_per_step": round(pf["wall"] / args.prefill_steps * 1e3, 4),
            "roofline": {"kernel": "prefill_mfma_kernel", "bound": "mfma", "achieved": round(tflops, 3),
                         "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 5),
                         "traffic": measured_traffic("prefill"), "flops_per_launch": pf["flops"],
                         "launch_ms": {"mean": round(pf["mean_ms"], 4), "median": round(pf["median_ms"], 4)}},
        }
    if not args.no_next:
        line["next"] = run_next(args)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(dec, args.cpu_budget)
        if "prefill" in line:
            line["prefill"]["cpu_baseline"] = cpu_baseline_prefill(pf, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
