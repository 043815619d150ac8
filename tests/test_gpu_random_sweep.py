"""Seeded random sweep of the HIP path against the fp64 oracle.

Fixed-seed draws of shapes, dtypes and options that the hand-picked parity
cases do not line up on purpose (plus a few larger draws, caches of 1000 to
4000 positions over up to 24 sequences and prompts of 400 to 1100 tokens, so
that sequences fall into many pieces): head/group layouts (MHA, MQA, odd group
sizes), d_h 64 and 128, cache lengths around and away from tile edges,
lengths out of range, appends into full and non-full caches, windows shorter
and longer than the span, caller-fixed split lengths, causal and full
prefill with and without a window, and pooling. Each case is checked to the
same bar as the other parity tests (bf16/fp16: max-abs 2e-2 and rel-L2
5e-3; fp32: max-abs 1e-5; caches after an append bit for bit).
"""
import random

import numpy as np
import pytest
import torch

import grouped_query_kv_gqa_amd as gq
import oracle as O
from grouped_query_kv_gqa_amd import inputs as I
from gpu_util import assert_parity, say, to_host

pytestmark = pytest.mark.gpu

DEV = "cuda"
LAYOUTS = [(8, 8), (8, 2), (16, 4), (32, 8), (64, 8), (64, 1), (24, 3), (12, 6), (40, 5), (16, 16), (48, 1)]
DTYPES = [torch.bfloat16, torch.float16, torch.float32]


def _decode_cases(n, seed=2024, big=False):
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        H, G = rng.choice(LAYOUTS)
        D = rng.choice([64, 128])
        dtype = rng.choice(DTYPES[:2] if big else DTYPES)
        B = rng.randint(4, 24) if big else rng.randint(1, 6)
        Tmax = rng.randint(1000, 4000) if big else rng.randint(1, 300 if dtype == torch.float32 else 700)
        seqlens = []
        for _ in range(B):
            kind = rng.random()
            if kind < 0.15:
                seqlens.append(Tmax)
            elif kind < 0.25:
                seqlens.append(max(0, Tmax - 1))
            elif kind < 0.32:
                seqlens.append(0)
            elif kind < 0.38:
                seqlens.append(rng.choice([-5, Tmax + 9]))
            else:
                seqlens.append(rng.randint(1, Tmax))
        append = rng.random() < 0.5
        window = 0 if rng.random() < 0.5 else rng.randint(1, Tmax + 5)
        split = 0 if rng.random() < 0.6 else rng.choice([32, 64, 96, 32 * rng.randint(1, 12)])
        cases.append((i, B, H, G, D, Tmax, tuple(seqlens), dtype, append, window, split))
    return cases


def _prefill_cases(n, seed=4096, big=False):
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        H, G = rng.choice(LAYOUTS)
        D = rng.choice([64, 128])
        dtype = rng.choice(DTYPES[:2] if big else DTYPES)
        B = rng.randint(1, 2)
        T = rng.randint(400, 1100) if big else rng.randint(1, 120 if dtype == torch.float32 else 333)
        causal = rng.random() < 0.7
        window = rng.randint(1, T + 3) if causal and rng.random() < 0.5 else 0
        cases.append((i, B, T, H, G, D, dtype, causal, window))
    return cases


def _bits(t):
    t = to_host(t)
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype in (torch.bfloat16, torch.float16) else t.numpy()


@pytest.mark.parametrize("case", _decode_cases(40) + [(100 + c[0],) + c[1:] for c in _decode_cases(12, 77, True)],
                         ids=lambda c: f"d{c[0]}")
def test_random_decode_step(case):
    i, B, H, G, D, Tmax, seqlens, dtype, append, window, split = case
    say(f"random decode #{i}: B={B} H={H} G={G} D={D} Tmax={Tmax} seqlens={list(seqlens)} {dtype} "
        f"append={append} window={window} split={split}")
    w = I.DecodeWorkload("rand", B, H, G, D, Tmax, dtype)
    x = I.decode_inputs(w, seed=100 + i, device=DEV, seqlens=list(seqlens))
    kn = I.random_tensor((B, G, D), seed=200 + i, dtype=dtype, device=DEV) if append else None
    vn = I.random_tensor((B, G, D), seed=300 + i, dtype=dtype, device=DEV) if append else None
    ref, k_ref, v_ref = O.decode_step(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]),
                                      to_host(x["seqlens"]), w.scale,
                                      k_new=to_host(kn) if append else None, v_new=to_host(vn) if append else None,
                                      window=window)
    torch.cuda.synchronize()
    out = gq.decode_step(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=w.scale, k_new=kn, v_new=vn,
                         window=window, split_tokens=split)
    torch.cuda.synchronize()
    assert_parity(out, ref, dtype, f"random decode #{i}")
    assert np.array_equal(_bits(x["k_cache"]), k_ref) and np.array_equal(_bits(x["v_cache"]), v_ref), \
        "cache contents after the call"


@pytest.mark.parametrize("case", _prefill_cases(24) + [(100 + c[0],) + c[1:] for c in _prefill_cases(6, 99, True)],
                         ids=lambda c: f"p{c[0]}")
def test_random_prefill(case):
    i, B, T, H, G, D, dtype, causal, window = case
    say(f"random prefill #{i}: B={B} T={T} H={H} G={G} D={D} {dtype} causal={causal} window={window}")
    w = I.PrefillWorkload("rand", B, T, H, G, D, dtype, causal)
    x = I.prefill_inputs(w, seed=500 + i, device=DEV)
    torch.cuda.synchronize()
    out = gq.prefill(x["q"], x["k"], x["v"], causal=causal, window=window)
    torch.cuda.synchronize()
    qh, kh, vh = to_host(x["q"]), to_host(x["k"]), to_host(x["v"])
    ref = O.prefill_window(qh, kh, vh, window) if window > 0 else O.prefill(qh, kh, vh, causal=causal)
    assert_parity(out, ref, dtype, f"random prefill #{i}")


@pytest.mark.parametrize("i", range(10), ids=lambda i: f"m{i}")
def test_random_pool(i):
    rng = random.Random(8000 + i)
    H, G = rng.choice(LAYOUTS)
    D = rng.choice([64, 128])
    dtype = rng.choice(DTYPES)
    N = rng.randint(1, 400)
    weighted = rng.random() < 0.5
    say(f"random pool #{i}: N={N} H={H} G={G} D={D} {dtype} weighted={weighted}")
    x = I.mean_pool_inputs(N, H, D, dtype=dtype, seed=900 + i, device=DEV)
    if not weighted:
        out = gq.mean_pool_kv(x, G)
        torch.cuda.synchronize()
        assert_parity(out, O.mean_pool(to_host(x), G), dtype, f"random mean pool #{i}")
        return
    wts = I.random_tensor((H,), seed=950 + i, dtype=torch.float32, device=DEV)
    out = gq.weighted_pool_kv(x, wts, G)
    torch.cuda.synchronize()
    wh = to_host(wts).double().numpy()
    ref = O.weighted_pool(to_host(x), G, wh)
    # the weighted sums are not bounded by 1, so the bound is relative: one
    # rounding of the fp32 sum to the output type plus the fp32 accumulation
    # error of r terms
    got = out.float().cpu().double().numpy()
    absum = O.weighted_pool(np.abs(to_host(x).double().numpy()), G, np.abs(wh))
    rel = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11, torch.float32: 0.0}[dtype]
    bound = np.abs(ref) * rel + absum * (H // G) * 2.0 ** -23 + 2.0 ** -24
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))


# Two fp32 draws of a wider sweep (128 and 96 heads over 2 groups) whose rows
# came out 1.008e-5 and 1.080e-5 off while the fp32 path kept its scores in
# fp32: at scores near 100 the rounding of the score itself is about 4e-6 in
# the exponent. The fp32 path now keeps scores and the running maximum in fp64.
FP32_LARGE_SCORES = [(96, 1, 117, 128, 2, 64, torch.float32, True, 0),
                     (126, 1, 15, 96, 2, 128, torch.float32, True, 0)]


@pytest.mark.parametrize("case", _prefill_cases(10, seed=555) + [(200 + c[0],) + c[1:] for c in _prefill_cases(2, 556, True)]
                         + FP32_LARGE_SCORES, ids=lambda c: f"q{c[0]}")
def test_random_prefill_large_scores(case):
    """Queries scaled by 8-16 (scores of tens of units, as outlier features
    give): the scale must reach the scores in fp32. (Rounding q*scale to 16
    bits once exceeded the bound here by up to 7x.)"""
    i, B, T, H, G, D, dtype, causal, window = case
    mult = random.Random(7000 + i).choice([8.0, 16.0])
    say(f"large-score prefill #{i}: B={B} T={T} H={H} G={G} D={D} {dtype} causal={causal} window={window} q*{mult}")
    w = I.PrefillWorkload("rand", B, T, H, G, D, dtype, causal)
    x = I.prefill_inputs(w, seed=500 + i, device=DEV)
    x["q"] = (x["q"].float() * mult).to(dtype)
    torch.cuda.synchronize()
    out = gq.prefill(x["q"], x["k"], x["v"], causal=causal, window=window)
    torch.cuda.synchronize()
    qh, kh, vh = to_host(x["q"]), to_host(x["k"]), to_host(x["v"])
    ref = O.prefill_window(qh, kh, vh, window) if window > 0 else O.prefill(qh, kh, vh, causal=causal)
    assert_parity(out, ref, dtype, f"large-score prefill #{i}")


@pytest.mark.parametrize("case", _decode_cases(8, seed=556), ids=lambda c: f"e{c[0]}")
def test_random_decode_large_scores(case):
    i, B, H, G, D, Tmax, seqlens, dtype, append, window, split = case
    mult = random.Random(7100 + i).choice([8.0, 16.0])
    say(f"large-score decode #{i}: B={B} H={H} G={G} D={D} Tmax={Tmax} {dtype} window={window} q*{mult}")
    w = I.DecodeWorkload("rand", B, H, G, D, Tmax, dtype)
    x = I.decode_inputs(w, seed=100 + i, device=DEV, seqlens=list(seqlens))
    x["q"] = (x["q"].float() * mult).to(dtype)
    ref, _, _ = O.decode_step(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]), to_host(x["seqlens"]),
                              w.scale, window=window)
    torch.cuda.synchronize()
    out = gq.decode_step(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=w.scale, window=window,
                         split_tokens=split)
    torch.cuda.synchronize()
    assert_parity(out, ref, dtype, f"large-score decode #{i}")


@pytest.mark.parametrize("B", [64, 65, 128, 129, 300])
@pytest.mark.parametrize("append,window,split", [(False, 0, 0), (True, 0, 0), (True, 37, 0), (False, 0, 64)])
def test_decode_many_sequences(B, append, window, split):
    """More than 64 sequences: the partition, the walk over the sequences and
    the merge go through the lengths 64 at a time."""
    rng = random.Random(B * 7 + window + split)
    Tmax = 200
    seqlens = [rng.choice([0, 1, 31, 32, 33, Tmax, rng.randint(1, Tmax)]) for _ in range(B)]
    say(f"decode with {B} sequences append={append} window={window} split={split}")
    w = I.DecodeWorkload("many", B, 8, 2, 128, Tmax, torch.bfloat16)
    x = I.decode_inputs(w, seed=B, device=DEV, seqlens=seqlens)
    kn = I.random_tensor((B, 2, 128), seed=B + 1, dtype=torch.bfloat16, device=DEV) if append else None
    vn = I.random_tensor((B, 2, 128), seed=B + 2, dtype=torch.bfloat16, device=DEV) if append else None
    ref, k_ref, v_ref = O.decode_step(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]),
                                      to_host(x["seqlens"]), w.scale,
                                      k_new=to_host(kn) if append else None, v_new=to_host(vn) if append else None,
                                      window=window)
    torch.cuda.synchronize()
    out = gq.decode_step(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=w.scale, k_new=kn, v_new=vn,
                         window=window, split_tokens=split)
    torch.cuda.synchronize()
    assert_parity(out, ref, torch.bfloat16, f"{B} sequences")
    assert np.array_equal(_bits(x["k_cache"]), k_ref) and np.array_equal(_bits(x["v_cache"]), v_ref)
