"""Overrun checks and invariances on the GPU.

* Guard bands: every output (and every cache a decode step writes) is a view
  into a larger buffer whose margins on both sides hold a NaN bit pattern;
  after the call the margins must be bit-identical and the interior (also
  poisoned beforehand) fully written and at oracle parity.
* Reads past the inputs: prefill K/V are views at the end of a larger buffer
  whose tail is NaN; with ragged last tiles (T % 64 in {1, 31, 33, 63}) the
  output must still be finite and at parity (the kernel's ranged loads must
  return zeros past the tensors, not the bytes that follow them).
* Decode is invariant to the order of cache positions within [0, L_b)
  ("Grouped-Query Attention" (llm-arch-kb), section 3: softmax over keys, a
  sum over positions).
"""
import numpy as np
import pytest
import torch

import grouped_query_kv_gqa_amd as gq
import oracle as O
from grouped_query_kv_gqa_amd import inputs as I
from gpu_util import assert_parity, say, to_host

pytestmark = pytest.mark.gpu

DEV = "cuda"
MARGIN = 4096  # elements on each side (8 or 16 KiB)
_POISON = {torch.bfloat16: (torch.int16, 0x7FA5), torch.float16: (torch.int16, 0x7E5A),
           torch.float32: (torch.int32, 0x7FC0DEAD)}


def guarded(shape, dtype):
    """(buffer, view): the view is contiguous, 16-byte aligned, surrounded by
    MARGIN poisoned elements, and poisoned itself."""
    n = int(np.prod(shape))
    ity, pat = _POISON[dtype]
    buf = torch.empty(n + 2 * MARGIN, dtype=dtype, device=DEV)
    buf.view(ity).fill_(pat)
    return buf, buf[MARGIN:MARGIN + n].view(*shape)


def guarded_copy(t):
    buf, view = guarded(tuple(t.shape), t.dtype)
    view.copy_(t)
    return buf, view


def _bits(t):
    """Stored bit patterns of a device tensor or an oracle array."""
    if isinstance(t, torch.Tensor):
        t = to_host(t)
        a = t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()
    else:
        a = np.asarray(t)
    return a.view(np.uint16 if a.dtype.itemsize == 2 else np.uint32)


def margins_intact(buf):
    ity, pat = _POISON[buf.dtype]
    bits = buf.view(ity)
    return bool((bits[:MARGIN] == pat).all()) and bool((bits[-MARGIN:] == pat).all())


@pytest.mark.parametrize("H,G,D,dtype", [(32, 8, 128, torch.bfloat16), (64, 1, 128, torch.bfloat16),
                                         (8, 8, 64, torch.float16), (12, 3, 64, torch.float32)])
@pytest.mark.parametrize("split", [0, 64])
def test_decode_out_guard_bands(H, G, D, dtype, split):
    say(f"decode guard bands H={H} G={G} D={D} {dtype} split={split}")
    B, Tmax = 5, 700
    w = I.DecodeWorkload("guard", B, H, G, D, Tmax, dtype)
    x = I.decode_inputs(w, seed=H + G + split, device=DEV, seqlens=[700, 1, 0, 333, 64])
    buf, out = guarded((B, H, D), dtype)
    torch.cuda.synchronize()
    gq.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=w.scale, out=out, split_tokens=split)
    torch.cuda.synchronize()
    assert margins_intact(buf), "decode wrote outside out"
    ref = O.decode(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]), to_host(x["seqlens"]), w.scale)
    assert_parity(out, ref, dtype, "decode")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("window", [0, 50])
def test_decode_step_guard_bands(dtype, window):
    """The caches are written at one position per sequence: their margins and
    every other position stay as they were."""
    say(f"decode_step guard bands {dtype} window={window}")
    B, H, G, D, Tmax = 4, 16, 4, 128, 300
    w = I.DecodeWorkload("guard_step", B, H, G, D, Tmax, dtype)
    lens = [299, 300, 0, 150]
    x = I.decode_inputs(w, seed=11 + window, device=DEV, seqlens=lens)
    kn = I.random_tensor((B, G, D), seed=12, dtype=dtype, device=DEV)
    vn = I.random_tensor((B, G, D), seed=13, dtype=dtype, device=DEV)
    kbuf, kc = guarded_copy(x["k_cache"])
    vbuf, vc = guarded_copy(x["v_cache"])
    obuf, out = guarded((B, H, D), dtype)
    torch.cuda.synchronize()
    gq.decode_step(x["q"], kc, vc, x["seqlens"], scale=w.scale, k_new=kn, v_new=vn, window=window, out=out,
                   split_tokens=64)
    torch.cuda.synchronize()
    assert margins_intact(obuf) and margins_intact(kbuf) and margins_intact(vbuf)
    ref, ref_k, ref_v = O.decode_step(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]),
                                      to_host(x["seqlens"]), w.scale, k_new=to_host(kn), v_new=to_host(vn),
                                      window=window)
    assert_parity(out, ref, dtype, "decode_step")
    assert np.array_equal(_bits(kc), _bits(ref_k)) and np.array_equal(_bits(vc), _bits(ref_v)), "cache contents"


_PREFILL_GUARD = [
    (2, 97, 8, 2, 128, torch.bfloat16, 0),
    (1, 200, 32, 8, 128, torch.bfloat16, 0),
    (1, 130, 64, 1, 128, torch.float16, 0),
    (2, 150, 16, 4, 64, torch.bfloat16, 40),
    (1, 40, 6, 3, 64, torch.float32, 0),
]


# every shape causal, and without a window also full attention (a window needs the causal mask)
@pytest.mark.parametrize("B,T,H,G,D,dtype,window,causal",
                         [c + (True,) for c in _PREFILL_GUARD] + [c + (False,) for c in _PREFILL_GUARD if not c[-1]])
def test_prefill_out_guard_bands(B, T, H, G, D, dtype, window, causal):
    say(f"prefill guard bands B={B} T={T} H={H} G={G} D={D} {dtype} window={window} causal={causal}")
    w = I.PrefillWorkload("guard", B, T, H, G, D, dtype, causal)
    x = I.prefill_inputs(w, seed=T + H, device=DEV)
    buf, out = guarded((B, T, H, D), dtype)
    torch.cuda.synchronize()
    gq.prefill(x["q"], x["k"], x["v"], causal=causal, window=window, out=out)
    torch.cuda.synchronize()
    assert margins_intact(buf), "prefill wrote outside out"
    if window:
        ref = O.prefill_window(to_host(x["q"]), to_host(x["k"]), to_host(x["v"]), window)
    else:
        ref = O.prefill(to_host(x["q"]), to_host(x["k"]), to_host(x["v"]), causal=causal)
    assert_parity(out, ref, dtype, "prefill")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("weighted", [False, True])
def test_pool_out_guard_bands(dtype, weighted):
    say(f"pool guard bands {dtype} weighted={weighted}")
    N, H, G, D = 333, 64, 8, 128
    x = I.mean_pool_inputs(N, H, D, dtype=dtype, seed=21, device=DEV)
    buf, out = guarded((N, G, D), dtype)
    torch.cuda.synchronize()
    if weighted:
        wts = I.random_tensor((H,), seed=22, dtype=torch.float32, device=DEV)
        gq.weighted_pool_kv(x, wts, G, out=out)
        ref = O.weighted_pool(to_host(x), G, to_host(wts))
    else:
        gq.mean_pool_kv(x, G, out=out)
        ref = O.mean_pool(to_host(x), G)
    torch.cuda.synchronize()
    assert margins_intact(buf), "pool wrote outside out"
    g = to_host(out).double().numpy()
    assert np.isfinite(g).all()
    # one rounding of the fp32 result to the output type, plus fp32 accumulation
    ulp = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11, torch.float32: 2.0 ** -23}[dtype]
    assert np.all(np.abs(g - ref) <= ulp * np.abs(ref) + 1e-5 * (1 + np.abs(ref)))


@pytest.mark.parametrize("T", [64 + 1, 64 + 31, 128 + 33, 128 + 63])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_prefill_reads_nothing_past_kv(T, causal, dtype):
    """K and V end where a NaN region begins, 64 rows long: the last, ragged
    key tile must bring zeros for rows past T, not those NaNs."""
    say(f"prefill NaN past K/V T={T} causal={causal} {dtype}")
    B, H, G, D = 2, 8, 2, 128
    w = I.PrefillWorkload("tail", B, T, H, G, D, dtype, causal)
    x = I.prefill_inputs(w, seed=T, device=DEV)
    n = B * T * G * D
    tail = 64 * G * D
    views = {}
    for name in ("k", "v"):
        buf = torch.full((n + tail,), float("nan"), dtype=dtype, device=DEV)
        buf[:n].copy_(x[name].view(-1))
        views[name] = buf[:n].view(B, T, G, D)
    torch.cuda.synchronize()
    out = gq.prefill(x["q"], views["k"], views["v"], causal=causal)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all(), "NaN from rows past the end of K/V"
    ref = O.prefill(to_host(x["q"]), to_host(x["k"]), to_host(x["v"]), causal=causal)
    assert_parity(out, ref, dtype, "prefill")


@pytest.mark.parametrize("H,G", [(32, 8), (64, 1), (16, 16)])
def test_decode_permutation_invariance(H, G):
    """Shuffling each sequence's first L_b cache positions (the same
    permutation for K and V) changes the result only by rounding."""
    say(f"decode permutation invariance H={H} G={G}")
    B, D, Tmax = 4, 128, 2048
    w = I.DecodeWorkload("perm", B, H, G, D, Tmax, torch.bfloat16)
    lens = [2048, 1000, 33, 1777]
    x = I.decode_inputs(w, seed=H * 3 + G, device=DEV, seqlens=lens)
    torch.cuda.synchronize()
    base = gq.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=w.scale)
    gen = torch.Generator(device="cpu").manual_seed(5)
    kp, vp = x["k_cache"].clone(), x["v_cache"].clone()
    for b, L in enumerate(lens):
        perm = torch.randperm(L, generator=gen).to(DEV)
        kp[b, :L] = x["k_cache"][b, perm]
        vp[b, :L] = x["v_cache"][b, perm]
    perm_out = gq.decode(x["q"], kp, vp, x["seqlens"], scale=w.scale)
    torch.cuda.synchronize()
    ref = O.decode(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]), to_host(x["seqlens"]), w.scale)
    assert_parity(base, ref, w.dtype, "unpermuted")
    assert_parity(perm_out, ref, w.dtype, "permuted")
    # the order changes which running maximum each probability is rounded
    # against, so the two agree to the rounding bar, not bit for bit
    assert_parity(perm_out, to_host(base).double().numpy(), w.dtype, "permuted against unpermuted")
