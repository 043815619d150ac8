"""GPU decode parity: libgqa's gqa_decode against the fp64 oracle.

Inputs come from grouped_query_kv_gqa_amd.inputs (seeded draws only); the
oracle reads host copies of the exact same bits.
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


def _oracle_rows(x, w_scale, bs):
    """Oracle output for the listed sequences (all heads), reading only their
    first L_b cache positions."""
    sl = to_host(x["seqlens"]).numpy()
    outs = []
    for b in bs:
        L = int(min(max(sl[b], 0), x["k_cache"].shape[1]))
        Lc = max(L, 1)
        k = to_host(x["k_cache"][b:b + 1, :Lc])
        v = to_host(x["v_cache"][b:b + 1, :Lc])
        q = to_host(x["q"][b:b + 1])
        outs.append(O.decode(q, k, v, np.array([L], np.int32), w_scale)[0])
    return np.stack(outs)


def _run(x, scale, split_tokens=0):
    torch.cuda.synchronize()
    out = gq.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=scale, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out


def test_decode_tiny_fp32_full():
    w = I.WORKLOADS["decode_tiny_fp32"]
    say(f"decode {w.name}")
    x = I.decode_inputs(w, seed=0, device=DEV)
    out = _run(x, w.scale)
    ref = O.decode(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]), to_host(x["seqlens"]), w.scale)
    assert_parity(out, ref, torch.float32, w.name)


SMALL = [
    # B, H, G, D, Tmax, seqlens, dtype
    (3, 8, 2, 128, 300, [300, 1, 37], torch.bfloat16),
    (2, 32, 8, 128, 257, [257, 200], torch.bfloat16),
    (2, 8, 8, 64, 100, [65, 100], torch.bfloat16),      # MHA, G = H
    (2, 16, 1, 128, 130, [130, 33], torch.bfloat16),    # MQA, G = 1
    (2, 64, 1, 128, 96, [96, 31], torch.bfloat16),      # 64 heads in one group
    (1, 40, 1, 64, 70, [70], torch.bfloat16),           # 40 heads: ragged head tile
    (2, 24, 4, 64, 45, [45, 32], torch.bfloat16),
    (2, 12, 3, 64, 50, [50, 17], torch.float32),
    (3, 4, 2, 128, 33, [33, 0, 5], torch.float32),
    (3, 32, 8, 128, 300, [300, 1, 170], torch.float16),
    (2, 64, 1, 128, 96, [96, 31], torch.float16),     # 64 heads in one group
    (2, 8, 8, 64, 100, [65, 100], torch.float16),     # MHA
]


@pytest.mark.parametrize("B,H,G,D,Tmax,seqlens,dtype", SMALL)
def test_decode_small_parity(B, H, G, D, Tmax, seqlens, dtype):
    say(f"decode small B={B} H={H} G={G} D={D} Tmax={Tmax} {dtype}")
    w = I.DecodeWorkload("small", B, H, G, D, Tmax, dtype)
    x = I.decode_inputs(w, seed=B * 1000 + H + G, device=DEV, seqlens=seqlens)
    for split in (0, 32, 64):
        out = _run(x, w.scale, split)
        ref = O.decode(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]), to_host(x["seqlens"]),
                       w.scale)
        assert_parity(out, ref, dtype, f"split={split}")


def test_decode_llama3_8b_full():
    w = I.WORKLOADS["decode_llama3_8b"]
    say(f"decode {w.name} full size")
    x = I.decode_inputs(w, seed=0, device=DEV)
    out = _run(x, w.scale)
    ref = O.decode(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]), to_host(x["seqlens"]), w.scale)
    ma, rl = assert_parity(out, ref, w.dtype, w.name)
    print(f"{w.name}: max-abs {ma:.3e} rel-L2 {rl:.3e}")


@pytest.mark.parametrize("G", [8, 1, 64])
def test_decode_llama2_70b_ragged_full(G):
    """The ragged Llama-2-70B batch at full size, launched as the benchmark
    launches it. G = 8 and G = 1: all 64 sequences against the oracle. G = 64
    (16 GiB of cache): 16 sequences spread over the length range (the
    shortest, the longest and 14 evenly spaced in sorted order), read back
    one by one; every output is checked to be finite."""
    base = I.WORKLOADS["decode_llama2_70b_ragged"]
    w = base if G == base.G else base.with_G(G)
    say(f"decode {w.name} full size")
    x = I.decode_inputs(w, seed=0, device=DEV)
    out = _run(x, w.scale)
    sl = to_host(x["seqlens"]).numpy()
    if G == 64:
        order = np.argsort(sl, kind="stable")
        bs = sorted({int(order[int(round(i * (w.B - 1) / 15))]) for i in range(16)})
        assert len(bs) == 16
        ref = _oracle_rows(x, w.scale, bs)
        got = out[bs]
        assert torch.isfinite(out.float()).all()
    else:
        bs = list(range(w.B))
        ref = O.decode(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]), to_host(x["seqlens"]),
                       w.scale)
        got = out
    ma, rl = assert_parity(got, ref, w.dtype, w.name)
    print(f"{w.name}: max-abs {ma:.3e} rel-L2 {rl:.3e} over {len(bs)} sequences")
    del x
    torch.cuda.empty_cache()


def test_decode_long_128k_full():
    w = I.WORKLOADS["decode_long_128k"]
    say(f"decode {w.name} full size")
    x = I.decode_inputs(w, seed=0, device=DEV)
    out = _run(x, w.scale)
    ref = _oracle_rows(x, w.scale, [0])
    ma, rl = assert_parity(out, ref, w.dtype, w.name)
    print(f"{w.name}: max-abs {ma:.3e} rel-L2 {rl:.3e}")


def test_decode_split_invariance():
    w = I.DecodeWorkload("split", 2, 16, 4, 128, 2000, torch.bfloat16)
    say("decode split invariance")
    x = I.decode_inputs(w, seed=3, device=DEV, seqlens=[2000, 1500])
    ref = O.decode(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]), to_host(x["seqlens"]), w.scale)
    outs = []
    for split in (32, 64, 96, 256, 1000, 2000, 0):
        out = _run(x, w.scale, split)
        assert_parity(out, ref, w.dtype, f"split={split}")
        outs.append(out.float())
    for o in outs[1:]:
        assert torch.max(torch.abs(o - outs[0])).item() <= 4e-3


def test_decode_nan_tail_never_read():
    w = I.DecodeWorkload("poison", 4, 16, 4, 128, 200, torch.bfloat16)
    say("decode NaN-poisoned tail")
    lens = [1, 31, 32, 33]
    x = I.decode_inputs(w, seed=5, device=DEV, seqlens=lens)
    for b, L in enumerate(lens):
        x["k_cache"][b, L:] = 0
        x["v_cache"][b, L:] = 0
    clean = _run(x, w.scale, 64).clone()
    for b, L in enumerate(lens):
        x["k_cache"][b, L:] = float("nan")
        x["v_cache"][b, L:] = float("nan")
    for split in (64, 0, 32):
        poisoned = _run(x, w.scale, split)
        assert torch.isfinite(poisoned.float()).all()
        if split == 64:
            assert torch.equal(poisoned, clean)
    # lengths at and around tile and cache edges
    w2 = I.DecodeWorkload("edges", 6, 8, 2, 64, 97, torch.bfloat16)
    lens = [1, 31, 32, 33, 96, 97]
    x = I.decode_inputs(w2, seed=6, device=DEV, seqlens=lens)
    for b, L in enumerate(lens):
        x["k_cache"][b, L:] = float("nan")
        x["v_cache"][b, L:] = float("nan")
    out = _run(x, w2.scale)
    kh, vh = to_host(x["k_cache"]), to_host(x["v_cache"])
    ref = O.decode(to_host(x["q"]), kh, vh, np.array(lens, np.int32), w2.scale)
    assert_parity(out, ref, w2.dtype, "edge lengths")


def test_decode_group_tag_exact():
    say("decode group tag")
    # (96, 2), (80, 2), (40, 1): 48, 40 and 40 heads per group, so the wide
    # kernel's last 16-head tile is partly or wholly past the group
    for H, G in [(32, 8), (64, 8), (8, 8), (16, 1), (64, 1), (24, 4), (96, 2), (80, 2), (40, 1)]:
        w = I.DecodeWorkload("tag", 2, H, G, 128, 150, torch.bfloat16)
        x = I.decode_inputs(w, seed=H + G, device=DEV, seqlens=[150, 77])
        tag = torch.arange(G, device=DEV, dtype=torch.float32).view(1, 1, G, 1)
        x["v_cache"] = tag.expand_as(x["v_cache"]).to(torch.bfloat16).contiguous()
        for split in (0, 32):
            out = _run(x, w.scale, split)
            expect = torch.arange(H, device=DEV) // (H // G)
            assert torch.equal(out.float(), expect.float().view(1, H, 1).expand_as(out).float()), (H, G, split)


def test_decode_lengths_clamp_and_zero():
    say("decode length clamping")
    w = I.DecodeWorkload("clamp", 4, 8, 2, 128, 64, torch.bfloat16)
    x = I.decode_inputs(w, seed=9, device=DEV, seqlens=[64, 0, -3, 10 ** 6])
    out = _run(x, w.scale, 32)
    assert torch.all(out[1] == 0) and torch.all(out[2] == 0)
    x2 = dict(x)
    x2["seqlens"] = torch.tensor([64, 0, 0, 64], dtype=torch.int32, device=DEV)
    out2 = _run(x2, w.scale, 32)
    assert torch.equal(out, out2)


def test_decode_deterministic():
    say("decode determinism")
    w = I.WORKLOADS["decode_llama3_8b"]
    x = I.decode_inputs(w, seed=1, device=DEV)
    a = _run(x, w.scale).clone()
    b = _run(x, w.scale)
    assert torch.equal(a, b)


def test_decode_empty_batch_and_errors():
    say("decode empty batch and argument errors")
    q = torch.empty(0, 8, 128, dtype=torch.bfloat16, device=DEV)
    kc = torch.empty(0, 16, 2, 128, dtype=torch.bfloat16, device=DEV)
    sl = torch.empty(0, dtype=torch.int32, device=DEV)
    assert gq.decode(q, kc, kc, sl).shape == (0, 8, 128)
    q = torch.zeros(1, 6, 128, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(1, 16, 4, 128, dtype=torch.bfloat16, device=DEV)
    sl = torch.tensor([16], dtype=torch.int32, device=DEV)
    with pytest.raises(gq.GqaError) as e:
        gq.decode(q, kc, kc, sl)
    assert e.value.status == gq.GQA_ERR_INVALID_ARG
    q = torch.zeros(1, 8, 96, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(1, 16, 2, 96, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gq.GqaError) as e:
        gq.decode(q, kc, kc, sl)
    assert e.value.status == gq.GQA_ERR_UNSUPPORTED


def test_decode_llama3_8b_fp16_full():
    """The Llama-3-8B decode layer with fp16 storage (the pages count 2-byte
    fp16 cache scalars)."""
    base = I.WORKLOADS["decode_llama3_8b"]
    w = I.DecodeWorkload(base.name + "_fp16", base.B, base.H, base.G, base.D, base.Tmax, torch.float16)
    say(f"decode {w.name} full size")
    x = I.decode_inputs(w, seed=0, device=DEV)
    out = _run(x, w.scale)
    ref = O.decode(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]), to_host(x["seqlens"]), w.scale)
    ma, rl = assert_parity(out, ref, w.dtype, w.name)
    print(f"{w.name}: max-abs {ma:.3e} rel-L2 {rl:.3e}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H,G", [(8, 2), (16, 4), (24, 3), (64, 1), (48, 1), (96, 2)])
def test_decode_shared_group_deterministic(H, G, D):
    """Layouts where several waves share a group (they combine their softmax
    states inside the workgroup): repeated calls give the same bits, and the
    result matches the oracle, with and without an append."""
    say(f"decode deterministic combine H={H} G={G} D={D}")
    B, Tmax = 6, 1500
    w = I.DecodeWorkload("det", B, H, G, D, Tmax, torch.bfloat16)
    x = I.decode_inputs(w, seed=H * 10 + G + D, device=DEV, seqlens=[1500, 1, 700, 0, 1499, 333])
    ref = O.decode(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]), to_host(x["seqlens"]), w.scale)
    first = _run(x, w.scale)
    for _ in range(5):
        assert torch.equal(_run(x, w.scale), first)
    assert_parity(first, ref, torch.bfloat16, "decode")
    kn = I.random_tensor((B, G, D), seed=7, dtype=torch.bfloat16, device=DEV)
    vn = I.random_tensor((B, G, D), seed=8, dtype=torch.bfloat16, device=DEV)
    outs = []
    for _ in range(3):
        kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
        torch.cuda.synchronize()
        outs.append(gq.decode_step(x["q"], kc, vc, x["seqlens"], scale=w.scale, k_new=kn, v_new=vn))
        torch.cuda.synchronize()
    assert all(torch.equal(o, outs[0]) for o in outs[1:])
    ref_a, _, _ = O.decode_step(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]), to_host(x["seqlens"]),
                                w.scale, k_new=to_host(kn), v_new=to_host(vn))
    assert_parity(outs[0], ref_a, torch.bfloat16, "decode_step append")


WIDE = [
    # B, H, G, D, Tmax, seqlens, dtype: 33 to 64 heads per group (one
    # workgroup per slice and group, K/V staged in LDS for all heads)
    (3, 64, 1, 128, 1000, [1000, 129, 1], torch.bfloat16),
    (2, 33, 1, 128, 700, [700, 300], torch.bfloat16),      # a 1-head second tile
    (4, 96, 2, 64, 600, [600, 0, 127, 128], torch.bfloat16),
    (2, 120, 3, 128, 450, [449, 450], torch.float16),      # 40 heads per group
    (5, 48, 1, 64, 2100, [2100, 1, 2048, 777, 1500], torch.float16),
]


@pytest.mark.parametrize("B,H,G,D,Tmax,seqlens,dtype", WIDE)
def test_decode_wide_groups(B, H, G, D, Tmax, seqlens, dtype):
    """Groups of 33 to 64 heads against the oracle, whole and cut into
    pieces, with an append into the cache and with a window."""
    say(f"decode wide B={B} H={H} G={G} D={D} Tmax={Tmax} {dtype}")
    w = I.DecodeWorkload("wide", B, H, G, D, Tmax, dtype)
    x = I.decode_inputs(w, seed=H * 7 + G + D, device=DEV, seqlens=seqlens)
    ref = O.decode(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]), to_host(x["seqlens"]), w.scale)
    for split in (0, 32, 160, 4096):
        out = _run(x, w.scale, split)
        assert_parity(out, ref, dtype, f"split={split}")
    kn = I.random_tensor((B, G, D), seed=31, dtype=dtype, device=DEV)
    vn = I.random_tensor((B, G, D), seed=32, dtype=dtype, device=DEV)
    for window, split in ((0, 0), (0, 96), (200, 0), (1, 64)):
        ref_s, kr, vr = O.decode_step(to_host(x["q"]), to_host(x["k_cache"]), to_host(x["v_cache"]),
                                      to_host(x["seqlens"]), w.scale, k_new=to_host(kn), v_new=to_host(vn),
                                      window=window)
        kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
        torch.cuda.synchronize()
        out = gq.decode_step(x["q"], kc, vc, x["seqlens"], scale=w.scale, k_new=kn, v_new=vn, window=window,
                             split_tokens=split)
        torch.cuda.synchronize()
        assert_parity(out, ref_s, dtype, f"append window={window} split={split}")
        assert np.array_equal(to_host(kc).view(torch.int16).numpy().view(np.uint16), kr)
        assert np.array_equal(to_host(vc).view(torch.int16).numpy().view(np.uint16), vr)


@pytest.mark.parametrize("D", [64, 128])
def test_decode_default_scale_is_inverse_sqrt_dh(D):
    # no scale given: the library's default, 1/sqrt(d_h), bit for bit the same
    # as passing it (both round to the same float)
    say(f"decode default scale D={D}")
    w = I.DecodeWorkload("scale", 3, 16, 4, D, 300, torch.bfloat16)
    x = I.decode_inputs(w, seed=21, device=DEV, seqlens=[300, 17, 0])
    a = gq.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"])
    b = gq.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=D ** -0.5)
    k0, v0 = x["k_cache"].clone(), x["v_cache"].clone()
    kn = I.random_tensor((3, 4, D), seed=22, dtype=torch.bfloat16, device=DEV)
    c = gq.decode_step(x["q"], k0, v0, x["seqlens"], k_new=kn, v_new=kn, window=64)
    k1, v1 = x["k_cache"].clone(), x["v_cache"].clone()
    d = gq.decode_step(x["q"], k1, v1, x["seqlens"], scale=D ** -0.5, k_new=kn, v_new=kn, window=64)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(c.view(torch.int16), d.view(torch.int16))
