"""GPU prefill parity: libgqa's gqa_prefill against the fp64 oracle."""
import numpy as np
import pytest
import torch

import grouped_query_kv_gqa_amd as gq
import oracle as O
from grouped_query_kv_gqa_amd import inputs as I
from gpu_util import assert_parity, say, to_host

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run(x, causal):
    torch.cuda.synchronize()
    out = gq.prefill(x["q"], x["k"], x["v"], causal=causal)
    torch.cuda.synchronize()
    return out


SMALL = [
    # B, T, H, G, D, dtype
    (2, 77, 8, 2, 128, torch.bfloat16),
    (1, 200, 32, 8, 128, torch.bfloat16),
    (2, 65, 4, 4, 64, torch.bfloat16),     # MHA
    (1, 130, 16, 1, 128, torch.bfloat16),  # MQA
    (1, 33, 24, 4, 64, torch.bfloat16),
    (2, 1, 8, 2, 128, torch.bfloat16),     # one token
    (1, 40, 6, 3, 64, torch.float32),
    (2, 77, 8, 2, 128, torch.float16),
    (1, 130, 16, 1, 128, torch.float16),
    (2, 65, 4, 4, 64, torch.float16),
]


@pytest.mark.parametrize("B,T,H,G,D,dtype", SMALL)
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_small_parity(B, T, H, G, D, dtype, causal):
    say(f"prefill small B={B} T={T} H={H} G={G} D={D} {dtype} causal={causal}")
    w = I.PrefillWorkload("small", B, T, H, G, D, dtype, causal)
    x = I.prefill_inputs(w, seed=T + H, device=DEV)
    out = _run(x, causal)
    ref = O.prefill(to_host(x["q"]), to_host(x["k"]), to_host(x["v"]), causal=causal)
    assert_parity(out, ref, dtype, "prefill")


def test_prefill_llama3_8b_prefix_and_late_rows():
    """Full-size causal prefill (B=4, T=8192): the first 512 positions equal a
    T=512 problem on the same prefix (causality), which the oracle checks in
    full; 16 late rows per sequence are checked one by one."""
    w = I.PREFILL_WORKLOADS["prefill_llama3_8b_causal"]
    say(f"prefill {w.name} full size")
    x = I.prefill_inputs(w, seed=0, device=DEV)
    out = _run(x, True)
    P = 512
    pre = {k: v[:, :P].contiguous() for k, v in x.items()}
    out_pre = _run(pre, True)
    assert torch.equal(out_pre, out[:, :P]), "prefix rows differ from a prefix-sized call"
    ref = O.prefill(to_host(pre["q"]), to_host(pre["k"]), to_host(pre["v"]), causal=True)
    ma, rl = assert_parity(out_pre, ref, w.dtype, "T=512 prefix")
    print(f"{w.name} prefix: max-abs {ma:.3e} rel-L2 {rl:.3e}")
    rng = np.random.default_rng(0)
    rb, rt, rh = [], [], []
    for b in range(w.B):
        for t in list(range(w.T - 8, w.T)) + list(rng.integers(P, w.T - 8, 8)):
            rb.append(b); rt.append(int(t)); rh.append(int(rng.integers(0, w.H)))
    ref_rows = O.prefill(to_host(x["q"]), to_host(x["k"]), to_host(x["v"]), causal=True, rows=(rb, rt, rh))
    got = out[rb, rt, rh]
    ma, rl = assert_parity(got, ref_rows, w.dtype, "late rows")
    print(f"{w.name} late rows: max-abs {ma:.3e} rel-L2 {rl:.3e}")


def test_prefill_row_equals_decode():
    """Causal prefill row t equals decode of q[:, t] over the first t+1 positions."""
    say("prefill vs decode")
    w = I.PrefillWorkload("pd", 2, 96, 16, 4, 128, torch.bfloat16)
    x = I.prefill_inputs(w, seed=4, device=DEV)
    out = _run(x, True)
    for t in (0, 31, 32, 95):
        sl = torch.full((w.B,), t + 1, dtype=torch.int32, device=DEV)
        dec = gq.decode(x["q"][:, t].contiguous(), x["k"], x["v"], sl, scale=w.D ** -0.5)
        torch.cuda.synchronize()
        assert torch.max(torch.abs(dec.float() - out[:, t].float())).item() <= 8e-3


@pytest.mark.parametrize("H,G,D,dtype", [
    (32, 8, 128, torch.bfloat16),
    (24, 8, 128, torch.bfloat16),    # 3 heads per group: a 256-row tile holds 85 1/3 tokens
    (20, 4, 64, torch.bfloat16),     # 5 heads per group
    (16, 16, 128, torch.bfloat16),   # multi-head
    (64, 1, 128, torch.bfloat16),    # multi-query, 64 heads
    (96, 2, 128, torch.bfloat16),    # 48 heads per group: 5 tokens per 256-row tile
    (32, 8, 128, torch.float16),
    (512, 1, 64, torch.bfloat16),    # a group wider than the MFMA tile: row kernel
])
def test_prefill_group_tag_exact(H, G, D, dtype):
    """Group map of the prefill, exactly ("Grouped-Query Attention"
    (llm-arch-kb), section 2 The grouping): with every value row of group g
    in sequence b set to the tag g + G*b, each output row is a convex
    combination of equal rows, so head h of sequence b must come out as
    exactly h // (H/G) + G*b (the tags are small integers, exact in 16 bits;
    the kernel's rounding is far below half a unit in their last place)."""
    say(f"prefill group tag H={H} G={G} d_h={D} {dtype}")
    B, T = 2, 150
    w = I.PrefillWorkload("tag", B, T, H, G, D, dtype)
    x = I.prefill_inputs(w, seed=H + G + D, device=DEV)
    tag = (torch.arange(G, device=DEV, dtype=torch.float32).view(1, 1, G, 1)
           + G * torch.arange(B, device=DEV, dtype=torch.float32).view(B, 1, 1, 1))
    x["v"] = tag.expand(B, T, G, D).to(dtype).contiguous()
    expect = (torch.arange(H, device=DEV) // (H // G)).view(1, 1, H, 1).float() \
        + G * torch.arange(B, device=DEV).view(B, 1, 1, 1).float()
    for causal, window in [(True, 0), (False, 0), (True, 40)]:
        torch.cuda.synchronize()
        out = gq.prefill(x["q"], x["k"], x["v"], causal=causal, window=window)
        torch.cuda.synchronize()
        assert torch.equal(out.float(), expect.expand(B, T, H, D)), (H, G, D, dtype, causal, window)


@pytest.mark.parametrize("H,G,D,dtype", [(32, 8, 128, torch.bfloat16), (64, 1, 128, torch.float16),
                                         (6, 3, 64, torch.bfloat16), (512, 1, 64, torch.bfloat16)])
def test_prefill_window_one_is_exact(H, G, D, dtype):
    """A causal window of one position leaves each query a single key: its
    weight is exactly 1, so row t of head h must equal v[t, h // (H/G)]
    bit for bit (the window edge, exactly)."""
    say(f"prefill window 1 H={H} G={G} d_h={D} {dtype}")
    B, T = 2, 131
    w = I.PrefillWorkload("w1", B, T, H, G, D, dtype)
    x = I.prefill_inputs(w, seed=H * 7 + G, device=DEV)
    torch.cuda.synchronize()
    out = gq.prefill(x["q"], x["k"], x["v"], causal=True, window=1)
    torch.cuda.synchronize()
    expect = x["v"].repeat_interleave(H // G, dim=2).contiguous()
    assert torch.equal(out, expect)


def test_prefill_deterministic():
    """Repeated prefill calls on the same inputs are bit-identical (no
    atomics; every output row is reduced in a fixed order)."""
    say("prefill determinism")
    w = I.PrefillWorkload("det", 2, 1000, 32, 8, 128, torch.bfloat16)
    x = I.prefill_inputs(w, seed=5, device=DEV)
    a = _run(x, True).clone()
    b = _run(x, True)
    assert torch.equal(a, b)


def test_prefill_errors():
    say("prefill argument errors")
    q = torch.zeros(1, 4, 6, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 4, 4, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gq.GqaError) as e:
        gq.prefill(q, k, k)
    assert e.value.status == gq.GQA_ERR_INVALID_ARG
    q = torch.zeros(0, 4, 8, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(0, 4, 2, 128, dtype=torch.bfloat16, device=DEV)
    assert gq.prefill(q, k, k).shape == q.shape


WINDOW_CASES = [
    # B, T, H, G, D, dtype
    (2, 300, 8, 2, 128, torch.bfloat16),
    (1, 260, 8, 8, 64, torch.bfloat16),    # MHA: 128 tokens per workgroup
    (1, 200, 32, 1, 128, torch.bfloat16),  # r = 32: 4 tokens per workgroup
    (2, 150, 16, 4, 64, torch.bfloat16),
    (1, 90, 6, 3, 64, torch.float32),
    (2, 300, 8, 2, 128, torch.float16),
]


@pytest.mark.parametrize("B,T,H,G,D,dtype", WINDOW_CASES)
@pytest.mark.parametrize("window", [1, 5, 64, 100, 1000])
def test_prefill_window_parity(B, T, H, G, D, dtype, window):
    say(f"prefill window={window} B={B} T={T} H={H} G={G} D={D} {dtype}")
    w = I.PrefillWorkload("win", B, T, H, G, D, dtype, True)
    x = I.prefill_inputs(w, seed=T + window, device=DEV)
    torch.cuda.synchronize()
    out = gq.prefill(x["q"], x["k"], x["v"], causal=True, window=window)
    torch.cuda.synchronize()
    ref = O.prefill_window(to_host(x["q"]), to_host(x["k"]), to_host(x["v"]), window)
    assert_parity(out, ref, dtype, f"window={window}")


def test_prefill_window_full_size_sampled():
    """Full-size causal prefill (B=4, T=8192) with a 4096-position window:
    rows on both sides of the window edge checked one by one, and the first
    4096 positions equal to plain causal prefill (the window covers them)."""
    w = I.PREFILL_WORKLOADS["prefill_llama3_8b_causal"]
    W = 4096
    say(f"prefill {w.name} full size, window {W}")
    x = I.prefill_inputs(w, seed=1, device=DEV)
    out = gq.prefill(x["q"], x["k"], x["v"], causal=True, window=W)
    full = gq.prefill(x["q"], x["k"], x["v"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :W], full[:, :W])
    rt = np.array([W - 1, W, W + 1, 5000, 8191, 8191, 6000, 4500])
    rb = np.array([0, 1, 2, 3, 0, 3, 1, 2])
    rh = np.array([0, 5, 31, 8, 17, 2, 30, 9])
    ref = O.prefill_window(to_host(x["q"]), to_host(x["k"]), to_host(x["v"]), W, rows=(rb, rt, rh))
    got = out[torch.as_tensor(rb), torch.as_tensor(rt), torch.as_tensor(rh)]
    assert_parity(got, ref, w.dtype, "window rows")


def test_prefill_window_errors():
    say("prefill window argument errors")
    w = I.PrefillWorkload("err", 1, 16, 4, 2, 64, torch.bfloat16, True)
    x = I.prefill_inputs(w, seed=0, device=DEV)
    with pytest.raises(gq.GqaError):
        gq.prefill(x["q"], x["k"], x["v"], causal=False, window=8)
    with pytest.raises(gq.GqaError):
        gq.prefill(x["q"], x["k"], x["v"], causal=True, window=-1)


def test_prefill_fp16_full_size_sampled():
    """Full-size causal prefill (B=4, T=8192) with fp16 storage: late rows
    checked one by one against the oracle."""
    base = I.PREFILL_WORKLOADS["prefill_llama3_8b_causal"]
    w = I.PrefillWorkload(base.name + "_fp16", base.B, base.T, base.H, base.G, base.D, torch.float16, True)
    say(f"prefill {w.name} full size")
    x = I.prefill_inputs(w, seed=2, device=DEV)
    out = _run(x, True)
    rb = np.array([0, 1, 2, 3, 0, 2])
    rt = np.array([8191, 8000, 4096, 5555, 1, 7777])
    rh = np.array([0, 31, 7, 12, 3, 20])
    ref = O.prefill(to_host(x["q"]), to_host(x["k"]), to_host(x["v"]), causal=True, rows=(rb, rt, rh))
    got = out[torch.as_tensor(rb), torch.as_tensor(rt), torch.as_tensor(rh)]
    assert_parity(got, ref, w.dtype, "fp16 rows")


@pytest.mark.parametrize("H,G", [(12, 4), (10, 2), (30, 5), (21, 3), (96, 32)])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_group_sizes_not_dividing_tile(H, G, causal):
    """Group sizes r = H/G of 3, 5, 6 and 7 leave a 256-row query tile partly
    unused (256 // r tokens of r heads), and r = 3 with d_h = 64; checked
    against the oracle over every row, with a sequence length that ends in a
    partial key tile."""
    say(f"prefill r={H // G} H={H} G={G} causal={causal}")
    D = 64 if H == 96 else 128
    w = I.PrefillWorkload("r", 2, 301, H, G, D, torch.bfloat16, causal)
    x = I.prefill_inputs(w, seed=H + G, device=DEV)
    out = _run(x, causal)
    ref = O.prefill(to_host(x["q"]), to_host(x["k"]), to_host(x["v"]), causal=causal)
    assert_parity(out, ref, torch.bfloat16, f"r={H // G}")
