"""The range-checked build, libgqa_debug.so: the same kernels compiled with
-DGQA_DEBUG, where every global-memory access checks its index (cache
positions against Tmax, rows against B*H or B*T*H, partial-row slots against
the workspace, tile rows against T) and records a flag instead of touching
memory out of range.

Every kernel family runs here from the debug library on shapes that reach its
edges (empty, clamped and full sequences, appends, windows, sequences cut
into many pieces or into slices long enough for the decode's falling wave
priority, T not a multiple of the 64-position tile, groups wider than 32
heads, the row kernels). No check may fire, and each result must equal the
release library's bit for bit: the checks add branches, never arithmetic.
Inputs come from the seeded generators of grouped_query_kv_gqa_amd.inputs.
"""
import pytest
import torch

import grouped_query_kv_gqa_amd as gq
from grouped_query_kv_gqa_amd import inputs as I
from gpu_util import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _same(a, b):
    if a.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def _release_and_debug(name, fn):
    """fn() -> tuple of result tensors; runs it on both libraries."""
    say(f"debug build: {name} (release)")
    rel = [t.clone() for t in fn()]
    torch.cuda.synchronize()
    with gq.debug_build():
        enabled, _ = gq.debug_checks()  # clears earlier flags
        assert enabled, "libgqa_debug.so was built without checks"
        say(f"debug build: {name} (range-checked)")
        dbg = [t.clone() for t in fn()]
        _, flags = gq.debug_checks()
    assert flags == 0, f"{name}: range checks fired, flags {flags:#010x}"
    for i, (a, b) in enumerate(zip(rel, dbg)):
        assert _same(a, b), f"{name}: result {i} differs between the release and the debug library"


def test_release_library_reports_no_checks():
    assert gq.debug_checks() == (False, 0)


def test_a_failed_check_reaches_the_host():
    # one check that fails by construction (it guards no memory access)
    with gq.debug_build():
        gq.debug_checks()
        lib = gq.load_library()
        say("debug build: self-test check")
        assert lib.gqa_debug_selftest(torch.cuda.current_stream().cuda_stream) == gq.GQA_OK
        assert gq.debug_checks() == (True, 1 << 31)
        assert gq.debug_checks() == (True, 0)  # cleared by the read


DECODE = [
    # B, H, G, D, Tmax, seqlens, dtype, split_tokens
    (5, 32, 8, 128, 700, [700, 0, 699, 1, 5000], torch.bfloat16, 0),   # full, empty, clamped long
    (3, 64, 1, 128, 1500, [0, 1200, 1500], torch.bfloat16, 0),         # one group of 64 heads
    (4, 40, 1, 64, 333, [333, 17, 200, 64], torch.bfloat16, 32),       # 40-head group, many pieces
    (70, 16, 4, 128, 96, [(7 * i) % 97 for i in range(70)], torch.bfloat16, 0),  # more than 64 sequences
    (2, 8, 8, 64, 200, [150, 200], torch.float16, 0),                  # multi-head, fp16
    (3, 12, 3, 64, 50, [50, 17, 0], torch.float32, 0),                 # fp32 path
    (2, 16, 4, 128, 2000, [2000, 1500], torch.bfloat16, 1024),        # slices long enough for the wave priority
]


@pytest.mark.parametrize("B,H,G,D,Tmax,seqlens,dtype,split", DECODE)
def test_decode_debug_build(B, H, G, D, Tmax, seqlens, dtype, split):
    w = I.DecodeWorkload("dbg", B, H, G, D, Tmax, dtype)
    x = I.decode_inputs(w, seed=11, device=DEV, seqlens=seqlens)

    def run():
        return (gq.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=w.scale, split_tokens=split),)

    _release_and_debug(f"decode B={B} H={H} G={G} D={D} Tmax={Tmax} {dtype} split={split}", run)


STEP = [
    # B, H, G, D, Tmax, seqlens, dtype, window
    (4, 16, 4, 128, 300, [0, 299, 300, 150], torch.bfloat16, 64),
    (2, 64, 1, 128, 260, [259, 31], torch.bfloat16, 0),
    (3, 12, 3, 64, 50, [50, 17, 0], torch.float32, 8),
]


@pytest.mark.parametrize("B,H,G,D,Tmax,seqlens,dtype,window", STEP)
def test_decode_step_debug_build(B, H, G, D, Tmax, seqlens, dtype, window):
    w = I.DecodeWorkload("dbg", B, H, G, D, Tmax, dtype)
    x = I.decode_inputs(w, seed=12, device=DEV, seqlens=seqlens)
    kn = I.random_tensor((B, G, D), seed=13, dtype=dtype, device=DEV)
    vn = I.random_tensor((B, G, D), seed=14, dtype=dtype, device=DEV)
    k0, v0 = x["k_cache"].clone(), x["v_cache"].clone()

    def run():
        k, v = k0.clone(), v0.clone()
        out = gq.decode_step(x["q"], k, v, x["seqlens"], scale=w.scale, k_new=kn, v_new=vn, window=window)
        return out, k, v

    _release_and_debug(f"decode_step B={B} H={H} G={G} D={D} Tmax={Tmax} {dtype} window={window}", run)


PREFILL = [
    # B, T, H, G, D, causal, window, dtype
    (2, 200, 8, 2, 128, True, 0, torch.bfloat16),
    (2, 130, 8, 2, 128, False, 0, torch.bfloat16),
    (1, 300, 12, 4, 64, True, 50, torch.bfloat16),
    (1, 97, 6, 2, 64, True, 0, torch.float16),
    (1, 70, 8, 2, 64, True, 0, torch.float32),      # row kernel
    (1, 40, 512, 1, 64, True, 0, torch.bfloat16),   # 512 heads in a group: row kernel
]


@pytest.mark.parametrize("B,T,H,G,D,causal,window,dtype", PREFILL)
def test_prefill_debug_build(B, T, H, G, D, causal, window, dtype):
    w = I.PrefillWorkload("dbg", B, T, H, G, D, dtype)
    x = I.prefill_inputs(w, seed=15, device=DEV)

    def run():
        return (gq.prefill(x["q"], x["k"], x["v"], causal=causal, window=window),)

    _release_and_debug(f"prefill B={B} T={T} H={H} G={G} D={D} causal={causal} window={window} {dtype}", run)


@pytest.mark.parametrize("weighted", [False, True])
def test_pool_debug_build(weighted):
    x = I.mean_pool_inputs(1000, 32, 128, dtype=torch.bfloat16, seed=16, device=DEV)
    wts = I.random_tensor((32,), seed=17, dtype=torch.float32, device=DEV)

    def run():
        return (gq.weighted_pool_kv(x, wts, 4) if weighted else gq.mean_pool_kv(x, 4),)

    _release_and_debug(f"pool weighted={weighted}", run)
