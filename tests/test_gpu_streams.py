"""Streams and graph capture: libgqa queues its kernels on the caller's
stream and keeps one split-decode workspace per (device, stream).

- Decode calls of different shapes on two streams, overlapping in time, give
  bit for bit the results of the same calls made one after the other (decode
  is deterministic), so neither stream's partial rows leak into the other's.
- A decode call and a prefill call captured into a HIP graph (after a
  warm-up call on the capture stream, which sizes the workspace outside the
  capture) and replayed with new inputs copied into the captured tensors give
  the eager results on every replay, with eager work and synchronisation
  between the replays.
"""
import pytest
import torch

import grouped_query_kv_gqa_amd as gq
from grouped_query_kv_gqa_amd import inputs as I
from gpu_util import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _decode(x, w):
    return gq.decode(x["q"], x["k_cache"], x["v_cache"], x["seqlens"], scale=w.scale)


def test_decode_two_streams_match_serial():
    say("decode on two concurrent streams")
    wa = I.DecodeWorkload("a", 16, 32, 8, 128, 2048, torch.bfloat16)
    wb = I.DecodeWorkload("b", 5, 64, 8, 128, 3000, torch.bfloat16, ragged=(1, 3000))
    xa = I.decode_inputs(wa, seed=11, device=DEV)
    xb = I.decode_inputs(wb, seed=12, device=DEV)
    ref_a = _decode(xa, wa).clone()
    ref_b = _decode(xb, wb).clone()
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(4):
        with torch.cuda.stream(sa):
            oa = _decode(xa, wa)
        with torch.cuda.stream(sb):
            ob = _decode(xb, wb)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        assert torch.equal(oa, ref_a)
        assert torch.equal(ob, ref_b)


def test_graph_capture_decode_and_prefill():
    say("decode and prefill captured in a HIP graph, replayed with new inputs")
    w = I.DecodeWorkload("g", 8, 32, 8, 128, 1500, torch.bfloat16, ragged=(1, 1500))
    pw = I.PrefillWorkload("g", 1, 300, 16, 4, 128, torch.bfloat16, True)
    x = I.decode_inputs(w, seed=21, device=DEV)
    px = I.prefill_inputs(pw, seed=22, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream: the workspace exists before capture
        _decode(x, w)
        gq.prefill(px["q"], px["k"], px["v"], causal=True)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        out = _decode(x, w)
        pout = gq.prefill(px["q"], px["k"], px["v"], causal=True)
    for rep in range(3):
        nx = I.decode_inputs(w, seed=30 + rep, device=DEV)
        npx = I.prefill_inputs(pw, seed=40 + rep, device=DEV)
        for key in ("q", "k_cache", "v_cache", "seqlens"):
            x[key].copy_(nx[key])
        for key in ("q", "k", "v"):
            px[key].copy_(npx[key])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = _decode(nx, w)
        pref = gq.prefill(npx["q"], npx["k"], npx["v"], causal=True)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"decode replay {rep}"
        assert torch.equal(pout, pref), f"prefill replay {rep}"


def test_graph_survives_workspace_growth():
    """A decode captured at a small shape keeps working after a larger eager
    call on the capture stream replaces the stream's workspace: the captured
    block is kept alive, and every replay matches the eager result bit for
    bit. A capture on a stream whose workspace is missing fails cleanly
    without allocating."""
    say("graph replay after workspace growth on the capture stream")
    small = I.DecodeWorkload("small", 4, 32, 8, 128, 1024, torch.bfloat16, ragged=(1, 1024))
    big = I.DecodeWorkload("big", 32, 64, 8, 128, 4096, torch.bfloat16, ragged=(1024, 4096))
    x = I.decode_inputs(small, seed=51, device=DEV)
    xb = I.decode_inputs(big, seed=52, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _decode(x, small)  # sizes the stream's workspace for the small shape
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        out = _decode(x, small)
    for rep in range(3):
        with torch.cuda.stream(s):  # larger eager call: the workspace grows
            bo = _decode(xb, big)
        s.synchronize()
        nx = I.decode_inputs(small, seed=60 + rep, device=DEV)
        for key in ("q", "k_cache", "v_cache", "seqlens"):
            x[key].copy_(nx[key])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = _decode(nx, small)
        bref = _decode(xb, big)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} after growth"
        assert torch.equal(bo, bref), f"large eager call {rep}"
    # a fresh stream has no workspace: capturing a split decode there is refused
    s2 = torch.cuda.Stream()
    s2.wait_stream(torch.cuda.current_stream())
    g2 = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(g2, stream=s2):
        try:
            _decode(x, small)
        except gq.GqaError as e:
            err = e
    assert err is not None and err.status == gq.GQA_ERR_INVALID_ARG and "captur" in str(err)
    torch.cuda.synchronize()
