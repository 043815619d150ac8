"""Pins that tie the fp64 oracle to facts fixed outside the oracle itself.

Every pin takes an oracle library handle, so the same pins run against the
real oracle (test_oracle_pins.py) and against copies of it with a mistake
planted (test_oracle_mutants.py), where at least one pin must fail.

What each pin compares against:
  * numbers the pages print (tests/golden/kv_cache_bytes.json);
  * torch's scaled_dot_product_attention in float64 on the CPU, a library
    routine: plain MHA at G = H, MQA by expanding one K/V head, and GQA both
    through its enable_gqa broadcast and through repeat_interleave, which is
    the broadcast the sketch in "Grouped-Query Attention" (llm-arch-kb),
    section 3, states;
  * pure-Python scalar loops on tiny inputs (brute force);
  * closed forms: one cached token, all-zero keys, zero scale, two keys with
    an analytic sigmoid weight, one dominant key, an exact group tag;
  * invariants: softmax weights sum to one, positions past the sequence length
    are never read, permuting cache positions changes nothing, causal prefill
    row t equals decode over the first t+1 positions;
  * mean-pooling: a hand-worked example, identity at G = H, the all-head mean
    at G = 1, numpy's reshape-mean over contiguous groups, and linearity
    (pooling weights then projecting equals projecting then pooling);
  * fp16 storage: all 65536 bit patterns against numpy's float16 widening;
  * cache append: the caches after the call against numpy assignment, the
    output against library attention over the appended cache, and the exact
    new value for an empty sequence;
  * sliding windows: library attention over the sliced cache (decode) or with
    a band mask (prefill), the exact value for a one-position window, and no
    change for a window covering the whole sequence;
  * weighted pooling: numpy's einsum, one-hot weights (exact head copies) and
    the mean at w = 1/r.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "kv_cache_bytes.json")


def _divisors(n):
    return [d for d in range(1, n + 1) if n % d == 0]


def _sdpa_decode(q, k, v, L, scale, mode="gqa"):
    """Library attention for one sequence. q [H,D], k/v [Tmax,G,D] fp64 numpy."""
    H, D = q.shape
    G = k.shape[1]
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(k[:L].transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v[:L].transpose(1, 0, 2)))[None]
    if mode == "gqa":
        o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)
    elif mode == "repeat":
        o = F.scaled_dot_product_attention(qt, kt.repeat_interleave(H // G, dim=1),
                                           vt.repeat_interleave(H // G, dim=1), scale=scale)
    elif mode == "mha":
        assert G == H
        o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    elif mode == "mqa":
        assert G == 1
        o = F.scaled_dot_product_attention(qt, kt.expand(1, H, L, D), vt.expand(1, H, L, D), scale=scale)
    else:
        raise ValueError(mode)
    return o[0, :, 0, :].numpy()


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# --------------------------------------------------------------------------
# Pins
# --------------------------------------------------------------------------

def pin_group_map(lib):
    for H in range(1, 129):
        for G in _divisors(H):
            expect = np.repeat(np.arange(G), H // G)  # repeat_interleave order
            got = [O.group_of_head(h, H, G, lib=lib) for h in range(H)]
            assert got == expect.tolist(), (H, G)


def pin_cache_golden(lib):
    with open(GOLDEN) as f:
        gold = json.load(f)
    for c in gold["cases"]:
        b = O.kv_cache_bytes_per_token(c["kv_heads"], c["d_h"], c["layers"], c["bytes_per_scalar"], lib=lib)
        assert b == c["bytes_per_token"], (c["what"], b)
        if "MiB_per_token" in c:
            assert b / 2 ** 20 == c["MiB_per_token"]
        if "KiB_per_token" in c:
            assert b / 2 ** 10 == c["KiB_per_token"]
        for T, gib in c["GiB_at_tokens"].items():
            assert b * int(T) / 2 ** 30 == gib, (c["what"], T)
    for r in gold["ratios"]:
        big = O.kv_cache_bytes_per_token(r["G_mha"], 128, 80, 2, lib=lib)
        small = O.kv_cache_bytes_per_token(r["G_mqa"], 128, 80, 2, lib=lib)
        assert big / small == r["factor"], r["what"]
    # MQA's per-token cache is 2 d_h L scalars.
    assert O.kv_cache_bytes_per_token(1, 128, 80, 1, lib=lib) == 2 * 128 * 80


def pin_sdpa_decode(lib):
    rng = np.random.default_rng(11)
    B, H, D, Tmax = 3, 8, 16, 23
    seqlens = np.array([23, 9, 1], dtype=np.int32)
    for G in _divisors(H):
        q, k, v = _rand(rng, B, H, D), _rand(rng, B, Tmax, G, D), _rand(rng, B, Tmax, G, D)
        scale = 0.37
        out = O.decode(q, k, v, seqlens, scale, lib=lib)
        for b in range(B):
            modes = ["gqa", "repeat"] + (["mha"] if G == H else []) + (["mqa"] if G == 1 else [])
            for mode in modes:
                ref = _sdpa_decode(q[b], k[b], v[b], int(seqlens[b]), scale, mode)
                np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12, err_msg=f"G={G} b={b} {mode}")


def pin_sdpa_decode_bf16_storage(lib):
    """bf16 storage is read bit-exactly: the oracle on bf16 bits equals library
    attention on the same values widened to fp64."""
    gen = torch.Generator().manual_seed(5)
    B, H, G, D, Tmax = 2, 8, 2, 64, 40
    q = torch.randn(B, H, D, generator=gen).to(torch.bfloat16)
    k = torch.randn(B, Tmax, G, D, generator=gen).to(torch.bfloat16)
    v = torch.randn(B, Tmax, G, D, generator=gen).to(torch.bfloat16)
    seqlens = np.array([40, 17], dtype=np.int32)
    out = O.decode(q, k, v, seqlens, 0.125, lib=lib)
    for b in range(B):
        ref = _sdpa_decode(q[b].double().numpy(), k[b].double().numpy(), v[b].double().numpy(),
                           int(seqlens[b]), 0.125)
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def _brute_attend(qrow, keys, vals, scale):
    s = [scale * sum(a * b for a, b in zip(qrow, kr)) for kr in keys]
    m = max(s)
    p = [math.exp(x - m) for x in s]
    z = sum(p)
    return [sum(p[t] * vals[t][d] for t in range(len(keys))) / z for d in range(len(qrow))]


def pin_brute_force(lib):
    rng = np.random.default_rng(3)
    for B, H, D, T in [(1, 1, 3, 1), (2, 4, 3, 5), (1, 4, 2, 6), (2, 2, 4, 3)]:
        for G in _divisors(H):
            r = H // G
            # decode
            q, k, v = _rand(rng, B, H, D), _rand(rng, B, T, G, D), _rand(rng, B, T, G, D)
            seqlens = rng.integers(1, T + 1, size=B).astype(np.int32)
            out = O.decode(q, k, v, seqlens, 0.5, lib=lib)
            for b in range(B):
                L = int(seqlens[b])
                for h in range(H):
                    g = h // r
                    ref = _brute_attend(list(q[b, h]), [list(k[b, t, g]) for t in range(L)],
                                        [list(v[b, t, g]) for t in range(L)], 0.5)
                    np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)
            # prefill, causal and not
            qp = _rand(rng, B, T, H, D)
            for causal in (True, False):
                outp = O.prefill(qp, k, v, causal=causal, lib=lib)
                for b in range(B):
                    for t in range(T):
                        for h in range(H):
                            g = h // r
                            n = t + 1 if causal else T
                            ref = _brute_attend(list(qp[b, t, h]), [list(k[b, s, g]) for s in range(n)],
                                                [list(v[b, s, g]) for s in range(n)], 1.0 / math.sqrt(D))
                            np.testing.assert_allclose(outp[b, t, h], ref, rtol=0, atol=1e-12)


def pin_closed_forms(lib):
    rng = np.random.default_rng(7)
    B, H, G, D, Tmax = 2, 8, 4, 8, 12
    r = H // G
    q, k, v = _rand(rng, B, H, D), _rand(rng, B, Tmax, G, D), _rand(rng, B, Tmax, G, D)
    # One cached token: the output is that token's value row, exactly.
    out = O.decode(q, k, v, np.array([1, 1], np.int32), 0.3, lib=lib)
    for b in range(B):
        for h in range(H):
            assert np.array_equal(out[b, h], v[b, 0, h // r])
    # All-zero keys, or zero scale: uniform weights, the mean of the values.
    L = np.array([12, 5], np.int32)
    for kk, sc in ((np.zeros_like(k), 0.3), (k, 0.0)):
        out = O.decode(q, kk, v, L, sc, lib=lib)
        for b in range(B):
            for h in range(H):
                np.testing.assert_allclose(out[b, h], v[b, :L[b], h // r].mean(axis=0), rtol=0, atol=1e-13)
    # Two keys: weights are sigmoid(+/- score difference).
    a, scale = 1.7, 0.6
    q2 = np.zeros((1, 1, 4)); q2[0, 0, 0] = a
    k2 = np.zeros((1, 2, 1, 4)); k2[0, 0, 0, 0] = 1.0
    v2 = _rand(rng, 1, 2, 1, 4)
    w0 = 1.0 / (1.0 + math.exp(-scale * a))
    out = O.decode(q2, k2, v2, np.array([2], np.int32), scale, lib=lib)
    np.testing.assert_allclose(out[0, 0], w0 * v2[0, 0, 0] + (1 - w0) * v2[0, 1, 0], rtol=0, atol=1e-15)
    # One key far above the rest: the output is that key's value row.
    kd = np.zeros((1, 6, 1, 4)); kd[0, 4, 0, 1] = 1.0
    qd = np.zeros((1, 1, 4)); qd[0, 0, 1] = 1000.0
    out = O.decode(qd, kd, v2.repeat(3, axis=1), np.array([6], np.int32), 1.0, lib=lib)
    np.testing.assert_allclose(out[0, 0], v2.repeat(3, axis=1)[0, 4, 0], rtol=0, atol=1e-300)


def pin_probs(lib):
    rng = np.random.default_rng(9)
    B, H, G, D, Tmax = 3, 6, 3, 5, 17
    q, k, v = _rand(rng, B, H, D) * 3, _rand(rng, B, Tmax, G, D), _rand(rng, B, Tmax, G, D)
    L = np.array([17, 4, 1], np.int32)
    out, p = O.decode(q, k, v, L, 0.9, return_probs=True, lib=lib)
    for b in range(B):
        assert np.all(p[b, :, L[b]:] == 0.0)
        assert np.all(p[b, :, :L[b]] > 0.0)
        np.testing.assert_allclose(p[b].sum(axis=-1), 1.0, rtol=0, atol=1e-12)
        # out is the probability-weighted value rows
        for h in range(H):
            np.testing.assert_allclose(out[b, h], p[b, h, :L[b]] @ v[b, :L[b], h // (H // G)], atol=1e-12)


def pin_group_tag(lib):
    rng = np.random.default_rng(13)
    for H, G in [(8, 2), (64, 8), (32, 8), (16, 16), (12, 1), (12, 3)]:
        B, D, Tmax = 2, 8, 9
        q, k = _rand(rng, B, H, D), _rand(rng, B, Tmax, G, D)
        v = np.broadcast_to(np.arange(G, dtype=np.float64)[None, None, :, None], (B, Tmax, G, D)).copy()
        out = O.decode(q, k, v, np.array([9, 4], np.int32), 0.5, lib=lib)
        expect = np.repeat(np.arange(G), H // G).astype(np.float64)
        np.testing.assert_allclose(out, np.broadcast_to(expect[None, :, None], out.shape), rtol=0, atol=1e-13)


def pin_masking(lib):
    rng = np.random.default_rng(17)
    B, H, G, D, Tmax = 4, 4, 2, 6, 10
    q, k, v = _rand(rng, B, H, D), _rand(rng, B, Tmax, G, D), _rand(rng, B, Tmax, G, D)
    L = np.array([10, 3, 0, 7], np.int32)
    base = O.decode(q, k, v, L, 0.4, lib=lib)
    kp, vp = k.copy(), v.copy()
    for b in range(B):
        kp[b, L[b]:] = np.nan
        vp[b, L[b]:] = np.nan
    poisoned = O.decode(q, kp, vp, L, 0.4, lib=lib)
    assert np.array_equal(base, poisoned)
    assert np.all(base[2] == 0.0)  # zero-length sequence -> zero row
    # Lengths are clamped to [0, Tmax].
    over = O.decode(q, k, v, np.array([99, 3, -5, 7], np.int32), 0.4, lib=lib)
    assert np.array_equal(over, base)


def pin_permutation(lib):
    rng = np.random.default_rng(19)
    B, H, G, D, Tmax = 2, 8, 2, 8, 15
    q, k, v = _rand(rng, B, H, D), _rand(rng, B, Tmax, G, D), _rand(rng, B, Tmax, G, D)
    L = np.array([15, 11], np.int32)
    base = O.decode(q, k, v, L, 0.3, lib=lib)
    kp, vp = k.copy(), v.copy()
    for b in range(B):
        perm = rng.permutation(L[b])
        kp[b, :L[b]] = k[b, perm]
        vp[b, :L[b]] = v[b, perm]
    np.testing.assert_allclose(O.decode(q, kp, vp, L, 0.3, lib=lib), base, rtol=0, atol=1e-13)


def pin_prefill(lib):
    rng = np.random.default_rng(23)
    B, T, H, G, D = 2, 13, 8, 2, 8
    q, k, v = _rand(rng, B, T, H, D), _rand(rng, B, T, G, D), _rand(rng, B, T, G, D)
    scale = 1.0 / math.sqrt(D)
    for causal in (True, False):
        out = O.prefill(q, k, v, causal=causal, lib=lib)
        # library attention with the same broadcast
        qt = torch.from_numpy(q).permute(0, 2, 1, 3)
        kt = torch.from_numpy(k).permute(0, 2, 1, 3)
        vt = torch.from_numpy(v).permute(0, 2, 1, 3)
        ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, enable_gqa=True)
        np.testing.assert_allclose(out, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)
        # row t equals decode of q[:, t] over the first t+1 (or all T) positions
        for t in range(T):
            n = t + 1 if causal else T
            dec = O.decode(np.ascontiguousarray(q[:, t]), k, v, np.full(B, n, np.int32), scale, lib=lib)
            np.testing.assert_allclose(out[:, t], dec, rtol=0, atol=1e-13)
        # causal row 0 is the first value row of each head's group
        if causal:
            for h in range(H):
                assert np.array_equal(out[:, 0, h], v[:, 0, h // (H // G)])
        # a listed subset of rows equals the same rows of the full result
        rb = rng.integers(0, B, 20); rt = rng.integers(0, T, 20); rh = rng.integers(0, H, 20)
        sub = O.prefill(q, k, v, causal=causal, rows=(rb, rt, rh), lib=lib)
        np.testing.assert_array_equal(sub, out[rb, rt, rh])


def pin_mean_pool(lib):
    # hand-worked: four heads of two values each into two groups
    x = np.array([[[1.0, 2.0], [3.0, 4.0], [5.0, 6.0], [7.0, 9.0]]])
    np.testing.assert_array_equal(O.mean_pool(x, 2, lib=lib), [[[2.0, 3.0], [6.0, 7.5]]])
    np.testing.assert_array_equal(O.mean_pool(x, 1, lib=lib), [[[4.0, 5.25]]])
    rng = np.random.default_rng(29)
    N, H, D = 7, 16, 8
    x = _rand(rng, N, H, D)
    assert np.array_equal(O.mean_pool(x, H, lib=lib), x)                      # G = H: identity
    np.testing.assert_allclose(O.mean_pool(x, 1, lib=lib)[:, 0], x.mean(axis=1), rtol=0, atol=1e-14)
    for G in _divisors(H):
        np.testing.assert_allclose(O.mean_pool(x, G, lib=lib), x.reshape(N, G, H // G, D).mean(axis=2),
                                   rtol=0, atol=1e-14)
    xb = torch.randn(N, H, D, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    assert np.array_equal(O.mean_pool(xb, H, lib=lib), xb.double().numpy())
    # linearity: pool(W) applied to h equals pool of (h W)
    d, T, G = 12, 5, 4
    W = _rand(rng, d, H * D)
    h = _rand(rng, T, d)
    pooled_w = O.mean_pool(W.reshape(d, H, D), G, lib=lib).reshape(d, G * D)
    pooled_k = O.mean_pool((h @ W).reshape(T, H, D), G, lib=lib).reshape(T, G * D)
    np.testing.assert_allclose(h @ pooled_w, pooled_k, rtol=0, atol=1e-12)


def pin_f16_widen(lib):
    # every one of the 65536 fp16 bit patterns widens to numpy's own float16
    # -> float64 conversion (G = H pooling copies each value through)
    x = np.arange(65536, dtype=np.uint16).view(np.float16).reshape(64, 8, 128)
    assert np.array_equal(O.mean_pool(x, 8, lib=lib), x.astype(np.float64), equal_nan=True)
    # fp16 storage through decode equals library attention on the widened values
    rng = np.random.default_rng(11)
    B, H, G, D, Tmax = 2, 4, 2, 16, 9
    q = rng.standard_normal((B, H, D)).astype(np.float16)
    k = rng.standard_normal((B, Tmax, G, D)).astype(np.float16)
    v = rng.standard_normal((B, Tmax, G, D)).astype(np.float16)
    v.reshape(-1)[:6] = np.array([65504.0, -0.0, 6.1035156e-05, 5.9604645e-08, -2.0, 0.33325195], np.float16)
    sl = np.array([9, 4], dtype=np.int32)
    out = O.decode(q, k, v, sl, 0.25, lib=lib)
    for b in range(B):
        ref = _sdpa_decode(q[b].astype(np.float64), k[b].astype(np.float64), v[b].astype(np.float64),
                           int(sl[b]), 0.25)
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-9)


def pin_decode_append(lib):
    rng = np.random.default_rng(12)
    B, H, G, D, Tmax = 5, 8, 2, 16, 10
    q, k, v = _rand(rng, B, H, D), _rand(rng, B, Tmax, G, D), _rand(rng, B, Tmax, G, D)
    kn, vn = _rand(rng, B, G, D), _rand(rng, B, G, D)
    sl = np.array([0, 3, 9, 10, -4], dtype=np.int32)  # empty, middle, last free slot, full, negative
    for W in (0, 2):
        out, ka, va = O.decode_step(q, k, v, sl, 0.3, k_new=kn, v_new=vn, window=W, lib=lib)
        for b in range(B):
            L = min(max(int(sl[b]), 0), Tmax)
            ek, ev = k[b].copy(), v[b].copy()
            if L < Tmax:
                ek[L], ev[L] = kn[b], vn[b]
                L += 1
            assert np.array_equal(ka[b], ek) and np.array_equal(va[b], ev)  # only position L_b written
            lo = max(0, L - W) if W else 0
            np.testing.assert_allclose(out[b], _sdpa_decode(q[b], ek[lo:], ev[lo:], L - lo, 0.3),
                                       rtol=1e-12, atol=1e-12)
        # an empty sequence attends to the new token alone: its value, exactly
        assert np.array_equal(out[0], np.repeat(vn[0], H // G, axis=0))
        assert np.array_equal(out[4], np.repeat(vn[4], H // G, axis=0))


def pin_decode_window(lib):
    rng = np.random.default_rng(13)
    B, H, G, D, Tmax = 3, 6, 3, 8, 12
    q, k, v = _rand(rng, B, H, D), _rand(rng, B, Tmax, G, D), _rand(rng, B, Tmax, G, D)
    sl = np.array([12, 5, 1], dtype=np.int32)
    full = O.decode(q, k, v, sl, 0.4, lib=lib)
    for W in (1, 3, 5, 12, 20):
        out, ka, _ = O.decode_step(q, k, v, sl, 0.4, window=W, lib=lib)
        assert np.array_equal(ka, k)  # no append: the cache is untouched
        for b in range(B):
            L = int(sl[b])
            lo = max(0, L - W)
            np.testing.assert_allclose(out[b], _sdpa_decode(q[b], k[b, lo:], v[b, lo:], L - lo, 0.4),
                                       rtol=1e-12, atol=1e-12)
            if W == 1:  # one key: its value, exactly
                assert np.array_equal(out[b], np.repeat(v[b, L - 1], H // G, axis=0))
            if W >= L:  # a window covering the sequence changes nothing
                np.testing.assert_allclose(out[b], full[b], rtol=1e-13, atol=1e-13)


def pin_prefill_window(lib):
    rng = np.random.default_rng(14)
    B, T, H, G, D = 2, 13, 4, 2, 8
    q, k, v = _rand(rng, B, T, H, D), _rand(rng, B, T, G, D), _rand(rng, B, T, G, D)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(H // G, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(H // G, dim=1)
    i = torch.arange(T)
    for W in (1, 4, 13, 30):
        out = O.prefill_window(q, k, v, W, lib=lib)
        band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)  # key s in [t-W+1, t]
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=band).permute(0, 2, 1, 3).numpy()
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
        if W == 1:  # each query sees only itself
            assert np.array_equal(out, np.repeat(v, H // G, axis=2))
    rb, rt, rh = np.array([1, 0, 1]), np.array([12, 5, 0]), np.array([3, 0, 2])
    np.testing.assert_array_equal(O.prefill_window(q, k, v, 4, rows=(rb, rt, rh), lib=lib),
                                  O.prefill_window(q, k, v, 4, lib=lib)[rb, rt, rh])


def pin_weighted_pool(lib):
    rng = np.random.default_rng(15)
    N, H, G, D = 5, 8, 2, 6
    r = H // G
    x = _rand(rng, N, H, D)
    w = rng.standard_normal(H)
    ref = np.einsum("ngjd,gj->ngd", x.reshape(N, G, r, D), w.reshape(G, r))
    np.testing.assert_allclose(O.weighted_pool(x, G, w, lib=lib), ref, rtol=1e-13, atol=1e-13)
    for j in range(r):  # one-hot weights pick head j of every group, exactly
        oh = np.zeros(H)
        oh[j::r] = 1.0
        assert np.array_equal(O.weighted_pool(x, G, oh, lib=lib), x[:, j::r, :])
    np.testing.assert_allclose(O.weighted_pool(x, G, np.full(H, 1.0 / r), lib=lib),
                               x.reshape(N, G, r, D).mean(axis=2), rtol=0, atol=1e-14)


PINS = [
    pin_group_map,
    pin_cache_golden,
    pin_sdpa_decode,
    pin_sdpa_decode_bf16_storage,
    pin_brute_force,
    pin_closed_forms,
    pin_probs,
    pin_group_tag,
    pin_masking,
    pin_permutation,
    pin_prefill,
    pin_mean_pool,
    pin_f16_widen,
    pin_decode_append,
    pin_decode_window,
    pin_prefill_window,
    pin_weighted_pool,
]
