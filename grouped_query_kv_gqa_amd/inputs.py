"""Seeded synthetic inputs for grouped-query attention workloads.

This module draws random numbers and nothing else: it holds none of the
attention arithmetic, so both the GPU path and the CPU oracle can be fed from
it. Draw order is fixed (seqlens, then q, then K, then V) so that workloads
that differ only in the number of key/value heads G share seqlens and q.
Values are N(0,1) in fp32, optionally multiplied by a power of two, then
rounded to the storage dtype (round-to-nearest-even for bf16).

Workload shapes follow the model shapes the pages name: Llama 2 70B has 64
query heads, 8 key/value heads and head dimension 128 ("Grouped-Query
Attention" (llm-arch-kb), section 1 Premise and section 2 KV-cache footprint;
crackai.dev paper card, Key Takeaways). The Llama-3-8B decode shape (32 query
heads, 8 key/value heads) is a commonly used GQA layer shape.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

_CHUNK_ELEMS = 1 << 28  # draw big tensors in pieces to bound fp32 temporaries


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H: int
    G: int
    D: int
    Tmax: int
    dtype: torch.dtype
    ragged: tuple | None = None  # (lo, hi) inclusive length range, else every length is Tmax
    q_mult: float = 1.0
    description: str = ""

    @property
    def scale(self) -> float:
        return self.D ** -0.5

    def with_G(self, G: int) -> "DecodeWorkload":
        return DecodeWorkload(f"{self.name}_G{G}", self.B, self.H, G, self.D, self.Tmax, self.dtype,
                              self.ragged, self.q_mult, self.description)


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    T: int
    H: int
    G: int
    D: int
    dtype: torch.dtype
    causal: bool = True
    description: str = ""


WORKLOADS = {
    "decode_tiny_fp32": DecodeWorkload(
        "decode_tiny_fp32", B=1, H=8, G=2, D=64, Tmax=256, dtype=torch.float32,
        description="tiny GQA decode, fp32 debug path, group size 4"),
    "decode_llama3_8b": DecodeWorkload(
        "decode_llama3_8b", B=16, H=32, G=8, D=128, Tmax=4096, dtype=torch.bfloat16,
        description="Llama-3-8B-shaped GQA decode layer, every sequence at context 4096"),
    "decode_llama2_70b_ragged": DecodeWorkload(
        "decode_llama2_70b_ragged", B=64, H=64, G=8, D=128, Tmax=8192, dtype=torch.bfloat16,
        ragged=(1024, 8192),
        description="Llama-2-70B-shaped ragged GQA decode, lengths uniform in [1024, 8192]"),
    "decode_long_128k": DecodeWorkload(
        "decode_long_128k", B=1, H=64, G=8, D=128, Tmax=131072, dtype=torch.bfloat16, q_mult=2.0,
        description="long-context split-K GQA decode, one sequence of 131072 tokens, q scaled by 2"),
}

PREFILL_WORKLOADS = {
    "prefill_llama3_8b_causal": PrefillWorkload(
        "prefill_llama3_8b_causal", B=4, T=8192, H=32, G=8, D=128, dtype=torch.bfloat16,
        description="causal GQA prefill, Llama-3-8B head shape, 8192 tokens"),
}


def _randn(shape, gen: torch.Generator, device, dtype, mult: float = 1.0) -> torch.Tensor:
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, _CHUNK_ELEMS):
        e = min(n, s + _CHUNK_ELEMS)
        x = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        if mult != 1.0:
            x.mul_(mult)
        flat[s:e].copy_(x.to(dtype))
    return out


def make_generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def decode_inputs(w: DecodeWorkload, seed: int = 0, device="cpu", seqlens=None):
    """Returns dict(q [B,H,D], k_cache, v_cache [B,Tmax,G,D], seqlens [B] int32)."""
    gen = make_generator(seed, device)
    if seqlens is None:
        if w.ragged is not None:
            lo, hi = w.ragged
            seqlens = torch.randint(lo, hi + 1, (w.B,), generator=gen, device=device, dtype=torch.int64)
        else:
            seqlens = torch.full((w.B,), w.Tmax, device=device, dtype=torch.int64)
    seqlens = torch.as_tensor(seqlens, device=device).to(torch.int32)
    q = _randn((w.B, w.H, w.D), gen, device, w.dtype, w.q_mult)
    k = _randn((w.B, w.Tmax, w.G, w.D), gen, device, w.dtype)
    v = _randn((w.B, w.Tmax, w.G, w.D), gen, device, w.dtype)
    return {"q": q, "k_cache": k, "v_cache": v, "seqlens": seqlens}


def prefill_inputs(w: PrefillWorkload, seed: int = 0, device="cpu", T: int | None = None):
    """Returns dict(q [B,T,H,D], k, v [B,T,G,D]). ``T`` overrides the length
    (a prefix-sized problem drawn from its own stream)."""
    T = w.T if T is None else T
    gen = make_generator(seed, device)
    q = _randn((w.B, T, w.H, w.D), gen, device, w.dtype)
    k = _randn((w.B, T, w.G, w.D), gen, device, w.dtype)
    v = _randn((w.B, T, w.G, w.D), gen, device, w.dtype)
    return {"q": q, "k": k, "v": v}


def mean_pool_inputs(N: int, H: int, D: int, dtype=torch.bfloat16, seed: int = 0, device="cpu"):
    gen = make_generator(seed, device)
    return _randn((N, H, D), gen, device, dtype)


def random_tensor(shape, seed: int, dtype=torch.float32, device="cpu", mult: float = 1.0):
    """A standalone seeded N(0,1) tensor (used by small tests)."""
    return _randn(tuple(shape), make_generator(seed, device), device, dtype, mult)
