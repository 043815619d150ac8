"""fp64 CPU oracle for grouped-query attention (test infrastructure).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
use this module. The GPU library and its Python binding never import it, and
it imports nothing from them.

The arithmetic lives in ``gqa_oracle.c`` (plain double-precision loops, one
OpenMP thread per output row); this module only builds that file with gcc,
loads it with ctypes and passes arrays through. Inputs may be numpy arrays or
CPU torch tensors holding bf16, fp32 or fp64; bf16 is passed as its raw 16-bit
pattern and widened exactly inside the C code.

Sources: "Grouped-Query Attention" (llm-arch-kb), sections 1-3; the crackai.dev
paper card "GQA: Training Generalized Multi-Query Transformer Models from
Multi-Head Checkpoints", How It Works; "Multi-Query and Grouped-Query
Attention" (praveentn.live). Every function cites its passage in the C file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BF16, F32, F64, F16 = 0, 1, 2, 3

_lib = None


def build(src: str = _SRC, out: str = _LIB_PATH, extra_flags=()) -> str:
    """Compile the oracle with gcc (fp64, no fast-math) into a shared library."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           *extra_flags, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _declare(lib):
    c_void_p, c_int, c_double, c_int64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_int64
    lib.oracle_group_of_head.argtypes = [c_int, c_int, c_int]
    lib.oracle_group_of_head.restype = c_int
    lib.oracle_kv_cache_bytes_per_token.argtypes = [c_int, c_int, c_int, c_int]
    lib.oracle_kv_cache_bytes_per_token.restype = c_double
    lib.oracle_decode.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_int, c_int, c_int,
                                  c_int, c_int, c_double, c_void_p, c_void_p]
    lib.oracle_decode.restype = None
    lib.oracle_prefill.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                   c_int, c_int, c_void_p, c_void_p, c_void_p, c_int64, c_void_p]
    lib.oracle_prefill.restype = None
    lib.oracle_mean_pool.argtypes = [c_void_p, c_int, c_int64, c_int, c_int, c_int, c_void_p]
    lib.oracle_mean_pool.restype = None
    lib.oracle_decode_step.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_int,
                                       c_int, c_int, c_int, c_int, c_double, c_int, c_void_p]
    lib.oracle_decode_step.restype = None
    lib.oracle_prefill_window.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                          c_int, c_int, c_void_p, c_void_p, c_void_p, c_int64, c_void_p]
    lib.oracle_prefill_window.restype = None
    lib.oracle_weighted_pool.argtypes = [c_void_p, c_int, c_int64, c_int, c_int, c_int, c_void_p, c_void_p]
    lib.oracle_weighted_pool.restype = None
    lib.oracle_set_threads.argtypes = [c_int]
    lib.oracle_set_threads.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = c_int
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle library. A custom ``path``
    loads another build of an oracle source, as the mutation tests do."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def _as_array(x):
    """Return (contiguous numpy array, dtype code). bf16 torch tensors become
    their uint16 bit patterns; everything else keeps its precision."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.device.type != "cpu":
                raise ValueError("oracle inputs must be CPU tensors")
            if x.dtype == torch.bfloat16:
                return np.ascontiguousarray(x.contiguous().view(torch.int16).numpy().view(np.uint16)), BF16
            if x.dtype == torch.float16:
                return np.ascontiguousarray(x.contiguous().view(torch.int16).numpy().view(np.uint16)), F16
            x = x.contiguous().numpy()
    except ImportError:
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, BF16
    if x.dtype == np.float16:
        return x.view(np.uint16), F16
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.float64:
        return x, F64
    raise TypeError(f"unsupported oracle input dtype {x.dtype}")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _same_kind(*arrs):
    codes = {c for _, c in arrs}
    if len(codes) != 1:
        raise TypeError("q, k, v must share one storage type")
    return codes.pop()


def group_of_head(h: int, H: int, G: int, lib=None) -> int:
    return (lib or load()).oracle_group_of_head(h, H, G)


def kv_cache_bytes_per_token(kv_heads: int, d_h: int, layers: int, bytes_per_scalar: int, lib=None) -> float:
    return (lib or load()).oracle_kv_cache_bytes_per_token(kv_heads, d_h, layers, bytes_per_scalar)


def decode(q, k_cache, v_cache, seqlens, scale: float, return_probs: bool = False, lib=None):
    """out[b,h,:] over cache positions [0, L_b); q [B,H,D], cache [B,Tmax,G,D]."""
    lib = lib or load()
    qa, ka, va = _as_array(q), _as_array(k_cache), _as_array(v_cache)
    dtype = _same_kind(qa, ka, va)
    qa, ka, va = qa[0], ka[0], va[0]
    B, H, D = qa.shape
    Bk, Tmax, G, Dk = ka.shape
    assert (Bk, Dk) == (B, D) and va.shape == ka.shape
    sl = np.ascontiguousarray(np.asarray(seqlens if not hasattr(seqlens, "numpy") else seqlens.numpy(),
                                         dtype=np.int32))
    assert sl.shape == (B,)
    out = np.empty((B, H, D), dtype=np.float64)
    probs = np.empty((B, H, Tmax), dtype=np.float64) if return_probs else None
    lib.oracle_decode(_ptr(qa), _ptr(ka), _ptr(va), dtype, _ptr(sl), B, H, G, D, Tmax, float(scale),
                      _ptr(out), _ptr(probs) if probs is not None else None)
    return (out, probs) if return_probs else out


def prefill(q, k, v, causal: bool = True, rows=None, lib=None):
    """q [B,T,H,D], k/v [B,T,G,D]. rows=None -> out [B,T,H,D]; rows = (b, t, h)
    index arrays -> out [len(rows), D]."""
    lib = lib or load()
    qa, ka, va = _as_array(q), _as_array(k), _as_array(v)
    dtype = _same_kind(qa, ka, va)
    qa, ka, va = qa[0], ka[0], va[0]
    B, T, H, D = qa.shape
    G = ka.shape[2]
    assert ka.shape == (B, T, G, D) and va.shape == ka.shape
    if rows is None:
        out = np.empty((B, T, H, D), dtype=np.float64)
        lib.oracle_prefill(_ptr(qa), _ptr(ka), _ptr(va), dtype, B, T, H, G, D, int(bool(causal)),
                           None, None, None, 0, _ptr(out))
        return out
    rb, rt, rh = (np.ascontiguousarray(np.asarray(a, dtype=np.int32)) for a in rows)
    n = rb.shape[0]
    out = np.empty((n, D), dtype=np.float64)
    lib.oracle_prefill(_ptr(qa), _ptr(ka), _ptr(va), dtype, B, T, H, G, D, int(bool(causal)),
                       _ptr(rb), _ptr(rt), _ptr(rh), n, _ptr(out))
    return out


def _seqlens(seqlens, B):
    sl = np.ascontiguousarray(np.asarray(seqlens if not hasattr(seqlens, "numpy") else seqlens.numpy(),
                                         dtype=np.int32))
    assert sl.shape == (B,)
    return sl


def decode_step(q, k_cache, v_cache, seqlens, scale: float, k_new=None, v_new=None, window: int = 0, lib=None):
    """Decode with an optional cache append (k_new, v_new [B,G,D]) and an
    optional sliding window. Returns (out [B,H,D] fp64, k_after, v_after):
    the caches after the append, as arrays of the stored bits (the inputs are
    not modified)."""
    lib = lib or load()
    qa, ka, va = _as_array(q), _as_array(k_cache), _as_array(v_cache)
    arrs = [qa, ka, va]
    if k_new is not None:
        kn, vn = _as_array(k_new), _as_array(v_new)
        arrs += [kn, vn]
    dtype = _same_kind(*arrs)
    qa = qa[0]
    ka, va = ka[0].copy(), va[0].copy()
    B, H, D = qa.shape
    Bk, Tmax, G, Dk = ka.shape
    assert (Bk, Dk) == (B, D) and va.shape == ka.shape
    kp = vp = None
    if k_new is not None:
        kn, vn = kn[0], vn[0]
        assert kn.shape == (B, G, D) and vn.shape == (B, G, D)
        kp, vp = _ptr(kn), _ptr(vn)
    sl = _seqlens(seqlens, B)
    out = np.empty((B, H, D), dtype=np.float64)
    lib.oracle_decode_step(_ptr(qa), kp, vp, _ptr(ka), _ptr(va), dtype, _ptr(sl), B, H, G, D, Tmax, float(scale),
                           int(window), _ptr(out))
    return out, ka, va


def prefill_window(q, k, v, window: int, rows=None, lib=None):
    """Causal prefill where query t sees keys [max(0, t+1-window), t]."""
    lib = lib or load()
    qa, ka, va = _as_array(q), _as_array(k), _as_array(v)
    dtype = _same_kind(qa, ka, va)
    qa, ka, va = qa[0], ka[0], va[0]
    B, T, H, D = qa.shape
    G = ka.shape[2]
    assert ka.shape == (B, T, G, D) and va.shape == ka.shape
    if rows is None:
        out = np.empty((B, T, H, D), dtype=np.float64)
        lib.oracle_prefill_window(_ptr(qa), _ptr(ka), _ptr(va), dtype, B, T, H, G, D, int(window),
                                  None, None, None, 0, _ptr(out))
        return out
    rb, rt, rh = (np.ascontiguousarray(np.asarray(a, dtype=np.int32)) for a in rows)
    out = np.empty((rb.shape[0], D), dtype=np.float64)
    lib.oracle_prefill_window(_ptr(qa), _ptr(ka), _ptr(va), dtype, B, T, H, G, D, int(window),
                              _ptr(rb), _ptr(rt), _ptr(rh), rb.shape[0], _ptr(out))
    return out


def weighted_pool(x, G: int, w, lib=None):
    """x [N,H,D], w [H] -> [N,G,D]: group g = sum of w[i] x[:, i, :] over its heads."""
    lib = lib or load()
    xa, dtype = _as_array(x)
    N, H, D = xa.shape
    wa = np.ascontiguousarray(np.asarray(w.numpy() if hasattr(w, "numpy") else w, dtype=np.float64))
    assert wa.shape == (H,)
    out = np.empty((N, G, D), dtype=np.float64)
    lib.oracle_weighted_pool(_ptr(xa), dtype, N, H, G, D, _ptr(wa), _ptr(out))
    return out


def mean_pool(x, G: int, lib=None):
    """x [N,H,D] -> [N,G,D], the mean of each group's heads."""
    lib = lib or load()
    xa, dtype = _as_array(x)
    N, H, D = xa.shape
    out = np.empty((N, G, D), dtype=np.float64)
    lib.oracle_mean_pool(_ptr(xa), dtype, N, H, G, D, _ptr(out))
    return out


def set_threads(n: int, lib=None):
    (lib or load()).oracle_set_threads(int(n))


def max_threads(lib=None) -> int:
    return (lib or load()).oracle_max_threads()
