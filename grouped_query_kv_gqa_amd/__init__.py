"""grouped_query_kv_gqa_amd -- grouped-query attention over a KV cache on
AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libgqa.so`` (C ABI in ``include/gqa.h``). Every
step of the computation runs in the library's HIP kernels; this module only
checks torch tensors (device, dtype, shape, contiguity), passes their data
pointers and the current HIP stream, and raises ``GqaError`` on a non-zero
status. There is no CPU fallback: if the library is missing, every call
raises.

  decode(q, k_cache, v_cache, seqlens, scale=None, out=None, split_tokens=0)
  prefill(q, k, v, causal=True, out=None)
  mean_pool_kv(x, G, out=None)

Inside ``with debug_build():`` the calls go to ``libgqa_debug.so`` instead,
the same kernels with a range check at every global memory access;
``debug_checks()`` reads (and clears) the violations they recorded.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

__all__ = ["GqaError", "decode", "decode_step", "prefill", "mean_pool_kv", "weighted_pool_kv", "decode_plan",
           "release_workspaces", "library_path", "load_library", "debug_build", "debug_checks"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libgqa.so")
_DEBUG_LIB_PATH = os.path.join(_PKG, "libgqa_debug.so")

GQA_OK, GQA_ERR_INVALID_ARG, GQA_ERR_UNSUPPORTED, GQA_ERR_HIP = 0, 1, 2, 3
GQA_BF16, GQA_FP32, GQA_FP16 = 0, 1, 2

_lib = None


class GqaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"gqa status {status}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


_debug_lib = None
_use_debug = False


def load_library():
    """Load libgqa.so (torch is imported first, so the library binds to the
    HIP runtime torch already loaded); libgqa_debug.so inside debug_build()."""
    global _lib, _debug_lib
    if _use_debug:
        if _debug_lib is None:
            _debug_lib = _open(_DEBUG_LIB_PATH)
        return _debug_lib
    if _lib is None:
        _lib = _open(_LIB_PATH)
    return _lib


@contextlib.contextmanager
def debug_build():
    """Route this module's calls to libgqa_debug.so inside the block."""
    global _use_debug
    prev = _use_debug
    _use_debug = True
    try:
        yield
    finally:
        _use_debug = prev


def debug_checks():
    """(enabled, flags) from gqa_debug_checks of the library in use: enabled
    is False for the release library; flags (0 = none) are the range-check
    violations recorded on the current device since the last call."""
    lib = load_library()
    en, fl = ctypes.c_int(), ctypes.c_uint32()
    _check(lib.gqa_debug_checks(ctypes.byref(en), ctypes.byref(fl)))
    return bool(en.value), fl.value


def _open(path: str):
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m grouped_query_kv_gqa_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.gqa_decode.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp]
    lib.gqa_decode_ex.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp, i32]
    lib.gqa_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, i32, vp, vp]
    lib.gqa_decode_step_noalloc.argtypes = list(lib.gqa_decode_step.argtypes)
    lib.gqa_prefill.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.gqa_prefill_ex.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.gqa_mean_pool_kv.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp]
    lib.gqa_weighted_pool_kv.argtypes = [vp, vp, i64, i32, i32, i32, i32, vp, vp]
    lib.gqa_decode_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(i32),
                                    ctypes.POINTER(i32), ctypes.POINTER(i64)]
    for fn in ("gqa_decode", "gqa_decode_ex", "gqa_decode_step", "gqa_decode_step_noalloc", "gqa_prefill",
               "gqa_prefill_ex",
               "gqa_mean_pool_kv", "gqa_weighted_pool_kv", "gqa_decode_plan"):
        getattr(lib, fn).restype = i32
    lib.gqa_status_string.argtypes = [i32]
    lib.gqa_status_string.restype = ctypes.c_char_p
    lib.gqa_last_hip_error.argtypes = []
    lib.gqa_last_hip_error.restype = ctypes.c_char_p
    lib.gqa_last_error.argtypes = []
    lib.gqa_last_error.restype = ctypes.c_char_p
    lib.gqa_release_workspaces.argtypes = []
    lib.gqa_release_workspaces.restype = i32
    lib.gqa_abi_version.argtypes = []
    lib.gqa_abi_version.restype = i32
    lib.gqa_debug_checks.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_uint32)]
    lib.gqa_debug_checks.restype = i32
    lib.gqa_debug_selftest.argtypes = [vp]
    lib.gqa_debug_selftest.restype = i32
    return lib


def _check(status: int):
    if status != GQA_OK:
        lib = load_library()
        raise GqaError(status, lib.gqa_last_hip_error().decode() or lib.gqa_status_string(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GQA_BF16
    if t.dtype == torch.float32:
        return GQA_FP32
    if t.dtype == torch.float16:
        return GQA_FP16
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16, float16 or float32")


def _need_device(*ts: torch.Tensor):
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    for t in ts:
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _stream_ptr(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def decode(q, k_cache, v_cache, seqlens, scale: float | None = None, out=None, split_tokens: int = 0):
    """One decode step. q [B,H,D]; k_cache, v_cache [B,Tmax,G,D]; seqlens [B]
    int32 on the device. Returns out [B,H,D] (same dtype as q)."""
    lib = load_library()
    B, H, D = q.shape
    Bk, Tmax, G, Dk = k_cache.shape
    if (Bk, Dk) != (B, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between q, k_cache and v_cache")
    if seqlens.dtype != torch.int32 or tuple(seqlens.shape) != (B,):
        raise ValueError("seqlens must be int32 of shape [B]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share a dtype")
    dev = _need_device(q, k_cache, v_cache, seqlens)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_device(out)
        if out.shape != q.shape or out.dtype != q.dtype or out.device != dev:
            raise ValueError("out must match q")
    if scale is None:
        scale = float("nan")  # the library's default, 1/sqrt(d_h)
    with torch.cuda.device(dev):
        _check(lib.gqa_decode_ex(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seqlens.data_ptr(),
                                 B, H, G, D, Tmax, float(scale), _dtype_code(q), out.data_ptr(),
                                 _stream_ptr(dev), int(split_tokens)))
    return out


def decode_step(q, k_cache, v_cache, seqlens, scale: float | None = None, k_new=None, v_new=None, window: int = 0,
                out=None, split_tokens: int = 0):
    """One decode step with an optional cache append and sliding window.
    k_new, v_new [B,G,D] (or None): written into the caches at position
    clamp(seqlens[b]) when that is below Tmax, and attended as the newest
    position; seqlens is not advanced. window > 0: only the `window` newest
    positions are read. Returns out [B,H,D]."""
    lib = load_library()
    B, H, D = q.shape
    Bk, Tmax, G, Dk = k_cache.shape
    if (Bk, Dk) != (B, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between q, k_cache and v_cache")
    if seqlens.dtype != torch.int32 or tuple(seqlens.shape) != (B,):
        raise ValueError("seqlens must be int32 of shape [B]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share a dtype")
    tensors = [q, k_cache, v_cache, seqlens]
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        if tuple(k_new.shape) != (B, G, D) or tuple(v_new.shape) != (B, G, D):
            raise ValueError("k_new and v_new must be [B, G, d_h]")
        if k_new.dtype != q.dtype or v_new.dtype != q.dtype:
            raise TypeError("k_new and v_new must share q's dtype")
        tensors += [k_new, v_new]
    dev = _need_device(*tensors)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_device(out)
        if out.shape != q.shape or out.dtype != q.dtype or out.device != dev:
            raise ValueError("out must match q")
    if scale is None:
        scale = float("nan")  # the library's default, 1/sqrt(d_h)
    kn = k_new.data_ptr() if k_new is not None else None
    vn = v_new.data_ptr() if v_new is not None else None
    with torch.cuda.device(dev):
        _check(lib.gqa_decode_step(q.data_ptr(), kn, vn, k_cache.data_ptr(), v_cache.data_ptr(),
                                   seqlens.data_ptr(), B, H, G, D, Tmax, float(scale), int(window),
                                   int(split_tokens), _dtype_code(q), out.data_ptr(), _stream_ptr(dev)))
    return out


def prefill(q, k, v, causal: bool = True, out=None, window: int = 0):
    """q [B,T,H,D]; k, v [B,T,G,D]. Returns out [B,T,H,D], scale 1/sqrt(D).
    window > 0 (causal only): query t sees keys [t + 1 - window, t]."""
    lib = load_library()
    B, T, H, D = q.shape
    if k.shape[:2] != (B, T) or k.shape[3] != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch between q, k and v")
    G = k.shape[2]
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    dev = _need_device(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != dev or not out.is_contiguous():
        raise ValueError("out must match q")
    with torch.cuda.device(dev):
        _check(lib.gqa_prefill_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, H, G, D, int(bool(causal)),
                                  int(window), _dtype_code(q), out.data_ptr(), _stream_ptr(dev)))
    return out


def mean_pool_kv(x, G: int, out=None):
    """x [N,H,D] -> [N,G,D]: each group is the mean of its H/G heads."""
    lib = load_library()
    N, H, D = x.shape
    dev = _need_device(x)
    if out is None:
        out = torch.empty((N, G, D), dtype=x.dtype, device=dev)
    elif tuple(out.shape) != (N, G, D) or out.dtype != x.dtype or out.device != dev or not out.is_contiguous():
        raise ValueError("out must be [N,G,D] like x")
    with torch.cuda.device(dev):
        _check(lib.gqa_mean_pool_kv(x.data_ptr(), N, H, G, D, _dtype_code(x), out.data_ptr(), _stream_ptr(dev)))
    return out


def weighted_pool_kv(x, weights, G: int, out=None):
    """x [N,H,D], weights [H] float32 on the device -> [N,G,D]: group g is
    sum_j weights[g*r + j] * x[:, g*r + j, :] (r = H/G)."""
    lib = load_library()
    N, H, D = x.shape
    if weights.dtype != torch.float32 or tuple(weights.shape) != (H,):
        raise ValueError("weights must be float32 of shape [H]")
    dev = _need_device(x, weights)
    if out is None:
        out = torch.empty((N, G, D), dtype=x.dtype, device=dev)
    elif tuple(out.shape) != (N, G, D) or out.dtype != x.dtype or out.device != dev or not out.is_contiguous():
        raise ValueError("out must be [N,G,D] like x")
    with torch.cuda.device(dev):
        _check(lib.gqa_weighted_pool_kv(x.data_ptr(), weights.data_ptr(), N, H, G, D, _dtype_code(x),
                                        out.data_ptr(), _stream_ptr(dev)))
    return out


def release_workspaces():
    """Free every decode workspace the library holds (waits for the devices
    first). Graphs captured earlier must not be replayed afterwards."""
    _check(load_library().gqa_release_workspaces())


def decode_plan(B, H, G, D, Tmax, dtype=torch.bfloat16, split_tokens=0, cu_count=256):
    """(chunk_tokens, num_splits, workspace_bytes) of the decode split plan; host only."""
    lib = load_library()
    chunk, splits, ws = ctypes.c_int(), ctypes.c_int(), ctypes.c_int64()
    code = {torch.bfloat16: GQA_BF16, torch.float16: GQA_FP16}.get(dtype, GQA_FP32)
    _check(lib.gqa_decode_plan(B, H, G, D, Tmax, code, split_tokens, cu_count, ctypes.byref(chunk),
                               ctypes.byref(splits), ctypes.byref(ws)))
    return chunk.value, splits.value, ws.value
