"""The C ABI library on the CPU: it loads, exports every function the header
declares, and its host-side checks and split planner behave as documented.
No call here reaches the GPU (each returns before touching HIP)."""
import ctypes
import os
import re
import subprocess

import pytest

import grouped_query_kv_gqa_amd as gq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gqa_\w+)\s*\(", text, re.M)))


def test_header_symbols_exported():
    names = _declared()
    assert {"gqa_decode", "gqa_decode_ex", "gqa_prefill", "gqa_mean_pool_kv", "gqa_decode_plan",
            "gqa_status_string", "gqa_last_error", "gqa_abi_version"} <= set(names)
    lib = ctypes.CDLL(gq.library_path())
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", gq.library_path()], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}\b", out), f"{n} not a defined text symbol"


def test_status_strings():
    lib = gq.load_library()
    assert lib.gqa_status_string(0) == b"ok"
    assert lib.gqa_status_string(1) == b"invalid argument"
    assert lib.gqa_status_string(2) == b"unsupported"
    assert lib.gqa_status_string(3) == b"HIP runtime error"
    assert lib.gqa_abi_version() == 1


def _decode(lib, **kw):
    a = dict(q=16, k=32, v=48, sl=64, B=2, H=8, G=2, D=128, T=10, scale=1.0, dt=0, out=4096, stream=None, split=0)
    a.update(kw)
    return lib.gqa_decode_ex(a["q"], a["k"], a["v"], a["sl"], a["B"], a["H"], a["G"], a["D"], a["T"], a["scale"],
                             a["dt"], a["out"], a["stream"], a["split"])


def test_decode_argument_checks():
    lib = gq.load_library()
    assert _decode(lib, G=3) == gq.GQA_ERR_INVALID_ARG
    assert b"divide" in lib.gqa_last_error()
    assert _decode(lib, H=0) == gq.GQA_ERR_INVALID_ARG
    assert _decode(lib, B=-1) == gq.GQA_ERR_INVALID_ARG
    assert _decode(lib, T=-1) == gq.GQA_ERR_INVALID_ARG
    assert _decode(lib, D=96) == gq.GQA_ERR_UNSUPPORTED
    assert _decode(lib, dt=7) == gq.GQA_ERR_UNSUPPORTED
    assert _decode(lib, scale=float("inf")) == gq.GQA_ERR_INVALID_ARG
    assert _decode(lib, q=None) == gq.GQA_ERR_INVALID_ARG
    assert _decode(lib, sl=None) == gq.GQA_ERR_INVALID_ARG
    assert _decode(lib, q=18) == gq.GQA_ERR_INVALID_ARG          # misaligned
    assert b"aligned" in lib.gqa_last_error()
    assert _decode(lib, out=48) == gq.GQA_ERR_INVALID_ARG         # out aliases v
    assert b"overlaps" in lib.gqa_last_error()
    assert _decode(lib, split=-5) == gq.GQA_ERR_INVALID_ARG
    assert _decode(lib, B=0, q=None, k=None, v=None, sl=None, out=None) == gq.GQA_OK  # empty batch


def test_prefill_and_pool_argument_checks():
    lib = gq.load_library()
    pf = lib.gqa_prefill
    assert pf(16, 32, 48, 1, 4, 6, 4, 128, 1, 0, 4096, None) == gq.GQA_ERR_INVALID_ARG  # G does not divide H
    assert pf(16, 32, 48, 1, 4, 8, 2, 128, 2, 0, 4096, None) == gq.GQA_ERR_INVALID_ARG  # causal not 0/1
    assert pf(16, 32, 48, 1, 4, 8, 2, 80, 1, 0, 4096, None) == gq.GQA_ERR_UNSUPPORTED
    assert pf(None, None, None, 0, 4, 8, 2, 128, 1, 0, None, None) == gq.GQA_OK      # empty batch
    assert pf(None, None, None, 3, 0, 8, 2, 128, 1, 0, None, None) == gq.GQA_OK      # empty sequences
    mp = lib.gqa_mean_pool_kv
    assert mp(16, 10, 8, 3, 128, 0, 1 << 20, None) == gq.GQA_ERR_INVALID_ARG
    assert mp(16, 10, 8, 2, 12, 0, 1 << 20, None) == gq.GQA_ERR_UNSUPPORTED
    assert mp(16, 10, 8, 2, 128, 0, 32, None) == gq.GQA_ERR_INVALID_ARG              # overlap
    assert mp(None, 0, 8, 2, 128, 0, None, None) == gq.GQA_OK


def test_decode_plan():
    # Llama-3-8B decode shape: one 8-wave workgroup (8 groups) per CU, the
    # 16 x 4096 positions cut into 256 slices of 256
    chunk, nwg, ws = gq.decode_plan(16, 32, 8, 128, 4096)
    assert (chunk, nwg) == (256, 256)
    slots = (256 + 16) * 32
    assert ws == slots * 128 * 4 + slots * 4
    # explicit slice lengths round up to 32 positions
    assert gq.decode_plan(2, 8, 2, 128, 1000, split_tokens=100)[:2] == (128, 16)
    assert gq.decode_plan(2, 8, 2, 128, 1000, split_tokens=5000)[:2] == (5024, 1)
    # one long sequence spread over every CU
    assert gq.decode_plan(1, 64, 8, 128, 131072)[:2] == (512, 256)
    # fp32 never splits
    import torch
    assert gq.decode_plan(1, 8, 2, 64, 256, dtype=torch.float32) == (256, 1, 0)


def test_host_plan_sanitized(tmp_path):
    """The planner and checks, built host-only with g++ under ASan/UBSan."""
    src = tmp_path / "t.cpp"
    src.write_text(r'''
#include "plan.h"
#include <cassert>
#include <cstdio>
int main() {
  std::string e; gqa::DecodePlan p;
  for (int B : {0, 1, 3, 64}) for (int H : {1, 8, 32, 64, 128}) for (int G = 1; G <= H; ++G) {
    if (H % G) continue;
    for (int T : {0, 1, 31, 32, 33, 4096, 131072}) for (int s : {0, 32, 100, 1 << 20}) for (int bpc : {0, 1, 2}) {
      assert(gqa::plan_decode(B, H, G, 128, T, GQA_BF16, s, 256, bpc, &p, &e) == GQA_OK);
      assert(p.head_tiles * 16 * p.nt >= H / G && G % p.gb == 0 && p.waves % p.gb == 0);
      if (B == 0) continue;
      assert(p.nwg >= 1 && p.full_P >= 32 && p.full_P % 32 == 0);
      assert((int64_t)p.full_P * p.nwg >= (int64_t)B * T);
      assert(p.workspace_bytes >= p.lse_offset + ((int64_t)p.nwg + B) * H * 4);
      assert(p.lse_offset >= ((int64_t)p.nwg + B) * H * 128 * 4);
    }
  }
  assert(gqa::plan_decode(1, 6, 4, 128, 10, GQA_BF16, 0, 256, 0, &p, &e) == GQA_ERR_INVALID_ARG);
  char buf[64];
  assert(gqa::check_decode(buf, buf + 16, buf + 32, (const int32_t*)buf, 1, 8, 2, 128, 1, 1.f, GQA_BF16, buf, &e) == GQA_ERR_INVALID_ARG);
  std::puts("ok");
  return 0;
}
''')
    exe = tmp_path / "t"
    csrc = os.path.join(ROOT, "grouped_query_kv_gqa_amd", "csrc")
    subprocess.run(["g++", "-std=c++20", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    f"-I{csrc}", f"-I{os.path.join(ROOT, 'include')}", str(src), os.path.join(csrc, "plan.cpp"),
                    "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "ok" in r.stdout, r.stderr
