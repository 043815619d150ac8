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
            "gqa_status_string", "gqa_last_hip_error", "gqa_last_error", "gqa_release_workspaces",
            "gqa_abi_version"} <= set(names)
    lib = ctypes.CDLL(gq.library_path())
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", gq.library_path()], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}\b", out), f"{n} not a defined text symbol"


def test_debug_library_exports_the_same_symbols():
    # libgqa_debug.so: the same sources with device range checks compiled in
    dbg = os.path.join(os.path.dirname(gq.library_path()), "libgqa_debug.so")
    out = subprocess.run(["nm", "-D", "--defined-only", dbg], capture_output=True, text=True).stdout
    for n in _declared():
        assert re.search(rf"\bT {n}\b", out), f"{n} not defined in libgqa_debug.so"


def test_release_library_has_no_debug_checks():
    lib = gq.load_library()
    en, fl = ctypes.c_int(-1), ctypes.c_uint32(7)
    assert lib.gqa_debug_checks(ctypes.byref(en), ctypes.byref(fl)) == gq.GQA_OK
    assert (en.value, fl.value) == (0, 0)
    assert lib.gqa_debug_checks(None, None) == gq.GQA_OK
    assert lib.gqa_debug_selftest(None) == gq.GQA_ERR_UNSUPPORTED


def test_status_strings():
    lib = gq.load_library()
    assert lib.gqa_status_string(0) == b"ok"
    assert lib.gqa_status_string(1) == b"invalid argument"
    assert lib.gqa_status_string(2) == b"unsupported"
    assert lib.gqa_status_string(3) == b"HIP runtime error"
    assert lib.gqa_abi_version() == 2


def _decode(lib, **kw):
    a = dict(q=16, k=32, v=48, sl=64, B=2, H=8, G=2, D=128, T=10, scale=1.0, dt=0, out=4096, stream=None, split=0)
    a.update(kw)
    return lib.gqa_decode_ex(a["q"], a["k"], a["v"], a["sl"], a["B"], a["H"], a["G"], a["D"], a["T"], a["scale"],
                             a["dt"], a["out"], a["stream"], a["split"])


def test_decode_argument_checks():
    lib = gq.load_library()
    assert _decode(lib, G=3) == gq.GQA_ERR_INVALID_ARG
    assert b"divide" in lib.gqa_last_hip_error()
    assert lib.gqa_last_error() == lib.gqa_last_hip_error()
    assert _decode(lib, H=0) == gq.GQA_ERR_INVALID_ARG
    assert _decode(lib, B=-1) == gq.GQA_ERR_INVALID_ARG
    assert _decode(lib, T=-1) == gq.GQA_ERR_INVALID_ARG
    assert _decode(lib, D=96) == gq.GQA_ERR_UNSUPPORTED
    assert _decode(lib, dt=7) == gq.GQA_ERR_UNSUPPORTED
    assert _decode(lib, scale=float("inf")) == gq.GQA_ERR_INVALID_ARG
    assert _decode(lib, scale=float("-inf")) == gq.GQA_ERR_INVALID_ARG  # NaN instead selects 1/sqrt(d_h)
    assert _decode(lib, q=None) == gq.GQA_ERR_INVALID_ARG
    assert _decode(lib, sl=None) == gq.GQA_ERR_INVALID_ARG
    assert _decode(lib, q=18) == gq.GQA_ERR_INVALID_ARG          # misaligned
    assert b"aligned" in lib.gqa_last_hip_error()
    assert _decode(lib, out=48) == gq.GQA_ERR_INVALID_ARG         # out aliases v
    assert b"overlaps" in lib.gqa_last_hip_error()
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
    # explicit slice lengths round up to 32 positions and charge no startup
    assert gq.decode_plan(2, 8, 2, 128, 1000, split_tokens=100)[:2] == (128, 16)
    assert gq.decode_plan(2, 8, 2, 128, 1000, split_tokens=5000)[:2] == (5024, 1)
    # one long sequence spread over every CU
    assert gq.decode_plan(1, 64, 8, 128, 131072)[:2] == (512, 256)
    # multi-query (one group of 64 heads, the wide kernel): one 8-wave
    # workgroup per CU reading 512 B per position, charged 512 KiB / 512 B =
    # 1024 startup positions per sequence: 64 x (8192 + 1024) / 256 = 2304
    assert gq.decode_plan(64, 64, 1, 128, 8192)[:2] == (2304, 256)
    # fp32 never splits
    import torch
    assert gq.decode_plan(1, 8, 2, 64, 256, dtype=torch.float32) == (256, 1, 0)
    # the plan applies the same size limits as the decode call
    for args in [(65536, 8, 2, 128, 16), (2, 8, 2, 128, 1 << 30)]:
        with pytest.raises(gq.GqaError) as e:
            gq.decode_plan(*args)
        assert e.value.status == gq.GQA_ERR_UNSUPPORTED
        assert _decode(gq.load_library(), B=args[0], T=args[4], q=1 << 40, k=2 << 40, v=3 << 40, sl=4 << 40,
                       out=5 << 40) == gq.GQA_ERR_UNSUPPORTED


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
      assert((p.wide ? 64 : p.head_tiles * 16 * p.nt) >= H / G && G % p.gb == 0 && p.waves % p.gb == 0);
      assert(p.wide == (H / G > 32 && H / G <= 64));
      if (B == 0) continue;
      assert(p.nwg >= 1 && p.full_P >= 32 && p.full_P % 32 == 0);
      assert((int64_t)p.full_P * p.nwg >= (int64_t)B * T);
      assert(p.workspace_bytes >= p.lse_offset + ((int64_t)p.nwg + B) * H * 4);
      assert(p.lse_offset >= ((int64_t)p.nwg + B) * H * 128 * 4);
    }
  }
  assert(gqa::plan_decode(1, 6, 4, 128, 10, GQA_BF16, 0, 256, 0, &p, &e) == GQA_ERR_INVALID_ARG);
  // launch limits: merge grid rows, 31-bit flat positions, 2^32 work-items
  assert(gqa::plan_decode(65535, 8, 2, 128, 16, GQA_BF16, 0, 256, 0, &p, &e) == GQA_OK);
  assert(gqa::plan_decode(65536, 8, 2, 128, 16, GQA_BF16, 0, 256, 0, &p, &e) == GQA_ERR_UNSUPPORTED);
  assert(gqa::plan_decode(65536, 8, 2, 128, 16, GQA_FP32, 0, 256, 0, &p, &e) == GQA_ERR_UNSUPPORTED);
  assert(gqa::plan_decode(2, 8, 2, 128, 1 << 30, GQA_BF16, 0, 256, 0, &p, &e) == GQA_ERR_UNSUPPORTED);
  assert(gqa::plan_decode(1, 8, 2, 128, 1 << 30, GQA_BF16, 0, 256, 0, &p, &e) == GQA_OK);
  assert(gqa::plan_decode(1, 8, 2, 128, 1 << 30, GQA_BF16, 32, 256, 0, &p, &e) == GQA_ERR_UNSUPPORTED);
  assert(gqa::plan_decode(1, 8, 2, 128, 1 << 30, GQA_BF16, 4096, 256, 0, &p, &e) == GQA_OK);
  assert(gqa::plan_decode(65535, 2048, 2, 128, 1, GQA_FP32, 0, 256, 0, &p, &e) == GQA_ERR_UNSUPPORTED);
  assert(gqa::check_prefill_launch(65535, 8, 8, 2, 128, GQA_BF16, &e) == GQA_OK);
  assert(gqa::check_prefill_launch(65536, 8, 8, 2, 128, GQA_BF16, &e) == GQA_ERR_UNSUPPORTED);
  assert(gqa::check_prefill_launch(1, 1 << 24, 64, 8, 128, GQA_BF16, &e) == GQA_OK);
  assert(gqa::check_prefill_launch(1, 1 << 24, 128, 8, 128, GQA_BF16, &e) == GQA_ERR_UNSUPPORTED);
  assert(gqa::check_prefill_launch(1, 1 << 21, 64, 8, 128, GQA_FP32, &e) == GQA_ERR_UNSUPPORTED);
  assert(gqa::check_prefill_launch(1, 1 << 19, 64, 8, 128, GQA_FP32, &e) == GQA_OK);
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


def test_workspace_registry_sanitized(tmp_path):
    """The decode workspace policy (allocate, grow, never allocate or free a
    graph's block during or after capture, release everything on request),
    built host-only with g++ under ASan/UBSan against a fake device whose
    blocks are host allocations: a block used past its size, freed twice or
    never freed fails the sanitizer."""
    src = tmp_path / "w.cpp"
    src.write_text(r'''
#include "workspace.h"
#include <cassert>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <set>
struct Fake : gqa::WsBackend {
  std::set<void*> live; int allocs = 0, async_frees = 0, now_frees = 0, syncs = 0;
  bool capturing = false, fail_alloc = false;
  int alloc(void **p, int64_t bytes, void *) override {
    if (fail_alloc) return 2;
    *p = std::malloc((size_t)bytes); live.insert(*p); ++allocs; return 0; }
  int free_async(void *p, void *) override { assert(live.erase(p) == 1); std::free(p); ++async_frees; return 0; }
  int free_now(int, void *p) override { assert(live.erase(p) == 1); std::free(p); ++now_frees; return 0; }
  int sync_device(int) override { ++syncs; return 0; }
  int is_capturing(void *, bool *c) override { *c = capturing; return 0; }
  std::string error_text(int c) override { return "fake error " + std::to_string(c); }
};
int main() {
  Fake f; gqa::WorkspaceRegistry reg(&f); std::string e; char *p = nullptr, *q = nullptr;
  void *s1 = (void*)0x10, *s2 = (void*)0x20;
  // nothing needed: nothing allocated
  assert(reg.get(0, s1, 0, &p, &e) == GQA_OK && p == nullptr && f.allocs == 0);
  // first use allocates; the whole requested size is usable
  assert(reg.get(0, s1, 1000, &p, &e) == GQA_OK && p && f.allocs == 1);
  std::memset(p, 1, 1000);
  // smaller and equal requests reuse the block
  assert(reg.get(0, s1, 500, &q, &e) == GQA_OK && q == p && f.allocs == 1);
  assert(reg.get(0, s1, 1000, &q, &e) == GQA_OK && q == p && f.allocs == 1);
  // another stream or device gets its own block
  assert(reg.get(0, s2, 1000, &q, &e) == GQA_OK && q != p && f.allocs == 2);
  assert(reg.get(1, s1, 1000, &q, &e) == GQA_OK && f.allocs == 3 && reg.live_count() == 3);
  // growth without capture frees the old block in stream order
  assert(reg.get(0, s1, 5000, &q, &e) == GQA_OK && q != p && f.allocs == 4 && f.async_frees == 1);
  std::memset(q, 2, 5000);
  p = q;
  // a failed allocation keeps the old block
  f.fail_alloc = true;
  assert(reg.get(0, s1, 100000, &q, &e) == GQA_ERR_HIP && e.find("fake error") != std::string::npos);
  f.fail_alloc = false;
  assert(reg.get(0, s1, 5000, &q, &e) == GQA_OK && q == p);
  // during capture: a block that fits is used and marked, nothing allocated
  f.capturing = true;
  assert(reg.get(0, s1, 4000, &q, &e) == GQA_OK && q == p && reg.live_captured(0, s1) && f.allocs == 4);
  // during capture: too small or missing is an error, nothing allocated or freed
  assert(reg.get(0, s1, 1 << 20, &q, &e) == GQA_ERR_INVALID_ARG && e.find("captur") != std::string::npos);
  assert(reg.get(2, s1, 10, &q, &e) == GQA_ERR_INVALID_ARG && f.allocs == 4 && f.async_frees == 1);
  assert(reg.live_bytes(0, s1) >= 5000);
  f.capturing = false;
  // growth after capture retires the graph's block instead of freeing it
  assert(reg.get(0, s1, 20000, &q, &e) == GQA_OK && q != p && f.async_frees == 1 && reg.retired_count() == 1);
  assert(f.live.count(p) == 1 && !reg.live_captured(0, s1));
  std::memset(p, 3, 5000);  // the retired block is still valid memory
  std::memset(q, 4, 20000);
  // release frees everything after waiting for both devices
  assert(reg.release_all(&e) == GQA_OK && f.live.empty() && f.syncs == 2);
  assert(reg.live_count() == 0 && reg.retired_count() == 0);
  // and the next call allocates afresh
  assert(reg.get(0, s1, 64, &q, &e) == GQA_OK && f.allocs == 6);
  assert(reg.release_all(&e) == GQA_OK && f.live.empty());
  std::puts("ok");
  return 0;
}
''')
    exe = tmp_path / "w"
    csrc = os.path.join(ROOT, "grouped_query_kv_gqa_amd", "csrc")
    subprocess.run(["g++", "-std=c++20", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    f"-I{csrc}", f"-I{os.path.join(ROOT, 'include')}", str(src), os.path.join(csrc, "workspace.cpp"),
                    "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for several (by flag or by a launcher's
    WORLD_SIZE) it exits with a message before touching any device."""
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *argv], capture_output=True, text=True,
                           timeout=120, env={**os.environ, **env})
        assert r.returncode == 2, (argv, env, r.returncode, r.stderr)
        assert "one GPU only" in r.stderr
