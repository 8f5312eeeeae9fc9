"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects invalid arguments on the host before touching HIP."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import chunk_causal_dit_wf_amd as wf
from chunk_causal_dit_wf_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wf_chunk_attn.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wf_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"wf_chunk_attn_fwd", "wf_kv_append", "wf_kv_evict", "wf_last_error", "wf_stream_copy"} <= set(names)
    L = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(r"\bT %s$" % n, out, flags=re.M), n


@pytest.mark.parametrize("header", HEADERS, ids=os.path.basename)
def test_header_compiles_as_c(header):
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", header],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_struct_layout_matches_binding():
    src = """
#include <stddef.h>
#include <stdio.h>
#include "wf_chunk_attn.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu\\n", sizeof(wf_kv_cache), offsetof(wf_kv_cache, page_table),
         offsetof(wf_kv_cache, table_len), offsetof(wf_kv_cache, kv_dtype), offsetof(wf_kv_cache, start));
  return 0;
}
"""
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "t")
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        got = subprocess.run([exe], capture_output=True, text=True).stdout.split()
    S = _lib.wf_kv_cache
    want = [ctypes.sizeof(S), S.page_table.offset, S.table_len.offset, S.kv_dtype.offset, S.start.offset]
    assert [int(x) for x in got] == want


def _cache(dtype="bf16", table=(0, 1, 2, 3), P=64, H=2, D=64):
    return wf.KVCache(4, P, H, D, dtype, list(table), device="cpu")


def _status(fn, *a, **k):
    try:
        fn(*a, **k)
    except wf.WfError as e:
        return e.status
    return wf.WF_OK


@pytest.mark.parametrize("mutate,status", [
    (lambda c: setattr(c.c, "head_dim", 96), wf.WF_ERR_UNSUPPORTED),
    (lambda c: setattr(c.c, "page_size", 12), wf.WF_ERR_UNSUPPORTED),
    (lambda c: setattr(c.c, "kv_dtype", 7), wf.WF_ERR_UNSUPPORTED),
    (lambda c: setattr(c.c, "table_len", 0), wf.WF_ERR_INVALID_ARG),
    (lambda c: setattr(c.c, "num_pages", 3), wf.WF_ERR_INVALID_ARG),
    (lambda c: setattr(c.c, "k", None), wf.WF_ERR_INVALID_ARG),
    (lambda c: setattr(c.c, "k", c.c.k + 4), wf.WF_ERR_INVALID_ARG),
    (lambda c: setattr(c.c, "v", c.c.k), wf.WF_ERR_INVALID_ARG),
    (lambda c: c.table.__setitem__(2, 0), wf.WF_ERR_INVALID_ARG),
    (lambda c: c.table.__setitem__(2, 9), wf.WF_ERR_INVALID_ARG),
    (lambda c: setattr(c.c, "end", -1), wf.WF_ERR_INVALID_ARG),
    (lambda c: setattr(c.c, "end", 300), wf.WF_ERR_INVALID_ARG),
])
def test_cache_check_rejects(mutate, status):
    c = _cache()
    wf.wf_kv_cache_check(c)
    mutate(c)
    assert _status(wf.wf_kv_cache_check, c) == status


def test_fp8_cache_needs_scales():
    c = _cache("fp8")
    wf.wf_kv_cache_check(c)
    c.c.k_scale = None
    assert _status(wf.wf_kv_cache_check, c) == wf.WF_ERR_INVALID_ARG


def test_cache_bytes():
    c = _cache("fp8", P=200)
    kb, sb = wf.wf_kv_cache_bytes(c)
    assert kb == 4 * 2 * 200 * 64 and sb == 4 * 2 * 2 * 4


def test_append_validation_before_any_launch():
    c = _cache()
    k = torch.zeros(8, 2, 64, dtype=torch.bfloat16)
    assert _status(wf.wf_kv_append, c, 1, k, k) == wf.WF_ERR_RANGE          # gap after end
    assert _status(wf.wf_kv_append, c, 0, torch.zeros(300, 2, 64, dtype=torch.bfloat16),
                   torch.zeros(300, 2, 64, dtype=torch.bfloat16)) == wf.WF_ERR_CAPACITY
    c.c.end = 256
    c.c.start = 2
    assert _status(wf.wf_kv_append, c, 260, k, k) == wf.WF_ERR_RANGE
    assert _status(wf.wf_kv_append, c, 256, k, k) == wf.WF_ERR_CAPACITY     # 264 > 2 + 256: wraps onto live tokens
    assert (c.start, c.end) == (2, 256)
    f = _cache("fp8")
    k8 = torch.zeros(8, 2, 64, dtype=torch.uint8)
    s = torch.ones(1, 2, 1)
    assert _status(wf.wf_kv_append, f, 0, k8, k8, s, s) == wf.WF_ERR_INVALID_ARG   # not whole pages


def test_append_without_device_reports_hip_error_and_keeps_metadata():
    c = _cache()
    k = torch.zeros(8, 2, 64, dtype=torch.bfloat16)
    if torch.cuda.is_available():
        pytest.skip("needs a machine without a GPU")
    assert _status(wf.wf_kv_append, c, 0, k, k) == wf.WF_ERR_HIP
    assert (c.start, c.end) == (0, 0)
    assert "launch" in wf.lib().wf_last_error().decode()


def test_evict_validation():
    c = _cache()
    c.c.end = 100
    assert _status(wf.wf_kv_evict, c, 101) == wf.WF_ERR_RANGE
    assert _status(wf.wf_kv_evict, c, -1) == wf.WF_ERR_RANGE
    wf.wf_kv_evict(c, 40)                     # metadata only, no launch
    assert (c.start, c.end) == (40, 100)


def test_stream_copy_validation_before_any_launch():
    """The reference copy rejects bad sizes, alignment and overlap on the host (nothing is
    launched: the pointers below are never dereferenced); zero bytes is a no-op."""
    L = wf.lib()
    vp = ctypes.c_void_p
    assert L.wf_stream_copy(vp(4096), vp(1 << 20), 0, None) == wf.WF_OK
    assert L.wf_stream_copy(vp(4096), vp(1 << 20), 24, None) == wf.WF_ERR_INVALID_ARG      # not 16-byte multiple
    assert L.wf_stream_copy(vp(4104), vp(1 << 20), 32, None) == wf.WF_ERR_INVALID_ARG      # misaligned source
    assert L.wf_stream_copy(vp(4096), vp((1 << 20) + 8), 32, None) == wf.WF_ERR_INVALID_ARG
    assert L.wf_stream_copy(None, vp(1 << 20), 32, None) == wf.WF_ERR_INVALID_ARG
    assert L.wf_stream_copy(vp(4096), vp(4096 + 64), 128, None) == wf.WF_ERR_INVALID_ARG   # overlap
    assert L.wf_stream_copy(vp(4096 + 64), vp(4096), 128, None) == wf.WF_ERR_INVALID_ARG
    assert "overlap" in L.wf_last_error().decode()


def test_attention_validation():
    c = _cache()
    c.c.start, c.c.end = 10, 200
    q = torch.zeros(16, 2, 64, dtype=torch.bfloat16)
    st = lambda *a, **k: _status(wf.wf_chunk_attn_fwd, c, *a, **k)
    assert st(q, [0, 16], [5], [20]) == wf.WF_ERR_RANGE          # begins before start
    assert st(q, [0, 16], [20], [20]) == wf.WF_ERR_RANGE         # empty
    assert st(q, [0, 16], [20], [201]) == wf.WF_ERR_RANGE        # beyond end
    assert st(q, [1, 16], [20], [30]) == wf.WF_ERR_INVALID_ARG   # q_off[0] != 0
    assert st(q, [0, 9, 8], [20, 20], [30, 30]) == wf.WF_ERR_INVALID_ARG
    assert st(q.float(), [0, 16], [20], [30]) == wf.WF_ERR_UNSUPPORTED   # f32 q with bf16 cache
    assert st(q, [0] * 66, [20] * 65, [30] * 65) == wf.WF_ERR_INVALID_ARG  # too many chunks
    assert st(q, [0, 16], [20], [30], softmax_scale=float("nan")) == wf.WF_ERR_INVALID_ARG
    assert st(q, [0, 16], [20], [30], o=q) == wf.WF_ERR_INVALID_ARG      # o aliases q
    assert st(q, [0, 0], [20], [30]) == wf.WF_OK                          # no rows: nothing to do
    ws = torch.zeros(4096, dtype=torch.uint8)
    assert st(q, [0, 16], [20], [30], workspace=ws[1:]) == wf.WF_ERR_INVALID_ARG   # misaligned workspace


def test_attention_workspace_needs_pointer_and_size_together():
    c = _cache()
    c.c.start, c.c.end = 0, 200
    q = torch.zeros(16, 2, 64, dtype=torch.bfloat16)
    o = torch.zeros_like(q)
    qo = (ctypes.c_int32 * 2)(0, 16)
    kb = (ctypes.c_int64 * 1)(0)
    ke = (ctypes.c_int64 * 1)(100)
    L = wf.lib()
    st = L.wf_chunk_attn_fwd(ctypes.byref(c.c), ctypes.c_void_p(q.data_ptr()), wf.WF_BF16,
                             ctypes.c_void_p(o.data_ptr()), None, 1, qo, kb, ke, 0.0, None, 4096, None)
    assert st == wf.WF_ERR_INVALID_ARG
    assert "workspace" in L.wf_last_error().decode()


def test_fastdiv_exhaustive_on_host(tmp_path):
    """The device's page addressing divides with a multiply-high; check it on the host."""
    src = r"""
#include <cstdio>
#include <cstdint>
#include <random>
#include "wf_internal.h"
int main() {
  std::mt19937_64 g(1); long bad = 0;
  for (uint32_t d : {1u,2u,3u,7u,8u,21u,64u,192u,1560u,4680u,32760u,65536u,1000003u,2147483647u}) {
    wf::FastDiv f = wf::make_fastdiv(d);
    for (uint32_t n = 0; n < 2000000; ++n) bad += wf::fastdiv(n, f) != n / d;
    for (int i = 0; i < 2000000; ++i) { uint32_t n = (uint32_t)g(); bad += wf::fastdiv(n, f) != n / d; }
    for (uint32_t n : {0xFFFFFFFFu, 0x80000000u, d - 1, d, d + 1}) bad += wf::fastdiv(n, f) != n / d;
  }
  for (uint32_t d = 1; d < 4000; ++d) { wf::FastDiv f = wf::make_fastdiv(d);
    for (int i = 0; i < 500; ++i) { uint32_t n = (uint32_t)g(); bad += wf::fastdiv(n, f) != n / d; } }
  printf("%ld\n", bad); return bad != 0;
}
"""
    c = tmp_path / "t.hip"
    c.write_text(src)
    exe = tmp_path / "t"
    r = subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-I", os.path.join(ROOT, "chunk_causal_dit_wf_amd", "csrc"),
                        "--offload-arch=gfx950", "-x", "hip", str(c), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "0"


def test_xcd_deal_is_a_bijection_on_host(tmp_path):
    """The attention kernels' item deal (wf_internal.h): for every chunk size N up to 5000 it is
    a bijection of [0, N) whose inverse is deal_index, XCD x = L % 8 runs one contiguous run of
    the head-major order, and for the Wan round (19 query tiles x 12 heads) the 8 XCDs hold 16
    (XCD, head) pairs, the fewest possible (at most 32 items fit one XCD, so 4 heads must split)."""
    src = r"""
#include <cstdio>
#include <vector>
#include <set>
#include "wf_internal.h"
int main() {
  long bad = 0;
  for (int N = 1; N <= 5000; ++N) {
    std::vector<int> seen(N, 0), lo(8, N), hi(8, -1), cnt(8, 0);
    for (int L = 0; L < N; ++L) {
      const int pos = wf::deal_position(N, L);
      if (pos < 0 || pos >= N) { ++bad; continue; }
      seen[pos]++;
      bad += wf::deal_index(N, pos) != L;
      const int x = L & 7;
      lo[x] = pos < lo[x] ? pos : lo[x]; hi[x] = pos > hi[x] ? pos : hi[x]; cnt[x]++;
    }
    for (int i = 0; i < N; ++i) bad += seen[i] != 1;
    for (int x = 0; x < 8; ++x) if (cnt[x]) bad += hi[x] - lo[x] + 1 != cnt[x];  // contiguous run
  }
  std::set<std::pair<int, int>> pairs;
  for (int L = 0; L < 228; ++L) pairs.insert({L & 7, wf::deal_position(228, L) / 19});
  printf("%ld %zu\n", bad, pairs.size());
  return bad != 0;
}
"""
    c = tmp_path / "t.hip"
    c.write_text(src)
    exe = tmp_path / "t"
    r = subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-I", os.path.join(ROOT, "chunk_causal_dit_wf_amd", "csrc"),
                        "--offload-arch=gfx950", "-x", "hip", str(c), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.split() == ["0", "16"], out.stdout


def test_quantizing_append_validation():
    k = torch.zeros(64, 2, 64, dtype=torch.bfloat16)
    b = _cache("bf16")
    assert _status(wf.wf_kv_append_quantize, b, 0, k, k) == wf.WF_ERR_UNSUPPORTED   # not an E4M3FN cache
    f = _cache("fp8")
    assert _status(wf.wf_kv_append_quantize, f, 8, k, k) == wf.WF_ERR_RANGE         # beyond end
    assert _status(wf.wf_kv_append_quantize, f, 0, k[:40], k[:40]) == wf.WF_ERR_INVALID_ARG  # not whole pages
    raw = torch.zeros(64 * 2 * 64 + 8, dtype=torch.bfloat16)
    mis = raw[1:1 + 64 * 2 * 64].view(64, 2, 64)
    assert _status(wf.wf_kv_append_quantize, f, 0, mis, k) == wf.WF_ERR_INVALID_ARG  # misaligned source
    assert _status(wf.wf_kv_append_quantize, f, 0, k[:0], k[:0]) == wf.WF_OK         # nothing to do
    assert (f.start, f.end) == (0, 0)
    if not torch.cuda.is_available():
        assert _status(wf.wf_kv_append_quantize, f, 0, k, k) == wf.WF_ERR_HIP
        assert (f.start, f.end) == (0, 0)


def test_host_logic_under_address_and_undefined_behavior_sanitizers(tmp_path):
    """api.cpp built for the host with AddressSanitizer and UndefinedBehaviorSanitizer, linked
    with host stand-ins of the kernel launchers (tests/sanitize/launch_stubs.cpp), and driven
    through validation, planning and metadata paths by tests/sanitize/abi_exercise.c.  A
    sanitizer report aborts the program; every status must match."""
    san = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    hip_host = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include")]
    csrc = os.path.join(ROOT, "chunk_causal_dit_wf_amd", "csrc")
    sdir = os.path.join(ROOT, "tests", "sanitize")
    steps = [
        ["g++", "-std=c++17"] + san + hip_host + ["-c", os.path.join(csrc, "api.cpp"), "-o", str(tmp_path / "api.o")],
        ["g++", "-std=c++17"] + san + hip_host + ["-c", os.path.join(sdir, "launch_stubs.cpp"),
                                                  "-o", str(tmp_path / "stubs.o")],
        ["gcc", "-std=c99"] + san + ["-I" + os.path.join(ROOT, "include"), "-c",
                                     os.path.join(sdir, "abi_exercise.c"), "-o", str(tmp_path / "main.o")],
        ["g++"] + san + [str(tmp_path / "main.o"), str(tmp_path / "api.o"), str(tmp_path / "stubs.o"),
                         "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(tmp_path / "ex")],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, (cmd, r.stderr[-2000:])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([str(tmp_path / "ex")], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), (r.stdout[-3000:], r.stderr[-3000:])


def test_bench_source_hash_ignores_comments_and_layout_only():
    """bench.py keeps a committed HBM-traffic figure only while the kernel code it was measured
    on is unchanged: comments and white space do not count, any code token does."""
    import bench
    base = 'int f(int a) {\n  // note\n  return a + 1; /* x */\n}\nconst char* s = "//not a comment";\n'
    same = 'int f(int a) { return a + 1;\n}   // other note\n/* block */ const char* s = "//not a comment";'
    diff = 'int f(int a) {\n  return a + 2;\n}\nconst char* s = "//not a comment";\n'
    lit = 'int f(int a) {\n  return a + 1;\n}\nconst char* s = "//not a Comment";\n'
    t = bench.code_text(base)
    assert t == bench.code_text(same)
    assert t != bench.code_text(diff) and t != bench.code_text(lit)
    assert "note" not in t and '"//not a comment"' in t
    for src in ("attn_fwd.hip", "attn_fp8.hip", "kv_cache.hip"):
        assert re.fullmatch(r"[0-9a-f]{64}", bench.source_sha(src))
