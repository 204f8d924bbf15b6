"""Sanitizer builds, on the CPU.

1. The oracle built with gcc's AddressSanitizer and UndefinedBehaviorSanitizer
   runs every oracle pin (the three pin files) in a child process: an
   out-of-bounds access, use after free, signed overflow or misaligned load
   anywhere in the oracle fails the run.
2. The library's host code (the C ABI: argument checks, pool set-up, the
   host-RAM check) built with the same sanitizers (host side only; the
   kernels are built as usual) is driven by a C program through every error
   path that needs no GPU.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hierarchical_sparse_attention_hisparse_amd", "csrc")
ROCM = "/opt/rocm"


def _gcc_runtime(name):
    out = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_address_and_ub_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    asan = _gcc_runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "oracle", "hisparse_oracle.c"), "-o", str(lib), "-lm"],
                   check=True)
    env = dict(os.environ, LD_PRELOAD=asan, HISPARSE_ORACLE_LIB=str(lib),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child really runs the sanitized build
    probe = subprocess.run(
        [sys.executable, "-c",
         "import sys; sys.path.insert(0, %r); import oracle.oracle as o; o.load_oracle(); "
         "m = open('/proc/self/maps').read(); "
         "print(int('liboracle_san.so' in m and 'libasan' in m))" % ROOT],
        env=env, capture_output=True, text=True, timeout=300, cwd=str(tmp_path))
    assert probe.stdout.strip().endswith("1"), probe.stdout + probe.stderr
    pins = [os.path.join(ROOT, "tests", f) for f in
            ("test_oracle_pins.py", "test_oracle_pins_steps.py",
             "test_oracle_pins_mirror_invalidate.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"] + pins,
                       env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    print(r.stdout.strip().splitlines()[-1])


_DRIVER = r"""
#include <stdio.h>
#include <string.h>
#include "hisparse.h"
static int fails = 0;
static void expect(int got, int want, const char* what) {
  if (got != want) {
    printf("FAIL %s: %d != %d (%s)\n", what, got, want, hisparse_last_error());
    ++fails;
  } else {
    printf("ok %s: %s\n", what, hisparse_last_error());
  }
}
int main(void) {
  hisparse_pool* pool = NULL;
  hisparse_pool_config c;
  memset(&c, 0, sizeof c);
  c.max_requests = 4; c.slots = 256; c.max_top_k = 64; c.max_batch = 4; c.row_bytes = 656;
  c.num_layers = 1; c.max_seq_len = 1024;
  expect(hisparse_init_pool(NULL, NULL, NULL, NULL, 0, &pool), HISPARSE_EINVAL, "null config");
  expect(hisparse_init_pool(&c, NULL, NULL, NULL, 1024, &pool), HISPARSE_EINVAL, "null arrays");
  c.max_heads = 8;
  expect(hisparse_init_pool(&c, NULL, NULL, NULL, 1024, &pool), HISPARSE_EINVAL, "max_heads");
  c.max_heads = 0; c.row_bytes = 650;
  expect(hisparse_init_pool(&c, NULL, NULL, NULL, 1024, &pool), HISPARSE_EINVAL, "row_bytes");
  c.row_bytes = 656; c.slots = 16384; c.max_top_k = 4096;
  expect(hisparse_init_pool(&c, NULL, NULL, NULL, 1 << 20, &pool), HISPARSE_EUNSUPPORTED, "lds");
  c.slots = 256; c.max_top_k = 64;
  {
    void* hp[1] = {(void*)0x10008};
    int64_t hr[1] = {16};
    void* dp[1] = {(void*)0x20000};
    expect(hisparse_init_pool(&c, hp, hr, dp, 1024, &pool), HISPARSE_EINVAL, "misaligned host pool");
  }
  void* p = NULL;
  expect(hisparse_host_alloc((size_t)1 << 60, &p), HISPARSE_ENOMEM, "host ram");
  expect(hisparse_host_alloc(0, &p), HISPARSE_EINVAL, "zero bytes");
  expect(hisparse_host_alloc(16, NULL), HISPARSE_EINVAL, "null out");
  expect(hisparse_resolve(NULL, NULL, 1, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                          NULL, NULL), HISPARSE_EINVAL, "resolve: null pool");
  expect(hisparse_gather_copy(NULL, NULL, 1, 0, 1, NULL), HISPARSE_EINVAL, "copy: null pool");
  expect(hisparse_sparse_mla_decode(NULL, NULL, 1, 16, 1, 0, NULL, NULL, 1.f, NULL),
         HISPARSE_EINVAL, "decode: null pool");
  expect(hisparse_mirror_rows(NULL, NULL, 1, NULL, NULL, 0, 1, NULL), HISPARSE_EINVAL,
         "mirror: null pool");
  hisparse_destroy_pool(NULL);
  expect(hisparse_host_free(NULL), HISPARSE_OK, "free null");
  return fails ? 1 : 0;
}
"""


def test_abi_host_code_under_address_and_ub_sanitizers(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    rt = None
    for base in (os.path.join(ROCM, "lib", "llvm", "lib", "clang"),
                 os.path.join(ROCM, "llvm", "lib", "clang")):
        if os.path.isdir(base):
            for ver in sorted(os.listdir(base)):
                d = os.path.join(base, ver, "lib", "linux")
                if os.path.exists(os.path.join(d, "libclang_rt.asan-x86_64.so")):
                    rt = d
    if not (os.path.exists(hipcc) and os.path.exists(clang) and rt):
        pytest.skip("no ROCm compiler or clang sanitizer runtime")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include")]
    # Host code of the ABI with the sanitizers (each flag for the host pass
    # only); the kernel sources unchanged, compiled in parallel.
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    procs = [subprocess.Popen([hipcc] + flags + san + ["-c", os.path.join(CSRC, "abi.hip"), "-o",
                                                       str(tmp_path / "abi.o")],
                              stdout=subprocess.DEVNULL, stderr=subprocess.PIPE)]
    for f in ("resolve", "gather", "mla_decode", "maintain"):
        procs.append(subprocess.Popen([hipcc] + flags + ["-c", os.path.join(CSRC, f + ".hip"), "-o",
                                                         str(tmp_path / (f + ".o"))],
                                      stdout=subprocess.DEVNULL, stderr=subprocess.PIPE))
    for pr in procs:
        _, err = pr.communicate(timeout=600)
        assert pr.returncode == 0, err.decode()[-2000:]
    lib = tmp_path / "libhisparse_san.so"
    objs = [str(tmp_path / (f + ".o")) for f in ("abi", "resolve", "gather", "mla_decode", "maintain")]
    subprocess.run([clangxx, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan"] +
                   objs + ["-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", str(lib)], check=True)
    src = tmp_path / "drive_abi.c"
    src.write_text(_DRIVER)
    exe = tmp_path / "drive_abi"
    subprocess.run([clang, "-std=c99", "-g", "-fsanitize=address,undefined", "-shared-libsan",
                    "-I", os.path.join(ROOT, "include"), str(src), "-L", str(tmp_path),
                    "-lhisparse_san", "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath," + rt,
                    "-o", str(exe)], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr[-3000:]
    assert r.stdout.count("ok ") == 14 and "FAIL" not in r.stdout, r.stdout
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
