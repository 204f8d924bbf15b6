"""CPU checks of the C-ABI library: it builds for gfx950, loads, and exports
every entry point include/hisparse.h declares (no compute calls); the
diagnostic build exports those and the ones of include/hisparse_diag.h."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hisparse.h")
DIAG_HEADER = os.path.join(ROOT, "include", "hisparse_diag.h")
DIAG_LIB = os.path.join(ROOT, "hierarchical_sparse_attention_hisparse_amd", "libhisparse_diag.so")


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(hisparse_[a-z_0-9]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("hisparse_init_pool", "hisparse_resolve", "hisparse_sparse_mla_decode",
                     "hisparse_destroy_pool", "hisparse_last_error"):
        assert required in names


def test_library_loads_and_exports_every_symbol():
    import hierarchical_sparse_attention_hisparse_amd as hs
    from hierarchical_sparse_attention_hisparse_amd.build import build_library
    if not os.path.exists(hs.library_path()):
        build_library(force=True)
    lib = ctypes.CDLL(hs.library_path())
    for name in _declared_functions():
        assert hasattr(lib, name), name
    # the binding loads the same library
    assert hs.load_library() is not None
    assert hs.hisparse_last_error() == ""


def test_diagnostic_library_exports_both_headers_and_the_library_only_its_own():
    import hierarchical_sparse_attention_hisparse_amd as hs
    from hierarchical_sparse_attention_hisparse_amd.build import build_library
    if not (os.path.exists(hs.library_path()) and os.path.exists(DIAG_LIB)):
        build_library(force=True)
    diag_names = _declared_functions(DIAG_HEADER)
    assert set(diag_names) == {"hisparse_diag_phase_clear", "hisparse_diag_phase_read",
                               "hisparse_diag_floor", "hisparse_diag_exchange",
                               "hisparse_diag_hit_detection"}
    diag = ctypes.CDLL(DIAG_LIB)
    for name in _declared_functions() + diag_names:
        assert hasattr(diag, name), name
    lib = ctypes.CDLL(hs.library_path())
    for name in diag_names:
        assert not hasattr(lib, name), name
    data = open(DIAG_LIB, "rb").read()
    device = [t for t in _offload_bundle_targets(data) if not t.startswith("host-")]
    assert set(device) == {"hipv4-amdgcn-amd-amdhsa--gfx950"}, device


def _offload_bundle_targets(data: bytes):
    """Target IDs of every clang offload bundle embedded in a shared library
    (magic, entry count, then per entry: offset, size, ID length, ID)."""
    import struct
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    ids, pos = [], 0
    while True:
        i = data.find(magic, pos)
        if i < 0:
            return ids
        j = i + len(magic)
        n, = struct.unpack_from("<Q", data, j)
        j += 8
        assert 0 < n < 16, "malformed bundle header at %d" % i
        for _ in range(n):
            _off, _size, idlen = struct.unpack_from("<QQQ", data, j)
            j += 24
            ids.append(data[j:j + idlen].decode("ascii"))
            j += idlen
        pos = i + 1


def test_library_is_gfx950_code_object():
    """Every offload bundle in the library holds host code and gfx950 device
    code only: no other GPU target is built."""
    import hierarchical_sparse_attention_hisparse_amd as hs
    data = open(hs.library_path(), "rb").read()
    ids = _offload_bundle_targets(data)
    device = [t for t in ids if not t.startswith("host-")]
    assert device, "no device code object in the library"
    assert set(device) == {"hipv4-amdgcn-amd-amdhsa--gfx950"}, ids
    assert all(t.startswith("host-x86_64") for t in ids if t.startswith("host-"))


def test_host_alloc_refuses_more_than_the_available_ram():
    """hisparse_host_alloc checks the request against 95% of MemAvailable
    before pinning anything: a request far beyond the host's memory is
    refused with ENOMEM and a message naming the limit (no GPU needed)."""
    import hierarchical_sparse_attention_hisparse_amd as hs
    lib = hs.load_library()
    out = ctypes.c_void_p(1)
    rc = lib.hisparse_host_alloc(ctypes.c_size_t(1 << 60), ctypes.byref(out))
    msg = hs.hisparse_last_error()
    assert rc == -2 and "MemAvailable" in msg and out.value is None, (rc, msg)
    avail = 0
    for line in open("/proc/meminfo"):
        if line.startswith("MemAvailable:"):
            avail = int(line.split()[1]) * 1024
    # just above the limit: refused by the same check
    rc = lib.hisparse_host_alloc(ctypes.c_size_t(int(0.96 * avail)), ctypes.byref(out))
    assert rc == -2 and "MemAvailable" in hs.hisparse_last_error()


def test_binding_rejects_bad_arguments_before_any_device_call():
    """Shape/dtype checks happen on the host; CPU tensors are refused."""
    import torch
    import hierarchical_sparse_attention_hisparse_amd as hs
    from hierarchical_sparse_attention_hisparse_amd._binding import _dev
    with pytest.raises(TypeError):
        _dev(torch.zeros(3, dtype=torch.int32), torch.int32, (3,), "x")
    with pytest.raises(ValueError):
        _dev(None, torch.int32, (3,), "x")
    assert _dev(None, torch.int32, (3,), "x", allow_none=True) is None
    assert hs.STAT_NAMES[4] == "tripwires"


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU; asked for more it says why and exits
    before touching a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_header_is_plain_c_and_the_library_links_from_c(tmp_path):
    """include/hisparse.h compiles as strict C99 and as C++17; a C program
    links libhisparse.so and gets a status code and message back from a call
    whose arguments are refused on the host (no GPU needed)."""
    import shutil
    import subprocess
    import hierarchical_sparse_attention_hisparse_amd as hs
    from hierarchical_sparse_attention_hisparse_amd.build import build_library
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("no host C/C++ compiler")
    if not os.path.exists(hs.library_path()):
        build_library(force=True)
    inc = os.path.join(ROOT, "include")
    libdir = os.path.dirname(hs.library_path())
    src = tmp_path / "use_abi.c"
    src.write_text(
        '#include <stdio.h>\n#include "hisparse.h"\n'
        "int main(void) {\n"
        "  hisparse_pool* pool = NULL;\n"
        "  int rc = hisparse_init_pool(NULL, NULL, NULL, NULL, 0, &pool);\n"
        '  printf("%d %s\\n", rc, hisparse_last_error());\n'
        "  return rc == HISPARSE_EINVAL && pool == NULL ? 0 : 1;\n"
        "}\n")
    exe = tmp_path / "use_abi"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", inc,
                    str(src), "-L", libdir, "-lhisparse", "-Wl,-rpath," + libdir, "-o", str(exe)],
                   check=True)
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror", "-fsyntax-only", "-x", "c++", "-I", inc,
                    str(src)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("-1 ") and "NULL" in res.stdout


def test_diagnostic_header_is_plain_c_and_links_from_c(tmp_path):
    """include/hisparse_diag.h compiles as strict C99 (with hisparse.h) and as
    C++17; a C program links libhisparse_diag.so and gets the stated refusal
    back from diagnostic calls with bad arguments (no GPU needed)."""
    import shutil
    import subprocess
    from hierarchical_sparse_attention_hisparse_amd.build import build_library
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("no host C/C++ compiler")
    if not os.path.exists(DIAG_LIB):
        build_library(force=True)
    inc = os.path.join(ROOT, "include")
    libdir = os.path.dirname(DIAG_LIB)
    src = tmp_path / "use_diag.c"
    src.write_text(
        '#include <stdio.h>\n#include "hisparse.h"\n#include "hisparse_diag.h"\n'
        "int main(void) {\n"
        "  uint64_t w[1];\n"
        "  int a = hisparse_diag_phase_read(w, 1);\n"
        "  int b = hisparse_diag_floor(NULL, 9, 1, 1, 1, 1, 1, NULL, NULL, NULL, NULL, NULL, NULL, 1);\n"
        "  int c = hisparse_diag_exchange(NULL, 1, 0, NULL, 1);\n"
        "  int d = hisparse_diag_hit_detection(NULL, 9, 1, 1, 1, 1, 1, NULL, NULL, NULL, NULL, NULL, 1);\n"
        '  printf("%d %d %d %d %d %s\\n", a, b, c, d, HISPARSE_TRACE_WORDS, hisparse_last_error());\n'
        "  return a == HISPARSE_EINVAL && b == HISPARSE_EINVAL && c == HISPARSE_EINVAL &&\n"
        "         d == HISPARSE_EINVAL ? 0 : 1;\n"
        "}\n")
    exe = tmp_path / "use_diag"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", inc,
                    str(src), "-L", libdir, "-l:libhisparse_diag.so", "-Wl,-rpath," + libdir,
                    "-o", str(exe)], check=True)
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror", "-fsyntax-only", "-x", "c++", "-I", inc,
                    str(src)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("-1 -1 -1 -1 73728 "), res.stdout


def _init_rc(cfg_kwargs, device_pool_rows=None, layer0=None):
    """hisparse_init_pool through the C ABI.  The pool arrays are NULL unless
    `layer0` = (host pointer, host rows, device pointer) is given; those
    pointers are only checked on the host, never dereferenced."""
    import hierarchical_sparse_attention_hisparse_amd as hs
    from hierarchical_sparse_attention_hisparse_amd._binding import _Config
    base = dict(max_requests=4, slots=256, max_top_k=64, max_batch=4, row_bytes=656, num_layers=1,
                page_size=0, max_steps=1, resident_pages=0, max_seq_len=1024)
    base.update(cfg_kwargs)
    cfg = _Config(**base)
    lib = hs.load_library()
    out = ctypes.c_void_p(1)
    rows = base["max_requests"] * base["slots"] if device_pool_rows is None else device_pool_rows
    if layer0 is not None:
        hp = (ctypes.c_void_p * 1)(layer0[0])
        hr = (ctypes.c_int64 * 1)(layer0[1])
        dp = (ctypes.c_void_p * 1)(layer0[2])
        rc = lib.hisparse_init_pool(ctypes.byref(cfg), hp, hr, dp, ctypes.c_int64(rows),
                                    ctypes.byref(out))
    else:
        rc = lib.hisparse_init_pool(ctypes.byref(cfg), None, None, None, ctypes.c_int64(rows),
                                    ctypes.byref(out))
    return rc, hs.hisparse_last_error(), out.value


@pytest.mark.parametrize("bad", [
    dict(max_requests=0), dict(slots=0), dict(slots=16385), dict(max_top_k=0),
    dict(max_top_k=257), dict(max_batch=0), dict(max_batch=65536), dict(row_bytes=650),
    dict(row_bytes=0), dict(num_layers=0), dict(page_size=-1), dict(max_steps=-1),
    dict(resident_pages=3), dict(max_seq_len=0), dict(max_seq_len=2 ** 31)])
def test_init_rejects_bad_configurations_on_the_host(bad):
    """Every configuration check of hisparse_init_pool runs before any device
    call: each bad field is refused with EINVAL, a message, and no pool."""
    rc, msg, out = _init_rc(bad)
    assert rc == -1, (bad, rc, msg)
    assert msg and out is None


def test_init_rejects_a_device_pool_too_small_for_the_hot_rows():
    rc, msg, out = _init_rc(dict(max_requests=4, slots=256), device_pool_rows=4 * 256 - 1)
    assert rc == -1 and "device_pool_rows" in msg and out is None
    rc, msg, _ = _init_rc(dict(max_requests=4, slots=256, page_size=16, resident_pages=10),
                          device_pool_rows=4 * 256 + 159)
    assert rc == -1 and "device_pool_rows" in msg


@pytest.mark.parametrize("S,k,fits", [(4096, 2048, True), (4096, 4096, True), (8192, 4096, True),
                                      (16384, 2004, True), (16384, 2008, False),
                                      (16384, 4096, False)])
def test_lds_budget_limits_stated_in_the_header(S, k, fits):
    """The header's limits on max_top_k per slot count: shapes within them
    pass every configuration check (the call then stops at the NULL pool
    arrays), shapes beyond them are refused with EUNSUPPORTED and the LDS
    bytes they would need."""
    rc, msg, out = _init_rc(dict(max_requests=2, slots=S, max_top_k=k, max_seq_len=1 << 20))
    if fits:
        assert rc == -1 and "pool arrays are NULL" in msg, (S, k, rc, msg)
    else:
        assert rc == -4 and "LDS" in msg, (S, k, rc, msg)
    assert out is None


@pytest.mark.parametrize("layer0,what", [((0x10000, 2 ** 31, 0x20000), "host_pool_rows"),
                                          ((0x10008, 16, 0x20000), "host_pools"),
                                          (((0), 16, 0x20000), "host_pools"),
                                          ((0x10000, 16, 0), "device_pools"),
                                          ((0x10000, 16, 0x20004), "device_pools")])
def test_init_rejects_bad_pool_arrays_on_the_host(layer0, what):
    """Per-layer pool checks (row count below 2^31, non-NULL 16-byte-aligned
    pointers) also run before any device call."""
    rc, msg, out = _init_rc({}, layer0=layer0)
    assert rc == -1 and what in msg and out is None, (layer0, rc, msg)
