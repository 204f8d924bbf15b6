"""CPU checks of the C-ABI library: it builds for gfx950, loads, and exports
every entry point include/hisparse.h declares (no compute calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hisparse.h")


def _declared_functions():
    text = open(HEADER).read()
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


def test_library_is_gfx950_code_object():
    import hierarchical_sparse_attention_hisparse_amd as hs
    data = open(hs.library_path(), "rb").read()
    assert b"gfx950" in data
    assert b"sm_" not in data[:0]  # nothing NVIDIA-specific is built


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
