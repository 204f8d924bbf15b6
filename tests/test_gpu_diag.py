"""The diagnostic library (libhisparse_diag.so: the plan kernel's phase trace
and the floor kernels) checked in a process of its own, since the binding
loads one library per process: bit-exact parity of the traced build, a
complete and ordered trace, and the floor kernels' stated results."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_diagnostic_library_in_its_own_process():
    lib = os.path.join(ROOT, "hierarchical_sparse_attention_hisparse_amd", "libhisparse_diag.so")
    assert os.path.exists(lib), "libhisparse_diag.so is not built"
    env = dict(os.environ, HISPARSE_LIBRARY="diag")
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "diag_check.py")],
                       env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    print(r.stdout[-3000:])
    assert r.returncode == 0 and "DIAG OK" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
