"""The binding loads the HIP library so that the process holds one HIP
runtime: PyTorch's copy, whose soname matches ROCm's. Checked in a fresh
interpreter that loads the library before anything else imports torch
(no GPU needed: only the mapped shared objects are inspected)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_SCRIPT = r"""
import dense_gemm_preshuffle_amd as gp
gp.load_library()
import torch
maps = open("/proc/self/maps").read().splitlines()
hip = sorted({l.split()[-1] for l in maps if "libamdhip64" in l})
hsa = sorted({l.split()[-1] for l in maps if "libhsa-runtime64" in l})
print(len(hip), len(hsa))
"""


def test_library_binds_to_the_one_hip_runtime():
    if not os.path.exists(os.path.join(ROOT, "dense_gemm_preshuffle_amd", "libgemm_preshuffle.so")):
        pytest.skip("library not built")
    r = subprocess.run([sys.executable, "-c", _SCRIPT], cwd=ROOT, capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, PYTHONPATH=ROOT))
    assert r.returncode == 0, r.stderr
    assert r.stdout.split()[-2:] == ["1", "1"], r.stdout
