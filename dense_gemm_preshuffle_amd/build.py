"""Build the gfx950 HIP library libgemm_preshuffle.so in-tree.

    python -m dense_gemm_preshuffle_amd.build        (or build() from Python)

Every translation unit under csrc/ is compiled with hipcc for gfx950 only,
in parallel, and linked into dense_gemm_preshuffle_amd/libgemm_preshuffle.so.
The build fails if any kernel spills registers or uses scratch memory.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgemm_preshuffle.so")
# the HBM streaming-read probe that bench.py --floor times (not the GEMM library)
PROBE_SRCS = [os.path.join(PKG, "probe", f) for f in ("stream_read.hip", "mfma_rate.hip")]
# The probes keep MFMA accumulators in VGPRs: with AGPR accumulators the
# compiler rotates a loop's eight 4-register accumulators through AGPR copies
# every iteration (24 accvgpr reads and writes per 8 MFMAs), which the rate
# probe would then measure instead of the MFMA.
PROBE_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
PROBE_LIB = os.path.join(PKG, "libgp_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 (v_pk_*_f32) instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


_REMARK = re.compile(r"remark: +(.*?) \[-Rpass-analysis=kernel-resource-usage\]")


def kernel_resources(text: str) -> dict:
    """Per-kernel resource remarks of one hipcc run -> {kernel: {field: value}}."""
    out, cur = {}, None
    for line in text.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        body = m.group(1)
        if body.startswith("Function Name:"):
            cur = out.setdefault(body.split(":", 1)[1].strip(), {})
        elif cur is not None and ":" in body:
            k, v = body.split(":", 1)
            cur[k.strip()] = v.strip()
    return out


def _compile(src: str) -> tuple:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj, kernel_resources(r.stdout + r.stderr)


def spilling(res: dict) -> list:
    """Kernels that keep values in scratch memory (register spills or an
    array the compiler could not keep in registers): each such access is a
    round trip to memory in the hot loop, tens of times slower."""
    bad = []
    for name, r in res.items():
        vals = [int(r.get(k, "0") or 0) for k in ("VGPRs Spill", "SGPRs Spill", "ScratchSize [bytes/lane]")]
        if any(vals):
            bad.append((name, vals))
    return bad


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        done = list(ex.map(_compile, srcs))
    objs = [o for o, _ in done]
    res = {k: v for _, r in done for k, v in r.items()}
    bad = spilling(res)
    if bad:
        lines = "\n".join(f"  {n}: VGPR spill {v[0]}, SGPR spill {v[1]}, scratch {v[2]} B/lane" for n, v in bad)
        raise RuntimeError(f"{len(bad)} kernels use scratch memory:\n{lines}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([HIPCC, *FLAGS, *PROBE_FLAGS, "-shared", "-o", tmp, *PROBE_SRCS], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)
    for f in (LIB, PROBE_LIB):
        if os.path.exists(f):
            os.remove(f)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
