"""Helpers shared by the GPU parity tests: run the HIP path on host inputs and
compare with the oracle (INT8 bit-exact, bf16 outputs within the tolerances of
oracle.compare)."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from dense_gemm_preshuffle_amd import workload


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_run(dtype, host, opts=None, repeat=1, act=None):
    import torch

    dev = workload.to_device(dtype, host)
    p = workload.prepare(dtype, dev)
    outs = []
    for _ in range(repeat):
        c = workload.run(dtype, p, opts=opts, act=act)
        torch.cuda.synchronize()
        outs.append(workload.to_host(c))
    return outs if repeat > 1 else outs[0]


def check(dtype, host, out, rows=None, cols=None, ref=None, act=None):
    """Compare a GPU result (int32, bf16 or fp16 bits) with the oracle; returns metrics."""
    if ref is None:
        ref = oracle.gemm(dtype, host, rows, cols, act=act)
    if rows is not None or cols is not None:
        r = np.arange(out.shape[0]) if rows is None else np.asarray(rows)
        c = np.arange(out.shape[1]) if cols is None else np.asarray(cols)
        out = out[np.ix_(r, c)]
    if dtype == "int8":
        assert out.dtype == np.int32
        bad = np.argwhere(out != ref)
        assert bad.size == 0, f"{len(bad)} INT8 mismatches, first at {bad[:5].tolist()}"
        return {"exact": True}
    m = oracle.compare_f16(out, ref) if dtype == "fp16" else oracle.compare_bf16(out, ref)
    assert m["ok"], f"{dtype}: {m}"
    return m
