"""Marshal host arrays of one GEMM problem onto the GPU and run it.

`to_device` copies the arrays (A, B and their scales) to device tensors,
`prepare` runs the library's B preshuffle pass once, and `run` launches the
GEMM entry point that matches the input type. Nothing here computes any part
of the GEMM.
"""
from __future__ import annotations

import numpy as np

from . import gemm_a8w8, gemm_bf16, gemm_ex, gemm_ex_ws, gemm_f16, gemm_mxfp4, gemm_preshuffle_b, gemm_w4a8


def to_device(dtype: str, host: dict, device="cuda") -> dict:
    import torch

    out = {}
    for k, v in host.items():
        arr = np.ascontiguousarray(v)
        if arr.dtype == np.uint16:
            t = torch.from_numpy(arr.view(np.int16)).view(torch.float16 if dtype == "fp16" else torch.bfloat16)
        else:
            t = torch.from_numpy(arr)
        out[k] = t.to(device)
    return out


def prepare(dtype: str, dev: dict, stream=None) -> dict:
    p = dict(dev)
    p["b_shuf"] = gemm_preshuffle_b(dev["b"], dtype, stream=stream)
    p["N"] = dev["b"].shape[0]
    return p


def run(dtype: str, p: dict, opts=None, c=None, stream=None, act=None):
    """Launch the type's own entry point, or gemm_ex with the fused epilogue
    (bias p["bias"] if present, activation `act`) when `act` is given, or
    gemm_ex_ws when p holds a "workspace" entry (a tensor, or None where the
    plan needs none)."""
    N = p["N"]
    if "workspace" in p:
        return gemm_ex_ws(dtype, p["a"], p["b_shuf"], p.get("scale_a"), p.get("scale_b"), p.get("bias"),
                          act or "none", c=c, N=N, opts=opts, workspace=p["workspace"], stream=stream)
    if act is not None:
        return gemm_ex(dtype, p["a"], p["b_shuf"], p.get("scale_a"), p.get("scale_b"), p.get("bias"), act,
                       c=c, N=N, opts=opts, stream=stream)
    if dtype in ("int8", "fp8"):
        return gemm_a8w8(p["a"], p["b_shuf"], p.get("scale_a"), p.get("scale_b"), c=c, N=N,
                         in_dtype=dtype, opts=opts, stream=stream)
    if dtype == "bf16":
        return gemm_bf16(p["a"], p["b_shuf"], c=c, N=N, opts=opts, stream=stream)
    if dtype == "mxfp4":
        return gemm_mxfp4(p["a"], p["scale_a"], p["b_shuf"], p["scale_b"], c=c, N=N, opts=opts, stream=stream)
    if dtype == "fp16":
        return gemm_f16(p["a"], p["b_shuf"], c=c, N=N, opts=opts, stream=stream)
    if dtype == "w4a8":
        return gemm_w4a8(p["a"], p["b_shuf"], p["scale_a"], p["scale_b"], c=c, N=N, opts=opts, stream=stream)
    raise ValueError(dtype)


def to_host(c) -> np.ndarray:
    """int32 result -> int32 array; bf16 / fp16 result -> uint16 bit patterns."""
    import torch

    c = c.cpu()
    if c.dtype in (torch.bfloat16, torch.float16):
        return c.view(torch.int16).numpy().view(np.uint16)
    return c.numpy()
