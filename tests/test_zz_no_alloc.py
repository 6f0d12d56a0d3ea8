"""gemm_ex_noalloc (the library's static workspace) against gemm_ex_ws (a
caller's workspace), through the C ABI: two calls in a row, the second on a
smaller problem, each bitwise equal to gemm_ex_ws with the same plan and
within the oracle's bounds; a plan larger than the static workspace is
refused before anything is launched."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from tests._parity import say

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_noalloc_matches_caller_workspace_twice(dtype):
    import torch

    import dense_gemm_preshuffle_amd as gp
    from dense_gemm_preshuffle_amd import workload

    lib = gp.load_library()
    shapes = {"fp8": [(256, 2048, 16384), (128, 2048, 8192)], "bf16": [(256, 1024, 8192), (192, 1024, 8192)]}[dtype]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for M, N, K in shapes:
        plan = gp.gemm_plan_ws(dtype, M, N, K)
        say(f"no-alloc {dtype} {M}x{N}x{K}: ksplit {plan['ksplit']} workspace {plan['workspace_bytes']}")
        assert plan["ksplit"] > 1 and 0 < plan["workspace_bytes"] <= 32 * 2**20 + 65536
        host = workloads.make_inputs(dtype, M, N, K, seed=M + K)
        p = workload.prepare(dtype, workload.to_device(dtype, host))
        ws = torch.zeros(plan["workspace_bytes"], dtype=torch.uint8, device="cuda")
        tdt = torch.bfloat16
        c_ws = torch.empty(M, N, dtype=tdt, device="cuda")
        c_na = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
        dt, out_dt = gp.DTYPES[dtype], 2
        args = (dt, out_dt, _p(p["a"]), _p(p["b_shuf"]), _p(p.get("scale_a")), _p(p.get("scale_b")), None, 0)
        st = lib.gemm_ex_ws(*args, _p(c_ws), M, N, K, None, _p(ws), ws.numel(), stream)
        assert st == 0, gp.gemm_status_string(st)
        st = lib.gemm_ex_noalloc(*args, _p(c_na), M, N, K, None, stream)
        assert st == 0, gp.gemm_status_string(st)
        torch.cuda.synchronize()
        o_ws, o_na = workload.to_host(c_ws), workload.to_host(c_na)
        assert np.array_equal(o_ws, o_na), "static-workspace result differs from the caller-workspace one"
        m = oracle.compare_bf16(o_na, oracle.gemm(dtype, host))
        assert m["ok"], m


def test_noalloc_refuses_plans_beyond_its_workspace():
    import dense_gemm_preshuffle_amd as gp

    lib = gp.load_library()
    # BF16 1024 x 2048 x 16384 in 8 K ranges of 128 x 256 tiles: 64 MiB of partial sums
    o = gp.GemmOpts(kernel=1, tile_m=128, tile_n=256, tile_k=64, ksplit=8)
    assert gp.gemm_workspace_size("bf16", 1024, 2048, 16384, o) > 32 * 2**20 + 65536
    fake = ctypes.c_void_p(0x100000)     # validation fails before any pointer is used
    st = lib.gemm_ex_noalloc(2, 2, fake, fake, None, None, None, 0, fake, 1024, 2048, 16384, ctypes.byref(o), None)
    assert st == gp.GP_EWORKSPACE
