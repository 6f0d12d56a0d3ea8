"""The planner's own choice on seeded random shapes (M 17-4096, N a multiple
of 16 in 64-8192, K a multiple of 256 in 512-16384), with and without a
workspace: whatever kernel, tile, row blocks, K chunks or K split it picks,
the outputs of a sample of rows (the first and last 8, 8 from the middle and
8 drawn at random, over every column) match the oracle to the bounds of
oracle.compare (INT8 bit-exact), and two calls with the workspace give
bitwise the same result."""
import random

import numpy as np
import pytest

import oracle
import workloads
from tests._parity import check, gpu_run, say

pytestmark = pytest.mark.gpu


def _shapes(per_type=10, seed=20261202):
    rnd = random.Random(seed)
    out = []
    for dtype in ("fp8", "int8", "bf16", "fp16", "w4a8", "mxfp4"):
        n = 0
        while n < per_type:
            M = int(round(np.exp(rnd.uniform(np.log(17), np.log(4096)))))
            N = 16 * max(4, int(round(np.exp(rnd.uniform(np.log(64), np.log(8192))) / 16)))
            K = 256 * max(2, int(round(np.exp(rnd.uniform(np.log(512), np.log(16384))) / 256)))
            if M * N * K > 2**36:
                continue
            out.append((dtype, M, N, K))
            n += 1
    return out


def _rows(M, seed):
    rnd = np.random.default_rng(seed)
    mid = M // 2
    pick = np.r_[0:8, max(0, mid - 4):mid + 4, M - 8:M, rnd.integers(0, M, 8)]
    return np.unique(np.clip(pick, 0, M - 1))


@pytest.mark.parametrize("dtype,M,N,K", _shapes(), ids=lambda v: str(v))
def test_planner_choice_parity(dtype, M, N, K):
    import torch

    import dense_gemm_preshuffle_amd as gp
    from dense_gemm_preshuffle_amd import workload

    p_ws, p_plain = gp.gemm_plan_ws(dtype, M, N, K), gp.gemm_plan(dtype, M, N, K)
    say(f"random {dtype} {M}x{N}x{K}: with workspace kernel {p_ws['kernel']} tile {p_ws['tile_m']}x"
        f"{p_ws['tile_n']}x{p_ws['tile_k']} ksplit {p_ws['ksplit']} grid {p_ws['grid']}; without kernel "
        f"{p_plain['kernel']} tile {p_plain['tile_m']}x{p_plain['tile_n']}x{p_plain['tile_k']}")
    host = workloads.make_inputs(dtype, M, N, K, seed=M * 31 + N * 7 + K)
    rows = _rows(M, M + N + K)
    ref = oracle.gemm(dtype, host, rows, None)
    # without a workspace
    check(dtype, host, gpu_run(dtype, host), rows=rows, ref=ref)
    # with one: the planner may split K; two calls, bitwise equal
    dev = workload.to_device(dtype, host)
    p = workload.prepare(dtype, dev)
    nbytes = gp.gemm_workspace_size(dtype, M, N, K)
    assert nbytes == p_ws["workspace_bytes"]
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
    outs = []
    for _ in range(2):
        c = gp.gemm_ex_ws(dtype, p["a"], p["b_shuf"], p.get("scale_a"), p.get("scale_b"), N=N, workspace=ws)
        torch.cuda.synchronize()
        outs.append(workload.to_host(c))
    assert np.array_equal(outs[0], outs[1]), "results differ between two calls"
    check(dtype, host, outs[0], rows=rows, ref=ref)


_ACTS = ("relu", "silu", "gelu")


@pytest.mark.parametrize("dtype,M,N,K", [s for s in _shapes() if s[0] != "int8"], ids=lambda v: str(v))
def test_planner_choice_fused_epilogue(dtype, M, N, K):
    """The same shapes with a bias and an activation (the floating-point
    types), given a workspace: every planner path runs the fused epilogue,
    after the partial sums where it splits K."""
    import torch

    import dense_gemm_preshuffle_amd as gp
    from dense_gemm_preshuffle_amd import workload

    act = _ACTS[(M + N + K) % 3]
    plan = gp.gemm_plan_ws(dtype, M, N, K)
    say(f"random fused {act} {dtype} {M}x{N}x{K}: kernel {plan['kernel']} tile {plan['tile_m']}x{plan['tile_n']} "
        f"ksplit {plan['ksplit']}")
    host = workloads.make_inputs(dtype, M, N, K, seed=M * 13 + N + K * 3, bias=True)
    p = workload.prepare(dtype, workload.to_device(dtype, host))
    p["workspace"] = gp.workspace(dtype, M, N, K, None)
    outs = []
    for _ in range(2):
        c = workload.run(dtype, p, act=act)
        torch.cuda.synchronize()
        outs.append(workload.to_host(c))
    assert np.array_equal(outs[0], outs[1]), "results differ between two calls"
    rows = _rows(M, M * 3 + N + K)
    check(dtype, host, outs[0], rows=rows, ref=oracle.gemm(dtype, host, rows, None, act=act), act=act)
