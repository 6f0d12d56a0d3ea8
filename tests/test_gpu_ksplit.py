"""K split across workgroups (gemm_ex_ws) and the scheduler-off variants,
through the C ABI, against the oracle.

A K split changes only how the fp32 / int32 sums are grouped: INT8 stays
bit-exact, the other types stay within the oracle.compare bounds. The
workgroups of a tile may finish in any order, yet the partial sums are added
in the fixed order of their K ranges, so two runs give the same bits; every
call leaves the workspace's arrival counters at zero."""
import numpy as np
import pytest

import oracle
import workloads
from tests._parity import check, say

pytestmark = pytest.mark.gpu


def _run_ws(dtype, host, opts, repeat=2, ws_extra=0):
    import torch

    import dense_gemm_preshuffle_amd as gp
    from dense_gemm_preshuffle_amd import workload

    dev = workload.to_device(dtype, host)
    p = workload.prepare(dtype, dev)
    M, K = host["a"].shape[0], (host["a"].shape[1] * (2 if dtype in ("mxfp4",) else 1))
    N = p["N"]
    plan = gp.gemm_plan_ws(dtype, M, N, K, opts)
    nbytes = gp.gemm_workspace_size(dtype, M, N, K, opts)
    assert nbytes == plan["workspace_bytes"]
    ws = torch.zeros(nbytes + ws_extra, dtype=torch.uint8, device="cuda") if nbytes else None
    outs = []
    for _ in range(repeat):
        c = gp.gemm_ex_ws(dtype, p["a"], p["b_shuf"], p.get("scale_a"), p.get("scale_b"), N=N, opts=opts,
                          workspace=ws)
        torch.cuda.synchronize()
        outs.append(workload.to_host(c))
    if ws is not None:
        tiles = -(-M // plan["tile_m"]) * -(-N // plan["tile_n"])
        cnt = ws[: 4 * tiles].view(torch.int32).cpu().numpy()
        assert not cnt.any(), "arrival counters not back to zero"
    return plan, outs


KSPLIT_CASES = [
    # dtype, M, N, K, opts (tile, ksplit)
    ("fp8", 128, 256, 2048, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, ksplit=2)),
    ("fp8", 128, 256, 2048, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, ksplit=8)),
    ("fp8", 256, 512, 2048, dict(kernel=1, tile_m=128, tile_n=128, tile_k=128, ksplit=4)),
    ("fp8", 256, 256, 3072, dict(kernel=1, tile_m=128, tile_n=128, tile_k=256, ksplit=3)),
    ("fp8", 128, 512, 1024, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128, ksplit=2, epilogue=2)),
    ("fp8", 64, 512, 2048, dict(kernel=1, tile_m=32, tile_n=256, tile_k=256, ksplit=4)),
    ("fp8", 200, 400, 2048, dict(kernel=1, tile_m=128, tile_n=128, tile_k=256, ksplit=2)),     # ragged M, N
    ("int8", 128, 256, 2048, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, ksplit=4)),
    ("int8", 256, 256, 1024, dict(kernel=1, tile_m=128, tile_n=128, tile_k=128, ksplit=2)),
    ("bf16", 256, 512, 1024, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, ksplit=4)),
    ("bf16", 128, 256, 512, dict(kernel=1, tile_m=64, tile_n=128, tile_k=64, ksplit=2)),
    ("fp16", 256, 512, 1024, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, ksplit=2)),
    ("fp16", 192, 384, 2048, dict(kernel=1, tile_m=64, tile_n=128, tile_k=64, ksplit=8)),
    ("fp16", 100, 208, 1024, dict(kernel=1, tile_m=64, tile_n=128, tile_k=64, ksplit=4)),   # ragged M, N
    # MXFP4: 8-tile scale groups; a split of 16 K tiles into 2 (whole groups)
    # and 4 (half groups: each range starts inside its first group's row)
    ("mxfp4", 128, 256, 4096, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, ksplit=2)),
    ("mxfp4", 128, 256, 4096, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, ksplit=4)),
    ("mxfp4", 256, 256, 2048, dict(kernel=1, tile_m=128, tile_n=128, tile_k=256, ksplit=2)),
    ("w4a8", 128, 256, 2048, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, ksplit=2)),
    ("w4a8", 128, 512, 4096, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128, ksplit=4)),
]


@pytest.mark.parametrize("dtype,M,N,K,opts", KSPLIT_CASES)
def test_ksplit_parity_and_repeatability(dtype, M, N, K, opts):
    say(f"ksplit {dtype} {M}x{N}x{K} {opts}")
    host = workloads.make_inputs(dtype, M, N, K, seed=M + N + K + opts["ksplit"])
    plan, (o1, o2) = _run_ws(dtype, host, opts)
    assert plan["ksplit"] == opts["ksplit"] and plan["workspace_bytes"] > 0
    assert np.array_equal(o1, o2), "K-split result differs between runs"
    check(dtype, host, o1)


def test_ksplit_full_size_fp8_512():
    """FP8 512x4096x4096 with a K split, every output, twice (bitwise equal)."""
    name = "fp8_512x4096x4096"
    dtype, M, N, K, seed, _ = workloads.CONFIGS[name]
    opts = dict(kernel=1, tile_m=128, tile_n=128, tile_k=256, ksplit=2)
    say(f"ksplit full size {name} {opts}")
    host = workloads.make_inputs(dtype, M, N, K, seed)
    plan, (o1, o2) = _run_ws(dtype, host, opts)
    assert np.array_equal(o1, o2)
    check(dtype, host, o1)


def test_workspace_errors():
    import torch

    import dense_gemm_preshuffle_amd as gp
    from dense_gemm_preshuffle_amd import workload

    say("workspace errors")
    host = workloads.make_inputs("fp8", 128, 256, 2048, seed=5)
    p = workload.prepare("fp8", workload.to_device("fp8", host))
    opts = dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, ksplit=2)
    need = gp.gemm_workspace_size("fp8", 128, 256, 2048, opts)
    assert need > 0
    for ws in (None, torch.zeros(need - 16, dtype=torch.uint8, device="cuda")):
        with pytest.raises(gp.GemmError) as e:
            gp.gemm_ex_ws("fp8", p["a"], p["b_shuf"], p["scale_a"], p["scale_b"], N=256, opts=opts, workspace=ws)
        assert e.value.status == gp.GP_EWORKSPACE
    # a split through an entry point without a workspace
    with pytest.raises(gp.GemmError) as e:
        gp.gemm_a8w8(p["a"], p["b_shuf"], p["scale_a"], p["scale_b"], N=256, in_dtype="fp8", opts=opts)
    assert e.value.status == gp.GP_EWORKSPACE
    # no split needed: no workspace needed
    assert gp.gemm_workspace_size("fp8", 128, 256, 2048, dict(ksplit=1)) == 0
    c = gp.gemm_ex_ws("fp8", p["a"], p["b_shuf"], p["scale_a"], p["scale_b"], N=256, opts=dict(ksplit=1))
    torch.cuda.synchronize()
    check("fp8", host, workload.to_host(c))


SCHED_OFF_CASES = [
    ("int8", 64, 128, 1024, dict(kernel=1, tile_m=16, tile_n=64, tile_k=256)),
    ("int8", 128, 256, 1024, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, pipeline=3)),
    ("fp8", 128, 256, 1024, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, pipeline=3)),
    ("fp8", 128, 512, 768, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128, pipeline=3)),
    ("fp8", 256, 512, 640, dict(kernel=1, tile_m=128, tile_n=256, tile_k=128, pipeline=3)),
    ("fp8", 256, 256, 768, dict(kernel=1, tile_m=128, tile_n=128, tile_k=256, pipeline=3)),
    ("bf16", 256, 512, 448, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, pipeline=3)),
    ("fp16", 256, 512, 448, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, pipeline=3)),
    ("bf16", 512, 512, 640, dict(kernel=1, tile_m=256, tile_n=256, tile_k=64, mfma=16, pipeline=3)),
    ("fp16", 512, 512, 384, dict(kernel=1, tile_m=256, tile_n=256, tile_k=64, mfma=16, pipeline=3)),
    ("bf16", 256, 1024, 448, dict(kernel=1, tile_m=128, tile_n=512, tile_k=64, mfma=16, pipeline=3)),
    ("fp16", 256, 1024, 320, dict(kernel=1, tile_m=128, tile_n=512, tile_k=64, mfma=16, pipeline=3)),
    ("mxfp4", 256, 512, 2816, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, mfma=32, pipeline=2)),
    ("w4a8", 128, 256, 1280, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, pipeline=3)),
]


@pytest.mark.parametrize("dtype,M,N,K,opts", SCHED_OFF_CASES)
def test_scheduler_off_parity(dtype, M, N, K, opts):
    """The same tiles with the compiler's own hot-loop order (scheduler off)
    and with the pinned one (scheduler on)."""
    import dense_gemm_preshuffle_amd as gp
    from tests._parity import gpu_run

    say(f"scheduler off {dtype} {M}x{N}x{K} {opts}")
    host = workloads.make_inputs(dtype, M, N, K, seed=M * 3 + K)
    for sched in (1, 2):
        o = dict(opts, scheduler=sched)
        assert gp.gemm_plan(dtype, M, N, K, o)["scheduler"] == sched
        check(dtype, host, gpu_run(dtype, host, o))


@pytest.mark.parametrize("dtype,M,N,K", [("fp8", 128, 4096, 8192), ("mxfp4", 256, 4096, 16384),
                                         ("bf16", 256, 1024, 8192), ("w4a8", 256, 4096, 8192),
                                         ("int8", 128, 1024, 16384), ("fp8", 200, 2000, 16384),
                                         # a full grid of small tiles, split over larger ones (BF16 / FP16)
                                         ("bf16", 512, 4096, 16384), ("fp16", 256, 4096, 8192),
                                         # from a 128 x 128 first choice onto 128 x 256 tiles in two ranges
                                         ("bf16", 512, 8192, 8192),
                                         # FP8 with 16 rows and long K: 16 x 64 tiles in 8 ranges (N = 1008:
                                         # the last column tile overlaps its neighbour)
                                         ("fp8", 16, 2048, 16384), ("fp8", 16, 1008, 16384),
                                         ("int8", 16, 2048, 16384), ("bf16", 16, 2048, 8192),
                                         ("fp16", 16, 1008, 8192), ("w4a8", 16, 1024, 32768),
                                         # 17 to 64 rows: ceil(M / 16) row tiles of 16 (M = 40, 17: the last
                                         # row tile overlaps its neighbour)
                                         ("fp8", 48, 1024, 32768), ("fp8", 40, 2048, 16384),
                                         ("fp8", 17, 1008, 16384), ("int8", 64, 1024, 16384),
                                         ("bf16", 32, 2048, 8192), ("fp16", 64, 1024, 16384),
                                         ("w4a8", 24, 1024, 32768),
                                         # 64 x 128 tiles: BF16 / FP16 in 2x the ranges from 64 tiles, INT8 in four
                                         ("bf16", 256, 2048, 8192), ("fp16", 192, 2048, 8192), ("int8", 192, 2048, 8192),
                                         # 4-bit B in ranges of 2048 K elements (1024 bytes)
                                         ("mxfp4", 384, 2048, 8192), ("w4a8", 128, 7168, 4096)])
def test_automatic_split_parity(dtype, M, N, K):
    """The planner's own split (no options) on long-K shapes, every output."""
    import dense_gemm_preshuffle_amd as gp

    plan = gp.gemm_plan_ws(dtype, M, N, K)
    say(f"automatic split {dtype} {M}x{N}x{K}: {plan}")
    assert plan["ksplit"] > 1
    host = workloads.make_inputs(dtype, M, N, K, seed=K + M)
    _, (o1, o2) = _run_ws(dtype, host, None)
    assert np.array_equal(o1, o2)
    check(dtype, host, o1)


def test_one_workspace_serves_shapes_of_any_size():
    """One zeroed workspace, calls with fewer, then more, then fewer tiles:
    the counters always sit in the same fixed area, so no call finds an
    earlier call's partial sums where its counters are."""
    import torch

    import dense_gemm_preshuffle_amd as gp
    from dense_gemm_preshuffle_amd import workload

    cases = [("fp8", 128, 2048, 8192), ("fp8", 256, 4096, 16384), ("fp8", 128, 1024, 16384), ("fp8", 200, 2000, 16384)]
    need = max(gp.gemm_workspace_size(*c) for c in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for dtype, M, N, K in cases:
        plan = gp.gemm_plan_ws(dtype, M, N, K)
        say(f"shared workspace {dtype} {M}x{N}x{K}: ksplit {plan['ksplit']} grid {plan['grid']}")
        assert plan["ksplit"] > 1
        host = workloads.make_inputs(dtype, M, N, K, seed=M + N)
        p = workload.prepare(dtype, workload.to_device(dtype, host))
        c = gp.gemm_ex_ws(dtype, p["a"], p["b_shuf"], p["scale_a"], p["scale_b"], N=N, workspace=ws)
        torch.cuda.synchronize()
        check(dtype, host, workload.to_host(c))
    assert not ws[:65536].any().item()


@pytest.mark.parametrize("dtype,M,N,K,act", [("fp8", 16, 2048, 16384, "gelu"), ("fp8", 128, 4096, 8192, "silu"),
                                             ("bf16", 512, 4096, 16384, "relu"), ("mxfp4", 256, 4096, 16384, "gelu"),
                                             ("w4a8", 256, 4096, 8192, "none"), ("fp16", 256, 4096, 8192, "silu"),
                                             ("bf16", 16, 2048, 8192, "relu"), ("w4a8", 16, 1024, 32768, "gelu"),
                                             ("fp8", 40, 2048, 16384, "silu"), ("bf16", 64, 1024, 16384, "gelu"),
                                             ("fp16", 192, 2048, 8192, "gelu")])
def test_split_with_fused_epilogue(dtype, M, N, K, act):
    """gemm_ex_ws with a bias and an activation on shapes the planner splits:
    the last workgroup of each tile adds the partial sums, then runs the
    fused epilogue (bias, activation) like an unsplit tile."""
    import torch

    import dense_gemm_preshuffle_amd as gp
    from dense_gemm_preshuffle_amd import workload

    plan = gp.gemm_plan_ws(dtype, M, N, K)
    say(f"split + fused {act} {dtype} {M}x{N}x{K}: ksplit {plan['ksplit']} tile {plan['tile_m']}x{plan['tile_n']}")
    assert plan["ksplit"] > 1
    host = workloads.make_inputs(dtype, M, N, K, seed=M + N + K + 5, bias=True)
    dev = workload.to_device(dtype, host)
    p = workload.prepare(dtype, dev)
    p["workspace"] = gp.workspace(dtype, M, N, K, None)
    outs = []
    for _ in range(2):
        c = workload.run(dtype, p, act=act)
        torch.cuda.synchronize()
        outs.append(workload.to_host(c))
    assert np.array_equal(outs[0], outs[1])
    check(dtype, host, outs[0], act=act)
