"""Parity at the workloads' full sizes, in the planner's default launch
configuration (the one the benchmark times). Every output is compared:
INT8 bit-exact, the floating-point types within the normwise and floored
elementwise bounds of oracle.compare, against the float64 oracle computed
in full on the host (BF16 / FP16 8192^3 take a few seconds of BLAS)."""
import pytest

import workloads
from tests._parity import check, gpu_run, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", sorted(workloads.CONFIGS))
def test_config_parity(name):
    import dense_gemm_preshuffle_amd as gp

    dtype, M, N, K, seed, tile = workloads.CONFIGS[name]
    plan = gp.gemm_plan(dtype, M, N, K)
    say(f"config {name}: plan {plan}")
    host = workloads.make_inputs(dtype, M, N, K, seed)
    out = gpu_run(dtype, host)
    m = check(dtype, host, out)
    say(f"config {name}: all {M * N} outputs: {m}")


@pytest.mark.parametrize("name", ["fp8_512x4096x4096", "bf16_8192x8192x8192"])
def test_named_tile_parity(name):
    """The tiles the workloads name (64x256x128 FP8, 128x256x64 BF16), every output."""
    dtype, M, N, K, seed, tile = workloads.CONFIGS[name]
    opts = dict(kernel=1, tile_m=tile[0], tile_n=tile[1], tile_k=tile[2])
    say(f"named tile {name} {opts}")
    host = workloads.make_inputs(dtype, M, N, K, seed)
    out = gpu_run(dtype, host, opts)
    m = check(dtype, host, out)
    say(f"named tile {name}: all {M * N} outputs: {m}")
