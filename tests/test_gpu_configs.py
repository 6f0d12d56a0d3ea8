"""Parity at the workloads' full sizes, in the planner's default launch
configuration (the one the benchmark times). INT8 is compared in full and
bit-exact; FP8 in full; BF16 8192^3 and MXFP4 4096x4096x8192 on a sample of
rows and columns that touches the first and last tiles in both dimensions."""
import numpy as np
import pytest

import workloads
from tests._parity import check, gpu_run, say

pytestmark = pytest.mark.gpu


def _sample(n, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.unique(np.concatenate([np.arange(16), np.arange(n - 16, n), rng.choice(n, k, replace=False)]))
    return idx


@pytest.mark.parametrize("name", sorted(workloads.CONFIGS))
def test_config_parity(name):
    import dense_gemm_preshuffle_amd as gp

    dtype, M, N, K, seed, tile = workloads.CONFIGS[name]
    plan = gp.gemm_plan(dtype, M, N, K)
    say(f"config {name}: plan {plan}")
    host = workloads.make_inputs(dtype, M, N, K, seed)
    out = gpu_run(dtype, host)
    if M * N * K <= 2 ** 34:
        m = check(dtype, host, out)
    else:
        rows, cols = _sample(M, 224, seed), _sample(N, 224, seed + 1)
        m = check(dtype, host, out, rows=rows, cols=cols)
    say(f"config {name}: {m}")


@pytest.mark.parametrize("name", ["fp8_512x4096x4096", "bf16_8192x8192x8192"])
def test_named_tile_parity(name):
    """The tiles the workloads name (64x256x128 FP8, 128x256x64 BF16)."""
    dtype, M, N, K, seed, tile = workloads.CONFIGS[name]
    opts = dict(kernel=1, tile_m=tile[0], tile_n=tile[1], tile_k=tile[2])
    say(f"named tile {name} {opts}")
    host = workloads.make_inputs(dtype, M, N, K, seed)
    out = gpu_run(dtype, host, opts)
    rows, cols = _sample(M, 128, seed + 2), _sample(N, 128, seed + 3)
    check(dtype, host, out, rows=rows, cols=cols)
