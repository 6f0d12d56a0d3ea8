"""GEMMs whose largest buffer is just under 2^31 bytes, the most the library
takes (its kernels address every buffer with 32-bit offsets), so that the
top of that range is exercised: B, A or C at 2 146 435 072 bytes. The first
and last 16 rows and columns and a block in the middle are compared with the
oracle on those rows and columns: bit for bit for INT8, within the bf16
bounds for BF16 (2-byte elements: other offset arithmetic). C starts filled
with a value no result can take (INT8: int32 min, as |a|, |b| <= 8 and
K <= 65536; BF16: NaN, as the inputs are finite), and none may be left."""
import numpy as np
import pytest

import oracle
import workloads
from tests._parity import check, say

pytestmark = pytest.mark.gpu

# (type, what sits at the limit, M, N, K); INT8 bytes: A = M*K, B = N*K, C = 4*M*N
CASES = [
    ("int8", "B", 16, 32752, 65536),       # small-M kernel, 16-column workgroups
    ("int8", "B", 256, 32752, 65536),      # tile kernel; the last column tile overlaps its neighbour
    ("int8", "A", 32752, 64, 65536),
    ("int8", "C", 16384, 32752, 64),
    ("bf16", "B", 256, 32752, 32768),
]


def _sample(n):
    mid = n // 2
    return np.unique(np.r_[0:16, mid - 8:mid + 8, n - 16:n])


@pytest.mark.parametrize("dtype,what,M,N,K", CASES, ids=lambda v: str(v))
def test_buffer_just_under_2_31_bytes(dtype, what, M, N, K):
    import torch

    import dense_gemm_preshuffle_amd as gp
    from dense_gemm_preshuffle_amd import workload

    eb = 1 if dtype == "int8" else 2
    size = {"A": M * K * eb, "B": N * K * eb, "C": M * N * (4 if dtype == "int8" else 2)}[what]
    assert 2**31 - 2**21 < size < 2**31
    plan = gp.gemm_plan(dtype, M, N, K)
    say(f"limit {what} {dtype} {M}x{N}x{K} ({size} bytes): kernel {plan['kernel']} "
        f"tile {plan['tile_m']}x{plan['tile_n']}x{plan['tile_k']} grid {plan['grid']}")
    host = workloads.make_inputs(dtype, M, N, K, seed=M + N + K)
    dev = workload.to_device(dtype, host)
    p = workload.prepare(dtype, dev)
    if dtype == "int8":
        c = torch.full((M, N), int(np.iinfo(np.int32).min), dtype=torch.int32, device="cuda")
    else:
        c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    workload.run(dtype, p, c=c)
    torch.cuda.synchronize()
    left = (c == int(np.iinfo(np.int32).min)) if dtype == "int8" else torch.isnan(c)
    assert int(left.sum().item()) == 0, "outputs left unwritten"
    rows, cols = _sample(M), _sample(N)
    got = workload.to_host(c[torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(cols, device="cuda")])
    check(dtype, host, got, ref=oracle.gemm(dtype, host, rows, cols))
    del dev, p, c
    torch.cuda.empty_cache()
