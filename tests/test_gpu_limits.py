"""GEMMs whose largest buffer is just under 2^31 bytes, the most the library
takes (its kernels address every buffer with 32-bit offsets), so that the
top of that range is exercised: B, A or C at 2 146 435 072 bytes. INT8, so
the sampled outputs are compared bit for bit: the first and last 16 rows and
columns and a block in the middle, against the oracle on those rows and
columns. C starts filled with a value no INT8 result can take
(|a|, |b| <= 8, K <= 65536), and none may be left."""
import numpy as np
import pytest

import oracle
import workloads
from tests._parity import say

pytestmark = pytest.mark.gpu

SENTINEL = np.iinfo(np.int32).min

# (what sits at the limit, M, N, K); INT8 bytes: A = M*K, B = N*K, C = 4*M*N
CASES = [
    ("B", 16, 32752, 65536),       # small-M kernel, 16-column workgroups
    ("B", 256, 32752, 65536),      # tile kernel; the last column tile overlaps its neighbour
    ("A", 32752, 64, 65536),
    ("C", 16384, 32752, 64),
]


def _sample(n):
    mid = n // 2
    return np.unique(np.r_[0:16, mid - 8:mid + 8, n - 16:n])


@pytest.mark.parametrize("what,M,N,K", CASES, ids=lambda v: str(v))
def test_buffer_just_under_2_31_bytes(what, M, N, K):
    import torch

    import dense_gemm_preshuffle_amd as gp
    from dense_gemm_preshuffle_amd import workload

    size = {"A": M * K, "B": N * K, "C": 4 * M * N}[what]
    assert 2**31 - 2**21 < size < 2**31
    plan = gp.gemm_plan("int8", M, N, K)
    say(f"limit {what} int8 {M}x{N}x{K} ({size} bytes): kernel {plan['kernel']} "
        f"tile {plan['tile_m']}x{plan['tile_n']}x{plan['tile_k']} grid {plan['grid']}")
    host = workloads.make_inputs("int8", M, N, K, seed=M + N + K)
    dev = workload.to_device("int8", host)
    p = workload.prepare("int8", dev)
    c = torch.full((M, N), int(SENTINEL), dtype=torch.int32, device="cuda")
    workload.run("int8", p, c=c)
    torch.cuda.synchronize()
    assert int((c == int(SENTINEL)).sum().item()) == 0, "outputs left unwritten"
    rows, cols = _sample(M), _sample(N)
    got = c[torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(cols, device="cuda")].cpu().numpy()
    ref = oracle.gemm("int8", host, rows, cols)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:5].tolist()}"
    del dev, p, c
    torch.cuda.empty_cache()
