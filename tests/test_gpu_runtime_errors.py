"""A HIP error left behind by an earlier runtime call of the caller is not
reported as the library's own.

HIP keeps one "last error" per thread, set by any failing runtime call and
read (and cleared) by hipGetLastError. The library reads it right after each
launch to learn the launch's status, so it clears it right before the
launch: otherwise an error from an unrelated, earlier call in the same
thread (the application's or a framework's: the process has one HIP runtime,
shared by everything that links it) would come back as GP_EHIP from a launch
that succeeded."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from tests._parity import say

pytestmark = pytest.mark.gpu


def _hip_runtimes():
    """Distinct HIP runtime files mapped into this process."""
    return {line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line}


def test_stale_error_of_an_earlier_call_is_not_a_launch_error():
    import torch

    import dense_gemm_preshuffle_amd as gp
    from dense_gemm_preshuffle_amd import workload

    say("stale runtime error before gemm_preshuffle_b / gemm_a8w8")
    lib = gp.load_library()
    host = workloads.make_inputs("fp8", 16, 512, 1024, seed=31)
    dev = workload.to_device("fp8", host)
    torch.cuda.synchronize()
    assert len(_hip_runtimes()) == 1, _hip_runtimes()   # the library and torch share one runtime
    hip = ctypes.CDLL("libamdhip64.so.7")                # that same runtime (matched by its soname)
    for call in ("preshuffle", "gemm"):
        # a failing call with no lasting effect: an attribute of a device that does not exist
        v = ctypes.c_int()
        assert hip.hipDeviceGetAttribute(ctypes.byref(v), 0, 4096) != 0
        assert hip.hipPeekAtLastError() != 0              # the thread's last error is now set
        if call == "preshuffle":
            b_shuf = torch.empty(dev["b"].numel(), dtype=torch.uint8, device="cuda")
            st = lib.gemm_preshuffle_b(ctypes.c_void_p(dev["b"].data_ptr()), ctypes.c_void_p(b_shuf.data_ptr()),
                                       512, 1024, gp.DTYPES["fp8"],
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        else:
            c = torch.empty(16, 512, dtype=torch.bfloat16, device="cuda")
            st = lib.gemm_a8w8(*(ctypes.c_void_p(t.data_ptr()) for t in (dev["a"], b_shuf, dev["scale_a"],
                                                                          dev["scale_b"], c)),
                               16, 512, 1024, gp.DTYPES["fp8"], 2, None,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, (call, st, lib.gemm_last_hip_error())
        assert lib.gemm_last_hip_error() == b"hipSuccess"
        assert lib.gemm_last_hip_call() == b""
    torch.cuda.synchronize()
    assert np.array_equal(b_shuf.cpu().numpy(), oracle.preshuffle(host["b"]))
    out = workload.to_host(c)
    assert oracle.compare_bf16(out, oracle.gemm("fp8", host))["ok"]
