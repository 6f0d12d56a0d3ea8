"""Python binding of the gfx950 preshuffle GEMM library (libgemm_preshuffle.so).

Argument marshalling only: every step of the GEMM runs in the library's HIP
kernels. PyTorch supplies device memory and the current stream. The entry
points have the names of the C ABI (include/gemm_preshuffle.h):

    gemm_preshuffle_b(b, dtype)                      -> preshuffled B (uint8, flat)
    gemm_a8w8(a, b_shuf, scale_a, scale_b, ...)      -> C int32 (INT8) or bf16 (FP8)
    gemm_bf16(a, b_shuf, ...)                        -> C bf16
    gemm_mxfp4(a, scale_a, b_shuf, scale_b, ...)     -> C bf16
    gemm_f16(a, b_shuf, ...)                         -> C fp16
    gemm_w4a8(a, b_shuf, scale_a, scale_b, ...)      -> C bf16 (int8 A, INT4 B)
    gemm_ex(dtype, a, b_shuf, ..., bias, act)        -> any type with the fused
                                                        bias / activation epilogue
    gemm_plan(dtype, M, N, K, opts)                  -> dict (host-only planner query)
    gemm_ex_ws(dtype, ..., workspace=ws)             -> gemm_ex with a device workspace, which
                                                        lets the planner split K across workgroups
    gemm_workspace_size(dtype, M, N, K, opts)        -> bytes gemm_ex_ws needs (0: none)
    gemm_plan_ws(dtype, M, N, K, opts)               -> dict, the plan of gemm_ex_ws
    workspace(dtype, M, N, K, opts)                  -> a zeroed device workspace of that size
    gemm_ex_noalloc(dtype, ...)                      -> gemm_ex_ws on the library's own static
                                                        device workspace (allocates nothing)

Tensors: A is [M, K] (INT8 / FP8 as any 1-byte dtype, BF16 / FP16 as
bfloat16 / float16 or a 2-byte integer view, MXFP4 as uint8 [M, K/2]; W4A8:
int8 [M, K]); B before the shuffle is [N, K] the same way (W4A8: packed INT4
uint8 [N, K/2]). If the library has not been built the first call raises
GemmLibraryMissing: there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "GemmError", "GemmLibraryMissing", "GemmOpts", "lib_path", "load_library",
    "gemm_preshuffle_b", "gemm_a8w8", "gemm_bf16", "gemm_mxfp4", "gemm_f16", "gemm_w4a8", "gemm_ex",
    "gemm_plan", "ACTS", "gemm_ex_ws", "gemm_ex_noalloc", "gemm_workspace_size", "gemm_plan_ws", "workspace",
    "gemm_status_string", "source_hash", "DTYPES", "EPI_DIRECT", "EPI_CSHUFFLE", "KERNEL_TILE", "KERNEL_SPLITK",
    "KERNEL_WIDE",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libgemm_preshuffle.so"

# gp_dtype values of the C ABI
GP_I8, GP_FP8_E4M3, GP_BF16, GP_FP4_E2M1, GP_I32, GP_F16, GP_I4 = 0, 1, 2, 3, 4, 5, 6
DTYPES = {"int8": GP_I8, "fp8": GP_FP8_E4M3, "bf16": GP_BF16, "mxfp4": GP_FP4_E2M1,
          "fp16": GP_F16, "w4a8": GP_I4}
_ELEM_BITS = {GP_I8: 8, GP_FP8_E4M3: 8, GP_BF16: 16, GP_FP4_E2M1: 4, GP_F16: 16, GP_I4: 4}   # of B
_OUT = {GP_I8: GP_I32, GP_FP8_E4M3: GP_BF16, GP_BF16: GP_BF16, GP_FP4_E2M1: GP_BF16, GP_F16: GP_F16,
        GP_I4: GP_BF16}
# gp_status values of a HIP runtime or launch error, and of a missing / too small workspace
GP_EHIP = 5
GP_EWORKSPACE = 6
# gp_act values of the C ABI
ACTS = {"none": 0, "relu": 1, "silu": 2, "gelu": 3}
EPI_AUTO, EPI_DIRECT, EPI_CSHUFFLE = 0, 1, 2
KERNEL_AUTO, KERNEL_TILE, KERNEL_SPLITK, KERNEL_WIDE = 0, 1, 2, 3


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: status {status} ({gemm_status_string(status)})"
        if status == GP_EHIP and _lib is not None:
            msg += f" [{_lib.gemm_last_hip_error().decode()} from {_lib.gemm_last_hip_call().decode()}]"
        super().__init__(msg)


class GemmLibraryMissing(ImportError):
    pass


class GemmOpts(ctypes.Structure):
    _fields_ = [("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int), ("tile_k", ctypes.c_int),
                ("epilogue", ctypes.c_int), ("kernel", ctypes.c_int), ("xcd_swizzle", ctypes.c_int),
                ("waves", ctypes.c_int), ("mfma", ctypes.c_int), ("pipeline", ctypes.c_int),
                ("ksplit", ctypes.c_int), ("scheduler", ctypes.c_int)]


class GemmPlanInfo(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int),
                ("tile_k", ctypes.c_int), ("epilogue", ctypes.c_int), ("xcd_swizzle", ctypes.c_int),
                ("waves", ctypes.c_int), ("threads", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("grid", ctypes.c_int64), ("k_tiles", ctypes.c_int64),
                ("mfma_per_wave_tile", ctypes.c_int64), ("mfma_total", ctypes.c_int64),
                ("mfma", ctypes.c_int), ("pipeline", ctypes.c_int), ("ksplit", ctypes.c_int),
                ("scheduler", ctypes.c_int), ("workspace_bytes", ctypes.c_int64)]


_lib = None


def lib_path() -> str:
    return os.environ.get("GEMM_PRESHUFFLE_LIB", os.path.join(_PKG, _LIB_NAME))


def load_library():
    """Load (once) and return the ctypes handle of the HIP library."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise GemmLibraryMissing(
            f"{path} is not built; run `python -m dense_gemm_preshuffle_amd.build` "
            "(or __graft_entry__.build()) first")
    # PyTorch ships its own HIP and HSA runtimes under the sonames of ROCm's
    # (libamdhip64.so.7, libhsa-runtime64.so.1). Loaded after torch, this
    # library binds to those copies: one runtime per process. Loaded before
    # torch, it would bind to /opt/rocm's copies and torch would then load
    # its own: two runtimes, and the second to start finds no device
    # (hipGetDevice: hipErrorNoDevice). So torch is imported first.
    import torch  # noqa: F401

    lib = ctypes.CDLL(path)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.gemm_preshuffle_b.argtypes = [vp, vp, i64, i64, ci, vp]
    lib.gemm_a8w8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ci, ci, ctypes.POINTER(GemmOpts), vp]
    lib.gemm_bf16.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.POINTER(GemmOpts), vp]
    lib.gemm_mxfp4.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.POINTER(GemmOpts), vp]
    lib.gemm_f16.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.POINTER(GemmOpts), vp]
    lib.gemm_w4a8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.POINTER(GemmOpts), vp]
    lib.gemm_ex.argtypes = [ci, ci, vp, vp, vp, vp, vp, ci, vp, i64, i64, i64, ctypes.POINTER(GemmOpts), vp]
    lib.gemm_plan.argtypes = [ci, i64, i64, i64, ctypes.POINTER(GemmOpts), ctypes.POINTER(GemmPlanInfo)]
    lib.gemm_plan_ws.argtypes = [ci, i64, i64, i64, ctypes.POINTER(GemmOpts), ctypes.POINTER(GemmPlanInfo)]
    lib.gemm_workspace_size.argtypes = [ci, i64, i64, i64, ctypes.POINTER(GemmOpts), ctypes.POINTER(ctypes.c_size_t)]
    lib.gemm_ex_ws.argtypes = [ci, ci, vp, vp, vp, vp, vp, ci, vp, i64, i64, i64, ctypes.POINTER(GemmOpts), vp,
                               ctypes.c_size_t, vp]
    lib.gemm_ex_noalloc.argtypes = [ci, ci, vp, vp, vp, vp, vp, ci, vp, i64, i64, i64, ctypes.POINTER(GemmOpts), vp]
    lib.gemm_status_string.argtypes = [ci]
    lib.gemm_status_string.restype = ctypes.c_char_p
    lib.gemm_last_hip_error.argtypes = []
    lib.gemm_last_hip_error.restype = ctypes.c_char_p
    lib.gemm_last_hip_call.argtypes = []
    lib.gemm_last_hip_call.restype = ctypes.c_char_p
    for f in ("gemm_preshuffle_b", "gemm_a8w8", "gemm_bf16", "gemm_mxfp4", "gemm_f16", "gemm_w4a8", "gemm_ex",
              "gemm_plan", "gemm_plan_ws", "gemm_workspace_size", "gemm_ex_ws", "gemm_ex_noalloc"):
        getattr(lib, f).restype = ci
    _lib = lib
    return lib


def source_hash() -> str:
    """SHA-256 over the HIP sources of the library (identifies a kernel build)."""
    import hashlib

    csrc = os.path.join(_PKG, "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def header_functions() -> list:
    """Names of the functions the public header declares."""
    hdr = os.path.join(os.path.dirname(_PKG), "include", "gemm_preshuffle.h")
    txt = open(hdr).read()
    return re.findall(r"^(?:int|const char\*)\s+(\w+)\(", txt, flags=re.M)


def gemm_status_string(status: int) -> str:
    try:
        return load_library().gemm_status_string(int(status)).decode()
    except GemmLibraryMissing:
        return "library not built"


def _opts(opts):
    if opts is None:
        return None
    if isinstance(opts, GemmOpts):
        return ctypes.byref(opts)
    o = GemmOpts()
    for k, v in dict(opts).items():
        setattr(o, k, int(v))
    return ctypes.byref(o)


def _dt(x) -> int:
    return DTYPES[x] if isinstance(x, str) else int(x)


def _stream(stream):
    import torch

    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(status: int, where: str):
    if status != 0:
        raise GemmError(status, where)


def _row_bytes(t) -> int:
    return t.shape[-1] * t.element_size()


def gemm_plan(dtype, M: int, N: int, K: int, opts=None) -> dict:
    """Host-only: the plan a GEMM call with these sizes and options would launch."""
    info = GemmPlanInfo()
    _check(load_library().gemm_plan(_dt(dtype), M, N, K, _opts(opts), ctypes.byref(info)), "gemm_plan")
    return {name: getattr(info, name) for name, _ in GemmPlanInfo._fields_}


def gemm_plan_ws(dtype, M: int, N: int, K: int, opts=None) -> dict:
    """Host-only: the plan of gemm_ex_ws with these sizes and options (it may split K)."""
    info = GemmPlanInfo()
    _check(load_library().gemm_plan_ws(_dt(dtype), M, N, K, _opts(opts), ctypes.byref(info)), "gemm_plan_ws")
    return {name: getattr(info, name) for name, _ in GemmPlanInfo._fields_}


def gemm_workspace_size(dtype, M: int, N: int, K: int, opts=None) -> int:
    """Host-only: workspace bytes a gemm_ex_ws call with these arguments needs (0: none)."""
    n = ctypes.c_size_t()
    _check(load_library().gemm_workspace_size(_dt(dtype), M, N, K, _opts(opts), ctypes.byref(n)),
           "gemm_workspace_size")
    return int(n.value)


def workspace(dtype, M: int, N: int, K: int, opts=None, device="cuda"):
    """A zero-filled device workspace for gemm_ex_ws with these arguments (None when none is needed).
    Zero once here; every call leaves its counters zero again."""
    import torch

    n = gemm_workspace_size(dtype, M, N, K, opts)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def gemm_preshuffle_b(b, dtype, out=None, stream=None):
    """B [N, K] (device tensor) -> preshuffled bytes (uint8, flat, N*Kb)."""
    import torch

    dt = _dt(dtype)
    N = b.shape[0]
    Kb = _row_bytes(b)
    K = Kb * 8 // _ELEM_BITS[dt]
    if out is None:
        out = torch.empty(N * Kb, dtype=torch.uint8, device=b.device)
    _check(load_library().gemm_preshuffle_b(_ptr(b), _ptr(out), N, K, dt, _stream(stream)),
           "gemm_preshuffle_b")
    return out


def gemm_a8w8(a, b_shuf, scale_a=None, scale_b=None, c=None, N=None, in_dtype="int8",
              opts=None, stream=None):
    """INT8 (-> int32, no scales) or FP8 E4M3 (-> bf16, fp32 scales) GEMM."""
    import torch

    dt = _dt(in_dtype)
    M, K = a.shape[0], _row_bytes(a)
    if N is None:
        N = b_shuf.numel() * b_shuf.element_size() // K
    out_dt = GP_I32 if dt == GP_I8 else GP_BF16
    if c is None:
        c = torch.empty(M, N, dtype=torch.int32 if out_dt == GP_I32 else torch.bfloat16, device=a.device)
    _check(load_library().gemm_a8w8(_ptr(a), _ptr(b_shuf), _ptr(scale_a), _ptr(scale_b), _ptr(c),
                                    M, N, K, dt, out_dt, _opts(opts), _stream(stream)), "gemm_a8w8")
    return c


def gemm_bf16(a, b_shuf, c=None, N=None, opts=None, stream=None):
    """BF16 GEMM, bf16 output."""
    import torch

    M, K = a.shape[0], a.shape[1]
    if N is None:
        N = b_shuf.numel() * b_shuf.element_size() // (2 * K)
    if c is None:
        c = torch.empty(M, N, dtype=torch.bfloat16, device=a.device)
    _check(load_library().gemm_bf16(_ptr(a), _ptr(b_shuf), _ptr(c), M, N, K, _opts(opts), _stream(stream)),
           "gemm_bf16")
    return c


def gemm_mxfp4(a, scale_a, b_shuf, scale_b, c=None, N=None, opts=None, stream=None):
    """MXFP4 GEMM: a uint8 [M, K/2], scale_a uint8 [M, K/32], bf16 output."""
    import torch

    M, K = a.shape[0], 2 * _row_bytes(a)
    if N is None:
        N = b_shuf.numel() * b_shuf.element_size() * 2 // K
    if c is None:
        c = torch.empty(M, N, dtype=torch.bfloat16, device=a.device)
    _check(load_library().gemm_mxfp4(_ptr(a), _ptr(scale_a), _ptr(b_shuf), _ptr(scale_b), _ptr(c),
                                     M, N, K, _opts(opts), _stream(stream)), "gemm_mxfp4")
    return c


def gemm_f16(a, b_shuf, c=None, N=None, opts=None, stream=None):
    """FP16 GEMM, fp16 output."""
    import torch

    M, K = a.shape[0], a.shape[1]
    if N is None:
        N = b_shuf.numel() * b_shuf.element_size() // (2 * K)
    if c is None:
        c = torch.empty(M, N, dtype=torch.float16, device=a.device)
    _check(load_library().gemm_f16(_ptr(a), _ptr(b_shuf), _ptr(c), M, N, K, _opts(opts), _stream(stream)),
           "gemm_f16")
    return c


def gemm_w4a8(a, b_shuf, scale_a, scale_b, c=None, N=None, opts=None, stream=None):
    """int8 A [M, K] x INT4 B (preshuffled as GP_I4), fp32 scales, bf16 output."""
    import torch

    M, K = a.shape[0], _row_bytes(a)
    if N is None:
        N = b_shuf.numel() * b_shuf.element_size() * 2 // K
    if c is None:
        c = torch.empty(M, N, dtype=torch.bfloat16, device=a.device)
    _check(load_library().gemm_w4a8(_ptr(a), _ptr(b_shuf), _ptr(scale_a), _ptr(scale_b), _ptr(c),
                                    M, N, K, _opts(opts), _stream(stream)), "gemm_w4a8")
    return c


def gemm_ex(dtype, a, b_shuf, scale_a=None, scale_b=None, bias=None, act="none", c=None, N=None,
            opts=None, stream=None):
    """Any input type with the fused epilogue: C = act(scaled accumulator + bias[n])."""
    import torch

    dt = _dt(dtype)
    out_dt = _OUT[dt]
    M = a.shape[0]
    K = _row_bytes(a) * 8 // (8 if dt == GP_I4 else _ELEM_BITS[dt])
    if N is None:
        N = b_shuf.numel() * b_shuf.element_size() * 8 // (K * _ELEM_BITS[dt])
    if c is None:
        tdt = {GP_I32: torch.int32, GP_BF16: torch.bfloat16, GP_F16: torch.float16}[out_dt]
        c = torch.empty(M, N, dtype=tdt, device=a.device)
    a_ = ACTS[act] if isinstance(act, str) else int(act)
    _check(load_library().gemm_ex(dt, out_dt, _ptr(a), _ptr(b_shuf), _ptr(scale_a), _ptr(scale_b), _ptr(bias),
                                  a_, _ptr(c), M, N, K, _opts(opts), _stream(stream)), "gemm_ex")
    return c


def gemm_ex_ws(dtype, a, b_shuf, scale_a=None, scale_b=None, bias=None, act="none", c=None, N=None,
               opts=None, workspace=None, stream=None):
    """gemm_ex with a device workspace (a uint8 tensor from `workspace()`), so
    that the planner may split K across workgroups."""
    import torch

    dt = _dt(dtype)
    out_dt = _OUT[dt]
    M = a.shape[0]
    K = _row_bytes(a) * 8 // (8 if dt == GP_I4 else _ELEM_BITS[dt])
    if N is None:
        N = b_shuf.numel() * b_shuf.element_size() * 8 // (K * _ELEM_BITS[dt])
    if c is None:
        tdt = {GP_I32: torch.int32, GP_BF16: torch.bfloat16, GP_F16: torch.float16}[out_dt]
        c = torch.empty(M, N, dtype=tdt, device=a.device)
    a_ = ACTS[act] if isinstance(act, str) else int(act)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().gemm_ex_ws(dt, out_dt, _ptr(a), _ptr(b_shuf), _ptr(scale_a), _ptr(scale_b), _ptr(bias),
                                     a_, _ptr(c), M, N, K, _opts(opts), _ptr(workspace), nbytes, _stream(stream)),
           "gemm_ex_ws")
    return c


def gemm_ex_noalloc(dtype, a, b_shuf, c, scale_a=None, scale_b=None, bias=None, act="none", N=None, opts=None,
                    stream=None):
    """gemm_ex_ws on the library's own static device workspace: nothing is
    allocated, so the output tensor `c` must be given. Calls that overlap in
    time on one device share that workspace and must not be made."""
    dt = _dt(dtype)
    out_dt = _OUT[dt]
    M = a.shape[0]
    K = _row_bytes(a) * 8 // (8 if dt == GP_I4 else _ELEM_BITS[dt])
    if N is None:
        N = b_shuf.numel() * b_shuf.element_size() * 8 // (K * _ELEM_BITS[dt])
    a_ = ACTS[act] if isinstance(act, str) else int(act)
    _check(load_library().gemm_ex_noalloc(dt, out_dt, _ptr(a), _ptr(b_shuf), _ptr(scale_a), _ptr(scale_b),
                                          _ptr(bias), a_, _ptr(c), M, N, K, _opts(opts), _stream(stream)),
           "gemm_ex_noalloc")
    return c
