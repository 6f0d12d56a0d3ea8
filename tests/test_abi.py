"""The C-ABI library: it loads, exports every function the header declares,
and its host-side logic (validation, planner) behaves as documented. Nothing
here launches GPU work: every call below fails validation or is the
host-only planner query."""
import ctypes
import os

import pytest

import dense_gemm_preshuffle_amd as gp
from oracle import formulas as F
from workloads import CONFIGS

GP_OK, GP_EINVAL, GP_ESHAPE, GP_EDTYPE = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    return gp.load_library()


def test_exports_every_header_function(lib):
    names = gp.header_functions()
    assert set(names) >= {"gemm_preshuffle_b", "gemm_a8w8", "gemm_bf16", "gemm_mxfp4", "gemm_f16",
                          "gemm_w4a8", "gemm_ex", "gemm_plan", "gemm_status_string"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(6):
        assert lib.gemm_status_string(s)
    assert b"unknown" in lib.gemm_status_string(99)


FAKE = ctypes.c_void_p(0x100000)   # aligned, never dereferenced: validation fails first
MIS = ctypes.c_void_p(0x100008)    # misaligned


@pytest.fixture
def fake_ptrs(lib):
    """The validation tests below pass addresses that are not device memory;
    each call is meant to fail validation before any HIP call. On a host
    with a GPU a wrong expectation would launch a kernel on them, so these
    tests run only where no GPU driver is present."""
    if os.path.exists("/dev/kfd"):
        pytest.skip("fake-pointer validation tests run on hosts without a GPU")
    return lib


def test_null_and_misaligned_pointers(fake_ptrs):
    lib = fake_ptrs
    assert lib.gemm_bf16(None, FAKE, FAKE, 128, 256, 64, None, None) == GP_EINVAL
    assert lib.gemm_bf16(MIS, FAKE, FAKE, 128, 256, 64, None, None) == GP_EINVAL
    assert lib.gemm_a8w8(FAKE, FAKE, None, None, None, 16, 16, 64, 0, 4, None, None) == GP_EINVAL
    assert lib.gemm_mxfp4(FAKE, None, FAKE, FAKE, FAKE, 16, 16, 128, None, None) == GP_EINVAL
    assert lib.gemm_preshuffle_b(FAKE, None, 16, 64, 0, None) == GP_EINVAL
    # overlapping preshuffle buffers
    assert lib.gemm_preshuffle_b(FAKE, ctypes.c_void_p(0x100000 + 512), 16, 64, 0, None) == GP_EINVAL


def test_sizes_and_shapes(fake_ptrs):
    lib = fake_ptrs
    assert lib.gemm_bf16(FAKE, FAKE, FAKE, 0, 256, 64, None, None) == GP_EINVAL      # empty
    assert lib.gemm_bf16(FAKE, FAKE, FAKE, 128, -16, 64, None, None) == GP_EINVAL
    assert lib.gemm_bf16(FAKE, FAKE, FAKE, 128, 250, 64, None, None) == GP_ESHAPE    # N % 16
    assert lib.gemm_bf16(FAKE, FAKE, FAKE, 128, 256, 48, None, None) == GP_ESHAPE    # Kb % 64
    assert lib.gemm_a8w8(FAKE, FAKE, None, None, FAKE, 16, 16, 96, 0, 4, None, None) == GP_ESHAPE
    assert lib.gemm_preshuffle_b(FAKE, ctypes.c_void_p(0x900000), 16, 32, 0, None) == GP_ESHAPE
    assert lib.gemm_preshuffle_b(FAKE, ctypes.c_void_p(0x900000), 24, 64, 0, None) == GP_ESHAPE
    # 2^31-byte limit of the 32-bit buffer offsets
    assert lib.gemm_bf16(FAKE, FAKE, FAKE, 65536, 65536, 65536, None, None) == GP_ESHAPE


@pytest.mark.parametrize("M,N,K", [(2 ** 61 + 64, 16, 64), (64, 2 ** 61 + 16, 64), (64, 16, 2 ** 61 + 64),
                                   (2 ** 31, 16, 64), (2 ** 30, 2 ** 30, 64), (2 ** 62, 2 ** 62, 2 ** 62)])
def test_huge_sizes_are_rejected_without_overflow(M, N, K):
    """Sizes whose byte counts overflow int64 when multiplied are GP_ESHAPE,
    not a plan for the wrapped-around size (host-only planner query)."""
    info = gp.GemmPlanInfo()
    for dt in (0, 1, 2, 3, 5, 6):
        assert gp.load_library().gemm_plan(dt, M, N, K, None, ctypes.byref(info)) == GP_ESHAPE, (dt, M, N, K)


@pytest.mark.parametrize("N,K", [(2 ** 61 + 16, 64), (16, 2 ** 61 + 64), (2 ** 30, 64), (2 ** 62, 2 ** 62)])
def test_huge_preshuffle_sizes_are_rejected(fake_ptrs, N, K):
    assert fake_ptrs.gemm_preshuffle_b(FAKE, ctypes.c_void_p(0x900000), N, K, 0, None) == GP_ESHAPE


def test_dtype_pairs(fake_ptrs):
    lib = fake_ptrs
    S = ctypes.c_void_p(0x200000)
    # INT8 must have int32 output and no scales
    assert lib.gemm_a8w8(FAKE, FAKE, None, None, FAKE, 16, 16, 64, 0, 2, None, None) == GP_EDTYPE
    assert lib.gemm_a8w8(FAKE, FAKE, S, S, FAKE, 16, 16, 64, 0, 4, None, None) == GP_EDTYPE
    # FP8 must have bf16 output and both scales
    assert lib.gemm_a8w8(FAKE, FAKE, None, None, FAKE, 16, 16, 64, 1, 2, None, None) == GP_EDTYPE
    assert lib.gemm_a8w8(FAKE, FAKE, S, S, FAKE, 16, 16, 64, 1, 4, None, None) == GP_EDTYPE
    assert lib.gemm_a8w8(FAKE, FAKE, S, S, FAKE, 16, 16, 64, 2, 2, None, None) == GP_EDTYPE
    assert lib.gemm_preshuffle_b(FAKE, ctypes.c_void_p(0x900000), 16, 64, 7, None) == GP_EDTYPE


def test_options_validation():
    with pytest.raises(gp.GemmError) as e:
        gp.gemm_plan("fp8", 512, 4096, 4096, dict(tile_m=64, tile_n=256, tile_k=96, kernel=1))
    assert e.value.status == GP_ESHAPE                  # tile not compiled
    with pytest.raises(gp.GemmError) as e:
        gp.gemm_plan("fp8", 512, 4096, 4096, dict(epilogue=7))
    assert e.value.status == GP_EINVAL
    with pytest.raises(gp.GemmError) as e:
        gp.gemm_plan("fp8", 512, 4096, 4096, dict(tile_m=64))   # partial tile spec
    assert e.value.status == GP_EINVAL
    with pytest.raises(gp.GemmError) as e:
        gp.gemm_plan("mxfp4", 64, 256, 192)             # FP4 needs K % 128
    assert e.value.status == GP_ESHAPE


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_plan_mfma_count_and_flops(name):
    dtype, M, N, K, _, _ = CONFIGS[name]
    p = gp.gemm_plan(dtype, M, N, K)
    assert p["mfma_total"] == F.mfma_count_gfx950(dtype, M, N, K, p["mfma"])
    assert p["mfma_total"] * F.flops_per_mfma_gfx950(dtype, p["mfma"]) == F.flops(M, N, K)
    assert p["grid"] > 0 and p["threads"] in (256, 512)


def test_named_tiles_plan():
    p = gp.gemm_plan("fp8", 512, 4096, 4096, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128, epilogue=1,
                                                   pipeline=1))
    # the pages' formula counts gfx942 K=32 instructions; gfx950 FP8 takes K=128
    assert p["mfma_per_wave_tile"] * 4 == F.mfma_per_tile_pages(64, 256, 128)
    assert p["grid"] == 128 and p["k_tiles"] == 32 and p["mfma"] == 16
    fp8_scales = 256 * (1 + 256 // 64)              # FP8 row / column scales staged in LDS
    assert p["lds_bytes"] == F.lds_bytes(64, 256, 128, 1) + fp8_scales
    p = gp.gemm_plan("bf16", 8192, 8192, 8192, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, epilogue=1, mfma=16,
                                                     pipeline=1))
    assert p["grid"] == 2048 and p["k_tiles"] == 128
    assert p["mfma_per_wave_tile"] == 64            # 2 K32 steps x 8 x 4
    p = gp.gemm_plan("bf16", 8192, 8192, 8192, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, epilogue=1,
                                                     pipeline=1, mfma=32))
    assert p["mfma"] == 32 and p["mfma_per_wave_tile"] == 32   # 4 K16 steps x 4 x 2 (32x32 blocks)
    assert p["lds_bytes"] == F.lds_bytes(128, 256, 64, 2)
    p = gp.gemm_plan("fp8", 512, 4096, 4096, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128, epilogue=2))
    assert p["lds_bytes"] == 64 * (256 * 2 + 16) + fp8_scales   # padded CShuffle tile (above 3 stages of A)
    p = gp.gemm_plan("fp8", 512, 4096, 4096, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128, epilogue=1, pipeline=3))
    assert p["lds_bytes"] == 3 * 64 * 128 + fp8_scales and p["pipeline"] == 3
    # default epilogue: CShuffle for tile_n >= 128 while two workgroups fit a CU
    assert gp.gemm_plan("bf16", 8192, 8192, 8192)["epilogue"] == gp.EPI_CSHUFFLE
    assert gp.gemm_plan("int8", 4096, 4096, 4096, dict(kernel=1, tile_m=128, tile_n=256, tile_k=128))["epilogue"] == gp.EPI_DIRECT


def test_worked_example_plan():
    # GEMM Optimization Guide §14: 5120 x 5120 x 8320, tile 64 x 256 x 128 FP8
    p = gp.gemm_plan("fp8", 5120, 5120, 8320, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128, pipeline=1))
    assert p["grid"] == 1600 and p["k_tiles"] == 65
    assert p["mfma_per_wave_tile"] * p["k_tiles"] * 4 == 4160   # in gfx942 K=32 instructions


def test_wide_kernel_plan():
    p = gp.gemm_plan("bf16", 8192, 8192, 8192, dict(kernel=3))
    assert p["kernel"] == gp.KERNEL_WIDE and (p["tile_m"], p["tile_n"]) == (256, 256)
    assert p["waves"] == 8 and p["threads"] == 512 and p["grid"] == 1024
    # every MFMA of the problem is issued once: per wave per K tile x waves x workgroups x K tiles
    assert p["mfma_per_wave_tile"] * 8 * p["grid"] * p["k_tiles"] == p["mfma_total"]
    assert p["mfma_total"] == F.mfma_count_gfx950("bf16", 8192, 8192, 8192, p["mfma"])
    # A and B stages (256 rows each) or the padded bf16 C tile, whichever is larger
    assert p["lds_bytes"] == max(p["pipeline"] * 512 * p["tile_k"] * 2, 256 * (256 * 2 + 16))
    q = gp.gemm_plan("int8", 512, 512, 512, dict(kernel=3, mfma=32))
    assert q["epilogue"] == gp.EPI_DIRECT and q["mfma"] == 32
    assert q["mfma_per_wave_tile"] * 8 * q["grid"] * q["k_tiles"] == q["mfma_total"]
    for bad in (dict(kernel=3, tile_m=128, tile_n=256, tile_k=64), dict(kernel=3, pipeline=1),
                dict(kernel=3, epilogue=1)):
        with pytest.raises(gp.GemmError) as e:
            gp.gemm_plan("bf16", 512, 512, 512, bad)
        assert e.value.status == GP_ESHAPE
    with pytest.raises(gp.GemmError):
        gp.gemm_plan("mxfp4", 512, 512, 512, dict(kernel=3))     # FP4 runs on the 4-wave kernel
    with pytest.raises(gp.GemmError):
        gp.gemm_plan("bf16", 192, 512, 512, dict(kernel=3))      # M below one 256-row tile


def test_small_m_uses_split_k():
    p = gp.gemm_plan("fp8", 16, 7168, 2048)
    assert p["kernel"] == gp.KERNEL_SPLITK and p["tile_m"] == 16


def test_every_gpu_case_has_a_plan():
    """Every option set the GPU parity tests use is accepted by the planner
    (host-only check, so planner mistakes show up without a GPU)."""
    from tests.test_gpu_parity import EPI_CASES, FP4_PLACEMENT_OPTS, PERM_CASES, RAGGED_CASES, TILE_CASES

    for dtype, M, N, K, opts in TILE_CASES + PERM_CASES + RAGGED_CASES + EPI_CASES:
        p = gp.gemm_plan(dtype, M, N, K, opts)
        assert p["grid"] > 0, (dtype, M, N, K, opts)
    for opts in FP4_PLACEMENT_OPTS:
        gp.gemm_plan("mxfp4", 128, 256, 1024, opts)
    for opts in (dict(kernel=1, tile_m=64, tile_n=256, tile_k=256), dict(kernel=1, tile_m=128, tile_n=256, tile_k=256)):
        gp.gemm_plan("mxfp4", 128, 256, 1024, opts)
    gp.gemm_plan("mxfp4", 16, 64, 1024, dict(kernel=2))


def test_gemm_ex_validation(fake_ptrs):
    lib = fake_ptrs
    S = ctypes.c_void_p(0x200000)
    B = ctypes.c_void_p(0x300000)
    GP_I8, GP_FP8, GP_BF16, GP_FP4, GP_I32, GP_F16, GP_I4 = 0, 1, 2, 3, 4, 5, 6
    ex = lib.gemm_ex
    # activation outside the enum; misaligned bias
    assert ex(GP_BF16, GP_BF16, FAKE, FAKE, None, None, B, 4, FAKE, 128, 256, 64, None, None) == GP_EINVAL
    assert ex(GP_BF16, GP_BF16, FAKE, FAKE, None, None, B, -1, FAKE, 128, 256, 64, None, None) == GP_EINVAL
    assert ex(GP_BF16, GP_BF16, FAKE, FAKE, None, None, MIS, 1, FAKE, 128, 256, 64, None, None) == GP_EINVAL
    # the exact INT8 -> int32 path takes no bias and no activation
    assert ex(GP_I8, GP_I32, FAKE, FAKE, None, None, B, 0, FAKE, 16, 16, 64, None, None) == GP_EDTYPE
    assert ex(GP_I8, GP_I32, FAKE, FAKE, None, None, None, 1, FAKE, 16, 16, 64, None, None) == GP_EDTYPE
    # output types: FP16 -> fp16 only, the others -> bf16
    assert ex(GP_F16, GP_BF16, FAKE, FAKE, None, None, None, 0, FAKE, 16, 16, 64, None, None) == GP_EDTYPE
    assert ex(GP_BF16, GP_F16, FAKE, FAKE, None, None, None, 0, FAKE, 16, 16, 64, None, None) == GP_EDTYPE
    assert ex(GP_I4, GP_I32, FAKE, FAKE, S, S, None, 0, FAKE, 16, 16, 512, None, None) == GP_EDTYPE
    # scale vectors: required for FP8 / MXFP4 / W4A8, refused for BF16 / FP16
    assert ex(GP_I4, GP_BF16, FAKE, FAKE, None, S, None, 0, FAKE, 16, 16, 512, None, None) == GP_EDTYPE
    assert ex(GP_BF16, GP_BF16, FAKE, FAKE, S, None, None, 0, FAKE, 16, 16, 64, None, None) == GP_EDTYPE
    assert ex(9, GP_BF16, FAKE, FAKE, None, None, None, 0, FAKE, 16, 16, 64, None, None) == GP_EDTYPE
    # named wrappers validate the same way
    assert lib.gemm_w4a8(FAKE, FAKE, None, S, FAKE, 16, 16, 512, None, None) == GP_EDTYPE
    assert lib.gemm_f16(FAKE, FAKE, None, 16, 16, 64, None, None) == GP_EINVAL
    assert lib.gemm_w4a8(FAKE, FAKE, S, S, FAKE, 16, 16, 320, None, None) == GP_ESHAPE   # K % 128 (INT4 layout)


def test_w4a8_plan():
    p = gp.gemm_plan("w4a8", 16, 7168, 2048)
    assert p["kernel"] == gp.KERNEL_SPLITK
    assert p["mfma_total"] == F.mfma_count_gfx950("w4a8", 16, 7168, 2048)
    with pytest.raises(gp.GemmError) as e:
        gp.gemm_plan("w4a8", 512, 512, 2048, dict(kernel=3))   # no 256 x 256 W4A8 kernel
    assert e.value.status == GP_EDTYPE
    with pytest.raises(gp.GemmError) as e:
        gp.gemm_plan("w4a8", 16, 256, 2 * 65536)               # int32 range of the 16x widened products
    assert e.value.status == GP_ESHAPE
    q = gp.gemm_plan("w4a8", 300, 512, 4096, dict(kernel=2, tile_m=64))   # small-M kernel, any M: 4 row blocks
    assert q["tile_m"] == 64 and q["grid"] == (512 // q["tile_n"]) * 5   # per workgroup, the last partial
    # larger M: the tile kernel, two int8 MFMAs per 64-byte INT4 piece; A
    # tiles (int8) are twice the bytes of the B tile's K extent
    t = gp.gemm_plan("w4a8", 512, 4096, 4096)
    assert t["kernel"] == gp.KERNEL_TILE and (t["tile_m"], t["tile_n"], t["tile_k"]) == (64, 128, 256)
    assert t["mfma_total"] == F.mfma_count_gfx950("w4a8", 512, 4096, 4096)
    assert t["lds_bytes"] == t["pipeline"] * 64 * 256 + 256 * (1 + 2)   # A stages + fp32 scale blocks
    assert gp.gemm_plan("w4a8", 4096, 4096, 128)["k_tiles"] == 1     # K % 128 on the tile kernel


@pytest.mark.parametrize("dtype,M,N,K", [("bf16", 100, 256, 256), ("fp8", 200, 272, 512), ("int8", 77, 208, 256),
                                         ("mxfp4", 130, 4096, 1024), ("fp16", 40, 128, 128), ("fp8", 5, 512, 2048)])
def test_ragged_plans(dtype, M, N, K):
    """M and N not multiples of the tile: edge tiles overlap inside M x N,
    the grid is the ceiling, and the issued MFMAs cover every output."""
    p = gp.gemm_plan(dtype, M, N, K)
    tm, tn = p["tile_m"], p["tile_n"]
    if p["kernel"] == gp.KERNEL_TILE:
        assert tm <= M and tn <= N
    assert p["grid"] == -(-M // tm) * -(-N // tn)
    assert p["mfma_total"] * F.flops_per_mfma_gfx950(dtype, p["mfma"]) >= F.flops(M, N, K)
    assert p["mfma_total"] == p["grid"] * p["waves"] * p["k_tiles"] * p["mfma_per_wave_tile"]


def test_tile_must_fit_inside_the_problem():
    with pytest.raises(gp.GemmError) as e:
        gp.gemm_plan("bf16", 100, 256, 256, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64))
    assert e.value.status == GP_ESHAPE
    # no tile fits a 48-column problem: the small-M kernel takes it for any M
    assert gp.gemm_plan("fp8", 200, 48, 1024)["kernel"] == gp.KERNEL_SPLITK


def test_fp4_plan_lds_matches_scale_groups():
    """MXFP4 with a 2-stage pipeline stages scales as a ring of two slots of
    8-tile groups (8 x (TM+TN) x 8 bytes each) beside the A stages: for the
    128 x 256 tile exactly the 80 KiB share of each of two workgroups per CU."""
    p = gp.gemm_plan("mxfp4", 4096, 4096, 8192, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256))
    assert p["pipeline"] == 2 and p["tile_k"] == 256 and (p["tile_m"], p["tile_n"]) == (128, 256)
    stages = 2 * p["tile_m"] * 128 + 2 * (8 * (p["tile_m"] + p["tile_n"]) * 8)
    assert stages == 80 * 1024
    cshuffle = p["tile_m"] * (p["tile_n"] * 2 + 16) if p["epilogue"] == gp.EPI_CSHUFFLE else 0
    assert p["lds_bytes"] == max(stages, cshuffle)
    # the default 128 x 512 tile runs 8 waves, one workgroup per CU (160 KiB share)
    q = gp.gemm_plan("mxfp4", 4096, 4096, 8192)
    assert (q["tile_m"], q["tile_n"], q["waves"], q["threads"]) == (128, 512, 8, 512)
    stages = 2 * 128 * 128 + 2 * (8 * (128 + 512) * 8)
    assert q["lds_bytes"] == max(stages, 128 * (512 * 2 + 16)) <= 160 * 1024


def test_k_group_plan():
    """waves=8 on the tile kernel: two groups of 4 waves split the K tiles
    (an even count), each with its own A stages; the issued MFMAs still
    cover the problem exactly once."""
    opts = dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, pipeline=3, waves=8)
    p = gp.gemm_plan("fp8", 512, 4096, 4096, opts)
    assert p["waves"] == 8 and p["threads"] == 512 and p["k_tiles"] == 16
    assert p["mfma_total"] == F.mfma_count_gfx950("fp8", 512, 4096, 4096, p["mfma"])
    q = gp.gemm_plan("fp8", 512, 4096, 4096, dict(opts, waves=4))
    assert q["waves"] == 4 and q["mfma_total"] == p["mfma_total"]
    # two groups' A stages (plus the FP8 scale blocks) against one group's
    assert p["lds_bytes"] == 2 * 3 * 64 * 256 + 256 * (1 + 2)
    assert q["lds_bytes"] == 3 * 64 * 256 + 256 * (1 + 2)
    for bad_k in (3 * 256, 1280):   # odd K-tile counts
        with pytest.raises(gp.GemmError) as e:
            gp.gemm_plan("fp8", 512, 4096, bad_k, opts)
        assert e.value.status == GP_ESHAPE
    with pytest.raises(gp.GemmError):   # a tile without a two-group build
        gp.gemm_plan("fp8", 512, 4096, 4096, dict(opts, tile_m=128, tile_n=256, tile_k=128))
    with pytest.raises(gp.GemmError):   # FP4 stages its scales per group: not built
        gp.gemm_plan("mxfp4", 512, 4096, 4096, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, waves=8))
    with pytest.raises(gp.GemmError):
        gp.gemm_plan("fp8", 512, 4096, 4096, dict(opts, waves=6))


def test_degenerate_shapes_plan():
    """One 16-column block and the shortest K of each type run on the
    small-M kernel with one wave; FP8 needs whole 128-element MFMA steps."""
    for dtype, M, N, K in [("int8", 1, 16, 64), ("fp8", 1, 16, 128), ("bf16", 1, 16, 32), ("fp16", 3, 16, 32),
                           ("mxfp4", 1, 16, 128), ("w4a8", 1, 16, 128), ("bf16", 1000, 16, 64)]:
        p = gp.gemm_plan(dtype, M, N, K)
        assert p["kernel"] == gp.KERNEL_SPLITK and p["waves"] == 1, (dtype, p)
        assert p["mfma_total"] * F.flops_per_mfma_gfx950(dtype, 16) >= F.flops(M, N, K)
    q = gp.gemm_plan("fp8", 16, 7168, 2048)           # the M=16 shape keeps 4 waves
    assert q["waves"] == 4
    with pytest.raises(gp.GemmError) as e:
        gp.gemm_plan("fp8", 16, 256, 64)               # half an FP8 MFMA step
    assert e.value.status == GP_ESHAPE


@pytest.mark.parametrize("dtype,M,N,K", [("int8", 512, 4096, 4160), ("fp16", 512, 4096, 4128),
                                         ("mxfp4", 512, 4096, 4224), ("bf16", 8192, 8192, 8224)])
def test_k_not_a_multiple_of_the_large_tiles(dtype, M, N, K):
    """K a whole number of 64-byte layout blocks but not of 128: the tile
    kernel with 64-byte K tiles, not the small-M kernel."""
    p = gp.gemm_plan(dtype, M, N, K)
    assert p["kernel"] == gp.KERNEL_TILE and p["grid"] >= 64
    assert p["tile_k"] * {"int8": 8, "fp16": 16, "bf16": 16, "mxfp4": 4}[dtype] // 8 == 64
    assert p["mfma_total"] == F.mfma_count_gfx950(dtype, M, N, K, p["mfma"])


@pytest.mark.parametrize("dtype", ["fp8", "bf16", "int8", "mxfp4", "fp16", "w4a8"])
def test_small_m_row_blocks(dtype):
    """The small-M kernel's rows per workgroup: 16, 32, or 64 on 8 waves
    (not MXFP4); more read B once for more rows but give fewer workgroups.
    On 7168 columns (224 workgroups of 32 columns) the largest block that
    holds the rows wins; on 4096, 32 rows; on 1024, 16 (one 256-workgroup
    round). The issued MFMAs still cover every output."""
    four = 2 if dtype == "mxfp4" else 4
    for M, N, mb in [(16, 7168, 1), (5, 7168, 1), (24, 7168, 2), (32, 7168, 2), (48, 7168, four),
                     (64, 7168, four), (100, 7168, four), (64, 4096, 2), (48, 4096, 2), (64, 1024, 1),
                     (33, 2048, 1), (24, 4096, 1)]:
        p = gp.gemm_plan(dtype, M, N, 2048, dict(kernel=2))
        assert p["tile_m"] == 16 * mb, (M, N, p)
        assert p["waves"] == (8 if mb == 4 else 4)
        assert p["grid"] == (N // p["tile_n"]) * -(-M // (16 * mb))
        assert p["mfma_total"] == p["grid"] * p["waves"] * p["k_tiles"] * p["mfma_per_wave_tile"]
        assert p["mfma_total"] * F.flops_per_mfma_gfx950(dtype, 16) >= F.flops(M, N, 2048)
    q = gp.gemm_plan(dtype, 64, 7168, 2048, dict(kernel=2, tile_m=16))
    assert q["tile_m"] == 16


def test_zero_filled_options_plan_like_null():
    """A zero-filled gemm_opts is all-automatic, as NULL is: the same plan on
    shapes that take each of the planner's rules (16-64 row K split, small-M
    kernel above 64 rows, row blocks, 4-bit fallback, the tile splits)."""
    shapes = [("fp8", 16, 2048, 16384), ("fp8", 48, 1024, 32768), ("bf16", 64, 1024, 16384), ("w4a8", 128, 1024, 7168),
              ("int8", 128, 1024, 4096), ("fp8", 64, 2048, 4096), ("mxfp4", 96, 2048, 16384), ("fp8", 128, 3072, 4096),
              ("bf16", 256, 2048, 8192), ("fp16", 192, 2048, 8192), ("fp8", 32, 576, 4352), ("bf16", 113, 1024, 1280),
              ("fp8", 16, 7168, 2048), ("bf16", 8192, 8192, 8192)]
    for dt, M, N, K in shapes:
        assert gp.gemm_plan_ws(dt, M, N, K) == gp.gemm_plan_ws(dt, M, N, K, {}), (dt, M, N, K)
        assert gp.gemm_plan(dt, M, N, K) == gp.gemm_plan(dt, M, N, K, {}), (dt, M, N, K)


def test_half_and_int8_split_on_64x128_tiles():
    """BF16 / FP16 split 64 x 128 tiles (not 128 x 256 where fewer than 32
    of those cover the output), in twice the ranges from 64 tiles up to 512
    workgroups, and only from 144 workgroups (else 16 x 64 tiles); INT8
    takes FP8's four-range and 256-workgroup rules."""
    for dt, M, N, K, tile, ks, grid in [("bf16", 128, 2048, 16384, (64, 128), 8, 256),
                                        ("bf16", 256, 2048, 8192, (64, 128), 8, 512),
                                        ("fp16", 192, 2048, 8192, (64, 128), 8, 384),
                                        ("fp16", 320, 512, 8192, (64, 128), 8, 160),
                                        ("bf16", 80, 512, 16384, (16, 64), 8, 320),
                                        ("bf16", 512, 2048, 16384, (128, 256), 8, 256),
                                        ("int8", 192, 2048, 8192, (64, 128), 4, 192)]:
        p = gp.gemm_plan_ws(dt, M, N, K)
        assert ((p["tile_m"], p["tile_n"]), p["ksplit"], p["grid"]) == (tile, ks, grid), (dt, M, N, K, p)


def test_fp8_split_on_64x128_tiles():
    """FP8's automatic split on 64 x 128 tiles: four ranges where 48 to 64
    tiles cover the output (rows at most 1.5 M, K from 4096 bytes), and no
    more than 256 workgroups where halving the split keeps 168 or more (not
    below two ranges past 8192 bytes of K)."""
    for M, N, K, tile, ks, grid in [(128, 3072, 4096, (64, 128), 4, 192), (256, 2048, 7168, (64, 128), 4, 256),
                                    (160, 4096, 8192, (64, 128), 2, 192), (128, 7168, 8192, (64, 128), 2, 224),
                                    (160, 7168, 16384, (64, 128), 2, 336), (384, 3072, 16384, (64, 128), 2, 288),
                                    (384, 7168, 4096, (128, 128), 1, 168), (80, 3072, 4096, (16, 64), 2, 480)]:
        p = gp.gemm_plan_ws("fp8", M, N, K)
        assert ((p["tile_m"], p["tile_n"]), p["ksplit"], p["grid"]) == (tile, ks, grid), (M, N, K, p)


def test_small_m_kernel_above_64_rows_on_small_outputs():
    """Above 64 rows the planner still takes the small-M kernel where the
    output is small: W4A8 / MXFP4 up to M*N = 2^19 with M*N*K up to 2^31;
    INT8 up to 3*2^18 with M*N*K up to 3*2^29; BF16 / FP16 3*2^18 and 2^30;
    FP8 2^17 and 2^30; K from 1024 (up to 8192 but for W4A8 / MXFP4), M up
    to 4096, and only when no option is set; the K bounds only given a
    workspace (without one the tiles cannot split K)."""
    for ws in (False, True):
        plan = gp.gemm_plan_ws if ws else gp.gemm_plan
        for dt, M, N, K, kern in [("w4a8", 128, 1024, 7168, 2), ("w4a8", 2048, 256, 2048, 2), ("w4a8", 2048, 512, 2048, 1),
                                  ("w4a8", 128, 512, 16384, 2), ("mxfp4", 1024, 512, 2048, 2), ("mxfp4", 4097, 128, 2048, 1),
                                  ("int8", 128, 1024, 4096, 2), ("int8", 128, 256, 512, 1), ("int8", 128, 1024, 16384, 1),
                                  ("int8", 1024, 512, 4096, 1), ("bf16", 128, 2048, 4096, 2), ("bf16", 256, 2048, 4096, 1),
                                  ("fp16", 96, 1024, 7168, 2), ("fp8", 128, 1024, 4096, 2), ("fp8", 128, 2048, 4096, 1),
                                  ("fp8", 65, 4096, 2048, 1), ("fp8", 64, 4096, 2048, 2)]:
            p = plan(dt, M, N, K)
            assert p["kernel"] == kern, (dt, M, N, K, ws, p)
            if kern == 2:
                assert p["grid"] == (N // p["tile_n"]) * -(-M // p["tile_m"])
    # W4A8 / MXFP4 past M*N*K = 2^31: split tiles given a workspace, the small-M kernel without one, or
    # where the tiles would leave fewer than 128 workgroups (no MXFP4 split tile below 128 rows)
    for dt, M, N, K in [("w4a8", 2048, 256, 7168), ("w4a8", 128, 4096, 16384), ("mxfp4", 128, 4096, 8192)]:
        assert gp.gemm_plan(dt, M, N, K)["kernel"] == 2
        p = gp.gemm_plan_ws(dt, M, N, K)
        assert p["kernel"] == 1 and p["ksplit"] > 1 and p["grid"] >= 128, (dt, M, N, K, p)
    assert gp.gemm_plan_ws("mxfp4", 96, 2048, 16384)["kernel"] == 2
    assert gp.gemm_plan("w4a8", 128, 1024, 7168, dict(xcd_swizzle=1))["kernel"] == 1   # an option set: the tile planner
    assert gp.gemm_plan("w4a8", 128, 1024, 7168, dict(kernel=2))["kernel"] == 2


# ---------------------------------------------------------------- K split across workgroups, scheduler option
@pytest.mark.parametrize("dtype,M,N,K,tile,ks", [
    ("fp8", 256, 2048, 16384, (64, 128, 256), 4), ("bf16", 512, 2048, 16384, (128, 256, 64), 8),
    ("w4a8", 256, 4096, 8192, (64, 128, 256), 2), ("fp8", 128, 4096, 8192, (64, 128, 256), 4),
    ("mxfp4", 256, 4096, 16384, (128, 128, 256), 4), ("bf16", 256, 1024, 8192, (64, 128, 64), 8)])
def test_automatic_k_split_on_long_k(dtype, M, N, K, tile, ks):
    """gemm_ex_ws splits K where the tiles alone cannot fill 256 CUs with a
    64 x 128 or larger tile; the entry points without a workspace never do."""
    p = gp.gemm_plan_ws(dtype, M, N, K)
    assert (p["tile_m"], p["tile_n"], p["tile_k"], p["ksplit"]) == (*tile, ks)
    assert p["grid"] == -(-M // tile[0]) * -(-N // tile[1]) * ks == 256
    T = -(-M // tile[0]) * -(-N // tile[1])
    assert p["workspace_bytes"] == gp.gemm_workspace_size(dtype, M, N, K) == \
        65536 + T * ks * tile[0] * tile[1] * 4
    q = gp.gemm_plan(dtype, M, N, K)
    assert q["ksplit"] == 1 and q["workspace_bytes"] == 0
    # the launch covers the same MFMAs as without a split
    assert p["mfma_total"] * 1 == (p["grid"] * p["waves"] * p["k_tiles"] * p["mfma_per_wave_tile"])


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_benchmark_workloads_are_not_split(name):
    """Short K (the workloads' K at most 8192 with grids of >= 256 tiles, or
    the small-M kernel): no split, no workspace."""
    dtype, M, N, K, seed, tile = CONFIGS[name]
    p = gp.gemm_plan_ws(dtype, M, N, K)
    assert p["ksplit"] == 1 and p["workspace_bytes"] == 0
    assert {k: v for k, v in p.items() if k not in ("ksplit", "scheduler", "workspace_bytes")} == \
        {k: v for k, v in gp.gemm_plan(dtype, M, N, K).items() if k not in ("ksplit", "scheduler", "workspace_bytes")}


def test_k_split_options():
    lib = gp.load_library()
    info = gp.GemmPlanInfo()
    o = gp.GemmOpts(kernel=1, tile_m=64, tile_n=128, tile_k=256, ksplit=2)
    # a split needs the workspace entry point
    assert lib.gemm_plan(1, 512, 4096, 4096, ctypes.byref(o), ctypes.byref(info)) == gp.GP_EWORKSPACE
    assert lib.gemm_plan_ws(1, 512, 4096, 4096, ctypes.byref(o), ctypes.byref(info)) == GP_OK
    assert info.ksplit == 2 and info.grid == 512 and info.k_tiles == 8
    # the split must divide the K tiles (16 here)
    o.ksplit = 3
    assert lib.gemm_plan_ws(1, 512, 4096, 4096, ctypes.byref(o), ctypes.byref(info)) == GP_ESHAPE
    # no split variant of this tile
    o2 = gp.GemmOpts(kernel=1, tile_m=32, tile_n=128, tile_k=128, ksplit=2)
    assert lib.gemm_plan_ws(1, 512, 4096, 4096, ctypes.byref(o2), ctypes.byref(info)) == GP_ESHAPE
    # small-M kernel: no split across workgroups
    o3 = gp.GemmOpts(kernel=2, ksplit=2)
    assert lib.gemm_plan_ws(1, 16, 7168, 2048, ctypes.byref(o3), ctypes.byref(info)) == GP_ESHAPE
    for bad in (-1, 65):
        o4 = gp.GemmOpts(ksplit=bad)
        assert lib.gemm_plan_ws(1, 512, 4096, 4096, ctypes.byref(o4), ctypes.byref(info)) == GP_EINVAL
    n = ctypes.c_size_t(7)
    assert lib.gemm_workspace_size(1, 512, 4096, 4096, None, ctypes.byref(n)) == GP_OK and n.value == 0
    assert lib.gemm_workspace_size(1, 512, 4096, 4096, None, None) == GP_EINVAL


def test_scheduler_option():
    # default tiles of the benchmark workloads have a scheduler-off variant
    for name in ("fp8_512x4096x4096", "bf16_8192x8192x8192", "mxfp4_4096x4096x8192", "fp16_8192x8192x8192",
                 "w4a8_512x4096x4096", "int8_128x256x512"):
        dtype, M, N, K, seed, tile = CONFIGS[name]
        assert gp.gemm_plan(dtype, M, N, K)["scheduler"] == 1
        assert gp.gemm_plan(dtype, M, N, K, dict(scheduler=2))["scheduler"] == 2
        assert gp.gemm_plan(dtype, M, N, K, dict(scheduler=1))["scheduler"] == 1
    with pytest.raises(gp.GemmError) as e:      # no scheduler-off variant of this tile
        gp.gemm_plan("fp8", 512, 4096, 4096, dict(kernel=1, tile_m=32, tile_n=128, tile_k=128, scheduler=2))
    assert e.value.status == GP_ESHAPE
    with pytest.raises(gp.GemmError) as e:      # the small-M kernel has no pinned schedule to turn off
        gp.gemm_plan("fp8", 16, 7168, 2048, dict(scheduler=2))
    assert e.value.status == GP_ESHAPE
    assert gp.gemm_plan("fp8", 16, 7168, 2048)["scheduler"] == 2
    with pytest.raises(gp.GemmError) as e:
        gp.gemm_plan("fp8", 512, 4096, 4096, dict(scheduler=3))
    assert e.value.status == GP_EINVAL


def test_workspace_validation(fake_ptrs):
    lib = fake_ptrs
    o = gp.GemmOpts(kernel=1, tile_m=64, tile_n=128, tile_k=256, ksplit=2)
    need = gp.gemm_workspace_size("fp8", 512, 4096, 4096, o)
    S = ctypes.c_void_p(0x200000)
    args = (1, 2, FAKE, FAKE, S, S, None, 0, FAKE, 512, 4096, 4096, ctypes.byref(o))
    assert lib.gemm_ex_ws(*args, None, need, None) == gp.GP_EWORKSPACE
    assert lib.gemm_ex_ws(*args, FAKE, need - 1, None) == gp.GP_EWORKSPACE
    assert lib.gemm_ex_ws(*args, MIS, need, None) == GP_EINVAL
    # a split with a fused epilogue passes the host checks (compiled; on a
    # host without a gfx950 GPU the call stops at the device check)
    args_b = (1, 2, FAKE, FAKE, S, S, FAKE, 1, FAKE, 512, 4096, 4096, ctypes.byref(o))
    assert lib.gemm_ex_ws(*args_b, FAKE, need, None) in (gp.GP_EHIP, 4)   # GP_EHIP or GP_EARCH
    # the scheduler-off variants have the plain epilogue only
    o2 = gp.GemmOpts(kernel=1, tile_m=64, tile_n=128, tile_k=256, pipeline=3, scheduler=2)
    args_c = (1, 2, FAKE, FAKE, S, S, FAKE, 1, FAKE, 512, 4096, 4096, ctypes.byref(o2))
    assert lib.gemm_ex_ws(*args_c, FAKE, need, None) == GP_ESHAPE


def test_split_tile_count_limit():
    """A split plan has at most 16384 tiles (the fixed counter area)."""
    ok = dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, ksplit=2)
    assert gp.gemm_plan_ws("fp8", 64 * 128, 128 * 128, 4096, ok)["ksplit"] == 2       # 16384 tiles
    with pytest.raises(gp.GemmError) as e:
        gp.gemm_plan_ws("fp8", 64 * 129, 128 * 128, 4096, ok)                         # 16512 tiles
    assert e.value.status == GP_ESHAPE


def test_planner_takes_large_edge_tiles_on_ragged_shapes():
    """A tile whose overlapping edge tiles add at most 1/8 to the computed
    area counts like one that divides M and N: BF16 8000 x 8192 x 8192 gets
    the 256 x 256 tile of the 8192^3 shape (2.4% of its rows computed twice),
    not the largest tile dividing 8000 (64 x 256); a tile that would compute
    far more than M x N still loses to a smaller one."""
    assert (gp.gemm_plan("bf16", 8192, 8192, 8192)["tile_m"], gp.gemm_plan("bf16", 8192, 8192, 8192)["tile_n"]) == (256, 256)
    for M, N, K in [(8000, 8192, 8192), (4000, 4096, 4096), (8192, 8000, 4096)]:
        p = gp.gemm_plan("bf16", M, N, K)
        assert (p["tile_m"], p["tile_n"], p["waves"]) == (256, 256, 8), (M, N, p)
    p = gp.gemm_plan("bf16", 300, 8192, 4096)      # 256-row tiles would compute 512 rows for 300
    assert p["tile_m"] <= 64 and p["grid"] >= 256
    p = gp.gemm_plan("mxfp4", 4000, 4096, 8192)
    assert (p["tile_m"], p["tile_n"]) == (128, 512)


def test_planner_splits_long_k_onto_larger_bf16_tiles():
    """With a workspace, BF16 / FP16 GEMMs whose grid of small tiles is full
    but whose K is long split K over a tile with fewer operand bytes per
    FLOP (each range keeping >= 4096 bytes of K); FP8 / INT8 do not."""
    p = gp.gemm_plan_ws("bf16", 512, 8192, 8192)
    assert (p["tile_m"], p["tile_n"], p["ksplit"], p["grid"]) == (128, 256, 2, 256)
    p = gp.gemm_plan_ws("bf16", 256, 8192, 8192)
    assert (p["tile_m"], p["tile_n"], p["ksplit"], p["grid"]) == (128, 256, 4, 256)
    assert gp.gemm_plan_ws("fp16", 512, 8192, 8192)["ksplit"] == 2
    for dt in ("fp8", "int8"):
        assert gp.gemm_plan_ws(dt, 512, 8192, 8192)["ksplit"] == 1
    assert gp.gemm_plan_ws("bf16", 512, 4096, 4096)["ksplit"] == 1     # 2048-byte ranges: no split
    assert gp.gemm_plan("bf16", 512, 8192, 8192)["ksplit"] == 1        # no workspace, no split


def test_planner_full_grid_and_fp8_order():
    """Three quarters of the CUs count as a full grid (7168 columns make 224
    tiles of 128 columns), and FP8 tiles are tried in the order of their
    operand bytes per FLOP."""
    def tile(dt, M, N, K):
        p = gp.gemm_plan_ws(dt, M, N, K)
        return p["tile_m"], p["tile_n"], p["grid"], p["ksplit"]
    assert tile("fp8", 256, 7168, 2048) == (64, 128, 224, 1)      # not 1792 tiles of 16 x 64
    assert tile("fp8", 128, 7168, 2048) == (32, 128, 224, 1)
    assert tile("fp8", 1024, 4096, 7168)[:2] == (128, 128)         # before 64 x 256
    assert tile("fp8", 512, 4096, 4096) == (64, 128, 256, 1)       # the benchmark shape: unchanged
    assert tile("fp8", 16, 7168, 2048)[:3] == (16, 32, 224)
    assert tile("bf16", 192, 8192, 8192) == (128, 256, 256, 4)     # 192 .. 255 tiles: BF16 larger-tile split
    assert tile("fp8", 256, 7168, 8192) == (64, 128, 224, 1)       # ... and no split for FP8
    # FP8: fewest operand bytes for the busiest CU, edge tiles up to a quarter more area
    for M in (80, 96, 112):
        assert tile("fp8", M, 7168, 2048)[:2] == (32, 128), M
    assert tile("fp8", 1536, 8192, 4096)[:2] == (128, 256)


def test_planner_splits_long_k_at_16_to_64_rows_over_16x64_tiles():
    """16 to 64 rows and long K, given a workspace: 16 x 64 tiles split along
    K into the largest power of two of ranges that keeps 2048 bytes of B's K
    per range and at most 256 workgroups (4 or more at 16 rows, 2 or more
    above), from 8192 bytes per B row for FP8 and 16384 for INT8, BF16, FP16
    and W4A8, where the busiest CU's bytes fall to 0.8 of the small-M plan's
    or less (FP8 from 16384 bytes: 0.95; W4A8: 0.5); not without a
    workspace, not for shorter K, not for other row counts, not for MXFP4."""
    p = gp.gemm_plan_ws("fp8", 16, 2048, 16384)
    assert (p["kernel"], p["tile_m"], p["tile_n"], p["tile_k"], p["ksplit"], p["grid"]) == (1, 16, 64, 512, 8, 256)
    assert gp.gemm_plan_ws("fp8", 16, 1024, 32768)["ksplit"] == 16
    assert gp.gemm_plan_ws("fp8", 16, 3072, 16384)["ksplit"] == 4
    assert gp.gemm_plan_ws("fp8", 16, 2048, 8192)["ksplit"] == 4
    assert gp.gemm_plan("fp8", 16, 2048, 16384)["kernel"] == 2            # no workspace
    assert gp.gemm_plan_ws("fp8", 16, 2048, 7168)["kernel"] == 2          # K too short
    assert gp.gemm_plan_ws("fp8", 16, 7168, 2048)["kernel"] == 2          # the M=16 workload is unchanged
    assert gp.gemm_plan_ws("fp8", 8, 2048, 16384)["kernel"] == 2
    # above 16 rows: ceil(M / 16) * ceil(N / 64) tiles, 2 or more ranges
    for M, N, K, S in ((32, 2048, 16384, 4), (64, 1024, 16384, 4), (64, 2048, 16384, 2),
                       (48, 1024, 32768, 4), (40, 2048, 16384, 2), (17, 2048, 16384, 4),
                       (64, 1024, 8192, 4)):
        q = gp.gemm_plan_ws("fp8", M, N, K)
        assert (q["kernel"], q["tile_m"], q["tile_n"], q["ksplit"]) == (1, 16, 64, S), (M, N, K, q)
        assert q["grid"] == -(-M // 16) * -(-N // 64) * S
    assert gp.gemm_plan_ws("fp8", 64, 4096, 16384)["kernel"] == 2         # 256 tiles: no room to split
    assert gp.gemm_plan_ws("fp8", 32, 2048, 7168)["kernel"] == 2          # K too short
    assert gp.gemm_plan_ws("fp8", 65, 2048, 16384)["tile_m"] != 16        # past 64 rows: the tile planner's own choice
    assert gp.gemm_plan("fp8", 64, 2048, 16384)["kernel"] == 2            # no workspace
    # the small-M plan takes two column blocks per workgroup (A read once per
    # 32 columns): the split's bytes are 0.9 of its, not enough below 16384
    # bytes of K for FP8, nor at all for INT8; W4A8 needs 0.5
    assert gp.gemm_plan_ws("fp8", 32, 4096, 8192)["kernel"] == 2
    assert gp.gemm_plan_ws("fp8", 64, 2048, 8192)["kernel"] == 2
    assert gp.gemm_plan_ws("int8", 64, 2048, 16384)["kernel"] == 2
    assert gp.gemm_plan_ws("int8", 64, 1024, 16384)["ksplit"] == 4
    assert gp.gemm_plan_ws("w4a8", 33, 1024, 32768)["kernel"] == 2
    assert gp.gemm_plan_ws("w4a8", 24, 1024, 32768)["ksplit"] == 8
    assert gp.gemm_plan_ws("bf16", 64, 1024, 16384)["ksplit"] == 4
    assert gp.gemm_plan_ws("bf16", 32, 2048, 4096)["kernel"] == 2
    q = gp.gemm_plan_ws("int8", 16, 2048, 16384)
    assert (q["kernel"], q["tile_m"], q["tile_n"], q["tile_k"], q["ksplit"]) == (1, 16, 64, 256, 8)
    assert gp.gemm_plan_ws("int8", 16, 2048, 8192)["kernel"] == 2         # 8192 bytes: INT8 keeps the small-M kernel
    for dt in ("bf16", "fp16"):
        q = gp.gemm_plan_ws(dt, 16, 2048, 8192)                             # 16384 bytes per row
        assert (q["kernel"], q["tile_k"], q["ksplit"]) == (1, 128, 8)
        assert gp.gemm_plan_ws(dt, 16, 2048, 4096)["kernel"] == 2
    q = gp.gemm_plan_ws("w4a8", 16, 1024, 32768)
    assert (q["kernel"], q["tile_k"], q["ksplit"]) == (1, 256, 8)
    assert gp.gemm_plan_ws("w4a8", 16, 2048, 16384)["kernel"] == 2
    assert gp.gemm_plan_ws("mxfp4", 16, 2048, 32768)["kernel"] == 2
