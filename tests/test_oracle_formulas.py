"""Pins for the planning / roofline formulas against the values the pages print
(tests/golden/pages_formulas.json, each entry with its page and section), plus
the gfx950 FLOP invariant (no GPU)."""
import json
import os

import pytest

from oracle import formulas as F
from workloads import CONFIGS

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_formulas.json")))


@pytest.mark.parametrize("e", GOLDEN["mfma_per_tile"])
def test_mfma_per_tile(e):
    assert F.mfma_per_tile_pages(*e["tile"], e["elem_bytes"]) == e["value"], e["cite"]


@pytest.mark.parametrize("e", GOLDEN["derived"])
def test_derived(e):
    d = F.derived(*e["tile"], e["elem_bytes"])
    for k in ("m_repeat", "num_acc_n", "k_unroll"):
        if k in e:
            assert d[k] == e[k], e["cite"]


def test_worked_example():
    w = GOLDEN["worked_example"]
    tm, tn, tk = w["tile"]
    assert F.grid(w["M"], w["N"], tm, tn) == w["grid"]
    assert w["K"] // tk == w["k_tiles"]
    assert F.mfma_total_pages(w["K"], tm, tn, tk, w["elem_bytes"]) == w["mfma_total_per_block"]
    assert F.lds_bytes(tm, tn, tk, w["elem_bytes"]) == w["lds_two_stage_bytes"]
    assert tm * tk * w["elem_bytes"] == w["lds_tile_bytes"]
    assert F.flops(w["M"], w["N"], w["K"]) == w["flops"]
    assert F.bytes_moved("fp8", w["M"], w["N"], w["K"]) == w["bytes_moved"]
    gbps = w["bytes_moved"] / (w["time_ms"] * 1e-3) / 1e9
    assert round(gbps) == w["bandwidth_GBps_rounded"]


@pytest.mark.parametrize("e", GOLDEN["lds_budget"])
def test_lds_budget(e):
    assert F.lds_bytes(e["tile_m"], 256, e["tile_k"], e["elem_bytes"]) == e["two_stage_bytes"], e["cite"]


def test_vgpr_estimate():
    e = GOLDEN["vgpr_estimate"]
    v = F.vgpr_estimate(*e["tile"], e["elem_bytes"], e["num_a_loads"])
    for k in ("accumulators", "b_tile", "a_prefetch", "a_tile"):
        assert v[k] == e[k], e["cite"]


@pytest.mark.parametrize("e", GOLDEN["occupancy"])
def test_occupancy(e):
    assert F.occupancy(e["vgprs"]) == e["waves"], e["cite"]


def test_occupancy_spill():
    assert F.occupancy(513) == 0


@pytest.mark.parametrize("name", sorted(CONFIGS))
@pytest.mark.parametrize("ms", [16, 32])
def test_gfx950_flop_invariant(name, ms):
    dtype, M, N, K, _, _ = CONFIGS[name]
    if M % ms or N % ms:
        pytest.skip("problem smaller than one MFMA block")
    assert F.mfma_count_gfx950(dtype, M, N, K, ms) * F.flops_per_mfma_gfx950(dtype, ms) == F.flops(M, N, K)


def test_config_bytes():
    # algorithmic bytes of the workloads (INT8 writes int32, the rest bf16)
    assert F.bytes_moved("int8", 128, 256, 512, out_bytes=4) == 327680
    assert F.bytes_moved("fp8", 16, 7168, 2048) == 14970944
    assert F.bytes_moved("fp8", 512, 4096, 4096) == 23087104
    assert F.bytes_moved("bf16", 8192, 8192, 8192) == 402653184
    assert F.bytes_moved("mxfp4", 4096, 4096, 8192) == 69206016
