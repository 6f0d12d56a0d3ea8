"""Planted mistakes in the oracle, for the mutation check of its pins.

A pytest plugin: with ORACLE_MUTANT=<name> in the environment it replaces
one oracle function by a plausible wrong version (a dropped term, a wrong
sign, index or constant, a transposed operand) before any test module is
imported, in every oracle module that binds the name. Used only by
tests/test_oracle_mutants.py, which runs the oracle's pins in a child
process per mutant and expects at least one of them to fail. Nothing here
runs on a GPU.
"""
from __future__ import annotations

import os

import numpy as np


def _mutants():
    import importlib

    import oracle

    # the submodules (the package's `gemm` attribute is the dispatch function)
    f, g, c, lay, fo = (importlib.import_module("oracle." + m)
                        for m in ("formats", "gemm", "compare", "layout", "formulas"))

    def fp8_drop_scale_a(a, b, scale_a, scale_b, rows=None, cols=None):
        A = f.decode_e4m3(g._take(a, rows))
        B = f.decode_e4m3(g._take(b, cols))
        sb = np.asarray(g._take(scale_b, cols), dtype=np.float32).astype(np.float64)
        return (A @ B.T) * sb[None, :]

    def fp8_reversed_k_of_b(a, b, scale_a, scale_b, rows=None, cols=None):
        A = f.decode_e4m3(g._take(a, rows))
        B = f.decode_e4m3(g._take(b, cols))[:, ::-1]
        sa = np.asarray(g._take(scale_a, rows), dtype=np.float32).astype(np.float64)
        sb = np.asarray(g._take(scale_b, cols), dtype=np.float32).astype(np.float64)
        return (A @ B.T) * sa[:, None] * sb[None, :]

    orig_e4m3 = f.decode_e4m3

    def e4m3_bias8(codes):
        cc = np.asarray(codes).astype(np.int64)
        e = (cc >> 3) & 0xF
        v = orig_e4m3(codes)
        return np.where(e == 0, v, v * 0.5)

    def e4m3_subnormal_as_normal(codes):
        cc = np.asarray(codes).astype(np.int64)
        e = (cc >> 3) & 0xF
        m = (cc & 7).astype(np.float64)
        sign = np.where(cc & 0x80, -1.0, 1.0)
        return np.where(e == 0, sign * (1.0 + m / 8.0) * 2.0 ** -7, orig_e4m3(codes))

    orig_e2m1 = f.decode_e2m1

    def e2m1_swapped_codes(codes):
        cc = np.asarray(codes).astype(np.int64)
        swap = np.where((cc & 7) == 3, (cc & 8) | 4, np.where((cc & 7) == 4, (cc & 8) | 3, cc))
        return orig_e2m1(swap)

    def e8m0_off_by_one(codes):
        cc = np.asarray(codes).astype(np.int64)
        return np.where(cc == 255, np.nan, np.exp2(cc.astype(np.float64) - 126.0))

    def bf16_wrong_shift(bits):
        b = np.asarray(bits).astype(np.uint32) << np.uint32(15)
        return b.view(np.float32).astype(np.float64)

    def int4_unsigned(codes):
        return np.asarray(codes).astype(np.int64) & 0xF

    def nibbles_high_first(packed):
        p = np.asarray(packed).astype(np.uint8)
        out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
        out[..., 0::2] = p >> 4
        out[..., 1::2] = p & 0xF
        return out

    def preshuffle_index_swapped(n, kb, Kb):
        n0, j = divmod(n, 16)
        k0, r = divmod(kb, 64)
        gg, b = divmod(r, 16)
        return (((n0 * (Kb // 64) + k0) * 16 + j) * 4 + gg) * 16 + b

    def preshuffle_swapped(b):
        bb = np.ascontiguousarray(b).view(np.uint8)
        N, Kb = bb.shape
        t = bb.reshape(N // 16, 16, Kb // 64, 4, 16)
        return np.ascontiguousarray(t.transpose(0, 2, 1, 3, 4)).reshape(-1)

    orig_act = g.activation

    def gelu_tanh(x, act):
        if act == "gelu":
            x = np.asarray(x, dtype=np.float64)
            return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))
        return orig_act(x, act)

    def silu_sign(x, act):
        if act == "silu":
            x = np.asarray(x, dtype=np.float64)
            with np.errstate(over="ignore"):
                return x / (1.0 + np.exp(x))
        return orig_act(x, act)

    def bias_after_activation(r, bias=None, act="none", cols=None):
        out = orig_act(np.asarray(r, dtype=np.float64), act)
        if bias is not None:
            out = out + np.asarray(g._take(bias, cols), dtype=np.float32).astype(np.float64)[None, :]
        return out

    def mx_scales_shifted(packed, scale):
        vals = f.decode_e2m1(f.unpack_fp4(packed))
        s = np.roll(f.decode_e8m0(scale), 1, axis=1)
        return vals * np.repeat(s, 32, axis=1)

    def w4a8_drop_scale_b(a, b, scale_a, scale_b, rows=None, cols=None):
        A = f.decode_int8(g._take(a, rows))
        B = f.decode_int4(f.unpack_nibbles(g._take(b, cols)))
        sa = np.asarray(g._take(scale_a, rows), dtype=np.float32).astype(np.float64)
        return (A @ B.T).astype(np.float64) * sa[:, None]

    def int8_as_unsigned(x):
        return np.asarray(x).astype(np.uint8).astype(np.int64)

    def bf16_rne_truncate(x):
        x = np.asarray(x, dtype=np.float64)
        m, e = np.frexp(x)
        return np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)

    def f16_rne_10_bits(x):
        x = np.asarray(x, dtype=np.float64)
        m, e = np.frexp(x)
        return np.ldexp(np.round(np.ldexp(m, 10)), e - 10)

    orig_dispatch = g._gemm

    def mxfp4_dispatch_swapped_scales(dtype, inputs, rows, cols):
        if dtype == "mxfp4":
            return g.gemm_mxfp4(inputs["a"], inputs["scale_b"], inputs["b"], inputs["scale_a"], rows, cols)
        return orig_dispatch(dtype, inputs, rows, cols)

    orig_bytes = fo.bytes_moved

    def bytes_without_scales(dtype, M, N, K, out_bytes=2):
        extra = {"fp8": (M + N) * 4, "w4a8": (M + N) * 4, "int4": (M + N) * 4, "mxfp4": (M + N) * (K // 32)}
        return orig_bytes(dtype, M, N, K, out_bytes) - extra.get(dtype, 0)

    def mfma_count_k_doubled(dtype, M, N, K, ms=16):
        return (M // ms) * (N // ms) * (K // (2 * fo._k_instr(dtype, ms)))

    def flops_single(M, N, K):
        return M * N * K

    orig_cv = c.compare_values

    def compare_ignores_elementwise(cc, ref):
        out = orig_cv(cc, ref)
        out["ok"] = bool(out["normwise"] <= c.NORMWISE_TOL and out["nonfinite"] == 0)
        return out

    return {
        "fp8_drop_scale_a": [("gemm_fp8", fp8_drop_scale_a)],
        "fp8_reversed_k_of_b": [("gemm_fp8", fp8_reversed_k_of_b)],
        "e4m3_bias8": [("decode_e4m3", e4m3_bias8)],
        "e4m3_subnormal_as_normal": [("decode_e4m3", e4m3_subnormal_as_normal)],
        "e2m1_swapped_codes": [("decode_e2m1", e2m1_swapped_codes)],
        "e8m0_off_by_one": [("decode_e8m0", e8m0_off_by_one)],
        "bf16_wrong_shift": [("decode_bf16", bf16_wrong_shift)],
        "int4_unsigned": [("decode_int4", int4_unsigned)],
        "nibbles_high_first": [("unpack_nibbles", nibbles_high_first), ("unpack_fp4", nibbles_high_first)],
        "preshuffle_swapped": [("preshuffle_index", preshuffle_index_swapped), ("preshuffle", preshuffle_swapped)],
        "gelu_tanh": [("activation", gelu_tanh)],
        "silu_sign": [("activation", silu_sign)],
        "bias_after_activation": [("apply_epilogue", bias_after_activation)],
        "mx_scales_shifted": [("_dec_mx", mx_scales_shifted)],
        "w4a8_drop_scale_b": [("gemm_w4a8", w4a8_drop_scale_b)],
        "int8_as_unsigned": [("decode_int8", int8_as_unsigned)],
        "bf16_rne_truncate": [("bf16_rne", bf16_rne_truncate)],
        "compare_ignores_elementwise": [("compare_values", compare_ignores_elementwise)],
        "bytes_without_scales": [("bytes_moved", bytes_without_scales)],
        "mfma_count_k_doubled": [("mfma_count_gfx950", mfma_count_k_doubled)],
        "flops_single": [("flops", flops_single)],
        "f16_rne_10_bits": [("f16_rne", f16_rne_10_bits)],
        "mxfp4_dispatch_swapped_scales": [("_gemm", mxfp4_dispatch_swapped_scales)],
    }, (oracle, f, g, c, lay, fo)


NAMES = (
    "fp8_drop_scale_a", "fp8_reversed_k_of_b", "e4m3_bias8", "e4m3_subnormal_as_normal", "e2m1_swapped_codes",
    "e8m0_off_by_one", "bf16_wrong_shift", "int4_unsigned", "nibbles_high_first", "preshuffle_swapped",
    "gelu_tanh", "silu_sign", "bias_after_activation", "mx_scales_shifted", "w4a8_drop_scale_b",
    "int8_as_unsigned", "bf16_rne_truncate", "compare_ignores_elementwise", "bytes_without_scales",
    "mfma_count_k_doubled", "flops_single", "f16_rne_10_bits", "mxfp4_dispatch_swapped_scales",
)


def pytest_configure(config):
    name = os.environ.get("ORACLE_MUTANT")
    if not name:
        return
    table, modules = _mutants()
    patches = table[name]
    for attr, fn in patches:
        hit = False
        for mod in modules:
            if hasattr(mod, attr):
                setattr(mod, attr, fn)
                hit = True
        assert hit, attr
