"""Pins of the oracle's fp16 and fp32 output variants, against what IEEE-754 fixes: fp16
round-to-nearest-even at ties, the overflow threshold and the subnormal range, written out from
the format's definition; fp32 outputs equal the binary32 products; canonical NaNs; and the
definition's consistency across output types (a value exactly representable in fp16 and bf16
gives the same number in all three)."""
import numpy as np
import pytest

import oracle
import synth
from tests.st_files import f32_bytes, make_file


def _h(bits):
    return np.array([bits], dtype=np.uint16)


def _f(x):
    return np.array([x], dtype=np.float32)


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3C00), (-2.0, 0xC000), (65504.0, 0x7BFF),
    (1 + 2 ** -11, 0x3C00),                 # a tie between 1 and 1 + 2^-10: to even (1)
    (1 + 3 * 2 ** -11, 0x3C02),             # a tie between 1 + 2^-10 and 1 + 2^-9: to even
    (1 + 2 ** -11 + 2 ** -20, 0x3C01),      # just above the tie
    (65519.0, 0x7BFF), (65520.0, 0x7C00),   # 65520 is the tie between 65504 and 2^16: inf
    (-1e9, 0xFC00),
    (2.0 ** -14, 0x0400), (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000),      # 2^-25 ties to 0
    (3 * 2.0 ** -26, 0x0001), (2.0 ** -25 + 2.0 ** -40, 0x0001), (-(2.0 ** -24), 0x8001),
    (1.5 * 2.0 ** -24, 0x0002),             # tie between 1 and 2 subnormal units: to even (2)
    (0.0, 0x0000), (-0.0, 0x8000), (float("inf"), 0x7C00), (-float("inf"), 0xFC00),
])
def test_f16_rounding_cases(x, bits):
    assert oracle.f16_rne(_f(x))[0] == bits


def test_f16_nan_is_canonical():
    for u in (0x7F800001, 0xFFC00000, 0x7FFFFFFF):
        assert oracle.f16_rne(np.array([u], np.uint32).view(np.float32))[0] == 0x7E00
    assert oracle.f32_bits(np.array([0xFF812345], np.uint32).view(np.float32))[0] == 0x7FC00000


def test_f16_brute_force_against_the_definition():
    """Every fp16 value and every midpoint between neighbours (in fp32): values map to
    themselves; midpoints go to the neighbour with an even significand."""
    codes = np.arange(0x7C00, dtype=np.uint32)                     # finite non-negative fp16
    vals = codes.astype(np.uint16).view(np.float16).astype(np.float32)
    assert np.array_equal(oracle.f16_rne(vals), codes.astype(np.uint16))
    lo, hi = vals[:-1].astype(np.float64), vals[1:].astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)                        # exact in fp32
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    want = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:]).astype(np.uint16)
    assert np.array_equal(oracle.f16_rne(mid), want)


def test_outputs_agree_across_types_for_representable_values():
    # e4m3 codes times 1.0: every e4m3 value is exact in bf16, fp16 and fp32
    buf = make_file([("w.weight", "F8_E4M3", (256,), np.arange(256, dtype=np.uint8)),
                     ("w.scale_weight", "F32", (), f32_bytes(1.0))])
    b = oracle.materialize(buf, "bf16")["w.weight"]
    h = oracle.materialize(buf, "f16")["w.weight"]
    f = oracle.materialize(buf, "f32")["w.weight"]
    assert f.dtype == np.uint32 and h.dtype == np.uint16
    ok = (np.arange(256) & 0x7F) != 0x7F
    vb = (b.astype(np.uint32) << 16).view(np.float32)
    vh = h.view(np.float16).astype(np.float32)
    vf = f.view(np.float32)
    assert np.array_equal(vb[ok], vf[ok]) and np.array_equal(vh[ok], vf[ok])
    assert np.all(h[~ok] == 0x7E00) and np.all(f[~ok] == 0x7FC00000) and np.all(b[~ok] == 0x7FC0)


def test_f32_output_is_the_binary32_product():
    buf = synth.config_bytes(3, small=True)
    h, outs = oracle.plan(buf)
    data = np.frombuffer(buf, np.uint8, offset=h.data_offset)
    o = next(o for o in outs if o.kind == "FP8_BLOCK128")
    idx = np.arange(o.numel)
    m, n = o.shape
    w = data[o.src.begin: o.src.begin + o.numel]
    gn = -(-n // 128)
    S = np.frombuffer(buf, "<f4", count=-(-m // 128) * gn, offset=h.data_offset + o.scale.begin).reshape(-1, gn)
    want = (oracle.E4M3[w] * S[(idx // n) // 128, (idx % n) // 128]).astype(np.float32)
    assert np.array_equal(oracle.decode(o, data, out_dtype="f32").reshape(-1), want.view(np.uint32))
    # and the fp16 output is that product rounded once more
    assert np.array_equal(oracle.decode(o, data, out_dtype="f16").reshape(-1), oracle.f16_rne(want))


def test_bf16_passthrough_only_keeps_bits_for_bf16():
    raw = np.array([0x3F80, 0x7F81, 0xFF80, 0x0001], dtype=np.uint16)   # 1, a signalling NaN, -inf, subnormal
    buf = make_file([("b", "BF16", (4,), raw)])
    assert np.array_equal(oracle.materialize(buf, "bf16")["b"], raw)
    assert np.array_equal(oracle.materialize(buf, "f32")["b"], np.array([0x3F800000, 0x7FC00000, 0xFF800000, 0x00010000],
                                                                         dtype=np.uint32))
    assert np.array_equal(oracle.materialize(buf, "f16")["b"], np.array([0x3C00, 0x7E00, 0xFC00, 0x0000], dtype=np.uint16))


def test_f16_equals_torch_cast_on_random_and_boundary_patterns():
    """An independent implementation: torch's fp32 -> fp16 cast (round to nearest even) on 2M
    random fp32 patterns and on every pattern within 64 ulps of the fp16 overflow threshold and of
    every power of two from 2^-26 to 2^-13 (the subnormal range and its edges)."""
    import torch
    rng = np.random.default_rng(11)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    edges = [np.float32(65520.0).view(np.uint32)] + [np.float32(2.0 ** e).view(np.uint32) for e in range(-26, -12)]
    near = np.concatenate([np.arange(int(b) - 64, int(b) + 65, dtype=np.int64) for b in edges]).astype(np.uint32)
    u = np.concatenate([u, near, near | np.uint32(0x80000000)])
    x = u.view(np.float32)
    finite = np.isfinite(x) | np.isinf(x)
    want = torch.from_numpy(x[finite].copy()).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f16_rne(x[finite]), want)
