"""Pins of the oracle's number formats and arithmetic against things other than itself:
torch's own float8 / bfloat16 / float16 conversions, exact rational arithmetic, closed forms."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import E2M1, E4M3, bf16_rne, e2m1_value, e4m3_value
from tests.st_files import f32_bytes, make_file


def _torch_bf16_bits(y_f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(y_f32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ E4M3 / E2M1 code tables

def test_e4m3_table_matches_torch_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(E4M3))
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan].view(np.uint32), E4M3[~nan].view(np.uint32))  # -0 included


@pytest.mark.parametrize("code,value", [(0x7E, 448.0), (0xFE, -448.0), (0x08, 2.0 ** -6), (0x01, 2.0 ** -9),
                                        (0x07, 7 * 2.0 ** -9), (0x38, 1.0), (0x39, 1.125), (0x00, 0.0)])
def test_e4m3_spot_values(code, value):
    assert e4m3_value(code) == value
    assert E4M3[code] == np.float32(value)


def test_e4m3_negative_zero():
    assert E4M3[0x80] == 0 and math.copysign(1.0, float(E4M3[0x80])) == -1.0


def test_e2m1_closed_form():
    pos = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [e2m1_value(c) for c in range(8)] == pos
    assert [e2m1_value(c) for c in range(8, 16)] == [-v for v in pos]
    assert math.copysign(1.0, e2m1_value(8)) == -1.0
    assert np.array_equal(E2M1, np.array(pos + [-v for v in pos], np.float32))


def test_e2m1_matches_mx_definition_via_e4m3_embedding():
    # An e2m1 value with exponent bits ee and mantissa bit m equals the e4m3 value whose
    # exponent is ee re-biased from 1 to 7 and whose top mantissa bit is m (subnormals included
    # only for the zero code).  Cross-checks the e2m1 table through torch's e4m3 decoding.
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for c in range(16):
        s, E, m = c >> 3, (c >> 1) & 3, c & 1
        if E == 0 and m == 1:
            expect = 0.5
        elif E == 0:
            expect = 0.0
        else:
            expect = float(ref[((E - 1 + 7) << 3) | (m << 2)])
        assert abs(e2m1_value(c)) == expect


# ------------------------------------------------------------------ bf16 rounding

def _rounding_classes():
    hi = np.arange(65536, dtype=np.uint64) << np.uint64(16)
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x4000, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xC000, 0xFFFE, 0xFFFF],
                    dtype=np.uint64)
    return (hi[:, None] | lows[None, :]).reshape(-1).astype(np.uint32)


def test_bf16_rne_matches_torch_every_rounding_class():
    # Every upper half (all 65,536 bf16 patterns) combined with low halves covering each
    # (lsb, round bit, sticky) class: below half, exactly half, above half, both lsb parities.
    u = _rounding_classes()
    y = u.view(np.float32)
    ours = bf16_rne(y)
    nan = np.isnan(y)
    assert np.array_equal(ours[~nan], _torch_bf16_bits(y)[~nan])
    assert np.all(ours[nan] == 0x7FC0)


def test_bf16_rne_matches_torch_random_patterns():
    rng = np.random.default_rng(1234)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    y = u.view(np.float32)
    ours = bf16_rne(y)
    nan = np.isnan(y)
    assert np.array_equal(ours[~nan], _torch_bf16_bits(y)[~nan])
    assert np.all(ours[nan] == 0x7FC0)


def test_bf16_rne_ties_and_limits():
    v = lambda bits: np.array([bits], np.uint32).view(np.float32)
    assert bf16_rne(v(0x3F808000))[0] == 0x3F80      # 1 + 2^-8: tie, lsb 0 stays
    assert bf16_rne(v(0x3F818000))[0] == 0x3F82      # 1 + 3*2^-8: tie, lsb 1 rounds up
    assert bf16_rne(v(0x7F7FFFFF))[0] == 0x7F80      # FLT_MAX rounds to +inf
    assert bf16_rne(v(0xFF7FFFFF))[0] == 0xFF80
    assert bf16_rne(v(0x7F800000))[0] == 0x7F80
    assert bf16_rne(v(0x00000001))[0] == 0x0000      # smallest subnormal: below half
    assert bf16_rne(v(0x00008001))[0] == 0x0001      # subnormal above half rounds up
    assert bf16_rne(v(0x80000000))[0] == 0x8000
    assert bf16_rne(v(0xFFC00001))[0] == 0x7FC0      # any NaN is canonical


def test_f16_widening_exhaustive_matches_torch():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    ours = bf16_rne(h.astype(np.float32))
    ref = torch.from_numpy(h.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(h)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(ours[nan] == 0x7FC0)


# ------------------------------------------------------------------ witnesses (exact arithmetic)

def _fraction_to_bf16_single_rounding(x: Fraction) -> int:
    """Round a positive normal rational once to bf16 (8 significant bits), ties to even."""
    e = math.floor(math.log2(x))
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    ulp = Fraction(2) ** (e - 7)
    q, r = divmod(x, ulp)
    q = int(q)
    if r > ulp / 2 or (r == ulp / 2 and q % 2 == 1):
        q += 1
    val = q * ulp
    return int(np.float32(float(val)).view(np.uint32) >> 16)


def _fp8_tensor_file(codes: np.ndarray, scale_bits: int):
    s = np.array([scale_bits], np.uint32).view(np.float32)
    return make_file([("w.weight", "F8_E4M3", (len(codes),), codes.astype(np.uint8)),
                      ("w.scale_weight", "F32", (), s.tobytes())])


def test_witness_double_rounding_w1():
    # e4m3 0x39 (1.125) times the fp32 scale 0x3F6471C8: the fp32 product is exactly
    # 1.00390625 (a bf16 tie that stays at 0x3F80); rounding the exact product once would give
    # 0x3F81.  The definition is the two-step one.
    s = Fraction(float(np.array([0x3F6471C8], np.uint32).view(np.float32)[0]))
    assert s == Fraction(14971336, 2 ** 24)
    exact = Fraction(9, 8) * s
    assert _fraction_to_bf16_single_rounding(exact) == 0x3F81
    assert np.float32(float(exact)) == np.float32(1.00390625)
    out = oracle.materialize(_fp8_tensor_file(np.array([0x39]), 0x3F6471C8))
    assert out["w.weight"][0] == 0x3F80


def test_witness_multiply_order_w2():
    # e2m1 code 0x7 (6.0), block scale e4m3 0x77 (240), global 0x3B2D27D2: left to right gives
    # 0x4073, folding block*global first would give 0x4074.
    g = np.array([0x3B2D27D2], np.uint32).view(np.float32)[0]
    ltr = bf16_rne(np.array([np.float32(np.float32(6.0) * np.float32(240.0)) * g], np.float32))[0]
    folded = bf16_rne(np.array([np.float32(6.0) * np.float32(np.float32(240.0) * g)], np.float32))[0]
    assert (ltr, folded) == (0x4073, 0x4074)
    f = make_file([("x.weight", "U8", (1, 8), np.array([0x77] * 8, np.uint8)),  # code 7 in both nibbles
                   ("x.weight_scale", "F8_E4M3", (1, 1), np.array([0x77], np.uint8)),
                   ("x.weight_scale_2", "F32", (), np.array([0x3B2D27D2], np.uint32).tobytes())])
    out = oracle.materialize(f)["x.weight"]
    assert out.shape == (1, 16) and np.all(out == 0x4073)


# ------------------------------------------------------------------ brute force vs float64

def _two_step_ref(*factors):
    """Each fp32 multiply done exactly in float64 (<= 53 significant bits here), rounded to
    fp32 by numpy's RNE cast, then bf16 via torch's cast (NaN handled by the caller)."""
    acc = np.float32(factors[0])
    for f in factors[1:]:
        acc = (np.asarray(acc, np.float64) * np.asarray(f, np.float64)).astype(np.float32)
    return acc


SCALES = [0x3F6471C8, 0x3B2D27D2, 0x3C23D70A, 0x3A83126F, 0x3F800000, 0x00000001, 0x00400000, 0x7F7FFFFF,
          0x4B800000, 0x33D6BF95]


@pytest.mark.parametrize("scale_bits", SCALES)
def test_fp8_tensor_all_codes_brute_force(scale_bits):
    codes = np.arange(256, dtype=np.uint8)
    out = oracle.materialize(_fp8_tensor_file(codes, scale_bits))["w.weight"]
    s = np.array([scale_bits], np.uint32).view(np.float32)[0]
    ref_vals = np.array([e4m3_value(int(c)) for c in codes])
    with np.errstate(invalid="ignore", over="ignore"):
        y = _two_step_ref(ref_vals, np.full(256, s))
    nan = np.isnan(y)
    assert np.array_equal(out[~nan], _torch_bf16_bits(y)[~nan])
    assert np.all(out[nan] == 0x7FC0) and set(np.nonzero(nan)[0]) == {0x7F, 0xFF}


@pytest.mark.parametrize("g_bits", [0x3B2D27D2, 0x3F800000, 0x3DCCCCCD, 0x3A83126F, 0x7F000000])
def test_nvfp4_all_nibbles_all_block_scales_brute_force(g_bits):
    # Every e2m1 code against every positive finite e4m3 block scale (126 codes), one row per
    # block scale; row r uses scale code sc[r] and its 16 elements run through all 16 codes.
    sc = np.array([c for c in range(1, 127)], np.uint8)
    rows = len(sc)
    nib = np.tile(np.arange(16, dtype=np.uint8), rows)          # element j -> code j % 16
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    f = make_file([("q.weight", "U8", (rows, 8), packed),
                   ("q.weight_scale", "F8_E4M3", (rows, 1), sc),
                   ("q.weight_scale_2", "F32", (), np.array([g_bits], np.uint32).tobytes())])
    out = oracle.materialize(f)["q.weight"]
    g = np.array([g_bits], np.uint32).view(np.float32)[0]
    e2 = np.array([e2m1_value(c) for c in range(16)])
    bs = np.array([e4m3_value(int(c)) for c in sc])
    with np.errstate(over="ignore"):
        y = _two_step_ref(np.tile(e2, rows), np.repeat(bs, 16), np.full(rows * 16, g))
    assert np.array_equal(out.reshape(-1), _torch_bf16_bits(y))


# ------------------------------------------------------------------ closed forms

@pytest.mark.parametrize("k", [-20, -7, 0, 3, 9])
def test_power_of_two_scale_requantises_exactly(k):
    # With s = 2^k every output is decode(code) * 2^k exactly (e4m3 has 4 significant bits,
    # bf16 has 8), so re-encoding out / 2^k with torch's e4m3 cast returns the code.
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    bits = int(np.array([2.0 ** k], np.float32).view(np.uint32)[0])
    out = oracle.materialize(_fp8_tensor_file(codes, bits))["w.weight"]
    vals = torch.from_numpy(out.view(np.int16).copy()).view(torch.bfloat16).float() / (2.0 ** k)
    back = vals.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(back, codes)


def test_nvfp4_requantises_with_unit_scales():
    # bs = 1.0 (0x38), g = 1.0: outputs are the e2m1 values themselves; re-encode by table search.
    nib = np.tile(np.arange(16, dtype=np.uint8), 4)
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    f = make_file([("q.weight", "U8", (4, 8), packed), ("q.weight_scale", "F8_E4M3", (4, 1), np.full(4, 0x38, np.uint8)),
                   ("q.weight_scale_2", "F32", (), f32_bytes(1.0))])
    out = oracle.materialize(f)["q.weight"].reshape(-1)
    vals = torch.from_numpy(out.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    pos = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    back = [pos.index(abs(v)) | (8 if math.copysign(1, v) < 0 else 0) for v in vals]
    assert back == nib.tolist()


def test_block_fp8_index_mapping_with_distinct_power_of_two_scales():
    # 300 x 200 (ragged 128-blocks) of the value 1.0 (code 0x38); block (bi, bj) carries
    # 2^(bi*G + bj - 4).  Each output's exponent must name the block of its (row, col).
    M, N = 300, 200
    gm, gn = 3, 2
    S = np.array([[2.0 ** (bi * gn + bj - 4) for bj in range(gn)] for bi in range(gm)], np.float32)
    f = make_file([("b.weight", "F8_E4M3", (M, N), np.full(M * N, 0x38, np.uint8)),
                   ("b.weight_scale_inv", "F32", (gm, gn), S)])
    out = oracle.materialize(f)["b.weight"]
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    expect_exp = (rows // 128) * gn + cols // 128 - 4
    got_exp = ((out.astype(np.int64) >> 7) & 0xFF) - 127
    assert np.array_equal(got_exp, expect_exp)
    assert np.all((out & 0x7F) == 0) and np.all(out >> 15 == 0)


def test_nvfp4_index_mapping_position_coded():
    # M x K = 5 x 48 with K % 32 == 16.  Nibble at (i, j) = code 2 (1.0) everywhere except the
    # sign, which encodes j's parity (negative on odd j: tests the nibble order); block scale
    # (i, j/16) = 2^(i*3 + j/16 - 6) (distinct powers of two, e4m3 normals).
    M, K = 5, 48
    nib = np.where((np.arange(M * K) % K) % 2 == 1, 0xA, 0x2).astype(np.uint8)   # 0xA = -1.0
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    ex = np.array([[i * 3 + b - 6 for b in range(K // 16)] for i in range(M)])
    bs = torch.from_numpy(np.exp2(ex).astype(np.float32).reshape(-1)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    f = make_file([("n.weight", "U8", (M, K // 2), packed), ("n.weight_scale", "F8_E4M3", (M, K // 16), bs),
                   ("n.weight_scale_2", "F32", (), f32_bytes(1.0))])
    out = oracle.materialize(f)["n.weight"]
    i, j = np.meshgrid(np.arange(M), np.arange(K), indexing="ij")
    assert np.array_equal(((out.astype(np.int64) >> 7) & 0xFF) - 127, i * 3 + j // 16 - 6)
    assert np.array_equal(out >> 15, (j % 2).astype(np.uint16))


def test_passthrough_is_identity_and_casts_follow_torch():
    rng = np.random.default_rng(7)
    bf = rng.integers(0, 65536, size=999, dtype=np.uint64).astype(np.uint16)
    h = rng.standard_normal(501).astype(np.float16)
    x = (rng.standard_normal(333) * 1e-39).astype(np.float32)   # fp32 subnormals round normally
    f = make_file([("a", "BF16", (999,), bf), ("b", "F16", (501,), h), ("c", "F32", (333,), x)])
    out = oracle.materialize(f)
    assert np.array_equal(out["a"], bf)
    assert np.array_equal(out["b"], torch.from_numpy(h).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(out["c"], _torch_bf16_bits(x))


def test_sampled_decode_equals_full_decode():
    import synth
    buf = synth.config_bytes(3, small=True)
    h, outs = oracle.plan(buf)
    data = np.frombuffer(buf, np.uint8, offset=h.data_offset)
    rng = np.random.default_rng(3)
    for o in outs:
        full = oracle.decode(o, data).reshape(-1)
        if o.numel == 0:
            continue
        idx = rng.integers(0, o.numel, size=64)
        assert np.array_equal(oracle.decode(o, data, idx), full[idx])
