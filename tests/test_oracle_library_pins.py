"""Pins of the oracle's block-scaled float8 decodes against an independent implementation: the
transformers library's block dequantiser (written for checkpoints that store e4m3 weights with a
``weight_scale_inv`` grid, and for E8M0 bytes per 32 elements).  It multiplies in fp32 and casts
once to the output type, as the oracle does, so the bits must agree.  Its inputs are the file's
own tensors; it needs shapes that are whole multiples of the scale grid."""
import numpy as np
import pytest
import torch

import oracle
from tests.st_files import make_file

transformers_fp8 = pytest.importorskip("transformers.integrations.finegrained_fp8")


def _dequantize(q, scales, out):
    return transformers_fp8.Fp8Dequantize(None)._dequantize_one(q, scales, out)


def _codes(rng, n):
    """e4m3 codes without the two NaN codes (the library would keep NaN payloads)."""
    c = rng.integers(0, 254, n, dtype=np.uint64).astype(np.uint8)
    return np.where(c >= 0x7F, c + 1, c).astype(np.uint8)


@pytest.mark.parametrize("m,n", [(128, 128), (256, 384), (384, 128)])
def test_block_fp8_equals_the_library_dequantiser(m, n):
    rng = np.random.default_rng(m + n)
    w = _codes(rng, m * n)
    S = np.power(10.0, rng.uniform(-4, -2, (m // 128) * (n // 128))).astype(np.float32)
    buf = make_file([("w.weight", "F8_E4M3", (m, n), w), ("w.weight_scale_inv", "F32", (m // 128, n // 128), S)])
    q = torch.from_numpy(w.copy()).view(torch.float8_e4m3fn).view(m, n)
    s = torch.from_numpy(S.copy()).view(m // 128, n // 128)
    for out_dtype, tdt, idt in (("bf16", torch.bfloat16, torch.int16), ("f32", torch.float32, torch.int32),
                                ("f16", torch.float16, torch.int16)):
        got = oracle.materialize(buf, out_dtype)["w.weight"]
        ref = _dequantize(q, s, tdt).contiguous().view(idt).numpy().view(got.dtype)
        assert np.array_equal(got, ref), out_dtype


def test_mxfp8_equals_the_library_dequantiser():
    rng = np.random.default_rng(5)
    m, k = 64, 256
    w = _codes(rng, m * k)
    e = rng.integers(90, 160, m * (k // 32), dtype=np.uint64).astype(np.uint8)
    buf = make_file([("w.weight", "F8_E4M3", (m, k), w), ("w.weight_scale", "F8_E8M0", (m, k // 32), e)])
    q = torch.from_numpy(w.copy()).view(torch.float8_e4m3fn).view(m, k)
    s = torch.from_numpy(e.copy()).view(m, k // 32)          # uint8 exponents: 2^(e - 127)
    for out_dtype, tdt, idt in (("bf16", torch.bfloat16, torch.int16), ("f32", torch.float32, torch.int32)):
        got = oracle.materialize(buf, out_dtype)["w.weight"]
        ref = _dequantize(q, s, tdt).contiguous().view(idt).numpy().view(got.dtype)
        assert np.array_equal(got, ref), out_dtype


def test_nvfp4_with_unit_global_scale_equals_the_library_dequantiser():
    """The library also dequantises packed e2m1 weights (int8 storage, two nibbles per byte) against
    a scale grid; with e4m3 block scales over [M, K/16] it computes NVFP4's first product.  With a
    global scale of 1.0 the oracle's NVFP4 output must equal it: this pins the [M, K/16] block-scale
    layout and the e4m3 scale decode of the NVFP4 branch against an independent implementation."""
    rng = np.random.default_rng(21)
    m, k = 32, 128
    packed = rng.integers(0, 256, m * k // 2, dtype=np.uint64).astype(np.uint8)
    bs = _codes(rng, m * k // 16)
    buf = make_file([("w.weight", "U8", (m, k // 2), packed), ("w.weight_scale", "F8_E4M3", (m, k // 16), bs),
                     ("w.weight_scale_2", "F32", (), np.array([1.0], np.float32).tobytes())])
    q = torch.from_numpy(packed.copy()).view(torch.int8).view(m, k // 2)
    s = torch.from_numpy(bs.copy()).view(torch.float8_e4m3fn).view(m, k // 16)
    for out_dtype, tdt, idt in (("f32", torch.float32, torch.int32), ("bf16", torch.bfloat16, torch.int16)):
        got = oracle.materialize(buf, out_dtype)["w.weight"]
        ref = _dequantize(q, s, tdt).contiguous().view(idt).numpy().view(got.dtype)
        assert np.array_equal(got, ref), out_dtype
