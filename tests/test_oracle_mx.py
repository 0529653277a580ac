"""Pins of the oracle's OCP Microscaling formats (MXFP8, MXFP4): the E8M0 scale table against
torch's float8_e8m0fnu decoding (an independent implementation), every element code times every
scale code against an exact float64 product, the scale-index mapping with position-coded scales,
files written by the safetensors library decoded by an independent torch computation, and the
classification rules with their rejections."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import OracleError
from tests.st_files import f32_bytes, make_file


def _bf16_torch(x64):
    """float64 values -> fp32 (NumPy, round to nearest even) -> bf16 bits (torch's cast)."""
    f = torch.from_numpy(np.asarray(x64, dtype=np.float64).astype(np.float32))
    return f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_e8m0_table_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert nan.tolist() == [c == 255 for c in range(256)]
    assert np.array_equal(oracle.E8M0[~nan], ref[~nan]) and np.isnan(oracle.E8M0[255])
    assert oracle.E8M0[127] == 1.0 and oracle.E8M0[0] == np.float32(2.0 ** -127) and oracle.E8M0[254] == np.float32(2.0 ** 127)


def _mx_file(kind, codes, scales, m, k, storage="U8"):
    if kind == "MXFP8":
        return make_file([("w.weight", "F8_E4M3", (m, k), codes.astype(np.uint8)),
                          ("w.weight_scale", "F8_E8M0", (m, k // 32), scales.astype(np.uint8))])
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    shape = (m, k // 2) if storage == "U8" else (m, k)
    return make_file([("w.weight", storage, shape, packed),
                      ("w.weight_scale", "F8_E8M0", (m, k // 32), scales.astype(np.uint8))])


def test_mxfp8_every_code_times_every_scale_brute_force():
    # row r uses scale code r; its 256 elements are every e4m3 code: 256 x 256 products
    m, k = 256, 256
    codes = np.tile(np.arange(256), m)
    scales = np.repeat(np.arange(256), k // 32)
    out = oracle.materialize(_mx_file("MXFP8", codes, scales, m, k))["w.weight"]
    f32 = oracle.materialize(_mx_file("MXFP8", codes, scales, m, k), "f32")["w.weight"]
    elem = np.array([oracle.e4m3_value(c) for c in range(256)])
    for r in range(256):
        exact = elem * (2.0 ** (r - 127) if r < 255 else np.nan)
        with np.errstate(invalid="ignore", over="ignore"):
            want = _bf16_torch(exact)
            want32 = exact.astype(np.float32).view(np.uint32)
        want = np.where(np.isnan(exact), np.uint16(0x7FC0), want)
        want32 = np.where(np.isnan(exact), np.uint32(0x7FC00000), want32)
        assert np.array_equal(out[r], want), r
        assert np.array_equal(f32[r], want32), r


@pytest.mark.parametrize("storage", ["U8", "F4"])
def test_mxfp4_every_nibble_times_every_scale_brute_force(storage):
    m, k = 256, 32
    codes = np.tile(np.arange(16), m * k // 16)
    scales = np.arange(256)
    out = oracle.materialize(_mx_file("MXFP4", codes, scales, m, k, storage))["w.weight"]
    elem = np.array([oracle.e2m1_value(c) for c in range(16)] * 2)
    for r in range(256):
        exact = elem * (2.0 ** (r - 127) if r < 255 else np.nan)
        with np.errstate(invalid="ignore", over="ignore"):
            want = np.where(np.isnan(exact), np.uint16(0x7FC0), _bf16_torch(exact))
        assert np.array_equal(out[r], want), r


def test_mx_scale_index_mapping_position_coded():
    # every element 1.0 (e4m3 0x38, e2m1 0x2): the output is its block's scale, and each
    # (row, block) has a distinct scale exponent
    m, k = 5, 160
    scales = 100 + np.arange(m * (k // 32))
    want_exp = (scales.reshape(m, k // 32) - 127).repeat(32, axis=1)
    for kind, one in (("MXFP8", 0x38), ("MXFP4", 0x2)):
        out = oracle.materialize(_mx_file(kind, np.full(m * k, one), scales, m, k), "f32")["w.weight"]
        assert np.array_equal(out.view(np.float32), np.exp2(want_exp).astype(np.float32)), kind


def test_mx_files_written_by_the_safetensors_library():
    """A file the safetensors library writes from torch float8_e4m3fn / float8_e8m0fnu tensors
    decodes to torch's own two-step computation: element times its block's scale in fp32, then
    a bf16 cast."""
    from safetensors.torch import save
    g = torch.Generator().manual_seed(3)
    m, k = 48, 96
    w = (torch.randn(m, k, generator=g) * 8).to(torch.float8_e4m3fn)
    sc = torch.randint(110, 140, (m, k // 32), generator=g, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu)
    buf = save({"layer.weight": w, "layer.weight_scale": sc})
    h, outs = oracle.plan(buf)
    assert [(o.name, o.kind, o.shape) for o in outs] == [("layer.weight", "MXFP8", (m, k))]
    got = oracle.materialize(buf)["layer.weight"]
    ref = (w.to(torch.float32) * sc.to(torch.float32).repeat_interleave(32, dim=1)).to(torch.bfloat16)
    assert np.array_equal(got, ref.view(torch.int16).numpy().view(np.uint16))


def test_mx_synthetic_families_classify():
    for k, kind in ((6, "MXFP8"), (7, "MXFP4")):
        h, outs = oracle.plan(synth.config_bytes(k, small=True))
        assert {o.kind for o in outs} - {"PASS_BF16"} == {kind}
        for o in outs:
            if o.kind == kind:
                assert o.scale.dtype == "F8_E8M0" and o.scale.shape == (o.shape[0], o.shape[1] // 32)


E8 = np.full(4, 127, np.uint8)


@pytest.mark.parametrize("tensors,match", [
    ([("w.weight", "F8_E4M3", (2, 48), np.zeros(96, np.uint8)), ("w.weight_scale", "F8_E8M0", (2, 1), E8[:2])],
     "multiple of 32"),
    ([("w.weight", "F8_E4M3", (64,), np.zeros(64, np.uint8)), ("w.weight_scale", "F8_E8M0", (2,), E8[:2])],
     "2-D"),
    ([("w.weight", "F8_E4M3", (2, 32), np.zeros(64, np.uint8)), ("w.weight_scale", "F8_E8M0", (2, 2), E8)],
     "F8_E8M0"),
    ([("w.weight", "F8_E4M3", (2, 32), np.zeros(64, np.uint8)), ("w.weight_scale", "F8_E4M3", (2, 1), E8[:2])],
     "F8_E8M0"),
    ([("w.weight", "F8_E4M3", (2, 32), np.zeros(64, np.uint8)), ("w.weight_scale", "F8_E8M0", (2, 1), E8[:2]),
      ("w.scale_weight", "F32", (), f32_bytes(1.0))], "more than one"),
    ([("w.weight", "F8_E4M3", (2, 32), np.zeros(64, np.uint8)), ("w.weight_scale", "F8_E8M0", (2, 1), E8[:2]),
      ("w.weight_scale_2", "F32", (), f32_bytes(1.0))], "weight_scale_2"),
    ([("w.weight", "U8", (2, 8), np.zeros(16, np.uint8)), ("w.weight_scale", "F8_E8M0", (2, 1), E8[:2])],
     "multiple of 32"),
    ([("w.weight", "U8", (2, 16), np.zeros(32, np.uint8)), ("w.weight_scale", "F8_E8M0", (2, 1), E8[:2]),
      ("w.weight_scale_2", "F32", (), f32_bytes(1.0))], "weight_scale_2"),
    ([("w.weight", "U8", (2, 16), np.zeros(32, np.uint8)), ("w.weight_scale", "F8_E8M0", (1, 2), E8[:2])],
     "F8_E8M0"),
    ([("w.weight_scale", "F8_E8M0", (2, 1), E8[:2])], "no matching weight"),
])
def test_mx_malformed_is_rejected(tensors, match):
    with pytest.raises(OracleError, match=match):
        oracle.plan(make_file(tensors))


def test_mxfp4_matches_an_independent_library_decoder():
    """transformers' MXFP4 dequantiser (written for checkpoints that store 32 e2m1 values as 16
    uint8 bytes per block with one E8M0 byte per block) is an implementation of the packed layout
    independent of the oracle.  Its fp32 output pins the nibble order (element 2k in the low
    nibble of byte k) and the block-scale mapping.  The file is built from the packed bytes
    themselves, so the test does not assume the order it checks."""
    pytest.importorskip("transformers")
    from transformers.integrations.mxfp4 import convert_moe_packed_tensors
    rng = np.random.default_rng(11)
    m, k = 24, 96
    packed = rng.integers(0, 256, m * k // 2, dtype=np.uint64).astype(np.uint8)
    scales = rng.integers(100, 150, m * (k // 32), dtype=np.uint64).astype(np.uint8)
    buf = make_file([("w.weight", "U8", (m, k // 2), packed), ("w.weight_scale", "F8_E8M0", (m, k // 32), scales)])
    got = oracle.materialize(buf, "f32")["w.weight"]
    blocks = torch.from_numpy(packed.copy()).view(1, m, k // 32, 16)
    sc = torch.from_numpy(scales.copy()).view(1, m, k // 32)
    ref = convert_moe_packed_tensors(blocks, sc, dtype=torch.float32)   # [1, k, m]: rows last
    ref = ref[0].transpose(0, 1).contiguous().numpy()
    assert ref.shape == (m, k)
    assert np.array_equal(got, ref.view(np.uint32))


def test_nvfp4_nibble_order_is_the_pinned_mxfp4_order():
    """The oracle's NVFP4 branch unpacks nibbles on its own; with every block scale 1.0 (e4m3 0x38)
    and a global scale of 1.0 it must equal the MXFP4 branch (pinned above) at scale 2^0."""
    rng = np.random.default_rng(12)
    m, k = 16, 64
    packed = rng.integers(0, 256, m * k // 2, dtype=np.uint64).astype(np.uint8)
    nv = make_file([("w.weight", "U8", (m, k // 2), packed), ("w.weight_scale", "F8_E4M3", (m, k // 16),
                    np.full(m * k // 16, 0x38, np.uint8)), ("w.weight_scale_2", "F32", (), f32_bytes(1.0))])
    mx = make_file([("w.weight", "U8", (m, k // 2), packed),
                    ("w.weight_scale", "F8_E8M0", (m, k // 32), np.full(m * k // 32, 127, np.uint8))])
    assert np.array_equal(oracle.materialize(nv, "f32")["w.weight"], oracle.materialize(mx, "f32")["w.weight"])
