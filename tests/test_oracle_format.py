"""Pins of the oracle's safetensors parsing, layout checks and classification: round trips
against the safetensors library (an independent implementation of the format), the
generator's own layout, and one negative case per error rule."""
import json

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import OracleError
from tests.st_files import f32_bytes, make_file, raw_header_file


def test_tiny_round_trip_against_writer_layout():
    groups, meta, pad = synth.make_config(1)
    lay = synth.layout(groups, meta, pad)
    buf = synth.config_bytes(1)
    h, outs = oracle.plan(buf)
    assert h.data_size == lay.data_size == 718_856
    assert list(h.entries) == lay.order
    for name, (b, e) in lay.offsets.items():
        assert (h.entries[name].begin, h.entries[name].end) == (b, e)
    assert h.metadata == {"synthetic": "tiny", "seed": "1"}
    assert [o.name for o in outs] == ["bf16.0", "bf16.1", "f32.0", "f32.1", "fp8.0.weight", "fp8.1.weight",
                                     "f16.0", "f16.1"]
    assert [o.kind for o in outs] == ["PASS_BF16"] * 2 + ["CAST_F32"] * 2 + ["FP8_TENSOR"] * 2 + ["CAST_F16"] * 2
    assert sum(o.numel for o in outs) * 2 == 913_408
    # back-to-back packing: tensors after the first 4-byte scale sit 4 bytes off a 16-byte line
    assert h.entries["fp8.1.weight"].begin % 16 == 4 and h.entries["f16.0"].begin % 16 == 8


def _safetensors_library_file():
    from safetensors.torch import save
    g = torch.Generator().manual_seed(0)
    tensors = {
        "a.weight": torch.randn(33, 17, generator=g).to(torch.bfloat16),
        "b": torch.randn(7, generator=g).to(torch.float16),
        "c": torch.randn(3, 5, generator=g),
        "q.weight": (torch.randn(64, 48, generator=g) * 50).to(torch.float8_e4m3fn),
        "q.scale_weight": torch.tensor(0.0125),
        "z": torch.zeros(0, 4, dtype=torch.bfloat16),
    }
    return tensors, save(tensors, metadata={"k": "v"})


def test_parse_matches_safetensors_library_output():
    tensors, buf = _safetensors_library_file()
    h, outs = oracle.plan(buf)
    names = {"a.weight": "BF16", "b": "F16", "c": "F32", "q.weight": "F8_E4M3", "q.scale_weight": "F32", "z": "BF16"}
    assert {n: e.dtype for n, e in h.entries.items()} == names
    for n, t in tensors.items():
        assert h.entries[n].shape == tuple(t.shape)
        raw = np.frombuffer(buf, np.uint8)[h.data_offset + h.entries[n].begin: h.data_offset + h.entries[n].end]
        assert raw.tobytes() == t.contiguous().reshape(-1).view(torch.uint8).numpy().tobytes()
    mats = oracle.materialize(buf)
    assert np.array_equal(mats["a.weight"], tensors["a.weight"].view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(mats["b"], tensors["b"].to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(mats["c"], tensors["c"].to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    q = (tensors["q.weight"].float() * tensors["q.scale_weight"]).to(torch.bfloat16)
    assert np.array_equal(mats["q.weight"], q.view(torch.int16).numpy().view(np.uint16))
    assert mats["z"].shape == (0, 4)
    assert h.metadata == {"k": "v"}


def test_safetensors_library_reads_unaligned_writer_output():
    from safetensors import safe_open
    buf = synth.config_bytes(1)
    h = oracle.parse_header(buf)
    import tempfile, os
    with tempfile.TemporaryDirectory() as d:
        p = os.path.join(d, "t.safetensors")
        open(p, "wb").write(buf)
        with safe_open(p, framework="pt") as f:
            assert set(f.keys()) == set(h.entries)
            for n, e in h.entries.items():
                t = f.get_tensor(n)
                assert tuple(t.shape) == e.shape
                raw = buf[h.data_offset + e.begin: h.data_offset + e.end]
                assert t.contiguous().reshape(-1).view(torch.uint8).numpy().tobytes() == raw


def test_f4_storage_parses_with_unpacked_shape():
    from safetensors.torch import save
    packed = torch.arange(64, dtype=torch.uint8).reshape(4, 16)
    t = packed.view(torch.float4_e2m1fn_x2)
    buf = save({"x.weight": t, "x.weight_scale": torch.full((4, 2), 0x38, dtype=torch.uint8).view(torch.float8_e4m3fn),
                "x.weight_scale_2": torch.tensor(1.0)})
    h, outs = oracle.plan(buf)
    assert h.entries["x.weight"].dtype == "F4" and h.entries["x.weight"].shape == (4, 32)
    assert outs[0].kind == "NVFP4" and outs[0].shape == (4, 32)
    # the same bytes stored as U8 [4, 16] decode identically
    u8 = make_file([("x.weight", "U8", (4, 16), packed.numpy()),
                    ("x.weight_scale", "F8_E4M3", (4, 2), np.full(8, 0x38, np.uint8)),
                    ("x.weight_scale_2", "F32", (), f32_bytes(1.0))])
    assert np.array_equal(oracle.materialize(buf)["x.weight"], oracle.materialize(u8)["x.weight"])


def test_padded_and_unpadded_headers_parse_alike():
    a = synth.config_bytes(2, small=True)
    groups, meta, _ = synth.make_config(2, small=True)
    b = synth.build_bytes(groups, meta, pad_header=False)
    ha, hb = oracle.parse_header(a), oracle.parse_header(b)
    assert ha.header_len % 8 == 0 and ha.entries == hb.entries


def test_empty_header_and_zero_size_tensors():
    assert oracle.materialize(raw_header_file("{}")) == {}
    f = make_file([("e", "BF16", (0,), b""), ("s", "F32", (), f32_bytes(2.0)), ("e2", "F16", (3, 0), b"")])
    m = oracle.materialize(f)
    assert m["e"].shape == (0,) and m["e2"].shape == (3, 0) and m["s"].shape == () and m["s"] == 0x4000


# ------------------------------------------------------------------ negative cases

def _entry(dtype="BF16", shape=(2,), offs=(0, 4)):
    return {"dtype": dtype, "shape": list(shape), "data_offsets": list(offs)}


BAD = {
    "short file": b"\x01\x00",
    "header past end": (100).to_bytes(8, "little") + b"{}",
    "header cap": (100_000_001).to_bytes(8, "little") + b"{}",
    "not utf8": raw_header_file(b'{"\xff":1}'),
    "not json": raw_header_file("{nope"),
    "not object": raw_header_file("[1,2]"),
    "trailing garbage": raw_header_file("{} x"),
    "NaN constant": raw_header_file('{"a":{"dtype":"BF16","shape":[NaN],"data_offsets":[0,0]}}'),
    "duplicate key": raw_header_file('{"a":' + json.dumps(_entry()) + ',"a":' + json.dumps(_entry()) + "}", b"\0" * 4),
    "unknown dtype": raw_header_file(json.dumps({"a": _entry("Q7")}), b"\0" * 4),
    "float shape": raw_header_file('{"a":{"dtype":"BF16","shape":[2.0],"data_offsets":[0,4]}}', b"\0" * 4),
    "bool shape": raw_header_file('{"a":{"dtype":"BF16","shape":[true],"data_offsets":[0,2]}}', b"\0" * 2),
    "negative dim": raw_header_file(json.dumps({"a": _entry(shape=(-2,))}), b"\0" * 4),
    "too many dims": raw_header_file(json.dumps({"a": _entry(shape=(1,) * 9, offs=(0, 2))}), b"\0" * 2),
    "extra field": raw_header_file(json.dumps({"a": dict(_entry(), extra=1)}), b"\0" * 4),
    "missing field": raw_header_file(json.dumps({"a": {"dtype": "BF16", "shape": [2]}}), b"\0" * 4),
    "begin > end": raw_header_file(json.dumps({"a": _entry(offs=(4, 0))}), b"\0" * 4),
    "span mismatch": raw_header_file(json.dumps({"a": _entry(offs=(0, 6))}), b"\0" * 6),
    "gap": raw_header_file(json.dumps({"a": _entry(offs=(2, 6))}), b"\0" * 6),
    "overlap": raw_header_file(json.dumps({"a": _entry(offs=(0, 4)), "b": _entry(offs=(2, 6))}), b"\0" * 6),
    "short data": raw_header_file(json.dumps({"a": _entry(offs=(0, 4))}), b"\0" * 3),
    "long data": raw_header_file(json.dumps({"a": _entry(offs=(0, 4))}), b"\0" * 5),
    "metadata not str": raw_header_file('{"__metadata__":{"k":1}}'),
    "lone surrogate": raw_header_file('{"\\ud800":' + json.dumps(_entry()) + "}", b"\0" * 4),
    "nul in name": raw_header_file('{"a\\u0000b":' + json.dumps(_entry()) + "}", b"\0" * 4),
    "int64 overflow": raw_header_file('{"a":{"dtype":"BF16","shape":[9223372036854775808,0],"data_offsets":[0,0]}}'),
    "odd F4 bytes": raw_header_file(json.dumps({"a": _entry("F4", (3,), (0, 1))}), b"\0"),
    "i64 output": raw_header_file(json.dumps({"a": _entry("I64", (1,), (0, 8))}), b"\0" * 8),
    "fp8 without scale": make_file([("w.weight", "F8_E4M3", (4,), b"\0" * 4)]),
    "fp8 not .weight": make_file([("w", "F8_E4M3", (4,), b"\0" * 4), ("w.scale_weight", "F32", (), f32_bytes(1))]),
    "orphan scale": make_file([("w.scale_weight", "F32", (), f32_bytes(1))]),
    "scale not scalar": make_file([("w.weight", "F8_E4M3", (4,), b"\0" * 4), ("w.scale_weight", "F32", (2,), f32_bytes(1, 1))]),
    "scale wrong dtype": make_file([("w.weight", "F8_E4M3", (4,), b"\0" * 4), ("w.scale_weight", "BF16", (), b"\0\0")]),
    "both scales": make_file([("w.weight", "F8_E4M3", (1, 4), b"\0" * 4), ("w.scale_weight", "F32", (), f32_bytes(1)),
                              ("w.weight_scale_inv", "F32", (1, 1), f32_bytes(1))]),
    "block grid shape": make_file([("w.weight", "F8_E4M3", (129, 4), b"\0" * 516), ("w.weight_scale_inv", "F32", (1, 1), f32_bytes(1))]),
    "block 1-D": make_file([("w.weight", "F8_E4M3", (4,), b"\0" * 4), ("w.weight_scale_inv", "F32", (1,), f32_bytes(1))]),
    "nvfp4 K%16": make_file([("w.weight", "U8", (1, 4), b"\0" * 4), ("w.weight_scale", "F8_E4M3", (1, 0), b""),
                             ("w.weight_scale_2", "F32", (), f32_bytes(1))]),
    "nvfp4 missing global": make_file([("w.weight", "U8", (1, 8), b"\0" * 8), ("w.weight_scale", "F8_E4M3", (1, 1), b"\0")]),
    "nvfp4 scale shape": make_file([("w.weight", "U8", (1, 8), b"\0" * 8), ("w.weight_scale", "F8_E4M3", (2, 1), b"\0\0"),
                                    ("w.weight_scale_2", "F32", (), f32_bytes(1))]),
    "u8 not .weight": make_file([("w", "U8", (4,), b"\0" * 4)]),
}


@pytest.mark.parametrize("case", sorted(BAD))
def test_malformed_input_is_rejected(case):
    with pytest.raises(OracleError):
        oracle.materialize(BAD[case])
