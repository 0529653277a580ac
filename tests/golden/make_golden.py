"""Writes format_boundaries.json: boundary values of every format, as the bits the oracle gives for
each output type.  Run from the repository root: ``python -m tests.golden.make_golden``.  It calls
only the oracle (and the shared file writer); no value comes from the GPU path.

Each case also states its first element's fp32 result, worked out from the public format
definitions (e4m3fn, e2m1, E8M0, IEEE binary16/32), so the test can check the stored bits against
independent casts of that value.
The pages name these formats (block-FP8 and ModelOpt NVFP4 checkpoints in "Resident Modal LLM
Architecture", section "Current Backend Boundary"; scaled FP8 in "Disk tier safetensors streaming
design audit", section "Mandatory research audit") but print no worked values."""
import json
import os

import numpy as np

import oracle
from tests.st_files import make_file

HERE = os.path.dirname(os.path.abspath(__file__))


def f32(x):
    return int(np.array([x], np.float32).view(np.uint32)[0])


# (name, kind, codes, scale fields, the first element's fp32 result as a string float() reads, why)
CASES = [
    ("e4m3 max normal x 1", "FP8_TENSOR", [0x7E], {"scale": f32(1.0)}, "448", "largest e4m3fn value"),
    ("e4m3 min subnormal x 1", "FP8_TENSOR", [0x01], {"scale": f32(1.0)}, str(2.0 ** -9), "smallest e4m3fn subnormal"),
    ("e4m3 -0 x 1", "FP8_TENSOR", [0x80], {"scale": f32(1.0)}, "-0.0", "signed zero kept"),
    ("e4m3 max x 2^119", "FP8_TENSOR", [0x7E], {"scale": f32(2.0 ** 119)}, str(448 * 2.0 ** 119),
     "fp32 product 1.75 x 2^127, finite; infinite in fp16"),
    ("e4m3 max x 2^120", "FP8_TENSOR", [0x7E], {"scale": f32(2.0 ** 120)}, "inf",
     "448 x 2^120 overflows the fp32 product to infinity"),
    ("e4m3 1.125 x 0x3F6471C8", "FP8_TENSOR", [0x39], {"scale": 0x3F6471C8},
     str(1.125 * float(np.array([0x3F6471C8], np.uint32).view(np.float32)[0])),
     "reading R1: fp32 product 1.00390625 ties to even in bf16 (witness W1)"),
    ("block fp8 max x 0.5", "FP8_BLOCK128", [0x7E], {"scale_inv": f32(0.5)}, "224", "weight_scale_inv is multiplied (R3)"),
    ("nvfp4 6 x 448 x 1", "NVFP4", [0x7, 0x0], {"block": 0x7E, "global": f32(1.0)}, "2688", "largest e2m1 times largest block scale"),
    ("nvfp4 0.5 x 2^-9 x 1", "NVFP4", [0x1, 0x9], {"block": 0x01, "global": f32(1.0)}, str(0.5 * 2.0 ** -9),
     "smallest e2m1 times smallest block scale (element 1: -0.5 x 2^-9)"),
    ("nvfp4 6 x 240 x 0x3B2D27D2", "NVFP4", [0x7, 0x7], {"block": 0x77, "global": 0x3B2D27D2},
     repr(float(np.float32(np.float32(1440.0) * np.array([0x3B2D27D2], np.uint32).view(np.float32)[0]))),
     "reading R2: (e2m1 x block) first, then the global scale (witness W2)"),
    ("mxfp8 max x 2^127", "MXFP8", [0x7E], {"e8m0": 254}, "inf", "448 x 2^127 overflows fp32 to infinity"),
    ("mxfp8 1 x 2^-127", "MXFP8", [0x38], {"e8m0": 0}, str(2.0 ** -127), "E8M0 code 0 is 2^-127, an fp32 subnormal"),
    ("mxfp4 0.5 x 2^-127", "MXFP4", [0x1, 0x0], {"e8m0": 0}, str(2.0 ** -128), "fp32 subnormal product, exact"),
    ("mxfp4 6 x 1", "MXFP4", [0x7, 0xF], {"e8m0": 127}, "6", "E8M0 code 127 is 1.0 (element 1: -6)"),
    ("fp16 max to bf16", "CAST_F16", [0x7BFF], {}, "65504", "rounds up to 65536 in bf16"),
    ("fp16 min subnormal", "CAST_F16", [0x0001], {}, str(2.0 ** -24), "fp16 subnormal, exact in bf16"),
    ("fp32 65520", "CAST_F32", [f32(65520.0)], {}, "65520", "the fp16 overflow boundary (to +inf in fp16)"),
    ("fp32 max", "CAST_F32", [0x7F7FFFFF], {}, repr(float(np.finfo(np.float32).max)), "rounds to +inf in bf16"),
]


def period(kind, codes):
    """Elements per repeat of a case's row: MX and packed fp4 rows are whole 32-element blocks."""
    return 32 if kind in ("MXFP8", "MXFP4", "NVFP4") else len(codes)


def case_file(kind, codes, sc, reps=1):
    """A one-tensor checkpoint whose row holds `codes` (zero-padded to the period), repeated `reps`
    times, with its scales (the same scale for every block)."""
    p = period(kind, codes)
    c = np.zeros(p * reps, np.uint64)
    for r in range(reps):
        c[r * p: r * p + len(codes)] = codes
    n = p * reps
    if kind == "FP8_TENSOR":
        return make_file([("w.weight", "F8_E4M3", (n,), c.astype(np.uint8)),
                          ("w.scale_weight", "F32", (), np.array([sc["scale"]], np.uint32).tobytes())])
    if kind == "FP8_BLOCK128":
        g = -(-n // 128)
        return make_file([("w.weight", "F8_E4M3", (1, n), c.astype(np.uint8)),
                          ("w.weight_scale_inv", "F32", (1, g), np.full(g, sc["scale_inv"], np.uint32).tobytes())])
    if kind == "MXFP8":
        return make_file([("w.weight", "F8_E4M3", (1, n), c.astype(np.uint8)),
                          ("w.weight_scale", "F8_E8M0", (1, n // 32), np.full(n // 32, sc["e8m0"], np.uint8))])
    if kind in ("NVFP4", "MXFP4"):
        c = c.astype(np.uint8)
        packed = (c[0::2] | (c[1::2] << 4)).astype(np.uint8)   # element 2k in the low nibble
        if kind == "MXFP4":
            return make_file([("w.weight", "U8", (1, n // 2), packed),
                              ("w.weight_scale", "F8_E8M0", (1, n // 32), np.full(n // 32, sc["e8m0"], np.uint8))])
        return make_file([("w.weight", "U8", (1, n // 2), packed),
                          ("w.weight_scale", "F8_E4M3", (1, n // 16), np.full(n // 16, sc["block"], np.uint8)),
                          ("w.weight_scale_2", "F32", (), np.array([sc["global"]], np.uint32).tobytes())])
    if kind == "CAST_F16":
        return make_file([("w", "F16", (n,), c.astype(np.uint16))])
    if kind == "CAST_F32":
        return make_file([("w", "F32", (n,), c.astype(np.uint32))])
    raise ValueError(kind)


def main():
    out = []
    for name, kind, codes, sc, exact, why in CASES:
        buf = case_file(kind, codes, sc)
        expect = {}
        for dt in ("bf16", "f16", "f32"):
            (bits,) = oracle.materialize(buf, dt).values()
            expect[dt] = [int(b) for b in np.asarray(bits).reshape(-1)[: len(codes)]]
        out.append({"name": name, "kind": kind, "codes": codes, "scales": sc, "value_first": exact, "why": why,
                    "expect": expect})
    with open(os.path.join(HERE, "format_boundaries.json"), "w") as f:
        json.dump({"written_by": "tests/golden/make_golden.py (the oracle)", "cases": out}, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
