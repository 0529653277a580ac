"""GPU: the boundary-value fixtures of tests/golden/format_boundaries.json through the C ABI, for
every output type, against the stored bits: once as a single row (partial units, the exact path)
and once repeated to 2048 elements or more (whole units, the vector fast path)."""
import json
import os

import numpy as np
import pytest
import torch

import device_checkpoint_dequantisation_amd as st
from tests.golden.make_golden import case_file, period

pytestmark = pytest.mark.gpu
HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
CASES = json.load(open(os.path.join(HERE, "format_boundaries.json")))["cases"]


@pytest.mark.parametrize("repeat", [False, True])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16", "f32"])
def test_golden_cases(out_dtype, repeat):
    mask = 0xFFFFFFFF if out_dtype == "f32" else 0xFFFF
    for c in CASES:
        p = period(c["kind"], c["codes"])
        reps = max(1, -(-2048 // p)) if repeat else 1
        print(f"golden case {c['name']} into {out_dtype}, {reps} repeats", flush=True)
        buf = case_file(c["kind"], c["codes"], c["scales"], reps)
        ix = st.SafeTensorIndex.from_bytes(buf, out_dtype=out_dtype)
        ck = st.DeviceCheckpoint(ix, None, "cuda:0")
        ck.load_bytes(buf[ix.data_offset:])
        ck.arena.view(torch.int16).fill_(0x5A5A)
        ck.materialize()
        torch.cuda.synchronize()
        (t,) = ck.tensors.values()
        bits = t.reshape(-1).view(torch.int32 if out_dtype == "f32" else torch.int16).cpu().numpy()
        want = c["expect"][out_dtype]
        for r in range(reps):
            got = [int(b) & mask for b in bits[r * p: r * p + len(want)]]
            assert got == want, (c["name"], out_dtype, r, [hex(x) for x in got], [hex(x) for x in want])
