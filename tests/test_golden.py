"""The boundary-value fixtures in tests/golden/format_boundaries.json: the oracle still gives the
stored bits (a regression check of the oracle), and each case's stored first element equals
independent casts of its fp32 value worked out from the format definitions (numpy's fp32, torch's
bf16 and fp16 casts)."""
import json
import os

import numpy as np
import torch

import oracle
from tests.golden.make_golden import case_file

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
CASES = json.load(open(os.path.join(HERE, "format_boundaries.json")))["cases"]


def test_the_oracle_reproduces_the_fixtures():
    for c in CASES:
        buf = case_file(c["kind"], c["codes"], c["scales"])
        for dt, want in c["expect"].items():
            (bits,) = oracle.materialize(buf, dt).values()
            assert [int(b) for b in np.asarray(bits).reshape(-1)[: len(want)]] == want, (c["name"], dt)


def test_first_elements_equal_independent_casts_of_their_values():
    for c in CASES:
        v = np.float32(float(c["value_first"]))
        assert c["expect"]["f32"][0] == int(np.array([v]).view(np.uint32)[0]), c["name"]
        t = torch.tensor([v], dtype=torch.float32)
        assert c["expect"]["bf16"][0] == int(t.to(torch.bfloat16).view(torch.int16)[0]) & 0xFFFF, c["name"]
        assert c["expect"]["f16"][0] == int(t.to(torch.float16).view(torch.int16)[0]) & 0xFFFF, c["name"]
