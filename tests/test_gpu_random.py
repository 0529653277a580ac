"""GPU: seeded random sweep.  Each case draws a checkpoint family, a generator seed, an output
type and a work-unit size; the whole decode must equal the oracle bit for bit, and so must a
random set of row / column / block slices through the strided kernel instance."""
import numpy as np
import pytest
import torch

import oracle
import synth
import device_checkpoint_dequantisation_amd as st
from tests.test_gpu_slices import _slices_for, _view

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits(t, out_dtype):
    t = t.contiguous()
    if out_dtype == "f32":
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("case", range(40))
def test_random_case(case):
    rng = np.random.default_rng(1000 + case)
    k = int(rng.integers(2, 8))
    seed = int(rng.integers(100, 10_000))
    out_dtype = ("bf16", "f16", "f32")[int(rng.integers(0, 3))]
    scale = int(rng.choice([0, 0, 1, 2]))
    print(f"random case {case}: family {k} seed {seed} {out_dtype} unit scale {scale}", flush=True)
    buf = synth.config_bytes(k, seed=seed, small=True)
    want = oracle.materialize(buf, out_dtype)
    ix = st.SafeTensorIndex.from_bytes(buf, out_dtype=out_dtype, unit_log2_scale=scale)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.load_bytes(buf[ix.data_offset:])
    ck.arena.view(torch.int16).fill_(0x5A5A)
    ck.materialize()
    torch.cuda.synchronize()
    for name, w in want.items():
        assert np.array_equal(_bits(ck.tensors[name], out_dtype).reshape(w.shape), w), (case, name)
    outs = ix.outputs()
    picks = rng.choice(len(outs), min(len(outs), 12), replace=False)
    slices = [(int(j), rows, cols) for j in picks for rows, cols in _slices_for(outs[int(j)], rng)]
    got = ck.materialize_slices(slices, strided_kernel=True)
    torch.cuda.synchronize()
    for (j, rows, cols), t in zip(slices, got):
        w = _view(want[outs[j].name])
        r0, r1 = rows if rows else (0, w.shape[0])
        c0, c1 = cols if cols else (0, w.shape[1])
        assert np.array_equal(_bits(t, out_dtype).reshape(r1 - r0, c1 - c0), w[r0:r1, c0:c1]), (case, outs[j].name, rows, cols)
