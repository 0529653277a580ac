"""GPU: a decode captured in a HIP graph (torch.cuda.CUDAGraph) replays correctly.  The launch
path allocates nothing and records no memset, so it can be captured; every replay, with eager
work and synchronisation between replays, must equal the eager decode and the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import device_checkpoint_dequantisation_amd as st

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("k,out_dtype", [(2, "bf16"), (4, "f32"), (5, "bf16")])
def test_captured_decode_replays(k, out_dtype):
    buf = synth.config_bytes(k, small=True)
    ix = st.SafeTensorIndex.from_bytes(buf, out_dtype=out_dtype)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.load_bytes(buf[ix.data_offset:])
    torch.cuda.synchronize()
    print(f"graph capture c{k} {out_dtype}", flush=True)
    ck.materialize()
    torch.cuda.synchronize()
    eager = {n: t.clone() for n, t in ck.tensors.items()}   # the outputs (not the arena's padding)
    want = oracle.materialize(buf, out_dtype)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ck.materialize(s)          # warm the launch path on the side stream before capturing
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        ck.materialize()
    for r in range(4):
        ck.arena.view(torch.int16).fill_(0x5A5A + r)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in ck.tensors.items():
            assert torch.equal(t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32),
                               eager[n].view(torch.int16) if t.element_size() == 2 else eager[n].view(torch.int32)), (r, n)
    for name, w in want.items():
        t = ck.tensors[name].contiguous()
        got = (t.view(torch.int32) if out_dtype == "f32" else t.view(torch.int16)).cpu().numpy().view(w.dtype)
        assert np.array_equal(got.reshape(w.shape), w), name
