"""GPU parity of the kernel instances with non-temporal output stores (ST_MAT_STREAM_STORES).  The
planner asks for them only for tables whose outputs exceed the last-level cache, which the small
checkpoints never do, so these tests pass the flag explicitly: every element must equal the oracle's,
through the whole-output and the slices instance, for every output type."""
import numpy as np
import pytest
import torch

import oracle
import synth
import device_checkpoint_dequantisation_amd as st

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BITS = {"bf16": torch.int16, "f16": torch.int16, "f32": torch.int32}


@pytest.mark.parametrize("slices", [False, True])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6, 7])
def test_whole_tables_with_stream_stores(k, out_dtype, slices):
    buf = synth.config_bytes(k, small=True)
    want = oracle.materialize(buf, out_dtype)
    ix = st.SafeTensorIndex.from_bytes(buf, out_dtype=out_dtype)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.load_bytes(buf[ix.data_offset:])
    assert not ck.stream_stores                    # small outputs: the planner keeps plain stores
    ck.arena.view(torch.int16).fill_(0x5A5A)       # poison: every element must be written
    print(f"stream stores c{k} {out_dtype} slices instance {slices}", flush=True)
    st.materialize(ck.blob, ck.table, ck.units, ck.outs, slices=slices, out_dtype=out_dtype, stream_stores=True)
    torch.cuda.synchronize()
    for name, w in want.items():
        g = ck.tensors[name].view(BITS[out_dtype]).cpu().numpy().view(w.dtype)
        assert np.array_equal(g.reshape(w.shape), w), name


@pytest.mark.parametrize("k", [2, 3, 4, 6, 7])
def test_column_slices_with_stream_stores(k):
    """One column slice per 2-d output (strided, not a complete shard set) through the slices instance
    with non-temporal stores, against the oracle's whole output."""
    buf = synth.config_bytes(k, small=True)
    want = oracle.materialize(buf)
    ix = st.SafeTensorIndex.from_bytes(buf)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.load_bytes(buf[ix.data_offset:])
    outs = ix.outputs()
    slices = []
    for j, o in enumerate(outs):
        if len(o.shape) != 2:
            continue
        q = 128 if o.kind == "FP8_BLOCK128" else 32 if o.kind in ("MXFP8", "MXFP4") else 16
        w = max(q, o.shape[1] // 2 // q * q)
        c0 = q if o.shape[1] >= q + w else 0
        slices.append((j, None, (c0, c0 + w)))
    assert slices
    raw, units = ix.table_slices(slices)
    table = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(DEV)
    shapes = [ix.slice_shape(*sl) for sl in slices]
    got = [torch.full((r, c), float("nan"), dtype=torch.bfloat16, device=DEV) for r, c in shapes]
    ptrs = torch.tensor([t.data_ptr() for t in got], dtype=torch.int64, device=DEV)
    st.materialize(ck.blob, table, units, ptrs, slices=True, stream_stores=True)
    torch.cuda.synchronize()
    for (j, _, (c0, c1)), t in zip(slices, got):
        w = want[outs[j].name].reshape(outs[j].shape[0], -1)
        assert np.array_equal(t.view(torch.int16).cpu().numpy().view(np.uint16), w[:, c0:c1]), (outs[j].name, c0, c1)



def _every_code_files():
    from tests.test_gpu_parity import (block_fp8_file, float_every_code_file, fp8_every_code_file, mx_every_code_file,
                                       nvfp4_every_code_file)
    return {"fp8": fp8_every_code_file, "nvfp4": nvfp4_every_code_file, "block": lambda s: block_fp8_file(257, 129, s),
            "float": float_every_code_file, "mxfp8": lambda s: mx_every_code_file("MXFP8", s),
            "mxfp4": lambda s: mx_every_code_file("MXFP4", s)}


@pytest.mark.parametrize("shift", [0, 1, 3, 9])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("name", ["fp8", "nvfp4", "block", "float", "mxfp8", "mxfp4"])
def test_every_code_with_stream_stores(name, out_dtype, shift):
    """The every-code files of each kind (NaN codes, special scales, ragged tails) behind a leading
    tensor that shifts every source off its natural alignment, through the streaming-store instance:
    its whole units of bf16 copies and MXFP8 load with non-temporal buffer loads, aligned and not."""
    buf = _every_code_files()[name](shift)
    want = oracle.materialize(buf, out_dtype)
    ix = st.SafeTensorIndex.from_bytes(buf, out_dtype=out_dtype)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.load_bytes(buf[ix.data_offset:])
    ck.arena.view(torch.int16).fill_(0x5A5A)
    print(f"stream stores, every code: {name} {out_dtype} shift {shift}", flush=True)
    st.materialize(ck.blob, ck.table, ck.units, ck.outs, out_dtype=out_dtype, stream_stores=True)
    torch.cuda.synchronize()
    for n, w in want.items():
        g = ck.tensors[n].view(BITS[out_dtype]).cpu().numpy().view(w.dtype)
        assert np.array_equal(g.reshape(w.shape), w), n
