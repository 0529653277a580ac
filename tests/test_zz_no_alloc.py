"""The allocation-free launch (st_materialize_noalloc) against the launch it varies
(st_materialize_as), called through the C ABI: bit-exact equal outputs, which the oracle also
checks, on two calls in a row on one stream (the second with a smaller table, so the scratch array
still holds the tail of the first), for every output type and for column slices; and its host-side
refusals, which enqueue nothing."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import synth
import device_checkpoint_dequantisation_amd as st
from device_checkpoint_dequantisation_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BITS = {"bf16": torch.int16, "f16": torch.int16, "f32": torch.int32}


def _staged(buf, out_dtype):
    ix = st.SafeTensorIndex.from_bytes(buf, out_dtype=out_dtype)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.load_bytes(buf[ix.data_offset:])
    return ix, ck


def _second_arena(ix, ck):
    """An arena of the same layout as ck's, poisoned, with its output pointers."""
    arena = torch.empty_like(ck.arena)
    arena.view(torch.int16).fill_(0x5A5A)
    esize = arena.element_size()
    ptrs = [arena.data_ptr() + o.offset for o in ix.outputs()]
    views = {o.name: arena[o.offset // esize: o.offset // esize + o.numel] for o in ix.outputs()}
    return arena, ptrs, views


@pytest.mark.parametrize("out_dtype", ["bf16", "f16", "f32"])
def test_noalloc_equals_materialize_two_calls(out_dtype):
    first = synth.config_bytes(5, small=True)    # thousands of small mixed tensors: the larger table
    second = synth.config_bytes(3, small=True)   # block FP8 + bf16: a smaller table
    calls = []
    for buf in (first, second):
        ix, ck = _staged(buf, out_dtype)
        ck.arena.view(torch.int16).fill_(0x5A5A)
        ck.materialize()                                      # the existing entry point
        arena, ptrs, views = _second_arena(ix, ck)
        raw, units = ix.table()
        calls.append((buf, ix, ck, arena, views, raw, units, ptrs))
    assert len(calls[1][5]) < len(calls[0][5]), "the second table must be the smaller one"
    stream = torch.cuda.current_stream(DEV)
    keep = []
    for buf, ix, ck, arena, views, raw, units, ptrs in calls:    # back to back, no sync between
        print(f"noalloc: {len(raw)}-byte table, {units} units, {len(ptrs)} outputs, {out_dtype}", flush=True)
        keep.append(st.materialize_noalloc(ck.blob, raw, units, ptrs, stream, out_dtype=out_dtype))
    torch.cuda.synchronize()
    for buf, ix, ck, arena, views, raw, units, ptrs in calls:
        want = oracle.materialize(buf, out_dtype)
        for name, w in want.items():
            ref = ck.tensors[name].reshape(-1).view(BITS[out_dtype])
            got = views[name].view(BITS[out_dtype])
            assert torch.equal(got, ref), f"{name}: st_materialize_noalloc differs from st_materialize_as"
            g = got.cpu().numpy().view(w.dtype)
            assert np.array_equal(g, w.reshape(-1)), f"{name}: differs from the oracle"


def test_noalloc_column_slices():
    buf = synth.config_bytes(4, small=True)        # NVFP4: column cuts at multiples of 16
    ix, ck = _staged(buf, "bf16")
    ck.materialize()
    slices = []
    for k, o in enumerate(ix.outputs()):
        if len(o.shape) == 2 and o.kind == "NVFP4":
            c = o.shape[1]
            slices.append((k, (1, o.shape[0] - 1), (16, c - 16)))
    raw, units = ix.table_slices(slices)
    outs = [torch.full(ix.slice_shape(*sl), float("nan"), dtype=torch.bfloat16, device=DEV) for sl in slices]
    keep = st.materialize_noalloc(ck.blob, raw, units, [t.data_ptr() for t in outs], slices=True)
    torch.cuda.synchronize()
    del keep
    for (k, (r0, r1), (c0, c1)), got in zip(slices, outs):
        whole = ck.tensors[ix.output(k).name]
        assert torch.equal(got.view(torch.int16), whole[r0:r1, c0:c1].view(torch.int16))


def test_noalloc_refusals_enqueue_nothing():
    buf = synth.config_bytes(1)
    ix, ck = _staged(buf, "bf16")
    raw, units = ix.table()
    ptrs = [0] * ix.num_outputs
    L = _lib.lib()
    s = C.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    tbl = C.create_string_buffer(raw, len(raw))
    pp = (C.c_void_p * len(ptrs))()
    blob = C.c_void_p(ck.blob.data_ptr())
    big = _lib.NOALLOC_SCRATCH_BYTES
    cases = [
        (tbl, big + 64, units, pp, len(ptrs), 0),                # table past the scratch size
        (tbl, len(raw), units, pp, big // 8, 0),                 # pointer array past it
        (tbl, len(raw), units + 4, pp, len(ptrs), 0),            # n disagrees with the header
        (tbl, len(raw), units, pp, len(ptrs), 2),                # output type disagrees
        (tbl, len(raw), units, pp, len(ptrs) - 1, 0),            # a descriptor's pointer is missing
        (tbl, 40, units, pp, len(ptrs), 0),                      # no header
    ]
    for t, nb, n, p, n_outs, odt in cases:
        r = L.st_materialize_noalloc(blob, t, nb, n, p, n_outs, odt, 0, s)
        assert r == -1, (nb, n, n_outs, odt, r)
        assert L.st_last_error().decode()
    torch.cuda.synchronize()
