"""GPU parity of sliced materialisation: each slice equals the same block of the oracle's whole
output, bit for bit, for row slices, column slices (fast and exact-only), empty and edge slices of
every kind; and tensor-parallel shards (8 row shards, 8 column shards where the cuts allow)
reassemble the whole output."""
import numpy as np
import pytest
import torch

import oracle
import synth
import device_checkpoint_dequantisation_amd as st
from tests.st_files import make_file

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _staged(buf):
    ix = st.SafeTensorIndex.from_bytes(buf)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.load_bytes(buf[ix.data_offset:])
    return ix, ck


def _view(w):
    """The oracle's whole output as the slicing matrix view."""
    if w.ndim == 0:
        return w.reshape(1, 1)
    if w.ndim == 1:
        return w.reshape(-1, 1)
    return w.reshape(w.shape[0], -1)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _slices_for(o, rng):
    """A spread of slices the cuts allow for output o."""
    shape = o.shape
    R = 1 if not shape else shape[0]
    C = 1 if len(shape) <= 1 else int(np.prod(shape[1:]))
    mx = o.kind in ("MXFP8", "MXFP4")
    rq = 128 if o.kind == "FP8_BLOCK128" else 1
    cq = 128 if o.kind == "FP8_BLOCK128" else 16 if o.kind == "NVFP4" else 32 if mx else 1
    wq = 16 if o.kind == "NVFP4" else 32 if mx else 1
    out = [(None, None), ((0, 0), None)]
    for _ in range(4):
        r0 = int(rng.integers(0, R // rq + 1)) * rq
        r1 = int(rng.integers(r0, R + 1))
        c0 = int(rng.integers(0, C // cq + 1)) * cq
        wmax = (C - c0) // wq
        c1 = c0 + int(rng.integers(0, wmax + 1)) * wq
        out += [((r0, r1), None), ((r0, r1), (c0, c1)), (None, (c0, c1))]
    if C >= 32 and o.kind not in ("FP8_BLOCK128",):
        out.append(((0, min(R, 3)), (0, C // 2 // wq * wq)))
    return out


@pytest.mark.parametrize("strided_kernel", [True, False])
@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6, 7])
def test_slices_match_the_oracle(k, strided_kernel):
    buf = synth.config_bytes(k, small=k != 1)
    want = oracle.materialize(buf)
    ix, ck = _staged(buf)
    rng = np.random.default_rng(k)
    outs = ix.outputs()
    picks = range(len(outs)) if len(outs) <= 60 else rng.choice(len(outs), 60, replace=False)
    slices = []
    for kk in picks:
        for rows, cols in _slices_for(outs[int(kk)], rng):
            slices.append((int(kk), rows, cols))
    print(f"slices c{k}: {len(slices)} (strided kernel {strided_kernel})", flush=True)
    got = ck.materialize_slices(slices, strided_kernel=strided_kernel)
    torch.cuda.synchronize()
    for (kk, rows, cols), t in zip(slices, got):
        w = _view(want[outs[kk].name])
        r0, r1 = rows if rows else (0, w.shape[0])
        c0, c1 = cols if cols else (0, w.shape[1])
        assert tuple(t.shape) == (r1 - r0, c1 - c0)
        assert np.array_equal(_bits(t).reshape(r1 - r0, c1 - c0), w[r0:r1, c0:c1]), (outs[kk].name, rows, cols)


def test_exact_only_column_slices():
    # rows of 60 (bf16) and 24 (f32) bytes break the word alignment; widths that split chunks
    rng = np.random.default_rng(9)
    b = rng.integers(0, 1 << 16, size=(7, 30), dtype=np.uint16)
    b[b & 0x7F80 == 0x7F80] = 0x3F80   # no NaN payloads in the passthrough source
    f = rng.standard_normal((5, 6)).astype(np.float32)
    h = rng.standard_normal((4, 33)).astype(np.float16)
    buf = make_file([("b", "BF16", (7, 30), b), ("f", "F32", (5, 6), f), ("h", "F16", (4, 33), h)])
    want = oracle.materialize(buf)
    ix, ck = _staged(buf)
    slices = [(0, None, (2, 9)), (0, (1, 6), (0, 30)), (1, (0, 5), (1, 4)), (2, None, (5, 30)), (2, (3, 4), (0, 33))]
    got = ck.materialize_slices(slices)
    torch.cuda.synchronize()
    names = [o.name for o in ix.outputs()]
    for (kk, rows, cols), t in zip(slices, got):
        w = _view(want[names[kk]])
        r0, r1 = rows if rows else (0, w.shape[0])
        c0, c1 = cols if cols else (0, w.shape[1])
        assert np.array_equal(_bits(t).reshape(r1 - r0, c1 - c0), w[r0:r1, c0:c1]), (names[kk], rows, cols)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_tensor_parallel_shards_reassemble(k):
    buf = synth.config_bytes(k, small=True)
    want = oracle.materialize(buf)
    ix, ck = _staged(buf)
    for kk, o in enumerate(ix.outputs()):
        if len(o.shape) != 2:
            continue
        R, C = o.shape
        q = 128 if o.kind == "FP8_BLOCK128" else 16 if o.kind == "NVFP4" else 1
        for axis, n in ((0, R), (1, C)):
            if o.kind == "FP8_BLOCK128" and n % (8 * 128):
                parts = [(b, min(n, b + 128)) for b in range(0, n, 128)]   # one shard per block row/col
            else:
                step = -(-n // 8 // q) * q if q > 1 else -(-n // 8)
                parts = [(b, min(n, b + step)) for b in range(0, n, step)]
            sl = [(kk, p, None) if axis == 0 else (kk, None, p) for p in parts]
            got = ck.materialize_slices(sl)
            torch.cuda.synchronize()
            whole = np.concatenate([_bits(t).reshape(t.shape) for t in got], axis=axis)
            assert np.array_equal(whole, want[o.name]), (o.name, axis)


@pytest.mark.parametrize("kind", ["NVFP4", "MXFP4"])
def test_interleaved_fp4_column_shards_match_the_whole_decode(kind):
    """8-way column shards of packed fp4 weights large enough that the planner interleaves them in
    many bands (index from the header alone, random bytes filled on the GPU, codes and scales free of
    NaN): every shard equals its block of the whole decode, which equals the oracle on sampled
    elements."""
    from synth.st_writer import Group, TensorSpec, layout
    m, k = 1536, 5120
    spec = [("w.weight", "U8", (m, k // 2))]
    if kind == "NVFP4":
        spec += [("w.weight_scale", "F8_E4M3", (m, k // 16)), ("w.weight_scale_2", "F32", ())]
    else:
        spec += [("w.weight_scale", "F8_E8M0", (m, k // 32))]
    lay = layout([Group([TensorSpec(n, d, s)], None) for n, d, s in spec])
    ix = st.SafeTensorIndex.from_bytes(lay.header, file_size=len(lay.header) + lay.data_size)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    gen = torch.Generator(device=DEV).manual_seed(17)
    blob = ck.blob
    b, e = lay.offsets["w.weight"]
    blob[b:e] = torch.randint(0, 256, (e - b,), device=DEV, dtype=torch.uint8, generator=gen)
    sb, se = lay.offsets["w.weight_scale"]
    lo, hi = (0x08, 0x68) if kind == "NVFP4" else (115, 130)
    blob[sb:se] = torch.randint(lo, hi, (se - sb,), device=DEV, dtype=torch.uint8, generator=gen)
    if kind == "NVFP4":
        gb, ge = lay.offsets["w.weight_scale_2"]
        blob[gb:ge] = torch.tensor([0.0123], device=DEV).view(torch.uint8)
    ck.arena.view(torch.int16).fill_(0x5A5A)
    ck.materialize()
    slices = [(0, None, (c, c + k // 8)) for c in range(0, k, k // 8)]
    raw, units = ix.table_slices(slices)
    n_desc = int(np.frombuffer(raw[:8], "<u4")[1])
    assert n_desc > 8, "the shards were not split into bands"
    got = ck.materialize_slices(slices)
    torch.cuda.synchronize()
    whole = ck.tensors["w.weight"]
    for (o, _, (c0, c1)), t in zip(slices, got):
        assert torch.equal(t.view(torch.int16), whole[:, c0:c1].view(torch.int16)), (c0, c1)
    # the whole decode against the oracle on sampled elements
    h = oracle.parse_header(lay.header)
    out = oracle.classify(h)[0]
    data = blob[: lay.data_size].cpu().numpy()
    idx = np.random.default_rng(3).integers(0, m * k, 4096)
    want = oracle.decode(out, data, idx)
    g = whole.reshape(-1)[torch.from_numpy(idx).to(DEV)].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(g, want)
