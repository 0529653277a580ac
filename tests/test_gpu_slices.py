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
    slices = [(0, None, (c, c + k // 8)) for c in range(0, k, k // 8)][::-1]   # reversed: bands, not a split
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


SPLIT_KINDS = ("NVFP4", "MXFP4")   # kinds whose complete shard sets become split descriptors


def _split_sets(o):
    """Complete, in-order column shard sets (2, 4 and 8 shards) an output allows for a split."""
    if len(o.shape) != 2 or o.kind == "FP8_BLOCK128":
        return []
    R, C = o.shape
    q = 32 if o.kind in ("MXFP8", "MXFP4") else 16 if o.kind == "NVFP4" else 8
    return [[(c, c + C // n) for c in range(0, C, C // n)] for n in (2, 4, 8) if C % (n * q) == 0]


def _split_config(k):
    """Config k's bytes; the packed fp4 families at widths that split (512 columns: 2, 4 and 8 shards;
    320 columns: 2 shards), as their small forms have none."""
    if k in (4, 7):
        from synth import configs
        from synth.st_writer import build_bytes
        groups, meta, pad = (configs.nvfp4 if k == 4 else configs.mxfp4)(seed=k, layers=2, big=512, small=320)
        return build_bytes(groups, meta, pad)
    return synth.config_bytes(k, small=k != 1)


@pytest.mark.parametrize("out_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("k", [1, 2, 4, 5, 6, 7])
def test_split_shards_match_the_oracle(k, out_dtype):
    """Complete shard sets of every 2-d output that allows them (one split descriptor each: the source
    read whole, each chunk stored to its shard), through the slices instance's fast path and through
    the plain instance's per-element path, against the oracle's whole output."""
    buf = _split_config(k)
    want = oracle.materialize(buf, out_dtype)
    ix = st.SafeTensorIndex.from_bytes(buf, out_dtype=out_dtype)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.load_bytes(buf[ix.data_offset:])
    outs = ix.outputs()
    sets = [(kk, cols) for kk, o in enumerate(outs) for cols in _split_sets(o)][:120]
    assert sets, "no output allows a split"
    slices = [(kk, None, c) for kk, cols in sets for c in cols]
    raw, units = ix.table_slices(slices)
    n_desc = int(np.frombuffer(raw[:8], "<u4")[1])
    if k in (4, 7):
        assert any(outs[kk].kind in SPLIT_KINDS for kk, _ in sets), "no set of a split kind"
    # one split descriptor per set of a split kind, one descriptor per shard otherwise
    assert n_desc == sum(1 if outs[kk].kind in SPLIT_KINDS else len(cols) for kk, cols in sets), n_desc
    bits = {"f32": torch.int32}.get(out_dtype, torch.int16)
    for strided_kernel in (True, False):
        print(f"split c{k} {out_dtype}: {len(sets)} sets, {len(slices)} shards, slices instance {strided_kernel}",
              flush=True)
        got = ck.materialize_slices(slices, strided_kernel=strided_kernel)
        torch.cuda.synchronize()
        for (kk, _, (c0, c1)), t in zip(slices, got):
            w = want[outs[kk].name].reshape(outs[kk].shape[0], -1)
            g = t.view(bits).cpu().numpy().view(w.dtype)
            assert np.array_equal(g, w[:, c0:c1]), (outs[kk].name, c0, c1, strided_kernel)


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [1, 3])
@pytest.mark.parametrize("k", [4, 7])
def test_split_shards_with_larger_units(k, scale, out_dtype):
    """Complete shard sets planned with units 2^scale times the default: every unit of a split
    descriptor takes the chunk-walking path (whole units of the default size take the other), against
    the oracle's whole output."""
    buf = _split_config(k)
    want = oracle.materialize(buf, out_dtype)
    ix = st.SafeTensorIndex.from_bytes(buf, unit_log2_scale=scale, out_dtype=out_dtype)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.load_bytes(buf[ix.data_offset:])
    outs = ix.outputs()
    sets = [(kk, cols) for kk, o in enumerate(outs) for cols in _split_sets(o) if o.kind in SPLIT_KINDS][:60]
    assert sets
    slices = [(kk, None, c) for kk, cols in sets for c in cols]
    raw, units = ix.table_slices(slices)
    assert int(np.frombuffer(raw[:8], "<u4")[1]) == len(sets)
    print(f"split c{k} units x{1 << scale} {out_dtype}: {len(sets)} sets, {len(slices)} shards", flush=True)
    got = ck.materialize_slices(slices)
    torch.cuda.synchronize()
    bits = {"f32": torch.int32}.get(out_dtype, torch.int16)
    for (kk, _, (c0, c1)), t in zip(slices, got):
        w = want[outs[kk].name].reshape(outs[kk].shape[0], -1)
        assert np.array_equal(t.view(bits).cpu().numpy().view(w.dtype), w[:, c0:c1]), (outs[kk].name, c0, c1)


def test_split_shards_with_misaligned_outputs():
    """A shard whose output is 2 bytes off a 16-byte boundary takes the per-element path; the other
    shards of the set keep the fast path; all equal the oracle."""
    buf = _split_config(4)
    want = oracle.materialize(buf)
    ix, ck = _staged(buf)
    outs = ix.outputs()
    kk = next(j for j, o in enumerate(outs) if _split_sets(o) and len(_split_sets(o)[-1]) == 8)
    o = outs[kk]
    cols = _split_sets(o)[-1]
    slices = [(kk, None, c) for c in cols]
    R = o.shape[0]
    sizes = [R * (c1 - c0) for c0, c1 in cols]
    arena = torch.full((sum(sizes) + 8 * 16,), float("nan"), dtype=torch.bfloat16, device=DEV)
    ptrs, views, pos = [], [], 8
    for i, n in enumerate(sizes):
        off = pos + (1 if i == 3 else 0)                     # shard 3 sits 2 bytes off 16
        ptrs.append(arena.data_ptr() + 2 * off)
        views.append(arena[off: off + n])
        pos = off + n + 8 - (off + n) % 8 + 8
    raw, units = ix.table_slices(slices)
    table = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(DEV)
    p = torch.tensor(ptrs, dtype=torch.int64, device=DEV)
    st.materialize(ck.blob, table, units, p, slices=True)
    torch.cuda.synchronize()
    w = want[o.name].reshape(R, -1)
    for (c0, c1), v in zip(cols, views):
        assert np.array_equal(_bits(v).reshape(R, c1 - c0), w[:, c0:c1]), (c0, c1)


def test_split_fp4_shards_of_a_large_weight():
    """Complete 8-way shard sets of large NVFP4 and MXFP4 weights (many full units; index from the
    header, random bytes on the GPU): one split descriptor each, every shard equal to its block of the
    whole decode."""
    from synth.st_writer import Group, TensorSpec, layout
    m, k = 1536, 5120
    spec = [("a.weight", "U8", (m, k // 2)), ("a.weight_scale", "F8_E4M3", (m, k // 16)), ("a.weight_scale_2", "F32", ()),
            ("b.weight", "U8", (m, k // 2)), ("b.weight_scale", "F8_E8M0", (m, k // 32))]
    lay = layout([Group([TensorSpec(n, d, s_)], None) for n, d, s_ in spec])
    ix = st.SafeTensorIndex.from_bytes(lay.header, file_size=len(lay.header) + lay.data_size)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    gen = torch.Generator(device=DEV).manual_seed(23)
    for name, (lo, hi) in (("a.weight", (0, 256)), ("b.weight", (0, 256)), ("a.weight_scale", (0x08, 0x68)),
                           ("b.weight_scale", (115, 130))):
        b, e = lay.offsets[name]
        ck.blob[b:e] = torch.randint(lo, hi, (e - b,), device=DEV, dtype=torch.uint8, generator=gen)
    gb, ge = lay.offsets["a.weight_scale_2"]
    ck.blob[gb:ge] = torch.tensor([0.0171], device=DEV).view(torch.uint8)
    ck.materialize()
    outs = ix.outputs()
    slices = [(j, None, (c, c + k // 8)) for j in range(2) for c in range(0, k, k // 8)]
    raw, units = ix.table_slices(slices)
    assert int(np.frombuffer(raw[:8], "<u4")[1]) == 2
    got = ck.materialize_slices(slices)
    torch.cuda.synchronize()
    for (j, _, (c0, c1)), t in zip(slices, got):
        whole = ck.tensors[outs[j].name]
        assert torch.equal(t.view(torch.int16), whole[:, c0:c1].view(torch.int16)), (j, c0, c1)
