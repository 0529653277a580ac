"""Slice tables on the CPU (st_index_table_slices): matrix views, descriptor fields of row and
column slices of every kind, the exact-only flag, and the cuts that are refused."""
import numpy as np
import pytest

import synth
import device_checkpoint_dequantisation_amd as st
from device_checkpoint_dequantisation_amd import _lib
from tests.st_files import f32_bytes, make_file
from tests.test_index import _table


@pytest.fixture(scope="module")
def ix3():
    return st.SafeTensorIndex.from_bytes(synth.config_bytes(3, small=True))


def _k(ix, name):
    return next(k for k, o in enumerate(ix.outputs()) if o.name == name)


def test_matrix_views():
    buf = make_file([("s", "BF16", (), b"\0\0"), ("v", "BF16", (10,), b"\0" * 20),
                     ("t", "BF16", (2, 3, 4), b"\0" * 48), ("z", "BF16", (0, 5), b"")])
    ix = st.SafeTensorIndex.from_bytes(buf)
    assert ix.slice_shape(_k(ix, "s")) == (1, 1)
    assert ix.slice_shape(_k(ix, "v")) == (10, 1) and ix.slice_shape(_k(ix, "v"), (2, 7)) == (5, 1)
    assert ix.slice_shape(_k(ix, "t")) == (2, 12) and ix.slice_shape(_k(ix, "t"), (1, 2), (4, 10)) == (1, 6)
    assert ix.slice_shape(_k(ix, "z")) == (0, 5)


def test_row_and_column_slice_descriptors(ix3):
    ents = ix3.tensors()
    q = _k(ix3, "model.layers.0.self_attn.q_proj.weight")      # FP8_BLOCK128 [320, 320]
    emb = _k(ix3, "model.embed_tokens.weight")                   # BF16 [1000, 320]
    o_q, o_e = ix3.output(q), ix3.output(emb)
    raw, units = ix3.table_slices([(q, (128, 320), None), (q, (0, 320), (128, 256)), (emb, (10, 20), (3, 11)),
                                   (emb, (5, 6), None)])
    h, d, m = _table(raw)
    gc = -(-320 // 128)
    # row slice of block FP8: contiguous, scale grid advanced by one block row
    assert d[0]["pitch"] == 0 and d[0]["flags"] == 0 and d[0]["cols"] == 320
    assert d[0]["src"] == ents[o_q.tensor].begin + 128 * 320
    assert d[0]["scale"] == ents[o_q.scale].begin + 4 * (1 * gc)
    # column slice of block FP8: pitch = row length, width = 128, grid advanced by one block column
    assert d[1]["pitch"] == 320 and d[1]["cols"] == 128 and d[1]["flags"] == 0 and d[1]["grid_cols"] == gc
    assert d[1]["src"] == ents[o_q.tensor].begin + 128 and d[1]["scale"] == ents[o_q.scale].begin + 4
    # a bf16 column slice 8 wide: whole chunks, rows of 640 bytes: fast path
    assert d[2]["pitch"] == 320 and d[2]["cols"] == 8 and d[2]["flags"] == 0
    assert d[2]["src"] == ents[o_e.tensor].begin + 2 * (10 * 320 + 3)
    assert d[3]["pitch"] == 0 and d[3]["src"] == ents[o_e.tensor].begin + 2 * 5 * 320
    assert units == 60 + 40 + 1 + 1   # 1024-element units: 61440, 40960, 80 and 320 elements
    numels = [192 * 320, 320 * 128, 10 * 8, 320]
    from tests.test_index import _check_map
    _check_map(d, m, units, numels)


def test_exact_only_when_chunks_would_split():
    w = np.arange(6 * 30, dtype=np.uint16)
    buf = make_file([("b", "BF16", (6, 30), w), ("f", "F32", (4, 6), np.arange(24, dtype=np.float32))])
    ix = st.SafeTensorIndex.from_bytes(buf)
    raw, _ = ix.table_slices([(0, None, (0, 8)), (0, None, (2, 9)), (1, None, (0, 3))])
    _, d, _ = _table(raw)
    # bf16 rows of 60 bytes are not whole 16-byte words: exact only, whatever the width
    assert d[0]["flags"] == _lib.DESC_EXACT and d[1]["flags"] == _lib.DESC_EXACT
    assert d[2]["flags"] == _lib.DESC_EXACT   # width 3 is not a whole 8-element chunk


def test_nvfp4_slices():
    ix = st.SafeTensorIndex.from_bytes(synth.config_bytes(4, small=True))
    k, o = next((k, o) for k, o in enumerate(ix.outputs()) if o.kind == "NVFP4")
    ents = ix.tensors()
    M, K = o.shape
    raw, _ = ix.table_slices([(k, (3, 9), (16, 48))])
    _, d, _ = _table(raw)
    first = 3 * K + 16
    assert d[0]["pitch"] == K and d[0]["cols"] == 32 and d[0]["flags"] == 0
    assert d[0]["src"] == ents[o.tensor].begin + first // 2 and d[0]["scale"] == ents[o.scale].begin + first // 16
    with pytest.raises(st.StError, match="multiples of 16"):
        ix.table_slices([(k, None, (8, 40))])
    with pytest.raises(st.StError, match="multiples of 16"):
        ix.table_slices([(k, None, (16, 40))])


@pytest.mark.parametrize("k,kind", [(6, "MXFP8"), (7, "MXFP4")])
def test_mx_slices(k, kind):
    ix = st.SafeTensorIndex.from_bytes(synth.config_bytes(k, small=True))
    kk, o = next((kk, o) for kk, o in enumerate(ix.outputs()) if o.kind == kind)
    ents = ix.tensors()
    M, K = o.shape
    raw, _ = ix.table_slices([(kk, (3, 9), (32, 96)), (kk, (5, 7), None)])
    _, d, _ = _table(raw)
    first = 3 * K + 32
    nbits = 8 if kind == "MXFP8" else 4
    assert d[0]["pitch"] == K and d[0]["cols"] == 64 and d[0]["flags"] == 0
    assert d[0]["src"] == ents[o.tensor].begin + first * nbits // 8
    assert d[0]["scale"] == ents[o.scale].begin + first // 32
    assert d[1]["pitch"] == 0 and d[1]["scale"] == ents[o.scale].begin + 5 * K // 32
    for cols in ((16, 48), (32, 48)):
        with pytest.raises(st.StError, match="multiples of 32"):
            ix.table_slices([(kk, None, cols)])


def test_refused_cuts(ix3):
    q = _k(ix3, "model.layers.0.self_attn.q_proj.weight")
    with pytest.raises(st.StError, match="multiples of 128"):
        ix3.table_slices([(q, (64, 320), None)])
    with pytest.raises(st.StError, match="multiples of 128"):
        ix3.table_slices([(q, None, (100, 200))])
    with pytest.raises(st.StError, match="outside"):
        ix3.table_slices([(q, (0, 321), None)])
    with pytest.raises(st.StError, match="outside"):
        ix3.table_slices([(q, (10, 5), None)])
    with pytest.raises(st.StError, match="ST_E_ARG"):
        ix3.table_slices([(10 ** 6, None, None)])
    ix3.table_slices([(q, (128, 128), None)])   # empty slices are fine


def _header_index(spec):
    """An index built from a header alone (no data bytes needed for planning)."""
    from synth.st_writer import Group, TensorSpec, layout
    lay = layout([Group([TensorSpec(n, d, sh)], None) for n, d, sh in spec])
    return st.SafeTensorIndex.from_bytes(lay.header, file_size=len(lay.header) + lay.data_size)


SIBLING_CASES = {
    "nvfp4": [("w.weight", "U8", (4096, 2560)), ("w.weight_scale", "F8_E4M3", (4096, 320)), ("w.weight_scale_2", "F32", ()),
              ("b.weight", "BF16", (100,))],
    "mxfp4": [("w.weight", "U8", (2048, 4096)), ("w.weight_scale", "F8_E8M0", (2048, 256)), ("b.weight", "BF16", (100,))],
    "fp8": [("w.weight", "F8_E4M3", (4096, 3072)), ("w.scale_weight", "F32", ()), ("b.weight", "BF16", (100,))],
    "mxfp8": [("w.weight", "F8_E4M3", (2048, 4096)), ("w.weight_scale", "F8_E8M0", (2048, 128)), ("b.weight", "BF16", (100,))],
    "bf16": [("w.weight", "BF16", (1024, 2048)), ("b.weight", "BF16", (100,))],
}
SPLIT_CASES = ("mxfp4", "nvfp4")   # the kinds whose complete shard sets are split


def _descs_by_out(d):
    return [int(r["out"]) for r in d]


@pytest.mark.parametrize("case", SPLIT_CASES)
def test_complete_shard_sets_become_split_descriptors(case):
    """Every column shard of a weight, equal widths, in column order, listed together: one split
    descriptor (source rows read whole, shard s written to outs[out + s]) covering the shards' units;
    other slices keep their own descriptors in request order."""
    ix = _header_index(SIBLING_CASES[case])
    o = ix.output(0)
    C = o.shape[1]
    for n in (2, 4, 8):
        W = C // n
        slices = [(1, None, None)] + [(0, None, (c, c + W)) for c in range(0, C, W)] + [(0, (0, 3), None)]
        raw, units = ix.table_slices(slices)
        h, d, m = _table(raw)
        assert len(d) == 3 and _descs_by_out(d) == [0, 1, n + 1]
        sd = d[1]
        assert sd["flags"] == _lib.DESC_SPLIT and sd["pitch"] == C and sd["cols"] == W
        assert sd["grid_cols"] == n.bit_length() - 1
        R = o.shape[0]
        shift = int(sd["unit_shift"])
        _, whole, _ = _table(ix.table_slices([(0, None, None)])[0])
        assert shift == int(whole[0]["unit_shift"])
        assert int(sd["unit_end"]) - int(sd["unit_begin"]) == -(-R * C // (1 << shift))
        ents = ix.tensors()
        assert sd["src"] == ents[o.tensor].begin            # whole rows from the first
        # the unit map still points every group at the descriptor holding its first unit
        ends = d["unit_end"].astype(np.int64)
        starts = np.concatenate([[0], ends[:-1]])
        for g, di in enumerate(m):
            assert starts[di] <= g * _lib.UNITS_PER_GROUP < ends[di]


@pytest.mark.parametrize("case", sorted(SIBLING_CASES))
def test_shards_that_are_not_a_complete_set_interleave_or_keep_order(case):
    """Shards listed in reverse order, or three of a weight, are not split: packed fp4 siblings
    interleave band by band, other kinds keep the request order; each slice's units are covered
    exactly once with the right element offsets."""
    from tests.test_index import _check_map
    ix = _header_index(SIBLING_CASES[case])
    o = ix.output(0)
    kind, cols = o.kind, o.shape[1]
    step = cols // 8
    for slices in ([(0, None, (c, c + step)) for c in range(0, cols, step)][::-1],
                   [(0, None, (c, c + step)) for c in range(0, 3 * step, step)]):
        slices = slices + [(1, None, None)]
        raw, units = ix.table_slices(slices)
        h, d, m = _table(raw)
        numels = [ix.slice_shape(*sl)[0] * ix.slice_shape(*sl)[1] for sl in slices]
        _check_map(d, m, units, numels)
        assert not any(int(r["flags"]) & _lib.DESC_SPLIT for r in d)
        outs = _descs_by_out(d)
        nsh = len(slices) - 1
        if kind in ("NVFP4", "MXFP4"):
            assert outs[: 2 * nsh] == list(range(nsh)) * 2     # band 0 of every shard, then band 1
            shard_units = -(-numels[0] // (1 << int(d[0]["unit_shift"])))
            assert len(d) == nsh * -(-shard_units // 16) + 1
        else:
            assert outs == list(range(len(slices)))


@pytest.mark.parametrize("case", ["block_fp8", "bf16", "fp8", "mxfp8"])
def test_other_kinds_keep_one_descriptor_per_shard(case):
    """Complete shard sets of the kinds outside the split set (block FP8, bf16, scaled FP8, MXFP8)
    keep one descriptor per shard, in request order."""
    spec = ([("w.weight", "F8_E4M3", (1024, 2048)), ("w.weight_scale_inv", "F32", (8, 16))] if case == "block_fp8"
            else SIBLING_CASES[case])
    ix = _header_index(spec)
    C = ix.output(0).shape[1]
    slices = [(0, None, (c, c + C // 8)) for c in range(0, C, C // 8)]
    raw, units = ix.table_slices(slices)
    h, d, m = _table(raw)
    assert len(d) == 8 and not any(int(r["flags"]) & _lib.DESC_SPLIT for r in d)
    assert _descs_by_out(d) == list(range(8))


def _full_header_index(k):
    """The index of benchmark config k at full size, built from its header alone."""
    from synth.st_writer import layout
    groups, meta, pad = synth.make_config(k)
    lay = layout(groups, meta, pad)
    return st.SafeTensorIndex.from_bytes(lay.header, file_size=len(lay.header) + lay.data_size)


SOURCE_BITS = {0: 16, 1: 16, 2: 32, 3: 8, 4: 8, 5: 4, 6: 8, 7: 4}


def _eighth_bytes(d, units):
    """Bytes (source + 2-byte output per element) of each eighth of the unit sequence."""
    ends = d["unit_end"].astype(np.int64)
    starts = np.concatenate([[0], ends[:-1]])
    e = np.zeros(8)
    for row, a, b in zip(d, starts, ends):
        per = (1 << int(row["unit_shift"])) * (SOURCE_BITS[int(row["kind"])] / 8 + 2)
        for x in range(8):
            lo, hi = max(a, units * x // 8), min(b, units * (x + 1) // 8)
            if hi > lo:
                e[x] += per * (hi - lo)
    return e


@pytest.mark.parametrize("axis", [0, 1])
def test_slice_tables_balance_the_xcd_eighths(axis):
    """8-way shards of every 2-d output of the block-FP8 checkpoint (fp8 layers and a bf16 embedding
    of more bytes per unit): in request order one eighth would carry the embedding's shards; the
    planner cuts every large slice into 8 pieces, one per eighth, so the eighths carry equal bytes,
    and every slice's units are still covered once with the kernel's unit offsets intact."""
    from tests.test_index import _check_map
    ix = _full_header_index(3)
    slices = []
    for k, o in enumerate(ix.outputs()):
        if len(o.shape) != 2:
            slices.append((k, None, None))
            continue
        dim = o.shape[axis]
        q = 128 if o.kind == "FP8_BLOCK128" else 1
        step = max(q, -(-dim // 8 // q) * q)
        for b in range(0, dim, step):
            part = (b, min(dim, b + step))
            slices.append((k, part, None) if axis == 0 else (k, None, part))
    raw, units = ix.table_slices(slices)
    h, d, m = _table(raw)
    assert len(d) > len(slices)                      # large slices were cut into pieces
    numels = [int(np.prod(ix.slice_shape(*sl))) for sl in slices]
    _check_map(d, m, units, numels)
    e = _eighth_bytes(d, units)
    assert e.max() / e.mean() < 1.01, e / e.mean()


def test_balanced_slice_tables_keep_request_order():
    """Homogeneous shard tables (the scaled-FP8 checkpoint's row shards) are balanced already and keep
    one descriptor per slice in request order."""
    ix = _full_header_index(2)
    slices = []
    for k, o in enumerate(ix.outputs()):
        if len(o.shape) != 2:
            slices.append((k, None, None))
            continue
        R = o.shape[0]
        slices += [(k, (b, min(R, b + R // 8)), None) for b in range(0, R, R // 8)]
    raw, units = ix.table_slices(slices)
    h, d, m = _table(raw)
    assert len(d) == len(slices) and [int(r["out"]) for r in d] == list(range(len(slices)))
