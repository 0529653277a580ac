"""Host-side tests of libstmat (no GPU): exported symbols, the C index against the oracle's
parse and classification, descriptor-table invariants, and malformed-input rejection."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
import synth
import device_checkpoint_dequantisation_amd as st
from device_checkpoint_dequantisation_amd import _lib
from tests.st_files import f32_bytes, make_file, raw_header_file
from tests.test_oracle_format import BAD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    text = open(os.path.join(ROOT, "include", "stmat.h")).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    declared = set(re.findall(r"\b(st_[a-z_0-9]+)\s*\(", text))
    assert declared, "no declarations found"
    lib = C.CDLL(_lib.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), f"{name} is declared in stmat.h but not exported"
    assert declared == set(_lib.SIGNATURES), "Python signatures out of sync with stmat.h"


def _index(buf):
    return st.SafeTensorIndex.from_bytes(buf)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6, 7])
def test_index_matches_oracle_on_configs(k):
    buf = synth.config_bytes(k, small=True)
    h, outs = oracle.plan(buf)
    ix = _index(buf)
    assert ix.data_offset == h.data_offset and ix.data_size == h.data_size
    ents = ix.tensors()
    assert [e.name for e in ents] == list(h.entries)
    for e in ents:
        o = h.entries[e.name]
        assert (e.dtype, e.shape, e.begin, e.end) == (o.dtype, o.shape, o.begin, o.end)
    couts = ix.outputs()
    assert [c.name for c in couts] == [o.name for o in outs]
    for c, o in zip(couts, outs):
        assert c.kind == o.kind and c.shape == o.shape and c.numel == o.numel
        assert ents[c.tensor].name == o.src.name
        assert (ents[c.scale].name if c.scale >= 0 else None) == (o.scale.name if o.scale else None)
        assert (ents[c.scale2].name if c.scale2 >= 0 else None) == (o.scale2.name if o.scale2 else None)
    assert ix.metadata == h.metadata
    assert ix.traffic_bytes == h.data_size + 2 * sum(o.numel for o in outs)


def test_tiny_traffic_is_the_documented_figure():
    ix = _index(synth.config_bytes(1))
    assert ix.data_size == 718_856 and ix.traffic_bytes == 718_856 + 913_408


STEP_SHIFT = {"PASS_BF16": 10, "CAST_F16": 10, "CAST_F32": 9, "FP8_TENSOR": 10, "FP8_BLOCK128": 10, "NVFP4": 11,
              "MXFP8": 10, "MXFP4": 11}


def step_shift(kind, out_dtype):
    """Default unit size (log2 elements): packed fp4 into fp32 outputs uses 1024-element units."""
    if kind in ("NVFP4", "MXFP4") and out_dtype == "f32":
        return 10
    return STEP_SHIFT[kind]

DESC = np.dtype([("src", "<u8"), ("scale", "<u8"), ("scale2", "<u8"), ("pitch", "<u4"), ("flags", "<u4"),
                 ("unit_begin", "<u4"),
                 ("unit_end", "<u4"), ("tail", "<u4"), ("out", "<u4"), ("cols", "<u4"), ("grid_cols", "<u4"),
                 ("div_magic", "<u4"), ("kind", "u1"), ("unit_shift", "u1"), ("div_shift", "u1"), ("r0", "u1")])
HEADER = np.dtype([("magic", "<u4"), ("n_desc", "<u4"), ("units", "<u8"), ("desc_offset", "<u8"),
                   ("map_offset", "<u8"), ("bytes", "<u8"), ("out_dtype", "<u4"), ("flags", "<u4"),
                   ("reserved", "<u8", 2)])


def _table(raw: bytes):
    h = np.frombuffer(raw, HEADER, count=1)[0]
    assert h["magic"] == _lib.TABLE_MAGIC and h["bytes"] == len(raw) and len(raw) % 64 == 0
    groups = -(-int(h["units"]) // _lib.UNITS_PER_GROUP)
    assert h["map_offset"] == 64 and h["desc_offset"] == 64 + -(-groups * 4 // 64) * 64
    d = np.frombuffer(raw, DESC, count=int(h["n_desc"]), offset=int(h["desc_offset"]))
    m = np.frombuffer(raw, "<u4", count=groups, offset=int(h["map_offset"]))
    return h, d, m


def _check_map(d, m, units, numels):
    """Table invariants: descriptors cover consecutive ranges of the unit sequence; each output's
    pieces (one descriptor each, or one for the whole output) cover its units exactly once, and
    the kernel's element offset (unit - unit_begin) << shift (modulo 2^32) lands on the right
    units; only the piece holding an output's last unit ends in its partial tail; every group of 4
    units maps to the descriptor holding its first unit."""
    numels = np.asarray(numels, dtype=np.int64)
    ends = d["unit_end"].astype(np.int64)
    starts = np.concatenate([[0], ends[:-1]])
    assert np.all(ends >= starts)
    covered = {}
    for i, row in enumerate(d):
        sh, out = int(row["unit_shift"]), int(row["out"])
        n = int(numels[out])
        nu = -(-n // (1 << sh))
        first = (int(starts[i]) - int(row["unit_begin"])) % (1 << 32)
        count = int(ends[i] - starts[i])
        assert first + count <= nu, (i, first, count, nu)
        covered.setdefault(out, []).append((first, count))
        if count:
            last = first + count == nu
            want_tail = n - ((nu - 1) << sh) if last else 1 << sh
            assert row["tail"] == want_tail and 1 <= row["tail"] <= 1 << sh, (i, int(row["tail"]), want_tail)
    for out, parts in covered.items():
        parts.sort()
        pos = 0
        for first, count in parts:
            assert first == pos, (out, parts)
            pos += count
        n = int(numels[out])
        assert pos == -(-n // (1 << int(d[[int(r["out"]) for r in d].index(out)]["unit_shift"])))
    for g, di in enumerate(m):
        u = g * _lib.UNITS_PER_GROUP
        assert starts[di] <= u < ends[di], (g, di)
    assert ends.max(initial=0) == units


@pytest.mark.parametrize("k,out_dtype", [(3, "bf16"), (4, "bf16"), (7, "f16"), (4, "f32"), (7, "f32"), (2, "f32")])
@pytest.mark.parametrize("scale", [0, 2])
def test_table_invariants(scale, k, out_dtype):
    buf = synth.config_bytes(k, small=True)
    ix = st.SafeTensorIndex.from_bytes(buf, unit_log2_scale=scale, out_dtype=out_dtype)
    esize = 4 if out_dtype == "f32" else 2
    raw, units = ix.table()
    h, d, m = _table(raw)
    outs = ix.outputs()
    ents = ix.tensors()
    assert h["units"] == units and h["n_desc"] == len(outs) == len(d)
    pos = 0
    for k, (row, o) in enumerate(zip(d, outs)):
        assert row["out"] == k and row["pitch"] == 0 and row["flags"] == 0 and _lib.KINDS[row["kind"]] == o.kind
        assert row["src"] == ents[o.tensor].begin
        if o.scale >= 0:
            assert row["scale"] == ents[o.scale].begin
        if o.scale2 >= 0:
            assert row["scale2"] == ents[o.scale2].begin
        assert row["unit_shift"] == step_shift(o.kind, out_dtype) + scale
        assert row["unit_begin"] == pos
        pos += -(-o.numel // (1 << int(row["unit_shift"])))
        if o.kind == "FP8_BLOCK128":
            assert row["cols"] == o.shape[1] and row["grid_cols"] == -(-o.shape[1] // 128)
    assert pos == units
    _check_map(d, m, units, [o.numel for o in outs])
    # arena: 256-byte aligned, disjoint, in order
    offs = [o.offset for o in outs]
    assert all(x % 256 == 0 for x in offs)
    assert all(offs[i] + esize * outs[i].numel <= offs[i + 1] for i in range(len(offs) - 1))
    assert ix.arena_bytes >= offs[-1] + esize * outs[-1].numel
    assert ix.blob_bytes % 256 == 0 and ix.blob_bytes >= ix.data_size
    assert ix.device_bytes >= ix.blob_bytes + ix.arena_bytes + len(raw)


def test_map_with_empty_and_tiny_outputs():
    f = make_file([("e", "BF16", (0,), b""), ("a", "F32", (3,), f32_bytes(1, 2, 3)), ("z", "F16", (0, 7), b""),
                   ("b", "BF16", (2000,), b"\0" * 4000), ("c", "BF16", (1,), b"\0\0"), ("y", "BF16", (0,), b"")])
    ix = st.SafeTensorIndex.from_bytes(f)
    raw, units = ix.table()
    h, d, m = _table(raw)
    assert units == 1 + 2 + 1
    _check_map(d, m, units, [o.numel for o in ix.outputs()])
    raw, units = st.SafeTensorIndex.from_bytes(make_file([])).table()
    h, d, m = _table(raw)
    assert units == 0 and len(d) == 0 and len(m) == 0


@pytest.mark.parametrize("cols", [1, 2, 3, 7, 100, 127, 128, 129, 200, 300, 4096, 12288, 65535, 999983, 2 ** 31 - 1,
                                  2 ** 31, 2 ** 31 + 1, 2 ** 32 - 1])
def test_block_division_constants_give_exact_quotients(cols):
    # The planner stores (magic, shift) for dividing a 32-bit element index by the width N; the
    # quotient rule is checked against exact integer division on edge and random numerators.
    hdr = ('{"w.weight":{"dtype":"F8_E4M3","shape":[%d,%d],"data_offsets":[0,0]},'
           '"w.weight_scale_inv":{"dtype":"F32","shape":[%d,%d],"data_offsets":[0,0]}}')
    # a zero-row weight keeps the file empty while the planner still derives the constants
    f = raw_header_file(hdr % (0, cols, 0, -(-cols // 128)))
    d = _table(_index(f).table()[0])[1][0]
    m, l = int(d["div_magic"]), int(d["div_shift"])
    rng = np.random.default_rng(cols)
    ns = [0, 1, cols - 1, cols, cols + 1, 2 ** 32 - 1, 2 ** 32 - 2, (2 ** 32 - 1) // cols * cols,
          (2 ** 32 - 1) // cols * cols - 1] + rng.integers(0, 2 ** 32, 2000).tolist()
    for n in ns:
        n %= 2 ** 32
        t = (m * n) >> 32
        q = n if l == 0 else (t + ((n - t) >> 1)) >> (l - 1)
        assert q == n // cols, (cols, n)


def test_subset_table_is_self_contained():
    buf = synth.config_bytes(5, small=True)
    ix = _index(buf)
    full = _table(ix.table()[0])[1]
    sel = [7, 3, 100, 3]
    raw, units = ix.table_subset(sel)
    h, d, m = _table(raw)
    assert h["n_desc"] == 4
    pos = 0
    outs = ix.outputs()
    for j, s in enumerate(sel):
        assert d[j]["out"] == j and d[j]["src"] == full[s]["src"] and d[j]["unit_end"] - d[j]["unit_begin"] == \
            full[s]["unit_end"] - full[s]["unit_begin"] and d[j]["tail"] == full[s]["tail"]
        assert d[j]["unit_begin"] == pos
        pos += -(-outs[s].numel // (1 << int(d[j]["unit_shift"])))
    assert units == pos
    _check_map(d, m, units, [outs[s].numel for s in sel])
    with pytest.raises(st.StError):
        ix.table_subset([10 ** 6])


@pytest.mark.parametrize("case", sorted(BAD))
def test_index_rejects_what_the_oracle_rejects(case):
    with pytest.raises(st.StError):
        _index(BAD[case])


def test_header_size_and_open(tmp_path):
    buf = synth.config_bytes(1)
    p = tmp_path / "c1.safetensors"
    p.write_bytes(buf)
    ix = st.SafeTensorIndex.open(str(p))
    assert ix.data_offset == oracle.parse_header(buf).data_offset
    n = C.c_uint64()
    assert _lib.lib().st_header_size(buf[:8], C.byref(n)) == 0 and n.value == ix.data_offset
    with pytest.raises(st.StError):
        st.SafeTensorIndex.open(str(tmp_path / "missing.safetensors"))
    (tmp_path / "trunc.safetensors").write_bytes(buf[:100])
    with pytest.raises(st.StError):
        st.SafeTensorIndex.open(str(tmp_path / "trunc.safetensors"))


def test_errors_name_the_tensor():
    f = make_file([("w.weight", "F8_E4M3", (4,), b"\0" * 4)])
    with pytest.raises(st.StError, match=r"ST_E_SCALE.*w\.weight"):
        _index(f)


def test_bad_options_rejected():
    with pytest.raises(st.StError):
        st.SafeTensorIndex.from_bytes(raw_header_file("{}"), unit_log2_scale=9)


def _mutations(buf: bytes, rng, count):
    n = int.from_bytes(buf[:8], "little")
    hdr = bytearray(buf[8:8 + n])
    data = buf[8 + n:]
    for _ in range(count):
        h = bytearray(hdr)
        for _ in range(int(rng.integers(1, 4))):
            op = int(rng.integers(3))
            i = int(rng.integers(len(h)))
            if op == 0:
                h[i] = int(rng.choice(list(b'{}[]":,0123456789-.eE \\u')))
            elif op == 1:
                del h[i]
            else:
                h.insert(i, int(rng.choice(list(b'{}[]":,09-'))))
        yield len(h).to_bytes(8, "little") + bytes(h) + data


MUTATION_BASES = {
    "fp8": make_file([("a.weight", "F8_E4M3", (2, 3), b"\x01" * 6), ("a.scale_weight", "F32", (), f32_bytes(0.5)),
                      ("b", "BF16", (2,), b"\0" * 4), ("c", "F16", (1, 1), b"\0\0")], metadata={"x": "y"}),
    "mx": make_file([("a.weight", "F8_E4M3", (2, 32), b"\x01" * 64), ("a.weight_scale", "F8_E8M0", (2, 1), b"\x7f" * 2),
                     ("m.weight", "U8", (1, 16), b"\x21" * 16), ("m.weight_scale", "F8_E8M0", (1, 1), b"\x80")]),
}


@pytest.mark.parametrize("base", sorted(MUTATION_BASES))
def test_random_header_mutations_accept_and_reject_alike(base):
    # The C reader and the oracle must agree on acceptance for corrupted headers and, when both
    # accept, on the parsed entries.
    base = MUTATION_BASES[base]
    rng = np.random.default_rng(11)
    agree = accepted = 0
    for m in _mutations(base, rng, 600):
        try:
            h, outs = oracle.plan(m)
            ok_o = True
        except oracle.OracleError:
            ok_o = False
        try:
            ix = _index(m)
            ok_c = True
        except st.StError:
            ok_c = False
        assert ok_o == ok_c, m[8:]
        agree += 1
        if ok_c:
            accepted += 1
            assert [e.name for e in ix.tensors()] == list(h.entries)
            assert [o.name for o in ix.outputs()] == [o.name for o in outs]
    assert agree == 600


@pytest.mark.parametrize("dt,esize,code", [("bf16", 2, 0), ("f16", 2, 1), ("f32", 4, 2)])
def test_output_types_size_the_arena_and_mark_the_tables(dt, esize, code):
    buf = synth.config_bytes(5, small=True)
    ix = st.SafeTensorIndex.from_bytes(buf, out_dtype=dt)
    outs = ix.outputs()
    assert ix.out_dtype == dt
    offs = [o.offset for o in outs]
    assert all(x % 256 == 0 for x in offs)
    assert all(offs[i] + esize * outs[i].numel <= offs[i + 1] for i in range(len(offs) - 1))
    assert ix.traffic_bytes == ix.data_size + esize * sum(o.numel for o in outs)
    for raw in (ix.table()[0], ix.table_subset([1, 2])[0], ix.table_slices([(3, None, None)])[0]):
        assert _table(raw)[0]["out_dtype"] == code
    plan = st.StreamPlan(ix, 64 << 10)
    for step in plan.steps:
        if step.outputs:
            assert np.frombuffer(plan.tables, HEADER, count=1, offset=step.table_offset)[0]["out_dtype"] == code


def test_bad_plan_options_are_refused():
    buf = synth.config_bytes(1)
    with pytest.raises(st.StError, match="ST_E_ARG"):
        _build(buf, 3, 0)
    with pytest.raises(st.StError, match="ST_E_ARG"):
        _build(buf, 4, 0)
    with pytest.raises(st.StError, match="ST_E_ARG"):
        _build(buf, 0, 7)


def _build(buf, flags, scale):
    import ctypes as C
    h = C.c_void_p()
    opts = _lib.PlanOpts(scale, flags)
    raw = C.create_string_buffer(bytes(buf), len(buf))
    st.check(_lib.lib().st_index_build(raw, len(buf), len(buf), C.byref(opts), C.byref(h)), "st_index_build")


def test_mx_rejections_match_the_oracle():
    from tests.test_oracle_mx import test_mx_malformed_is_rejected as case
    for mark in case.pytestmark:
        if mark.name == "parametrize":
            for tensors, _ in mark.args[1]:
                buf = make_file(tensors)
                with pytest.raises(oracle.OracleError):
                    oracle.plan(buf)
                with pytest.raises(st.StError):
                    _index(buf)


def test_large_outputs_are_cut_into_eight_pieces():
    """When the file-order eighths of the unit sequence carry unequal bytes (here a bf16 copy at
    4 KB per unit, then fp8 at 3 KB), outputs of at least 2048 units are cut into 8 equal pieces,
    piece p in the p-th eighth; small outputs fill the eighths in file order."""
    rng = np.random.default_rng(2)
    big_bf16 = 2048 * 1024 + 5              # 2049 units, the last one partial
    big_fp8 = 3000 * 1024                   # 3000 units
    tensors = [("a", "BF16", (big_bf16,), rng.integers(0, 2 ** 16, big_bf16, dtype=np.uint64).astype(np.uint16))]
    tensors += [(f"s{i}", "F32", (3000 + i,), rng.standard_normal(3000 + i).astype(np.float32)) for i in range(20)]
    tensors += [("q.weight", "F8_E4M3", (big_fp8,), np.full(big_fp8, 0x38, np.uint8)),
                ("q.scale_weight", "F32", (), f32_bytes(0.5))]
    buf = make_file(tensors)
    ix = _index(buf)
    raw, units = ix.table()
    h, d, m = _table(raw)
    outs = ix.outputs()
    _check_map(d, m, units, [o.numel for o in outs])
    kk = {o.name: k for k, o in enumerate(outs)}
    for name in ("a", "q.weight"):
        rows = [i for i, r in enumerate(d) if r["out"] == kk[name]]
        assert len(rows) == 8
        ends = d["unit_end"].astype(np.int64)
        starts = np.concatenate([[0], ends[:-1]])
        for p, i in enumerate(rows):          # piece p sits in eighth p of the sequence
            assert p * units // 8 - 64 <= starts[i] <= (p + 1) * units // 8, (name, p, starts[i], units)
    small = [i for i, r in enumerate(d) if outs[int(r["out"])].name.startswith("s")]
    assert [outs[int(d[i]["out"])].name for i in small] == [f"s{i}" for i in range(20)]   # file order kept
    # a subset table of the two large outputs is still unbalanced, and cut; one output alone is not
    raw, units = ix.table_subset([kk["a"], kk["q.weight"]])
    h, d, m = _table(raw)
    assert len(d) == 16 and units == 2049 + 3000
    _check_map(d, m, units, [outs[kk["a"]].numel, outs[kk["q.weight"]].numel])
    raw, units = ix.table_subset([kk["a"]])
    h, d, m = _table(raw)
    assert len(d) == 1 and units == 2049


def test_balanced_checkpoints_keep_file_order():
    # two large fp8 outputs: every eighth carries the same bytes, so nothing is cut
    n = 3000 * 1024
    buf = make_file([("a.weight", "F8_E4M3", (n,), np.full(n, 0x38, np.uint8)), ("a.scale_weight", "F32", (), f32_bytes(1.0)),
                     ("b.weight", "F8_E4M3", (n,), np.full(n, 0x38, np.uint8)), ("b.scale_weight", "F32", (), f32_bytes(1.0))])
    ix = _index(buf)
    raw, units = ix.table()
    h, d, m = _table(raw)
    assert len(d) == 2 and list(d["unit_begin"]) == [0, 3000]
    _check_map(d, m, units, [o.numel for o in ix.outputs()])


def test_launch_arguments_are_checked_before_any_gpu_call():
    """st_materialize_as (and its bf16 forms) and st_stage_file reject bad arguments with ST_E_ARG
    and a message, before touching the GPU: fake, well-aligned device addresses stand in."""
    import ctypes as C
    L = _lib.lib()
    ok = C.c_void_p(1 << 20)        # 256-byte aligned stand-ins; never dereferenced on these paths
    cases = [
        ((None, ok, 5, ok, 0, 0), "null pointer"),
        ((ok, None, 5, ok, 0, 0), "null pointer"),
        ((ok, ok, 5, None, 0, 0), "null pointer"),
        ((C.c_void_p((1 << 20) + 16), ok, 5, ok, 0, 0), "blob is not 256-byte aligned"),
        ((ok, C.c_void_p((1 << 20) + 32), 5, ok, 0, 0), "work table is not 64-byte aligned"),
        ((ok, ok, 1 << 32, ok, 0, 0), "at most 2^32 - 1"),
        ((ok, ok, 5, ok, 3, 0), "unknown output type 3"),
        ((ok, ok, 5, ok, 0, 4), "unknown flags 0x4"),
    ]
    for (blob, descs, n, outs, dt, flags), msg in cases:
        assert L.st_materialize_as(blob, descs, n, outs, dt, flags, None) == -1, msg
        assert msg.encode() in L.st_last_error(), (msg, L.st_last_error())
    # n == 0 is a no-op, whatever the pointers
    assert L.st_materialize_as(None, None, 0, None, 7, 9, None) == 0
    assert L.st_materialize(None, None, 0, None, None) == 0
    assert L.st_materialize(ok, None, 1, ok, None) == -1 and L.st_materialize_slices(None, ok, 1, ok, None) == -1
    ix = _index(synth.config_bytes(1))
    assert L.st_stage_file(b"/nonexistent", ix._h, None, ok, 1 << 30, None, None, None) == -1
    assert b"null pointer" in L.st_last_error()
    assert L.st_stage_file(b"/nonexistent", ix._h, ok, ok, 1024, None, None, None) == -1
    assert b"pinned buffer" in L.st_last_error()
    assert L.st_stage_file(b"/nonexistent", ix._h, C.c_void_p((1 << 20) + 8), ok, 1 << 30, None, None, None) == -1
    assert b"blob is not" in L.st_last_error()


@pytest.mark.parametrize("delta", [-1, 1])
def test_staging_refuses_a_file_of_the_wrong_size_before_any_gpu_call(delta, tmp_path):
    """st_stage_file and st_stream_file open the file and compare its size with the index before
    any GPU call; a file one byte shorter or longer fails with ST_E_IO and both sizes named.  A
    missing file fails the same way."""
    import ctypes as C
    L = _lib.lib()
    ok = C.c_void_p(1 << 20)        # aligned stand-ins; these paths stop before using them
    buf = synth.config_bytes(1)
    ix = _index(buf)
    p = tmp_path / "c1.safetensors"
    p.write_bytes(buf[:-1] if delta < 0 else buf + b"\0")
    want = f"the index expects {len(buf)}".encode()
    assert L.st_stage_file(str(p).encode(), ix._h, ok, ok, 1 << 30, None, None, None) == -2
    assert want in L.st_last_error() and f"{len(buf) + delta} bytes".encode() in L.st_last_error()
    plan = st.StreamPlan(ix, 1 << 20)
    assert L.st_stream_file(str(p).encode(), ix._h, plan._h, ok, ok, ok, ok, 64 << 20, None, None, None, None) == -2
    assert want in L.st_last_error()
    assert L.st_stage_file(str(tmp_path / "missing").encode(), ix._h, ok, ok, 1 << 30, None, None, None) == -2
    assert b"cannot open" in L.st_last_error()


def _header_only(k, out_dtype="bf16"):
    from synth.st_writer import layout
    lay = layout(*synth.configs.make_config(k))
    return st.SafeTensorIndex.from_bytes(lay.header, file_size=len(lay.header) + lay.data_size, out_dtype=out_dtype)


def test_tables_with_outputs_past_the_cache_ask_for_stream_stores():
    """The planner sets ST_TABLE_STREAM_STORES exactly when a table's outputs exceed 256 MiB (the
    MI355X's Infinity Cache): the large checkpoints, not the tiny or the many-small one (211 MB);
    subset and slice tables by their own outputs; each streaming step by its own."""
    limit = 256 << 20
    for k in (1, 2, 3, 4, 5, 6, 7):
        ix = _header_only(k)
        out_bytes = sum(o.numel for o in ix.outputs()) * 2
        flags = int(_table(ix.table()[0])[0]["flags"])
        assert flags == (_lib.TABLE_STREAM_STORES if out_bytes > limit else 0), (k, out_bytes, flags)
        assert st.table_stream_stores(ix.table()[0]) == (out_bytes > limit)
    ix = _header_only(4)        # 80 weights of 25600 x 5120 (250 MiB each in bf16)
    outs = ix.outputs()
    assert outs[0].numel * 2 <= limit
    assert int(_table(ix.table_subset([0])[0])[0]["flags"]) == 0
    assert int(_table(ix.table_subset([0, 1])[0])[0]["flags"]) == _lib.TABLE_STREAM_STORES
    assert int(_table(ix.table_slices([(0, None, (0, 640))])[0])[0]["flags"]) == 0
    assert int(_table(ix.table_slices([(j, None, None) for j in range(3)])[0])[0]["flags"]) == _lib.TABLE_STREAM_STORES
    ix32 = _header_only(4, "f32")    # the same weight is 500 MiB in fp32
    assert int(_table(ix32.table_subset([0])[0])[0]["flags"]) == _lib.TABLE_STREAM_STORES
