"""The streaming plan (st_stream_plan_build) on the CPU: its staging steps tile the data section,
every output is attached to the first step after which all of its input bytes are copied, each
step's work table is the subset table of its outputs, and the error paths."""
import bisect
import ctypes as C

import numpy as np
import pytest

import synth
import device_checkpoint_dequantisation_amd as st
from device_checkpoint_dequantisation_amd._lib import lib
from tests.st_files import f32_bytes, make_file

CHUNKS = [64 << 10, 100_000, 1 << 20]


def _inputs(ents, co):
    return [ents[i] for i in (co.tensor, co.scale, co.scale2) if i >= 0]


def check_plan(ix, plan):
    size = ix.data_size
    # ranges: step-major, each step within the chunk size, together tiling [0, size) once
    assert all(s.bytes <= plan.chunk_bytes for s in plan.steps)
    assert sum(s.bytes for s in plan.steps) == size
    flat = [r for s in plan.steps for r in s.ranges]
    assert flat == plan.ranges
    assert all(b < e for b, e in flat)
    cover = sorted(flat)
    pos = 0
    for b, e in cover:
        assert b == pos
        pos = e
    assert pos == size
    for s in plan.steps:
        assert sum(e - b for b, e in s.ranges) == s.bytes
    step_of_byte = sorted((b, e, k) for k, s in enumerate(plan.steps) for b, e in s.ranges)
    starts = [b for b, _, _ in step_of_byte]

    def steps_of(ent):  # steps copying any byte of the tensor
        i = bisect.bisect_right(starts, ent.begin) - 1
        out = []
        while i < len(step_of_byte) and step_of_byte[i][0] < ent.end:
            if step_of_byte[i][1] > ent.begin:
                out.append(step_of_byte[i][2])
            i += 1
        return out

    def last_step(ent):  # step that copies the tensor's last byte (-1: no bytes)
        if ent.end == ent.begin:
            return -1
        return step_of_byte[bisect.bisect_right(starts, ent.end - 1) - 1][2]

    # outputs: a permutation, each in the first step completing all its inputs
    outs = ix.outputs()
    ents = ix.tensors()
    assert sorted(plan.order) == list(range(len(outs)))
    assert [o for s in plan.steps for o in s.outputs] == plan.order
    for k, s in enumerate(plan.steps):
        for o in s.outputs:
            ins = _inputs(ents, outs[o])
            for ent in ins:
                assert all(j <= k for j in steps_of(ent)), (outs[o].name, ent.name)
            assert max([last_step(ent) for ent in ins] + [0]) == k
    # each step's table is the subset table of its outputs
    for s in plan.steps:
        if not s.outputs:
            assert s.units == 0
            continue
        table, units = ix.table_subset(list(s.outputs))
        assert plan.tables[s.table_offset: s.table_offset + len(table)] == table
        assert units == s.units
        assert s.table_offset % 64 == 0
    return step_of_byte


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("chunk", CHUNKS)
def test_plan_invariants_small_configs(k, chunk):
    ix = st.SafeTensorIndex.from_bytes(synth.config_bytes(k, small=True))
    check_plan(ix, st.StreamPlan(ix, chunk))


def test_file_order_when_scales_follow_their_weights():
    ix = st.SafeTensorIndex.from_bytes(synth.config_bytes(2, small=True))
    plan = st.StreamPlan(ix, 64 << 10)
    assert plan.ranges == sorted(plan.ranges)  # pure file order
    # a step is one contiguous range
    assert all(len(s.ranges) == 1 for s in plan.steps)


def test_scales_at_the_end_are_staged_first():
    ix = st.SafeTensorIndex.from_bytes(synth.config_bytes(2, small=True, scales_last=True))
    chunk = 64 << 10
    plan = st.StreamPlan(ix, chunk)
    check_plan(ix, plan)
    ents = {e.name: e for e in ix.tensors()}
    # scales lying more than one chunk past their weight's end are staged before everything else
    far = {n for n, e in ents.items() if n.endswith(".scale_weight")
           and e.end > ents[n[: -len(".scale_weight")] + ".weight"].end + chunk}
    assert len(far) >= 10
    early = set()
    for s in plan.steps:
        covered = {n for n in ents if any(b <= ents[n].begin and ents[n].end <= e for b, e in s.ranges)}
        if not covered <= far:
            break
        early |= covered
    assert early == far
    # so the first weights are decoded long before the file's end
    assert any(s.outputs for s in plan.steps[1: len(plan.steps) // 2])


def test_scale_far_after_weight_moves_first():
    w = (np.arange(300 * 256) % 120).astype(np.uint8)
    fill = np.zeros(100_000, dtype=np.uint16)
    buf = make_file([("a.weight", "F8_E4M3", (300, 256), w), ("b", "BF16", (100_000,), fill),
                     ("a.scale_weight", "F32", (), f32_bytes(0.5))])
    ix = st.SafeTensorIndex.from_bytes(buf)
    plan = st.StreamPlan(ix, 64 << 10)
    check_plan(ix, plan)
    ents = {e.name: e for e in ix.tensors()}
    s = ents["a.scale_weight"]
    assert plan.steps[0].ranges == ((s.begin, s.end),)
    assert plan.steps[0].outputs == ()
    names = [o.name for o in ix.outputs()]
    a_step = next(k for k, st_ in enumerate(plan.steps) if names.index("a.weight") in st_.outputs)
    assert a_step == 2  # 76,800 weight bytes: steps 1 and 2 of 64 KiB


def test_scale_just_after_weight_stays_in_file_order():
    w = (np.arange(300 * 256) % 120).astype(np.uint8)
    buf = make_file([("a.weight", "F8_E4M3", (300, 256), w), ("a.scale_weight", "F32", (), f32_bytes(0.5))])
    ix = st.SafeTensorIndex.from_bytes(buf)
    plan = st.StreamPlan(ix, 64 << 10)
    check_plan(ix, plan)
    assert plan.ranges == [(0, 65536), (65536, ix.data_size)]


def test_empty_checkpoint_and_empty_tensors():
    ix = st.SafeTensorIndex.from_bytes(make_file([("e", "BF16", (0, 4), b"")]))
    plan = st.StreamPlan(ix, 64 << 10)
    assert len(plan.steps) == 1 and plan.steps[0].bytes == 0 and plan.steps[0].units == 0
    assert plan.order == [0] and plan.steps[0].outputs == (0,)
    buf = make_file([("e", "BF16", (0,), b""), ("x", "BF16", (40_000,), np.ones(40_000, np.uint16))])
    ix = st.SafeTensorIndex.from_bytes(buf)
    plan = st.StreamPlan(ix, 64 << 10)
    check_plan(ix, plan)


def test_chunk_too_small_is_rejected():
    ix = st.SafeTensorIndex.from_bytes(synth.config_bytes(1))
    with pytest.raises(st.StError, match="ST_E_ARG"):
        st.StreamPlan(ix, 4096)


def test_stream_file_rejects_a_plan_of_another_index_before_any_gpu_call(tmp_path):
    buf = synth.config_bytes(1)
    a = st.SafeTensorIndex.from_bytes(buf)
    b = st.SafeTensorIndex.from_bytes(buf)
    plan = st.StreamPlan(a, 64 << 10)
    path = tmp_path / "c1.safetensors"
    path.write_bytes(buf)
    st_ = st.StreamStats()
    fake = C.c_void_p(1 << 20)
    rc = lib().st_stream_file(str(path).encode(), b._h, plan._h, fake, fake, fake, fake, 1 << 30, None, None, None,
                              C.byref(st_))
    assert rc == -1 and b"another index" in lib().st_last_error()
    rc = lib().st_stream_file(str(path).encode(), a._h, plan._h, fake, fake, fake, fake, 1024, None, None, None,
                              C.byref(st_))
    assert rc == -1 and b"pinned buffer" in lib().st_last_error()


# ---------------------------------------------------------------- selected and packed plans

def _descs(table):
    from device_checkpoint_dequantisation_amd._lib import Desc, TableHeader
    h = TableHeader.from_buffer_copy(table[:64])
    size = C.sizeof(Desc)
    return [Desc.from_buffer_copy(table[h.desc_offset + j * size: h.desc_offset + (j + 1) * size])
            for j in range(h.n_desc)]


@pytest.mark.parametrize("k", [2, 3, 4, 5])
@pytest.mark.parametrize("pack", [False, True])
def test_selected_plan_reads_only_what_it_needs(k, pack, tmp_path):
    buf = synth.config_bytes(k, small=True, **({"scales_last": True} if k == 2 and pack else {}))
    path = tmp_path / "c.safetensors"
    path.write_bytes(buf)
    ix = st.SafeTensorIndex.open(str(path))
    outs, ents = ix.outputs(), ix.tensors()
    rng = np.random.default_rng(k)
    sel = sorted(rng.choice(len(outs), size=max(1, len(outs) // 3), replace=False).tolist(), reverse=True)
    plan = st.StreamPlan(ix, 64 << 10, select=sel, pack=pack)
    assert sorted(plan.order) == sorted(sel)
    # within a step, outputs keep the selection's order
    for s in plan.steps:
        assert list(s.outputs) == [o for o in sel if o in s.outputs]
    needed = sorted({(ents[i].begin, ents[i].end) for o in sel for i in (outs[o].tensor, outs[o].scale, outs[o].scale2)
                     if i >= 0 and ents[i].end > ents[i].begin})
    # every needed byte is read exactly once; nothing else except small gaps between needed tensors
    cover = sorted(plan.ranges)
    for (b0, e0), (b1, e1) in zip(cover, cover[1:]):
        assert e0 <= b1
    read = sum(e - b for b, e in plan.ranges)
    need = sum(e - b for b, e in needed)
    assert need <= read <= need + 4096 * len(needed)
    union = []
    for b, e in cover:
        if union and union[-1][1] == b:
            union[-1][1] = e
        else:
            union.append([b, e])
    for b, e in needed:
        assert any(rb <= b and e <= re for rb, re in union)
    # destinations: identity, or a compact blob keeping each byte's offset mod 256
    for (b, e), d in zip(plan.ranges, plan.range_dsts):
        if pack:
            assert d % 256 == b % 256 and d + (e - b) + 64 <= plan.blob_bytes
        else:
            assert d == b
    if pack:
        spans = sorted((d, d + e - b) for (b, e), d in zip(plan.ranges, plan.range_dsts))
        for (d0, e0), (d1, e1) in zip(spans, spans[1:]):
            assert e0 <= d1
        assert plan.blob_bytes <= need + 256 * (len(needed) + 1) + 4096 * len(needed)
    else:
        assert plan.blob_bytes == ix.blob_bytes
    # the tables point at where the bytes land
    for s in plan.steps:
        if not s.outputs:
            continue
        hdr_bytes = int.from_bytes(plan.tables[s.table_offset + 32: s.table_offset + 40], "little")
        descs = _descs(plan.tables[s.table_offset: s.table_offset + hdr_bytes])
        for j, o in enumerate(s.outputs):
            co = outs[o]
            assert descs[j].src == plan.tensor_offset(ents[co.tensor].begin) or ents[co.tensor].end == ents[co.tensor].begin
            if co.scale >= 0:
                assert descs[j].scale == plan.tensor_offset(ents[co.scale].begin)
            if co.scale2 >= 0:
                assert descs[j].scale2 == plan.tensor_offset(ents[co.scale2].begin)
    # st_read_plans lands every needed byte at its destination (host only, no GPU)
    import torch
    host = torch.full((plan.blob_bytes,), 0xEE, dtype=torch.uint8)
    st.read_plans(str(path), ix, [plan], [host])
    data = np.frombuffer(buf, np.uint8)[ix.data_offset:]
    hb = host.numpy()
    for b, e in needed:
        d = plan.tensor_offset(b)
        assert np.array_equal(hb[d: d + e - b], data[b:e])


def test_select_errors():
    ix = st.SafeTensorIndex.from_bytes(synth.config_bytes(2, small=True))
    with pytest.raises(st.StError, match="out of range"):
        st.StreamPlan(ix, 64 << 10, select=[ix.num_outputs])
    with pytest.raises(st.StError, match="twice"):
        st.StreamPlan(ix, 64 << 10, select=[1, 1])
    with pytest.raises(ValueError):
        st.StreamPlan(ix, 64 << 10, pack=True)
    plan = st.StreamPlan(ix, 64 << 10, select=[], pack=True)
    assert plan.order == [] and len(plan.steps) == 1 and plan.steps[0].units == 0


def test_read_plans_several_and_errors(tmp_path):
    buf = synth.config_bytes(4, small=True)
    path = tmp_path / "c4.safetensors"
    path.write_bytes(buf)
    ix = st.SafeTensorIndex.open(str(path))
    import torch
    plans = [st.StreamPlan(ix, 64 << 10, select=[k], pack=True) for k in range(ix.num_outputs)]
    hosts = [torch.zeros(p.blob_bytes, dtype=torch.uint8) for p in plans]
    st.read_plans(str(path), ix, plans, hosts)
    data = np.frombuffer(buf, np.uint8)[ix.data_offset:]
    ents = ix.tensors()
    for k, (p, h) in enumerate(zip(plans, hosts)):
        co = ix.output(k)
        for i in (co.tensor, co.scale, co.scale2):
            if i >= 0:
                e = ents[i]
                d = p.tensor_offset(e.begin)
                assert np.array_equal(h.numpy()[d: d + e.end - e.begin], data[e.begin:e.end])
    with pytest.raises(st.StError, match="needed"):
        st.read_plans(str(path), ix, plans[:1], [torch.zeros(8, dtype=torch.uint8)])
    other = st.SafeTensorIndex.open(str(path))
    with pytest.raises(st.StError, match="another index"):
        st.read_plans(str(path), other, plans[:1], hosts[:1])
    (tmp_path / "short.safetensors").write_bytes(buf[:-1])
    with pytest.raises(st.StError, match="ST_E_IO"):
        st.read_plans(str(tmp_path / "short.safetensors"), ix, plans[:1], hosts[:1])


def test_read_plans_from_several_threads_and_files(tmp_path):
    """The reader pool is shared by the process: repeated calls reuse it, calls on different files
    and calls from several threads at once (one takes the shared pool, the others a pool of their
    own) all land their bytes exactly."""
    import threading
    import torch
    files = []
    for k in (2, 4, 6):
        buf = synth.config_bytes(k, small=True)
        path = tmp_path / f"c{k}.safetensors"
        path.write_bytes(buf)
        ix = st.SafeTensorIndex.open(str(path))
        plan = st.StreamPlan(ix, 64 << 10, select=list(range(ix.num_outputs)), pack=True)
        files.append((str(path), ix, plan, np.frombuffer(buf, np.uint8)[ix.data_offset:]))

    def check(path, ix, plan, data, host):
        for k in range(ix.num_outputs):
            co = ix.output(k)
            for i in (co.tensor, co.scale, co.scale2):
                if i >= 0:
                    e = ix.tensors()[i]
                    d = plan.tensor_offset(e.begin)
                    assert np.array_equal(host.numpy()[d: d + e.end - e.begin], data[e.begin:e.end])

    for _ in range(3):                       # sequential calls, alternating files
        for path, ix, plan, data in files:
            host = torch.zeros(plan.blob_bytes, dtype=torch.uint8)
            st.read_plans(path, ix, [plan], [host])
            check(path, ix, plan, data, host)
    errors = []

    def worker(j):
        try:
            path, ix, plan, data = files[j % len(files)]
            for _ in range(5):
                host = torch.zeros(plan.blob_bytes, dtype=torch.uint8)
                st.read_plans(path, ix, [plan], [host])
                check(path, ix, plan, data, host)
        except Exception as e:   # reported below, on the test's thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(j,)) for j in range(6)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors


def test_read_plans_after_dropping_the_page_cache(tmp_path):
    """Ranges whose pages are not in the page cache are read in larger pieces than cached ones
    (the reader pool asks the kernel, without waiting for the disk, whether the range's first, middle
    and last bytes are cached).  Both ways land the same bytes: read the file with its pages dropped
    from the cache (advisory: fsync, then POSIX_FADV_DONTNEED), then again with them cached, and
    compare every byte.  Three tensors, two of them longer than one cold piece (64 MiB)."""
    import os
    import torch
    rng = np.random.default_rng(11)
    sizes = [(70 << 20) + 3, 5, (130 << 20) + 1]   # bf16 element counts x 2 bytes, odd offsets after the second
    tensors = []
    for k, n in enumerate(sizes):
        raw = rng.integers(0, 256, size=2 * n, dtype=np.uint8)
        tensors.append((f"t{k}", "BF16", (n,), raw))
    buf = make_file(tensors)
    path = tmp_path / "big.safetensors"
    path.write_bytes(buf)
    ix = st.SafeTensorIndex.open(str(path))
    data = np.frombuffer(buf, np.uint8)[ix.data_offset:]
    plans = [st.StreamPlan(ix, 96 << 20), st.StreamPlan(ix, 96 << 20, select=[2, 0], pack=True)]
    for cached in (False, True):
        for plan in plans:
            if not cached:   # drop the file's pages before each read
                fd = os.open(str(path), os.O_RDONLY)
                try:
                    os.fsync(fd)
                    os.posix_fadvise(fd, 0, 0, os.POSIX_FADV_DONTNEED)
                finally:
                    os.close(fd)
            host = torch.full((plan.blob_bytes,), 0xEE, dtype=torch.uint8)
            st.read_plans(str(path), ix, [plan], [host])
            hb = host.numpy()
            for b, e in plan.ranges:
                d = plan.tensor_offset(b)
                assert np.array_equal(hb[d: d + e - b], data[b:e])
    del buf, data
