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
