"""GPU parity of the fp16 and fp32 output types: the kernel instances for each type against the
oracle's rounding of the same exact values, bit for bit, over every checkpoint family, every code
of every format with special scales, column slices (both kernels), the streamed pipeline and lazy
loads; outputs that are not aligned to 16 bytes; and a launch whose output type disagrees with the
table's writes nothing."""
import numpy as np
import pytest
import torch

import oracle
import synth
import device_checkpoint_dequantisation_amd as st
from tests.test_gpu_parity import (block_fp8_file, float_every_code_file, fp4_scales_last_file, fp8_every_code_file,
                                   mx_every_code_file, nvfp4_every_code_file, pieces_file)
from tests.test_gpu_slices import _slices_for, _view
from tests.st_files import make_file

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TYPES = ["f16", "f32"]


def _bits(t):
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _staged(buf, out_dtype, **kw):
    ix = st.SafeTensorIndex.from_bytes(buf, out_dtype=out_dtype, **kw)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.load_bytes(buf[ix.data_offset:])
    return ix, ck


def _assert_equal(name, g, w):
    assert g.shape == w.shape, name
    if not np.array_equal(g, w):
        bad = np.nonzero(g.reshape(-1) != w.reshape(-1))[0]
        raise AssertionError(f"{name}: {len(bad)} of {w.size} differ; first at {bad[:8].tolist()}: "
                             f"gpu {[hex(x) for x in g.reshape(-1)[bad[:8]]]} "
                             f"oracle {[hex(x) for x in w.reshape(-1)[bad[:8]]]}")


def assert_parity(buf, out_dtype, **kw):
    print(f"{out_dtype} parity case: {len(buf)} bytes {kw}", flush=True)
    want = oracle.materialize(buf, out_dtype)
    ix, ck = _staged(buf, out_dtype, **kw)
    assert ck.arena.dtype == {"f16": torch.float16, "f32": torch.float32}[out_dtype]
    ck.arena.view(torch.int16).fill_(0x5A5A)     # poison: every element must be written
    ck.materialize()
    torch.cuda.synchronize()
    assert list(ck.tensors) == list(want)
    for name, w in want.items():
        _assert_equal(name, _bits(ck.tensors[name]), w)


@pytest.mark.parametrize("out_dtype", TYPES)
@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6, 7])
def test_configs_small(k, out_dtype):
    assert_parity(synth.config_bytes(k, small=k != 1), out_dtype)


@pytest.mark.parametrize("out_dtype", TYPES)
@pytest.mark.parametrize("k,scale", [(1, 3), (3, 1), (4, 6), (5, 3)])
def test_larger_work_units(k, scale, out_dtype):
    assert_parity(synth.config_bytes(k, small=k != 1), out_dtype, unit_log2_scale=scale)


@pytest.mark.parametrize("out_dtype", TYPES)
@pytest.mark.parametrize("shift", [0, 1, 2, 3, 9])
def test_fp8_tensor_every_code(shift, out_dtype):
    assert_parity(fp8_every_code_file(shift), out_dtype)


@pytest.mark.parametrize("out_dtype", TYPES)
@pytest.mark.parametrize("shift", [0, 1, 6])
def test_nvfp4_every_code(shift, out_dtype):
    assert_parity(nvfp4_every_code_file(shift), out_dtype)


@pytest.mark.parametrize("out_dtype", TYPES)
@pytest.mark.parametrize("M,N,shift", [(300, 200, 0), (130, 7, 2), (257, 129, 7), (128, 4096, 0), (1, 16, 1)])
def test_block_fp8_ragged_shapes(M, N, shift, out_dtype):
    assert_parity(block_fp8_file(M, N, shift), out_dtype)


@pytest.mark.parametrize("out_dtype", TYPES)
@pytest.mark.parametrize("shift", [0, 1, 2, 3, 7])
def test_float_sources_every_code(shift, out_dtype):
    assert_parity(float_every_code_file(shift), out_dtype)


@pytest.mark.parametrize("out_dtype", TYPES)
@pytest.mark.parametrize("kind", ["MXFP8", "MXFP4"])
@pytest.mark.parametrize("shift", [0, 3])
def test_mx_every_code(kind, shift, out_dtype):
    assert_parity(mx_every_code_file(kind, shift), out_dtype)


@pytest.mark.parametrize("out_dtype", TYPES)
@pytest.mark.parametrize("kind", ["NVFP4", "MXFP4"])
@pytest.mark.parametrize("shift", [0, 1, 2, 3])
def test_fp4_block_scales_last_in_the_file(kind, shift, out_dtype):
    """The unit-wide scale-code fetch of both fp4 unit forms (fp32: the paired-lane unit) at every
    alignment of a scale tensor that ends the data section."""
    assert_parity(fp4_scales_last_file(kind, shift), out_dtype)


@pytest.mark.parametrize("out_dtype", TYPES)
@pytest.mark.parametrize("k", [2, 4, 7])
def test_outputs_not_aligned_to_16_bytes(k, out_dtype):
    """Every output shifted by one element: the exact path writes them one at a time (for packed
    fp4 into fp32, from the paired-lane unit too)."""
    buf = synth.config_bytes(k, small=True)
    ix, ck = _staged(buf, out_dtype)
    esize = 4 if out_dtype == "f32" else 2
    arena = torch.empty(ix.arena_bytes // esize + 8, dtype=ix.torch_dtype, device=DEV)
    outs = ix.outputs()
    ptrs = torch.tensor([arena.data_ptr() + o.offset + esize for o in outs], dtype=torch.int64).to(DEV)
    st.materialize(ck.blob, ck.table, ck.units, ptrs, out_dtype=out_dtype)
    torch.cuda.synchronize()
    want = oracle.materialize(buf, out_dtype)
    for o in outs:
        start = o.offset // esize + 1
        _assert_equal(o.name, _bits(arena[start: start + o.numel]).reshape(o.shape), want[o.name])


@pytest.mark.parametrize("planned,launch", [(p, q) for p in ("bf16", "f16", "f32") for q in ("bf16", "f16", "f32")
                                             if p != q])
def test_output_type_mismatch_writes_nothing(planned, launch):
    buf = synth.config_bytes(1)
    ix, ck = _staged(buf, planned)
    ck.arena.view(torch.int16).fill_(0x1234)
    for slices in (False, True):
        st.materialize(ck.blob, ck.table, ck.units, ck.outs, slices=slices, out_dtype=launch)
    torch.cuda.synchronize()
    assert bool((ck.arena.view(torch.int16) == 0x1234).all())


@pytest.mark.parametrize("strided_kernel", [True, False])
@pytest.mark.parametrize("out_dtype", TYPES)
@pytest.mark.parametrize("k", [2, 3, 4, 5, 6, 7])
def test_slices(k, out_dtype, strided_kernel):
    buf = synth.config_bytes(k, small=True)
    want = oracle.materialize(buf, out_dtype)
    ix, ck = _staged(buf, out_dtype)
    rng = np.random.default_rng(100 + k)
    outs = ix.outputs()
    picks = range(len(outs)) if len(outs) <= 40 else rng.choice(len(outs), 40, replace=False)
    slices = [(int(kk), rows, cols) for kk in picks for rows, cols in _slices_for(outs[int(kk)], rng)]
    print(f"{out_dtype} slices c{k}: {len(slices)} (strided kernel {strided_kernel})", flush=True)
    got = ck.materialize_slices(slices, strided_kernel=strided_kernel)
    torch.cuda.synchronize()
    for (kk, rows, cols), t in zip(slices, got):
        assert t.dtype == ix.torch_dtype
        w = _view(want[outs[kk].name])
        r0, r1 = rows if rows else (0, w.shape[0])
        c0, c1 = cols if cols else (0, w.shape[1])
        _assert_equal((outs[kk].name, rows, cols), _bits(t).reshape(r1 - r0, c1 - c0), w[r0:r1, c0:c1])


@pytest.mark.parametrize("out_dtype", TYPES)
@pytest.mark.parametrize("k", [2, 4, 5])
def test_streamed_load(k, out_dtype, tmp_path):
    buf = synth.config_bytes(k, small=True)
    p = tmp_path / f"c{k}.safetensors"
    p.write_bytes(buf)
    want = oracle.materialize(buf, out_dtype)
    print(f"{out_dtype} streamed c{k}", flush=True)
    for streamed in (True, False):
        got = st.load(str(p), DEV, streamed=streamed, chunk_mb=1, out_dtype=out_dtype)
        for name, w in want.items():
            assert got[name].dtype == {"f16": torch.float16, "f32": torch.float32}[out_dtype]
            _assert_equal((streamed, name), _bits(got[name]), w)


@pytest.mark.parametrize("out_dtype", TYPES)
@pytest.mark.parametrize("k", [3, 4])
def test_lazy_loads(k, out_dtype, tmp_path):
    buf = synth.config_bytes(k, small=True)
    p = tmp_path / f"c{k}.safetensors"
    p.write_bytes(buf)
    want = oracle.materialize(buf, out_dtype)
    print(f"{out_dtype} lazy c{k}", flush=True)
    for ram in (0, 1 << 30):
        sd = st.StreamStateDict(str(p), DEV, ram_cache_bytes=ram, out_dtype=out_dtype)
        names = list(sd)
        for _ in range(2 if ram else 1):          # the second pass hits the RAM tier
            got = sd.load(names)
            torch.cuda.synchronize()
            for name, w in want.items():
                _assert_equal((ram, name), _bits(got[name]).reshape(w.shape), w)
        for name in names[:: max(1, len(names) // 10)]:
            _assert_equal(name, _bits(sd[name]).reshape(want[name].shape), want[name])


def _f16_rounding_file():
    """fp32 inputs covering every fp16 rounding class: every finite fp16 value, every midpoint
    between neighbours (ties, including the subnormal ties down to 2^-25), one fp32 ulp either
    side of each midpoint, the overflow boundary, and both signs."""
    codes = np.arange(0x7C00, dtype=np.uint32)
    vals = codes.astype(np.uint16).view(np.float16).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    mid32 = mids.astype(np.float32)
    extra = np.array([2.0 ** -25, 65504.0, 65519.99, 65520.0, 1e30], dtype=np.float32)
    x = np.concatenate([vals.astype(np.float32), mid32, np.nextafter(mid32, np.float32(np.inf)),
                        np.nextafter(mid32, np.float32(0)), extra])
    x = np.concatenate([x, -x])
    return make_file([("f", "F32", (x.size,), x)])


@pytest.mark.parametrize("shift", [0, 1])
def test_f16_rounding_every_class_both_paths(shift):
    """Aligned outputs take the vector conversion; outputs shifted by one element take the exact
    path's software rounding.  Both must equal the oracle on every rounding class."""
    buf = _f16_rounding_file()
    ix, ck = _staged(buf, "f16")
    want = oracle.materialize(buf, "f16")["f"]
    o = ix.outputs()[0]
    arena = torch.empty(o.numel + 64, dtype=torch.float16, device=DEV)
    arena.view(torch.int16).fill_(0x5A5A)
    ptrs = torch.tensor([arena.data_ptr() + 2 * shift], dtype=torch.int64).to(DEV)
    st.materialize(ck.blob, ck.table, ck.units, ptrs, out_dtype="f16")
    torch.cuda.synchronize()
    _assert_equal(("f16 rounding", shift), _bits(arena[shift: shift + o.numel]), want)


@pytest.mark.parametrize("out_dtype", TYPES)
def test_large_outputs_cut_into_pieces(out_dtype):
    assert_parity(pieces_file(), out_dtype)
