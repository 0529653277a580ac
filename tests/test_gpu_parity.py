"""GPU parity: the HIP path through the C ABI against the CPU oracle, bit for bit, on seeded
inputs that span several work units, ragged tails, every code of every format, unaligned
sources and outputs, special scales, subsets and empty cases."""
import numpy as np
import pytest
import torch

import oracle
import synth
import device_checkpoint_dequantisation_amd as st
from tests.st_files import f32_bytes, make_file

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _gpu_outputs(buf: bytes, unit_log2_scale=0):
    ix = st.SafeTensorIndex.from_bytes(buf, unit_log2_scale=unit_log2_scale)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.load_bytes(buf[ix.data_offset:])
    ck.arena.view(torch.int16).fill_(0x5A5A)     # poison: every element must be written
    ck.materialize()
    torch.cuda.synchronize()
    return {k: v.view(torch.int16).cpu().numpy().view(np.uint16) for k, v in ck.tensors.items()}, ck


def assert_parity(buf: bytes, **kw):
    print(f"parity case: {len(buf)} bytes {kw}", flush=True)
    want = oracle.materialize(buf)
    got, ck = _gpu_outputs(buf, **kw)
    assert list(got) == list(want)
    for name in want:
        w, g = want[name], got[name]
        assert g.shape == w.shape, name
        if not np.array_equal(g, w):
            bad = np.nonzero(g.reshape(-1) != w.reshape(-1))[0]
            raise AssertionError(f"{name}: {len(bad)} of {w.size} differ; first at {bad[:8].tolist()}: "
                                 f"gpu {g.reshape(-1)[bad[:8]].tolist()} oracle {w.reshape(-1)[bad[:8]].tolist()}")
    return ck


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6, 7])
def test_configs_small(k):
    assert_parity(synth.config_bytes(k, small=k != 1))


@pytest.mark.parametrize("k", [1, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("scale", [1, 3, 6])
def test_larger_work_units(k, scale):
    assert_parity(synth.config_bytes(k, small=k != 1), unit_log2_scale=scale)


def _pad(k):
    """A leading tensor of k + 4 bytes (F8 [k] + its scale), shifting later offsets by k + 4."""
    if k == 0:
        return []
    return [("pad.weight", "F8_E4M3", (k,), np.full(k, 0x38, np.uint8)), ("pad.scale_weight", "F32", (), f32_bytes(1.0))]


SPECIAL_SCALES = [0x3F6471C8, 0x3C23D70A, 0x00000001, 0x00400000, 0x7F7FFFFF, 0x7F000000, 0x7F800000, 0xFF800000,
                  0x7FC00000, 0x80000000, 0x00000000, 0xBF800000, 0x3B2D27D2]


def fp8_every_code_file(shift):
    """Every e4m3 code (10240 elements: full units and a ragged tail) under special fp32 scales."""
    codes = np.tile(np.arange(256, dtype=np.uint8), 40)
    tensors = list(_pad(shift))
    for i, s in enumerate(SPECIAL_SCALES):
        tensors += [(f"q{i}.weight", "F8_E4M3", (len(codes),), np.roll(codes, i)),
                    (f"q{i}.scale_weight", "F32", (), np.array([s], np.uint32).tobytes())]
    return make_file(tensors)


def nvfp4_every_code_file(shift, storage="U8"):
    """Rows of K = 48 (K % 32 == 16): every e2m1 code against every e4m3 block-scale code,
    including NaN codes and subnormals, under several global scales."""
    sc = np.arange(256, dtype=np.uint8)
    M, K = 256 * 2, 48
    nib = np.tile(np.arange(16, dtype=np.uint8), M * K // 16)
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    bs = np.repeat(sc, 6)[: M * K // 16]
    tensors = list(_pad(shift))
    for i, g in enumerate([0x3B2D27D2, 0x3F800000, 0x00000001, 0x7F7FFFFF, 0x7F800000, 0x7FC00000, 0x00000000]):
        wshape = (M, K // 2) if storage == "U8" else (M, K)   # F4: the shape counts unpacked elements
        tensors += [(f"n{i}.weight", storage, wshape, packed), (f"n{i}.weight_scale", "F8_E4M3", (M, K // 16), np.roll(bs, i)),
                    (f"n{i}.weight_scale_2", "F32", (), np.array([g], np.uint32).tobytes())]
    return make_file(tensors)


def block_fp8_file(M, N, shift):
    """Random codes in [M, N] with 128x128 scales, one huge, one NaN and one infinite."""
    rng = np.random.default_rng(M * 1000 + N)
    w = rng.integers(0, 256, size=M * N, dtype=np.uint64).astype(np.uint8)
    gm, gn = -(-M // 128), -(-N // 128)
    S = rng.uniform(1e-4, 1e-2, size=gm * gn).astype(np.float32)
    S[0] = np.float32(2.0 ** 125)   # not foldable
    if S.size > 2:
        S[1] = np.float32("nan")
        S[2] = np.float32("inf")
    tensors = list(_pad(shift)) + [("b.weight", "F8_E4M3", (M, N), w), ("b.weight_scale_inv", "F32", (gm, gn), S)]
    return make_file(tensors)


def mx_every_code_file(kind, shift, storage="U8"):
    """MXFP8: rows of K = 288 (9 scale blocks), every e4m3 code against every E8M0 scale code
    (NaN and the subnormal 2^-127 included); MXFP4: every e2m1 code against every scale code."""
    if kind == "MXFP8":
        M, K = 256, 288
        codes = np.tile(np.arange(256, dtype=np.uint8), M * K // 256 + 1)[: M * K]
        scales = np.arange(M * K // 32, dtype=np.uint32).astype(np.uint8)
        tensors = list(_pad(shift)) + [("x.weight", "F8_E4M3", (M, K), codes),
                                       ("x.weight_scale", "F8_E8M0", (M, K // 32), scales)]
    else:
        M, K = 256, 96
        nib = np.tile(np.arange(16, dtype=np.uint8), M * K // 16)
        packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
        scales = np.roll(np.arange(M * K // 32, dtype=np.uint32).astype(np.uint8), 7)
        shape = (M, K // 2) if storage == "U8" else (M, K)
        tensors = list(_pad(shift)) + [("x.weight", storage, shape, packed),
                                       ("x.weight_scale", "F8_E8M0", (M, K // 32), scales)]
    return make_file(tensors)


def float_every_code_file(shift):
    """Every fp16 code, random fp32 words with their specials, random bf16 words."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(5)
    f = rng.integers(0, 2 ** 32, size=50_001, dtype=np.uint64).astype(np.uint32)
    f[:12] = [0x7F800000, 0xFF800000, 0x7FC00000, 0xFFFFFFFF, 0x00000001, 0x80000001, 0x007FFFFF, 0x7F7FFFFF,
              0x3F808000, 0x3F818000, 0x00008000, 0x00018000]
    bf = rng.integers(0, 2 ** 16, size=9_999, dtype=np.uint64).astype(np.uint16)
    tensors = list(_pad(shift)) + [("h", "F16", (256, 256), h), ("f", "F32", (50_001,), f), ("p", "BF16", (9_999,), bf)]
    return make_file(tensors)


@pytest.mark.parametrize("shift", [0, 1, 2, 3, 5, 9, 12, 15])
def test_fp8_tensor_every_code_every_alignment(shift):
    assert_parity(fp8_every_code_file(shift))


@pytest.mark.parametrize("storage", ["U8", "F4"])
@pytest.mark.parametrize("shift", [0, 1, 3, 6])
def test_nvfp4_every_nibble_every_block_scale(shift, storage):
    assert_parity(nvfp4_every_code_file(shift, storage))


@pytest.mark.parametrize("M,N", [(300, 200), (5, 1), (130, 7), (257, 129), (128, 4096), (1, 16), (129, 48)])
@pytest.mark.parametrize("shift", [0, 2, 7])
def test_block_fp8_ragged_shapes(M, N, shift):
    assert_parity(block_fp8_file(M, N, shift))


@pytest.mark.parametrize("shift", [0, 1, 2, 3, 7])
def test_f16_every_code_and_f32_specials(shift):
    assert_parity(float_every_code_file(shift))


@pytest.mark.parametrize("kind,storage", [("MXFP8", None), ("MXFP4", "U8"), ("MXFP4", "F4")])
@pytest.mark.parametrize("shift", [0, 1, 2, 3, 5, 9])
def test_mx_every_code_every_scale(kind, storage, shift):
    assert_parity(mx_every_code_file(kind, shift, storage or "U8"))


def fp4_scales_last_file(kind, shift):
    """Packed fp4 [64, 256] (8 whole units into 2-byte outputs, 16 into fp32) with its block-scale
    tensor last in the data section, at offset shift mod 4, and NaN codes among the scales."""
    rng = np.random.default_rng(40 + shift)
    M, K = 64, 256
    packed = rng.integers(0, 256, size=M * K // 2, dtype=np.uint64).astype(np.uint8)
    tensors = list(_pad(shift))
    if kind == "NVFP4":
        sc = rng.integers(0x08, 0x60, size=M * K // 16, dtype=np.uint64).astype(np.uint8)  # e4m3, finite
        sc[[3, 500, 1023]] = [0x7F, 0xFF, 0x7F]          # NaN codes
        tensors += [("w.weight_scale_2", "F32", (), f32_bytes(0.75)), ("w.weight", "U8", (M, K // 2), packed),
                    ("w.weight_scale", "F8_E4M3", (M, K // 16), sc)]
    else:
        sc = rng.integers(100, 150, size=M * K // 32, dtype=np.uint64).astype(np.uint8)     # e8m0
        sc[[5, 300]] = 0xFF                                # NaN codes
        tensors += [("w.weight", "U8", (M, K // 2), packed), ("w.weight_scale", "F8_E8M0", (M, K // 32), sc)]
    buf = make_file(tensors)
    ix = st.SafeTensorIndex.from_bytes(buf)
    last = max(ix.tensors(), key=lambda t: t.begin)
    assert last.name == "w.weight_scale" and last.begin % 4 == shift and last.end == ix.data_size
    return buf


@pytest.mark.parametrize("kind", ["NVFP4", "MXFP4"])
@pytest.mark.parametrize("shift", [0, 1, 2, 3])
def test_fp4_block_scales_last_in_the_file(kind, shift):
    """Whole packed-fp4 units fetch their block-scale codes as one word per lane, from the 4-byte
    boundary below them, reading up to 4 bytes past a unit's codes.  With the scale tensor last in
    the data section, at each alignment, those bytes are the blob's tail padding; NaN codes among
    the scales send their chunks down the exact path."""
    assert_parity(fp4_scales_last_file(kind, shift))


def test_many_small_full_stress_config():
    assert_parity(synth.config_bytes(5, count=6000))


def test_misaligned_output_pointers_take_the_exact_path():
    buf = synth.config_bytes(1)
    ix = st.SafeTensorIndex.from_bytes(buf)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.load_bytes(buf[ix.data_offset:])
    outs = ix.outputs()
    # a second arena, every output shifted by 2 bytes (bf16-aligned, not 16-byte aligned)
    arena = torch.empty(ix.arena_bytes // 2 + 8, dtype=torch.bfloat16, device=DEV)
    ptrs = torch.tensor([arena.data_ptr() + o.offset + 2 for o in outs], dtype=torch.int64).to(DEV)
    st.materialize(ck.blob, ck.table, ck.units, ptrs)
    torch.cuda.synchronize()
    want = oracle.materialize(buf)
    for o in outs:
        start = o.offset // 2 + 1
        got = arena[start: start + o.numel].view(torch.int16).cpu().numpy().view(np.uint16).reshape(o.shape)
        assert np.array_equal(got, want[o.name]), o.name


def test_subset_table_writes_only_selected_outputs():
    buf = synth.config_bytes(3, small=True)
    ix = st.SafeTensorIndex.from_bytes(buf)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.load_bytes(buf[ix.data_offset:])
    outs = ix.outputs()
    sel = [len(outs) - 1, 2, 0]
    raw, units = ix.table_subset(sel)
    table = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(DEV)
    bufs = [torch.full((outs[s].numel,), -1, dtype=torch.int16, device=DEV) for s in sel]
    ptrs = torch.tensor([b.data_ptr() for b in bufs], dtype=torch.int64).to(DEV)
    st.materialize(ck.blob, table, units, ptrs)
    torch.cuda.synchronize()
    want = oracle.materialize(buf)
    for s, b in zip(sel, bufs):
        assert np.array_equal(b.cpu().numpy().view(np.uint16), want[outs[s].name].reshape(-1))


def test_wrong_unit_count_writes_nothing():
    buf = synth.config_bytes(1)
    ix = st.SafeTensorIndex.from_bytes(buf)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.load_bytes(buf[ix.data_offset:])
    ck.arena.view(torch.int16).fill_(0x1234)
    st.materialize(ck.blob, ck.table, ck.units - 1, ck.outs)
    torch.cuda.synchronize()
    assert bool((ck.arena.view(torch.int16) == 0x1234).all())


def test_empty_outputs_and_empty_table():
    f = make_file([("e", "BF16", (0,), b""), ("a", "F32", (3,), f32_bytes(1, 2, 3)), ("z", "F16", (0, 7), b""),
                   ("q.weight", "F8_E4M3", (0, 16), b""), ("q.weight_scale_inv", "F32", (0, 1), b"")])
    assert_parity(f)
    ix = st.SafeTensorIndex.from_bytes(make_file([]))
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.materialize()
    torch.cuda.synchronize()
    assert ck.tensors == {}


def test_staging_from_file_matches_bytes(tmp_path):
    buf = synth.config_bytes(5, small=True)
    p = tmp_path / "c5.safetensors"
    p.write_bytes(buf)
    ix = st.SafeTensorIndex.open(str(p))
    ck = st.DeviceCheckpoint(ix, str(p), DEV, pinned_mb=2)
    host = ck.blob[: ix.data_size].cpu().numpy().tobytes()
    assert host == buf[ix.data_offset:]
    want = oracle.materialize(buf)
    for streamed in (True, False):
        out = st.load(str(p), DEV, streamed=streamed)
        for name, w in want.items():
            assert np.array_equal(out[name].view(torch.int16).cpu().numpy().view(np.uint16), w), (streamed, name)


def pieces_file():
    """Outputs of at least 2048 units, which the planner cuts into 8 pieces, between small ones and
    at odd byte offsets: bf16 (2049 units, the last partial), scaled FP8 (3001 units) and NVFP4
    (2080 units of 2048 elements)."""
    rng = np.random.default_rng(9)
    nb, nf = 2048 * 1024 + 5, 3000 * 1024 + 77
    M, K = 1024, 4160
    tensors = list(_pad(3))
    tensors += [("a", "BF16", (nb,), rng.integers(0, 2 ** 16, nb, dtype=np.uint64).astype(np.uint16))]
    tensors += [(f"s{i}", "F16", (100 + 7 * i,), rng.standard_normal(100 + 7 * i).astype(np.float16)) for i in range(9)]
    tensors += [("q.weight", "F8_E4M3", (nf,), rng.integers(0, 256, nf, dtype=np.uint64).astype(np.uint8)),
                ("q.scale_weight", "F32", (), f32_bytes(0.013))]
    tensors += [("n.weight", "U8", (M, K // 2), rng.integers(0, 256, M * K // 2, dtype=np.uint64).astype(np.uint8)),
                ("n.weight_scale", "F8_E4M3", (M, K // 16), np.full(M * K // 16, 0x38, np.uint8)),
                ("n.weight_scale_2", "F32", (), f32_bytes(0.25))]
    return make_file(tensors)


def test_large_outputs_cut_into_pieces():
    ck = assert_parity(pieces_file())
    h = np.frombuffer(ck.table.cpu().numpy().tobytes()[:64], dtype=np.uint32)
    assert ck.units > 7000 and h[1] > len(ck.tensors)   # n_desc: the large outputs were cut


def test_concurrent_decodes_on_separate_streams():
    """The library keeps no device state between launches, so decodes of different checkpoints
    (and output types) enqueued on separate streams may run at the same time: each must still
    equal the oracle.  Each stream decodes its checkpoint three times in a row."""
    cases = [(2, "bf16"), (4, "f32"), (7, "f16"), (3, "bf16")]
    cks, wants, streams = [], [], []
    for k, dt in cases:
        buf = synth.config_bytes(k, small=True)
        ix = st.SafeTensorIndex.from_bytes(buf, out_dtype=dt)
        ck = st.DeviceCheckpoint(ix, None, DEV)
        ck.load_bytes(buf[ix.data_offset:])
        ck.arena.view(torch.int16).fill_(0x5A5A)
        cks.append(ck)
        wants.append(oracle.materialize(buf, dt))
        streams.append(torch.cuda.Stream(DEV))
    torch.cuda.synchronize()
    print(f"concurrent decodes: {cases}", flush=True)
    for _ in range(3):
        for ck, s in zip(cks, streams):
            ck.materialize(s)
    torch.cuda.synchronize()
    for (k, dt), ck, want in zip(cases, cks, wants):
        for name, w in want.items():
            t = ck.tensors[name].contiguous()
            g = (t.view(torch.int32) if dt == "f32" else t.view(torch.int16)).cpu().numpy().view(w.dtype)
            assert np.array_equal(g.reshape(w.shape), w), (k, dt, name)
