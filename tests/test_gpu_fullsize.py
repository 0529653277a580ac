"""GPU parity at full checkpoint sizes and at maximum sizes, in the launch configuration bench.py
times (one st_materialize over the whole staged blob).  The five benchmark checkpoints are compared
with the oracle element by element in full in test_gpu_fullsize_oracle.py; here:

* The MXFP8 and MXFP4 checkpoints at full size: every output is checked against the CPU oracle on
  sampled elements the oracle computes one by one: first, last, row and 128-block boundaries, and
  random positions.
* A spread of the quantised outputs is also checked whole against an independent GPU computation of
  the same definition with torch (float8_e4m3fn decode, fp32 products in the pages' order, RNE cast
  to bfloat16). The generated checkpoints hold no NaN code, where torch's NaN bits would differ.
* The fp16 and fp32 kernel instances at full size (scaled FP8, block FP8, NVFP4, MXFP4): sampled
  elements against the oracle's rounding to that type, whole quantised outputs against torch.
* Maximum sizes (index built from the header alone, blob filled on the GPU): a bf16 tensor of more
  than 2^32 elements, a 128-block FP8 tensor just under the 2^32-element limit, a per-tensor
  FP8 tensor whose source starts unaligned and ends past 2^31 bytes, and a checkpoint of more than
  2^24 work units, whose launch needs more than 2^22 workgroups and so a second grid row.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.st_writer import Group, TensorSpec, layout
import device_checkpoint_dequantisation_amd as st

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
QUANT = ("FP8_TENSOR", "FP8_BLOCK128", "NVFP4", "MXFP8", "MXFP4")
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def _sample_idx(shape, numel, rng, n_rand=256):
    idx = [0, numel - 1] + rng.integers(0, numel, n_rand).tolist()
    if len(shape) == 2:
        rows, cols = shape
        for r in (0, 127, 128, rows // 2, rows - 1):
            for c in (0, 15, 16, 31, 32, 127, 128, cols // 2, cols - 1):
                if r < rows and c < cols:
                    idx.append(r * cols + c)
    return np.unique(np.array(idx, dtype=np.int64))


def _bits(t):
    return t.contiguous().view(torch.int16)


def _e4m3(u8):
    return u8.view(torch.float8_e4m3fn).float()


def _f32(blob, begin, count):
    return blob[begin: begin + 4 * count].clone().view(torch.float32)   # scales may sit 2 bytes off


def _expand_grid(S, m, n):
    return S.repeat_interleave(128, 0)[:m].repeat_interleave(128, 1)[:, :n]


def _torch_reference(kind, shape, blob, src, scale, scale2, out=torch.bfloat16):
    """Value of one quantised output in the output type ``out``, computed whole with torch ops on
    the GPU (the fp32 result, then torch's round-to-nearest-even cast)."""
    return _torch_f32(kind, shape, blob, src, scale, scale2).to(out)


def _torch_f32(kind, shape, blob, src, scale, scale2):
    numel = int(np.prod(shape))
    if kind == "FP8_TENSOR":
        return _e4m3(blob[src: src + numel]) * _f32(blob, scale, 1)
    if kind == "FP8_BLOCK128":
        m, n = shape
        gm, gn = -(-m // 128), -(-n // 128)
        S = _expand_grid(_f32(blob, scale, gm * gn).view(gm, gn), m, n)
        return (_e4m3(blob[src: src + numel]).view(m, n) * S).view(-1)
    if kind == "NVFP4":
        packed = blob[src: src + numel // 2]
        nib = torch.stack([packed & 15, packed >> 4], dim=1).view(-1).long()
        table = torch.tensor(E2M1, dtype=torch.float32, device=blob.device)
        bs = _e4m3(blob[scale: scale + numel // 16]).repeat_interleave(16)
        return (table[nib] * bs) * _f32(blob, scale2, 1)
    if kind in ("MXFP8", "MXFP4"):   # E8M0 scale per 32 elements, decoded by torch on the CPU
        S = blob[scale: scale + numel // 32].cpu().view(torch.float8_e8m0fnu).float().to(blob.device)
        S = S.repeat_interleave(32)
        if kind == "MXFP8":
            return _e4m3(blob[src: src + numel]) * S
        packed = blob[src: src + numel // 2]
        nib = torch.stack([packed & 15, packed >> 4], dim=1).view(-1).long()
        return torch.tensor(E2M1, dtype=torch.float32, device=blob.device)[nib] * S
    raise ValueError(kind)


@pytest.mark.parametrize("k", [6, 7])
def test_full_size_checkpoint(k, tmp_path):
    path = str(tmp_path / f"c{k}.safetensors")
    print(f"full-size config {k}: writing", flush=True)
    synth.write_config(k, path)
    try:
        print(f"config {k}: staging {os.path.getsize(path) / 1e9:.2f} GB", flush=True)
        ix = st.SafeTensorIndex.open(path)
        ck = st.DeviceCheckpoint(ix, path, DEV)
        ck.arena.view(torch.int16).fill_(0x5A5A)
        ck.materialize()
        torch.cuda.synchronize()
        mm = np.memmap(path, dtype=np.uint8, mode="r")
        h, outs = oracle.plan(mm)
        data = mm[h.data_offset:]
        rng = np.random.default_rng(k)
        ents = ix.tensors()
        couts = ix.outputs()
        assert [o.name for o in outs] == [co.name for co in couts]
        where, want = [], []
        for o, co in zip(outs, couts):          # sampled elements of every output, one gather
            assert o.kind == co.kind and o.shape == co.shape
            if o.numel:
                idx = _sample_idx(o.shape, o.numel, rng)
                where.append(co.offset // 2 + idx)
                want.append(oracle.decode(o, data, idx))
        where = torch.from_numpy(np.concatenate(where)).to(DEV)
        got = ck.arena.view(torch.int16)[where].cpu().numpy().view(np.uint16)
        bad = np.flatnonzero(got != np.concatenate(want))
        assert bad.size == 0, f"{bad.size} sampled elements differ from the oracle"
        whole = {kind: 0 for kind in QUANT}
        for o, co in zip(outs, couts):
            got_t = ck.tensors[o.name].reshape(-1)
            if o.kind in QUANT and whole[o.kind] < 8:
                ref = _torch_reference(o.kind, o.shape, ck.blob, ents[co.tensor].begin,
                                       ents[co.scale].begin, ents[co.scale2].begin if co.scale2 >= 0 else 0)
                assert torch.equal(_bits(got_t), _bits(ref)), f"{o.name}: whole tensor differs"
                whole[o.kind] += 1
            elif o.kind == "PASS_BF16":
                e = ents[co.tensor]
                assert torch.equal(got_t.view(torch.uint8), ck.blob[e.begin: e.end]), f"{o.name}: passthrough"
        print(f"config {k}: {len(outs)} outputs sampled; checked whole: {whole}", flush=True)
        del ck
    finally:
        os.remove(path)
        torch.cuda.empty_cache()


@pytest.mark.parametrize("k,out_dtype", [(2, "f32"), (4, "f32"), (7, "f32"), (4, "f16"), (3, "f32")])
def test_full_size_output_types(k, out_dtype, tmp_path):
    """The fp16 and fp32 kernel instances at full size, in the bench's launch configuration: sampled
    elements of every output against the oracle, and whole quantised outputs against torch."""
    path = str(tmp_path / f"c{k}.safetensors")
    print(f"full-size config {k} into {out_dtype}: writing", flush=True)
    synth.write_config(k, path)
    tdt, ibits = {"f16": (torch.float16, torch.int16), "f32": (torch.float32, torch.int32)}[out_dtype]
    try:
        ix = st.SafeTensorIndex.open(path, out_dtype=out_dtype)
        ck = st.DeviceCheckpoint(ix, path, DEV)
        ck.arena.view(torch.int16).fill_(0x5A5A)
        ck.materialize()
        torch.cuda.synchronize()
        mm = np.memmap(path, dtype=np.uint8, mode="r")
        h, outs = oracle.plan(mm)
        data = mm[h.data_offset:]
        rng = np.random.default_rng(100 + k)
        ents = ix.tensors()
        couts = ix.outputs()
        esize = 4 if out_dtype == "f32" else 2
        where, want = [], []
        for o, co in zip(outs, couts):
            if o.numel:
                idx = _sample_idx(o.shape, o.numel, rng)
                where.append(co.offset // esize + idx)
                want.append(oracle.decode(o, data, idx, out_dtype))
        where = torch.from_numpy(np.concatenate(where)).to(DEV)
        got = ck.arena.view(ibits)[where].cpu().numpy()
        want = np.concatenate(want)
        bad = np.flatnonzero(got.view(want.dtype) != want)
        assert bad.size == 0, f"{bad.size} sampled elements differ from the oracle"
        whole = {kind: 0 for kind in QUANT}
        for o, co in zip(outs, couts):
            if o.kind in QUANT and whole[o.kind] < 4:
                ref = _torch_reference(o.kind, o.shape, ck.blob, ents[co.tensor].begin,
                                       ents[co.scale].begin, ents[co.scale2].begin if co.scale2 >= 0 else 0, tdt)
                got_t = ck.tensors[o.name].reshape(-1)
                assert got_t.dtype == tdt
                assert torch.equal(got_t.view(ibits), ref.view(ibits)), f"{o.name}: whole tensor differs"
                whole[o.kind] += 1
        print(f"config {k} into {out_dtype}: {len(outs)} outputs sampled; checked whole: {whole}", flush=True)
        del ck
    finally:
        os.remove(path)
        torch.cuda.empty_cache()


def _staged_from_header(tensors, fill):
    """A checkpoint too large to write out: the index is built from its header alone and the blob
    is filled on the GPU by ``fill(data_section, offsets)``."""
    lay = layout([Group([TensorSpec(n, d, s)], None) for n, d, s in tensors])
    ix = st.SafeTensorIndex.from_bytes(lay.header, file_size=len(lay.header) + lay.data_size)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    fill(ck.blob[: lay.data_size], lay.offsets)
    ck.arena.view(torch.int16).fill_(0x5A5A)
    return ck, lay


def _random_bytes(dst, gen, no_nan_e4m3=False):
    for start in range(0, dst.numel(), 1 << 30):
        end = min(dst.numel(), start + (1 << 30))
        if no_nan_e4m3:   # every code but 0x7F and 0xFF
            r = torch.randint(0, 254, (end - start,), device=DEV, dtype=torch.int32, generator=gen)
            dst[start:end] = (r + (r >= 0x7F).int()).to(torch.uint8)
        else:
            dst[start:end] = torch.randint(0, 256, (end - start,), device=DEV, dtype=torch.uint8, generator=gen)


def test_passthrough_beyond_2_32_elements():
    n = (1 << 32) + 1000           # element and byte offsets past 32 bits; the bytes never repeat
    print(f"max size: BF16 [{n}]", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(11)
    ck, lay = _staged_from_header([("big", "BF16", (n,))], lambda blob, offs: _random_bytes(blob, gen))
    ck.materialize()
    torch.cuda.synchronize()
    assert torch.equal(ck.tensors["big"].view(torch.uint8), ck.blob[: 2 * n])
    del ck
    torch.cuda.empty_cache()


def test_block_fp8_near_the_2_32_element_limit():
    m, n = 65535, 65536 - 16       # numel just under 2^32; ragged last block row and column
    gm, gn = -(-m // 128), -(-n // 128)
    print(f"max size: block FP8 [{m}, {n}]", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(7)

    def fill(blob, offs):
        b, e = offs["w.weight"]
        _random_bytes(blob[b:e], gen, no_nan_e4m3=True)
        sb, se = offs["w.weight_scale_inv"]
        S = torch.pow(10.0, torch.rand(gm * gn, device=DEV, generator=gen) * 2 - 4)
        blob[sb:se].copy_(S.float().view(torch.uint8))

    ck, lay = _staged_from_header([("w.weight", "F8_E4M3", (m, n)),
                                   ("w.weight_scale_inv", "F32", (gm, gn))], fill)
    ck.materialize()
    torch.cuda.synchronize()
    out = ck.tensors["w.weight"]
    b, _ = lay.offsets["w.weight"]
    S = _f32(ck.blob, lay.offsets["w.weight_scale_inv"][0], gm * gn).view(gm, gn)
    for r0 in range(0, m, 8192):   # the whole tensor, in bands of 64 block rows
        r1 = min(m, r0 + 8192)
        w = _e4m3(ck.blob[b + r0 * n: b + r1 * n]).view(r1 - r0, n)
        ref = (w * _expand_grid(S[r0 // 128:], r1 - r0, n)).to(torch.bfloat16)
        assert torch.equal(out[r0:r1].view(torch.int16), ref.view(torch.int16)), f"rows {r0}:{r1}"
    del ck
    torch.cuda.empty_cache()


def test_scaled_fp8_unaligned_beyond_2_31_bytes():
    n = (1 << 31) + (1 << 20) + 3  # source starts 9 bytes in, ends past 2^31 bytes, ragged tail
    print(f"max size: scaled FP8 [{n}]", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(3)

    def fill(blob, offs):
        _random_bytes(blob[slice(*offs["pad.weight"])], gen, no_nan_e4m3=True)
        blob[slice(*offs["pad.scale_weight"])].copy_(torch.tensor([1.0], device=DEV).view(torch.uint8))
        _random_bytes(blob[slice(*offs["q.weight"])], gen, no_nan_e4m3=True)
        blob[slice(*offs["q.scale_weight"])].copy_(torch.tensor([0.0123], device=DEV).view(torch.uint8))

    ck, lay = _staged_from_header([("pad.weight", "F8_E4M3", (5,)), ("pad.scale_weight", "F32", ()),
                                   ("q.weight", "F8_E4M3", (n,)), ("q.scale_weight", "F32", ())], fill)
    ck.materialize()
    torch.cuda.synchronize()
    for name, size in (("pad", 5), ("q", n)):
        b, _ = lay.offsets[f"{name}.weight"]
        s = _f32(ck.blob, lay.offsets[f"{name}.scale_weight"][0], 1)
        out = ck.tensors[f"{name}.weight"]
        for start in range(0, size, 1 << 28):
            end = min(size, start + (1 << 28))
            ref = (_e4m3(ck.blob[b + start: b + end]) * s).to(torch.bfloat16)
            assert torch.equal(out[start:end].view(torch.int16), ref.view(torch.int16)), f"{name} {start}:{end}"
    del ck
    torch.cuda.empty_cache()


def test_launch_beyond_2_22_workgroups():
    """Five per-tensor FP8 tensors of 2^32 elements each (the last one 777 elements longer, starting
    off its 8-byte word): 20,971,521 work units of 1024 elements, 5,242,881 workgroups, so the grid
    takes a second row (its first holds 2^22 workgroups).  Every element is checked in bands
    against torch's e4m3 decode times the scale rounded to bf16, and sampled elements of every
    tensor against the oracle."""
    n = 1 << 32
    sizes = [n, n, n, n, n + 777]
    names = [f"b{i}" for i in range(5)]
    spec = []
    for nm, size in zip(names, sizes):
        spec += [(f"{nm}.weight", "F8_E4M3", (size,)), (f"{nm}.scale_weight", "F32", ())]
    scales = [0.001 * (i + 1) + 0.0007 for i in range(5)]
    print(f"grid beyond 2^22 workgroups: 5 scaled-FP8 tensors, {sum(sizes)} elements", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(5)

    def fill(blob, offs):
        for nm, sc in zip(names, scales):
            _random_bytes(blob[slice(*offs[f"{nm}.weight"])], gen, no_nan_e4m3=True)
            blob[slice(*offs[f"{nm}.scale_weight"])].copy_(torch.tensor([sc], device=DEV).view(torch.uint8))

    ck, lay = _staged_from_header(spec, fill)
    assert ck.units > 1 << 24, ck.units
    assert -(-ck.units // 4) > 1 << 22
    ck.materialize()
    torch.cuda.synchronize()
    band = 1 << 28
    for nm, size in zip(names, sizes):
        b, _ = lay.offsets[f"{nm}.weight"]
        s = _f32(ck.blob, lay.offsets[f"{nm}.scale_weight"][0], 1)
        out = ck.tensors[f"{nm}.weight"]
        for start in range(0, size, band):
            end = min(size, start + band)
            ref = (_e4m3(ck.blob[b + start: b + end]) * s).to(torch.bfloat16)
            assert torch.equal(out[start:end].view(torch.int16), ref.view(torch.int16)), f"{nm} {start}:{end}"
    # sampled elements against the oracle, from the header and the bytes around each sample
    h = oracle.parse_header(lay.header)
    outs = {o.name: o for o in oracle.classify(h)}
    rng = np.random.default_rng(22)
    checked = 0
    for nm, size in zip(names, sizes):
        o = outs[f"{nm}.weight"]
        idx = np.unique(np.concatenate([[0, size - 1, size - 777, (1 << 32) - 1], rng.integers(0, size, 4096)]))
        idx = idx[idx < size]
        lo = o.src.begin
        codes = ck.blob[lo + torch.from_numpy(idx).to(DEV)].cpu().numpy()
        data = np.zeros(o.scale.end, dtype=np.uint8)   # the data section, sparse: sampled codes + the scale
        data[lo + idx] = codes
        data[o.scale.begin: o.scale.end] = ck.blob[o.scale.begin: o.scale.end].cpu().numpy()
        want = oracle.decode(o, data, idx)
        got = ck.tensors[o.name][torch.from_numpy(idx).to(DEV)].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want), o.name
        checked += idx.size
    print(f"grid beyond 2^22 workgroups: {ck.units} units, bands exact, {checked} sampled elements equal the oracle",
          flush=True)
    del ck
    torch.cuda.empty_cache()
