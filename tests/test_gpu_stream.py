"""GPU parity of the overlapped streaming load (st_stream_file): every output equals the oracle on
the small checkpoints (whole tensors, many steps), and at full size the streamed arena equals the
one a serial stage + materialise produces, bit for bit."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import device_checkpoint_dequantisation_amd as st

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _write(tmp_path, name, buf):
    path = str(tmp_path / name)
    with open(path, "wb") as f:
        f.write(buf)
    return path


def _stream(path, chunk_mb=None, chunk_bytes=None, stream=None):
    ix = st.SafeTensorIndex.open(path)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.arena.view(torch.int16).fill_(0x5A5A)
    plan = st.StreamPlan(ix, chunk_bytes) if chunk_bytes else None
    stats = ck.stream(path, chunk_mb=chunk_mb or 64, stream=stream, plan=plan)
    ck.synchronize()
    return ck, stats


@pytest.mark.parametrize("variant", ["c1", "c2", "c3", "c4", "c5", "c6", "c7", "c2_scales_last"])
@pytest.mark.parametrize("chunk", [64 << 10, 300_000])
def test_stream_small_matches_oracle(variant, chunk, tmp_path):
    k = int(variant[1])
    buf = synth.config_bytes(k, small=k != 1, **({"scales_last": True} if "scales_last" in variant else {}))
    path = _write(tmp_path, f"{variant}.safetensors", buf)
    print(f"stream {variant} chunk {chunk}", flush=True)
    ck, stats = _stream(path, chunk_bytes=chunk)
    assert stats["bytes_read"] == ck.index.data_size
    assert stats["launches"] >= 1 and 0 <= stats["seconds_first_launch"] <= stats["seconds_read"] + 1.0
    want = oracle.materialize(buf)
    for name, w in want.items():
        got = ck.tensors[name].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got.reshape(w.shape), w), name


def test_stream_on_a_side_stream_and_twice(tmp_path):
    buf = synth.config_bytes(4, small=True)
    path = _write(tmp_path, "c4.safetensors", buf)
    ix = st.SafeTensorIndex.open(path)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    s = torch.cuda.Stream(DEV)
    plan = st.StreamPlan(ix, 64 << 10)
    ck.stream(path, stream=s, plan=plan)
    ck.synchronize()
    first = ck.arena.clone()
    ck.arena.view(torch.int16).fill_(0)
    ck.stream(path, stream=s, plan=plan)  # the same plan and ring again
    ck.synchronize()
    assert torch.equal(first.view(torch.int16), ck.arena.view(torch.int16))
    want = oracle.materialize(buf)
    for name, w in want.items():
        assert np.array_equal(ck.tensors[name].view(torch.int16).cpu().numpy().view(np.uint16), w), name


@pytest.mark.parametrize("k,extra", [(2, {}), (2, {"scales_last": True}), (3, {}), (4, {}), (5, {})])
def test_stream_full_size_equals_serial(k, extra, tmp_path):
    path = str(tmp_path / f"c{k}.safetensors")
    print(f"full-size stream c{k} {extra}: writing", flush=True)
    synth.write_config(k, path, **extra)
    try:
        ix = st.SafeTensorIndex.open(path)
        serial = st.DeviceCheckpoint(ix, path, DEV)
        serial.arena.view(torch.int16).fill_(0x5A5A)  # the gaps between outputs match the streamed arena's
        serial.materialize()
        torch.cuda.synchronize()
        ref = serial.arena.view(torch.int16).clone()
        del serial
        torch.cuda.empty_cache()
        ck, stats = _stream(path, chunk_mb=64)
        print(f"c{k}: {stats}", flush=True)
        assert stats["bytes_read"] == ix.data_size
        assert torch.equal(ck.arena.view(torch.int16), ref)
        # and a sample against the oracle, straight from the file
        mm = np.memmap(path, dtype=np.uint8, mode="r")
        h, outs = oracle.plan(mm)
        data = mm[h.data_offset:]
        rng = np.random.default_rng(k)
        for o in outs[:: max(1, len(outs) // 50)]:
            if o.numel == 0:
                continue
            idx = np.unique(np.concatenate([[0, o.numel - 1], rng.integers(0, o.numel, 64)]))
            got = ck.tensors[o.name].reshape(-1)[torch.from_numpy(idx).to(DEV)].view(torch.int16).cpu().numpy()
            assert np.array_equal(got.view(np.uint16), oracle.decode(o, data, idx)), o.name
        del ck
    finally:
        os.remove(path)
        torch.cuda.empty_cache()
