"""Checkpoints of several shard files on the GPU: load_checkpoint (from the index JSON and from the
directory) and ShardedStateDict equal the oracle's decode of each shard file, element for element, and
progress reports every shard against the known total."""
import numpy as np
import pytest
import torch

import oracle
import device_checkpoint_dequantisation_amd as st
from tests.st_files import write_sharded

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _want(bufs, out_dtype="bf16"):
    want = {}
    for b in bufs:
        want.update(oracle.materialize(b, out_dtype))
    return want


def _bits(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("streamed", [True, False])
def test_load_checkpoint_equals_the_oracle(k, streamed, tmp_path):
    files, where, bufs = write_sharded(tmp_path, k, 3)
    want = _want(bufs)
    seen = []
    print(f"sharded load c{k} streamed {streamed}: {len(files)} shards", flush=True)
    got = st.load_checkpoint(str(tmp_path / "model.safetensors.index.json"), DEV, streamed=streamed,
                             progress=lambda *a: seen.append(a))
    torch.cuda.synchronize()
    assert sorted(got) == sorted(want)
    for name, w in want.items():
        assert np.array_equal(_bits(got[name]).reshape(w.shape).view(w.dtype), w), name
    total = sum(len(b) - (8 + int.from_bytes(b[:8], "little")) for b in bufs)
    assert [s[:2] for s in seen] == [(i + 1, len(files)) for i in range(len(files))]
    assert seen[-1][3] == seen[-1][4] == total


def test_directory_without_index_and_fp32_outputs(tmp_path):
    files, _, bufs = write_sharded(tmp_path, 4, 2, index_name=None)
    want = _want(bufs, "f32")
    got = st.load_checkpoint(str(tmp_path), DEV, out_dtype="f32")
    torch.cuda.synchronize()
    for name, w in want.items():
        assert got[name].dtype == torch.float32
        assert np.array_equal(_bits(got[name]).reshape(w.shape).view(w.dtype), w), name


@pytest.mark.parametrize("ram", [0, 1 << 28])
def test_sharded_state_dict(ram, tmp_path):
    files, where, bufs = write_sharded(tmp_path, 3, 3)
    want = _want(bufs)
    sd = st.ShardedStateDict(str(tmp_path), DEV, ram_cache_bytes=ram)
    assert sorted(sd) == sorted(want) and len(sd) == len(want)
    names = list(sd)
    pick = names[::3] + names[1::7]            # keys from every shard in one load
    got = sd.load(pick)
    torch.cuda.synchronize()
    assert list(got) == list(dict.fromkeys(pick))
    for name in got:
        w = want[name]
        assert sd.meta(name).shape == w.shape and sd.file_of(name) == where[name]
        assert np.array_equal(_bits(got[name]).reshape(w.shape).view(w.dtype), w), name
    one = sd[names[-1]]
    torch.cuda.synchronize()
    assert np.array_equal(_bits(one).reshape(want[names[-1]].shape).view(np.uint16), want[names[-1]])
