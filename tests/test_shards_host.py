"""Checkpoints of several shard files, on the CPU: finding the shard files (one file, a directory, an
index JSON), indexing their headers without reading tensor bytes, and every refusal (missing files,
tensors in two shards, an index that disagrees with the headers, a weight split from its scales)."""
import json
import os

import pytest

import device_checkpoint_dequantisation_amd as st
from tests.st_files import write_sharded


def test_shard_files_of_a_file_a_directory_and_an_index(tmp_path):
    files, where, _ = write_sharded(tmp_path, 3, 3)
    assert st.shard_files(files[1]) == ([files[1]], None)
    idx = str(tmp_path / "model.safetensors.index.json")
    got, wm = st.shard_files(idx)
    assert got == sorted(files) and wm == where
    assert st.shard_files(str(tmp_path)) == (got, wm)          # the directory uses its index JSON
    os.remove(idx)
    assert st.shard_files(str(tmp_path)) == (sorted(files), None)   # otherwise every .safetensors file


def test_index_shards_reads_headers_only(tmp_path):
    files, where, bufs = write_sharded(tmp_path, 2, 4)
    shards = st.index_shards(str(tmp_path))
    assert [f for f, _ in shards] == sorted(files)
    names = [t.name for _, ix in shards for t in ix.tensors()]
    assert sorted(names) == sorted(where)
    outs = [o.name for _, ix in shards for o in ix.outputs()]
    assert len(outs) == len(set(outs)) and all(not n.endswith("scale_weight") for n in outs)
    # peak device memory of a sequential load: all outputs plus the largest shard's blob and table
    need = st.shards.device_bytes_needed(shards)
    assert need == sum(ix.arena_bytes for _, ix in shards) + max(ix.device_bytes - ix.arena_bytes for _, ix in shards)


def test_refusals(tmp_path):
    files, where, _ = write_sharded(tmp_path, 2, 3)
    idx = tmp_path / "model.safetensors.index.json"
    doc = json.loads(idx.read_text())
    # a listed file that does not exist
    bad = dict(doc, weight_map=dict(doc["weight_map"], extra="model-00009-of-00009.safetensors"))
    p = tmp_path / "missing.index.json"
    p.write_text(json.dumps(bad))
    with pytest.raises(FileNotFoundError, match="missing"):
        st.shard_files(str(p))
    # an index that puts a tensor in the wrong file
    name = next(iter(doc["weight_map"]))
    other = [os.path.basename(f) for f in files if os.path.basename(f) != doc["weight_map"][name]][0]
    wrong = dict(doc, weight_map=dict(doc["weight_map"], **{name: other}))
    p = tmp_path / "wrong.index.json"
    p.write_text(json.dumps(wrong))
    with pytest.raises(ValueError, match="lists"):
        st.index_shards(str(p))
    # an index that leaves a tensor out
    short = dict(doc, weight_map={k: v for k, v in doc["weight_map"].items() if k != name})
    p = tmp_path / "short.index.json"
    p.write_text(json.dumps(short))
    with pytest.raises(ValueError, match="does not list"):
        st.index_shards(str(p))
    # not an index
    p = tmp_path / "bad.index.json"
    p.write_text("[1, 2]")
    with pytest.raises(ValueError, match="weight_map"):
        st.shard_files(str(p))
    # two index files in one directory
    (tmp_path / "second.safetensors.index.json").write_text(json.dumps(doc))
    with pytest.raises(ValueError, match="several index files"):
        st.shard_files(str(tmp_path))


def test_tensor_in_two_shards(tmp_path):
    files, _, bufs = write_sharded(tmp_path, 2, 3, index_name=None)
    with open(str(tmp_path / "model-00004-of-00005.safetensors"), "wb") as fh:
        fh.write(bufs[0])                          # a copy of the first shard's tensors
    with pytest.raises(ValueError, match="two shards"):
        st.index_shards(str(tmp_path))


def test_weight_split_from_its_scales(tmp_path):
    write_sharded(tmp_path, 2, 3, split_pair=True)
    with pytest.raises(st.ShardError, match="must share a shard file") as e:
        st.index_shards(str(tmp_path / "model.safetensors.index.json"))
    assert e.value.code == -8   # ST_E_SCALE
