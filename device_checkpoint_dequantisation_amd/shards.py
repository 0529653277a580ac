"""Checkpoints stored as several safetensors files (shards).

A large checkpoint is usually split into shard files plus an index JSON whose ``weight_map`` names
the file of every tensor; the serving document tracks loading progress against the checkpoint's known
shard totals ("Resident Modal LLM Architecture", "Request Path" and "Progress And Streaming").  Each
shard is an ordinary safetensors file and goes through the same path as one file: its own metadata
index, staging and one grouped decode.  Before any device memory is touched, every shard's header is
indexed (metadata only), the index JSON is checked against the headers, and the device memory the
whole checkpoint needs is compared with what is free, failing with both numbers.

A quantised weight and its scale tensors must sit in the same shard, since each file is decoded on its
own; a checkpoint that splits them fails with the names and files involved.
"""
from __future__ import annotations

import json
import os
from collections.abc import Mapping

from . import SafeTensorIndex, StError, _torch, load
from .lazy import StreamStateDict


class ShardError(RuntimeError):
    """A shard whose header cannot be indexed; ``code`` is the library's st_status."""

    def __init__(self, msg: str, code: int):
        super().__init__(msg)
        self.code = code


# scale tensors that belong to the weight "X.weight" (the suffixes the index pairs by name)
_SCALE_SUFFIXES = (".scale_weight", ".weight_scale_inv", ".weight_scale_2", ".weight_scale")


def _weight_of(name: str):
    for s in _SCALE_SUFFIXES:
        if name.endswith(s):
            return name[: -len(s)] + ".weight"
    return None


def shard_files(path: str) -> tuple:
    """(files, weight_map) of the checkpoint at ``path``: one ``.safetensors`` file; an index JSON
    (``weight_map``: tensor name -> file name relative to the JSON's directory); or a directory,
    which uses its single ``*.safetensors.index.json`` if it has one and otherwise every
    ``*.safetensors`` file in it, in name order.  ``weight_map`` is None without an index JSON."""
    if os.path.isdir(path):
        idx = sorted(f for f in os.listdir(path) if f.endswith(".safetensors.index.json"))
        if len(idx) > 1:
            raise ValueError(f"{path}: several index files ({', '.join(idx)}); pass the one to load")
        if idx:
            return shard_files(os.path.join(path, idx[0]))
        files = sorted(os.path.join(path, f) for f in os.listdir(path) if f.endswith(".safetensors"))
        if not files:
            raise FileNotFoundError(f"{path}: no .safetensors files")
        return files, None
    if path.endswith(".json"):
        with open(path) as fh:
            doc = json.load(fh)
        wm = doc.get("weight_map") if isinstance(doc, dict) else None
        if not isinstance(wm, dict) or not wm or not all(isinstance(k, str) and isinstance(v, str) for k, v in wm.items()):
            raise ValueError(f"{path}: no weight_map of tensor names to file names")
        base = os.path.dirname(os.path.abspath(path))
        files = sorted({os.path.join(base, v) for v in wm.values()})
        missing = [f for f in files if not os.path.isfile(f)]
        if missing:
            raise FileNotFoundError(f"{path}: shard files listed in weight_map are missing: {', '.join(missing)}")
        return files, {k: os.path.join(base, v) for k, v in wm.items()}
    if not os.path.isfile(path):
        raise FileNotFoundError(path)
    return [path], None


def index_shards(path: str, out_dtype: str = "bf16") -> list:
    """[(file, SafeTensorIndex)] of every shard, from the headers alone, after checking that the
    shards' tensors are distinct, that the index JSON (if any) lists exactly the tensors each header
    holds, and that no weight is split from its scales."""
    files, wm = shard_files(path)
    where = {}
    out = []
    for f in files:
        try:
            ix = SafeTensorIndex.open(f, out_dtype=out_dtype)
        except StError as e:
            pair = _split_pairs(f, wm)
            raise ShardError(f"shard {f}: {e}" + (f"; {pair}" if pair else ""), e.code) from e
        for t in ix.tensors():
            if t.name in where:
                raise ValueError(f"tensor {t.name} is in two shards: {where[t.name]} and {f}")
            where[t.name] = f
        out.append((f, ix))
    if wm is not None:
        for name, f in wm.items():
            if where.get(name) != f:
                raise ValueError(f"the index lists {name} in {f}, but "
                                 + (f"its header is in {where[name]}" if name in where else "no shard holds it"))
        extra = sorted(set(where) - set(wm))
        if extra:
            raise ValueError(f"shard headers hold tensors the index does not list: {', '.join(extra[:8])}")
    return out


def _split_pairs(f: str, wm) -> str:
    """A description of the scale tensors the index JSON puts in another file than their weight."""
    if not wm:
        return ""
    bad = []
    for name, file in wm.items():
        w = _weight_of(name)
        if w is not None and w in wm and wm[w] != file and f in (file, wm[w]):
            bad.append(f"{w} is in {wm[w]} but {name} is in {file}")
    if not bad:
        return ""
    return ("a quantised weight and its scales must share a shard file, since each file is decoded on its own: "
            + "; ".join(bad[:4]) + (" ..." if len(bad) > 4 else ""))


def device_bytes_needed(shards) -> int:
    """Device memory a sequential load of ``shards`` ([(file, SafeTensorIndex)]) holds at its peak:
    every shard's outputs, plus the largest shard's staging blob and work table."""
    outs = sum(ix.arena_bytes for _, ix in shards)
    return outs + max((ix.device_bytes - ix.arena_bytes for _, ix in shards), default=0)


def load_checkpoint(path: str, device="cuda", out_dtype: str = "bf16", streamed: bool = True, chunk_mb: int = 128,
                    progress=None, check_vram: bool = True) -> dict:
    """Every output of a checkpoint of one or several shard files (see shard_files) as tensors on
    ``device``, one shard after the other through ``load``.  ``progress(done, total, file,
    bytes_done, bytes_total)`` is called after each shard, with the shard total known up front."""
    shards = index_shards(path, out_dtype)
    torch = _torch()
    dev = torch.device(device)
    if check_vram and dev.type == "cuda":
        free, total = torch.cuda.mem_get_info(dev)
        need = device_bytes_needed(shards)
        if need > free:
            raise MemoryError(f"checkpoint of {len(shards)} shards needs {need} bytes of device memory; "
                              f"{free} of {total} are free")
    total_bytes = sum(ix.data_size for _, ix in shards)
    done_bytes = 0
    tensors = {}
    for k, (f, ix) in enumerate(shards):
        tensors.update(load(f, dev, streamed=streamed, chunk_mb=chunk_mb, out_dtype=out_dtype))
        done_bytes += ix.data_size
        if progress is not None:
            progress(k + 1, len(shards), f, done_bytes, total_bytes)
    return tensors


class ShardedStateDict(Mapping):
    """StreamStateDict over the shard files of one checkpoint: keys from every header (metadata
    only), each load decoded from the shards that hold the requested keys.  ``ram_cache_bytes`` is
    the RAM tier of each shard."""

    def __init__(self, path: str, device="cuda", ram_cache_bytes: int = 0, out_dtype: str = "bf16", **kw):
        shards = index_shards(path, out_dtype)
        self.files = [f for f, _ in shards]
        self.parts = [StreamStateDict(f, device, ram_cache_bytes=ram_cache_bytes, index=ix, out_dtype=out_dtype, **kw)
                      for f, ix in shards]
        self._where = {}
        for part in self.parts:
            for key in part:
                self._where[key] = part
        self._keys = [key for part in self.parts for key in part]

    def __iter__(self):
        return iter(self._keys)

    def __len__(self):
        return len(self._keys)

    def __contains__(self, name):
        return name in self._where

    def meta(self, name: str):
        return self._where[name].meta(name)

    def meta_tensor(self, name: str):
        return self._where[name].meta_tensor(name)

    def file_of(self, name: str) -> str:
        return self._where[name].path

    def __getitem__(self, name: str):
        return self.load([name])[name]

    def load(self, names, stream=None) -> dict:
        """Decode ``names`` (grouped by shard, one load per shard) into fresh tensors."""
        names = list(dict.fromkeys(names))
        by_part = {}
        for n in names:
            by_part.setdefault(id(self._where[n]), (self._where[n], []))[1].append(n)  # KeyError for an unknown name
        out = {}
        for part, group in by_part.values():
            out.update(part.load(group, stream=stream))
        return {n: out[n] for n in names}
