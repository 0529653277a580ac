"""A plain safetensors writer for synthetic checkpoints.

File layout written (the safetensors format): an 8-byte little-endian header length N, N bytes
of JSON header, then the data section.  Each header entry maps a tensor name to its dtype
string, shape and ``data_offsets = [begin, end]`` relative to the data section; an optional
``__metadata__`` object maps strings to strings.

Unlike the safetensors library, which orders tensors by dtype alignment and pads the header to
a multiple of 8, this writer keeps the caller's order and can leave the header unpadded, so
tensors may start at any byte offset (the back-to-back packing the synthetic checkpoints ask
for).  Tensor bytes come from *groups*: one seeded callable produces the bytes of a weight and
of the scale tensors that belong to it, so a weight is always quantised with its own scale.
"""
from __future__ import annotations

import json
import os
import threading
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Callable, Sequence

import numpy as np

# Bits per element of the safetensors dtype strings the writer accepts.
DTYPE_BITS = {
    "BOOL": 8, "U8": 8, "I8": 8, "F8_E4M3": 8, "F8_E5M2": 8, "F8_E8M0": 8,
    "I16": 16, "U16": 16, "F16": 16, "BF16": 16,
    "I32": 32, "U32": 32, "F32": 32,
    "I64": 64, "U64": 64, "F64": 64,
    "F4": 4,
}


def nbytes_of(dtype: str, shape: Sequence[int]) -> int:
    numel = 1
    for s in shape:
        numel *= int(s)
    bits = numel * DTYPE_BITS[dtype]
    if bits % 8:
        raise ValueError(f"{dtype}{list(shape)} is not a whole number of bytes")
    return bits // 8


@dataclass
class TensorSpec:
    name: str
    dtype: str
    shape: tuple

    @property
    def nbytes(self) -> int:
        return nbytes_of(self.dtype, self.shape)


@dataclass
class Group:
    """Tensors whose bytes one seeded callable produces together (a weight and its scales)."""
    tensors: list
    make: Callable  # (np.random.Generator) -> list of uint8 arrays, one per tensor
    seed: tuple = ()
    cost: int = field(default=0)  # bytes produced; used to order parallel work


@dataclass
class Layout:
    header: bytes          # 8-byte length + JSON (+ padding)
    data_size: int
    offsets: dict          # name -> (begin, end) within the data section
    order: list            # tensor names in file order


def layout(groups: Sequence[Group], metadata: dict | None = None, pad_header: bool = False) -> Layout:
    obj = {}
    if metadata:
        obj["__metadata__"] = {str(k): str(v) for k, v in metadata.items()}
    pos = 0
    offsets = {}
    order = []
    for g in groups:
        for t in g.tensors:
            if t.name in offsets or t.name == "__metadata__":
                raise ValueError(f"duplicate tensor name {t.name!r}")
            b, e = pos, pos + t.nbytes
            obj[t.name] = {"dtype": t.dtype, "shape": [int(s) for s in t.shape], "data_offsets": [b, e]}
            offsets[t.name] = (b, e)
            order.append(t.name)
            pos = e
    text = json.dumps(obj, separators=(",", ":")).encode("utf-8")
    if pad_header:
        text += b" " * ((-len(text)) % 8)
    return Layout(header=len(text).to_bytes(8, "little") + text, data_size=pos, offsets=offsets, order=order)


def _group_bytes(g: Group) -> list:
    rng = np.random.default_rng(list(g.seed))
    parts = g.make(rng)
    if len(parts) != len(g.tensors):
        raise RuntimeError("group produced the wrong number of tensors")
    out = []
    for t, p in zip(g.tensors, parts):
        p = np.ascontiguousarray(p).view(np.uint8).reshape(-1)
        if p.size != t.nbytes:
            raise RuntimeError(f"{t.name}: generated {p.size} bytes, expected {t.nbytes}")
        out.append(p)
    return out


def build_bytes(groups: Sequence[Group], metadata: dict | None = None, pad_header: bool = False) -> bytes:
    """Whole file in memory (small checkpoints)."""
    lay = layout(groups, metadata, pad_header)
    buf = bytearray(len(lay.header) + lay.data_size)
    buf[: len(lay.header)] = lay.header
    base = len(lay.header)
    for g in groups:
        for t, p in zip(g.tensors, _group_bytes(g)):
            b, e = lay.offsets[t.name]
            buf[base + b: base + e] = p.tobytes()
    return bytes(buf)


def write_file(path: str, groups: Sequence[Group], metadata: dict | None = None,
               pad_header: bool = False, workers: int | None = None, progress=None) -> Layout:
    """Write the checkpoint to ``path``; groups are generated in parallel threads and written
    with positioned writes, so peak memory is a few groups, not the whole file."""
    lay = layout(groups, metadata, pad_header)
    base = len(lay.header)
    fd = os.open(path, os.O_RDWR | os.O_CREAT | os.O_TRUNC, 0o644)
    try:
        os.ftruncate(fd, base + lay.data_size)
        os.pwrite(fd, lay.header, 0)
        lock = threading.Lock()
        done = [0]

        def job(g: Group):
            for t, p in zip(g.tensors, _group_bytes(g)):
                b, _ = lay.offsets[t.name]
                mv = memoryview(p)
                off = 0
                while off < len(mv):
                    off += os.pwrite(fd, mv[off:], base + b + off)
            if progress is not None:
                with lock:
                    done[0] += 1
                    progress(done[0], len(groups))

        nw = workers or min(16, os.cpu_count() or 1)
        # Largest groups first keeps the pool busy to the end.
        todo = sorted(groups, key=lambda g: -g.cost)
        with ThreadPoolExecutor(max_workers=nw) as ex:
            for f in [ex.submit(job, g) for g in todo]:
                f.result()
    finally:
        os.close(fd)
    return lay
