"""Lazy, on-demand materialisation over the C ABI: a state dict whose keys come from the header
alone and whose tensors are decoded on the GPU when asked for, views over it, a RAM tier of raw
(still quantised) checkpoint bytes, and modules whose weights stay meta tensors until a
forward_pre_hook materialises them.

The design follows the pages' disk tier ("Disk tier safetensors streaming design audit",
"Strategy summary / Streaming safetensors mapping", "Range reads and tiering" and "Disk tier
integration"): a mapping with metadata-only keys that loads tensors on demand; prefix, filter and
rename views that load nothing; range reads into pinned memory, copied to the GPU; an LRU RAM cache
with a byte limit; meta tensors plus a registry of where each weight lives, materialised by a
forward_pre_hook.  Here the RAM tier keeps the checkpoint's own bytes (1 byte per fp8 element, half a
byte per e2m1 element) rather than decoded tensors, and every decode runs in the grouped kernel.
"""
from __future__ import annotations

import collections
import fnmatch
import re
import threading
import time
from collections.abc import Mapping
from dataclasses import dataclass

from . import (SafeTensorIndex, StreamPlan, _quantized, _torch, materialize, read_plans, stream_file,
               table_stream_stores)

_ONE_STEP = 1 << 60  # chunk size that keeps a whole selection in one staging step


def _round_up(x: int, a: int) -> int:
    return (x + a - 1) // a * a


def _batches(sizes, n):
    """Indices 0..len(sizes)-1 in order, cut into at most n runs of about equal total size."""
    total = sum(sizes)
    out, cur, acc = [], [], 0
    for i, sz in enumerate(sizes):
        cur.append(i)
        acc += sz
        if acc * n >= total * (len(out) + 1) and len(out) < n - 1:
            out.append(cur)
            cur = []
    if cur:
        out.append(cur)
    return out


@dataclass(frozen=True)
class OutputMeta:
    """What a key materialises to, known from the header alone."""
    name: str
    index: int          # output index in the checkpoint
    shape: tuple
    kind: str           # PASS_BF16, CAST_F16, CAST_F32, FP8_TENSOR, FP8_BLOCK128, NVFP4, MXFP8, MXFP4
    source_dtype: str   # safetensors dtype of the stored weight
    source_bytes: int   # bytes read to materialise it (weight and scale tensors)

    out_dtype: str = "bf16"  # output element type: bf16, f16 or f32

    @property
    def dtype(self):
        torch = _torch()
        return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[self.out_dtype]

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n


class PinnedArena:
    """Pinned host memory carved from slabs (first fit, coalescing frees), so that the RAM tier
    does not pin a fresh allocation for every entry.  Slabs are ``slab_bytes`` (or one entry's
    size, if larger) and are allocated on demand, never more than ``max_bytes`` in total.

    With ``prefetch`` (the default for real pinned memory), a background thread keeps one spare
    slab allocated and touched ahead of need: the first write to a freshly pinned page maps it, and
    done inside a file read that mapping made filling the tier several times slower than reading
    into pages already touched (measured on MI355X hosts: about 12 against 70 GB/s)."""

    def __init__(self, max_bytes: int, slab_bytes: int = 256 << 20, allocate=None, prefetch: bool | None = None):
        self.max_bytes = int(max_bytes)
        self.slab_bytes = max(256, min(int(slab_bytes), self.max_bytes))
        self.allocate = allocate or (lambda n: _torch().empty(n, dtype=_torch().uint8, pin_memory=True))
        self.slabs = []      # pinned uint8 tensors
        self.free = []       # per slab: sorted list of [offset, size] holes
        self.allocated = 0
        self.prefetch = (allocate is None) if prefetch is None else bool(prefetch)
        self._spare = None         # a touched slab of slab_bytes, not yet in use
        self._spare_thread = None
        self._spare_error = None
        if self.prefetch:
            self._start_spare()

    @property
    def capacity(self) -> int:
        """Bytes of the slabs in use, plus a spare slab being prepared or ready."""
        spare = self.slab_bytes if (self._spare_thread is not None or self._spare is not None) else 0
        return sum(t.numel() for t in self.slabs) + spare

    def _start_spare(self):
        """Allocate and touch the next slab in a background thread, if one more slab fits."""
        if not self.prefetch or self._spare_thread is not None or self._spare is not None:
            return
        if sum(t.numel() for t in self.slabs) + 2 * self.slab_bytes > self.max_bytes:
            return   # keep room for a slab of one large entry

        def work(size=self.slab_bytes):
            try:
                t = self.allocate(size)
                t.fill_(0)   # first touch of every page, off the read path
                self._spare = t
            except BaseException as e:  # reported when the slab is wanted
                self._spare_error = e

        self._spare_thread = threading.Thread(target=work, name="pinned-arena-prefetch", daemon=True)
        self._spare_thread.start()

    def reserve_slabs(self, nbytes: int) -> int:
        """Allocate and touch slabs now until they hold ``nbytes`` (within ``max_bytes``), so that
        later entries land in memory that is already pinned and mapped; returns the bytes of slabs
        held.  Creating pinned memory is the slow part of filling the tier (measured on MI355X
        hosts: about 12 GB/s, and other HIP calls of the process wait meanwhile)."""
        if self._spare_thread is not None:
            self._spare_thread.join()
            self._spare_thread = None
        if self._spare is not None:      # a spare already prepared becomes a slab first
            t, self._spare = self._spare, None
            self.slabs.append(t)
            self.free.append([[0, t.numel()]])
        while sum(t.numel() for t in self.slabs) < nbytes:
            size = self.slab_bytes
            if self.capacity + size > self.max_bytes:
                break
            t = self.allocate(size)
            t.fill_(0)
            self.slabs.append(t)
            self.free.append([[0, size]])
        return self.capacity

    def _take_spare(self, n: int):
        """The spare slab if it holds n bytes (waiting for it if it is still being prepared)."""
        if self._spare_thread is not None:
            self._spare_thread.join()
            self._spare_thread = None
        if self._spare_error is not None:
            e, self._spare_error = self._spare_error, None
            raise e
        t = self._spare
        if t is None or t.numel() < n:
            return None
        self._spare = None
        return t

    def alloc(self, n: int):
        """(slab, offset) of n free bytes (256-byte aligned), or None if none is free and no new
        slab fits under max_bytes."""
        n = _round_up(max(n, 1), 256)
        for si, holes in enumerate(self.free):
            for h in holes:
                if h[1] >= n:
                    off = h[0]
                    h[0] += n
                    h[1] -= n
                    if h[1] == 0:
                        holes.remove(h)
                    self.allocated += n
                    return si, off
        slab = self._take_spare(n)
        if slab is None:
            size = max(self.slab_bytes, n)
            if self.capacity + size > self.max_bytes:
                if self._spare is None:
                    return None
                self._spare = None   # a slab of one large entry takes the spare's place
                if self.capacity + size > self.max_bytes:
                    return None
            slab = self.allocate(size)
        size = slab.numel()
        self.slabs.append(slab)
        self.free.append([[n, size - n]] if size > n else [])
        self.allocated += n
        self._start_spare()
        return len(self.slabs) - 1, 0

    def release(self, si: int, off: int, n: int):
        n = _round_up(max(n, 1), 256)
        holes = self.free[si]
        holes.append([off, n])
        holes.sort()
        merged = []
        for h in holes:
            if merged and merged[-1][0] + merged[-1][1] == h[0]:
                merged[-1][1] += h[1]
            else:
                merged.append(h)
        self.free[si] = merged
        self.allocated -= n

    def view(self, si: int, off: int, n: int):
        return self.slabs[si][off: off + n]


class _Entry:
    """One output's packed checkpoint bytes in pinned host memory, with its plan."""
    __slots__ = ("plan", "host", "table_dev", "table_ready", "nbytes", "where", "last_use")

    def __init__(self, plan, host, where=None):
        self.plan = plan
        self.host = host
        self.table_dev = None
        self.table_ready = None  # event after the upload of table_dev
        self.nbytes = host.numel()
        self.where = where     # (slab, offset) in the RAM tier's arena
        self.last_use = None   # event after the latest upload from `host`


class RamCache:
    """LRU of packed checkpoint bytes, bounded by ``max_bytes`` (0 disables it).  An entry larger
    than the bound is not kept.  Entries live in a :class:`PinnedArena`; an entry's memory is handed
    out again only after its last upload has completed, and keys in ``protected`` (the entries a
    load is using) are never evicted."""

    def __init__(self, max_bytes: int = 0, slab_bytes: int = 256 << 20):
        self.max_bytes = int(max_bytes)
        self._d = collections.OrderedDict()
        self.bytes = 0
        self.evictions = 0
        self.protected = set()
        self.arena = PinnedArena(max_bytes, slab_bytes) if max_bytes > 0 else None

    def get(self, key):
        e = self._d.get(key)
        if e is not None:
            self._d.move_to_end(key)
        return e

    def reserve(self, n: int):
        """(slab, offset) of pinned host bytes for a new entry of n bytes, evicting least recently
        used entries as needed; None if it does not fit."""
        if self.arena is None or n > self.max_bytes:
            return None
        while True:
            if self.bytes + n <= self.max_bytes:
                where = self.arena.alloc(n)
                if where is not None:
                    return where
            if not self._evict_one():
                return None

    def put(self, key, entry) -> bool:
        if entry.nbytes > self.max_bytes:
            return False
        old = self._d.pop(key, None)
        if old is not None:
            self._drop(old)
        self._d[key] = entry
        self.bytes += entry.nbytes
        while self.bytes > self.max_bytes and self._evict_one(keep=key):
            pass
        return True

    def _evict_one(self, keep=None) -> bool:
        """Evicts the least recently used entry that is neither protected nor ``keep``; the cache
        may stay above its bound while protected entries fill it."""
        for key in self._d:
            if key not in self.protected and key != keep:
                self._drop(self._d.pop(key))
                self.evictions += 1
                return True
        return False

    def _drop(self, e):
        self.bytes -= e.nbytes
        if getattr(e, "where", None) is not None and self.arena is not None:
            if e.last_use is not None:
                e.last_use.synchronize()  # an upload may still be reading these bytes
            self.arena.release(e.where[0], e.where[1], e.nbytes)
            e.where = None

    def __contains__(self, key):
        return key in self._d

    def __len__(self):
        return len(self._d)

    def keys(self):
        return list(self._d)

    def clear(self):
        for e in self._d.values():
            self._drop(e)
        self._d.clear()
        self.bytes = 0


class StreamStateDict(Mapping):
    """Mapping from output name to a tensor on ``device`` (bf16, or ``out_dtype`` f16 / f32), over
    one safetensors file.

    ``keys()``, ``len()``, ``in`` and :meth:`meta` read nothing but the header.  Indexing decodes one
    tensor on the GPU; :meth:`load` decodes several with one read and one upload.  With
    ``ram_cache_bytes`` > 0 the checkpoint bytes of recently loaded outputs stay in pinned host
    memory (LRU) and later loads of them skip the file.  By default (``ram_preallocate``) that memory is
    pinned and touched when the mapping is created, up to the checkpoint's size or the bound if smaller:
    creating pinned memory holds up the process's other HIP calls, and done while loads fill the tier it
    made filling about 3x slower than reading into memory already pinned (measured on MI355X hosts:
    9-13 against 35-38 GB/s); ``ram_preallocate=False`` pins slabs as loads need them instead."""

    def __init__(self, path: str, device="cuda", ram_cache_bytes: int = 0, index: SafeTensorIndex | None = None,
                 out_dtype: str = "bf16", steps_per_load: int = 8, ram_preallocate: bool = True):
        self.path = path
        self.index = index if index is not None else SafeTensorIndex.open(path, out_dtype=out_dtype)
        self.device = _torch().device(device)
        ents = self.index.tensors()
        self._meta = {}
        for k, o in enumerate(self.index.outputs()):
            src = sum(ents[i].end - ents[i].begin for i in (o.tensor, o.scale, o.scale2) if i >= 0)
            self._meta[o.name] = OutputMeta(o.name, k, tuple(o.shape), o.kind, ents[o.tensor].dtype, src,
                                            self.index.out_dtype)
        self._keys = list(self._meta)
        self.ram = RamCache(ram_cache_bytes)
        self.stats = collections.Counter()
        self._ring = None   # pinned staging ring of the direct path
        self._ring_free = None  # event after the last copy out of the ring
        self._side = None   # its copy stream
        self._stage = None  # pinned buffer for small uploads
        self._stage_done = None
        self.steps_per_load = max(1, int(steps_per_load))  # staging steps of a direct load
        self.fill_batches = 4   # file reads per load that fills the RAM tier (overlapping the uploads)
        self.ram_preallocate_seconds = 0.0
        if ram_preallocate and self.ram.arena is not None:
            # pinned slabs for the whole checkpoint (each entry is its weight and scale bytes, runs
            # aligned to 256 bytes), or for the tier's bound if that is smaller
            need = sum(m.source_bytes + 1024 for m in self._meta.values())
            t0 = time.perf_counter()
            self.ram.arena.reserve_slabs(min(need, self.ram.max_bytes))
            self.ram_preallocate_seconds = time.perf_counter() - t0

    # ---- metadata only
    def __iter__(self):
        return iter(self._keys)

    def __len__(self):
        return len(self._keys)

    def __contains__(self, name):
        return name in self._meta

    def meta(self, name: str) -> OutputMeta:
        return self._meta[name]

    def meta_tensor(self, name: str):
        """A tensor on the meta device with the output's shape and dtype (no data)."""
        m = self._meta[name]
        return _torch().empty(m.shape, dtype=m.dtype, device="meta")

    def __getitem__(self, name: str):
        return self.load([name])[name]

    # ---- loading
    def load(self, names, stream=None) -> dict:
        """Decode the outputs ``names`` into fresh tensors of the output type, enqueued on ``stream``
        (default: the current stream); returns ``{name: tensor}``."""
        torch = _torch()
        names = list(dict.fromkeys(names))
        metas = [self._meta[n] for n in names]  # KeyError for an unknown name
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        self.stats["loads"] += 1
        self.stats["outputs"] += len(names)
        if not names:
            return {}
        with torch.cuda.stream(s):
            outs = {m.name: torch.empty(m.shape, dtype=m.dtype, device=self.device) for m in metas}
            if self.ram.max_bytes > 0:
                self._load_cached(metas, outs, s)
            else:
                self._load_direct(metas, outs, s)
        return outs

    def load_quantized(self, names, stream=None) -> dict:
        """The quantised weights ``names`` as stored (no decode), read with one packed plan into a
        device blob that the returned weight tensors view; see QuantizedWeight."""
        torch = _torch()
        metas = [self._meta[n] for n in names]
        plan = StreamPlan(self.index, _ONE_STEP, select=[m.index for m in metas], pack=True)
        host = torch.empty(plan.blob_bytes, dtype=torch.uint8, pin_memory=True)
        read_plans(self.path, self.index, [plan], [host])
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        with torch.cuda.stream(s):
            blob = torch.empty(plan.blob_bytes, dtype=torch.uint8, device=self.device)
            blob.copy_(host, non_blocking=True)
            ents = self.index.tensors()
            return {m.name: _quantized(self.index, blob, m.index, lambda i: plan.tensor_offset(ents[i].begin), False)
                    for m in metas}

    def _load_direct(self, metas, outs, s):
        """One packed plan over the outputs, streamed: the steps are read into a pinned ring, copied
        on a side stream and decoded on ``s`` while later steps are read."""
        torch = _torch()
        ks = [m.index for m in metas]
        total = sum(m.source_bytes for m in metas)
        chunk = min(64 << 20, max(1 << 20, _round_up(total // self.steps_per_load + 1, 1 << 20)))
        plan = StreamPlan(self.index, chunk, select=ks, pack=True)
        need = 4 * plan.chunk_bytes
        if self._ring is None or self._ring.numel() < need:
            if self._ring_free is not None:  # the old ring's last copies must be done before it is freed
                self._ring_free.synchronize()
            self._ring = torch.empty(max(need, 4 << 20), dtype=torch.uint8, pin_memory=True)
        if self._side is None:
            self._side = torch.cuda.Stream(self.device)
        blob = torch.empty(plan.blob_bytes, dtype=torch.uint8, device=self.device)
        by_index = {m.index: m.name for m in metas}
        table, ptrs = self._upload_parts([plan.tables, self._pointer_bytes([outs[by_index[k]] for k in plan.order])])
        ptrs = ptrs.view(_torch().int64)
        self._side.wait_stream(s)  # the blob and the ring are free for this load
        t0 = time.perf_counter()
        st = stream_file(self.path, self.index, plan, blob, table, ptrs, self._ring, self._side, s)
        self.stats["stream_call_seconds"] += time.perf_counter() - t0
        self.stats["read_seconds"] += st["seconds_read"]
        self.stats["ring_wait_seconds"] += st["seconds_wait"]
        self.stats["file_bytes"] += st["bytes_read"]
        self.stats["launches"] += st["launches"]
        blob.record_stream(self._side)
        self._ring_free = torch.cuda.Event()
        self._ring_free.record(self._side)  # after this load's last copy out of the ring

    def _load_cached(self, metas, outs, s):
        """Per-output packed entries, read from the file once and then kept in the RAM tier.  Misses
        are read in a few batches of about equal bytes, and each batch's uploads and decodes are
        enqueued before the next batch is read, so that file reads overlap the host-to-device copies."""
        torch = _torch()
        entries, miss = {}, []
        plans, wheres, hosts = [], [], []
        entered = 0   # misses whose reserved memory now belongs to an entry
        try:
            for m in metas:
                e = self.ram.get(m.index)
                if e is None:
                    miss.append(m)
                else:
                    entries[m.index] = e
                    self.ram.protected.add(m.index)
                    s.wait_event(e.table_ready)  # uploaded by an earlier load, maybe on another stream
                    self.stats["ram_hits"] += 1
            if miss:
                plans = [StreamPlan(self.index, _ONE_STEP, select=[m.index], pack=True) for m in miss]
                for p in plans:  # arena memory when the entry can be kept, a transient buffer otherwise
                    w = self.ram.reserve(p.blob_bytes)
                    wheres.append(w)
                    hosts.append(self.ram.arena.view(w[0], w[1], p.blob_bytes) if w is not None
                                 else torch.empty(p.blob_bytes, dtype=torch.uint8, pin_memory=True))
                    if w is not None:  # held until the entry is in the cache, then protected
                        self.ram.bytes += p.blob_bytes
            # the tables of all new entries and the output pointers in one upload
            *tables, ptrs = self._upload_parts([p.tables for p in plans] +
                                               [self._pointer_bytes([outs[m.name] for m in metas])])
            uploaded = torch.cuda.Event()
            uploaded.record(s)
            ptrs = ptrs[: 8 * len(metas)].view(torch.int64)
            # one device blob with a 256-byte aligned segment per output, one launch per output
            nbytes = {m.index: e.nbytes for m, e in ((m, entries.get(m.index)) for m in metas) if e is not None}
            nbytes.update({m.index: p.blob_bytes for m, p in zip(miss, plans)})
            segs, total = {}, 0
            for j, m in enumerate(metas):
                segs[m.index] = (j, total)
                total += _round_up(nbytes[m.index], 256)
            blob = torch.empty(max(total, 256), dtype=torch.uint8, device=self.device)

            def decode(m, e):
                j, off = segs[m.index]
                blob[off: off + e.nbytes].copy_(e.host, non_blocking=True)
                ev = torch.cuda.Event()
                ev.record(s)
                e.last_use = ev
                for step in e.plan.steps:
                    if step.units:
                        materialize(blob[off:], e.table_dev[step.table_offset:], step.units, ptrs[j:], s,
                                    out_dtype=self.index.out_dtype,
                                    stream_stores=table_stream_stores(e.plan.tables, step.table_offset))
                        self.stats["launches"] += 1

            for m in metas:
                if m.index in entries:
                    decode(m, entries[m.index])
            for batch in _batches([p.blob_bytes for p in plans], self.fill_batches):
                t0 = time.perf_counter()
                read_plans(self.path, self.index, [plans[i] for i in batch], [hosts[i] for i in batch])
                self.stats["read_seconds"] += time.perf_counter() - t0
                self.stats["file_bytes"] += sum(e - b for i in batch for b, e in plans[i].ranges)
                for i in batch:
                    m, p, w = miss[i], plans[i], wheres[i]
                    e = _Entry(p, hosts[i], w)
                    e.table_dev = tables[i]
                    e.table_ready = uploaded
                    entries[m.index] = e
                    if w is not None:
                        self.ram.bytes -= p.blob_bytes
                        self.ram.protected.add(m.index)
                        self.ram.put(m.index, e)
                    entered = i + 1
                    self.stats["ram_misses"] += 1
                    decode(m, e)
        except BaseException:
            for p, w in list(zip(plans, wheres))[entered:]:  # give back memory no entry took
                if w is not None:
                    self.ram.bytes -= p.blob_bytes
                    self.ram.arena.release(w[0], w[1], p.blob_bytes)
            raise
        finally:
            self.ram.protected.clear()

    def _upload(self, data: bytes):
        """A device copy of a few bytes (work tables, pointer arrays), through a pinned staging
        buffer that is reused once its previous upload has completed."""
        torch = _torch()
        n = max(len(data), 1)
        if self._stage is None or self._stage.numel() < n:
            self._stage = torch.empty(max(n, 1 << 20), dtype=torch.uint8, pin_memory=True)
            self._stage_done = None
        if self._stage_done is not None:
            self._stage_done.synchronize()
        if data:
            self._stage[: len(data)].numpy()[:] = memoryview(data).cast("B")
        dev = torch.empty(_round_up(n, 256), dtype=torch.uint8, device=self.device)
        dev[:n].copy_(self._stage[:n], non_blocking=True)
        self._stage_done = torch.cuda.Event()
        self._stage_done.record(torch.cuda.current_stream(self.device))
        return dev

    def _upload_parts(self, parts):
        """Device copies of several byte strings in one upload, each 256-byte aligned."""
        offs, blob = [], bytearray()
        for part in parts:
            offs.append(len(blob))
            blob += part
            blob += bytes(_round_up(len(blob), 256) - len(blob))
        dev = self._upload(bytes(blob))
        return [dev[o: o + len(part)] for o, part in zip(offs, parts)]

    @staticmethod
    def _pointer_bytes(tensors) -> bytes:
        import struct
        return struct.pack(f"<{len(tensors)}q", *[t.data_ptr() for t in tensors])


# ----------------------------------------------------------------------------- views

class _View(Mapping):
    """A lazy view: key translation over a base mapping that has ``load``; loads nothing itself."""

    def __init__(self, base):
        self.base = base
        self._map = None

    def _build(self):  # view key -> base key, in base order
        raise NotImplementedError

    @property
    def mapping(self) -> dict:
        if self._map is None:
            self._map = self._build()
        return self._map

    def __iter__(self):
        return iter(self.mapping)

    def __len__(self):
        return len(self.mapping)

    def __contains__(self, key):
        return key in self.mapping

    def __getitem__(self, key):
        return self.base[self.mapping[key]]

    def meta(self, key) -> OutputMeta:
        return self.base.meta(self.mapping[key])

    def meta_tensor(self, key):
        return self.base.meta_tensor(self.mapping[key])

    def load(self, keys, stream=None) -> dict:
        keys = list(keys)
        got = self.base.load([self.mapping[k] for k in keys], stream=stream)
        return {k: got[self.mapping[k]] for k in keys}


class PrefixViewStateDict(_View):
    """Keys of ``base`` that start with ``prefix``, with the prefix removed (``strip=True``), or every
    key with ``prefix`` prepended (``strip=False``)."""

    def __init__(self, base, prefix: str, strip: bool = True):
        super().__init__(base)
        self.prefix, self.strip = prefix, strip

    def _build(self):
        if self.strip:
            n = len(self.prefix)
            return {k[n:]: k for k in self.base if k.startswith(self.prefix)}
        return {self.prefix + k: k for k in self.base}


class FilterViewStateDict(_View):
    """Keys of ``base`` for which ``keep(key)`` is true; ``keep`` may also be a glob pattern."""

    def __init__(self, base, keep):
        super().__init__(base)
        self.keep = (lambda k, pat=keep: fnmatch.fnmatchcase(k, pat)) if isinstance(keep, str) else keep

    def _build(self):
        return {k: k for k in self.base if self.keep(k)}


class RenameViewStateDict(_View):
    """Keys of ``base`` renamed by ``rename``: a dict (old -> new; other keys unchanged), a list of
    ``(regex, replacement)`` pairs applied in order, or a function.  Two keys renamed to the same
    name is an error."""

    def __init__(self, base, rename):
        super().__init__(base)
        if isinstance(rename, dict):
            self.fn = lambda k, d=rename: d.get(k, k)
        elif callable(rename):
            self.fn = rename
        else:
            rules = [(re.compile(p), r) for p, r in rename]

            def fn(k, rules=rules):
                for p, r in rules:
                    k = p.sub(r, k)
                return k
            self.fn = fn

    def _build(self):
        out = {}
        for k in self.base:
            n = self.fn(k)
            if n in out:
                raise KeyError(f"rename maps both {out[n]!r} and {k!r} to {n!r}")
            out[n] = k
        return out


# ----------------------------------------------------------------------------- modules

@dataclass(frozen=True)
class DiskRef:
    """Where a module parameter's data lives: a key of a lazy state dict (or view)."""
    source: object
    key: str
    meta: OutputMeta


class LazyModuleLoader:
    """Turns the parameters of ``module`` that ``state_dict`` holds into meta tensors with a
    :class:`DiskRef` each, and registers a ``forward_pre_hook`` on every submodule owning such a
    parameter: before the submodule runs, all of its meta parameters are decoded in one
    ``state_dict.load`` call.  With ``max_resident_bytes`` the materialised parameters form an LRU
    (by submodule) on the device; going over the bound turns the least recently used submodules'
    parameters back into meta tensors (their DiskRefs stay).  Parameters take the state dict's
    output type (bf16 unless the index plans f16 or f32) and do not require grad."""

    def __init__(self, module, state_dict, max_resident_bytes: int | None = None, strict: bool = True):
        torch = _torch()
        self.module = module
        self.sd = state_dict
        self.max_resident_bytes = max_resident_bytes
        self.refs = {}            # (submodule, param name) -> DiskRef
        self._owned = collections.defaultdict(list)  # submodule -> [param name]
        self._resident = collections.OrderedDict()   # submodule -> bytes, LRU order
        self.resident_bytes = 0
        self.stats = collections.Counter()
        names = {}
        for mod_name, mod in module.named_modules():
            for pname, p in list(mod.named_parameters(recurse=False)):
                full = f"{mod_name}.{pname}" if mod_name else pname
                names[full] = (mod, pname, p)
        missing = [n for n in names if n not in state_dict]
        if strict and missing:
            raise KeyError(f"{len(missing)} parameters are not in the state dict, e.g. {missing[:3]}")
        for full, (mod, pname, p) in names.items():
            if full not in state_dict:
                continue
            meta = state_dict.meta(full)
            if tuple(p.shape) != tuple(meta.shape):
                raise ValueError(f"{full}: module shape {tuple(p.shape)} != checkpoint shape {meta.shape}")
            self.refs[(mod, pname)] = DiskRef(state_dict, full, meta)
            self._owned[mod].append(pname)
            mod._parameters[pname] = torch.nn.Parameter(state_dict.meta_tensor(full), requires_grad=False)
        self._hooks = [mod.register_forward_pre_hook(self._pre_hook) for mod in self._owned]

    def _pre_hook(self, mod, args):
        self.materialize(mod)

    def materialize(self, mod):
        """Decode every meta parameter of submodule ``mod`` now (one load)."""
        torch = _torch()
        todo = [p for p in self._owned[mod] if mod._parameters[p].is_meta]
        if todo:
            keys = [self.refs[(mod, p)].key for p in todo]
            got = self.sd.load(keys)
            nbytes = 0
            for p, k in zip(todo, keys):
                t = got[k]
                mod._parameters[p] = torch.nn.Parameter(t, requires_grad=False)
                nbytes += t.numel() * t.element_size()
            self.stats["materialized"] += len(todo)
            self._resident[mod] = self._resident.get(mod, 0) + nbytes
            self.resident_bytes += nbytes
        if mod in self._resident:
            self._resident.move_to_end(mod)
            self._enforce(keep=mod)

    def evict(self, mod):
        """Turn submodule ``mod``'s materialised parameters back into meta tensors."""
        torch = _torch()
        for p in self._owned[mod]:
            ref = self.refs[(mod, p)]
            if not mod._parameters[p].is_meta:
                mod._parameters[p] = torch.nn.Parameter(ref.source.meta_tensor(ref.key), requires_grad=False)
        self.resident_bytes -= self._resident.pop(mod, 0)
        self.stats["evicted"] += 1

    def _enforce(self, keep=None):
        if self.max_resident_bytes is None:
            return
        for mod in list(self._resident):
            if self.resident_bytes <= self.max_resident_bytes:
                break
            if mod is not keep:
                self.evict(mod)

    def evict_all(self):
        for mod in list(self._resident):
            self.evict(mod)

    def detach(self):
        """Remove the hooks (parameters keep their current state)."""
        for h in self._hooks:
            h.remove()
        self._hooks = []
