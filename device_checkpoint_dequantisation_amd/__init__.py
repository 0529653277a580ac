"""stmat: materialise safetensors checkpoint weights as bf16 (or fp16 / fp32) tensors on an MI355X.

Python binding of libstmat.so (include/stmat.h).  It only marshals arguments: the header index,
the descriptor plan, staging and the decode all run in the library; torch provides device
memory and streams.

    idx = SafeTensorIndex.open(path)           # metadata only, no tensor bytes read
    ckpt = DeviceCheckpoint(idx, path)         # VRAM pre-check, blob + outputs, staging
    ckpt.materialize()                         # one grouped kernel launch
    ckpt.tensors["model.layers.0.mlp.up_proj.weight"]   # bf16 torch tensor on the GPU

or simply ``load(path)`` -> {name: bf16 tensor}.
"""
from __future__ import annotations

import ctypes as C
import json
import os
from dataclasses import dataclass

from ._lib import (DTYPES, KINDS, MAT_SLICES, MAT_STREAM_STORES, TABLE_STREAM_STORES, OUT_DTYPES, PLAN_PACK, TABLE_MAGIC, Desc, OutputInfo,  # noqa: F401
                   PlanOpts, Slice, StError, StreamStats, StreamStep, TableHeader, TensorMeta, check, lib)

__all__ = ["SafeTensorIndex", "StreamPlan", "DeviceCheckpoint", "QuantizedWeight", "load", "materialize",
           "materialize_noalloc", "stage_file", "stream_file", "read_plans", "StError", "KINDS", "QUANTIZED_KINDS"]


@dataclass(frozen=True)
class TensorEntry:
    name: str
    dtype: str
    shape: tuple
    begin: int
    end: int


@dataclass(frozen=True)
class OutputEntry:
    name: str
    kind: str
    shape: tuple
    numel: int
    tensor: int
    scale: int
    scale2: int
    offset: int      # byte offset in the output arena


class SafeTensorIndex:
    """Metadata-only index of one safetensors file (the header alone is read)."""

    def __init__(self, handle: int):
        self._h = C.c_void_p(handle)

    @classmethod
    def open(cls, path: str, unit_log2_scale: int = 0, out_dtype: str = "bf16") -> "SafeTensorIndex":
        """Index of the file at ``path``; every output is planned as ``out_dtype`` (bf16, f16 or
        f32)."""
        h = C.c_void_p()
        opts = PlanOpts(unit_log2_scale, OUT_DTYPES.index(out_dtype))
        check(lib().st_index_open(os.fsencode(path), C.byref(opts), C.byref(h)), f"st_index_open({path})")
        return cls(h.value)

    @classmethod
    def from_bytes(cls, buf: bytes, file_size: int | None = None, unit_log2_scale: int = 0,
                   out_dtype: str = "bf16") -> "SafeTensorIndex":
        """Index from the leading bytes of a file (at least 8 + N) of ``file_size`` bytes
        (default: ``buf`` is the whole file)."""
        h = C.c_void_p()
        opts = PlanOpts(unit_log2_scale, OUT_DTYPES.index(out_dtype))
        size = len(buf) if file_size is None else file_size
        raw = C.create_string_buffer(bytes(buf), len(buf))
        check(lib().st_index_build(raw, len(buf), size, C.byref(opts), C.byref(h)), "st_index_build")
        return cls(h.value)

    def close(self):
        if self._h and self._h.value:
            lib().st_index_free(self._h)
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- sizes
    @property
    def out_dtype(self) -> str:
        """Output element type the index plans for: "bf16", "f16" or "f32"."""
        return OUT_DTYPES[lib().st_index_out_dtype(self._h)]

    @property
    def torch_dtype(self):
        torch = _torch()
        return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[self.out_dtype]

    @property
    def data_offset(self) -> int:
        return lib().st_index_data_offset(self._h)

    @property
    def data_size(self) -> int:
        return lib().st_index_data_size(self._h)

    @property
    def blob_bytes(self) -> int:
        return lib().st_index_blob_bytes(self._h)

    @property
    def arena_bytes(self) -> int:
        return lib().st_index_output_arena_bytes(self._h)

    @property
    def traffic_bytes(self) -> int:
        return lib().st_index_traffic_bytes(self._h)

    @property
    def device_bytes(self) -> int:
        return lib().st_index_device_bytes(self._h)

    @property
    def metadata(self) -> dict:
        return json.loads(lib().st_index_metadata_json(self._h).decode("utf-8"))

    # ---- entries
    def __len__(self) -> int:
        return lib().st_index_count(self._h)

    def tensor(self, i: int) -> TensorEntry:
        m = TensorMeta()
        check(lib().st_index_tensor(self._h, i, C.byref(m)), "st_index_tensor")
        return TensorEntry(m.name.decode("utf-8"), DTYPES[m.dtype], tuple(m.shape[: m.ndim]), m.begin, m.end)

    def tensors(self) -> list:
        return [self.tensor(i) for i in range(len(self))]

    def find(self, name: str) -> int:
        return lib().st_index_find(self._h, name.encode("utf-8"))

    @property
    def num_outputs(self) -> int:
        return lib().st_index_num_outputs(self._h)

    def output(self, k: int) -> OutputEntry:
        o = OutputInfo()
        check(lib().st_index_output(self._h, k, C.byref(o)), "st_index_output")
        return OutputEntry(o.name.decode("utf-8"), KINDS[o.kind], tuple(o.shape[: o.ndim]), o.numel, o.tensor,
                           o.scale, o.scale2, lib().st_index_output_offset(self._h, k))

    def outputs(self) -> list:
        return [self.output(k) for k in range(self.num_outputs)]

    def keys(self) -> list:
        """Output (weight) names, in output order; metadata only."""
        return [self.output(k).name for k in range(self.num_outputs)]

    # ---- slices
    @staticmethod
    def _slices(slices):
        arr = (Slice * max(1, len(slices)))()
        for j, sl in enumerate(slices):
            out, rows, cols = (sl + (None, None))[:3] if isinstance(sl, tuple) else (sl, None, None)
            r0, r1 = rows if rows is not None else (0, -1)
            c0, c1 = cols if cols is not None else (0, -1)
            arr[j] = Slice(int(out), 0, int(r0), int(-1 if r1 is None else r1), int(c0), int(-1 if c1 is None else c1))
        return arr

    def slice_shape(self, output: int, rows=None, cols=None) -> tuple:
        """(rows, cols) of a slice of the output's matrix view (st_index_slice_numel)."""
        arr = self._slices([(output, rows, cols)])
        r, c = C.c_uint64(), C.c_uint64()
        check(lib().st_index_slice_numel(self._h, arr, C.byref(r), C.byref(c)), "st_index_slice_numel")
        return r.value, c.value

    def has_column_slices(self, slices) -> bool:
        """True if any slice takes part of its output's columns (a strided source)."""
        for sl in slices:
            out, rows, cols = (sl + (None, None))[:3] if isinstance(sl, tuple) else (sl, None, None)
            if cols is not None and self.slice_shape(out, None, cols)[1] != self.slice_shape(out)[1]:
                return True
        return False

    def table_slices(self, slices):
        """Work table for slices, each ``(output, (row_begin, row_end), (col_begin, col_end))`` with
        None for a whole dimension and -1 for "to the end"; descriptor j writes outs[j]."""
        arr = self._slices(list(slices))
        k = len(slices)
        nb, units = C.c_size_t(), C.c_uint64()
        check(lib().st_index_table_slices(self._h, arr, k, None, 0, C.byref(nb), C.byref(units)), "st_index_table_slices")
        dst = C.create_string_buffer(nb.value)
        check(lib().st_index_table_slices(self._h, arr, k, dst, nb.value, C.byref(nb), C.byref(units)),
              "st_index_table_slices")
        return dst.raw[: nb.value], units.value

    # ---- work tables
    def table(self):
        """(bytes of the work table for every output, work units = the n st_materialize takes)."""
        nb, units = C.c_size_t(), C.c_uint64()
        p = lib().st_index_table(self._h, C.byref(nb), C.byref(units))
        return C.string_at(p, nb.value), units.value

    def table_subset(self, sel):
        """Self-contained work table for outputs ``sel`` (descriptor j writes outs[j])."""
        k = len(sel)
        arr = (C.c_uint32 * max(1, k))(*sel)
        nb, units = C.c_size_t(), C.c_uint64()
        check(lib().st_index_table_subset(self._h, arr, k, None, 0, C.byref(nb), C.byref(units)), "st_index_table_subset")
        dst = C.create_string_buffer(nb.value)
        check(lib().st_index_table_subset(self._h, arr, k, dst, nb.value, C.byref(nb), C.byref(units)),
              "st_index_table_subset")
        return dst.raw[: nb.value], units.value


@dataclass(frozen=True)
class StagingStep:
    bytes: int
    ranges: tuple       # ((begin, end), ...) of the data section
    outputs: tuple      # output indices this step completes
    table_offset: int   # byte offset of its work table in StreamPlan.tables
    units: int          # work units of that table (0: nothing to decode)


class StreamPlan:
    """Staging steps of at most ``chunk_bytes`` over a checkpoint's bytes, each with the outputs it
    completes and their work table.  ``select=None`` plans every output, laid out like the data
    section (st_stream_plan_build); a list of output indices plans those only
    (st_stream_plan_select), in a compact blob if ``pack``."""

    def __init__(self, index: SafeTensorIndex, chunk_bytes: int = 128 << 20, select=None, pack: bool = False):
        h = C.c_void_p()
        if select is None:
            if pack:
                raise ValueError("pack needs a selection of outputs")
            check(lib().st_stream_plan_build(index._h, chunk_bytes, C.byref(h)), "st_stream_plan_build")
        else:
            sel = list(select)
            arr = (C.c_uint32 * max(1, len(sel)))(*sel)
            check(lib().st_stream_plan_select(index._h, arr, len(sel), chunk_bytes, PLAN_PACK if pack else 0,
                                              C.byref(h)), "st_stream_plan_select")
        self._h = h.value
        self.index = index
        self.packed = bool(pack)
        L = lib()
        self.chunk_bytes = L.st_stream_plan_chunk_bytes(self._h)
        self.blob_bytes = L.st_stream_plan_blob_bytes(self._h)
        n = C.c_size_t()
        p = L.st_stream_plan_order(self._h, C.byref(n))
        self.order = [p[i] for i in range(n.value)]
        p = L.st_stream_plan_ranges(self._h, C.byref(n))
        self.ranges = [(p[i].begin, p[i].end) for i in range(n.value)]
        self.range_dsts = [p[i].dst for i in range(n.value)]
        self.range_steps = [p[i].step for i in range(n.value)]
        nb = C.c_size_t()
        tp = L.st_stream_plan_tables(self._h, C.byref(nb))
        self.tables = C.string_at(tp, nb.value) if nb.value else b""
        steps = []
        for k in range(L.st_stream_plan_num_steps(self._h)):
            st = StreamStep()
            check(L.st_stream_plan_step(self._h, k, C.byref(st)), "st_stream_plan_step")
            steps.append(StagingStep(st.bytes, tuple(self.ranges[st.first_range: st.first_range + st.n_ranges]),
                                     tuple(self.order[st.first_out: st.first_out + st.n_out]), st.table_offset,
                                     st.units))
        self.steps = steps

    def tensor_offset(self, begin: int) -> int:
        """Blob offset of the data-section byte ``begin`` (which the plan reads)."""
        for (b, e), d in zip(self.ranges, self.range_dsts):
            if b <= begin < e:
                return d + (begin - b)
        raise KeyError(begin)

    def close(self):
        if getattr(self, "_h", None):
            lib().st_stream_plan_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _torch():
    import torch
    return torch


def table_stream_stores(raw, offset: int = 0) -> bool:
    """Whether the work table at ``offset`` of the host bytes ``raw`` asks for non-temporal output
    stores (ST_TABLE_STREAM_STORES: its outputs are larger than the last-level cache)."""
    return bool(TableHeader.from_buffer_copy(bytes(raw[offset:offset + 64])).flags & TABLE_STREAM_STORES)


def check_table(raw: bytes, units: int, out_dtype: str) -> bool:
    """Raise ValueError unless the host copy ``raw`` of a work table records ``units`` work units
    and the output type ``out_dtype``: the kernel would leave every output unwritten otherwise.
    Returns the table's store policy (table_stream_stores)."""
    if len(raw) < 64:
        raise ValueError(f"work table of {len(raw)} bytes has no header")
    h = TableHeader.from_buffer_copy(bytes(raw[:64]))
    if h.magic != TABLE_MAGIC:
        raise ValueError(f"not a work table (magic 0x{h.magic:08x})")
    if h.units != units:
        raise ValueError(f"work table holds {h.units} units, the launch was given {units}")
    if h.out_dtype >= len(OUT_DTYPES) or OUT_DTYPES[h.out_dtype] != out_dtype:
        raise ValueError(f"work table was planned for output type code {h.out_dtype}, the launch asks for {out_dtype}")
    return bool(h.flags & TABLE_STREAM_STORES)


def stage_file(path: str, index: SafeTensorIndex, blob, pinned, side_stream) -> float:
    """Copy the file's data section into ``blob`` (device uint8 tensor of index.blob_bytes) through
    the pinned uint8 host tensor ``pinned`` on ``side_stream``; returns seconds spent reading."""
    secs = C.c_double()
    check(lib().st_stage_file(os.fsencode(path), index._h, C.c_void_p(blob.data_ptr()), C.c_void_p(pinned.data_ptr()),
                              pinned.numel(), C.c_void_p(side_stream.cuda_stream), None, C.byref(secs)),
          "st_stage_file")
    return secs.value


def materialize(blob, table, units: int, outs, stream=None, slices: bool = False, out_dtype: str = "bf16",
                stream_stores: bool = False):
    """Enqueue the grouped kernel (st_materialize_as): ``blob`` (the staged data section),
    ``table`` (a work table) and ``outs`` (device pointers, int64) are device tensors; ``units`` is
    the table's work-unit count; ``out_dtype`` the output type the table was planned for;
    ``slices`` selects the kernel with the strided path for column slices; ``stream_stores`` the
    non-temporal stores its header asks for (table_stream_stores)."""
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(blob.device)
    flags = (MAT_SLICES if slices else 0) | (MAT_STREAM_STORES if stream_stores else 0)
    check(lib().st_materialize_as(C.c_void_p(blob.data_ptr()), C.c_void_p(table.data_ptr()), units,
                                  C.c_void_p(outs.data_ptr()), OUT_DTYPES.index(out_dtype), flags,
                                  C.c_void_p(s.cuda_stream)), "st_materialize_as")


def materialize_noalloc(blob, table_raw: bytes, units: int, out_ptrs, stream=None, slices: bool = False,
                        out_dtype: str = "bf16"):
    """The allocation-free launch (st_materialize_noalloc): the work table ``table_raw`` (host bytes)
    and the device output pointers ``out_ptrs`` (ints) are copied into the library's own device
    array on ``stream`` and decoded from there.  Returns the host buffers handed to the copies; keep
    them until ``stream`` has passed the launch."""
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(blob.device)
    table = C.create_string_buffer(bytes(table_raw), len(table_raw))
    ptrs = (C.c_void_p * max(1, len(out_ptrs)))(*[int(p) for p in out_ptrs])
    check(lib().st_materialize_noalloc(C.c_void_p(blob.data_ptr()), table, len(table_raw), units, ptrs, len(out_ptrs),
                                       OUT_DTYPES.index(out_dtype), MAT_SLICES if slices else 0,
                                       C.c_void_p(s.cuda_stream)), "st_materialize_noalloc")
    return table, ptrs


def read_plans(path: str, index: SafeTensorIndex, plans, hosts) -> float:
    """Read each plan's ranges into the matching host uint8 tensor (st_read_plans); returns seconds."""
    n = len(plans)
    ph = (C.c_void_p * max(1, n))(*[p._h for p in plans])
    hb = (C.c_void_p * max(1, n))(*[h.data_ptr() for h in hosts])
    nb = (C.c_size_t * max(1, n))(*[h.numel() for h in hosts])
    secs = C.c_double()
    check(lib().st_read_plans(os.fsencode(path), index._h, ph, hb, nb, n, C.byref(secs)), "st_read_plans")
    return secs.value


def stream_file(path: str, index: SafeTensorIndex, plan: StreamPlan, blob, tables, outs_plan, pinned, side_stream,
                stream) -> dict:
    """Read, copy and decode ``path`` step by step (st_stream_file).  ``tables``: device copy of
    plan.tables; ``outs_plan``: device int64 pointers in plan order; ``pinned``: pinned uint8 host
    tensor of at least 4 * plan.chunk_bytes.  Returns once everything is enqueued."""
    st = StreamStats()
    check(lib().st_stream_file(os.fsencode(path), index._h, plan._h, C.c_void_p(blob.data_ptr()),
                               C.c_void_p(tables.data_ptr() if tables is not None else 0),
                               C.c_void_p(outs_plan.data_ptr()), C.c_void_p(pinned.data_ptr()), pinned.numel(),
                               C.c_void_p(side_stream.cuda_stream), C.c_void_p(stream.cuda_stream), None,
                               C.byref(st)), "st_stream_file")
    return {"seconds_read": st.seconds_read, "seconds_wait": st.seconds_wait, "bytes_read": st.bytes_read,
            "seconds_first_launch": st.seconds_first_launch,
            "steps": st.steps, "launches": st.launches}


@dataclass
class QuantizedWeight:
    """A quantised weight as stored, for consumers that compute on the quantised form (FP8 matrix
    cores): no decode, the checkpoint's own bytes on the device.
      FP8_TENSOR    data float8_e4m3fn [M, N...], scale fp32 []
      FP8_BLOCK128  data float8_e4m3fn [M, N],    scale fp32 [ceil(M/128), ceil(N/128)] (multiplied)
      NVFP4         data uint8 [M, K/2] (element 2k in the low nibble of byte k),
                    scale float8_e4m3fn [M, K/16], scale2 fp32 []
      MXFP8         data float8_e4m3fn [M, K],    scale float8_e8m0fnu [M, K/32]
      MXFP4         data uint8 [M, K/2] (as NVFP4), scale float8_e8m0fnu [M, K/32]"""
    name: str
    kind: str
    shape: tuple        # logical shape of the weight
    data: object
    scale: object
    scale2: object = None


QUANTIZED_KINDS = ("FP8_TENSOR", "FP8_BLOCK128", "NVFP4", "MXFP8", "MXFP4")


def _quantized(index: SafeTensorIndex, blob, k: int, at, copy: bool) -> QuantizedWeight:
    """QuantizedWeight of output k from a device blob in which tensor t's bytes start at at(t)."""
    torch = _torch()
    o = index.output(k)
    if o.kind not in QUANTIZED_KINDS:
        raise ValueError(f"{o.name}: {o.kind} is not a quantised weight")
    ents = index.tensors()

    def raw(i):
        e = ents[i]
        return blob[at(i): at(i) + (e.end - e.begin)]

    def f32(i, shape):  # fp32 scales may sit at any byte offset: always a copy
        return raw(i).clone().view(torch.float32).view(shape)

    w = raw(o.tensor)
    if o.kind in ("MXFP8", "MXFP4"):
        m, kk = o.shape
        data = w.view(m, kk // 2) if o.kind == "MXFP4" else w.view(torch.float8_e4m3fn).view(m, kk)
        sc = raw(o.scale).view(torch.float8_e8m0fnu).view(m, kk // 32)
        if copy:
            data, sc = data.clone(), sc.clone()
        return QuantizedWeight(o.name, o.kind, tuple(o.shape), data, sc)
    if o.kind == "NVFP4":
        m, kk = o.shape
        data = w.view(m, kk // 2)
        sc = raw(o.scale).view(torch.float8_e4m3fn).view(m, kk // 16)
        if copy:
            data, sc = data.clone(), sc.clone()
        return QuantizedWeight(o.name, o.kind, tuple(o.shape), data, sc, f32(o.scale2, ()))
    data = w.view(torch.float8_e4m3fn).view(o.shape)
    if copy:
        data = data.clone()
    if o.kind == "FP8_TENSOR":
        return QuantizedWeight(o.name, o.kind, tuple(o.shape), data, f32(o.scale, ()))
    m, n = o.shape
    return QuantizedWeight(o.name, o.kind, tuple(o.shape), data, f32(o.scale, (-(-m // 128), -(-n // 128))))


class DeviceCheckpoint:
    """A checkpoint staged on one GPU: the blob, the descriptor table and an output arena of the
    index's output type, in which every output starts on a 256-byte boundary."""

    def __init__(self, index: SafeTensorIndex, path: str | None = None, device="cuda", pinned_mb: int = 256,
                 check_vram: bool = True):
        torch = _torch()
        self.index = index
        self.device = torch.device(device)
        if self.device.type != "cuda":
            raise ValueError("DeviceCheckpoint needs a GPU device")
        if check_vram:
            free, total = torch.cuda.mem_get_info(self.device)
            need = index.device_bytes
            if need > free:
                raise MemoryError(f"checkpoint needs {need} bytes of device memory; {free} of {total} are free")
        self.blob = torch.empty(index.blob_bytes, dtype=torch.uint8, device=self.device)
        table, units = index.table()
        self.stream_stores = check_table(table, units, index.out_dtype)
        self.units = units
        self.table = torch.frombuffer(bytearray(table), dtype=torch.uint8).to(self.device)
        dt = index.torch_dtype
        esize = 4 if index.out_dtype == "f32" else 2
        self.arena = torch.empty(max(1, index.arena_bytes // esize), dtype=dt, device=self.device)
        outs = index.outputs()
        base = self.arena.data_ptr()
        self.outs = torch.tensor([base + o.offset for o in outs] or [0], dtype=torch.int64).to(self.device)
        self.tensors = {}
        for o in outs:
            start = o.offset // esize
            self.tensors[o.name] = self.arena[start: start + o.numel].view(o.shape)
        self.stage_seconds_read = None
        if path is not None:
            self.stage(path, pinned_mb)

    def stage(self, path: str, pinned_mb: int = 256):
        """Copy the file's data section into the blob (returns once the copy is complete).  Work
        already enqueued on the current stream (an earlier decode reading the blob) runs first."""
        torch = _torch()
        self.synchronize()
        pinned = torch.empty(max(2, pinned_mb) << 20, dtype=torch.uint8, pin_memory=True)
        side = torch.cuda.Stream(self.device)
        side.wait_stream(torch.cuda.current_stream(self.device))
        self.stage_seconds_read = stage_file(path, self.index, self.blob, pinned, side)
        side.synchronize()
        del pinned

    def stream(self, path: str, chunk_mb: int = 128, stream=None, plan: StreamPlan | None = None) -> dict:
        """Stage and decode ``path`` with the overlapped pipeline: each staging step's outputs are
        decoded on ``stream`` (default: the current stream) while later steps are read and copied.
        Returns the pipeline's statistics once everything is enqueued; the outputs are ready when
        ``stream`` reaches this point (the pinned ring is held until then, see ``synchronize``)."""
        torch = _torch()
        self.synchronize()  # an earlier streamed load's copies may still read the pinned ring
        plan = plan or StreamPlan(self.index, chunk_mb << 20)
        compute = stream if stream is not None else torch.cuda.current_stream(self.device)
        need = 4 * plan.chunk_bytes
        if getattr(self, "_pinned", None) is None or self._pinned.numel() < need:
            self._pinned = torch.empty(need, dtype=torch.uint8, pin_memory=True)
        tables = (torch.frombuffer(bytearray(plan.tables), dtype=torch.uint8).to(self.device, non_blocking=False)
                  if plan.tables else None)
        order = torch.tensor(plan.order or [0], dtype=torch.int64, device=self.device)
        outs_plan = self.outs[order] if plan.order else self.outs
        side = torch.cuda.Stream(self.device)
        compute.wait_stream(torch.cuda.current_stream(self.device))  # tables and outs_plan are ready
        side.wait_stream(compute)  # earlier decodes of this blob are done before it is overwritten
        for t in (tables, outs_plan):
            if t is not None:
                t.record_stream(compute)
        stats = stream_file(path, self.index, plan, self.blob, tables, outs_plan, self._pinned, side, compute)
        self._inflight = (plan, tables, outs_plan, side, compute)
        return stats

    def synchronize(self):
        """Wait for a streamed load and release its transient buffers (the pinned ring is kept)."""
        inflight = getattr(self, "_inflight", None)
        if inflight:
            inflight[4].synchronize()
            inflight[3].synchronize()
            self._inflight = None

    def load_bytes(self, data_section: bytes):
        """Stage from bytes already in host memory (tests): the data section only."""
        torch = _torch()
        assert len(data_section) == self.index.data_size
        if data_section:
            host = torch.frombuffer(bytearray(data_section), dtype=torch.uint8)
            self.blob[: len(data_section)].copy_(host)

    def quantized(self, names=None, copy: bool = True) -> dict:
        """The quantised weights (FP8_TENSOR, FP8_BLOCK128, NVFP4, MXFP8, MXFP4 outputs) as stored, from the
        staged blob: ``copy=True`` gives fresh, 256-byte aligned tensors; ``copy=False`` gives
        views into the blob for the weight bytes (the fp32 scales are always copied)."""
        outs = self.index.outputs()
        pos = {o.name: k for k, o in enumerate(outs)}
        want = [o.name for o in outs if o.kind in QUANTIZED_KINDS] if names is None else names
        ents = self.index.tensors()
        return {n: _quantized(self.index, self.blob, pos[n], lambda i: ents[i].begin, copy) for n in want}

    def materialize_slices(self, slices, stream=None, strided_kernel: bool | None = None) -> list:
        """Tensors [rows, cols] of the output type for slices of outputs (see SafeTensorIndex.table_slices),
        decoded in one launch from the staged blob.  ``strided_kernel`` (default: whether any
        slice cuts columns) picks st_materialize_slices; with False, the whole-output kernel's
        exact path decodes column slices element by element."""
        torch = _torch()
        slices = list(slices)
        shapes = [self.index.slice_shape(*((sl + (None, None))[:3] if isinstance(sl, tuple) else (sl,))) for sl in slices]
        outs = [torch.empty(shp, dtype=self.index.torch_dtype, device=self.device) for shp in shapes]
        raw, units = self.index.table_slices(slices)
        stream_stores = check_table(raw, units, self.index.out_dtype)
        if strided_kernel is None:
            strided_kernel = self.index.has_column_slices(slices)
        table = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(self.device)
        ptrs = torch.tensor([o.data_ptr() for o in outs] or [0], dtype=torch.int64).to(self.device)
        if units:
            s = self._launch_stream(stream)
            for t in [table, ptrs] + outs:  # allocated on the current stream, used on s
                t.record_stream(s)
            materialize(self.blob, table, units, ptrs, s, slices=strided_kernel, out_dtype=self.index.out_dtype,
                        stream_stores=stream_stores)
        return outs

    def _launch_stream(self, stream):
        """The stream a decode runs on: ``stream``, ordered after the work already enqueued on the
        current stream (uploads, staging), or the current stream itself."""
        torch = _torch()
        cur = torch.cuda.current_stream(self.device)
        if stream is None or stream == cur:
            return cur
        stream.wait_stream(cur)
        return stream

    def materialize(self, stream=None):
        if self.units:
            materialize(self.blob, self.table, self.units, self.outs, self._launch_stream(stream),
                        out_dtype=self.index.out_dtype, stream_stores=self.stream_stores)
        return self.tensors


def load(path: str, device="cuda", unit_log2_scale: int = 0, streamed: bool = True, chunk_mb: int = 128,
         out_dtype: str = "bf16") -> dict:
    """Every output of the checkpoint at ``path`` as a tensor on ``device`` (bf16 by default, or
    ``out_dtype`` f16 / f32).  By default the overlapped pipeline decodes each staging step while
    later steps are read and copied; ``streamed=False`` stages the whole data section first and
    then decodes it in one launch."""
    idx = SafeTensorIndex.open(path, unit_log2_scale, out_dtype)
    ck = DeviceCheckpoint(idx, None, device)
    if streamed:
        ck.stream(path, chunk_mb=chunk_mb)
        ck.synchronize()
        ck._pinned = None
        return ck.tensors
    ck.stage(path)
    out = ck.materialize()
    _torch().cuda.current_stream(ck.device).synchronize()
    return out


from .lazy import (DiskRef, FilterViewStateDict, LazyModuleLoader, OutputMeta, PrefixViewStateDict,  # noqa: E402,F401
                   RamCache, RenameViewStateDict, StreamStateDict)

from .shards import (ShardedStateDict, ShardError, index_shards, load_checkpoint, shard_files)  # noqa: E402,F401

__all__ += ["StreamStateDict", "PrefixViewStateDict", "FilterViewStateDict", "RenameViewStateDict", "RamCache",
            "LazyModuleLoader", "DiskRef", "OutputMeta", "ShardedStateDict", "ShardError", "index_shards",
            "load_checkpoint", "shard_files"]
