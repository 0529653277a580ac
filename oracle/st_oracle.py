"""Plain, slow CPU definition of what materialising a safetensors checkpoint as bf16 computes.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product never calls this module.

Sources.  The pages ("Disk tier safetensors streaming design audit", sections "FastSageTensors
capability audit" and "Strategy summary / Streaming safetensors mapping") describe a
metadata-only index built from the safetensors header: per tensor a dtype, a shape and
``data_offsets``, read without loading tensors.  The pages' serving document ("Resident Modal
LLM Architecture", section "Current Backend Boundary") names the quantised checkpoint families
(Qwen block-FP8, NVIDIA ModelOpt NVFP4) and the design audit (section "Mandatory research
audit") names ComfyUI's scaled-FP8 conversion.  The bit-level definitions used below are the
public ones those names refer to: the safetensors file layout, OCP 8-bit E4M3 ("fn": no
infinities, NaN at S.1111.111), OCP-MX E2M1, and IEEE-754 binary32 arithmetic with
round-to-nearest-even followed by round-to-nearest-even to bfloat16.

Readings where the pages are silent (each listed in the design notes):
  * one fp32 multiply per scale, each rounded RNE, then RNE to bf16 (double rounding); the fp16
    and fp32 output variants round the same fp32 result RNE to fp16, or keep it;
  * NVFP4 multiplies left to right: (e2m1 * block_scale) * global_scale;
  * ``weight_scale_inv`` is multiplied, despite its name;
  * every NaN result becomes the output type's canonical quiet NaN (bf16 0x7FC0, fp16 0x7E00,
    fp32 0x7FC00000); bf16 passthrough to a bf16 output copies bits unchanged;
  * no flush of subnormals anywhere;
  * packed e2m1: element 2k in bits 0-3, element 2k+1 in bits 4-7 of byte k;
  * tensor names: ``X.weight`` + ``X.scale_weight`` (fp32 scalar) = per-tensor scaled FP8;
    ``X.weight`` + ``X.weight_scale_inv`` (fp32 [ceil(M/128), ceil(N/128)]) = block FP8;
    ``X.weight`` (U8 [M, K/2] or F4 [M, K]) + ``X.weight_scale`` (e4m3 [M, K/16]) +
    ``X.weight_scale_2`` (fp32 scalar) = NVFP4;
    ``X.weight`` (F8_E4M3 [M, K]; or U8 [M, K/2] / F4 [M, K]) + ``X.weight_scale`` (F8_E8M0
    [M, K/32]) = MXFP8 / MXFP4, the OCP Microscaling formats: blocks of 32 consecutive elements
    of a row share one E8M0 scale 2^(e - 127) (e = 255 is NaN), applied by one fp32 multiply;
  * any byte offset is legal for any dtype; header length capped at 100,000,000 bytes;
  * header integers must fit in a signed 64-bit value; at most 8 dimensions.

Everything is NumPy elementwise work on explicit byte gathers; there is no blocking, fusion or
reordering.  Multi-byte values are assembled little-endian, byte by byte, from any offset.
"""
from __future__ import annotations

import json
import math
from dataclasses import dataclass

import numpy as np

HEADER_CAP = 100_000_000
INT64_MAX = (1 << 63) - 1
MAX_NDIM = 8

# Bits per element of every dtype string the safetensors format defines.
DTYPE_BITS = {
    "BOOL": 8, "U8": 8, "I8": 8, "F8_E4M3": 8, "F8_E5M2": 8, "F8_E8M0": 8,
    "I16": 16, "U16": 16, "F16": 16, "BF16": 16,
    "I32": 32, "U32": 32, "F32": 32,
    "I64": 64, "U64": 64, "F64": 64,
    "F4": 4, "F6_E2M3": 6, "F6_E3M2": 6,
}

SCALE_SUFFIXES = (".scale_weight", ".weight_scale_inv", ".weight_scale_2", ".weight_scale")


class OracleError(ValueError):
    pass


@dataclass(frozen=True)
class Entry:
    name: str
    dtype: str
    shape: tuple
    begin: int   # relative to the data section
    end: int

    @property
    def numel(self) -> int:
        return math.prod(self.shape)


@dataclass
class Header:
    header_len: int          # N
    data_offset: int         # 8 + N: file offset of the data section
    data_size: int           # bytes after the header
    entries: dict            # name -> Entry, in header order
    metadata: dict | None


@dataclass(frozen=True)
class Output:
    name: str
    kind: str                # PASS_BF16 CAST_F16 CAST_F32 FP8_TENSOR FP8_BLOCK128 NVFP4
    shape: tuple             # logical bf16 shape
    src: Entry
    scale: Entry | None = None
    scale2: Entry | None = None

    @property
    def numel(self) -> int:
        return math.prod(self.shape)


# ----------------------------------------------------------------------------- parsing

def _no_duplicates(pairs):
    d = {}
    for k, v in pairs:
        if k in d:
            raise OracleError(f"duplicate key {k!r} in header")
        d[k] = v
    return d


def _reject_constant(s):
    raise OracleError(f"non-JSON constant {s} in header")


def _is_int(x) -> bool:
    return isinstance(x, int) and not isinstance(x, bool)


def _check_name(s: str):
    try:
        s.encode("utf-8")
    except UnicodeEncodeError:
        raise OracleError("string with an unpaired surrogate in header") from None
    if "\x00" in s:
        raise OracleError("string with a NUL character in header")


def parse_header(buf) -> Header:
    """Parse the 8-byte little-endian length N and the N-byte JSON header of a safetensors
    file.  ``buf`` must hold at least the first 8 + N bytes; ``file_size`` checks use len(buf)
    when the whole file is given (see validate_layout)."""
    mv = memoryview(buf)
    if len(mv) < 8:
        raise OracleError("file shorter than the 8-byte header length")
    n = int.from_bytes(bytes(mv[:8]), "little")
    if n > HEADER_CAP:
        raise OracleError(f"header length {n} exceeds the cap {HEADER_CAP}")
    if 8 + n > len(mv):
        raise OracleError(f"header length {n} runs past the end of the file ({len(mv)} bytes)")
    try:
        text = bytes(mv[8:8 + n]).decode("utf-8")
    except UnicodeDecodeError as e:
        raise OracleError(f"header is not UTF-8: {e}") from None
    try:
        obj = json.loads(text, object_pairs_hook=_no_duplicates, parse_constant=_reject_constant)
    except json.JSONDecodeError as e:
        raise OracleError(f"header is not JSON: {e}") from None
    if not isinstance(obj, dict):
        raise OracleError("header is not a JSON object")
    metadata = None
    entries = {}
    for name, val in obj.items():
        _check_name(name)
        if name == "__metadata__":
            if not isinstance(val, dict) or not all(isinstance(v, str) for v in val.values()):
                raise OracleError("__metadata__ must map strings to strings")
            for k, v in val.items():
                _check_name(k)
                _check_name(v)
            metadata = dict(val)
            continue
        if not isinstance(val, dict) or set(val) != {"dtype", "shape", "data_offsets"}:
            raise OracleError(f"{name}: entry must have exactly dtype, shape, data_offsets")
        dtype, shape, offs = val["dtype"], val["shape"], val["data_offsets"]
        if not isinstance(dtype, str) or dtype not in DTYPE_BITS:
            raise OracleError(f"{name}: unknown dtype {dtype!r}")
        if not isinstance(shape, list) or not all(_is_int(s) and 0 <= s <= INT64_MAX for s in shape):
            raise OracleError(f"{name}: shape must be a list of non-negative integers")
        if len(shape) > MAX_NDIM:
            raise OracleError(f"{name}: more than {MAX_NDIM} dimensions")
        if (not isinstance(offs, list) or len(offs) != 2
                or not all(_is_int(o) and 0 <= o <= INT64_MAX for o in offs)):
            raise OracleError(f"{name}: data_offsets must be two non-negative integers")
        b, e = offs
        if b > e:
            raise OracleError(f"{name}: data_offsets begin {b} > end {e}")
        bits = math.prod(shape) * DTYPE_BITS[dtype]
        if bits % 8 or bits // 8 != e - b:
            raise OracleError(f"{name}: {dtype}{shape} needs {bits / 8:g} bytes, offsets span {e - b}")
        entries[name] = Entry(name, dtype, tuple(shape), b, e)
    return Header(n, 8 + n, len(mv) - 8 - n, entries, metadata)


def validate_layout(h: Header, file_size: int | None = None):
    """Offsets must tile the data section exactly: sorted by (begin, end) the first begins at 0,
    each begins where the previous ended, and the last ends at the end of the file."""
    size = h.data_size if file_size is None else file_size - h.data_offset
    pos = 0
    for e in sorted(h.entries.values(), key=lambda t: (t.begin, t.end)):
        if e.begin != pos:
            what = "overlaps" if e.begin < pos else "leaves a gap before"
            raise OracleError(f"{e.name}: data_offsets [{e.begin}, {e.end}] {what} byte {pos}")
        pos = e.end
    if pos != size:
        raise OracleError(f"tensors cover {pos} bytes but the data section has {size}")


# ----------------------------------------------------------------------------- classification

def _is_scalar(e: Entry) -> bool:
    return e.shape == () or e.shape == (1,)


def classify(h: Header) -> list:
    """Pair quantised weights with their scale tensors and give every other tensor a kind.
    Returns the outputs ordered by the weight's data offset, then name."""
    ents = h.entries
    used = set()
    outs = []
    for name, e in ents.items():
        if name.endswith(SCALE_SUFFIXES):
            continue
        if e.dtype == "BF16":
            outs.append(Output(name, "PASS_BF16", e.shape, e))
        elif e.dtype == "F16":
            outs.append(Output(name, "CAST_F16", e.shape, e))
        elif e.dtype == "F32":
            outs.append(Output(name, "CAST_F32", e.shape, e))
        elif e.dtype == "F8_E4M3":
            if not name.endswith(".weight"):
                raise OracleError(f"{name}: float8 tensor without a scale (not named X.weight)")
            x = name[: -len(".weight")]
            st, sb = ents.get(x + ".scale_weight"), ents.get(x + ".weight_scale_inv")
            sm = ents.get(x + ".weight_scale")
            if sum(v is not None for v in (st, sb, sm)) > 1:
                raise OracleError(f"{name}: more than one of scale_weight, weight_scale_inv, weight_scale present")
            if sm is not None:
                outs.append(_mx_output(name, e, sm, ents.get(x + ".weight_scale_2"), "MXFP8", e.shape))
                used.add(sm.name)
            elif st is not None:
                if st.dtype != "F32" or not _is_scalar(st):
                    raise OracleError(f"{st.name}: scale_weight must be an fp32 scalar")
                outs.append(Output(name, "FP8_TENSOR", e.shape, e, st))
                used.add(st.name)
            elif sb is not None:
                if len(e.shape) != 2:
                    raise OracleError(f"{name}: block-scaled float8 weight must be 2-D")
                m, n = e.shape
                grid = (-(-m // 128), -(-n // 128))
                if sb.dtype != "F32" or sb.shape != grid:
                    raise OracleError(f"{sb.name}: must be F32 {list(grid)}, got {sb.dtype}{list(sb.shape)}")
                outs.append(Output(name, "FP8_BLOCK128", e.shape, e, sb))
                used.add(sb.name)
            else:
                raise OracleError(f"{name}: float8 weight has no scale_weight, weight_scale_inv or weight_scale")
        elif e.dtype in ("U8", "F4"):
            if not name.endswith(".weight"):
                raise OracleError(f"{name}: {e.dtype} tensor is not an NVFP4 weight")
            x = name[: -len(".weight")]
            if len(e.shape) != 2:
                raise OracleError(f"{name}: NVFP4 weight must be 2-D")
            m = e.shape[0]
            k = e.shape[1] * 2 if e.dtype == "U8" else e.shape[1]
            bs, g = ents.get(x + ".weight_scale"), ents.get(x + ".weight_scale_2")
            if bs is not None and bs.dtype == "F8_E8M0":
                outs.append(_mx_output(name, e, bs, g, "MXFP4", (m, k)))
                used.add(bs.name)
                continue
            if k % 16:
                raise OracleError(f"{name}: NVFP4 K={k} is not a multiple of 16")
            if bs is None or g is None:
                raise OracleError(f"{name}: NVFP4 weight needs weight_scale and weight_scale_2")
            if bs.dtype != "F8_E4M3" or bs.shape != (m, k // 16):
                raise OracleError(f"{bs.name}: must be F8_E4M3 [{m}, {k // 16}]")
            if g.dtype != "F32" or not _is_scalar(g):
                raise OracleError(f"{g.name}: weight_scale_2 must be an fp32 scalar")
            outs.append(Output(name, "NVFP4", (m, k), e, bs, g))
            used.update((bs.name, g.name))
        else:
            raise OracleError(f"{name}: dtype {e.dtype} cannot be materialised as bf16")
    for name in ents:
        if name.endswith(SCALE_SUFFIXES) and name not in used:
            raise OracleError(f"{name}: scale tensor with no matching weight")
    outs.sort(key=lambda o: (o.src.begin, o.name))
    return outs


def _mx_output(name: str, e: Entry, sc: Entry, g, kind: str, shape: tuple) -> Output:
    """An MX weight of logical shape [M, K] with its E8M0 scale [M, K/32]."""
    if len(shape) != 2:
        raise OracleError(f"{name}: {kind} weight must be 2-D")
    m, k = shape
    if k % 32:
        raise OracleError(f"{name}: {kind} K={k} is not a multiple of 32")
    if g is not None:
        raise OracleError(f"{g.name}: an E8M0-scaled weight takes no weight_scale_2")
    if sc.dtype != "F8_E8M0" or sc.shape != (m, k // 32):
        raise OracleError(f"{sc.name}: must be F8_E8M0 [{m}, {k // 32}], got {sc.dtype}{list(sc.shape)}")
    return Output(name, kind, (m, k), e, sc)


def plan(buf):
    h = parse_header(buf)
    validate_layout(h, len(buf))
    return h, classify(h)


# ----------------------------------------------------------------------------- code tables

def e4m3_value(c: int) -> float:
    """OCP E4M3 'fn' code -> exact value (Python float): sign bit, 4 exponent bits (bias 7),
    3 mantissa bits; exponent field 0 is subnormal; S.1111.111 is NaN; no infinities."""
    s, E, m = c >> 7, (c >> 3) & 15, c & 7
    if E == 15 and m == 7:
        return math.nan
    v = (m / 8) * 2.0 ** -6 if E == 0 else (1 + m / 8) * 2.0 ** (E - 7)
    return -v if s else v


def e8m0_value(c: int) -> float:
    """OCP-MX E8M0 scale code -> exact value: 8 exponent bits, bias 127, no sign or mantissa;
    0xFF is NaN.  Code 0 is 2^-127, a binary32 subnormal."""
    return math.nan if c == 255 else 2.0 ** (c - 127)


def e2m1_value(c: int) -> float:
    """OCP-MX E2M1 code -> exact value: sign bit, 2 exponent bits (bias 1), 1 mantissa bit;
    exponent field 0 is subnormal (0 or 0.5); no NaN or infinities."""
    s, E, m = c >> 3, (c >> 1) & 3, c & 1
    v = m * 0.5 if E == 0 else (1 + m / 2) * 2.0 ** (E - 1)
    return -v if s else v


E4M3 = np.array([e4m3_value(c) for c in range(256)], dtype=np.float32)
E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float32)
E8M0 = np.array([e8m0_value(c) for c in range(256)], dtype=np.float32)


def bf16_rne(y: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16 bits, round to nearest, ties to even; any NaN -> 0x7FC0."""
    y = np.asarray(y, dtype=np.float32)
    u = y.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return np.where(np.isnan(y), np.uint64(0x7FC0), r).astype(np.uint16)


def f16_rne(y: np.ndarray) -> np.ndarray:
    """binary32 -> binary16 bits, round to nearest, ties to even (NumPy's IEEE conversion: overflow
    to infinity, subnormals kept); any NaN -> 0x7E00."""
    y = np.asarray(y, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        h = y.astype(np.float16).view(np.uint16)
    return np.where(np.isnan(y), np.uint16(0x7E00), h).astype(np.uint16)


def f32_bits(y: np.ndarray) -> np.ndarray:
    """binary32 bits of y; any NaN -> 0x7FC00000."""
    y = np.asarray(y, dtype=np.float32)
    return np.where(np.isnan(y), np.uint32(0x7FC00000), y.view(np.uint32)).astype(np.uint32)


OUT_ROUND = {"bf16": bf16_rne, "f16": f16_rne, "f32": f32_bits}


# ----------------------------------------------------------------------------- decoding

def _gather_le(data: np.ndarray, base: int, itemsize: int, idx: np.ndarray) -> np.ndarray:
    """Little-endian unsigned value of ``itemsize`` bytes starting at base + idx*itemsize."""
    off = base + idx * itemsize
    v = np.zeros(idx.shape, dtype=np.uint64)
    for k in range(itemsize):
        v |= data[off + k].astype(np.uint64) << np.uint64(8 * k)
    return v


def _f32_at(data, base, idx):
    return _gather_le(data, base, 4, idx).astype(np.uint32).view(np.float32)


def value(o: Output, data, idx) -> np.ndarray:
    """The exact binary32 result of output ``o`` at flat element indices ``idx``, before the
    output rounding: each scale applied by one RNE fp32 multiply, in the pages' order."""
    b = o.src.begin
    if o.kind == "PASS_BF16":
        return (_gather_le(data, b, 2, idx).astype(np.uint32) << np.uint32(16)).view(np.float32)
    if o.kind == "CAST_F16":
        return _gather_le(data, b, 2, idx).astype(np.uint16).view(np.float16).astype(np.float32)
    if o.kind == "CAST_F32":
        return _f32_at(data, b, idx)
    if o.kind == "FP8_TENSOR":
        s = _f32_at(data, o.scale.begin, np.zeros(1, np.int64))[0]
        return E4M3[_gather_le(data, b, 1, idx).astype(np.int64)] * s
    if o.kind == "FP8_BLOCK128":
        m, n = o.shape
        gn = -(-n // 128)
        i, j = idx // n, idx % n
        S = _f32_at(data, o.scale.begin, (i // 128) * gn + j // 128)
        return E4M3[_gather_le(data, b, 1, idx).astype(np.int64)] * S
    if o.kind in ("MXFP8", "MXFP4"):
        m, k = o.shape
        i, j = idx // k, idx % k
        S = E8M0[_gather_le(data, o.scale.begin, 1, i * (k // 32) + j // 32).astype(np.int64)]
        if o.kind == "MXFP8":
            return E4M3[_gather_le(data, b, 1, idx).astype(np.int64)] * S
        byte = _gather_le(data, b, 1, idx // 2)
        nib = (byte >> (np.uint64(4) * (idx & 1).astype(np.uint64))) & np.uint64(15)
        return E2M1[nib.astype(np.int64)] * S
    if o.kind == "NVFP4":
        m, k = o.shape
        i, j = idx // k, idx % k
        byte = _gather_le(data, b, 1, idx // 2)
        nib = (byte >> (np.uint64(4) * (idx & 1).astype(np.uint64))) & np.uint64(15)
        bs = E4M3[_gather_le(data, o.scale.begin, 1, i * (k // 16) + j // 16).astype(np.int64)]
        g = _f32_at(data, o.scale2.begin, np.zeros(1, np.int64))[0]
        t = E2M1[nib.astype(np.int64)] * bs
        return t * g
    raise OracleError(f"unknown kind {o.kind}")


def decode(o: Output, data, idx=None, out_dtype: str = "bf16") -> np.ndarray:
    """Output bits of ``o`` at flat element indices ``idx`` (all elements if None): uint16 for bf16
    and f16 outputs, uint32 for f32.  ``data`` is the data section (bytes after the header) as a
    uint8 array."""
    data = np.asarray(data, dtype=np.uint8)
    flat = idx is None
    if flat:
        idx = np.arange(o.numel, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    if o.kind == "PASS_BF16" and out_dtype == "bf16":
        out = _gather_le(data, o.src.begin, 2, idx).astype(np.uint16)
    else:
        with np.errstate(invalid="ignore", over="ignore"):
            out = OUT_ROUND[out_dtype](value(o, data, idx))
    return out.reshape(o.shape) if flat else out


def materialize(buf, out_dtype: str = "bf16") -> dict:
    """{name: output bits of the logical shape} for every output of a whole file's bytes."""
    h, outs = plan(buf)
    data = np.frombuffer(memoryview(buf), dtype=np.uint8, offset=h.data_offset)
    with np.errstate(invalid="ignore", over="ignore"):
        return {o.name: decode(o, data, out_dtype=out_dtype) for o in outs}
