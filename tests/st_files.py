"""Hand-built safetensors files for tests (input construction only, no decode arithmetic)."""
import numpy as np

from synth.st_writer import Group, TensorSpec, build_bytes


def make_file(tensors, metadata=None, pad=False):
    """tensors: list of (name, dtype, shape, raw) with raw a bytes-like or numpy array."""
    groups = []
    for name, dtype, shape, raw in tensors:
        arr = np.frombuffer(bytes(raw) if not isinstance(raw, np.ndarray) else raw.tobytes(), np.uint8)
        groups.append(Group([TensorSpec(name, dtype, tuple(shape))], (lambda a: lambda rng: [a])(arr), (0,)))
    return build_bytes(groups, metadata, pad)


def raw_header_file(header_text, data=b""):
    """A file whose header is exactly ``header_text`` (str or bytes), for malformed-input tests."""
    h = header_text.encode() if isinstance(header_text, str) else header_text
    return len(h).to_bytes(8, "little") + h + data


def f32_bytes(*vals):
    return np.array(vals, dtype="<f4").tobytes()
