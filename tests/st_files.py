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


def write_sharded(dirpath, k, n_shards=3, index_name="model.safetensors.index.json", split_pair=False):
    """Config k (small) cut into n_shards files of consecutive tensor groups (a weight stays with its
    scales unless split_pair moves the first quantised group's scales into the next file), plus an
    index JSON; returns (file paths, {tensor name: file path}, [file bytes])."""
    import json
    import os

    import synth
    from synth.st_writer import Group, build_bytes
    groups, meta, pad = synth.make_config(k, small=True)
    per = -(-len(groups) // n_shards)
    parts = [list(groups[i:i + per]) for i in range(0, len(groups), per)]
    if split_pair:
        for p, part in enumerate(parts[:-1]):
            for gi, g in enumerate(part):
                if len(g.tensors) > 1:   # a weight with scales: its scales go to the next shard
                    w, scales = g.tensors[0], g.tensors[1:]
                    make = g.make
                    part[gi] = Group([w], (lambda m: lambda rng: m(rng)[:1])(make), g.seed)
                    parts[p + 1].insert(0, Group(scales, (lambda m: lambda rng: m(rng)[1:])(make), g.seed))
                    break
            else:
                continue
            break
    files, where, bufs = [], {}, []
    for i, part in enumerate(parts):
        name = f"model-{i + 1:05d}-of-{len(parts):05d}.safetensors"
        path = os.path.join(str(dirpath), name)
        buf = build_bytes(part, meta, pad)
        with open(path, "wb") as fh:
            fh.write(buf)
        files.append(path)
        bufs.append(buf)
        for g in part:
            for t in g.tensors:
                where[t.name] = name
    if index_name:
        with open(os.path.join(str(dirpath), index_name), "w") as fh:
            json.dump({"metadata": {"total_size": sum(len(b) for b in bufs)}, "weight_map": where}, fh)
    return files, {n: os.path.join(str(dirpath), f) for n, f in where.items()}, bufs
