"""The five seeded synthetic checkpoint families, full size and scaled down.

Each family stands in for a checkpoint kind the pages name (ComfyUI's scaled-FP8 diffusion
models, Qwen block-FP8 LLMs, NVIDIA ModelOpt NVFP4); the trained weights themselves are not
needed, only their shapes, dtypes, value distributions and byte layout.

* ``tiny``       8 tensors + 2 scales, back-to-back (unaligned), about 1.6 MB of traffic.
* ``scaled_fp8`` DiT-style blocks of e4m3fn weights with one fp32 ``scale_weight`` each.
* ``block_fp8``  LLM-style layers of e4m3fn weights with an fp32 ``weight_scale_inv`` grid of
                 one value per 128x128 block, plus a bf16 embedding and norms.
* ``nvfp4``      packed e2m1 weights (U8 [M, K/2]) with e4m3fn ``weight_scale`` per 16
                 elements along K and an fp32 ``weight_scale_2`` per tensor.
* ``many_small`` 20,000 tensors of 64 B - 64 KB, mixed dtypes, packed unaligned.
* ``mxfp8``      the block-FP8 layer shapes as OCP MXFP8: e4m3fn weights with one E8M0
                 ``weight_scale`` per 32 elements along K.
* ``mxfp4``      the NVFP4 layer shapes as OCP MXFP4: packed e2m1 (U8 [M, K/2]) with one E8M0
                 ``weight_scale`` per 32 elements along K.

Seeds: the checkpoint's seed defaults to its config number (1..7); every group of tensors
draws from ``default_rng([seed, group_index])`` so generation can run in parallel and stays
reproducible.  Weights are N(0, 0.02) before quantisation; quantised weights are
``e4m3(clip(w / scale, -448, 448))`` with torch's round-to-nearest-even float8_e4m3fn cast.
"""
from __future__ import annotations

import math
import os

import numpy as np

from .st_writer import Group, TensorSpec, build_bytes, write_file

E4M3_MAX = 448.0


def _torch():
    import torch
    return torch


def _normal(rng, n):
    x = rng.standard_normal(n, dtype=np.float32)
    x *= np.float32(0.02)
    return x


def _bf16(x):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy()


def _e4m3(x):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _numel(shape):
    n = 1
    for s in shape:
        n *= int(s)
    return n


# ----------------------------------------------------------------------------- group makers

def g_plain(name, dtype, shape, seed):
    """A BF16 / F16 / F32 tensor of N(0, 0.02) values."""
    n = _numel(shape)

    def make(rng):
        x = _normal(rng, n)
        if dtype == "BF16":
            return [_bf16(x)]
        if dtype == "F16":
            return [x.astype(np.float16)]
        if dtype == "F32":
            return [x]
        raise ValueError(dtype)

    return Group([TensorSpec(name, dtype, tuple(shape))], make, seed, cost=n)


def g_scaled_fp8(prefix, shape, seed, scale_lo=0.001, scale_hi=0.01):
    """``prefix.weight`` e4m3fn + ``prefix.scale_weight`` fp32 scalar, s ~ U(lo, hi)."""
    n = _numel(shape)

    def make(rng):
        s = np.float32(rng.uniform(scale_lo, scale_hi))
        w = _normal(rng, n)
        w /= s
        np.clip(w, -E4M3_MAX, E4M3_MAX, out=w)
        return [_e4m3(w), np.array(s, dtype=np.float32)]

    return Group([TensorSpec(prefix + ".weight", "F8_E4M3", tuple(shape)),
                  TensorSpec(prefix + ".scale_weight", "F32", ())], make, seed, cost=n)


def g_scaled_fp8_split(prefix, shape, seed, scale_lo=0.001, scale_hi=0.01):
    """The same pair as two groups (weight, scale) so the scale can sit elsewhere in the file;
    the scale comes from its own stream, default_rng([*seed, 1]), which both groups draw."""
    n = _numel(shape)

    def scale():
        return np.float32(np.random.default_rng([*seed, 1]).uniform(scale_lo, scale_hi))

    def make_w(rng):
        w = _normal(rng, n)
        w /= scale()
        np.clip(w, -E4M3_MAX, E4M3_MAX, out=w)
        return [_e4m3(w)]

    return (Group([TensorSpec(prefix + ".weight", "F8_E4M3", tuple(shape))], make_w, seed, cost=n),
            Group([TensorSpec(prefix + ".scale_weight", "F32", ())], lambda rng: [np.array(scale(), np.float32)],
                  (*seed, 2), cost=1))


def g_block_fp8(prefix, shape, seed, block=128):
    """``prefix.weight`` e4m3fn [M, N] + ``prefix.weight_scale_inv`` fp32 [ceil(M/128), ceil(N/128)]
    drawn log-uniform in [1e-4, 1e-2]; each weight is divided by its own block's value."""
    M, N = shape
    gm, gn = -(-M // block), -(-N // block)

    def make(rng):
        S = (10.0 ** rng.uniform(-4.0, -2.0, size=(gm, gn))).astype(np.float32)
        w = _normal(rng, M * N).reshape(M, N)
        for bi in range(gm):
            rows = w[bi * block:(bi + 1) * block]
            rows /= np.repeat(S[bi], block)[:N][None, :]
        np.clip(w, -E4M3_MAX, E4M3_MAX, out=w)
        return [_e4m3(w.reshape(-1)), S]

    return Group([TensorSpec(prefix + ".weight", "F8_E4M3", (M, N)),
                  TensorSpec(prefix + ".weight_scale_inv", "F32", (gm, gn))], make, seed, cost=M * N)


def g_nvfp4(prefix, shape, seed, storage="U8"):
    """NVFP4 weight of logical shape [M, K]: packed bytes uniform over all 256 values (so both
    nibbles are uniform over the 16 e2m1 codes), ``weight_scale`` e4m3fn [M, K/16] holding
    e4m3(2^U(-6, 6)), ``weight_scale_2`` fp32 scalar ~ U(1e-3, 1e-1)."""
    M, K = shape
    assert K % 16 == 0
    wshape = (M, K // 2) if storage == "U8" else (M, K)

    def make(rng):
        packed = np.frombuffer(rng.bytes(M * K // 2), dtype=np.uint8)
        bs = _e4m3(np.exp2(rng.uniform(-6.0, 6.0, size=M * K // 16)).astype(np.float32))
        g = np.float32(rng.uniform(1e-3, 1e-1))
        return [packed, bs, np.array(g, dtype=np.float32)]

    return Group([TensorSpec(prefix + ".weight", storage, wshape),
                  TensorSpec(prefix + ".weight_scale", "F8_E4M3", (M, K // 16)),
                  TensorSpec(prefix + ".weight_scale_2", "F32", ())], make, seed, cost=M * K // 2)


def g_mxfp8(prefix, shape, seed):
    """OCP MXFP8 weight [M, K]: N(0, 0.02) values quantised per block of 32 along K with the
    spec's shared exponent floor(log2(amax)) - 8 (8 = E4M3's largest exponent), stored as E8M0
    code exponent + 127, and elements e4m3(clip(v / 2^exponent, -448, 448))."""
    M, K = shape
    assert K % 32 == 0

    def make(rng):
        w = _normal(rng, M * K).reshape(M, K // 32, 32)
        amax = np.abs(w).max(axis=2)
        ex = np.where(amax > 0, np.floor(np.log2(np.maximum(amax, np.float32(1e-30)))) - 8, -127)
        code = np.clip(ex + 127, 0, 254).astype(np.uint8)
        q = w / np.exp2(code.astype(np.float64) - 127)[:, :, None].astype(np.float32)
        np.clip(q, -E4M3_MAX, E4M3_MAX, out=q)
        return [_e4m3(q.reshape(-1)), code.reshape(-1)]

    return Group([TensorSpec(prefix + ".weight", "F8_E4M3", (M, K)),
                  TensorSpec(prefix + ".weight_scale", "F8_E8M0", (M, K // 32))], make, seed, cost=M * K)


def g_mxfp4(prefix, shape, seed, storage="U8"):
    """OCP MXFP4 weight of logical shape [M, K]: packed bytes uniform over all 256 values, and
    ``weight_scale`` E8M0 [M, K/32] with exponents uniform in [-12, 2] (codes 115..129)."""
    M, K = shape
    assert K % 32 == 0
    wshape = (M, K // 2) if storage == "U8" else (M, K)

    def make(rng):
        packed = np.frombuffer(rng.bytes(M * K // 2), dtype=np.uint8)
        code = rng.integers(115, 130, size=M * K // 32, dtype=np.int64).astype(np.uint8)
        return [packed, code]

    return Group([TensorSpec(prefix + ".weight", storage, wshape),
                  TensorSpec(prefix + ".weight_scale", "F8_E8M0", (M, K // 32))], make, seed, cost=M * K // 2)


# ----------------------------------------------------------------------------- the families

def tiny(seed=1):
    gs = []
    k = 0

    def sd():
        nonlocal k
        k += 1
        return (seed, k)

    gs += [g_plain(f"bf16.{i}", "BF16", (256, 256), sd()) for i in range(2)]
    gs += [g_plain(f"f32.{i}", "F32", (512,), sd()) for i in range(2)]
    gs += [g_scaled_fp8(f"fp8.{i}", (384, 256), sd()) for i in range(2)]
    gs += [g_plain(f"f16.{i}", "F16", (64, 1000), sd()) for i in range(2)]
    return gs, {"synthetic": "tiny", "seed": seed}, False


def scaled_fp8(seed=2, blocks=57, hidden=3072, mlp=12288, scales_last=False):
    """Scales follow their weights (most weights then start 4, 8 or 12 bytes off a 16-byte line);
    with scales_last=True every scale moves to the end of the file and every weight is 16-byte
    aligned (same shapes and distributions, different draws)."""
    gs = []
    tail = []
    k = 0

    def sd():
        nonlocal k
        k += 1
        return (seed, k)

    def fp8(prefix, shape):
        if scales_last:
            w, sc = g_scaled_fp8_split(prefix, shape, sd())
            gs.append(w)
            tail.append(sc)
        else:
            gs.append(g_scaled_fp8(prefix, shape, sd()))

    for b in range(blocks):
        p = f"blocks.{b}."
        gs.append(g_plain(p + "norm1.weight", "BF16", (hidden,), sd()))
        for proj in ("q", "k", "v", "o"):
            fp8(p + f"attn.{proj}", (hidden, hidden))
            gs.append(g_plain(p + f"attn.{proj}.bias", "BF16", (hidden,), sd()))
        gs.append(g_plain(p + "norm2.weight", "BF16", (hidden,), sd()))
        fp8(p + "mlp.up", (mlp, hidden))
        fp8(p + "mlp.down", (hidden, mlp))
        gs.append(g_plain(p + "mlp.down.bias", "BF16", (hidden,), sd()))
    return gs + tail, {"synthetic": "scaled_fp8" + ("_aligned" if scales_last else ""), "seed": seed}, True


def block_fp8(seed=3, layers=28, hidden=4096, inter=12288, vocab=151936):
    gs = []
    k = 0

    def sd():
        nonlocal k
        k += 1
        return (seed, k)

    gs.append(g_plain("model.embed_tokens.weight", "BF16", (vocab, hidden), sd()))
    for l in range(layers):
        p = f"model.layers.{l}."
        gs.append(g_plain(p + "input_layernorm.weight", "BF16", (hidden,), sd()))
        for proj in ("q_proj", "k_proj", "v_proj", "o_proj"):
            gs.append(g_block_fp8(p + "self_attn." + proj, (hidden, hidden), sd()))
        gs.append(g_plain(p + "post_attention_layernorm.weight", "BF16", (hidden,), sd()))
        gs.append(g_block_fp8(p + "mlp.gate_proj", (inter, hidden), sd()))
        gs.append(g_block_fp8(p + "mlp.up_proj", (inter, hidden), sd()))
        gs.append(g_block_fp8(p + "mlp.down_proj", (hidden, inter), sd()))
    gs.append(g_plain("model.norm.weight", "BF16", (hidden,), sd()))
    return gs, {"synthetic": "block_fp8", "seed": seed}, True


def nvfp4(seed=4, layers=40, big=25600, small=5120, storage="U8"):
    gs = []
    k = 0

    def sd():
        nonlocal k
        k += 1
        return (seed, k)

    for l in range(layers):
        p = f"model.layers.{l}.mlp."
        gs.append(g_nvfp4(p + "up_proj", (big, small), sd(), storage))
        gs.append(g_nvfp4(p + "down_proj", (small, big), sd(), storage))
    return gs, {"synthetic": "nvfp4", "seed": seed}, True


def mxfp8(seed=6, layers=28, hidden=4096, inter=12288):
    gs = []
    k = 0

    def sd():
        nonlocal k
        k += 1
        return (seed, k)

    for l in range(layers):
        p = f"model.layers.{l}."
        gs.append(g_plain(p + "input_layernorm.weight", "BF16", (hidden,), sd()))
        for n in ("q_proj", "k_proj", "v_proj", "o_proj"):
            gs.append(g_mxfp8(p + "self_attn." + n, (hidden, hidden), sd()))
        gs.append(g_mxfp8(p + "mlp.gate_proj", (inter, hidden), sd()))
        gs.append(g_mxfp8(p + "mlp.up_proj", (inter, hidden), sd()))
        gs.append(g_mxfp8(p + "mlp.down_proj", (hidden, inter), sd()))
    return gs, {"synthetic": "mxfp8", "seed": seed}, True


def mxfp4(seed=7, layers=40, big=25600, small=5120, storage="U8"):
    gs = []
    k = 0

    def sd():
        nonlocal k
        k += 1
        return (seed, k)

    for l in range(layers):
        p = f"model.layers.{l}.mlp."
        gs.append(g_mxfp4(p + "up_proj", (big, small), sd(), storage))
        gs.append(g_mxfp4(p + "down_proj", (small, big), sd(), storage))
    return gs, {"synthetic": "mxfp4", "seed": seed}, True


def _divisors(n):
    out = []
    i = 1
    while i * i <= n:
        if n % i == 0:
            out.append(i)
            if i != n // i:
                out.append(n // i)
        i += 1
    return sorted(out)


def many_small(seed=5, count=20000, lo=64, hi=65536):
    meta = np.random.default_rng([seed, 0])
    gs = []
    kinds = ("BF16", "F16", "F32", "F8")
    item = {"BF16": 2, "F16": 2, "F32": 4, "F8": 1}
    for i in range(count):
        kind = kinds[int(meta.integers(4))]
        size = int(math.floor(math.exp(meta.uniform(math.log(lo), math.log(hi)))))
        numel = max(1, size // item[kind])
        if meta.random() < 0.5:
            shape = (numel,)
        else:
            d = _divisors(numel)
            r = d[int(meta.integers(len(d)))]
            shape = (r, numel // r)
        if kind == "F8":
            gs.append(g_scaled_fp8(f"t{i}", shape, (seed, i + 1)))
        else:
            gs.append(g_plain(f"t{i}.weight", kind, shape, (seed, i + 1)))
    return gs, {"synthetic": "many_small", "seed": seed}, False


CONFIGS = {
    1: ("tiny", tiny),
    2: ("scaled_fp8", scaled_fp8),
    3: ("block_fp8", block_fp8),
    4: ("nvfp4", nvfp4),
    5: ("many_small", many_small),
    6: ("mxfp8", mxfp8),
    7: ("mxfp4", mxfp4),
}

# Scaled-down variants that keep every structural feature (ragged 128-blocks, K % 32 == 16,
# 4-byte skews, mixed dtypes) at sizes the CPU oracle decodes in seconds.
SMALL = {
    1: {},
    2: {"blocks": 2, "hidden": 320, "mlp": 1280},
    3: {"layers": 2, "hidden": 320, "inter": 960, "vocab": 1000},
    4: {"layers": 2, "big": 400, "small": 208},
    5: {"count": 2000},
    6: {"layers": 2, "hidden": 320, "inter": 960},
    7: {"layers": 2, "big": 416, "small": 224},
}


def make_config(k, seed=None, small=False, **overrides):
    """Groups, metadata and header padding flag of config ``k`` (1..7)."""
    name, fn = CONFIGS[k]
    kw = dict(SMALL[k]) if small else {}
    kw.update(overrides)
    return fn(seed=k if seed is None else seed, **kw)


def config_bytes(k, seed=None, small=False, **overrides) -> bytes:
    groups, meta, pad = make_config(k, seed, small, **overrides)
    return build_bytes(groups, meta, pad)


def write_config(k, path, seed=None, small=False, workers=None, progress=None, **overrides):
    groups, meta, pad = make_config(k, seed, small, **overrides)
    torch = _torch()
    prev = torch.get_num_threads()
    nw = workers or min(16, os.cpu_count() or 1)
    if nw > 1:
        torch.set_num_threads(1)
    try:
        return write_file(path, groups, meta, pad, workers=nw, progress=progress)
    finally:
        torch.set_num_threads(prev)
