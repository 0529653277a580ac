"""GPU parity of lazy, on-demand materialisation: every key of every small checkpoint equals the
oracle through the direct path (one packed plan per load) and through the RAM tier (hits and
evictions); views load the same tensors; and a module whose weights are meta tensors runs a forward
pass whose forward_pre_hooks decode exactly the oracle's weights, under a device-memory bound."""
import numpy as np
import pytest
import torch

import oracle
import synth
import device_checkpoint_dequantisation_amd as st
from tests.test_lazy_host import _c2_block

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _file(tmp_path, k, **kw):
    buf = synth.config_bytes(k, small=k != 1, **kw)
    path = tmp_path / f"c{k}.safetensors"
    path.write_bytes(buf)
    return str(path), buf


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6, 7])
def test_every_key_matches_the_oracle(k, tmp_path):
    path, buf = _file(tmp_path, k)
    want = oracle.materialize(buf)
    sd = st.StreamStateDict(path, DEV)
    print(f"lazy c{k}: {len(sd)} keys", flush=True)
    got = sd.load(list(sd))                       # one packed plan for everything
    torch.cuda.synchronize()
    for name, w in want.items():
        assert np.array_equal(_bits(got[name]).reshape(w.shape), w), name
    names = list(sd)
    for name in names[:: max(1, len(names) // 25)]:   # single keys
        assert np.array_equal(_bits(sd[name]).reshape(want[name].shape), want[name]), name
    assert sd.stats["launches"] >= 1 and sd.stats["file_bytes"] > 0


def test_scales_last_layout(tmp_path):
    path, buf = _file(tmp_path, 2, scales_last=True)
    want = oracle.materialize(buf)
    sd = st.StreamStateDict(path, DEV, ram_cache_bytes=1 << 30)
    got = sd.load(list(sd)[::-1])
    torch.cuda.synchronize()
    for name, w in want.items():
        assert np.array_equal(_bits(got[name]).reshape(w.shape), w), name


@pytest.mark.parametrize("k", [2, 4, 5])
def test_ram_tier_hits_and_evictions(k, tmp_path):
    path, buf = _file(tmp_path, k)
    want = oracle.materialize(buf)
    sd = st.StreamStateDict(path, DEV, ram_cache_bytes=1 << 30)
    names = list(sd)
    sd.load(names)
    read_once = sd.stats["file_bytes"]
    got = sd.load(names)                          # every output from pinned RAM, no file reads
    torch.cuda.synchronize()
    assert sd.stats["ram_hits"] == len(names) and sd.stats["file_bytes"] == read_once
    for name, w in want.items():
        assert np.array_equal(_bits(got[name]).reshape(w.shape), w), name
    # a bound of a third of the bytes: evictions, and still exact results in mixed hit/miss loads
    total = sd.ram.bytes
    small = st.StreamStateDict(path, DEV, ram_cache_bytes=total // 3, ram_preallocate=False)  # slabs on demand
    rng = np.random.default_rng(k)
    for _ in range(4):
        pick = [names[i] for i in rng.choice(len(names), size=max(1, len(names) // 2), replace=False)]
        got = small.load(pick)
        torch.cuda.synchronize()
        for name in pick:
            assert np.array_equal(_bits(got[name]).reshape(want[name].shape), want[name]), name
    assert small.ram.evictions > 0 and small.ram.bytes <= total // 3
    # an output loaded on its own is kept (evicting others); loading it again is a hit
    x = max(names, key=lambda n: small.meta(n).source_bytes)
    small.load([x])
    hits = small.stats["ram_hits"]
    again = small.load([x])
    torch.cuda.synchronize()
    assert small.stats["ram_hits"] == hits + 1 and small.ram.bytes <= total // 3
    assert np.array_equal(_bits(again[x]).reshape(want[x].shape), want[x])


def test_views_load_the_same_tensors(tmp_path):
    path, buf = _file(tmp_path, 3)
    want = oracle.materialize(buf)
    sd = st.StreamStateDict(path, DEV)
    v = st.RenameViewStateDict(st.PrefixViewStateDict(sd, "model.layers.1."), [(r"_proj", "")])
    got = v.load(list(v))
    torch.cuda.synchronize()
    assert "self_attn.q.weight" in got
    for key, t in got.items():
        base = "model.layers.1." + key.replace("self_attn.q", "self_attn.q_proj").replace(
            "self_attn.k", "self_attn.k_proj").replace("self_attn.v", "self_attn.v_proj").replace(
            "self_attn.o", "self_attn.o_proj").replace("mlp.gate", "mlp.gate_proj").replace(
            "mlp.up", "mlp.up_proj").replace("mlp.down", "mlp.down_proj")
        assert np.array_equal(_bits(t).reshape(want[base].shape), want[base]), key


def _forward(blk, x):
    h = x * blk.norm1.weight.float()
    a = blk.attn
    h = h + torch.nn.functional.linear(
        torch.nn.functional.linear(h, a.q.weight.float(), a.q.bias.float())
        + torch.nn.functional.linear(h, a.k.weight.float(), a.k.bias.float())
        + torch.nn.functional.linear(h, a.v.weight.float(), a.v.bias.float()), a.o.weight.float(), a.o.bias.float())
    h = h * blk.norm2.weight.float()
    return h + torch.nn.functional.linear(torch.relu(torch.nn.functional.linear(h, blk.mlp.up.weight.float())),
                                          blk.mlp.down.weight.float(), blk.mlp.down.bias.float())


def test_module_forward_pre_hooks_decode_the_oracle_weights(tmp_path):
    path, buf = _file(tmp_path, 2)
    want = oracle.materialize(buf)
    sd = st.StreamStateDict(path, DEV, ram_cache_bytes=64 << 20)
    Block = _c2_block()

    class Model(torch.nn.Module):
        def __init__(self):
            super().__init__()
            self.blocks = torch.nn.ModuleList([Block(), Block()])

    model = Model()
    layer_bytes = sum(2 * m.numel for m in (sd.meta(k) for k in sd if k.startswith("blocks.0.")))
    loader = st.LazyModuleLoader(model, sd, max_resident_bytes=layer_bytes)
    assert all(p.is_meta for p in model.parameters())
    x = torch.randn(3, 320, device=DEV)
    y0 = _forward_all(model, loader, x)
    # decoded weights equal the oracle's, and the bound held: block 0 went back to meta
    for name in ("blocks.1.attn.q.weight", "blocks.1.mlp.down.weight", "blocks.1.attn.o.bias"):
        mod_name, pname = name.rsplit(".", 1)
        p = model.get_submodule(mod_name)._parameters[pname]
        assert not p.is_meta and np.array_equal(_bits(p.data).reshape(want[name].shape), want[name]), name
    assert loader.stats["evicted"] > 0 and model.blocks[0].attn.q.weight.is_meta
    assert loader.resident_bytes <= layer_bytes
    # the reference: the oracle's weights, the same float32 arithmetic
    ref = x
    for i in range(2):
        ref = _forward_ref(want, f"blocks.{i}.", ref)
    torch.testing.assert_close(y0, ref, rtol=1e-4, atol=1e-4)
    # a second pass reloads the evicted block (from the RAM tier) and gives the same result
    hits = sd.stats["ram_hits"]
    y1 = _forward_all(model, loader, x)
    assert torch.equal(y0, y1) and sd.stats["ram_hits"] > hits
    loader.evict_all()
    assert all(p.is_meta for p in model.parameters()) and loader.resident_bytes == 0
    loader.detach()


def _forward_all(model, loader, x):
    """Runs each leaf module once so its forward_pre_hook fires (the norms have no forward of their
    own and are materialised through the loader), then the block's arithmetic."""
    for b in model.blocks:
        for m in (b.norm1, b.norm2, b.attn.q, b.attn.k, b.attn.v, b.attn.o, b.mlp.up, b.mlp.down):
            if isinstance(m, torch.nn.Linear):
                m(torch.zeros(1, m.in_features, device=DEV, dtype=torch.bfloat16))  # fires the hook
            else:
                loader.materialize(m)
        x = _forward(b, x)
    torch.cuda.synchronize()
    return x


def _forward_ref(want, p, x):
    def w(n):
        return torch.from_numpy((want[p + n].astype(np.uint32) << 16).view(np.float32)).to(DEV)
    lin = torch.nn.functional.linear
    h = x * w("norm1.weight")
    h = h + lin(lin(h, w("attn.q.weight"), w("attn.q.bias")) + lin(h, w("attn.k.weight"), w("attn.k.bias"))
                + lin(h, w("attn.v.weight"), w("attn.v.bias")), w("attn.o.weight"), w("attn.o.bias"))
    h = h * w("norm2.weight")
    return h + lin(torch.relu(lin(h, w("mlp.up.weight"))), w("mlp.down.weight"), w("mlp.down.bias"))


def _busy(ms_target=300):
    """Keep the current stream busy for a while with matrix products (fp32, no transposed views)."""
    a = torch.randn(4096, 4096, device=DEV)
    for _ in range(max(1, ms_target // 2)):
        a = torch.mm(a, a) * 1e-3
    return a


def test_back_to_back_loads_behind_a_busy_stream(tmp_path):
    """The side stream's copies wait for the compute stream, so with a busy compute stream the first
    load's copies out of the pinned ring are still queued when it returns; the second load must not
    read the file into that ring before they have run.  Several keys per load, so every load spans
    several ring steps; no synchronisation between the loads."""
    path, buf = _file(tmp_path, 2)
    want = oracle.materialize(buf)
    sd = st.StreamStateDict(path, DEV, steps_per_load=8)
    names = list(sd)
    half = len(names) // 2
    first, second = names[:half], names[half:]
    print(f"back-to-back loads: {len(first)} + {len(second)} keys behind a busy stream", flush=True)
    busy = _busy()
    got1 = sd.load(first)
    got2 = sd.load(second)
    busy = _busy(100)
    got3 = sd.load(first[::-1])                   # and once more through a larger ring
    torch.cuda.synchronize()
    del busy
    for got in (got1, got2, got3):
        for name, t in got.items():
            assert np.array_equal(_bits(t).reshape(want[name].shape), want[name]), name


def test_device_checkpoint_restream_behind_a_busy_stream(tmp_path):
    """DeviceCheckpoint.stream twice on the same pinned ring and arena, the second call made while the
    first one's copies wait behind a busy compute stream."""
    path, buf = _file(tmp_path, 4)
    want = oracle.materialize(buf)
    ix = st.SafeTensorIndex.open(path)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    busy = _busy()
    ck.stream(path, chunk_mb=1)
    ck.stream(path, chunk_mb=1)
    ck.synchronize()
    del busy
    for name, w in want.items():
        assert np.array_equal(_bits(ck.tensors[name]).reshape(w.shape), w), name


def test_preallocated_ram_tier(tmp_path):
    """A tier whose pinned memory is created up front: loads fill it without new slabs, and later
    loads hit it; every tensor equals the oracle."""
    path, buf = _file(tmp_path, 2)
    want = oracle.materialize(buf)
    sd = st.StreamStateDict(path, DEV, ram_cache_bytes=1 << 30, ram_preallocate=True)
    slabs = len(sd.ram.arena.slabs)
    assert slabs >= 1 and sd.ram.arena.capacity >= sum(sd.meta(k).source_bytes for k in sd)
    names = list(sd)
    for rnd in range(2):
        got = sd.load(names)
        torch.cuda.synchronize()
        for name, t in got.items():
            assert np.array_equal(_bits(t).reshape(want[name].shape), want[name]), name
    assert len(sd.ram.arena.slabs) == slabs        # no slab was added while filling
    assert sd.stats["ram_hits"] == len(names)
