"""The lazy state dict's host side, on the CPU: keys, shapes and dtypes from the header alone, the
prefix/filter/rename views, the RAM tier's LRU, and module attachment turning parameters into meta
tensors with their disk references (no tensor is read by any of these)."""
import numpy as np
import pytest
import torch

import synth
import device_checkpoint_dequantisation_amd as st
from device_checkpoint_dequantisation_amd.lazy import _Entry


@pytest.fixture(scope="module")
def c2(tmp_path_factory):
    path = tmp_path_factory.mktemp("lazy") / "c2.safetensors"
    path.write_bytes(synth.config_bytes(2, small=True))
    return str(path)


class _NoReads(st.StreamStateDict):
    def load(self, names, stream=None):
        raise AssertionError("a metadata operation loaded tensors")


def test_keys_and_meta_from_the_header_only(c2):
    sd = _NoReads(c2, device="cpu")
    ix = st.SafeTensorIndex.open(c2)
    outs = ix.outputs()
    assert list(sd) == [o.name for o in outs] and len(sd) == len(outs)
    assert "blocks.0.attn.q.weight" in sd and "blocks.0.attn.q.scale_weight" not in sd
    m = sd.meta("blocks.0.attn.q.weight")
    assert m.shape == (320, 320) and m.kind == "FP8_TENSOR" and m.source_dtype == "F8_E4M3"
    assert m.source_bytes == 320 * 320 + 4 and m.dtype == torch.bfloat16 and m.numel == 320 * 320
    t = sd.meta_tensor("blocks.0.mlp.up.weight")
    assert t.is_meta and t.shape == (1280, 320) and t.dtype == torch.bfloat16
    with pytest.raises(KeyError):
        sd.meta("nope")


def test_views(c2):
    sd = _NoReads(c2, device="cpu")
    blk = st.PrefixViewStateDict(sd, "blocks.1.")
    assert "attn.q.weight" in blk and "blocks.1.attn.q.weight" not in blk
    assert len(blk) == sum(1 for k in sd if k.startswith("blocks.1."))
    assert blk.meta("attn.q.weight") == sd.meta("blocks.1.attn.q.weight")
    added = st.PrefixViewStateDict(sd, "model.", strip=False)
    assert list(added) == ["model." + k for k in sd]
    w = st.FilterViewStateDict(sd, "*.weight")
    assert all(k.endswith(".weight") for k in w) and len(w) == sum(k.endswith(".weight") for k in sd)
    odd = st.FilterViewStateDict(sd, lambda k: k.startswith("blocks.0."))
    assert set(odd) == {k for k in sd if k.startswith("blocks.0.")}
    ren = st.RenameViewStateDict(sd, [(r"^blocks\.(\d+)\.", r"layers.\1."), (r"\.attn\.", ".self_attn.")])
    assert "layers.0.self_attn.q.weight" in ren and ren.meta("layers.1.mlp.up.weight").shape == (1280, 320)
    d = st.RenameViewStateDict(sd, {"blocks.0.norm1.weight": "first_norm"})
    assert "first_norm" in d and "blocks.0.norm2.weight" in d and len(d) == len(sd)
    with pytest.raises(KeyError, match="maps both"):
        list(st.RenameViewStateDict(sd, lambda k: "same"))
    # views compose and still load nothing
    nested = st.PrefixViewStateDict(st.FilterViewStateDict(sd, "blocks.1.*"), "blocks.1.attn.")
    assert sorted(nested) == sorted(k[len("blocks.1.attn."):] for k in sd if k.startswith("blocks.1.attn."))


def test_ram_cache_lru():
    class E:
        def __init__(self, n):
            self.nbytes = n
            self.where = None
    c = st.RamCache(100)
    assert c.put("a", E(40)) and c.put("b", E(40))
    assert c.get("a") is not None          # a is now the most recent
    assert c.put("c", E(40))               # evicts b
    assert c.keys() == ["a", "c"] and c.bytes == 80 and c.evictions == 1
    assert not c.put("big", E(101)) and "big" not in c
    assert c.put("a", E(10)) and c.bytes == 50
    c.clear()
    assert len(c) == 0 and c.bytes == 0
    assert not st.RamCache(0).put("x", E(1))


def _c2_block(hidden=320, mlp=1280):
    nn = torch.nn

    class Attn(nn.Module):
        def __init__(self):
            super().__init__()
            for n in "qkvo":
                setattr(self, n, nn.Linear(hidden, hidden))

    class Mlp(nn.Module):
        def __init__(self):
            super().__init__()
            self.up = nn.Linear(hidden, mlp, bias=False)
            self.down = nn.Linear(mlp, hidden)

    class Norm(nn.Module):
        def __init__(self):
            super().__init__()
            self.weight = nn.Parameter(torch.ones(hidden))

    class Block(nn.Module):
        def __init__(self):
            super().__init__()
            self.norm1, self.attn, self.norm2, self.mlp = Norm(), Attn(), Norm(), Mlp()

    return Block


def test_module_attach_makes_meta_parameters(c2):
    sd = _NoReads(c2, device="cpu")
    Block = _c2_block()
    blk = Block()
    loader = st.LazyModuleLoader(blk, st.PrefixViewStateDict(sd, "blocks.0."))
    assert all(p.is_meta for p in blk.parameters())
    assert len(loader.refs) == len(list(blk.parameters())) == 13
    ref = loader.refs[(blk.attn.q, "weight")]
    assert ref.key == "attn.q.weight" and ref.meta.kind == "FP8_TENSOR"
    assert blk.mlp.up.weight.dtype == torch.bfloat16 and blk.mlp.up.weight.shape == (1280, 320)
    loader.detach()


def test_module_attach_errors(c2):
    sd = _NoReads(c2, device="cpu")
    Block = _c2_block(hidden=320, mlp=640)
    with pytest.raises(ValueError, match="checkpoint shape"):
        st.LazyModuleLoader(Block(), st.PrefixViewStateDict(sd, "blocks.0."))
    extra = torch.nn.Linear(4, 4)
    with pytest.raises(KeyError, match="not in the state dict"):
        st.LazyModuleLoader(extra, sd)
    st.LazyModuleLoader(torch.nn.Linear(4, 4), sd, strict=False)  # nothing to attach: allowed


def test_pinned_arena_first_fit_and_coalescing():
    a = st.lazy.PinnedArena(4096, slab_bytes=2048, allocate=lambda n: torch.empty(n, dtype=torch.uint8))
    x = a.alloc(600)            # rounded to 768
    y = a.alloc(512)
    z = a.alloc(700)            # 768: slab 0 now holds 2048 bytes exactly
    assert x == (0, 0) and y == (0, 768) and z == (0, 1280) and a.free[0] == []
    w = a.alloc(100)            # a second slab
    assert w == (1, 0) and a.capacity == 4096
    assert a.alloc(4000) is None               # no room and no new slab under the bound
    a.release(0, 768, 512)
    a.release(0, 0, 600)
    assert a.free[0] == [[0, 1280]]            # the two holes merged
    assert a.alloc(1200) == (0, 0)             # first fit reuses it
    assert a.view(0, 0, 10).numel() == 10
    assert a.allocated == 1280 + 768 + 256


def test_ram_cache_protects_entries_in_use():
    class E:
        def __init__(self, n):
            self.nbytes, self.where, self.last_use = n, None, None
    c = st.RamCache(100)
    c.put("a", E(60))
    c.protected = {"a"}
    assert c.put("b", E(60))                   # over the bound, but "a" may not go
    assert "a" in c and "b" in c and c.evictions == 0
    c.protected = set()
    c.put("c", E(10))
    assert "a" not in c and c.evictions >= 1


def test_arena_slab_never_exceeds_the_bound():
    a = st.lazy.PinnedArena(1000, slab_bytes=256 << 20, allocate=lambda n: torch.empty(n, dtype=torch.uint8))
    assert a.slab_bytes == 1000
    assert a.alloc(300) == (0, 0) and a.capacity == 1000


def test_arena_prefetches_a_touched_spare_slab_within_the_bound():
    made = []

    def alloc(n):
        t = torch.full((n,), 7, dtype=torch.uint8)   # not zero: the spare must come back touched (zeroed)
        made.append(n)
        return t

    a = st.lazy.PinnedArena(8192, slab_bytes=2048, allocate=alloc, prefetch=True)
    assert a.capacity == 2048                 # the first spare, prepared in the background
    x = a.alloc(1000)
    assert x == (0, 0) and int(a.slabs[0].sum()) == 0
    for _ in range(4):                         # fill slabs; spares stop once another slab would not fit
        a.alloc(2000)
    assert sum(t.numel() for t in a.slabs) <= 8192 and a.capacity <= 8192
    assert a.alloc(2000) is None               # the bound is full
    big = st.lazy.PinnedArena(8192, slab_bytes=2048, allocate=alloc, prefetch=True)
    assert big.alloc(5000) == (0, 0)           # an entry larger than a slab gets a slab of its own
    assert big.slabs[0].numel() == 5120 and big.capacity <= 8192   # rounded to 256


def test_arena_reserve_slabs_up_front():
    a = st.lazy.PinnedArena(8192, slab_bytes=2048, allocate=lambda n: torch.full((n,), 9, dtype=torch.uint8),
                            prefetch=False)
    assert a.reserve_slabs(5000) == 6144            # three slabs, touched (zeroed)
    assert all(int(t.sum()) == 0 for t in a.slabs)
    assert a.alloc(2000) == (0, 0) and a.alloc(2000) == (1, 0)   # entries land in the reserved slabs
    assert a.reserve_slabs(1 << 20) == 8192         # never past the bound


def test_arena_reserve_takes_the_prepared_spare():
    a = st.lazy.PinnedArena(8192, slab_bytes=2048, allocate=lambda n: torch.zeros(n, dtype=torch.uint8), prefetch=True)
    assert a.reserve_slabs(1000) == 2048 and len(a.slabs) == 1   # the spare, now a slab
    assert a.alloc(1000) == (0, 0) and len(a.slabs) == 1


def test_fill_batches_cover_every_miss_in_order():
    from device_checkpoint_dequantisation_amd.lazy import _batches
    assert _batches([], 4) == []
    assert _batches([5], 4) == [[0]]
    assert _batches([10] * 13, 4) == [[0, 1, 2, 3], [4, 5, 6], [7, 8, 9], [10, 11, 12]]
    assert _batches([100, 1, 1, 1], 2) == [[0], [1, 2, 3]]
