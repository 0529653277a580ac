"""GPU: checkpoints written by the safetensors library itself (its header padding, its tensor
order, its dtype strings), loaded end to end with ``load`` (streamed and serial) and compared with
the oracle bit for bit, and with torch's own decoding of the same tensors."""
import numpy as np
import pytest
import torch

import oracle
import device_checkpoint_dequantisation_amd as st

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _checkpoint(seed):
    from safetensors.torch import save
    g = torch.Generator().manual_seed(seed)
    t = {}
    t["embed.weight"] = (torch.randn(1000, 256, generator=g) * 0.02).to(torch.bfloat16)
    t["norm.weight"] = torch.randn(256, generator=g).to(torch.float16)
    t["head.bias"] = torch.randn(300, generator=g)
    w = torch.randn(300, 256, generator=g) * 4
    t["q.weight"] = w.to(torch.float8_e4m3fn)
    t["q.weight_scale_inv"] = torch.rand(3, 2, generator=g) * 0.01 + 1e-4
    t["s.weight"] = (torch.randn(64, 96, generator=g) * 8).to(torch.float8_e4m3fn)
    t["s.scale_weight"] = torch.tensor(0.0123)
    t["m.weight"] = (torch.randn(48, 128, generator=g) * 8).to(torch.float8_e4m3fn)
    t["m.weight_scale"] = torch.randint(115, 135, (48, 4), generator=g, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu)
    t["n.weight"] = torch.randint(0, 256, (32, 64), generator=g, dtype=torch.int32).to(torch.uint8)
    t["n.weight_scale"] = (torch.rand(32, 8, generator=g) * 8 + 0.1).to(torch.float8_e4m3fn)
    t["n.weight_scale_2"] = torch.tensor(0.037)
    return save(t), t


@pytest.mark.parametrize("streamed", [True, False])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_library_written_checkpoint(streamed, out_dtype, tmp_path):
    buf, t = _checkpoint(7)
    p = tmp_path / "lib.safetensors"
    p.write_bytes(buf)
    print(f"library-written checkpoint: {len(buf)} bytes, streamed={streamed}, {out_dtype}", flush=True)
    got = st.load(str(p), DEV, streamed=streamed, chunk_mb=1, out_dtype=out_dtype)
    want = oracle.materialize(buf, out_dtype)
    assert sorted(got) == sorted(want)
    for name, w in want.items():
        g = got[name].contiguous()
        bits = (g.view(torch.int32) if out_dtype == "f32" else g.view(torch.int16)).cpu().numpy().view(w.dtype)
        assert np.array_equal(bits.reshape(w.shape), w), name
    # torch's own decoding of the two-step definition agrees too
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    ref = (t["s.weight"].float() * t["s.scale_weight"]).to(tdt)
    assert torch.equal(got["s.weight"].cpu(), ref)
    S = t["q.weight_scale_inv"].repeat_interleave(128, 0)[:300].repeat_interleave(128, 1)[:, :256]
    assert torch.equal(got["q.weight"].cpu(), (t["q.weight"].float() * S).to(tdt))
    E = t["m.weight_scale"].float().repeat_interleave(32, 1)
    assert torch.equal(got["m.weight"].cpu(), (t["m.weight"].float() * E).to(tdt))
    if out_dtype == "bf16":     # a bf16 source keeps its bits
        assert torch.equal(got["embed.weight"].cpu().view(torch.int16), t["embed.weight"].view(torch.int16))
