"""GPU checks of the quantised passthrough: weights and scales handed over as stored (views or
aligned copies of the staged bytes, lazily from a packed blob too) equal the file's bytes, and
decoding them with plain torch arithmetic gives exactly the kernel's bf16 outputs."""
import numpy as np
import pytest
import torch

import synth
import device_checkpoint_dequantisation_amd as st

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def _decode(q):
    """bf16 from a QuantizedWeight with torch: the pages' products in order, one rounding each."""
    if q.kind == "FP8_TENSOR":
        return (q.data.float() * q.scale).to(torch.bfloat16)
    if q.kind == "FP8_BLOCK128":
        m, n = q.shape
        S = q.scale.repeat_interleave(128, 0)[:m].repeat_interleave(128, 1)[:, :n]
        return (q.data.float() * S).to(torch.bfloat16)
    m, k = q.shape
    if q.kind in ("MXFP8", "MXFP4"):   # torch's E8M0 decoding, on the CPU
        S = q.scale.cpu().float().to(q.data.device).repeat_interleave(32, 1)
        if q.kind == "MXFP8":
            return (q.data.float() * S).to(torch.bfloat16)
        nib = torch.stack([q.data & 15, q.data >> 4], dim=-1).reshape(m, k).long()
        return (torch.tensor(E2M1, device=q.data.device)[nib] * S).to(torch.bfloat16)
    nib = torch.stack([q.data & 15, q.data >> 4], dim=-1).reshape(m, k).long()
    t = torch.tensor(E2M1, device=q.data.device)[nib] * q.scale.float().repeat_interleave(16, 1)
    return (t * q.scale2).to(torch.bfloat16)


@pytest.mark.parametrize("k", [2, 3, 4, 6, 7])
@pytest.mark.parametrize("copy", [True, False])
def test_quantized_passthrough(k, copy, tmp_path):
    buf = synth.config_bytes(k, small=True)
    ix = st.SafeTensorIndex.from_bytes(buf)
    ck = st.DeviceCheckpoint(ix, None, DEV)
    ck.load_bytes(buf[ix.data_offset:])
    ck.materialize()
    qs = ck.quantized(copy=copy)
    torch.cuda.synchronize()
    data = np.frombuffer(buf, np.uint8)[ix.data_offset:]
    ents = ix.tensors()
    outs = {o.name: o for o in ix.outputs()}
    assert qs and set(qs) == {n for n, o in outs.items() if o.kind in st.QUANTIZED_KINDS}
    for name, q in qs.items():
        o = outs[name]
        w = ents[o.tensor]
        assert np.array_equal(q.data.reshape(-1).view(torch.uint8).cpu().numpy(), data[w.begin:w.end])
        s = ents[o.scale]
        assert np.array_equal(q.scale.reshape(-1).view(torch.uint8).cpu().numpy(), data[s.begin:s.end])
        if copy:
            assert q.data.data_ptr() % 256 == 0
        else:
            assert q.data.data_ptr() == ck.blob.data_ptr() + w.begin
        assert torch.equal(_decode(q).view(torch.int16), ck.tensors[name].view(torch.int16)), name
    plain = [n for n, o in outs.items() if o.kind not in st.QUANTIZED_KINDS]
    if plain:
        with pytest.raises(ValueError):
            ck.quantized(plain[:1])


def test_lazy_quantized_matches(tmp_path):
    buf = synth.config_bytes(4, small=True)
    path = tmp_path / "c4.safetensors"
    path.write_bytes(buf)
    sd = st.StreamStateDict(str(path), DEV)
    names = [n for n in sd if sd.meta(n).kind == "NVFP4"]
    qs = sd.load_quantized(names)
    full = sd.load(names)
    torch.cuda.synchronize()
    for n in names:
        assert torch.equal(_decode(qs[n]).view(torch.int16), full[n].view(torch.int16)), n
