"""The torch module on the host side (no GPU): converting a model compresses
every linear layer's weight losslessly, and a converted layer survives a
state_dict round trip through torch.save / torch.load(weights_only=True)."""
import io

import numpy as np
import pytest
import torch

import oracle
from decode_gemv_byte_amd.linear import NWCLinear, convert


def _bits(t):
    return t.detach().to(torch.bfloat16).contiguous().view(torch.int16).numpy().view(np.uint16)


def _model(seed=0):
    g = torch.Generator().manual_seed(seed)
    m = torch.nn.Sequential(torch.nn.Linear(96, 200), torch.nn.GELU(),
                            torch.nn.Sequential(torch.nn.Linear(200, 64, bias=False)), torch.nn.Linear(64, 8))
    with torch.no_grad():
        for p in m.parameters():
            p.copy_(torch.randn(p.shape, generator=g) * 0.05)
    return m


def test_convert_compresses_every_linear_losslessly():
    m = _model()
    originals = [(_bits(l.weight), l.bias) for l in m.modules() if isinstance(l, torch.nn.Linear)]
    convert(m, device="cpu")
    conv = [l for l in m.modules() if isinstance(l, NWCLinear)]
    assert not any(isinstance(l, torch.nn.Linear) for l in m.modules())
    assert len(conv) == len(originals) == 3
    for layer, (w, bias) in zip(conv, originals):
        blob = layer.blob.numpy()
        assert np.array_equal(oracle.decode(blob), w)          # the oracle reads the library's blob back exactly
        assert (layer.out_features, layer.in_features) == w.shape
        if bias is None:
            assert layer.bias is None
        else:
            assert torch.equal(layer.bias, bias.detach().to(torch.bfloat16))
        assert layer.compressed_bytes() == blob.size


def test_state_dict_round_trip():
    lin = torch.nn.Linear(300, 40)
    a = NWCLinear.from_linear(lin, device="cpu")
    buf = io.BytesIO()
    torch.save(a.state_dict(), buf)
    buf.seek(0)
    sd = torch.load(buf, weights_only=True)
    b = NWCLinear(sd["blob"].numpy(), sd["bias"], device="cpu")
    assert torch.equal(a.blob, b.blob) and torch.equal(a.bias, b.bias)
    assert (b.in_features, b.out_features) == (300, 40)
    b.load_state_dict(sd)                                   # same shapes: loads in place


def test_forward_rejects_wrong_feature_count():
    a = NWCLinear.from_linear(torch.nn.Linear(16, 8), device="cpu")
    with pytest.raises(ValueError):
        a(torch.zeros(3, 17))
