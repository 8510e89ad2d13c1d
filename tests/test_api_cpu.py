"""CPU tests of the Python layer's module state: a CompressedLinear loads a state_dict
whose blob has another length (another weight or target rate), and a corrupt blob is
refused before the module changes.  Host code only (compress / serialize)."""
import os

import numpy as np
import pytest

L = pytest.importorskip("decode_tile_rans_amd._lib")
if not os.path.exists(L.LIB_PATH):
    pytest.skip("libentropack_hip.so not built", allow_module_level=True)

import torch  # noqa: E402

import decode_tile_rans_amd as ep  # noqa: E402


def _layer(seed, target, rows=64, cols=256):
    g = torch.Generator().manual_seed(seed)
    lin = torch.nn.Linear(cols, rows, dtype=torch.bfloat16)
    with torch.no_grad():
        lin.weight.copy_((torch.randn(rows, cols, generator=g) * 0.02).to(torch.bfloat16))
        lin.bias.copy_(torch.linspace(-1, 1, rows).to(torch.bfloat16))
    return ep.CompressedLinear.from_linear(lin, target_bpp=target)


def test_load_state_dict_of_another_length():
    a = _layer(1, 2.0)
    b = _layer(2, 5.0)
    assert a.packed.numel() != b.packed.numel()
    sd = a.state_dict()
    b.load_state_dict(sd)
    assert b.packed.numel() == a.packed.numel()
    assert torch.equal(b.packed, a.packed)
    assert b._c.to_bytes() == bytes(b.packed.numpy().tobytes())
    assert b._c.to_bytes() == a._c.to_bytes()
    assert b.compressed_bits == a.compressed_bits
    assert torch.equal(b.bias, a.bias)
    # and back: a smaller blob into the bigger one's module
    c = _layer(3, 6.0)
    c.load_state_dict(b.state_dict())
    assert c._c.to_bytes() == a._c.to_bytes()


def test_load_state_dict_other_shape_changes_features():
    a = _layer(4, 3.0, rows=32, cols=128)
    b = _layer(5, 3.0, rows=64, cols=256)
    sd = a.state_dict()
    b.bias = None                       # a layer without bias takes the blob only
    b.load_state_dict({"packed": sd["packed"]}, strict=False)
    assert (b.out_features, b.in_features) == (32, 128)
    assert b._c.to_bytes() == a._c.to_bytes()


def test_corrupt_blob_refused_without_change():
    a = _layer(6, 4.0)
    before = a._c.to_bytes()
    sd = a.state_dict()
    bad = sd["packed"].clone()[:-3]
    with pytest.raises(L.EPError):
        a.load_state_dict({"packed": bad, "bias": sd["bias"]})
    assert a._c.to_bytes() == before
    assert bytes(a.packed.numpy().tobytes()) == before
