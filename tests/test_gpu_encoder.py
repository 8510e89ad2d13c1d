"""The GPU encoder against the oracle: byte-identical blobs.

Inputs are copied to the device as raw container values; the blob that
ep_compress_device returns must equal oracle.compress byte for byte, and its recorded
distortion must equal the host encoder's (same summation order).
"""
import numpy as np
import pytest

import synth
import oracle
from oracle import numerics as nx

pytestmark = pytest.mark.gpu

from gpu_util import say, stream_ptr  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    from decode_tile_rans_amd import _lib as L
    L.lib()
    yield


def _gpu_blob(src, dt, t, S=0):
    import torch
    from decode_tile_rans_amd import _lib as L
    src = np.ascontiguousarray(src)
    d = torch.from_numpy(src.view(np.uint8).reshape(-1).copy()).cuda()
    torch.cuda.synchronize()
    h = L.ep_compress_device(d.data_ptr(), dt, src.shape[0], src.shape[1], t, S, stream_ptr())
    try:
        return L.ep_serialize(h), L.ep_blob_distortion(h)
    finally:
        L.ep_blob_free(h)


def _host_dist(src, dt, t, S=0):
    from decode_tile_rans_amd import _lib as L
    src = np.ascontiguousarray(src)
    h = L.ep_compress(src.ctypes.data, dt, src.shape[0], src.shape[1], t, S)
    try:
        return L.ep_blob_distortion(h)
    finally:
        L.ep_blob_free(h)


CASES = [
    ("small_gauss_3.5", lambda: synth.small_gauss(), nx.DT_BF16, 3.5, 0),
    ("odd_37x13", lambda: synth.rowscaled(37, 13, 5), nx.DT_BF16, 4.0, 0),
    ("r512_8_escapes", lambda: synth.rowscaled(512, 512, 70), nx.DT_BF16, 8.0, 0),
    ("r512_2.3", lambda: synth.rowscaled(512, 512, 30), nx.DT_BF16, 2.3, 0),
    ("r512_11_wide", lambda: synth.rowscaled(256, 512, 31), nx.DT_BF16, 11.0, 0),
    ("outliers", lambda: synth.rowscaled(300, 1000, 40, 0.001), nx.DT_BF16, 4.0, 0),
    ("S8", lambda: synth.rowscaled(300, 520, 32), nx.DT_BF16, 4.0, 8),
    ("S64", lambda: synth.rowscaled(200, 512, 33), nx.DT_BF16, 3.0, 64),
    ("S2", lambda: synth.rowscaled(129, 777, 34), nx.DT_BF16, 5.0, 2),
    ("fp16", lambda: synth.rowscaled_f32(96, 200, 4).astype(np.float16).view(np.uint16), nx.DT_FP16, 4.0, 0),
    ("fp32", lambda: synth.rowscaled_f32(64, 256, 4), nx.DT_FP32, 6.0, 0),
    ("fp8", lambda: synth.fp8_codes(128, 256, 4)[0], nx.DT_FP8, 5.0, 0),
    ("int8", lambda: synth.int8_codes(128, 256, 4)[0], nx.DT_INT8, 4.0, 0),
    ("zeros", lambda: np.zeros((40, 48), np.uint16), nx.DT_BF16, 2.0, 0),
    ("low", lambda: synth.rowscaled(64, 256, 9), nx.DT_BF16, 0.001, 0),
    ("1x1", lambda: synth.rowscaled(1, 1, 9), nx.DT_BF16, 4.0, 0),
    ("4M default S=8", lambda: synth.rowscaled(1024, 4096, 41), nx.DT_BF16, 4.0, 0),
    ("sampled rows", lambda: synth.rowscaled(2048, 640, 42), nx.DT_BF16, 3.0, 0),
]


@pytest.mark.parametrize("name,gen,dt,t,S", CASES, ids=[c[0] for c in CASES])
def test_gpu_encoder_byte_parity(name, gen, dt, t, S):
    src = gen()
    say("gpu encoder", name, src.shape, dt, t, S)
    got, dist = _gpu_blob(src, dt, t, S)
    want = oracle.compress(src, dt, t, chains_per_tile=S or None)
    assert got == want
    assert dist == _host_dist(src, dt, t, S)


def test_gpu_encoder_random_small():
    rng = np.random.default_rng(4242)
    for i in range(12):
        R, C = int(rng.integers(1, 90)), int(rng.integers(1, 300))
        t = float(rng.choice([0.7, 1.0, 2.3, 3.5, 4.0, 6.0, 9.0]))
        S = int(rng.choice([0, 1, 2, 4, 8, 16]))
        src = synth.rowscaled(R, C, 600 + i, outlier_frac=0.01 if i % 3 == 0 else 0.0)
        say("gpu encoder random", R, C, t, S)
        got, _ = _gpu_blob(src, nx.DT_BF16, t, S)
        assert got == oracle.compress(src, nx.DT_BF16, t, chains_per_tile=S or None), (R, C, t, S)


def test_gpu_encoder_errors():
    from decode_tile_rans_amd import _lib as L
    bad = synth.rowscaled(8, 16, 1).copy()
    bad[3, 5] = 0x7FC0                     # a BF16 NaN
    with pytest.raises(L.EPError) as ei:
        _gpu_blob(bad, nx.DT_BF16, 4.0)
    assert ei.value.name == "EP_E_NONFINITE"
    with pytest.raises(L.EPError) as ei:
        _gpu_blob(synth.rowscaled(8, 16, 1), nx.DT_BF16, 12.0)
    assert ei.value.name == "EP_E_RANGE"


def test_api_compress_on_gpu_tensor():
    # ep.compress of a CUDA tensor goes through the GPU encoder and gives the same bytes
    # as compressing the host copy
    import torch
    import decode_tile_rans_amd as ep
    w = torch.from_numpy(synth.rowscaled(256, 1024, 77)).view(torch.bfloat16)
    c_gpu = ep.compress(w.cuda(), 3.5)
    c_cpu = ep.compress(w, 3.5)
    assert c_gpu.to_bytes() == c_cpu.to_bytes()
    y = ep.decompress(c_gpu)
    torch.cuda.synchronize()
    assert y.shape == w.shape and y.dtype == torch.bfloat16


def test_host_pointer_source_refused():
    from decode_tile_rans_amd import _lib as L
    src = np.ascontiguousarray(synth.rowscaled(16, 64, 1))
    with pytest.raises(L.EPError) as ei:
        L.ep_compress_device(src.ctypes.data, nx.DT_BF16, 16, 64, 4.0, 0, 0)
    assert ei.value.name == "EP_E_ARG"


def test_batch_entry_equals_single_calls():
    """ep_compress_device_batch over matrices of several shapes: every blob equals the
    single-matrix entry's, byte for byte; a bad matrix fails the call and names it."""
    import torch
    from decode_tile_rans_amd import _lib as L
    say("gpu encoder batch")
    shapes = [(256, 512), (37, 13), (300, 1000), (1024, 4096), (129, 777), (64, 256), (8, 16)]
    ws = [torch.from_numpy(synth.rowscaled(r, c, 500 + i)).view(torch.bfloat16).cuda() for i, (r, c) in enumerate(shapes)]
    sp = stream_ptr()
    torch.cuda.synchronize()
    hs = L.ep_compress_device_batch([w.data_ptr() for w in ws], shapes, L.EP_BF16, 3.5, 0, sp)
    try:
        for w, h, shp in zip(ws, hs, shapes):
            one = L.ep_compress_device(w.data_ptr(), L.EP_BF16, shp[0], shp[1], 3.5, 0, sp)
            try:
                assert L.ep_serialize(h) == L.ep_serialize(one), f"shape {shp}"
            finally:
                L.ep_blob_free(one)
    finally:
        for h in hs:
            L.ep_blob_free(h)
    bad = torch.full((16, 16), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.EPError, match="matrix 1"):
        L.ep_compress_device_batch([ws[0].data_ptr(), bad.data_ptr()], [shapes[0], (16, 16)], L.EP_BF16, 3.5, 0, sp)


def test_python_compress_many():
    import torch
    import decode_tile_rans_amd as ep
    say("compress_many")
    ws = [torch.from_numpy(synth.rowscaled(r, c, 600 + r)).view(torch.bfloat16).cuda() for r, c in ((64, 256), (96, 512), (40, 48))]
    many = ep.compress_many(ws, 3.0)
    for w, c in zip(ws, many):
        assert c.to_bytes() == ep.compress(w, 3.0).to_bytes()
        assert c.shape == tuple(w.shape) and c.dtype == torch.bfloat16
