"""GPU parity of TileANS (lossless) decoding: every byte equal to the input.

Blobs are made by the oracle (``oracle.tileans``); the GPU decodes them through the
C ABI into byte buffers.  Every chain must end in its initial state (device error
count 0).
"""
import os

import numpy as np
import pytest

import synth
from oracle import tileans

pytestmark = pytest.mark.gpu

from gpu_util import say, stream_ptr  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    from decode_tile_rans_amd import _lib as L
    L.lib()
    yield


def _raw(a):
    return np.frombuffer(np.ascontiguousarray(a).tobytes(), dtype=np.uint8).copy()


class DevTA:
    def __init__(self, blob):
        from decode_tile_rans_amd import _lib as L
        self.L = L
        self.h = L.ep_deserialize(blob)
        L.ep_blob_upload(self.h, stream_ptr())
        self.n = tileans.parse(blob).n_bytes

    def out(self, fill=0):
        import torch
        t = torch.empty(self.n, dtype=torch.uint8, device="cuda")
        t.fill_(fill)
        return t

    def decode(self, fill=0):
        import torch
        o = self.out(fill)
        self.L.ep_decompress(self.h, o.data_ptr(), stream_ptr())
        torch.cuda.synchronize()
        return o.cpu().numpy()

    def errors(self):
        return self.L.ep_blob_device_errors(self.h)

    def __del__(self):
        try:
            self.L.ep_blob_free(self.h)
        except Exception:
            pass


def _with_env(env, fn):
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        return fn()
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


CASES = [
    ("bf16", lambda: synth.rowscaled(96, 200, 1), 2, None),
    ("bf16 S8 4 MiB", lambda: synth.rowscaled(1024, 2048, 9), 2, None),
    ("fp32 3-d", lambda: synth.rowscaled_f32(8, 24, 3).reshape(2, 4, 24), 4, 2),
    ("fp16 1-d ragged", lambda: synth.rowscaled_f32(1, 1001, 4).astype(np.float16).reshape(-1), 2, 1),
    ("fp8", lambda: synth.fp8_codes(64, 136, 5)[0], 1, 4),
    ("int8 S64", lambda: synth.int8_codes(32, 520, 6)[0], 1, 64),
    ("int64 4-d", lambda: np.random.default_rng(7).integers(-5, 5, size=(2, 3, 5, 7)), 8, None),
    ("one byte", lambda: np.array([200], dtype=np.uint8), 1, None),
    ("zeros", lambda: np.zeros((33, 17), dtype=np.uint16), 2, None),
    ("random", lambda: np.random.default_rng(8).integers(0, 256, size=5000, dtype=np.uint8), 1, None),
    ("odd length S8", lambda: np.random.default_rng(10).integers(0, 9, size=(3, 100003), dtype=np.uint8), 1, 8),
]


@pytest.mark.parametrize("name,gen,E,S", CASES, ids=[c[0] for c in CASES])
def test_decode_parity(name, gen, E, S):
    a = gen()
    raw = _raw(a)
    blob = tileans.compress(raw, E, a.shape, 3, chains_per_tile=S)
    say("tileans", name, a.shape, E, S)
    d = DevTA(blob)
    got = d.decode(fill=0x5A)
    assert np.array_equal(got, raw)
    assert d.errors() == 0


@pytest.mark.parametrize("env", [{"EP_DECODE_ILP": "2", "EP_DECODE_WAVES": "3"}, {"EP_DECODE_WAVES": "1"},
                                 {"EP_DECODE_WAVES": "5", "EP_DECODE_BPW": "7"}])
def test_launch_shapes(env):
    a = synth.rowscaled(300, 520, 20)
    raw = _raw(a)
    blob = tileans.compress(raw, 2, a.shape, 0, chains_per_tile=8)
    say("tileans shape", env)
    d = DevTA(blob)
    got = _with_env(env, lambda: d.decode())
    assert np.array_equal(got, raw) and d.errors() == 0


def test_tile_ranges():
    import torch
    a = synth.rowscaled(64, 1032, 21)      # 132 096 bytes = 32.25 tiles
    raw = _raw(a)
    blob = tileans.compress(raw, 2, a.shape, 0, chains_per_tile=4)
    d = DevTA(blob)
    n_tiles = tileans.parse(blob).n_tiles
    for (t0, t1) in [(0, 1), (n_tiles - 1, n_tiles), (3, 10), (n_tiles // 2, n_tiles)]:
        say("tileans tiles", t0, t1)
        o = d.out(0x5A)
        d.L.ep_decompress_tiles(d.h, t0, t1, o.data_ptr(), stream_ptr())
        torch.cuda.synchronize()
        got = o.cpu().numpy()
        sel = np.zeros(len(raw), dtype=bool)
        sel[4096 * t0: 4096 * t1] = True
        assert np.array_equal(got[sel], raw[sel]) and (got[~sel] == 0x5A).all()
    assert d.errors() == 0


def test_batch():
    import torch
    rng = np.random.default_rng(22)
    arrs = [synth.rowscaled(int(rng.integers(10, 300)), int(rng.choice([64, 200, 1000])), 30 + i) for i in range(14)]
    arrs.append(np.random.default_rng(23).integers(0, 256, size=70000, dtype=np.uint8))
    devs, raws = [], []
    for i, a in enumerate(arrs):
        raw = _raw(a)
        E = 1 if a.dtype == np.uint8 else 2
        devs.append(DevTA(tileans.compress(raw, E, a.shape, 0, chains_per_tile=int(rng.choice([1, 2, 8])))))
        raws.append(raw)
    outs = [d.out(0x5A) for d in devs]
    say("tileans batch", len(devs))
    devs[0].L.ep_decompress_batch([d.h for d in devs], [o.data_ptr() for o in outs], stream_ptr())
    torch.cuda.synchronize()
    for d, o, r in zip(devs, outs, raws):
        assert np.array_equal(o.cpu().numpy(), r) and d.errors() == 0


def test_api_round_trip_dtypes():
    import torch
    import decode_tile_rans_amd as ep
    g = torch.Generator().manual_seed(5)
    tensors = [torch.randn(7, 9, 11, generator=g).to(torch.bfloat16), torch.randn(1000, generator=g).to(torch.float16),
               torch.randn(4, 257, generator=g, dtype=torch.float64), torch.randint(0, 2, (33, 5), generator=g).bool(),
               torch.randint(-1000, 1000, (3, 3, 3, 3), generator=g, dtype=torch.int16),
               (torch.randn(64, 64, generator=g) * 3).to(torch.float8_e4m3fn),
               torch.randint(-5, 5, (513,), generator=g, dtype=torch.int64)]
    for t in tensors:
        say("tileans api", t.dtype, tuple(t.shape))
        c = ep.compress_lossless(t)
        raw = t.contiguous().reshape(-1).view(torch.uint8).numpy()
        assert c.to_bytes() == tileans.compress(raw, t.element_size(), tuple(t.shape), c_tag(c))
        y = ep.decompress(c)
        torch.cuda.synchronize()
        assert y.dtype == t.dtype and tuple(y.shape) == tuple(t.shape)
        assert torch.equal(y.cpu().view(torch.uint8), t.view(torch.uint8))
        assert c.device_errors() == 0


def c_tag(c):
    from decode_tile_rans_amd import _lib as L
    return L.ep_blob_dtype(c.handle)
