"""GPU tests of the decoder's container casts (ep_test_cast runs the same device code the
decode kernel stores with) against the oracle's casts, element by element, bit for bit:
every finite value with a BF16 bit pattern, the FP8 rounding boundaries (each code's
value, the midpoints to its neighbours and one float32 ulp either side, the subnormal
steps, the saturation edge) and log-uniform random values, with both signs."""
import numpy as np
import pytest

from oracle import numerics as nx

pytestmark = pytest.mark.gpu

from gpu_util import say, stream_ptr  # noqa: E402


def _inputs():
    parts = []
    bits = np.arange(1 << 16, dtype=np.uint32) << 16           # every BF16 pattern as float32
    f = bits.view(np.float32)
    parts.append(f[np.isfinite(f)])
    # FP8 E4M3FN grid: codes 0..126 (0x7f is NaN), their midpoints, +-1 ulp around each
    codes = nx.fp8_e4m3fn_to_f64(np.arange(127, dtype=np.uint8)).astype(np.float32)
    mids = ((codes[:-1].astype(np.float64) + codes[1:]) / 2).astype(np.float32)
    edge = np.concatenate([codes, mids, np.float32([464.0, 480.0, 500.0, 1e6, 3e38, 2.0 ** -10, 2.0 ** -11,
                                                    1e-30, 0.0])])
    parts += [edge, np.nextafter(edge, np.float32(np.inf)), np.nextafter(edge, np.float32(-np.inf))]
    # INT8 rounding: halves and their neighbours up to the clamp edges
    halves = (np.arange(-140, 141, dtype=np.float32) + np.float32(0.5))
    parts += [halves, np.nextafter(halves, np.float32(np.inf)), np.nextafter(halves, np.float32(-np.inf))]
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-24, 12, 1 << 20)).astype(np.float32)
    parts.append(mag)
    x = np.concatenate(parts).astype(np.float32)
    x = np.concatenate([x, -x])
    # a ragged tail (not a multiple of 8)
    return np.concatenate([x, np.float32([0.3, -0.7, 5.5])])


CASES = [("bf16", nx.DT_BF16, 0, np.uint16, nx.cast_bf16_sat),
         ("fp16", nx.DT_FP16, 0, np.uint16, nx.cast_fp16_sat),
         ("fp8-bits", nx.DT_FP8, 0, np.uint8, nx.cast_fp8_sat),
         ("fp8-instruction", nx.DT_FP8, 1, np.uint8, nx.cast_fp8_sat),
         ("int8", nx.DT_INT8, 0, np.int8, nx.cast_int8_sat)]


@pytest.mark.parametrize("name,dt,hw,npdt,ref", CASES, ids=[c[0] for c in CASES])
def test_container_cast_matches_oracle(name, dt, hw, npdt, ref):
    import torch
    from decode_tile_rans_amd import _lib as L
    x = _inputs()
    if dt == nx.DT_INT8:            # the INT8 cast takes values the decoder can produce
        x = x[np.abs(x) < 1e9]
    say("cast", name, x.size)
    xin = torch.from_numpy(x).cuda()
    out = torch.empty(x.size * np.dtype(npdt).itemsize, dtype=torch.uint8, device="cuda")
    L.ep_test_cast(dt, xin.data_ptr(), out.data_ptr(), x.size, hw, stream_ptr())
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(npdt)
    want = np.asarray(ref(x)).view(npdt)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} differ, first x={x[bad[0]]!r} got {got[bad[0]]} want {want[bad[0]]}"


def test_cast_refusals():
    import torch
    from decode_tile_rans_amd import _lib as L
    x = torch.zeros(8, device="cuda")
    with pytest.raises(L.EPError):
        L.ep_test_cast(nx.DT_FP32, x.data_ptr(), x.data_ptr(), 8, 0, stream_ptr())
    with pytest.raises(L.EPError):
        L.ep_test_cast(nx.DT_BF16, np.zeros(8, np.float32).ctypes.data, x.data_ptr(), 8, 0, stream_ptr())
