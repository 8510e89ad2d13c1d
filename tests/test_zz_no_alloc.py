"""GPU test of ep_compressed_matvec_noalloc (the fused product whose partial sums live in
the library's own scratch array, for callers that cannot allocate): its outputs equal
ep_compressed_matvec's (same kernels, same summation order) bit for bit, on two calls
in a row, the second with a smaller input, and both within the per-element bound of the
oracle product; a blob whose partial sums exceed the array is refused before any launch."""
import numpy as np
import pytest

import synth
import oracle
from oracle import numerics as nx
from oracle.gemm import linear_ref

pytestmark = pytest.mark.gpu

from gpu_util import DevBlob, check_linear, say, stream_ptr  # noqa: E402


def _t(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).view(dtype).cuda()


def _bits(y):
    import torch
    return y.cpu().view(torch.int16).numpy().view(np.uint16)


def _case(L, R, C, T, bpp, seed, with_bias):
    import torch
    say("no-alloc matvec", R, C, T, bpp, seed)
    blob = oracle.compress(synth.rowscaled(R, C, seed), nx.DT_BF16, bpp, chains_per_tile=8)
    _, w_hat, _ = oracle.decode(blob)
    x = synth.activations(T, C, seed + 1)
    bias = synth.f32_to_bf16_bits(np.linspace(-0.5, 0.5, R).astype(np.float32)) if with_bias else None
    db = DevBlob(blob)
    xt = _t(x, torch.bfloat16)
    bt = _t(bias, torch.bfloat16) if bias is not None else None
    bp = bt.data_ptr() if bt is not None else 0
    need = L.ep_matvec_workspace_bytes(db.h, T)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y_ws = torch.full((T, R), 3.0, dtype=torch.bfloat16, device="cuda")
    y_na = torch.full((T, R), 5.0, dtype=torch.bfloat16, device="cuda")
    L.ep_compressed_matvec(db.h, xt.data_ptr(), T, bp, y_ws.data_ptr(), ws.data_ptr(), need, stream_ptr())
    L.ep_compressed_matvec_noalloc(db.h, xt.data_ptr(), T, bp, y_na.data_ptr(), stream_ptr())
    torch.cuda.synchronize()
    got_ws, got_na = _bits(y_ws), _bits(y_na)
    assert np.array_equal(got_na, got_ws)
    xf, wf = nx.bf16_to_f64(x), nx.bf16_to_f64(w_hat)
    bf = nx.bf16_to_f64(bias) if bias is not None else None
    ref = linear_ref(xf, wf, bf)
    mag = linear_ref(np.abs(xf), np.abs(wf), np.abs(bf) if bf is not None else None)
    check_linear(nx.bf16_to_f64(got_na), ref, mag, C)
    assert db.errors() == 0


def test_noalloc_matches_workspace_entry_twice():
    from decode_tile_rans_amd import _lib as L
    # a larger call, then a smaller one (fewer chains, fewer rows, fewer tokens): the
    # second reads only the slots its own decode wrote, whatever the first left behind
    _case(L, 3000, 1024, 8, 4.0, 301, True)
    _case(L, 200, 512, 3, 3.0, 302, False)


def test_noalloc_refuses_oversize_and_bad_arguments():
    import torch
    from decode_tile_rans_amd import _lib as L
    say("no-alloc refusals")
    # 65536 x 64 at S = 8: 8192 chains x 65 row slots x 8 tokens x 4 bytes = 17 MB of
    # partial sums, more than the 16 MiB array
    big = oracle.compress(synth.rowscaled(65536, 64, 303), nx.DT_BF16, 4.0, chains_per_tile=8)
    db = DevBlob(big)
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((8, 65536), dtype=torch.bfloat16, device="cuda")
    assert L.ep_matvec_workspace_bytes(db.h, 8) - 256 > 16 << 20
    with pytest.raises(L.EPError) as e:
        L.ep_compressed_matvec_noalloc(db.h, x.data_ptr(), 8, 0, y.data_ptr(), stream_ptr())
    assert e.value.code == -9
    # 4 tokens fit (half the slots per chain)
    assert L.ep_matvec_workspace_bytes(db.h, 4) - 256 <= 16 << 20
    small = DevBlob(oracle.compress(synth.rowscaled(64, 256, 304), nx.DT_BF16, 4.0))
    xs = torch.zeros((9, 256), dtype=torch.bfloat16, device="cuda")
    ys = torch.empty((9, 64), dtype=torch.bfloat16, device="cuda")
    for T in (0, 9):
        with pytest.raises(L.EPError):
            L.ep_compressed_matvec_noalloc(small.h, xs.data_ptr(), T, 0, ys.data_ptr(), stream_ptr())
    with pytest.raises(L.EPError):   # activations in pageable host memory
        xh = np.zeros((4, 256), np.uint16)
        L.ep_compressed_matvec_noalloc(small.h, xh.ctypes.data, 4, 0, ys.data_ptr(), stream_ptr())
    torch.cuda.synchronize()
