"""GPU tests of the fused prefill product (ep_compressed_linear_prefill): y = x W^T + b for
1..256 activation rows and 4096 or 8192 columns, with each K slab of W decoded into an LDS
operand tile of an MFMA product, against the float64 oracle product of the oracle's
decoded weights.

The weights the product uses are the BF16 container values (bit-exact against the oracle
in the decode tests); only the fp32 accumulation order differs from the oracle's exact
sum.  Bound per output element: half a BF16 ulp of the result (<= 2^-8 |y|) plus the fp32
summation error, far below 2^-14 sum_i |x_i w_i| for 4096 or 8192 products.  A slab written to
the wrong rows or columns, a dropped group of 8 weights or a wrong activation row moves
an output by about 8/4096 of that sum or more, far outside the bound."""
import numpy as np
import pytest

import synth
import oracle
from oracle import numerics as nx
from oracle.gemm import linear_ref

pytestmark = pytest.mark.gpu

from gpu_util import DevBlob, say, stream_ptr  # noqa: E402

C = 4096


def _t(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).view(dtype).cuda()


def _bits(y):
    import torch
    return y.cpu().view(torch.int16).numpy().view(np.uint16)


def _check(got_bits, x, w_hat, bias):
    xf, wf = nx.bf16_to_f64(x), nx.bf16_to_f64(w_hat)
    ref = linear_ref(xf, wf, nx.bf16_to_f64(bias) if bias is not None else None)
    mag = np.abs(xf) @ np.abs(wf).T
    got = nx.bf16_to_f64(got_bits)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * mag + 1e-30
    bad = np.argwhere(~(err <= bound))
    assert bad.size == 0, f"{len(bad)} outputs off, first {bad[0]}: got {got[tuple(bad[0])]} ref {ref[tuple(bad[0])]}"


def _run(blob, T, seed, with_bias, x_log2=0):
    import torch
    from decode_tile_rans_amd import _lib as L
    _, w_hat, _ = oracle.decode(blob)
    R, C = w_hat.shape
    x = synth.activations(T, C, seed + 1)
    if x_log2:   # (scaled by a power of two: exact in BF16)
        x = synth.f32_to_bf16_bits((nx.bf16_to_f64(x) * 2.0 ** x_log2).astype(np.float32))
    bias = synth.f32_to_bf16_bits(np.linspace(-0.5, 0.5, R).astype(np.float32)) if with_bias else None
    db = DevBlob(blob)
    xt = _t(x, torch.bfloat16)
    bt = _t(bias, torch.bfloat16) if bias is not None else None
    y = torch.full((T, R), 7.0, dtype=torch.bfloat16, device="cuda")
    L.ep_compressed_linear_prefill(db.h, xt.data_ptr(), T, bt.data_ptr() if bt is not None else 0, y.data_ptr(),
                                   stream_ptr())
    torch.cuda.synchronize()
    _check(_bits(y), x, w_hat, bias)
    assert db.errors() == 0
    return db, xt, y


# (rows, T, target bpp, seed): one workgroup (64 rows), rows not a multiple of 8 (a
# block with chains past the matrix) or of 64 (a workgroup with waves past the matrix),
# activation rows 1..256 on both kernel variants (<= 128 and <= 256 rows), ragged
# 16-row blocks; narrow tables at 2.3 / 3 / 4 bpp, wide tables at 5 bpp, escapes at 8
CASES = [
    (64, 1, 4.0, 201),
    (64, 16, 4.0, 202),
    (130, 9, 3.0, 203),
    (200, 100, 4.0, 204),
    (72, 128, 2.3, 205),
    (136, 129, 4.0, 206),
    (257, 200, 5.0, 207),
    (128, 256, 4.0, 208),
    (96, 77, 8.0, 209),
]


@pytest.mark.parametrize("R,T,bpp,seed", CASES)
def test_prefill_matches_oracle(R, T, bpp, seed):
    say("prefill", R, T, bpp, seed)
    blob = oracle.compress(synth.rowscaled(R, C, seed), nx.DT_BF16, bpp, chains_per_tile=8)
    b = oracle.parse_blob(blob)
    if bpp >= 8:
        assert b.flags & 1    # escape symbols exercised
    _run(blob, T, seed, seed % 2 == 1)


# 8192 columns (two tiles a row: 32 rows of W a workgroup, two K segments a slab)
CASES_8192 = [
    (32, 16, 4.0, 221),
    (100, 128, 4.0, 222),
    (70, 129, 3.0, 223),
    (40, 256, 5.0, 224),
    (36, 50, 8.0, 225),
]


@pytest.mark.parametrize("R,T,bpp,seed", CASES_8192)
def test_prefill_8192_columns(R, T, bpp, seed):
    say("prefill 8192", R, T, bpp, seed)
    blob = oracle.compress(synth.rowscaled(R, 2 * C, seed), nx.DT_BF16, bpp, chains_per_tile=8)
    _run(blob, T, seed, seed % 2 == 1)


@pytest.mark.parametrize("T", [3, 160])
def test_prefill_narrow_escapes(T):
    # escape symbols with narrow tables (outliers in rows the rate search does not sample)
    say("prefill narrow escapes", T)
    blob = oracle.compress(synth.rowscaled_row_outliers(256, C, 92), nx.DT_BF16, 4.0, chains_per_tile=8)
    b = oracle.parse_blob(blob)
    assert b.k <= 5 and (b.flags & 1), (b.k, b.flags)
    _run(blob, T, 92, True)


def test_prefill_saturating_blob():
    # a BF16 blob some of whose reconstructions overflow BF16 (the container saturates)
    # (activations scaled by 2^-100 keep the products finite)
    say("prefill saturating")
    w = np.clip(synth.rowscaled_f32(64, C, 93) * np.float32(1e38 / 0.02), -3.3e38, 3.3e38).astype(np.float32)
    blob = oracle.compress(synth.f32_to_bf16_bits(w), nx.DT_BF16, 1.0, chains_per_tile=8)
    assert oracle.parse_blob(blob).flags & 2
    _run(blob, 20, 93, False, x_log2=-100)


def test_prefill_against_decode_then_gemm_and_linear_entry():
    # the same layer decoded to memory and multiplied by the GEMM: equal within two
    # bounds; and ep_compressed_linear_forward takes the fused product here (same bits)
    import torch
    from decode_tile_rans_amd import _lib as L
    say("prefill vs decode then GEMM")
    blob = oracle.compress(synth.rowscaled(192, C, 210), nx.DT_BF16, 4.0, chains_per_tile=8)
    db, xt, y = _run(blob, 64, 210, False)
    wd = db.decode()
    wt = torch.from_numpy(np.ascontiguousarray(wd)).view(torch.bfloat16).cuda()
    y2 = torch.empty_like(y)
    L.ep_gemm_bf16_nt(xt.data_ptr(), wt.data_ptr(), 0, y2.data_ptr(), 64, 192, C, stream_ptr())
    need = L.ep_linear_workspace_bytes(db.h)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y3 = torch.empty_like(y)
    L.ep_compressed_linear_forward(db.h, xt.data_ptr(), 64, 0, y3.data_ptr(), ws.data_ptr(), need, stream_ptr())
    torch.cuda.synchronize()
    a, b2 = y.float(), y2.float()
    assert torch.all((a - b2).abs() <= 2.0 ** -7 * torch.maximum(a.abs(), b2.abs()) + 1e-3)
    assert torch.equal(y.view(torch.int16), y3.view(torch.int16))


def test_prefill_refusals():
    import torch
    from decode_tile_rans_amd import _lib as L
    say("prefill refusals")
    db = DevBlob(oracle.compress(synth.rowscaled(64, C, 211), nx.DT_BF16, 4.0, chains_per_tile=8))
    x = torch.zeros((257, C), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((257, 64), dtype=torch.bfloat16, device="cuda")
    for T in (0, 257):
        with pytest.raises(L.EPError):
            L.ep_compressed_linear_prefill(db.h, x.data_ptr(), T, 0, y.data_ptr(), stream_ptr())
    with pytest.raises(L.EPError):   # activations not 16-byte aligned
        L.ep_compressed_linear_prefill(db.h, x.data_ptr() + 2, 8, 0, y.data_ptr(), stream_ptr())
    with pytest.raises(L.EPError):   # output not 8-byte aligned
        L.ep_compressed_linear_prefill(db.h, x.data_ptr(), 8, 0, y.data_ptr() + 2, stream_ptr())
    with pytest.raises(L.EPError):   # activations in pageable host memory
        xh = np.zeros((8, C), np.uint16)
        L.ep_compressed_linear_prefill(db.h, xh.ctypes.data, 8, 0, y.data_ptr(), stream_ptr())
    # other widths, chains per tile other than 8, FP16 blobs: not taken
    for b in (oracle.compress(synth.rowscaled(64, 2048, 212), nx.DT_BF16, 4.0, chains_per_tile=8),
              oracle.compress(synth.rowscaled(16, 3 * C, 212), nx.DT_BF16, 4.0, chains_per_tile=8),
              oracle.compress(synth.rowscaled(64, C, 212), nx.DT_BF16, 4.0, chains_per_tile=4),
              oracle.compress((np.random.default_rng(9).standard_normal((64, C)) * 0.02).astype(np.float16)
                              .view(np.uint16), nx.DT_FP16, 4.0, chains_per_tile=8)):
        d = DevBlob(b)
        with pytest.raises(L.EPError):
            L.ep_compressed_linear_prefill(d.h, x.data_ptr(), 8, 0, y.data_ptr(), stream_ptr())
    torch.cuda.synchronize()
