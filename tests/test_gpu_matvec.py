"""GPU tests of the fused decode-and-product path (ep_compressed_matvec): y = x W^T + b
for 1..8 activation rows with W decoded inside the product, against the float64 oracle
product of the oracle's decoded weights.

Bound per output element: the BF16 rounding of the result (half an ulp, <= 2^-8 |y|)
plus the fp32 summation error of the partial sums, which stays far below
2^-14 sum_i |x_i w_i| for rows of <= 4096 products (about C 2^-24 of it).  A group of
eight weights dropped or taken from the wrong row or column moves an output by about
8/C of that sum, far outside the bound for these shapes."""
import numpy as np
import pytest

import synth
import oracle
from oracle import numerics as nx
from oracle.gemm import linear_ref

pytestmark = pytest.mark.gpu

from gpu_util import DevBlob, say, stream_ptr  # noqa: E402


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
    bad = np.argwhere(~(err <= bound))   # a NaN anywhere fails
    assert bad.size == 0, f"{len(bad)} outputs off, first {bad[0]}: got {got[tuple(bad[0])]} ref {ref[tuple(bad[0])]}"


# (rows, cols, T, target bpp, chains per tile S, seed): groups per row G = cols / 8
# against the tile's 512 groups: many rows per tile (G 32, 9, 8), rows across tiles
# (480, 129), one row per tile (512); chains of a tile switching rows at different steps
# (G not a multiple of S); ragged last tiles; escapes at 8 bpp; 1..8 activation rows
CASES = [
    (384, 256, 1, 4.0, 8, 101),
    (300, 3840, 3, 4.0, 8, 102),
    (64, 4096, 8, 3.0, 8, 103),
    (130, 1032, 5, 2.3, 8, 104),
    (200, 512, 2, 8.0, 8, 105),
    (1000, 64, 4, 4.0, 8, 106),
    (1000, 64, 4, 4.0, 1, 106),
    (37, 72, 7, 4.0, 8, 107),
    (96, 2048, 6, 5.0, 4, 108),
    (250, 1000, 8, 3.5, 2, 109),
    (300, 3840, 3, 4.0, 16, 110),
    (130, 1032, 5, 2.3, 16, 111),
    (96, 2048, 1, 8.0, 16, 112),
]


@pytest.mark.parametrize("R,C,T,bpp,S,seed", CASES)
def test_matvec_matches_oracle(R, C, T, bpp, S, seed):
    import torch
    from decode_tile_rans_amd import _lib as L
    say("matvec", R, C, T, bpp, S, seed)
    src = synth.rowscaled(R, C, seed)
    blob = oracle.compress(src, nx.DT_BF16, bpp, chains_per_tile=S)
    _, w_hat, _ = oracle.decode(blob)
    x = synth.activations(T, C, seed + 1)
    bias = synth.f32_to_bf16_bits(np.linspace(-0.5, 0.5, R).astype(np.float32)) if seed % 2 else None
    db = DevBlob(blob)
    xt = _t(x, torch.bfloat16)
    bt = _t(bias, torch.bfloat16) if bias is not None else None
    bp = bt.data_ptr() if bt is not None else 0
    need = L.ep_matvec_workspace_bytes(db.h, T)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y = torch.full((T, R), 7.0, dtype=torch.bfloat16, device="cuda")
    L.ep_compressed_matvec(db.h, xt.data_ptr(), T, bp, y.data_ptr(), ws.data_ptr(), need, stream_ptr())
    torch.cuda.synchronize()
    first = _bits(y)
    _check(first, x, w_hat, bias)
    # a second call (workspace holding the first call's partial sums) gives the same bits
    ws.fill_(0xFF)
    L.ep_compressed_matvec(db.h, xt.data_ptr(), T, bp, y.data_ptr(), ws.data_ptr(), need, stream_ptr())
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), first)
    # the linear layer entry takes the fused path when its partial sums fit its workspace
    # (5-8 rows of whole-tile rows: the fused prefill product), else decodes and runs the
    # GEMM (same result within the bound)
    n1 = L.ep_linear_workspace_bytes(db.h)
    w1 = torch.empty(n1, dtype=torch.uint8, device="cuda")
    y1 = torch.empty_like(y)
    L.ep_compressed_linear_forward(db.h, xt.data_ptr(), T, bp, y1.data_ptr(), w1.data_ptr(), n1, stream_ptr())
    torch.cuda.synchronize()
    prefill = T > 4 and S == 8 and C in (4096, 8192)
    if need <= n1 and not prefill:
        assert np.array_equal(_bits(y1), first)
    else:
        _check(_bits(y1), x, w_hat, bias)
    assert db.errors() == 0


@pytest.mark.parametrize("T,t", [(1, 3.0), (5, 4.0)])
def test_matvec_narrow_escapes(T, t):
    # the fused product on a blob with escape symbols and a small escape threshold (the
    # outliers sit in rows the rate search does not sample)
    import torch
    from decode_tile_rans_amd import _lib as L
    say("matvec narrow escapes", T, t)
    src = synth.rowscaled_row_outliers(1024, 1024, 91)
    blob = oracle.compress(src, nx.DT_BF16, t)
    b = oracle.parse_blob(blob)
    assert b.k <= 5 and (b.flags & 1), (b.k, b.flags)
    _, w_hat, _ = oracle.decode(blob)
    x = synth.activations(T, 1024, 77)
    db = DevBlob(blob)
    xt = _t(x, torch.bfloat16)
    need = L.ep_matvec_workspace_bytes(db.h, T)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y = torch.empty((T, 1024), dtype=torch.bfloat16, device="cuda")
    L.ep_compressed_matvec(db.h, xt.data_ptr(), T, 0, y.data_ptr(), ws.data_ptr(), need, stream_ptr())
    torch.cuda.synchronize()
    _check(_bits(y), x, w_hat, None)
    assert db.errors() == 0


def test_matvec_python_layer_small_batch():
    """CompressedLinear on 1..8 tokens goes through the fused path; result against the
    oracle product of the oracle's decode of the layer's own blob."""
    import torch
    import decode_tile_rans_amd as ep
    say("matvec python layer")
    torch.manual_seed(1)
    lin = torch.nn.Linear(1024, 640, dtype=torch.bfloat16, device="cuda")
    layer = ep.CompressedLinear.from_linear(lin, target_bpp=4.0)
    blob = layer._c.to_bytes()
    _, w_hat, _ = oracle.decode(blob)
    b_bits = lin.bias.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    for T in (1, 4, 8):
        x = torch.randn(T, 1024, dtype=torch.bfloat16, device="cuda")
        with torch.inference_mode():
            y = layer(x)
        assert y.shape == (T, 640)
        _check(_bits(y), x.cpu().view(torch.int16).numpy().view(np.uint16), w_hat, b_bits)


def test_matvec_sequence_matches_one_layer_path():
    """The layer sequence with 4 activation rows: fused layers and decode-then-GEMM
    layers (rows too short for the fused path's workspace) mixed; every output equals the
    one-layer entry's bits."""
    import torch
    from decode_tile_rans_amd import _lib as L
    shapes = [(512, 768), (256, 64), (640, 512), (384, 1024)]
    T = 4
    dbs, xs, ys, bs = [], [], [], []
    for i, (R, C) in enumerate(shapes):
        blob = oracle.compress(synth.rowscaled(R, C, 70 + i), nx.DT_BF16, 3.0 + 0.5 * i, chains_per_tile=8)
        dbs.append(DevBlob(blob))
        xs.append(_t(synth.activations(T, C, 80 + i), torch.bfloat16))
        b = synth.f32_to_bf16_bits(np.linspace(-0.25, 0.25, R).astype(np.float32)) if i % 2 == 0 else None
        bs.append(_t(b, torch.bfloat16) if b is not None else None)
        ys.append(torch.empty((T, R), dtype=torch.bfloat16, device="cuda"))
    hs = [d.h for d in dbs]
    # the 64-column layer's partial sums do not fit its linear workspace: GEMM path
    assert L.ep_matvec_workspace_bytes(hs[1], T) > L.ep_linear_workspace_bytes(hs[1])
    need = L.ep_linear_seq_workspace_bytes(hs)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    say("matvec sequence", len(shapes), T)
    L.ep_compressed_linear_seq_forward(hs, [x.data_ptr() for x in xs], T, [b.data_ptr() if b is not None else 0 for b in bs],
                                       [y.data_ptr() for y in ys], ws.data_ptr(), need, stream_ptr(), int(side.cuda_stream))
    torch.cuda.synchronize()
    for i, (db, x, b, y) in enumerate(zip(dbs, xs, bs, ys)):
        one = torch.empty_like(y)
        n1 = L.ep_linear_workspace_bytes(db.h)
        w1 = torch.empty(n1, dtype=torch.uint8, device="cuda")
        L.ep_compressed_linear_forward(db.h, x.data_ptr(), T, b.data_ptr() if b is not None else 0, one.data_ptr(),
                                       w1.data_ptr(), n1, stream_ptr())
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), one.view(torch.int16)), f"layer {i} differs from the one-layer path"


def test_matvec_refusals():
    import torch
    from decode_tile_rans_amd import _lib as L
    say("matvec refusals")
    blob = oracle.compress(synth.rowscaled(64, 256, 9), nx.DT_BF16, 4.0)
    db = DevBlob(blob)
    x = torch.zeros((9, 256), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((9, 64), dtype=torch.bfloat16, device="cuda")
    need = L.ep_matvec_workspace_bytes(db.h, 8)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    assert L.ep_matvec_workspace_bytes(db.h, 0) == 0 and L.ep_matvec_workspace_bytes(db.h, 9) == 0
    for T in (0, 9):
        with pytest.raises(L.EPError):
            L.ep_compressed_matvec(db.h, x.data_ptr(), T, 0, y.data_ptr(), ws.data_ptr(), need, stream_ptr())
    with pytest.raises(L.EPError):   # workspace too small
        L.ep_compressed_matvec(db.h, x.data_ptr(), 8, 0, y.data_ptr(), ws.data_ptr(), need - 1, stream_ptr())
    with pytest.raises(L.EPError):   # activations not 16-byte aligned
        L.ep_compressed_matvec(db.h, x.data_ptr() + 2, 8, 0, y.data_ptr(), ws.data_ptr(), need, stream_ptr())
    with pytest.raises(L.EPError):   # activations in pageable host memory
        xh = np.zeros((8, 256), np.uint16)
        L.ep_compressed_matvec(db.h, xh.ctypes.data, 8, 0, y.data_ptr(), ws.data_ptr(), need, stream_ptr())
    # rows of a width that is not a multiple of 8, rows of fewer groups than chains per
    # tile (16 columns = 2 groups at S = 8), FP16 blobs: not taken
    for b in (oracle.compress(synth.rowscaled(64, 100, 9), nx.DT_BF16, 4.0),
              oracle.compress(synth.rowscaled(64, 16, 9), nx.DT_BF16, 4.0, chains_per_tile=8),
              oracle.compress((np.random.default_rng(9).standard_normal((64, 256)) * 0.02).astype(np.float16)
                              .view(np.uint16), nx.DT_FP16, 4.0)):
        d = DevBlob(b)
        assert L.ep_matvec_workspace_bytes(d.h, 4) == 0
        with pytest.raises(L.EPError):
            L.ep_compressed_matvec(d.h, x.data_ptr(), 4, 0, y.data_ptr(), ws.data_ptr(), need, stream_ptr())
    torch.cuda.synchronize()


def _single(L, db, x, T, bias):
    import torch
    need = L.ep_matvec_workspace_bytes(db.h, T)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y = torch.empty((T, db.R), dtype=torch.bfloat16, device="cuda")
    L.ep_compressed_matvec(db.h, x.data_ptr(), T, bias.data_ptr() if bias is not None else 0, y.data_ptr(),
                           ws.data_ptr(), need, stream_ptr())
    return y


@pytest.mark.parametrize("specs,T,C", [
    # (rows, target bpp, chains per tile) sharing 768 columns: narrow and wide tables,
    # with and without escapes, several chain counts, in one call
    ([(384, 4.0, 8), (640, 8.0, 8), (200, 2.3, 1), (1000, 5.0, 4)], 3, 768),
    # more blobs than one launch takes
    ([(64 + 8 * i, 3.0 + 0.25 * (i % 4), 8) for i in range(14)], 1, 768),
    # rows of whole tiles (row sums in the decode kernel at 8 and 16 chains per tile)
    # beside a blob whose sums take the finishing kernel, in one call
    ([(96, 4.0, 8), (64, 4.0, 16), (40, 3.0, 4), (33, 5.0, 16)], 2, 4096),
])
def test_matvec_batch_equals_single_calls(specs, T, C):
    import torch
    from decode_tile_rans_amd import _lib as L
    say("matvec batch", len(specs), T, C)
    dbs, biases, blobs = [], [], []
    for i, (R, bpp, S) in enumerate(specs):
        blob = oracle.compress(synth.rowscaled(R, C, 200 + i), nx.DT_BF16, bpp, chains_per_tile=S)
        blobs.append(blob)
        dbs.append(DevBlob(blob))
        b = synth.f32_to_bf16_bits(np.linspace(-0.3, 0.3, R).astype(np.float32)) if i % 3 != 1 else None
        biases.append(_t(b, torch.bfloat16) if b is not None else None)
    x_bits = synth.activations(T, C, 300)
    x = _t(x_bits, torch.bfloat16)
    hs = [d.h for d in dbs]
    need = L.ep_matvec_batch_workspace_bytes(hs, T)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ys = [torch.empty((T, d.R), dtype=torch.bfloat16, device="cuda") for d in dbs]
    bp = [b.data_ptr() if b is not None else 0 for b in biases]
    with pytest.raises(L.EPError):
        L.ep_compressed_matvec_batch(hs, x.data_ptr(), T, bp, [y.data_ptr() for y in ys], ws.data_ptr(), need - 1,
                                     stream_ptr())
    L.ep_compressed_matvec_batch(hs, x.data_ptr(), T, bp, [y.data_ptr() for y in ys], ws.data_ptr(), need,
                                 stream_ptr())
    torch.cuda.synchronize()
    for i, (db, y, b) in enumerate(zip(dbs, ys, biases)):
        one = _single(L, db, x, T, b)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), one.view(torch.int16)), f"blob {i} differs from its single call"
    # one of them against the oracle product
    _, w_hat, _ = oracle.decode(blobs[1])
    _check(_bits(ys[1]), x_bits, w_hat, None if biases[1] is None else _bits(biases[1]))
    for db in dbs:
        assert db.errors() == 0


def test_matvec_batch_refuses_mixed_widths():
    import torch
    from decode_tile_rans_amd import _lib as L
    say("matvec batch refusals")
    a = DevBlob(oracle.compress(synth.rowscaled(64, 256, 1), nx.DT_BF16, 4.0))
    b = DevBlob(oracle.compress(synth.rowscaled(64, 512, 2), nx.DT_BF16, 4.0))
    x = torch.zeros((2, 512), dtype=torch.bfloat16, device="cuda")
    ys = [torch.empty((2, 64), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    need = L.ep_matvec_batch_workspace_bytes([a.h, b.h], 2)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.EPError):
        L.ep_compressed_matvec_batch([a.h, b.h], x.data_ptr(), 2, None, [y.data_ptr() for y in ys], ws.data_ptr(),
                                     need, stream_ptr())
    assert L.ep_matvec_batch_workspace_bytes([a.h, b.h], 9) == 0
    torch.cuda.synchronize()


def test_python_linear_batch_equals_layers():
    """ep.linear_batch over three layers sharing an input: the same bits as calling each
    layer, for 2 tokens (fused, one batched call) and for 20 (decode then GEMM)."""
    import torch
    import decode_tile_rans_amd as ep
    say("python linear_batch")
    torch.manual_seed(3)
    layers = [ep.CompressedLinear.from_linear(torch.nn.Linear(512, r, dtype=torch.bfloat16, device="cuda"),
                                              target_bpp=4.0) for r in (256, 384, 128)]
    for T in (2, 20):
        x = torch.randn(T, 512, dtype=torch.bfloat16, device="cuda")
        with torch.inference_mode():
            got = ep.linear_batch(layers, x)
            want = [m(x) for m in layers]
        for g, w in zip(got, want):
            assert g.shape == w.shape and torch.equal(g.view(torch.int16), w.view(torch.int16))


def test_linear_falls_back_when_product_not_taken():
    """Rows shorter than S groups: the linear entry decodes and runs the GEMM instead."""
    import torch
    from decode_tile_rans_amd import _lib as L
    say("matvec fallback")
    R, C, T = 200, 16, 3
    blob = oracle.compress(synth.rowscaled(R, C, 11), nx.DT_BF16, 4.0, chains_per_tile=8)
    _, w_hat, _ = oracle.decode(blob)
    db = DevBlob(blob)
    assert L.ep_matvec_workspace_bytes(db.h, T) == 0
    x = synth.activations(T, C, 12)
    xt = _t(x, torch.bfloat16)
    y = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
    need = L.ep_linear_workspace_bytes(db.h)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    L.ep_compressed_linear_forward(db.h, xt.data_ptr(), T, 0, y.data_ptr(), ws.data_ptr(), need, stream_ptr())
    torch.cuda.synchronize()
    _check(_bits(y), x, w_hat, None)


@pytest.mark.parametrize("R,C,T,S", [(200, 4096, 1, 8), (130, 4096, 3, 8), (96, 8192, 8, 8), (40, 8192, 5, 8),
                                     (200, 4096, 1, 16), (70, 4096, 4, 16), (96, 8192, 2, 16), (33, 8192, 7, 16)])
def test_matvec_rows_of_whole_tiles_summed_in_kernel(R, C, T, S, monkeypatch):
    """Rows of whole tiles (4096 / 8192 columns at S = 8 or 16): the decode kernel adds a row's
    chain sums itself, in the finishing kernel's order, so the output equals the
    two-kernel path bit for bit and stays within the oracle bound."""
    import torch
    from decode_tile_rans_amd import _lib as L
    say("matvec in-kernel sums", R, C, T, S)
    blob = oracle.compress(synth.rowscaled(R, C, 120 + T), nx.DT_BF16, 4.0, chains_per_tile=S)
    _, w_hat, _ = oracle.decode(blob)
    x = synth.activations(T, C, 121)
    bias = synth.f32_to_bf16_bits(np.linspace(-0.5, 0.5, R).astype(np.float32))
    db = DevBlob(blob)
    xt, bt = _t(x, torch.bfloat16), _t(bias, torch.bfloat16)
    need = L.ep_matvec_workspace_bytes(db.h, T)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ys = []
    for flag in ("1", "0"):
        monkeypatch.setenv("EP_MATVEC_DIRECT", flag)
        y = torch.full((T, R), 7.0, dtype=torch.bfloat16, device="cuda")
        L.ep_compressed_matvec(db.h, xt.data_ptr(), T, bt.data_ptr(), y.data_ptr(), ws.data_ptr(), need, stream_ptr())
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16))
    _check(_bits(ys[0]), x, w_hat, bias)
    assert db.errors() == 0
