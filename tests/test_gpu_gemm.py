"""GPU tests of the MFMA GEMMs and the compressed linear layer against the
float64 oracle GEMM: every output within the per-element bound of an fp32-accumulated
BF16-out product (gpu_util.linear_bound), which a wrong tile, row or K-slice exceeds by
far; the layer outputs also within 1e-2 relative L2 (the pages' bar)."""
import numpy as np
import pytest

import synth
import oracle
from oracle import numerics as nx
from oracle.gemm import linear_ref, linear_fp8_ref, rel_l2

pytestmark = pytest.mark.gpu

from gpu_util import DevBlob, check_linear, say, stream_ptr  # noqa: E402

TOL = 1e-2


def _t(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).view(dtype).cuda()


# Small shapes and (2048, 9000, 256) take 128-wide tiles (they fill the CUs' rounds
# better).  The four-wave 256 x 256 kernel (K % 64 == 0): (2000, 8001, 320) ragged rows
# and an odd column count (element stores), five K tiles; (2048, 8192, 64) one K tile;
# (1800, 7000, 4096); (3300, 10000, 192) 256-wide tiles over the columns of the whole
# rounds and 128-wide ones over the rest.  (3328, 10000, 136): the same split with the
# eight-wave 256-wide kernel (K % 64 != 0, a partial last K tile).
@pytest.mark.parametrize("T,N,K", [(128, 128, 64), (256, 384, 512), (100, 200, 72), (1, 1, 8), (300, 129, 1032),
                                   (1024, 1024, 4096), (2048, 9000, 256), (2000, 8001, 320), (2048, 8192, 64),
                                   (1800, 7000, 4096), (3300, 10000, 192), (3328, 10000, 136)])
def test_gemm_bf16(T, N, K):
    import torch
    from decode_tile_rans_amd import _lib as L
    say("gemm bf16", T, N, K)
    x = synth.activations(T, K, 1)
    w = synth.rowscaled(N, K, 2)
    bias = synth.f32_to_bf16_bits(np.linspace(-1, 1, N).astype(np.float32))
    xt, wt, bt = _t(x, torch.bfloat16), _t(w, torch.bfloat16), _t(bias, torch.bfloat16)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    L.ep_gemm_bf16_nt(xt.data_ptr(), wt.data_ptr(), bt.data_ptr(), y.data_ptr(), T, N, K, stream_ptr())
    torch.cuda.synchronize()
    xf, wf, bf = nx.bf16_to_f64(x), nx.bf16_to_f64(w), nx.bf16_to_f64(bias)
    ref = linear_ref(xf, wf, bf)
    mag = linear_ref(np.abs(xf), np.abs(wf), np.abs(bf))
    got = nx.bf16_to_f64(y.cpu().view(torch.int16).numpy().view(np.uint16))
    check_linear(got, ref, mag, K)
    assert rel_l2(got, ref) <= TOL


@pytest.mark.parametrize("bias_offset", [0, 1, None], ids=["bias", "unaligned-bias", "no-bias"])
def test_gemm_bf16_kernels_agree(bias_offset, monkeypatch):
    """The four-wave and the eight-wave 256-wide kernels accumulate every output in the
    same K order, so they give the same bits; a bias pointer off its 8-byte alignment
    takes the element-wise bias reads."""
    import torch
    from decode_tile_rans_amd import _lib as L
    T, N, K = 2000, 8192, 576
    say("gemm bf16 kernels agree", T, N, K, bias_offset)
    xt = _t(synth.activations(T, K, 5), torch.bfloat16)
    wt = _t(synth.rowscaled(N, K, 6), torch.bfloat16)
    braw = _t(synth.f32_to_bf16_bits(np.linspace(-2, 2, N + 1).astype(np.float32)), torch.bfloat16)
    bp = None if bias_offset is None else braw.data_ptr() + 2 * bias_offset
    ys = []
    for flag in ("0", "1"):
        monkeypatch.setenv("EP_GEMM_W4", flag)
        y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        L.ep_gemm_bf16_nt(xt.data_ptr(), wt.data_ptr(), bp, y.data_ptr(), T, N, K, stream_ptr())
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16))


@pytest.mark.parametrize("T,N,K", [(128, 128, 128), (256, 384, 512), (100, 200, 144), (512, 1024, 2048), (2048, 9000, 256)])
def test_gemm_fp8(T, N, K):
    import torch
    from decode_tile_rans_amd import _lib as L
    say("gemm fp8", T, N, K)
    wq, aw = synth.fp8_codes(N, K, 3)
    xq, ax_rows = synth.fp8_codes(T, K, 4)
    a_x = float(ax_rows.max())
    xt, wt = _t(xq, torch.uint8), _t(wq, torch.uint8)
    awt = torch.from_numpy(aw).cuda()
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    L.ep_gemm_fp8_nt(xt.data_ptr(), wt.data_ptr(), a_x, awt.data_ptr(), y.data_ptr(), T, N, K, stream_ptr())
    torch.cuda.synchronize()
    xf, wf = nx.fp8_e4m3fn_to_f64(xq), nx.fp8_e4m3fn_to_f64(wq)
    ref = linear_fp8_ref(xf, wf, a_x, aw)
    mag = linear_fp8_ref(np.abs(xf), np.abs(wf), a_x, aw)
    got = nx.bf16_to_f64(y.cpu().view(torch.int16).numpy().view(np.uint16))
    check_linear(got, ref, mag, K, scale_roundings=2)
    assert rel_l2(got, ref) <= TOL


def test_compressed_linear_forward():
    import torch
    from decode_tile_rans_amd import _lib as L
    R, C, T = 1024, 768, 300
    src = synth.rowscaled(R, C, 21)
    blob = oracle.compress(src, nx.DT_BF16, 4.0)
    _, w_hat, _ = oracle.decode(blob)
    x = synth.activations(T, C, 22)
    bias = synth.f32_to_bf16_bits(np.linspace(-0.5, 0.5, R).astype(np.float32))
    db = DevBlob(blob)
    xt, bt = _t(x, torch.bfloat16), _t(bias, torch.bfloat16)
    y = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
    need = L.ep_linear_workspace_bytes(db.h)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    say("compressed linear", R, C, T)
    with pytest.raises(L.EPError):
        L.ep_compressed_linear_forward(db.h, xt.data_ptr(), T, bt.data_ptr(), y.data_ptr(), ws.data_ptr(), need - 1,
                                       stream_ptr())
    L.ep_compressed_linear_forward(db.h, xt.data_ptr(), T, bt.data_ptr(), y.data_ptr(), ws.data_ptr(), need,
                                   stream_ptr())
    torch.cuda.synchronize()
    xf, wf, bf = nx.bf16_to_f64(x), nx.bf16_to_f64(w_hat), nx.bf16_to_f64(bias)
    ref = linear_ref(xf, wf, bf)
    got = nx.bf16_to_f64(y.cpu().view(torch.int16).numpy().view(np.uint16))
    check_linear(got, ref, linear_ref(np.abs(xf), np.abs(wf), np.abs(bf)), C)
    assert rel_l2(got, ref) <= TOL
    assert db.errors() == 0


def test_linear_and_gemm_refuse_host_memory():
    """Pageable host pointers are refused before any launch, for every token count."""
    import torch
    from decode_tile_rans_amd import _lib as L
    say("host-memory refusals")
    R, C = 256, 512
    db = DevBlob(oracle.compress(synth.rowscaled(R, C, 23), nx.DT_BF16, 4.0))
    need = L.ep_linear_workspace_bytes(db.h)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for T in (4, 64):
        xd = torch.zeros((T, C), dtype=torch.bfloat16, device="cuda")
        yd = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
        xh = np.zeros((T, C), np.uint16)
        yh = np.zeros((T, R), np.uint16)
        bh = np.zeros(R, np.uint16)
        wsh = np.zeros(need, np.uint8)
        for args in ((xh.ctypes.data, 0, yd.data_ptr(), ws.data_ptr()),
                     (xd.data_ptr(), 0, yh.ctypes.data, ws.data_ptr()),
                     (xd.data_ptr(), bh.ctypes.data, yd.data_ptr(), ws.data_ptr()),
                     (xd.data_ptr(), 0, yd.data_ptr(), wsh.ctypes.data)):
            x_, b_, y_, w_ = args
            with pytest.raises(L.EPError):
                L.ep_compressed_linear_forward(db.h, x_, T, b_, y_, w_, need, stream_ptr())
    T, N, K = 64, 128, 256
    xd = torch.zeros((T, K), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    yd = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    host = np.zeros((N, K), np.uint16)
    with pytest.raises(L.EPError):
        L.ep_gemm_bf16_nt(xd.data_ptr(), host.ctypes.data, None, yd.data_ptr(), T, N, K, stream_ptr())
    with pytest.raises(L.EPError):
        L.ep_gemm_bf16_nt(host.ctypes.data, wd.data_ptr(), None, yd.data_ptr(), T, N, K, stream_ptr())
    aw = np.ones(N, np.float32)
    with pytest.raises(L.EPError):
        L.ep_gemm_fp8_nt(xd.data_ptr(), wd.data_ptr(), 1.0, aw.ctypes.data, yd.data_ptr(), T, N, K, stream_ptr())
    torch.cuda.synchronize()
    assert db.errors() == 0


def test_python_api_module_and_state_dict():
    import torch
    import decode_tile_rans_amd as ep
    say("python api")
    torch.manual_seed(0)
    lin = torch.nn.Linear(512, 384, dtype=torch.bfloat16, device="cuda")
    layer = ep.CompressedLinear.from_linear(lin, target_bpp=4.0)
    assert 4.0 <= layer.compressed_bits <= 4.1
    x = torch.randn(8, 512, dtype=torch.bfloat16, device="cuda")
    with torch.inference_mode():
        y = layer(x)
    assert y.shape == (8, 384) and y.dtype == torch.bfloat16
    # the layer's blob is the oracle's blob of the same weight; reference output from the oracle
    w_bits = lin.weight.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    blob = oracle.compress(w_bits, nx.DT_BF16, 4.0)
    assert layer._c.to_bytes() == blob
    _, w_hat, _ = oracle.decode(blob)
    xf, wf = x.float().cpu().numpy().astype(np.float64), nx.bf16_to_f64(w_hat)
    bf = lin.bias.detach().float().cpu().numpy().astype(np.float64)
    ref = linear_ref(xf, wf, bf)
    got = y.float().cpu().numpy().astype(np.float64)
    check_linear(got, ref, linear_ref(np.abs(xf), np.abs(wf), np.abs(bf)), 512)
    assert rel_l2(got, ref) <= TOL
    sd = layer.state_dict()
    layer2 = ep.CompressedLinear(ep.Compressed.from_bytes(blob), torch.zeros(384, dtype=torch.bfloat16, device="cuda"))
    layer2.load_state_dict(sd)
    with torch.inference_mode():
        y2 = layer2(x)
    assert torch.equal(y, y2)
    # compress / decompress round trip restores shape and dtype
    w = (torch.randn(256, 256, device="cuda") * 0.02).to(torch.bfloat16)
    c = ep.compress(w, 3.5)
    r = ep.decompress(c)
    assert r.shape == w.shape and r.dtype == w.dtype
    blob_w = oracle.compress(w.cpu().view(torch.int16).numpy().view(np.uint16), nx.DT_BF16, 3.5)
    assert c.to_bytes() == blob_w
    _, ref_w, _ = oracle.decode(blob_w)
    assert np.array_equal(r.cpu().view(torch.int16).numpy().view(np.uint16), ref_w)


# (T, [(rows = out, cols = in), ...]): at 200 tokens every GEMM leaves CUs idle, so every
# decode after the first runs on the side stream; at 4096 tokens the 4096-row layers'
# GEMMs take 256 tiles (one per CU) and the next decode runs in order on the main stream,
# while the 512-row layer's 32-tile GEMM lets the decode after it go to the side stream;
# at 200 tokens with S = 8 the 4096-column layers take the fused prefill product between
# decoded ones (chains per tile: None = the encoder's default)
SEQ_CASES = [
    (200, [(512, 768), (768, 512), (1024, 768), (768, 1024), (512, 768)], None),
    (4096, [(4096, 256), (512, 256), (4096, 256), (4096, 256)], None),
    (200, [(512, 4096), (4096, 512), (768, 512), (264, 4096), (512, 768)], 8),
]


@pytest.mark.parametrize("T,shapes,S", SEQ_CASES, ids=["side", "mixed", "prefill"])
def test_compressed_linear_sequence(T, shapes, S):
    """A sequence of layers: every output is bit-identical to the one-layer path and
    every element within the per-element bound of the oracle GEMM."""
    import torch
    from decode_tile_rans_amd import _lib as L
    dbs, xs, ys, refs, mags, bs = [], [], [], [], [], []
    for i, (R, C) in enumerate(shapes):
        blob = oracle.compress(synth.rowscaled(R, C, 40 + i), nx.DT_BF16, 3.0 + 0.5 * i, chains_per_tile=S)
        _, w_hat, _ = oracle.decode(blob)
        x = synth.activations(T, C, 60 + i)
        b = synth.f32_to_bf16_bits(np.linspace(-0.25, 0.25, R).astype(np.float32)) if i % 2 == 0 else None
        dbs.append(DevBlob(blob))
        xs.append(_t(x, torch.bfloat16))
        bs.append(_t(b, torch.bfloat16) if b is not None else None)
        ys.append(torch.empty((T, R), dtype=torch.bfloat16, device="cuda"))
        xf, wf = nx.bf16_to_f64(x), nx.bf16_to_f64(w_hat)
        bf = nx.bf16_to_f64(b) if b is not None else None
        refs.append(linear_ref(xf, wf, bf))
        mags.append(linear_ref(np.abs(xf), np.abs(wf), np.abs(bf) if bf is not None else None))
    hs = [d.h for d in dbs]
    need = L.ep_linear_seq_workspace_bytes(hs)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    say("linear sequence", len(shapes), T)
    with pytest.raises(L.EPError):
        L.ep_compressed_linear_seq_forward(hs, [x.data_ptr() for x in xs], T, [b.data_ptr() if b is not None else 0 for b in bs],
                                           [y.data_ptr() for y in ys], ws.data_ptr(), need - 1, stream_ptr(),
                                           int(side.cuda_stream))
    for rep in range(2):
        for y in ys:
            y.zero_()
        L.ep_compressed_linear_seq_forward(hs, [x.data_ptr() for x in xs], T, [b.data_ptr() if b is not None else 0 for b in bs],
                                           [y.data_ptr() for y in ys], ws.data_ptr(), need, stream_ptr(),
                                           int(side.cuda_stream))
        torch.cuda.synchronize()
        for i, (db, x, b, y, ref) in enumerate(zip(dbs, xs, bs, ys, refs)):
            one = torch.empty_like(y)
            n1 = L.ep_linear_workspace_bytes(db.h)
            w1 = torch.empty(n1, dtype=torch.uint8, device="cuda")
            L.ep_compressed_linear_forward(db.h, x.data_ptr(), T, b.data_ptr() if b is not None else 0, one.data_ptr(),
                                           w1.data_ptr(), n1, stream_ptr())
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), one.view(torch.int16)), f"layer {i} differs from the one-layer path"
            got = nx.bf16_to_f64(y.cpu().view(torch.int16).numpy().view(np.uint16))
            check_linear(got, ref, mags[i], shapes[i][1])
            assert rel_l2(got, ref) <= TOL
    for db in dbs:
        assert db.errors() == 0
