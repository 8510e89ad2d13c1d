"""GPU tests of the MFMA GEMMs and the compressed linear layer against the
float64 oracle GEMM (relative L2 <= 1e-2, the bound BF16 outputs allow)."""
import numpy as np
import pytest

import synth
import oracle
from oracle import numerics as nx
from oracle.gemm import linear_ref, linear_fp8_ref, rel_l2

pytestmark = pytest.mark.gpu

from gpu_util import DevBlob, say, stream_ptr  # noqa: E402

TOL = 1e-2


def _t(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).view(dtype).cuda()


# (2048, 9000, 256): 288 tiles of 256 x 256, more than one round of the CUs, so the
# columns of the whole round take 256-wide tiles and the ragged rest 128-wide ones
@pytest.mark.parametrize("T,N,K", [(128, 128, 64), (256, 384, 512), (100, 200, 72), (1, 1, 8), (300, 129, 1032),
                                   (1024, 1024, 4096), (2048, 9000, 256)])
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
    ref = linear_ref(nx.bf16_to_f64(x), nx.bf16_to_f64(w), nx.bf16_to_f64(bias))
    got = nx.bf16_to_f64(y.cpu().view(torch.int16).numpy().view(np.uint16))
    assert rel_l2(got, ref) <= TOL


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
    ref = linear_fp8_ref(nx.fp8_e4m3fn_to_f64(xq), nx.fp8_e4m3fn_to_f64(wq), a_x, aw)
    got = nx.bf16_to_f64(y.cpu().view(torch.int16).numpy().view(np.uint16))
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
    ref = linear_ref(nx.bf16_to_f64(x), nx.bf16_to_f64(w_hat), nx.bf16_to_f64(bias))
    got = nx.bf16_to_f64(y.cpu().view(torch.int16).numpy().view(np.uint16))
    assert rel_l2(got, ref) <= TOL
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
    ref = linear_ref(x.float().cpu().numpy().astype(np.float64), nx.bf16_to_f64(w_hat),
                     lin.bias.detach().float().cpu().numpy())
    assert rel_l2(y.float().cpu().numpy(), ref) <= TOL
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


def test_compressed_linear_sequence_overlapped():
    """Layers run with the next layer's decode on a second stream: every output is
    bit-identical to the one-layer path and within tolerance of the oracle GEMM."""
    import torch
    from decode_tile_rans_amd import _lib as L
    shapes = [(512, 768), (768, 512), (1024, 768), (768, 1024), (512, 768)]   # (rows = out, cols = in)
    T = 200
    dbs, xs, ys, refs, bs = [], [], [], [], []
    for i, (R, C) in enumerate(shapes):
        blob = oracle.compress(synth.rowscaled(R, C, 40 + i), nx.DT_BF16, 3.0 + 0.5 * i)
        _, w_hat, _ = oracle.decode(blob)
        x = synth.activations(T, C, 60 + i)
        b = synth.f32_to_bf16_bits(np.linspace(-0.25, 0.25, R).astype(np.float32)) if i % 2 == 0 else None
        dbs.append(DevBlob(blob))
        xs.append(_t(x, torch.bfloat16))
        bs.append(_t(b, torch.bfloat16) if b is not None else None)
        ys.append(torch.empty((T, R), dtype=torch.bfloat16, device="cuda"))
        refs.append(linear_ref(nx.bf16_to_f64(x), nx.bf16_to_f64(w_hat), nx.bf16_to_f64(b) if b is not None else None))
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
            assert rel_l2(got, ref) <= TOL
    for db in dbs:
        assert db.errors() == 0
