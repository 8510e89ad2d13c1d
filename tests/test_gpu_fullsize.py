"""Full-size GPU parity in the launch configurations the benchmark times.  Every
decoded element is compared with the oracle's decode of the same blob (the library's
host encoder writes the blob; its bytes equal the oracle encoder's, checked here for
one matrix of each shape and on the CPU for many more):

* DiT stack: all 9 matrices of the first transformer block, decoded by one batched
  launch on a side stream, and the 6 extra matrices in their own launch -- container
  bits and lattice coordinates of every element, every chain ending in L.
* Fused linear prefill (14336 x 4096 @ 4.0 bpp, 4096 tokens): the decoded weights in
  the layer's workspace bit for bit, then each output of 256 sampled token rows within
  the per-element bound of an fp32-accumulated product (a wrong weight row, tile or
  K-slice moves outputs far outside it).
* 8192^2 bitrate / container sweep (BF16 @2.3/3/5/8, FP8 @5, INT8 @4): every element
  and coordinate, tile subsets equal to the full decode, distortion at the high-rate
  prediction.
* The outlier recipe (3072^2, 0.1 % of entries at +-10 s_r) at 6 bpp, where the
  outliers are coded as escapes: every element and coordinate.
"""
import math

import numpy as np
import pytest

import synth
import oracle
from oracle import numerics as nx
from oracle.gemm import linear_fp8_ref, linear_ref

pytestmark = pytest.mark.gpu

from gpu_util import DevBlob, check_linear, say, stream_ptr, to_np  # noqa: E402

SQRT_G = math.sqrt(929 / 12960)


def _bits(t):
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _tile_mask(R, C, tiles):
    """Element mask of the columns-by-8 groups that the given tiles cover."""
    G = -(-C // 8)
    gm = np.zeros(R * G, dtype=bool)
    for t in tiles:
        gm[512 * t: 512 * (t + 1)] = True
    return np.repeat(gm, 8).reshape(R, G * 8)[:, :C]


def _product_blob(src, dt, t, S=0):
    from decode_tile_rans_amd import _lib as L
    src = np.ascontiguousarray(src)
    return L.ep_compress(src.ctypes.data, dt, src.shape[0], src.shape[1], t, S)


def _coords(h, R, C):
    import torch
    from decode_tile_rans_amd import _lib as L
    u = torch.zeros((R, C), dtype=torch.int32, device="cuda")
    L.ep_test_decode_coords(h, u.data_ptr(), stream_ptr())
    torch.cuda.synchronize()
    return u.cpu().numpy()


def _full_parity(h, got_bits, dt, what):
    """Every element and coordinate of a device decode against the oracle's decode of
    the same blob; returns (blob, coordinates, container values)."""
    from decode_tile_rans_amd import _lib as L
    blob = L.ep_serialize(h)
    say("oracle decode", what, len(blob))
    u_o, out_o, info = oracle.decode(blob)
    assert info["final_state_ok"] and info["reads_in_bounds"]
    R, C = out_o.shape
    assert got_bits.shape == (R, C)
    assert np.array_equal(got_bits.view(np.uint8), out_o.view(np.uint8)), what
    assert np.array_equal(_coords(h, R, C), u_o), what
    assert L.ep_blob_device_errors(h) == 0
    return blob, u_o, out_o


def _batch_fixture(indices):
    import torch
    from decode_tile_rans_amd import _lib as L
    say("stack matrices", indices[0], "..", indices[-1], ": drawing and compressing")
    srcs = [_bits(synth.dit_stack_torch(i)) for i in indices]
    handles = [_product_blob(s, nx.DT_BF16, 4.0) for s in srcs]
    side = torch.cuda.Stream()
    for h in handles:
        L.ep_blob_upload(h, int(side.cuda_stream))
    outs = [torch.empty(s.shape, dtype=torch.bfloat16, device="cuda") for s in srcs]
    L.ep_decompress_batch(handles, [o.data_ptr() for o in outs], int(side.cuda_stream))
    side.synchronize()
    return srcs, handles, outs


@pytest.fixture(scope="module")
def dit_block():
    from decode_tile_rans_amd import _lib as L
    srcs, handles, outs = _batch_fixture(list(range(9)))
    yield srcs, handles, outs
    for h in handles:
        L.ep_blob_free(h)


@pytest.fixture(scope="module")
def dit_extras():
    from decode_tile_rans_amd import _lib as L
    srcs, handles, outs = _batch_fixture(list(range(270, 276)))
    yield srcs, handles, outs
    for h in handles:
        L.ep_blob_free(h)


def test_dit_block_rate(dit_block):
    from decode_tile_rans_amd import _lib as L
    for h in dit_block[1]:
        assert 4.0 <= L.ep_actual_bpp(h) <= 4.1


def test_dit_block_device_residency(dit_block):
    """What a compressed weight costs in HBM: the stored bytes, plus the 56 KB of
    expanded decode tables, float32 row half-scales and section alignment -- within
    0.03 bpp of actual_bpp over the block (nothing is expanded per chain)."""
    from decode_tile_rans_amd import _lib as L
    srcs, handles, _ = dit_block
    params = sum(s.size for s in srcs)
    stored = sum(L.ep_serialized_size(h) for h in handles)
    dev = sum(L.ep_device_bytes(h) for h in handles)
    for s, h in zip(srcs, handles):
        extra = L.ep_device_bytes(h) - L.ep_serialized_size(h)
        assert 0 < extra <= 57344 + 4 * (s.shape[0] + 128) + 7 * 256 + 512
    assert 8.0 * dev / params <= 8.0 * stored / params + 0.03


@pytest.mark.timeout(600)
@pytest.mark.parametrize("index", list(range(9)))     # q, k, v, o, w1, w3, w2, mod1, mod2
def test_dit_block_parity_full(dit_block, index):
    srcs, handles, outs = dit_block
    _full_parity(handles[index], to_np(outs[index], nx.DT_BF16), nx.DT_BF16, f"stack matrix {index}")


def test_dit_block_spread_launch_equal(dit_block):
    """The block's launch (6300 blocks: more than one round of 256 CUs x 16 waves) with
    its blocks spread evenly over the CUs (EP_DECODE_SPREAD=1, waves looping over their
    share) writes the same bits as the default launch shape, which the parity tests
    above compare with the oracle."""
    import os
    import torch
    from decode_tile_rans_amd import _lib as L
    srcs, handles, outs = dit_block
    outs2 = [torch.full(s.shape, 7.0, dtype=torch.bfloat16, device="cuda") for s in srcs]
    os.environ["EP_DECODE_SPREAD"] = "1"
    try:
        L.ep_decompress_batch(handles, [o.data_ptr() for o in outs2], stream_ptr())
        torch.cuda.synchronize()
    finally:
        os.environ.pop("EP_DECODE_SPREAD", None)
    for a, b in zip(outs, outs2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for h in handles:
        assert L.ep_blob_device_errors(h) == 0


@pytest.mark.timeout(600)
@pytest.mark.parametrize("index", list(range(6)))
def test_dit_extras_parity_full(dit_extras, index):
    srcs, handles, outs = dit_extras
    _full_parity(handles[index], to_np(outs[index], nx.DT_BF16), nx.DT_BF16, f"stack matrix {270 + index}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("index", [0, 4, 6])        # q (3840^2), w1 (10240x3840), w2 (3840x10240)
def test_dit_block_encoder_bytes(dit_block, index):
    from decode_tile_rans_amd import _lib as L
    srcs, handles, _ = dit_block
    say("oracle full-size encode", srcs[index].shape)
    assert L.ep_serialize(handles[index]) == oracle.compress(srcs[index], nx.DT_BF16, 4.0)


@pytest.mark.timeout(600)
def test_fused_linear_full_size():
    import torch
    from decode_tile_rans_amd import _lib as L
    R, C, T = 14336, 4096, 4096
    say("fused linear: encode", R, C)
    wbits = synth.rowscaled(R, C, 5)
    h = _product_blob(wbits, nx.DT_BF16, 4.0)
    try:
        blob = L.ep_serialize(h)
        assert blob == oracle.compress(wbits, nx.DT_BF16, 4.0)
        L.ep_blob_upload(h, stream_ptr())
        xb = synth.activations(T, C, 50)
        x = torch.from_numpy(xb).view(torch.bfloat16).cuda()
        y = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
        need = L.ep_linear_workspace_bytes(h)
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        L.ep_compressed_linear_forward(h, x.data_ptr(), T, None, y.data_ptr(), ws.data_ptr(), need, stream_ptr())
        torch.cuda.synchronize()
        # the decoded weights the GEMM read: the 256-byte aligned start of the workspace
        off = (256 - ws.data_ptr() % 256) % 256
        wdec = ws[off:off + 2 * R * C].cpu().numpy().view(np.uint16).reshape(R, C)
        _, _, w_hat = _full_parity(h, wdec, nx.DT_BF16, "14336x4096 linear weight")   # (blob, coords, weights)
        rows = np.random.default_rng(1).choice(T, 256, replace=False)
        xf, wf = nx.bf16_to_f64(xb[rows]), nx.bf16_to_f64(w_hat)
        ref = linear_ref(xf, wf)
        mag = np.abs(xf) @ np.abs(wf).T
        check_linear(nx.bf16_to_f64(to_np(y, nx.DT_BF16)[rows]), ref, mag, C)
    finally:
        L.ep_blob_free(h)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("R,C,T,seed", [(14336, 4096, 256, 5), (8192, 8192, 96, 6)])
def test_fused_prefill_full_size(R, C, T, seed):
    # the 14336 x 4096 layer at 256 tokens and an 8192 x 8192 one (two tiles a row) at 96
    # through the fused prefill product (what the linear entry takes at these sizes):
    # every output element within the bound of the float64 product with the oracle's
    # decoded weights
    import torch
    from decode_tile_rans_amd import _lib as L
    say("fused prefill full size: encode", R, C, T)
    wbits = synth.rowscaled(R, C, seed)
    h = _product_blob(wbits, nx.DT_BF16, 4.0)
    try:
        blob = L.ep_serialize(h)
        L.ep_blob_upload(h, stream_ptr())
        xb = synth.activations(T, C, 52)
        x = torch.from_numpy(xb).view(torch.bfloat16).cuda()
        bias = synth.f32_to_bf16_bits(np.linspace(-1.0, 1.0, R).astype(np.float32))
        bt = torch.from_numpy(bias).view(torch.bfloat16).cuda()
        y = torch.full((T, R), 7.0, dtype=torch.bfloat16, device="cuda")
        L.ep_compressed_linear_prefill(h, x.data_ptr(), T, bt.data_ptr(), y.data_ptr(), stream_ptr())
        torch.cuda.synchronize()
        say("fused prefill full size: oracle")
        _, w_hat, _ = oracle.decode(blob)
        xf, wf = nx.bf16_to_f64(xb), nx.bf16_to_f64(w_hat)
        ref = linear_ref(xf, wf, nx.bf16_to_f64(bias))
        mag = np.abs(xf) @ np.abs(wf).T
        check_linear(nx.bf16_to_f64(to_np(y, nx.DT_BF16)), ref, mag, C)
        assert L.ep_blob_device_errors(h) == 0
    finally:
        L.ep_blob_free(h)


@pytest.mark.timeout(600)
def test_sixteen_chains_full_size():
    # the 14336 x 4096 layer encoded with 16 chains per tile: every decoded weight and
    # coordinate against the oracle's decode of the same blob, and the fused product on
    # 1 and 3 tokens (rows summed inside the decode kernel) within the float64 bound
    import torch
    from decode_tile_rans_amd import _lib as L
    R, C = 14336, 4096
    say("16 chains per tile full size: encode", R, C)
    wbits = synth.rowscaled(R, C, 5)
    h = _product_blob(wbits, nx.DT_BF16, 4.0, 16)
    try:
        assert L.ep_blob_params(h)[0] == 16
        data = L.ep_serialize(h)
    finally:
        L.ep_blob_free(h)
    db = DevBlob(data)
    full = db.decode()
    _, _, w_hat = _full_parity(db.h, full, nx.DT_BF16, "14336x4096 at S = 16")
    wf = nx.bf16_to_f64(w_hat)
    bias = synth.f32_to_bf16_bits(np.linspace(-1.0, 1.0, R).astype(np.float32))
    bt = torch.from_numpy(bias).view(torch.bfloat16).cuda()
    for T in (1, 3):
        say("16 chains per tile full size: product", T)
        xb = synth.activations(T, C, 53 + T)
        x = torch.from_numpy(xb).view(torch.bfloat16).cuda()
        y = torch.full((T, R), 7.0, dtype=torch.bfloat16, device="cuda")
        need = L.ep_linear_workspace_bytes(db.h)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        L.ep_compressed_linear_forward(db.h, x.data_ptr(), T, bt.data_ptr(), y.data_ptr(), ws.data_ptr(), need,
                                       stream_ptr())
        torch.cuda.synchronize()
        xf = nx.bf16_to_f64(xb)
        ref = linear_ref(xf, wf, nx.bf16_to_f64(bias))
        mag = np.abs(xf) @ np.abs(wf).T
        check_linear(nx.bf16_to_f64(to_np(y, nx.DT_BF16)), ref, mag, C)
    assert db.errors() == 0


SWEEP = [("bf16@2.3", nx.DT_BF16, 2.3), ("bf16@3.0", nx.DT_BF16, 3.0), ("bf16@5.0", nx.DT_BF16, 5.0),
         ("bf16@8.0", nx.DT_BF16, 8.0), ("fp8@5.0", nx.DT_FP8, 5.0), ("int8@4.0", nx.DT_INT8, 4.0)]


def _sweep_src(dt, n, seed=4):
    if dt == nx.DT_FP8:
        return synth.fp8_codes(n, n, seed)[0]
    if dt == nx.DT_INT8:
        return synth.int8_codes(n, n, seed)[0]
    return synth.rowscaled(n, n, seed)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,dt,t", SWEEP, ids=[s[0] for s in SWEEP])
def test_sweep_full_size_parity(name, dt, t):
    from decode_tile_rans_amd import _lib as L
    say("8192^2 sweep", name)
    src = _sweep_src(dt, 8192)
    h = _product_blob(src, dt, t)
    try:
        a = L.ep_actual_bpp(h)
        assert t <= a <= t + 0.1
        data = L.ep_serialize(h)
    finally:
        L.ep_blob_free(h)
    db = DevBlob(data)
    full = db.decode()
    assert db.errors() == 0
    _full_parity(db.h, full, dt, "8192^2 " + name)
    b = oracle.parse_blob(data)
    if name == "bf16@8.0":
        assert b.flags & 1            # the escape path at full size
    # tile subsets reproduce the full decode
    rng = np.random.default_rng(3)
    for t0 in list(rng.integers(0, b.n_tiles - 4, 3)) + [b.n_tiles - 3]:
        t0 = int(t0)
        t1 = min(t0 + 4, b.n_tiles)
        part = db.decode_tiles(t0, t1)
        cm = _tile_mask(b.R, b.C, range(t0, t1))
        assert np.array_equal(part[cm], full[cm])
    # distortion at the high-rate prediction (relative L2 = 2 delta sqrt(G) for
    # RMS-normalised rows; the excess at 8 bpp is the container's own rounding)
    w = nx.source_to_f64(src, dt)
    back = nx.source_to_f64(full, dt)
    err = np.linalg.norm(w - back) / np.linalg.norm(w)
    theory = 2.0 * float(b.delta) * SQRT_G
    assert abs(err / theory - 1.0) < 0.1, (err, theory)


@pytest.mark.timeout(600)
def test_outliers_escapes_full_size():
    say("outlier recipe 3072^2 @6.0")
    src = synth.rowscaled(3072, 3072, 2, 0.001)
    h = _product_blob(src, nx.DT_BF16, 6.0)
    from decode_tile_rans_amd import _lib as L
    try:
        data = L.ep_serialize(h)
    finally:
        L.ep_blob_free(h)
    b = oracle.parse_blob(data)
    assert b.S == 8 and (b.flags & 1)
    db = DevBlob(data)
    _full_parity(db.h, db.decode(), nx.DT_BF16, "outliers 3072^2 @6.0")


def test_fp8_gemm_sweep_shape():
    import torch
    from decode_tile_rans_amd import _lib as L
    T, N, K = 4096, 8192, 8192
    say("fp8 gemm", T, N, K)
    wq, aw = synth.fp8_codes(N, K, 4)
    xq, axr = synth.fp8_codes(T, K, 41)
    a_x = float(axr.max())
    xt = torch.from_numpy(xq).cuda()
    wt = torch.from_numpy(wq).cuda()
    awt = torch.from_numpy(aw).cuda()
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    L.ep_gemm_fp8_nt(xt.data_ptr(), wt.data_ptr(), a_x, awt.data_ptr(), y.data_ptr(), T, N, K, stream_ptr())
    torch.cuda.synchronize()
    rows = np.random.default_rng(2).choice(T, 64, replace=False)
    xf, wf = nx.fp8_e4m3fn_to_f64(xq[rows]), nx.fp8_e4m3fn_to_f64(wq)
    ref = linear_fp8_ref(xf, wf, a_x, aw)
    mag = linear_fp8_ref(np.abs(xf), np.abs(wf), a_x, aw)
    check_linear(nx.bf16_to_f64(to_np(y, nx.DT_BF16)[rows]), ref, mag, K, scale_roundings=2)
