"""Full-size GPU checks in the launch configuration the benchmark times.

* DiT stack: the first transformer block (9 matrices, drawn as bench.py draws them) is
  compressed by the library and decoded with one batched launch on a side stream.  For
  one matrix of each of the three shapes the oracle compresses the same input, the
  library's blob must be byte-identical, and sampled tiles decoded by the oracle from its
  own blob must match the GPU output bit for bit.  All 9 must end every chain in L.
* Fused linear prefill (14336 x 4096 @ 4.0 bpp, 4096 tokens): same blob check, then
  relative L2 of sampled output rows against the float64 oracle GEMM.
* 8192^2 bitrate / container sweep: full-size properties (rate bar, chains end in L,
  tile subsets equal the full decode, distortion close to high-rate theory); bit parity
  with the oracle at 1024^2 with the same recipe.
"""
import math

import numpy as np
import pytest

import synth
import oracle
from oracle import numerics as nx
from oracle.gemm import linear_fp8_ref, linear_ref, rel_l2

pytestmark = pytest.mark.gpu

from gpu_util import DevBlob, say, stream_ptr, to_np  # noqa: E402

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
    h = L.ep_compress(src.ctypes.data, dt, src.shape[0], src.shape[1], t, S)
    return h


@pytest.fixture(scope="module")
def dit_block():
    import torch
    from decode_tile_rans_amd import _lib as L
    say("dit block: drawing and compressing 9 matrices")
    srcs = [_bits(synth.dit_stack_torch(i)) for i in range(9)]
    handles = [_product_blob(s, nx.DT_BF16, 4.0) for s in srcs]
    side = torch.cuda.Stream()
    for h in handles:
        L.ep_blob_upload(h, int(side.cuda_stream))
    outs = [torch.empty(s.shape, dtype=torch.bfloat16, device="cuda") for s in srcs]
    L.ep_decompress_batch(handles, [o.data_ptr() for o in outs], int(side.cuda_stream))
    side.synchronize()
    yield srcs, handles, outs
    for h in handles:
        L.ep_blob_free(h)


def test_dit_block_all_chains_and_rate(dit_block):
    from decode_tile_rans_amd import _lib as L
    srcs, handles, outs = dit_block
    for s, h in zip(srcs, handles):
        assert L.ep_blob_device_errors(h) == 0
        assert 4.0 <= L.ep_actual_bpp(h) <= 4.1


@pytest.mark.timeout(400)
@pytest.mark.parametrize("index", [0, 4, 6])        # q (3840^2), w1 (10240x3840), w2 (3840x10240)
def test_dit_block_parity_sampled(dit_block, index):
    from decode_tile_rans_amd import _lib as L
    srcs, handles, outs = dit_block
    src = srcs[index]
    say("oracle full-size encode", src.shape)
    blob = oracle.compress(src, nx.DT_BF16, 4.0)
    assert L.ep_serialize(handles[index]) == blob
    b = oracle.parse_blob(blob)
    rng = np.random.default_rng(index)
    tiles = sorted(set([0, 1, b.n_tiles - 1] + rng.integers(0, b.n_tiles, 40).tolist()))
    _, out_o, info = oracle.decode(blob, tiles=tiles)
    assert info["final_state_ok"]
    got = to_np(outs[index], nx.DT_BF16)
    cm = _tile_mask(b.R, b.C, tiles)
    assert np.array_equal(got[cm], out_o[cm])


@pytest.mark.timeout(400)
def test_fused_linear_full_size():
    import torch
    from decode_tile_rans_amd import _lib as L
    R, C, T = 14336, 4096, 4096
    say("fused linear: oracle full-size encode", R, C)
    wbits = synth.rowscaled(R, C, 5)
    blob = oracle.compress(wbits, nx.DT_BF16, 4.0)
    h = _product_blob(wbits, nx.DT_BF16, 4.0)
    try:
        assert L.ep_serialize(h) == blob
        L.ep_blob_upload(h, stream_ptr())
        xb = synth.activations(T, C, 50)
        x = torch.from_numpy(xb).view(torch.bfloat16).cuda()
        y = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
        need = L.ep_linear_workspace_bytes(h)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        L.ep_compressed_linear_forward(h, x.data_ptr(), T, None, y.data_ptr(), ws.data_ptr(), need, stream_ptr())
        torch.cuda.synchronize()
        assert L.ep_blob_device_errors(h) == 0
        _, w_hat, _ = oracle.decode(blob)
        rows = np.random.default_rng(1).choice(T, 96, replace=False)
        ref = linear_ref(nx.bf16_to_f64(xb[rows]), nx.bf16_to_f64(w_hat))
        got = nx.bf16_to_f64(to_np(y, nx.DT_BF16)[rows])
        assert rel_l2(got, ref) <= 1e-2
    finally:
        L.ep_blob_free(h)


SWEEP = [("bf16@2.3", nx.DT_BF16, 2.3), ("bf16@3.0", nx.DT_BF16, 3.0), ("bf16@5.0", nx.DT_BF16, 5.0),
         ("bf16@8.0", nx.DT_BF16, 8.0), ("fp8@5.0", nx.DT_FP8, 5.0), ("int8@4.0", nx.DT_INT8, 4.0)]


def _sweep_src(dt, n, seed=4):
    if dt == nx.DT_FP8:
        return synth.fp8_codes(n, n, seed)[0]
    if dt == nx.DT_INT8:
        return synth.int8_codes(n, n, seed)[0]
    return synth.rowscaled(n, n, seed)


@pytest.mark.parametrize("name,dt,t", SWEEP, ids=[s[0] for s in SWEEP])
def test_sweep_full_size_properties(name, dt, t):
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
    b = oracle.parse_blob(data)
    # tile subsets reproduce the full decode
    rng = np.random.default_rng(3)
    for t0 in list(rng.integers(0, b.n_tiles - 4, 3)) + [b.n_tiles - 3]:
        t0 = int(t0)
        t1 = min(t0 + 4, b.n_tiles)
        part = db.decode_tiles(t0, t1)
        cm = _tile_mask(b.R, b.C, range(t0, t1))
        assert np.array_equal(part[cm], full[cm])
    # distortion at the high-rate prediction (relative L2 = 2 delta sqrt(G) for
    # RMS-normalised rows; the oracle meets it within 6 % at 1024^2 on every point,
    # the excess at 8 bpp being the container's own rounding)
    w = nx.source_to_f64(src, dt)
    back = nx.source_to_f64(full, dt)
    err = np.linalg.norm(w - back) / np.linalg.norm(w)
    theory = 2.0 * float(b.delta) * SQRT_G
    assert abs(err / theory - 1.0) < 0.1, (err, theory)


@pytest.mark.parametrize("name,dt,t", SWEEP, ids=[s[0] for s in SWEEP])
def test_sweep_reduced_parity(name, dt, t):
    say("1024^2 sweep parity", name)
    src = _sweep_src(dt, 1024, seed=40)
    blob = oracle.compress(src, dt, t, chains_per_tile=8)
    u_o, out_o, info = oracle.decode(blob)
    assert info["final_state_ok"]
    db = DevBlob(blob)
    assert np.array_equal(db.coords(), u_o)
    assert np.array_equal(db.decode().view(np.uint8), out_o.view(np.uint8))
    assert db.errors() == 0


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
    ref = linear_fp8_ref(nx.fp8_e4m3fn_to_f64(xq[rows]), nx.fp8_e4m3fn_to_f64(wq), a_x, aw)
    got = nx.bf16_to_f64(to_np(y, nx.DT_BF16)[rows])
    assert rel_l2(got, ref) <= 1e-2
