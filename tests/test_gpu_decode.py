"""GPU parity of the fused decode kernel against the oracle.

Blobs are made by the oracle (so no oracle input comes from the product); the
GPU decodes them through the C ABI.  Integer results (doubled lattice
coordinates, container bit patterns) must match bit for bit; every rANS chain
must end in its initial state (device error count 0).
"""
import os

import numpy as np
import pytest

import synth
import oracle
from oracle import numerics as nx

pytestmark = pytest.mark.gpu

from gpu_util import DevBlob, say, to_np  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    from decode_tile_rans_amd import _lib as L
    L.lib()        # fails loudly when the HIP library is missing
    yield


def _check(name, src, dt, t, S=None, env=None):
    say(name, src.shape, dt, t, S, env)
    blob = oracle.compress(src, dt, t, chains_per_tile=S)
    u_o, out_o, info = oracle.decode(blob)
    assert info["final_state_ok"]
    old = {}
    for k, v in (env or {}).items():
        old[k] = os.environ.get(k)
        os.environ[k] = v
    try:
        db = DevBlob(blob)
        u_g = db.coords()
        assert np.array_equal(u_g, u_o), f"{name}: coords differ at {np.argwhere(u_g != u_o)[:5]}"
        out_g = db.decode()
        assert np.array_equal(out_g.view(np.uint8), out_o.view(np.uint8)), f"{name}: container values differ"
        assert db.errors() == 0
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return blob, u_o, out_o


def test_small_gauss_config():
    _check("small_gauss 256x256 @3.5", synth.small_gauss(), nx.DT_BF16, 3.5)


@pytest.mark.parametrize("t,S", [(2.3, None), (3.0, 8), (4.0, None), (4.0, 2)])
def test_escapes_outside_the_rate_sample(t, S):
    # 1024 x 1024: the rate search samples every fourth row from row 0, so outliers in rows
    # 1, 5, 9, ... stay out of its escape count: a small escape threshold (K <= 32, the
    # narrow one-word tables of 1024 slots) with escape symbols in the blob
    src = synth.rowscaled_row_outliers(1024, 1024, 91)
    blob, _, _ = _check(f"outliers outside the sample 1024^2 @{t} S={S}", src, nx.DT_BF16, t, S)
    b = oracle.parse_blob(blob)
    assert b.k <= 5 and (b.flags & 1), (b.k, b.flags)


@pytest.mark.parametrize("t", [9.0, 11.0])
def test_huge_magnitudes_two_bypass_fields(t):
    # one entry per row 1e4 times the others: magnitudes of 2^19 and more, whose raw bits
    # (more than 16) are read as two bypass fields
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((4, 65536)) * 0.01).astype(np.float32)
    w[:, 5] = 100.0
    w[2, 70000 % 65536] = -100.0
    blob, u_o, _ = _check(f"huge magnitudes 4x65536 @{t}", synth.f32_to_bf16_bits(w), nx.DT_BF16, t)
    assert (np.abs(u_o) >> 1).max() >= 1 << 19


def test_rowscaled_outliers_3072():
    _check("rowscaled+outliers 3072x3072 @4.0", synth.rowscaled(3072, 3072, 2, 0.001), nx.DT_BF16, 4.0)


@pytest.mark.parametrize("R,C", [(1, 1), (37, 13), (5, 4097), (600, 7), (3, 8), (129, 1000)])
def test_ragged_shapes(R, C):
    _check(f"ragged {R}x{C}", synth.rowscaled(R, C, R + C), nx.DT_BF16, 4.0)


@pytest.mark.parametrize("S", [1, 2, 4, 8, 16, 32, 64])
def test_chains_per_tile(S):
    _check(f"S={S}", synth.rowscaled(200, 512 + 24, 90 + S), nx.DT_BF16, 3.0, S=S)


@pytest.mark.parametrize("t", [0.001, 0.5, 2.3, 8.0, 11.0])
def test_rates_and_escapes(t):
    blob, _, _ = _check(f"rate {t}", synth.rowscaled(256, 512, 120), nx.DT_BF16, t, S=8)
    if t >= 8:
        assert oracle.parse_blob(blob).flags & 1      # escapes exercised


@pytest.mark.parametrize("waves", ["1", "2", "5", "16"])
def test_workgroup_sizes(waves):
    _check(f"waves={waves}", synth.rowscaled(257, 1024, 8), nx.DT_BF16, 4.0, S=8, env={"EP_DECODE_WAVES": waves})


# Two chains per lane (two blocks interleaved, 64-byte rings without a mirror, reads
# wrapping): a spread launch takes this shape by itself when its blocks fit one round of
# it; here it is forced on small cases that cover odd chain counts, chains that finish a
# group earlier than their partner, several blocks per workgroup, escapes and containers.
ILP2_CASES = [
    ("ragged 37x13", lambda: synth.rowscaled(37, 13, 50), nx.DT_BF16, 4.0, None, "1"),
    ("ragged 129x1000", lambda: synth.rowscaled(129, 1000, 51), nx.DT_BF16, 4.0, None, "3"),
    ("S=8 odd tail", lambda: synth.rowscaled(257, 1024, 52), nx.DT_BF16, 4.0, 8, "2"),
    ("S=2", lambda: synth.rowscaled(200, 536, 53), nx.DT_BF16, 3.0, 2, "13"),
    ("S=64", lambda: synth.rowscaled(200, 536, 54), nx.DT_BF16, 3.0, 64, "5"),
    ("S=1", lambda: synth.rowscaled(300, 520, 55), nx.DT_BF16, 4.0, 1, "4"),
    ("escapes 8 bpp", lambda: synth.rowscaled(256, 512, 56), nx.DT_BF16, 8.0, 8, "2"),
    ("escapes 11 bpp", lambda: synth.rowscaled(256, 512, 57), nx.DT_BF16, 11.0, 8, "1"),
    ("outliers", lambda: synth.rowscaled(512, 1024, 58, 0.001), nx.DT_BF16, 4.0, 8, "13"),
    ("low rate", lambda: synth.rowscaled(256, 512, 59), nx.DT_BF16, 0.001, 8, "2"),
    ("fp8", lambda: synth.fp8_codes(512, 520, 60)[0], nx.DT_FP8, 5.0, 8, "3"),
    ("int8", lambda: synth.int8_codes(512, 520, 61)[0], nx.DT_INT8, 4.0, 8, "3"),
    ("fp32", lambda: synth.rowscaled_f32(256, 264, 62), nx.DT_FP32, 6.0, 8, "2"),
]


@pytest.mark.parametrize("case", ILP2_CASES, ids=[c[0] for c in ILP2_CASES])
def test_two_chains_per_lane(case):
    name, make, dt, t, S, waves = case
    _check(f"ilp2 {name}", make(), dt, t, S=S, env={"EP_DECODE_ILP": "2", "EP_DECODE_WAVES": waves})


def test_two_chains_per_lane_tiles():
    src = synth.rowscaled(512, 1032, 63)
    blob = oracle.compress(src, nx.DT_BF16, 4.0, chains_per_tile=8)
    b = oracle.parse_blob(blob)
    old = {k: os.environ.get(k) for k in ("EP_DECODE_ILP", "EP_DECODE_WAVES")}
    os.environ["EP_DECODE_ILP"] = "2"
    os.environ["EP_DECODE_WAVES"] = "2"
    try:
        db = DevBlob(blob)
        full = db.decode()
        G = -(-b.C // 8)
        for (t0, t1) in [(0, 1), (1, 2), (3, 10), (b.n_tiles - 3, b.n_tiles)]:
            say("ilp2 tiles", t0, t1)
            part = db.decode_tiles(t0, t1, fill=0x5A)
            gm = np.zeros(b.R * G, dtype=bool)
            gm[512 * t0: 512 * t1] = True
            cm = np.repeat(gm, 8).reshape(b.R, G * 8)[:, :b.C]
            assert np.array_equal(part[cm], full[cm])
            assert (part.view(np.uint8).reshape(b.R, -1)[np.repeat(~cm, 2, axis=1)] == 0x5A).all()
        assert db.errors() == 0
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


@pytest.mark.parametrize("dt", [nx.DT_FP16, nx.DT_FP32, nx.DT_FP8, nx.DT_INT8])
def test_containers(dt):
    R, C = 512, 520
    if dt == nx.DT_FP8:
        src, t = synth.fp8_codes(R, C, 4)[0], 5.0
    elif dt == nx.DT_INT8:
        src, t = synth.int8_codes(R, C, 4)[0], 4.0
    elif dt == nx.DT_FP16:
        src, t = synth.rowscaled_f32(R, C, 4).astype(np.float16).view(np.uint16), 4.0
    else:
        src, t = synth.rowscaled_f32(R, C, 4), 6.0
    _check(f"container {dt}", src, dt, t, S=8)


def test_saturating_bf16():
    # rows near the BF16 maximum force the clamping variant of the kernel
    w = synth.rowscaled_f32(64, 256, 11) * np.float32(1e38 / 0.02)
    w = np.clip(w, -3.3e38, 3.3e38).astype(np.float32)
    src = synth.f32_to_bf16_bits(w)
    blob, _, _ = _check("bf16 near max", src, nx.DT_BF16, 2.0)


@pytest.mark.parametrize("dt", [nx.DT_BF16, nx.DT_FP32])
def test_huge_row_scales_narrow(dt):
    # escape-free narrow tables (1 bpp, k = 3) with row half-scales h_r near 1e38: the
    # kernel's fma(u + 128, h, -128 h) would overflow in -128 h, so these blobs take the
    # plain product (BF16: the container also saturates)
    w = np.clip(synth.rowscaled_f32(48, 512, 94) * np.float32(1e38 / 0.02), -3.3e38, 3.3e38).astype(np.float32)
    src = synth.f32_to_bf16_bits(w) if dt == nx.DT_BF16 else w
    b = oracle.parse_blob(oracle.compress(src, dt, 1.0))
    assert b.k <= 5 and not (b.flags & 1)
    _check(f"huge row scales {dt}", src, dt, 1.0)


def test_tile_independence():
    src = synth.rowscaled(512, 1032, 12)
    blob = oracle.compress(src, nx.DT_BF16, 4.0, chains_per_tile=8)
    b = oracle.parse_blob(blob)
    db = DevBlob(blob)
    full = db.decode()
    G = -(-b.C // 8)
    rng = np.random.default_rng(0)
    ranges = [(0, 1), (b.n_tiles - 1, b.n_tiles), (3, 9), (b.n_tiles // 2, b.n_tiles)]
    ranges += [tuple(sorted(rng.integers(0, b.n_tiles, 2) + np.array([0, 1]))) for _ in range(4)]
    for (t0, t1) in ranges:
        say("tiles", t0, t1)
        part = db.decode_tiles(int(t0), int(t1), fill=0xA5)
        gm = np.zeros(b.R * G, dtype=bool)
        gm[512 * t0: 512 * t1] = True
        cm = np.repeat(gm, 8).reshape(b.R, G * 8)[:, :b.C]
        assert np.array_equal(part[cm], full[cm])
        assert (part.view(np.uint8).reshape(b.R, -1)[np.repeat(~cm, 2, axis=1)] == 0xA5).all()
        # the oracle decoding only these tiles agrees too
        _, out_o, _ = oracle.decode(blob, tiles=range(t0, t1))
        assert np.array_equal(part[cm], out_o[cm])
    assert db.errors() == 0


def test_batch_matches_single():
    import torch
    from decode_tile_rans_amd import _lib as L
    from gpu_util import stream_ptr
    shapes = [(256, 512, 3.0, 8), (100, 200, 4.0, 1), (64, 4096, 5.0, 8), (513, 264, 2.3, 8), (1, 8, 4.0, 1),
              (300, 300, 8.0, 8), (128, 1024, 4.0, 2), (77, 640, 4.5, 8), (512, 512, 3.5, 64),
              (40, 2000, 4.0, 8), (1000, 24, 4.0, 4), (64, 64, 1.0, 1), (200, 200, 6.0, 16)]
    dbs, refs = [], []
    for i, (R, C, t, S) in enumerate(shapes):
        blob = oracle.compress(synth.rowscaled(R, C, 700 + i), nx.DT_BF16, t, chains_per_tile=S)
        dbs.append(DevBlob(blob))
        refs.append(oracle.decode(blob)[1])
    outs = [torch.zeros((d.R, d.C), dtype=torch.bfloat16, device="cuda") for d in dbs]
    say("batch of", len(dbs))
    L.ep_decompress_batch([d.h for d in dbs], [o.data_ptr() for o in outs], stream_ptr())
    torch.cuda.synchronize()
    for d, o, r in zip(dbs, outs, refs):
        assert np.array_equal(to_np(o, nx.DT_BF16), r)
        assert d.errors() == 0


def _batch_parity(cases, env, label):
    import torch
    from decode_tile_rans_amd import _lib as L
    from gpu_util import stream_ptr
    dbs, refs = [], []
    for (src, dt, t, S) in cases:
        blob = oracle.compress(src, dt, t, chains_per_tile=S)
        dbs.append(DevBlob(blob))
        refs.append(oracle.decode(blob)[1])
    outs = [d.empty_out(0x5A) for d in dbs]
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        say(label, "batch of", len(dbs), "blocks", sum(oracle.parse_blob(d.data).n_blocks for d in dbs))
        L.ep_decompress_batch([d.h for d in dbs], [o.data_ptr() for o in outs], stream_ptr())
        torch.cuda.synchronize()
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    for i, (d, o, r) in enumerate(zip(dbs, outs, refs)):
        assert np.array_equal(to_np(o, d.dt).view(np.uint8), r.view(np.uint8)), (label, i)
        assert d.errors() == 0, (label, i)


# Batches: blobs with and without escapes and with narrow and wide tables go to separate
# launches of at most 12 blobs; small and ragged blobs, containers, more blobs than
# one launch holds.
def test_batch_small_and_ragged():
    cases = [(synth.rowscaled(R, C, 800 + i), nx.DT_BF16, t, S)
             for i, (R, C, t, S) in enumerate([(37, 13, 4.0, None), (256, 512, 3.0, 8), (1, 8, 4.0, 1),
                                               (129, 1000, 4.5, 8), (64, 64, 1.0, 1), (300, 300, 2.3, 8)])]
    _batch_parity(cases, {}, "batch small")


def test_batch_many_shapes():
    rng = np.random.default_rng(7)
    cases = []
    for i in range(24):
        R, C = int(rng.integers(64, 700)), int(rng.choice([256, 520, 1024, 1032]))
        cases.append((synth.rowscaled(R, C, 820 + i), nx.DT_BF16, float(rng.choice([2.3, 3.0, 4.0, 5.0])),
                      int(rng.choice([1, 2, 4, 8]))))
    _batch_parity(cases, {}, "batch shapes")


def test_batch_escapes_and_wide_tables():
    cases = [(synth.rowscaled(256, 512, 840), nx.DT_BF16, 8.0, 8), (synth.rowscaled(512, 1024, 841, 0.001),
             nx.DT_BF16, 4.0, 8), (synth.rowscaled(256, 512, 842), nx.DT_BF16, 11.0, 8),
             (synth.rowscaled(200, 536, 843), nx.DT_BF16, 3.0, 2), (synth.rowscaled(128, 1024, 844), nx.DT_BF16, 9.0, 4)]
    _batch_parity(cases, {}, "batch escapes")


@pytest.mark.parametrize("dt", [nx.DT_FP16, nx.DT_FP32, nx.DT_FP8, nx.DT_INT8])
def test_batch_containers(dt):
    if dt == nx.DT_FP8:
        mk = lambda i: synth.fp8_codes(256, 520, 850 + i)[0]
    elif dt == nx.DT_INT8:
        mk = lambda i: synth.int8_codes(256, 520, 850 + i)[0]
    elif dt == nx.DT_FP16:
        mk = lambda i: synth.rowscaled_f32(256, 520, 850 + i).astype(np.float16).view(np.uint16)
    else:
        mk = lambda i: synth.rowscaled_f32(256, 264, 850 + i)
    cases = [(mk(i), dt, 4.0 + i, 8) for i in range(3)]
    _batch_parity(cases, {}, f"batch dt {dt}")


def test_batch_more_blobs_than_one_launch():
    cases = [(synth.rowscaled(16 + i % 5, 64 + 8 * (i % 7), 900 + i), nx.DT_BF16, 4.0, 1) for i in range(170)]
    _batch_parity(cases, {}, "batch 170 blobs")


def test_budgeted_mixed_rate_stack():
    # a stack planned under one bit budget (matrices of different norms get different
    # targets) decodes in one batch launch, every matrix bit-exact with the oracle
    import torch
    import decode_tile_rans_amd as ep
    from decode_tile_rans_amd import _lib as L
    from gpu_util import stream_ptr
    shapes = [(256, 512, 1.0), (128, 1024, 8.0), (300, 200, 0.125), (64, 2048, 2.0), (512, 256, 0.5),
              (96, 640, 4.0), (200, 384, 0.25), (128, 128, 16.0)]
    mats = [synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(synth.rowscaled(R, C, 900 + i)) * np.float32(f))
            for i, (R, C, f) in enumerate(shapes)]
    cs, targets = ep.plan_bitrates(mats, 3.0, (2.0, 2.5, 3.0, 3.5, 4.0, 5.0), dtype=torch.bfloat16)
    say("mixed-rate stack, targets", targets)
    assert len(set(targets)) >= 3
    assert sum(c.actual_bpp * m.size for c, m in zip(cs, mats)) <= 3.0 * sum(m.size for m in mats)
    refs = []
    for m, t, c in zip(mats, targets, cs):
        blob = oracle.compress(m, nx.DT_BF16, t)
        assert c.to_bytes() == blob
        refs.append(oracle.decode(blob)[1])
    outs = ep.decompress_batch(cs)
    torch.cuda.synchronize()
    for c, o, r in zip(cs, outs, refs):
        assert np.array_equal(to_np(o, nx.DT_BF16), r)
        assert c.device_errors() == 0


def test_corrupt_stream_flags_error():
    src = synth.rowscaled(256, 1024, 13)
    blob = bytearray(oracle.compress(src, nx.DT_BF16, 4.0, chains_per_tile=8))
    b = oracle.parse_blob(bytes(blob))
    nw = len(b.stream)
    stream_off = len(blob) - 2 * nw
    for q in (nw // 3, nw // 2, 2 * nw // 3):
        blob[stream_off + 2 * q] ^= 0x5A
    blob = bytes(blob)
    _, _, info = oracle.decode(blob)
    assert not info["final_state_ok"]
    say("corrupt stream")
    db = DevBlob(blob)
    db.decode()
    assert db.errors() > 0


def test_host_pointer_destination_refused():
    # a pageable host buffer as the destination is refused before any launch
    from decode_tile_rans_amd import _lib as L
    blob = oracle.compress(synth.rowscaled(64, 64, 3), nx.DT_BF16, 4.0)
    db = DevBlob(blob)
    host = np.zeros(64 * 64 + 64, dtype=np.uint16)
    p = host.ctypes.data + ((16 - host.ctypes.data % 16) % 16)
    with pytest.raises(L.EPError) as ei:
        L.ep_decompress(db.h, p, 0)
    assert ei.value.name == "EP_E_ARG"
    with pytest.raises(L.EPError) as ei:
        L.ep_decompress_batch([db.h], [p], 0)
    assert ei.value.name == "EP_E_ARG"
