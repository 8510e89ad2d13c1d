"""Pins for the oracle codec: the rate bar, high-rate distortion theory,
sampled estimate vs full data, tile independence, containers, validation and
corruption detection."""
import json
import math
import os

import numpy as np
import pytest

import synth
import oracle
from oracle import codec, numerics as nx, rate, model as mdl

API = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "api_facts.json")))
SQRT_G = math.sqrt(929 / 12960)


def _rel_l2(src_bits, out_bits):
    w = nx.bf16_to_f64(src_bits)
    wh = nx.bf16_to_f64(out_bits)
    return np.linalg.norm(w - wh) / np.linalg.norm(w)


@pytest.fixture(scope="module")
def c1():
    src = synth.small_gauss()
    blob = oracle.compress(src, nx.DT_BF16, 3.5)
    return src, blob


def test_config1_round_trip_and_bar(c1):
    src, blob = c1
    u, out, info = oracle.decode(blob)
    assert info["final_state_ok"] and info["reads_in_bounds"]
    a = codec.actual_bpp(blob)
    assert 3.5 <= a <= 3.6
    assert u.shape == src.shape and out.dtype == np.uint16
    b = codec.parse_blob(blob)
    # high-rate theory: rel-L2 = 2 delta sqrt(G) for RMS-normalised Gaussian rows
    theory = 2.0 * float(b.delta) * SQRT_G
    assert abs(_rel_l2(src, out) / theory - 1.0) < 0.05
    # reconstruction is exactly h_r * u cast to BF16
    h = rate.half_steps(b.s_bits, b.delta)
    assert np.array_equal(out, nx.cast_bf16_sat((h[:, None] * u.astype(np.float32)).astype(np.float32)))


def test_tile_independence(c1):
    _, blob = c1
    u_all, out_all, _ = oracle.decode(blob)
    b = codec.parse_blob(blob)
    G = -(-b.C // 8)
    for tiles in ([3], [b.n_tiles - 1, 0], [5, 2, 9]):
        u_t, out_t, info = oracle.decode(blob, tiles=tiles)
        assert info["final_state_ok"]
        gmask = np.zeros(b.R * G, dtype=bool)
        for t in tiles:
            gmask[512 * t: 512 * (t + 1)] = True
        cmask = np.repeat(gmask, 8).reshape(b.R, G * 8)[:, :b.C]
        assert np.array_equal(u_t[cmask], u_all[cmask])
        assert (u_t[~cmask] == 0).all()


@pytest.mark.slow
def test_config2_bar_and_estimate():
    src = synth.rowscaled(3072, 3072, 2, 0.001)
    tr = []
    blob = oracle.compress(src, nx.DT_BF16, 4.0, trace=tr)
    a = codec.actual_bpp(blob)
    assert 4.0 <= a <= 4.1
    b = codec.parse_blob(blob)
    # the +-10 s_r outliers sit at |m| ~ 40 lattice steps: K = 64 codes them directly,
    # so the sample (and the whole matrix) holds no escape symbol
    assert b.S == 8 and b.k == 6 and not (b.flags & codec.FLAG_ESC)
    u, out, info = oracle.decode(blob)
    assert info["final_state_ok"] and info["reads_in_bounds"]
    # full-data code length within 0.02 bpp of the sampled estimate at the chosen delta
    est = dict(tr)[rate.f32_bits(b.delta)]
    rows = rate.sample_rows(3072, 3072)
    est_bpp = est / 65536.0 / (len(rows) * 3072)
    data_bpp = 16.0 * len(b.stream) / src.size + 32.0 * b.n_chains / src.size
    assert abs(data_bpp - est_bpp) < 0.02 + 24.0 * b.n_chains / src.size


def test_outliers_take_the_escape_path():
    """The outlier recipe (log-normal rows, 0.1 % of entries at +-10 s_r) at 6 bpp: the
    outliers land beyond the largest direct magnitude (K = 128), so they are coded as
    escape buckets with raw bits.  Every decoded coordinate must equal the E8 point of
    the encoder's lattice input, and most outliers must be among the escaped ones."""
    R = C = 768
    src = synth.rowscaled(R, C, 2, 0.001)
    blob = oracle.compress(src, nx.DT_BF16, 6.0)
    b = codec.parse_blob(blob)
    assert b.k == 7 and (b.flags & codec.FLAG_ESC)
    assert 6.0 <= codec.actual_bpp(blob) <= 6.1
    u, out, info = oracle.decode(blob)
    assert info["final_state_ok"] and info["reads_in_bounds"]
    h = rate.half_steps(b.s_bits, b.delta)
    w = nx.bf16_to_f64(src)
    assert np.array_equal(u, rate.quantize_rows(w, h).reshape(R, C))
    big = np.abs(u) >> 1 >= 128
    outl = np.abs(w) >= 9.0 * np.sqrt((w * w).mean(axis=1, keepdims=True))
    assert (big & outl).sum() >= 0.5 * outl.sum() > 0      # most outliers take escapes


@pytest.mark.parametrize("t", [1.0, 2.3, 3.0, 5.0, 8.0, 11.0])
def test_rate_bar_sweep(t):
    src = synth.rowscaled(512, 512, 40 + int(t * 10))
    blob = oracle.compress(src, nx.DT_BF16, t)
    a = codec.actual_bpp(blob)
    # 512 rows x 16-bit scales alone cost 0.03 bpp at C = 512
    assert t <= a <= t + 0.1, (t, a)
    u, out, info = oracle.decode(blob)
    assert info["final_state_ok"] and info["reads_in_bounds"]


def test_low_targets_and_estimate_monotone():
    src = synth.rowscaled(256, 512, 77)
    for t in (API["target_bpp_min"], 0.1, 0.5):
        blob = oracle.compress(src, nx.DT_BF16, t)
        u, out, info = oracle.decode(blob)
        assert info["final_state_ok"]
        assert codec.actual_bpp(blob) < t + 0.2
    w = nx.bf16_to_f64(src)
    wp = w
    s = rate.row_scales_bf16(w)
    ests = [rate.estimate(wp, s, np.float32(2.0 ** (j / 4)))[0] for j in range(-40, 8)]
    assert all(ests[i] >= ests[i + 1] for i in range(len(ests) - 1))


def test_rate_theory_gaussian():
    # High-rate theory: y = w / (2 h_r) is N(0, 1/(4 delta^2)) for RMS-normalised Gaussian
    # rows and E8 cells have unit volume, so rate = h(y) = 0.5 log2(2 pi e) - log2(2 delta).
    src = synth.rowscaled(1024, 256, 5)
    for t in (5.0, 7.0):
        blob = oracle.compress(src, nx.DT_BF16, t)
        b = codec.parse_blob(blob)
        predicted = 0.5 * math.log2(2 * math.pi * math.e) - math.log2(2.0 * float(b.delta))
        assert abs(t - predicted) < 0.08, (t, predicted)


@pytest.mark.parametrize("dtype", [nx.DT_FP16, nx.DT_FP32, nx.DT_FP8, nx.DT_INT8])
def test_containers(dtype):
    R, C = 96, 200
    if dtype == nx.DT_FP8:
        src, _ = synth.fp8_codes(R, C, 4)
        t = 5.0
    elif dtype == nx.DT_INT8:
        src, _ = synth.int8_codes(R, C, 4)
        t = 4.0
    elif dtype == nx.DT_FP16:
        src = synth.rowscaled_f32(R, C, 4).astype(np.float16).view(np.uint16)
        t = 4.0
    else:
        src = synth.rowscaled_f32(R, C, 4)
        t = 6.0
    blob = oracle.compress(src, dtype, t)
    u, out, info = oracle.decode(blob)
    assert info["final_state_ok"]
    assert out.shape == (R, C)
    assert out.dtype == {nx.DT_FP16: np.uint16, nx.DT_FP32: np.float32, nx.DT_FP8: np.uint8,
                         nx.DT_INT8: np.int8}[dtype]
    w = nx.source_to_f64(src, dtype)
    back = nx.source_to_f64(out if dtype != nx.DT_FP32 else out, dtype)
    assert np.linalg.norm(w - back) / np.linalg.norm(w) < 0.1
    if dtype == nx.DT_FP8:
        assert np.abs(back).max() <= 448.0


@pytest.mark.parametrize("R,C", [(1, 1), (1, 8), (3, 13), (37, 13), (5, 4097), (600, 7)])
def test_odd_shapes(R, C):
    rng = np.random.default_rng(R * 100 + C)
    src = synth.f32_to_bf16_bits((rng.standard_normal((R, C)) * 0.05).astype(np.float32))
    blob = oracle.compress(src, nx.DT_BF16, 4.0)
    u, out, info = oracle.decode(blob)
    assert info["final_state_ok"] and info["reads_in_bounds"] and out.shape == (R, C)


def test_zero_and_constant_matrices():
    z = np.zeros((64, 64), dtype=np.uint16)
    u, out, info = oracle.decode(oracle.compress(z, nx.DT_BF16, 2.0))
    assert (out == 0).all() and info["final_state_ok"]
    one = np.full((16, 40), 0x3F80, dtype=np.uint16)    # 1.0
    u, out, info = oracle.decode(oracle.compress(one, nx.DT_BF16, 3.0))
    assert info["final_state_ok"]
    assert np.abs(nx.bf16_to_f64(out) - 1.0).max() < 0.1


def test_validation_errors():
    src = synth.small_gauss(8, 8)
    for t in (API["target_bpp_min"] / 2, API["target_bpp_max"] + 0.01, float("nan"), float("inf")):
        with pytest.raises(codec.CompressError) as e:
            oracle.compress(src, nx.DT_BF16, t)
        assert e.value.code == "range"
    with pytest.raises(codec.CompressError) as e:
        oracle.compress(src.reshape(-1), nx.DT_BF16, 4.0)
    assert e.value.code == "shape"
    with pytest.raises(codec.CompressError) as e:
        oracle.compress(src, 9, 4.0)
    assert e.value.code == "dtype"
    bad = src.copy()
    bad[0, 0] = 0x7FC0    # NaN
    with pytest.raises(codec.CompressError) as e:
        oracle.compress(bad, nx.DT_BF16, 4.0)
    assert e.value.code == "nonfinite"
    with pytest.raises(codec.CompressError):
        oracle.compress(np.zeros((4, 4), np.int8), nx.DT_INT8, 9.0)


def test_corruption_detected(c1):
    _, blob = c1
    with pytest.raises(ValueError):
        codec.parse_blob(blob[:-2])
    with pytest.raises(ValueError):
        codec.parse_blob(b"XXXX" + blob[4:])
    b = codec.parse_blob(blob)
    b.stream = b.stream.copy()
    b.stream[len(b.stream) // 2] ^= 0x5A5A
    u, out, info = oracle.decode(b)
    assert not info["final_state_ok"]
