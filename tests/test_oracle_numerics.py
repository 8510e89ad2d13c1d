"""Pins for the oracle's container casts against torch's CPU casts and the OCP
E4M3FN definition (value table enumerated from sign/exponent/mantissa)."""
import numpy as np
import pytest
import torch

from oracle import numerics as nx


def _rand_f32(n, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n) * scale * np.exp2(rng.integers(-20, 20, n))
    return x.astype(np.float32)


def test_bf16_vs_torch():
    x = _rand_f32(200000, 1)
    ours = nx.cast_bf16_sat(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.uint16).numpy()
    assert np.array_equal(ours, ref)
    # exact ties round to even
    t = np.array([0x3F808000, 0x3F818000, 0xBF808000], dtype=np.uint32).view(np.float32)
    assert list(nx.cast_bf16_sat(t)) == [0x3F80, 0x3F82, 0xBF80]
    # saturation instead of infinity
    big = np.array([3.4e38, -3.4e38], dtype=np.float32)
    assert list(nx.cast_bf16_sat(big)) == [0x7F7F, 0xFF7F]


def test_fp16_vs_torch():
    x = _rand_f32(200000, 2, 1e-3)
    x = x[np.abs(x) < 60000]
    ours = nx.cast_fp16_sat(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert list(nx.cast_fp16_sat(np.array([1e6, -70000.0], np.float32))) == [0x7BFF, 0xFBFF]


def _e4m3fn_values():
    vals = {}
    for b in range(256):
        s = -1.0 if b & 0x80 else 1.0
        e = (b >> 3) & 15
        m = b & 7
        if e == 15 and m == 7:
            continue
        v = s * (m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
        vals[b] = v
    return vals


def test_fp8_table_and_rounding():
    vals = _e4m3fn_values()
    codes = np.array(sorted(vals), dtype=np.uint8)
    v = np.array([vals[c] for c in codes], dtype=np.float64)
    # every representable value maps to its own code (except -0 -> sign kept)
    got = nx.cast_fp8_sat(v.astype(np.float32))
    assert np.array_equal(got, codes)
    assert max(vals.values()) == 448.0
    # midpoints between neighbours round to the even code
    pos = sorted(set(x for x in vals.values() if x >= 0))
    mids = np.array([(a + b) / 2 for a, b in zip(pos[:-1], pos[1:])], dtype=np.float32)
    r = nx.cast_fp8_sat(mids)
    assert (r & 1 == 0).all()
    # agreement with torch's float8 cast inside the range
    x = np.clip(_rand_f32(100000, 3, 1.0), -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(nx.cast_fp8_sat(x), ref)
    # saturation
    assert list(nx.cast_fp8_sat(np.array([1000.0, -1e9], np.float32))) == [0x7E, 0xFE]
    assert np.array_equal(nx.fp8_e4m3fn_to_f64(codes), v)


def test_int8():
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, 126.6, 127.5, 300.0, -128.4, -129.0, -1000.0], np.float32)
    want = [round(float(a)) for a in x]
    want = [max(-128, min(127, a)) for a in want]
    assert list(nx.cast_int8_sat(x)) == want
