"""Pins of the TileANS (lossless) oracle: exact round trips, the entropy bound,
uniform tables on incompressible bytes, tile independence."""
import numpy as np
import pytest

import synth
from oracle import tileans as ta
from oracle.tileans import P, M


def _bytes_of(a):
    return np.frombuffer(np.ascontiguousarray(a).tobytes(), dtype=np.uint8)


def _check(a, E, S=None):
    raw = _bytes_of(a)
    blob = ta.compress(raw, E, a.shape, 7, chains_per_tile=S)
    out, info = ta.decode(blob)
    assert np.array_equal(out, raw)
    assert info["final_state_ok"] and info["reads_in_bounds"]
    b = ta.parse(blob)
    assert b.dims == tuple(a.shape) and b.E == E and b.dtype_tag == 7
    return blob, b


CASES = [
    ("bf16 weights", lambda: synth.rowscaled(96, 200, 1), 2, None),
    ("bf16 S8", lambda: synth.rowscaled(64, 1024, 2), 2, 8),
    ("fp32 3-d", lambda: synth.rowscaled_f32(8, 24, 3).reshape(2, 4, 24), 4, 2),
    ("fp16 1-d ragged", lambda: synth.rowscaled_f32(1, 1001, 4).astype(np.float16).reshape(-1), 2, 1),
    ("fp8 codes", lambda: synth.fp8_codes(64, 136, 5)[0], 1, 4),
    ("int8 codes", lambda: synth.int8_codes(32, 520, 6)[0], 1, 64),
    ("int64 4-d", lambda: np.random.default_rng(7).integers(-5, 5, size=(2, 3, 5, 7)), 8, 1),
    ("one byte", lambda: np.array([200], dtype=np.uint8), 1, 1),
    ("zeros", lambda: np.zeros((33, 17), dtype=np.uint16), 2, 1),
    ("random bytes", lambda: np.random.default_rng(8).integers(0, 256, size=5000, dtype=np.uint8), 1, 1),
]


@pytest.mark.parametrize("name,gen,E,S", CASES, ids=[c[0] for c in CASES])
def test_round_trip(name, gen, E, S):
    _check(gen(), E, S)


def test_coded_size_within_entropy_bound():
    # total stream bits <= sum of -log2(f/M) over all coded bytes + per chain the
    # final flush (at most 32 bits plus one partial word)
    a = synth.rowscaled(128, 512, 11)
    blob, b = _check(a, 2, 8)
    raw = _bytes_of(a)
    ctx = np.arange(len(raw)) % ta.n_contexts(2)
    f = b.tables.F[ctx, raw].astype(np.float64)
    ideal = float(np.sum(P - np.log2(f)))
    n_ch = b.n_tiles * b.S
    assert 16 * int(b.chain_lens.astype(np.int64).sum()) <= ideal + n_ch * 48
    # BF16 weights: the high byte (sign, exponent) is modelled, the low byte is close
    # to uniform, so the ratio sits well above 1 and below 2
    bits_per_elem = 8 * len(blob) / a.size
    assert 9.0 < bits_per_elem < 14.0


def test_uniform_tables_on_random_bytes():
    raw = np.random.default_rng(12).integers(0, 256, size=64 * 1024, dtype=np.uint8)
    blob, b = _check(raw, 1, 8)
    assert b.mask == 1 and (b.tables.F == M // 256).all()
    # a uniform table codes exactly 8 bits a byte: the words are the bytes plus at most
    # two words of state per chain
    n_ch = b.n_tiles * b.S
    words = int(b.chain_lens.astype(np.int64).sum())
    assert len(raw) // 2 - 2 * n_ch <= words <= len(raw) // 2 + 2 * n_ch


def test_mixed_tables():
    # int16 codes with a skewed high byte and a random low byte: context 1 coded,
    # context 0 uniform
    rng = np.random.default_rng(13)
    v = (rng.integers(0, 256, size=4096) | (rng.geometric(0.6, size=4096).clip(0, 255) << 8)).astype(np.uint16)
    blob, b = _check(v, 2, 1)
    assert b.mask == 0b01


def test_tile_independence():
    a = synth.rowscaled(64, 512, 14)        # 64 KB = 16 tiles
    raw = _bytes_of(a)
    blob = ta.compress(raw, 2, a.shape, 0, chains_per_tile=4)
    full, _ = ta.decode(blob)
    for tiles in ([0], [3, 7], [15], list(range(5, 11))):
        part, info = ta.decode(blob, tiles=tiles)
        sel = np.zeros(len(raw), dtype=bool)
        for t in tiles:
            sel[4096 * t: 4096 * (t + 1)] = True
        assert np.array_equal(part[sel], full[sel]) and not part[~sel].any()
        assert info["final_state_ok"]


def test_validation():
    with pytest.raises(ta.TileAnsError):
        ta.compress(np.zeros(10, np.uint8), 2, (4,))
    with pytest.raises(ta.TileAnsError):
        ta.compress(np.zeros(12, np.uint8), 3, (4,))
    blob = bytearray(ta.compress(np.arange(64, dtype=np.uint8), 1, (64,)))
    with pytest.raises(ta.TileAnsError):
        ta.parse(bytes(blob[:-2]))
    blob[0] = ord("X")
    with pytest.raises(ta.TileAnsError):
        ta.parse(bytes(blob))
