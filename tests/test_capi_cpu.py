"""CPU tests of the C ABI: every declared symbol is exported, the host encoder's
blobs are byte-identical to the oracle's, validation errors and blob parsing.

No GPU work is launched here (ep_compress / ep_serialize / ep_deserialize are host code).
"""
import os
import re

import numpy as np
import pytest

import synth
import oracle
from oracle import numerics as nx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

L = pytest.importorskip("decode_tile_rans_amd._lib")
if not os.path.exists(L.LIB_PATH):
    pytest.skip("libentropack_hip.so not built", allow_module_level=True)


def declared_symbols():
    txt = open(os.path.join(ROOT, "include", "entropack.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    lib = L.lib()
    names = declared_symbols()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES), set(names) ^ set(L.SIGNATURES)


def lib_blob(src, dt, t, S=0):
    src = np.ascontiguousarray(src)
    h = L.ep_compress(src.ctypes.data, dt, src.shape[0], src.shape[1], t, S)
    try:
        return L.ep_serialize(h), L.ep_actual_bpp(h)
    finally:
        L.ep_blob_free(h)


CASES = [
    ("small_gauss_3.5", lambda: synth.small_gauss(), nx.DT_BF16, 3.5, 0),
    ("odd_37x13", lambda: synth.rowscaled(37, 13, 5), nx.DT_BF16, 4.0, 0),
    ("r512_8", lambda: synth.rowscaled(512, 512, 70), nx.DT_BF16, 8.0, 0),
    ("r512_2.3", lambda: synth.rowscaled(512, 512, 30), nx.DT_BF16, 2.3, 0),
    ("r512_11", lambda: synth.rowscaled(256, 512, 31), nx.DT_BF16, 11.0, 0),
    ("S8", lambda: synth.rowscaled(300, 520, 32), nx.DT_BF16, 4.0, 8),
    ("S64", lambda: synth.rowscaled(200, 512, 33), nx.DT_BF16, 3.0, 64),
    ("S2", lambda: synth.rowscaled(129, 777, 34), nx.DT_BF16, 5.0, 2),
    ("fp16", lambda: synth.rowscaled_f32(96, 200, 4).astype(np.float16).view(np.uint16), nx.DT_FP16, 4.0, 0),
    ("fp32", lambda: synth.rowscaled_f32(64, 256, 4), nx.DT_FP32, 6.0, 0),
    ("fp8", lambda: synth.fp8_codes(128, 256, 4)[0], nx.DT_FP8, 5.0, 0),
    ("int8", lambda: synth.int8_codes(128, 256, 4)[0], nx.DT_INT8, 4.0, 0),
    ("zeros", lambda: np.zeros((40, 48), np.uint16), nx.DT_BF16, 2.0, 0),
    ("low", lambda: synth.rowscaled(64, 256, 9), nx.DT_BF16, 0.001, 0),
    ("1x1", lambda: synth.rowscaled(1, 1, 9), nx.DT_BF16, 4.0, 0),
]


@pytest.mark.parametrize("name,gen,dt,t,S", CASES, ids=[c[0] for c in CASES])
def test_encoder_byte_parity(name, gen, dt, t, S):
    src = gen()
    want = oracle.compress(src, dt, t, chains_per_tile=S or None)
    got, bpp = lib_blob(src, dt, t, S)
    assert got == want
    assert abs(bpp - 8.0 * len(want) / src.size) < 1e-12


def test_encoder_byte_parity_random_small():
    rng = np.random.default_rng(2024)
    for i in range(25):
        R = int(rng.integers(1, 90))
        C = int(rng.integers(1, 300))
        t = float(rng.choice([0.7, 1.0, 2.3, 3.5, 4.0, 6.0, 9.0]))
        S = int(rng.choice([0, 1, 2, 4, 8, 16]))
        src = synth.rowscaled(R, C, 500 + i, outlier_frac=0.01 if i % 3 == 0 else 0.0)
        assert lib_blob(src, nx.DT_BF16, t, S)[0] == oracle.compress(src, nx.DT_BF16, t, chains_per_tile=S or None), \
            (R, C, t, S)


@pytest.mark.slow
def test_encoder_byte_parity_config2():
    src = synth.rowscaled(3072, 3072, 2, 0.001)
    got, bpp = lib_blob(src, nx.DT_BF16, 4.0)
    assert got == oracle.compress(src, nx.DT_BF16, 4.0)
    assert 4.0 <= bpp <= 4.1


def test_validation_codes():
    src = np.ascontiguousarray(synth.small_gauss(8, 8))
    p = src.ctypes.data
    for t in (0.0005, 11.01, float("nan"), float("inf")):
        with pytest.raises(L.EPError) as e:
            L.ep_compress(p, nx.DT_BF16, 8, 8, t)
        assert e.value.name == "EP_E_RANGE"
    with pytest.raises(L.EPError) as e:
        L.ep_compress(p, 9, 8, 8, 4.0)
    assert e.value.name == "EP_E_DTYPE"
    with pytest.raises(L.EPError) as e:
        L.ep_compress(p, nx.DT_BF16, 0, 8, 4.0)
    assert e.value.name == "EP_E_ARG"
    with pytest.raises(L.EPError) as e:
        L.ep_compress(p, nx.DT_BF16, 8, 8, 4.0, 3)
    assert e.value.name == "EP_E_ARG"
    bad = src.copy()
    bad[3, 3] = 0x7F80   # +Inf
    with pytest.raises(L.EPError) as e:
        L.ep_compress(bad.ctypes.data, nx.DT_BF16, 8, 8, 4.0)
    assert e.value.name == "EP_E_NONFINITE"
    i8 = np.ones((4, 4), np.int8)
    with pytest.raises(L.EPError) as e:
        L.ep_compress(i8.ctypes.data, nx.DT_INT8, 4, 4, 8.5)
    assert e.value.name == "EP_E_RANGE"
    assert "target_bpp" in L.ep_last_error()


def test_serialize_deserialize_and_corruption():
    src = synth.small_gauss()
    blob, _ = lib_blob(src, nx.DT_BF16, 3.5)
    h = L.ep_deserialize(blob)
    assert L.ep_serialize(h) == blob
    assert L.ep_blob_shape(h) == (256, 256)
    assert L.ep_blob_dtype(h) == nx.DT_BF16
    S, k, flags = L.ep_blob_params(h)
    ob = oracle.parse_blob(blob)
    assert (S, k, flags) == (ob.S, ob.k, ob.flags)
    L.ep_blob_free(h)
    bad = [blob[:-2], b"XXXX" + blob[4:], blob + b"\0\0"]
    b2 = bytearray(blob)
    b2[44] = 1                              # reserved field
    bad.append(bytes(b2))
    b3 = bytearray(blob)
    off = 48 + 2 * 256 + ob.model_bytes.__len__()
    b3[off] ^= 2                            # block 0's offset no longer 0
    bad.append(bytes(b3))
    b4 = bytearray(blob)
    b4[48 + 1] |= 0x80                      # negative row scale
    bad.append(bytes(b4))
    for bb in bad:
        with pytest.raises(L.EPError) as e:
            L.ep_deserialize(bb)
        assert e.value.name == "EP_E_CORRUPT"
        with pytest.raises(ValueError):
            oracle.parse_blob(bb)


def _mutations(blob, rng, n):
    """n corrupted copies of blob: 1-4 random bytes changed, cut short or lengthened."""
    out = []
    for i in range(n):
        b = bytearray(blob)
        kind = i % 4
        if kind == 0:
            b = b[:int(rng.integers(0, len(b)))]
        elif kind == 1:
            b += bytes(rng.integers(0, 256, int(rng.integers(1, 64)), dtype=np.uint8))
        else:
            for _ in range(int(rng.integers(1, 5))):
                # bias toward the header and the model, where the parser makes most checks
                hi = len(b) if rng.random() < 0.3 else min(len(b), 48 + 4 * 256 + 1024)
                b[int(rng.integers(0, hi))] = int(rng.integers(0, 256))
        out.append(bytes(b))
    return out


def test_deserialize_random_corruptions():
    """The parser of untrusted bytes on corrupted blobs (lossy with and without escapes,
    TileANS): every copy is either refused as EP_E_CORRUPT or accepted, and an accepted
    copy serializes back to exactly its bytes.  (Run under ASan/UBSan by
    test_host_sanitizers.)"""
    rng = np.random.default_rng(11)
    blobs = [lib_blob(synth.small_gauss(), nx.DT_BF16, 3.5)[0],
             lib_blob(synth.rowscaled(64, 256, 31), nx.DT_BF16, 11.0)[0]]
    blobs.append(_lossless_blob(synth.rowscaled(64, 256, 5), 2)[0])
    accepted = 0
    for blob in blobs:
        for bb in _mutations(blob, rng, 400):
            try:
                h = L.ep_deserialize(bb)
            except L.EPError as e:
                assert e.name == "EP_E_CORRUPT", e
                continue
            try:
                assert L.ep_serialize(h) == bb
                assert np.isfinite(L.ep_actual_bpp(h))
                accepted += 1
            finally:
                L.ep_blob_free(h)
    assert accepted < 3 * 400


DIST_CASES = [c for c in CASES if c[0] in ("odd_37x13", "r512_8", "r512_2.3", "S8", "fp16", "fp32", "fp8", "int8",
                                           "zeros", "low", "1x1")]


@pytest.mark.parametrize("name,gen,dt,t,S", DIST_CASES, ids=[c[0] for c in DIST_CASES])
def test_encoder_distortion_matches_oracle(name, gen, dt, t, S):
    from oracle import plan
    src = np.ascontiguousarray(gen())
    h = L.ep_compress(src.ctypes.data, dt, src.shape[0], src.shape[1], t, S)
    try:
        e, r = L.ep_blob_distortion(h)
        blob = L.ep_serialize(h)
    finally:
        L.ep_blob_free(h)
    we, wr = plan.distortion(src, dt, blob)
    assert e == pytest.approx(we, rel=1e-12, abs=1e-300) and r == pytest.approx(wr, rel=1e-12, abs=1e-300)
    # a blob read back from bytes carries no source: the accessor says so
    h2 = L.ep_deserialize(blob)
    try:
        with pytest.raises(L.EPError) as ei:
            L.ep_blob_distortion(h2)
        assert ei.value.name == "EP_E_STATE"
    finally:
        L.ep_blob_free(h2)


def test_plan_bitrates_matches_oracle():
    from oracle import plan
    rng = np.random.default_rng(77)
    for it in range(60):
        n, m = int(rng.integers(1, 9)), int(rng.integers(1, 6))
        bits = np.sort(rng.uniform(1.0, 10.0, size=(n, m)), axis=1) * rng.integers(100, 10 ** 6, size=(n, 1))
        cost = np.sort(rng.uniform(0.0, 5.0, size=(n, m)), axis=1)[:, ::-1].copy()
        cost[rng.random((n, m)) < 0.15] *= 3.0
        if it % 5 == 0:                      # exact ties in bits and in cost
            bits = np.round(bits / 1000.0) * 1000.0
            cost = np.round(cost)
        lo = sum(float(v) for v in bits.min(axis=1))        # in matrix order, as both sides add
        hi = sum(float(v) for v in bits.max(axis=1))
        for budget in np.linspace(lo, hi * 1.05, 7):
            want = plan.plan(bits, cost, float(budget))
            assert L.ep_plan_bitrates(bits.tolist(), cost.tolist(), float(budget)) == want, (it, budget)
        with pytest.raises(L.EPError) as ei:
            L.ep_plan_bitrates(bits.tolist(), cost.tolist(), lo * 0.999 - 1.0)
        assert ei.value.name == "EP_E_RANGE"
    with pytest.raises(L.EPError) as ei:
        L.ep_plan_bitrates([[1.0, -2.0]], [[1.0, 0.5]], 10.0)
    assert ei.value.name == "EP_E_ARG"


def test_plan_bitrates_api_matches_oracle_pipeline():
    # the whole pipeline (compress at every candidate, measure, plan, recompress) against
    # the same steps done with the oracle encoder, bpp and distortion
    import torch
    from oracle import plan
    import decode_tile_rans_amd as ep
    from oracle.codec import actual_bpp
    mats = [synth.rowscaled(96, 256, 41), synth.rowscaled(64, 320, 42, outlier_frac=0.01),
            synth.rowscaled(128, 128, 43), synth.rowscaled(40, 200, 44)]
    # matrices of different norms (exact power-of-two scalings): the squared error of the
    # larger ones falls by more per bit, so they should get more bits
    mats = [synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(m) * np.float32(f)) for m, f in zip(mats, (1, 8, 0.125, 1))]
    cands = (2.0, 3.0, 4.0, 5.0)
    budget = 3.2
    got, targets = ep.plan_bitrates(mats, budget, cands, dtype=torch.bfloat16)
    bits = [[actual_bpp(oracle.compress(m, nx.DT_BF16, t)) * m.size for t in cands] for m in mats]
    cost = [[plan.distortion(m, nx.DT_BF16, oracle.compress(m, nx.DT_BF16, t))[0] for t in cands] for m in mats]
    want = plan.plan(np.array(bits), np.array(cost), budget * sum(m.size for m in mats))
    assert targets == [cands[j] for j in want]
    assert sum(c.actual_bpp * m.size for c, m in zip(got, mats)) <= budget * sum(m.size for m in mats)
    for c, m, j in zip(got, mats, want):
        assert c.to_bytes() == oracle.compress(m, nx.DT_BF16, cands[j])
    assert len(set(targets)) > 1            # the matrices differ enough to get different rates
    # uniform 3.0 fits the same budget; the plan does better on the summed error
    assert sum(cost[i][j] for i, j in enumerate(want)) < sum(cost[i][1] for i in range(len(mats)))


# ---------------------------------------------------------------- TileANS (lossless)
def _lossless_blob(a, E, S=0, tag=7):
    raw = np.frombuffer(np.ascontiguousarray(a).tobytes(), dtype=np.uint8).copy()
    h = L.ep_compress_lossless(raw.ctypes.data, len(raw), E, a.shape, tag, S)
    try:
        return L.ep_serialize(h), L.ep_actual_bpp(h), L.ep_blob_kind(h), L.ep_blob_dims(h), L.ep_blob_dtype(h), \
            L.ep_blob_elem_bytes(h), L.ep_blob_shape(h)
    finally:
        L.ep_blob_free(h)


TA_CASES = [
    ("bf16", lambda: synth.rowscaled(96, 200, 1), 2, 0),
    ("bf16 S8", lambda: synth.rowscaled(64, 1024, 2), 2, 8),
    ("fp32 3-d", lambda: synth.rowscaled_f32(8, 24, 3).reshape(2, 4, 24), 4, 2),
    ("fp16 1-d ragged", lambda: synth.rowscaled_f32(1, 1001, 4).astype(np.float16).reshape(-1), 2, 1),
    ("fp8", lambda: synth.fp8_codes(64, 136, 5)[0], 1, 4),
    ("int8 S64", lambda: synth.int8_codes(32, 520, 6)[0], 1, 64),
    ("int64 4-d", lambda: np.random.default_rng(7).integers(-5, 5, size=(2, 3, 5, 7)), 8, 0),
    ("one byte", lambda: np.array([200], dtype=np.uint8), 1, 0),
    ("zeros", lambda: np.zeros((33, 17), dtype=np.uint16), 2, 0),
    ("random", lambda: np.random.default_rng(8).integers(0, 256, size=5000, dtype=np.uint8), 1, 0),
    ("bf16 4 MiB", lambda: synth.rowscaled(1024, 2048, 9), 2, 0),
]


@pytest.mark.parametrize("name,gen,E,S", TA_CASES, ids=[c[0] for c in TA_CASES])
def test_tileans_byte_parity(name, gen, E, S):
    from oracle import tileans
    a = gen()
    got, bpp, kind, dims, tag, eb, shape = _lossless_blob(a, E, S)
    raw = np.frombuffer(np.ascontiguousarray(a).tobytes(), dtype=np.uint8)
    want = tileans.compress(raw, E, a.shape, 7, chains_per_tile=S or None)
    assert got == want
    assert kind == 1 and dims == tuple(a.shape) and tag == 7 and eb == E and shape == (1, a.size)
    assert abs(bpp - 8.0 * len(want) / a.size) < 1e-12
    h = L.ep_deserialize(got)          # read back: same accessors
    try:
        assert L.ep_blob_kind(h) == 1 and L.ep_blob_dims(h) == tuple(a.shape)
    finally:
        L.ep_blob_free(h)


def test_tileans_validation():
    from oracle import tileans
    raw = np.zeros(64, np.uint8)
    for args, code in [((raw.ctypes.data, 64, 3, (64,)), "EP_E_ARG"), ((raw.ctypes.data, 60, 2, (32,)), "EP_E_SHAPE"),
                       ((raw.ctypes.data, 64, 1, (0, 64)), "EP_E_SHAPE"), ((raw.ctypes.data, 64, 1, (64,), 300), "EP_E_ARG")]:
        with pytest.raises(L.EPError) as ei:
            L.ep_compress_lossless(*args)
        assert ei.value.name == code, args
    blob = bytearray(tileans.compress(np.arange(4096, dtype=np.uint16), 2, (4096,)))
    for cut in (len(blob) - 2, 40, 60):
        with pytest.raises(L.EPError) as ei:
            L.ep_deserialize(bytes(blob[:cut]))
        assert ei.value.name == "EP_E_CORRUPT"
    bad = bytearray(blob)
    bad[48 + 8 + 5] ^= 0x40            # a table entry: the table no longer sums to 2048
    with pytest.raises(L.EPError) as ei:
        L.ep_deserialize(bytes(bad))
    assert ei.value.name == "EP_E_CORRUPT"
    # lossy-only calls refuse a lossless blob
    h = L.ep_deserialize(bytes(blob))
    try:
        with pytest.raises(L.EPError):
            L.ep_blob_distortion(h)
    finally:
        L.ep_blob_free(h)


def test_device_entries_refuse_blobs_not_uploaded():
    """The decode and fused-product entries check the blob's device copy first, so a blob
    never uploaded is refused (EP_E_STATE) before any device call."""
    if not hasattr(L.lib(), "ep_compressed_linear_prefill"):
        pytest.skip("host-only build: no device entry points")
    src = np.ascontiguousarray(synth.rowscaled(64, 4096, 31))
    h = L.ep_compress(src.ctypes.data, nx.DT_BF16, 64, 4096, 4.0, 8)
    try:
        for call in (lambda: L.ep_compressed_linear_prefill(h, 16, 16, 0, 16),
                     lambda: L.ep_decompress(h, 16),
                     lambda: L.ep_test_decode_coords(h, 16)):
            with pytest.raises(L.EPError) as e:
                call()
            assert e.value.name == "EP_E_STATE"
    finally:
        L.ep_blob_free(h)
