"""Container conversions for the oracle (IEEE-754 / OCP FP8 definitions).

[ABS]: the method supports floating-point and integer weight containers such as
BF16, FP16, FP8 and INT8, with storage bitrate independent of numerical
precision.  [NEWS]: decompression restores the original dtype.

Reading taken (pages silent): every float container is written with
round-to-nearest-even after clamping to the container's largest finite value
("saturating"), INT8 with round-half-even to integer and clamp to [-128, 127],
FP32 unchanged.  So decoding never produces Inf/NaN from a valid blob.

Pins (tests): BF16 and FP16 against torch's CPU casts inside the range, FP8
against the OCP E4M3FN value table enumerated from its definition and against
torch's CPU float8 cast, INT8 against Python's round().
"""
from __future__ import annotations

import numpy as np

DT_BF16, DT_FP16, DT_FP32, DT_FP8, DT_INT8 = 1, 2, 3, 4, 5
DTYPES = (DT_BF16, DT_FP16, DT_FP32, DT_FP8, DT_INT8)
ELEM_BYTES = {DT_BF16: 2, DT_FP16: 2, DT_FP32: 4, DT_FP8: 1, DT_INT8: 1}

BF16_MAX = float(np.uint32(0x7F7F0000).view(np.float32))
FP16_MAX = 65504.0
FP8_MAX = 448.0


# ---------------------------------------------------------------- decode inputs
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp8_e4m3fn_to_f64(bits: np.ndarray) -> np.ndarray:
    """OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; S.1111.111 is NaN."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & ((b & 7) == 7), np.nan, val)
    return s * val


def source_to_f64(src, dtype: int) -> np.ndarray:
    """Raw container values (bit patterns for BF16/FP8) -> float64."""
    if dtype == DT_BF16:
        return bf16_to_f64(src)
    if dtype == DT_FP16:
        return np.asarray(src).view(np.float16).astype(np.float64) if np.asarray(src).dtype == np.uint16 \
            else np.asarray(src, dtype=np.float16).astype(np.float64)
    if dtype == DT_FP32:
        return np.asarray(src, dtype=np.float32).astype(np.float64)
    if dtype == DT_FP8:
        return fp8_e4m3fn_to_f64(src)
    if dtype == DT_INT8:
        return np.asarray(src, dtype=np.int8).astype(np.float64)
    raise ValueError("unsupported dtype")


# ---------------------------------------------------------------- float32 -> BF16
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to BF16, nearest-even (plain bit definition)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    return ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- container casts
def cast_bf16_sat(x32: np.ndarray) -> np.ndarray:
    x = np.clip(np.asarray(x32, dtype=np.float32), np.float32(-BF16_MAX), np.float32(BF16_MAX))
    return f32_to_bf16_bits(x)


def cast_fp16_sat(x32: np.ndarray) -> np.ndarray:
    x = np.clip(np.asarray(x32, dtype=np.float32), np.float32(-FP16_MAX), np.float32(FP16_MAX))
    return x.astype(np.float16).view(np.uint16)


def cast_fp8_sat(x32: np.ndarray) -> np.ndarray:
    """float32 -> OCP E4M3FN bits, nearest-even, clamped to +-448 first.

    Normal numbers: value = 2^e (1 + n/8), e in [-6, 8]; subnormals:
    value = n 2^-9, n in [0, 8).  Rounding is done on the exact scaled value
    (scaling by powers of two is exact in float64), ties to even.
    """
    x = np.clip(np.asarray(x32, dtype=np.float32).astype(np.float64), -FP8_MAX, FP8_MAX)
    sign = (x < 0) | ((x == 0) & np.signbit(x))
    a = np.abs(x)
    out = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: units of 2^-9; n == 8 lands exactly on the first normal (bits 0x08)
    out[sub] = np.rint(a[sub] * 512.0).astype(np.int64)
    nrm = ~sub
    mnt, ex = np.frexp(a[nrm])           # a = mnt * 2^ex, mnt in [0.5, 1)
    e = ex.astype(np.int64) - 1          # a = (2 mnt) 2^e, 2 mnt in [1, 2)
    n = np.rint((2.0 * mnt - 1.0) * 8.0).astype(np.int64)
    carry = n == 8
    e = np.where(carry, e + 1, e)
    n = np.where(carry, 0, n)
    out[nrm] = ((e + 7) << 3) | n
    out = out | np.where(sign, 0x80, 0)
    return out.astype(np.uint8)


def cast_int8_sat(x32: np.ndarray) -> np.ndarray:
    x = np.rint(np.asarray(x32, dtype=np.float32).astype(np.float64))
    return np.clip(x, -128, 127).astype(np.int8)


def cast_container(x32: np.ndarray, dtype: int) -> np.ndarray:
    """Write reconstructed float32 weights into the container (raw element bits)."""
    if dtype == DT_BF16:
        return cast_bf16_sat(x32)
    if dtype == DT_FP16:
        return cast_fp16_sat(x32)
    if dtype == DT_FP32:
        return np.asarray(x32, dtype=np.float32).copy()
    if dtype == DT_FP8:
        return cast_fp8_sat(x32)
    if dtype == DT_INT8:
        return cast_int8_sat(x32)
    raise ValueError("unsupported dtype")


def container_max(dtype: int) -> float:
    return {DT_BF16: BF16_MAX, DT_FP16: FP16_MAX, DT_FP8: FP8_MAX,
            DT_INT8: 127.0, DT_FP32: float(np.finfo(np.float32).max)}[dtype]


def needs_saturation(x32: np.ndarray, dtype: int) -> bool:
    """True if the plain (non-clamping) cast of some value would leave the container range."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    if x.size == 0:
        return False
    if dtype == DT_INT8:
        r = np.rint(x)
        return bool((r > 127).any() or (r < -128).any())
    if dtype == DT_FP32:
        return False
    return bool((np.abs(x) > container_max(dtype)).any())
