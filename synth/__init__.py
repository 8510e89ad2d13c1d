"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws numbers and rounds them to the input container
(BF16 / FP8-E4M3FN / INT8 bit patterns).  It holds none of the compression
method's arithmetic: no row scales, no lattice, no entropy coding.

Workloads (all seeded, all synthetic; the trained diffusion-transformer
weights the EntroPack pages measure on are not available here):

* ``small_gauss``     256 x 256 BF16, 0.02 * N(0,1), seed 0            (target 3.5 bpp)
* ``rowscaled``       R x C BF16, per-row scale s_r = exp(ln 0.02 + 0.5 z_r),
                      w = s_r * N(0,1); optionally a fraction of entries replaced by
                      +-10 s_r outliers (drawn without replacement, fair sign)
* ``dit_stack``       276 matrices shaped like a 30-block DiT (3840 wide) + 6 extras
* ``fp8_codes`` / ``int8_codes``  per-row absmax code tensors of a rowscaled matrix
* ``activations``     T x C BF16, N(0,1)

Draw order inside one matrix: row scales, then entries, then outlier positions,
then outlier signs.  NumPy PCG64 (``numpy.random.default_rng``) everywhere, except
``dit_stack_torch`` which draws on the GPU with torch's Philox generator so the
6.28 G-parameter stack can be produced in seconds.
"""
from __future__ import annotations

import math
import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "small_gauss", "rowscaled",
    "dit_stack_shapes", "fp8_codes", "int8_codes", "activations",
    "dit_stack_torch", "DT_BF16", "DT_FP16", "DT_FP32", "DT_FP8", "DT_INT8",
]

# container ids (same numbering as the C ABI's ep_dtype)
DT_BF16, DT_FP16, DT_FP32, DT_FP8, DT_INT8 = 1, 2, 3, 4, 5


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (round-to-nearest-even); returns uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def small_gauss(rows: int = 256, cols: int = 256, seed: int = 0, std: float = 0.02) -> np.ndarray:
    """i.i.d. N(0, std^2) BF16 matrix (uint16 bit patterns)."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((rows, cols)) * std).astype(np.float32)
    return f32_to_bf16_bits(w)


def rowscaled_f32(rows: int, cols: int, seed: int, outlier_frac: float = 0.0) -> np.ndarray:
    """Log-normal row scales times N(0,1) entries, optional +-10 s_r outliers (float32)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(rows)
    s = np.exp(math.log(0.02) + 0.5 * z)
    w = s[:, None] * rng.standard_normal((rows, cols))
    n_out = int(round(outlier_frac * rows * cols))
    if n_out:
        pos = rng.choice(rows * cols, size=n_out, replace=False)
        sign = rng.integers(0, 2, size=n_out) * 2 - 1
        w.reshape(-1)[pos] = sign * 10.0 * s[pos // cols]
    return w.astype(np.float32)


def rowscaled_row_outliers(rows: int, cols: int, seed: int, every: int = 4, first: int = 1,
                           mult: float = 12.0) -> np.ndarray:
    """BF16 bit patterns of :func:`rowscaled_f32` with one +-mult x s_r entry in each of
    rows first, first + every, ... (random column and sign; s_r the row's scale)."""
    w = rowscaled_f32(rows, cols, seed)
    rng = np.random.default_rng(seed + 7919)
    r = np.arange(first, rows, every)
    c = rng.integers(0, cols, r.size)
    rms = np.sqrt((w[r].astype(np.float64) ** 2).mean(axis=1))
    w[r, c] = (mult * rms * np.where(rng.random(r.size) < 0.5, -1.0, 1.0)).astype(np.float32)
    return f32_to_bf16_bits(w)


def rowscaled(rows: int, cols: int, seed: int, outlier_frac: float = 0.0) -> np.ndarray:
    """BF16 bit patterns of :func:`rowscaled_f32`."""
    return f32_to_bf16_bits(rowscaled_f32(rows, cols, seed, outlier_frac))


def dit_stack_shapes():
    """(rows, cols, seed) of the 276-matrix DiT-shaped stack.

    30 blocks x {q, k, v, o: 3840x3840; w1, w3: 10240x3840; w2: 3840x10240;
    mod1, mod2: 3840x3840} followed by 6 extra 3840x3840 matrices; matrix i
    uses seed 3000 + i.  Also returns the block index (30 = the extras).
    """
    d, h = 3840, 10240
    block = [(d, d), (d, d), (d, d), (d, d), (h, d), (h, d), (d, h), (d, d), (d, d)]
    out = []
    i = 0
    for b in range(30):
        for (r, c) in block:
            out.append((r, c, 3000 + i, b))
            i += 1
    for _ in range(6):
        out.append((d, d, 3000 + i, 30))
        i += 1
    return out


def _fp8_e4m3fn_bits_torch(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def fp8_codes(rows: int, cols: int, seed: int):
    """Per-row absmax FP8-E4M3FN codes of a rowscaled matrix.

    a_r = max|w_r| / 448, codes = E4M3FN(w / a_r) (torch's round-to-nearest-even
    cast).  Returns (uint8 code bits, float32 per-row scales a_r).
    """
    w = rowscaled_f32(rows, cols, seed)
    a = (np.abs(w).max(axis=1) / np.float32(448.0)).astype(np.float32)
    a[a == 0] = 1.0
    q = (w / a[:, None]).astype(np.float32)
    q = np.clip(q, -448.0, 448.0)
    return _fp8_e4m3fn_bits_torch(q), a


def int8_codes(rows: int, cols: int, seed: int):
    """Per-row absmax INT8 codes: a_r = max|w_r|/127, codes = clamp(rint(w/a_r), +-127)."""
    w = rowscaled_f32(rows, cols, seed)
    a = (np.abs(w).max(axis=1) / np.float32(127.0)).astype(np.float32)
    a[a == 0] = 1.0
    q = np.clip(np.rint(w / a[:, None]), -127, 127).astype(np.int8)
    return q, a


def activations(tokens: int, cols: int, seed: int) -> np.ndarray:
    """N(0,1) activations rounded to BF16 (uint16 bits)."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal((tokens, cols)).astype(np.float32))


def dit_stack_torch(index: int, device="cuda"):
    """Matrix ``index`` of the DiT stack drawn on the GPU (torch Philox, seed 3000+index).

    Same distribution as :func:`rowscaled` (log-normal row scales, N(0,1)
    entries, no outliers) but a different generator, so the whole stack can be
    drawn in seconds.  Returns a BF16 torch tensor on ``device``.
    """
    import torch
    r, c, seed, _ = dit_stack_shapes()[index]
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = torch.randn(r, 1, generator=g, device=device, dtype=torch.float32)
    s = torch.exp(math.log(0.02) + 0.5 * z)
    w = torch.randn(r, c, generator=g, device=device, dtype=torch.float32) * s
    return w.to(torch.bfloat16)
