"""Compress / decode and the blob v1 byte layout (oracle).

[README] quick start: ``compress(tensor, config)`` / ``decompress`` restore
shape and dtype; ``target_bpp`` is finite in [0.001, 11] and may be
non-integer; ``actual_bpp`` includes the metadata.  [NEWS]: lossy mode is for
2-D floating and integer tensors only.  [ABS]/[SUM]: tiles are independently
decodable and rANS-coded.

Blob v1 (little-endian, packed, this project's format):

  header (48 B)   'EPK1' | u16 version=1 | u8 dtype | u8 P=11 | u8 S | u8 k |
                  u8 flags (bit0: some escape, bit1: some value needs clamping)
                  | u8 tile_log2=12 | u32 R | u32 C | f32 delta | u32 n_tiles |
                  u32 n_blocks | u64 n_words | u32 model_bytes | u32 0
  row scales      bf16[R]
  model           model_bytes (bit-packed coset weight + magnitude frequencies)
  checkpoints     u32[n_blocks]   word offset of each block of 64 chains
  region lengths  u16[ceil(n_chains/2)]  (even; chains 2i / 2i+1 share a region)
  states          u32[n_chains]
  stream          u16[n_words]

Groups: row-major 8-wide column groups (columns padded with zeros to a
multiple of 8; padded coordinates are coded and dropped).  Tile t holds
groups [512 t, 512 t + 512) (4096 coordinates); chain j of tile t decodes
its local groups j, j + S, j + 2S, ...  Chains are numbered t*S + j.  Chain
2i reads its words forward from the region start, chain 2i+1 backward from
the region end; one zero word separates them when their total is odd.

actual_bpp = 8 * len(blob) / (R * C).

Reconstruction: w_hat = fl32(h_r * fl32(u)), h_r = fl32(s_r * delta), then
the container cast of ``numerics``.
"""
from __future__ import annotations

import math
import struct
from dataclasses import dataclass

import numpy as np

from . import numerics as nx
from .model import Model, group_symbols, count_symbols, build_model, n_msym
from .rans import encode_chains, decode_chains, WordReader, L
from .rate import row_scales_bf16, half_steps, quantize_rows, select_delta

MAGIC = b"EPK1"
VERSION = 1
HEADER = struct.Struct("<4sHBBBBBBIIfIIQII")
assert HEADER.size == 48
TILE_LOG2 = 12
TILE_GROUPS = 512
BLOCK_CHAINS = 64
FLAG_ESC = 1
FLAG_SAT = 2


class CompressError(ValueError):
    def __init__(self, code, msg):
        super().__init__(msg)
        self.code = code


def default_chains_per_tile(n: int) -> int:
    return 8 if n >= (1 << 22) else 1


def validate(shape, dtype, target_bpp):
    if len(shape) != 2:
        raise CompressError("shape", "lossy compression takes 2-D tensors only")
    R, C = shape
    if R < 1 or C < 1:
        raise CompressError("arg", "rows and cols must be >= 1")
    if dtype not in nx.DTYPES:
        raise CompressError("dtype", "unsupported dtype")
    t = float(target_bpp)
    if not math.isfinite(t) or t < 0.001 or t > 11.0:
        raise CompressError("range", "target_bpp must be finite and in [0.001, 11]")
    if dtype in (nx.DT_FP8, nx.DT_INT8) and t > 8.0:
        raise CompressError("range", "target_bpp above 8 for an 8-bit container")


def chain_layout(n_groups: int, S: int):
    """(n_tiles, chain_groups (n_chains, steps) of global group ids, -1 padded)."""
    n_tiles = max(1, -(-n_groups // TILE_GROUPS))
    steps = TILE_GROUPS // S
    n_ch = n_tiles * S
    ch = np.arange(n_ch)
    t, j = ch // S, ch % S
    k = np.arange(steps)
    local = j[:, None] + S * k[None, :]
    g = TILE_GROUPS * t[:, None] + local
    g = np.where(g < n_groups, g, -1)
    return n_tiles, g


@dataclass
class Blob:
    dtype: int
    S: int
    k: int
    flags: int
    R: int
    C: int
    delta: np.float32
    n_tiles: int
    s_bits: np.ndarray
    model: Model
    model_bytes: bytes
    checkpoints: np.ndarray
    region_len: np.ndarray
    states: np.ndarray
    stream: np.ndarray

    @property
    def n_chains(self):
        return self.n_tiles * self.S

    @property
    def n_blocks(self):
        return -(-self.n_chains // BLOCK_CHAINS)

    def to_bytes(self) -> bytes:
        hdr = HEADER.pack(MAGIC, VERSION, self.dtype, 11, self.S, self.k, self.flags, TILE_LOG2,
                          self.R, self.C, float(self.delta), self.n_tiles, self.n_blocks,
                          len(self.stream), len(self.model_bytes), 0)
        return b"".join([hdr, self.s_bits.astype("<u2").tobytes(), self.model_bytes,
                         self.checkpoints.astype("<u4").tobytes(), self.region_len.astype("<u2").tobytes(),
                         self.states.astype("<u4").tobytes(), self.stream.astype("<u2").tobytes()])


def _layout_regions(words, n_ch):
    """Paired regions: returns (region_len u16[], stream u16[], checkpoints u32[])."""
    n_reg = -(-n_ch // 2)
    parts = []
    rl = np.zeros(n_reg, dtype=np.int64)
    for r in range(n_reg):
        a = words[2 * r]
        b = words[2 * r + 1] if 2 * r + 1 < n_ch else np.zeros(0, np.uint16)
        pad = (len(a) + len(b)) & 1
        parts.append(a)
        if pad:
            parts.append(np.zeros(1, np.uint16))
        parts.append(b[::-1])
        rl[r] = len(a) + len(b) + pad
    assert (rl <= 0xFFFF).all()
    stream = np.concatenate(parts) if parts else np.zeros(0, np.uint16)
    starts = np.concatenate([[0], np.cumsum(rl)[:-1]]) if n_reg else np.zeros(0, np.int64)
    n_blocks = -(-n_ch // BLOCK_CHAINS)
    ck = starts[np.arange(n_blocks) * (BLOCK_CHAINS // 2)] if n_reg else np.zeros(n_blocks, np.int64)
    return rl.astype(np.uint16), stream.astype(np.uint16), ck.astype(np.uint32)


def compress(src, dtype: int, target_bpp: float, chains_per_tile=None, trace=None) -> bytes:
    """Compress a 2-D container array (BF16/FP8 as bit patterns) to blob v1 bytes."""
    src = np.asarray(src)
    validate(src.shape, dtype, target_bpp)
    R, C = src.shape
    w = nx.source_to_f64(src, dtype)
    if not np.isfinite(w).all():
        raise CompressError("nonfinite", "input holds NaN or Inf")
    s_bits = row_scales_bf16(w)
    s = nx.bf16_bits_to_f32(s_bits)
    live = (w != 0).any(axis=1)
    s_exp = (s_bits.astype(np.int64) >> 7) & 0xFF
    if (live & (s_exp == 0)).any():
        raise CompressError("range", "a nonzero row has an RMS below the BF16 normal range")
    G = -(-C // 8)
    wp = np.zeros((R, G * 8), dtype=np.float64)
    wp[:, :C] = w
    delta, k, _est, _ns = select_delta(w, wp, s_bits, float(target_bpp), trace=trace)
    h = half_steps(s_bits, delta)
    u = quantize_rows(wp, h)                       # (R*G, 8)
    sym = group_symbols(u, k)
    cc, m0, m1 = count_symbols(sym, n_msym(k))
    model = build_model(k, cc, m0, m1)
    n_groups = R * G
    S = chains_per_tile or default_chains_per_tile(R * C)
    assert S in (1, 2, 4, 8, 16, 32, 64)
    n_tiles, cg = chain_layout(n_groups, S)
    states, words = encode_chains(sym, model, cg)
    rl, stream, ck = _layout_regions(words, n_tiles * S)
    flags = 0
    if (sym["msym"] >= (1 << k)).any():
        flags |= FLAG_ESC
    wh = reconstruct_f32(u.reshape(R, G * 8)[:, :C], h)
    if nx.needs_saturation(wh, dtype):
        flags |= FLAG_SAT
    blob = Blob(dtype, S, k, flags, R, C, np.float32(delta), n_tiles, s_bits, model, model.to_bytes(),
                ck, rl, states, stream)
    return blob.to_bytes()


def parse_blob(buf: bytes) -> Blob:
    if len(buf) < HEADER.size:
        raise ValueError("blob truncated")
    (magic, ver, dtype, p, S, k, flags, tl, R, C, delta, n_tiles, n_blocks, n_words, mb, z) = \
        HEADER.unpack_from(buf, 0)
    if magic != MAGIC or ver != VERSION or p != 11 or tl != TILE_LOG2 or z != 0:
        raise ValueError("bad header")
    if dtype not in nx.DTYPES or S not in (1, 2, 4, 8, 16, 32, 64) or not (3 <= k <= 7) or flags > 3:
        raise ValueError("bad header fields")
    if R < 1 or C < 1:
        raise ValueError("bad shape")
    n_groups = R * (-(-C // 8))
    if n_tiles != max(1, -(-n_groups // TILE_GROUPS)):
        raise ValueError("bad tile count")
    n_ch = n_tiles * S
    if n_blocks != -(-n_ch // BLOCK_CHAINS):
        raise ValueError("bad block count")
    n_reg = -(-n_ch // 2)
    off = HEADER.size
    need = off + 2 * R + mb + 4 * n_blocks + 2 * n_reg + 4 * n_ch + 2 * n_words
    if len(buf) != need:
        raise ValueError("blob size mismatch")
    s_bits = np.frombuffer(buf, "<u2", R, off).copy(); off += 2 * R
    if ((s_bits & 0x8000) != 0).any() or (((s_bits >> 7) & 0xFF) == 0xFF).any():
        raise ValueError("bad row scale")
    mbytes = bytes(buf[off:off + mb]); off += mb
    model = Model.from_bytes(mbytes, k)
    ck = np.frombuffer(buf, "<u4", n_blocks, off).copy(); off += 4 * n_blocks
    rl = np.frombuffer(buf, "<u2", n_reg, off).copy(); off += 2 * n_reg
    st = np.frombuffer(buf, "<u4", n_ch, off).copy(); off += 4 * n_ch
    stream = np.frombuffer(buf, "<u2", n_words, off).copy()
    if (rl & 1).any():
        raise ValueError("odd region length")
    starts = np.concatenate([[0], np.cumsum(rl.astype(np.int64))[:-1]])
    if int(rl.astype(np.int64).sum()) != n_words:
        raise ValueError("region lengths do not cover the stream")
    if not np.array_equal(ck.astype(np.int64), starts[np.arange(n_blocks) * (BLOCK_CHAINS // 2)]):
        raise ValueError("checkpoints inconsistent")
    if (st < L).any():
        raise ValueError("state below L")
    return Blob(dtype, S, k, flags, R, C, np.float32(delta), n_tiles, s_bits, model, mbytes, ck, rl, st, stream)


def reconstruct_f32(u: np.ndarray, h: np.ndarray) -> np.ndarray:
    """w_hat = fl32(h_r * fl32(u))."""
    return (h[:, None] * np.asarray(u).astype(np.float32)).astype(np.float32)


def chain_readers(b: Blob):
    n_ch = b.n_chains
    rl = b.region_len.astype(np.int64)
    starts = np.concatenate([[0], np.cumsum(rl)[:-1]])
    ch = np.arange(n_ch)
    r = ch // 2
    fwd = (ch % 2) == 0
    start = np.where(fwd, starts[r], starts[r] + rl[r] - 1)
    step = np.where(fwd, 1, -1)
    lo = starts[r]
    hi = starts[r] + rl[r]
    return WordReader(b.stream, start, step, lo, hi)


def decode(buf, tiles=None):
    """Decode a blob.  Returns (u int32 (R, C) doubled coordinates, container array (R, C), info).

    ``tiles`` restricts decoding to an iterable of tile indices (other
    outputs stay zero): the tile-independence property.
    """
    b = parse_blob(buf) if not isinstance(buf, Blob) else buf
    R, C = b.R, b.C
    G = -(-C // 8)
    n_groups = R * G
    n_tiles, cg = chain_layout(n_groups, b.S)
    reader = chain_readers(b)
    if tiles is not None:
        keep = np.zeros(n_tiles, dtype=bool)
        keep[np.asarray(list(tiles), dtype=np.int64)] = True
        chain_keep = np.repeat(keep, b.S)
        cg = np.where(chain_keep[:, None], cg, -1)
    u, xend = decode_chains(b.model, b.states, cg, reader, n_groups)
    active = (cg >= 0).any(axis=1)
    ok_state = bool((xend[active] == L).all())
    ok_reads = not bool(reader.overrun.any())
    u = u.reshape(R, G * 8)[:, :C]
    h = half_steps(b.s_bits, b.delta)
    wh = reconstruct_f32(u, h)
    out = nx.cast_container(wh, b.dtype)
    info = dict(final_state_ok=ok_state, reads_in_bounds=ok_reads, S=b.S, k=b.k, flags=b.flags,
                actual_bpp=8.0 * (len(buf) if not isinstance(buf, Blob) else len(b.to_bytes())) / (R * C))
    return u.astype(np.int32), out, info


def actual_bpp(buf: bytes) -> float:
    b = parse_blob(buf)
    return 8.0 * len(buf) / (b.R * b.C)
