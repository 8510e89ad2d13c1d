"""Compress / decode and the blob v3 byte layout (oracle).

[README] quick start: ``compress(tensor, config)`` / ``decompress`` restore
shape and dtype; ``target_bpp`` is finite in [0.001, 11] and may be
non-integer; ``actual_bpp`` includes the metadata.  [NEWS]: lossy mode is for
2-D floating and integer tensors only.  [ABS]/[SUM]: tiles are independently
decodable and rANS-coded.

Blob v3 (little-endian, packed, this project's format):

  header (48 B)   'EPK1' | u16 version=3 | u8 dtype | u8 P | u8 S | u8 k |
                  u8 flags (bit0: some escape, bit1: some value needs clamping)
                  | u8 tile_log2=12 | u32 R | u32 C | f32 delta | u32 n_tiles |
                  u32 n_blocks | u64 n_words | u32 model_bytes | u32 0
  row scales      bf16[R]
  model           model_bytes (bit-packed coset weight + magnitude frequencies)
  block offsets   u32[n_blocks]  start of each block's area, in 8-word chunks
  full chunks     u8[n_chains] if S >= 8 else u16[n_chains]: len // 8 per chain
  tail lengths    u8[ceil(n_chains / 2)]: len % 8 of chain 2i (low nibble) and
                  2i + 1 (high nibble)
  states          u32[n_chains]
  stream          u16[n_words]   the block areas, back to back (``layout``)

Groups: row-major 8-wide column groups (columns padded with zeros to a
multiple of 8; padded coordinates are coded and dropped).  Tile t holds
groups [512 t, 512 t + 512) (4096 coordinates); chain j of tile t decodes
its local groups j, j + S, j + 2S, ...  Chains are numbered t*S + j; a block
is 64 consecutive chains (n_blocks = ceil(n_chains / 64)).  A tile's area
holds its tiles' chains' words: 8-word chunks in the order a reader with a
32-word window per chain requests them, then the short tails (``layout``).

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
from .model import Model, group_symbols, count_symbols, build_model, n_msym, precision
from .rans import encode_chains, ChainDecoder, L
from .layout import CHUNK, TileSchedule, request_ranks, block_geometry, build_stream
from .rate import row_scales_bf16, half_steps, quantize_rows, select_delta

MAGIC = b"EPK1"
VERSION = 3
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
    block_offsets: np.ndarray
    chain_lens: np.ndarray
    states: np.ndarray
    stream: np.ndarray

    @property
    def n_chains(self):
        return self.n_tiles * self.S

    @property
    def n_blocks(self):
        return -(-self.n_chains // BLOCK_CHAINS)

    def to_bytes(self) -> bytes:
        hdr = HEADER.pack(MAGIC, VERSION, self.dtype, precision(self.k), self.S, self.k, self.flags, TILE_LOG2,
                          self.R, self.C, float(self.delta), self.n_tiles, self.n_blocks,
                          len(self.stream), len(self.model_bytes), 0)
        lens = self.chain_lens.astype(np.int64)
        full = (lens // CHUNK).astype("<u1" if self.S >= 8 else "<u2")
        tails = np.zeros(2 * (-(-len(lens) // 2)), dtype=np.int64)
        tails[:len(lens)] = lens % CHUNK
        nib = (tails[0::2] | (tails[1::2] << 4)).astype("<u1")
        return b"".join([hdr, self.s_bits.astype("<u2").tobytes(), self.model_bytes,
                         self.block_offsets.astype("<u4").tobytes(), full.tobytes(), nib.tobytes(),
                         self.states.astype("<u4").tobytes(), self.stream.astype("<u2").tobytes()])


def chain_group_counts(n_groups: int, S: int, n_tiles: int):
    """Groups decoded by each chain, shaped (n_tiles, S)."""
    t = np.arange(n_tiles)[:, None]
    j = np.arange(S)[None, :]
    gt = np.minimum(n_groups - TILE_GROUPS * t, TILE_GROUPS)
    return np.where(gt > j, (gt - j + S - 1) // S, 0)


def compress(src, dtype: int, target_bpp: float, chains_per_tile=None, trace=None) -> bytes:
    """Compress a 2-D container array (BF16/FP8 as bit patterns) to blob v3 bytes."""
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
    states, words, cons = encode_chains(sym, model, cg)
    lens = np.array([len(w) for w in words], dtype=np.int64).reshape(n_tiles, S)
    assert (lens // CHUNK <= (0xFF if S >= 8 else 0xFFFF)).all()
    flags = 0
    if (sym["msym"] >= (1 << k)).any():
        flags |= FLAG_ESC
    ngr = chain_group_counts(n_groups, S, n_tiles)
    steps = cg.shape[1]
    rank = request_ranks(lens, ngr, cons.reshape(n_tiles, S, steps), esc=bool(flags & FLAG_ESC))
    offsets, stream = build_stream(words, lens.reshape(-1), rank, S)
    wh = reconstruct_f32(u.reshape(R, G * 8)[:, :C], h)
    if nx.needs_saturation(wh, dtype):
        flags |= FLAG_SAT
    blob = Blob(dtype, S, k, flags, R, C, np.float32(delta), n_tiles, s_bits, model, model.to_bytes(),
                offsets, lens.reshape(-1).astype(np.uint16), states, stream)
    return blob.to_bytes()


def parse_blob(buf: bytes) -> Blob:
    if len(buf) < HEADER.size:
        raise ValueError("blob truncated")
    (magic, ver, dtype, p, S, k, flags, tl, R, C, delta, n_tiles, n_blocks, n_words, mb, z) = \
        HEADER.unpack_from(buf, 0)
    if magic != MAGIC or ver != VERSION or tl != TILE_LOG2 or z != 0:
        raise ValueError("bad header")
    if dtype not in nx.DTYPES or S not in (1, 2, 4, 8, 16, 32, 64) or not (3 <= k <= 7) or flags > 3:
        raise ValueError("bad header fields")
    if p != precision(k):
        raise ValueError("table precision does not match the escape threshold")
    if R < 1 or C < 1:
        raise ValueError("bad shape")
    n_groups = R * (-(-C // 8))
    if n_tiles != max(1, -(-n_groups // TILE_GROUPS)):
        raise ValueError("bad tile count")
    n_ch = n_tiles * S
    if n_blocks != -(-n_ch // BLOCK_CHAINS):
        raise ValueError("bad block count")
    off = HEADER.size
    fw = 1 if S >= 8 else 2
    n_nib = -(-n_ch // 2)
    need = off + 2 * R + mb + 4 * n_blocks + fw * n_ch + n_nib + 4 * n_ch + 2 * n_words
    if len(buf) != need:
        raise ValueError("blob size mismatch")
    s_bits = np.frombuffer(buf, "<u2", R, off).copy(); off += 2 * R
    if ((s_bits & 0x8000) != 0).any() or (((s_bits >> 7) & 0xFF) == 0xFF).any():
        raise ValueError("bad row scale")
    mbytes = bytes(buf[off:off + mb]); off += mb
    model = Model.from_bytes(mbytes, k)
    offs = np.frombuffer(buf, "<u4", n_blocks, off).copy(); off += 4 * n_blocks
    full = np.frombuffer(buf, "<u1" if fw == 1 else "<u2", n_ch, off).astype(np.int64); off += fw * n_ch
    nib = np.frombuffer(buf, "<u1", n_nib, off).astype(np.int64); off += n_nib
    st = np.frombuffer(buf, "<u4", n_ch, off).copy(); off += 4 * n_ch
    stream = np.frombuffer(buf, "<u2", n_words, off).copy()
    tails = np.stack([nib & 15, nib >> 4], axis=1).reshape(-1)[:n_ch]
    if (tails >= CHUNK).any() or (n_ch % 2 and (nib[-1] >> 4) != 0):
        raise ValueError("bad tail length")
    lens = CHUNK * full + tails
    size = block_geometry(lens, S)[3]
    if n_words != CHUNK * int(size.sum()):
        raise ValueError("chain lengths do not cover the stream")
    if not np.array_equal(offs.astype(np.int64), np.concatenate([[0], np.cumsum(size)[:-1]])):
        raise ValueError("block offsets inconsistent")
    if (st < L).any():
        raise ValueError("state below L")
    return Blob(dtype, S, k, flags, R, C, np.float32(delta), n_tiles, s_bits, model, mbytes, offs,
                lens.astype(np.uint16), st, stream)


def reconstruct_f32(u: np.ndarray, h: np.ndarray) -> np.ndarray:
    """w_hat = fl32(h_r * fl32(u))."""
    return (h[:, None] * np.asarray(u).astype(np.float32)).astype(np.float32)


class ChunkReader:
    """Reads every chain's words from its tile area: full chunks where the
    schedule placed them, the tail from the tile's tails.  A word is readable
    only once a sync round of the schedule has fetched its chunk (a site's
    last, asynchronous round lands at the next site)."""

    def __init__(self, b: Blob, sched: TileSchedule):
        self.b = b
        self.sched = sched
        n_ch = b.n_tiles * b.S
        self.nfull, self.main_start, self.tail_pos, _ = block_geometry(b.chain_lens, b.S)
        self.base = CHUNK * b.block_offsets.astype(np.int64)[np.arange(n_ch) // BLOCK_CHAINS]
        self.q = np.zeros(n_ch, dtype=np.int64)
        self.overrun = np.zeros(n_ch, dtype=bool)

    def _pos(self, c, i, checked):
        S = self.b.S
        t, j = c // S, c % S
        n = i // CHUNK
        full = n < self.nfull[c]
        fetched = i < self.sched.landed[t, j]
        rk = self.sched.rank[t, j, np.minimum(n, self.sched.rank.shape[2] - 1)]
        pos = np.where(full, self.base[c] + self.main_start[c] + CHUNK * rk + i % CHUNK,
                       self.base[c] + self.tail_pos[c] + i - CHUNK * self.nfull[c])
        ok = (i < self.b.chain_lens[c]) & (fetched | (not checked)) & ((~full) | (rk >= 0))
        return np.where(ok, pos, -1), ok

    def _read(self, pos):
        w = np.zeros(len(pos), dtype=np.uint64)
        good = pos >= 0
        w[good] = self.b.stream[pos[good]]
        return w

    def take(self, idx):
        pos, ok = self._pos(idx, self.q[idx], checked=True)
        self.overrun[idx[~ok]] = True
        self.q[idx] += 1
        return self._read(pos)


def decode(buf, tiles=None):
    """Decode a blob.  Returns (u int32 (R, C) doubled coordinates, container array (R, C), info).

    ``tiles`` restricts decoding to an iterable of tile indices (other
    outputs stay zero): the tile-independence property.  Each tile runs the
    request schedule of ``layout`` while it decodes, group by group.
    """
    b = parse_blob(buf) if not isinstance(buf, Blob) else buf
    R, C = b.R, b.C
    G = -(-C // 8)
    n_groups = R * G
    n_tiles, cg = chain_layout(n_groups, b.S)
    S = b.S
    ngr = chain_group_counts(n_groups, S, n_tiles)
    if tiles is not None:
        keep = np.zeros(n_tiles, dtype=bool)
        keep[np.asarray(list(tiles), dtype=np.int64)] = True
    else:
        keep = np.ones(n_tiles, dtype=bool)
    ngr = np.where(keep[:, None], ngr, 0)
    lens = np.where(keep[:, None], b.chain_lens.astype(np.int64).reshape(n_tiles, S), 0)
    sched = TileSchedule(lens, ngr, esc=bool(b.flags & FLAG_ESC))
    reader = ChunkReader(b, sched)
    dec = ChainDecoder(b.model, b.states, n_groups)
    sched.prime()
    for g in range(cg.shape[1]):
        act = (g < ngr).reshape(-1)
        if sched.serves(g):
            sched.service(g)
        idx = np.nonzero(act)[0]
        if idx.size == 0:
            continue
        q0 = reader.q.copy()
        dec.decode_group(idx, cg[idx, g], reader)
        sched.consume(act.reshape(n_tiles, S), (reader.q - q0).reshape(n_tiles, S))
    active = keep.repeat(S) & (ngr.reshape(-1) > 0)
    ok_state = bool((dec.x[active] == L).all())
    ok_reads = not bool(reader.overrun.any())
    u = dec.u.reshape(R, G * 8)[:, :C]
    h = half_steps(b.s_bits, b.delta)
    wh = reconstruct_f32(u, h)
    out = nx.cast_container(wh, b.dtype)
    info = dict(final_state_ok=ok_state, reads_in_bounds=ok_reads, S=b.S, k=b.k, flags=b.flags,
                actual_bpp=8.0 * (len(buf) if not isinstance(buf, Blob) else len(b.to_bytes())) / (R * C))
    return u.astype(np.int32), out, info


def actual_bpp(buf: bytes) -> float:
    b = parse_blob(buf)
    return 8.0 * len(buf) / (b.R * b.C)
