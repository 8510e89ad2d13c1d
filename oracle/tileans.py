"""TileANS: lossless tile-rANS coding of raw tensor bytes (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[README] Config：压缩配置 lists a lossless TileANS configuration next to the
lossy one: any of the dtypes (BF16, FP16, FP32, FP8, INT8, ...) is restored
bit for bit and the ratio depends on the data.  [NEWS] 任意位元率的本體: lossy
mode takes 2-D tensors only; other shapes go the lossless way.  The pages say
nothing more, so the format is this project's reading, built on the same tile
rANS machinery as the lossy blob (``codec``, ``rans``, ``layout``):

* the tensor is its raw bytes (C order, little-endian elements of E bytes,
  E in {1, 2, 4, 8}), zero-padded to a multiple of 8: groups of 8 bytes,
  tiles of 512 groups (4096 bytes), S chains per tile (8 when the tensor has
  at least 2^22 bytes, else 1), chain j of a tile decoding its groups j, j+S,
  ... exactly as for the lossy coordinates;
* a byte's context is its position inside its element, at most 4 contexts
  (byte index mod min(E, 4): an 8-byte element shares them), each
  context has a table over the 256 byte values: Q(counts, 2048) of ``model``
  over all of the context's bytes (padding included), unless the coded size
  estimated with LOG2Q plus the 4096 bits of the stored table is not below the
  raw 8 bits per byte, in which case the table is uniform and not stored
  (f = 8 for every value: exactly 8 bits a byte);
* the rANS coder (32-bit state, 16-bit words, the final state L) and the
  request-order stream layout are those of the lossy blob (no escapes); the
  byte tables keep P = 11 (2048 slots).

Blob (little-endian, packed):

  header (48 B)  'EPT1' | u16 version=1 | u8 dtype tag (opaque) | u8 E | u8 P=11 |
                 u8 S | u8 ndim | u8 uniform mask (bit p: context p uniform) |
                 u8 tile_log2=12 | 3 x u8 0 | u64 n_bytes | u32 n_tiles |
                 u32 n_blocks | u64 n_words | u64 0
  dims           u64[ndim]
  tables         u16[256] per non-uniform context, in context order
  then block offsets, full-chunk counts, tail nibbles, states and stream
  exactly as in the lossy blob.

Pins (tests): round trip of every element size, shapes of every rank,
ragged sizes and both table kinds; coded size within the LOG2Q estimate plus
the per-chain flush bound; uniform tables on random bytes (exactly 8 bits per
byte of stream); tile independence.
"""
from __future__ import annotations

import struct

import numpy as np

from .codec import chain_layout, chain_group_counts, ChunkReader, BLOCK_CHAINS, TILE_GROUPS
from .layout import CHUNK, TileSchedule, request_ranks, build_stream, block_geometry
from .model import quantize_freqs, LOG2Q
from .rans import encode_chains, L

P = 11                # table precision of the byte tables (2048 slots)
M = 1 << P

MAGIC = b"EPT1"
VERSION = 1
HEADER = struct.Struct("<4sHBBBBBBB3xQIIQQ")
assert HEADER.size == 48
TILE_LOG2 = 12
ELEM_SIZES = (1, 2, 4, 8)


def n_contexts(E: int) -> int:
    return min(E, 4)


class TileAnsError(ValueError):
    pass


class Tables:
    """Per-context frequencies over the 256 byte values (the ``rans`` model
    interface: F, CUM indexed [context, value]; SLOT2ID for decoding; the
    precision P and slot count M)."""

    P = P
    M = M

    def __init__(self, F):
        self.F = np.asarray(F, dtype=np.int64)
        self.CUM = np.concatenate([np.zeros((len(self.F), 1), np.int64), np.cumsum(self.F, axis=1)[:, :-1]], axis=1)
        self.SLOT2ID = np.zeros((len(self.F), M), dtype=np.int64)
        for p in range(len(self.F)):
            self.SLOT2ID[p] = np.repeat(np.arange(256), self.F[p])


def default_chains_per_tile(n_bytes: int) -> int:
    return 8 if n_bytes >= (1 << 22) else 1


def context_tables(padded: np.ndarray, E: int):
    """(F (contexts, 256), uniform mask): Q-quantised counts or uniform per context."""
    nc = n_contexts(E)
    F = np.zeros((nc, 256), dtype=np.int64)
    mask = 0
    for p in range(nc):
        counts = np.bincount(padded[p::nc], minlength=256).astype(np.int64)
        f = quantize_freqs(counts, np.arange(256), M)
        used = counts > 0
        # (the stored table, 256 x 16 bits, counts against the coded side)
        coded = int((counts[used] * (P * 65536 - LOG2Q[f[used]])).sum()) + 256 * 16 * 65536
        raw = 8 * 65536 * int(counts.sum())
        if coded >= raw:
            F[p] = M // 256
            mask |= 1 << p
        else:
            F[p] = f
    return F, mask


def compress(raw, E: int, dims, dtype_tag: int = 0, chains_per_tile=None) -> bytes:
    """raw: the tensor's bytes (uint8, C order); E: element size; dims: its shape."""
    raw = np.frombuffer(np.ascontiguousarray(raw).tobytes(), dtype=np.uint8)
    dims = tuple(int(d) for d in dims)
    if E not in ELEM_SIZES:
        raise TileAnsError("element size must be 1, 2, 4 or 8 bytes")
    if not (1 <= len(dims) <= 8) or any(d < 1 for d in dims):
        raise TileAnsError("rank 1..8, every extent >= 1")
    n_bytes = len(raw)
    if n_bytes != E * int(np.prod(dims, dtype=object)):
        raise TileAnsError("byte count does not match the shape")
    n_groups = -(-n_bytes // 8)
    padded = np.zeros(8 * n_groups, dtype=np.uint8)
    padded[:n_bytes] = raw
    F, mask = context_tables(padded, E)
    tabs = Tables(F)
    by = padded.reshape(n_groups, 8).astype(np.int64)
    ctx = np.broadcast_to(np.arange(8) % n_contexts(E), (n_groups, 8))
    sym = {"ctx": ctx, "id": by, "rawval": np.zeros_like(by), "rawbits": np.zeros_like(by)}
    S = chains_per_tile or default_chains_per_tile(n_bytes)
    assert S in (1, 2, 4, 8, 16, 32, 64)
    n_tiles, cg = chain_layout(n_groups, S)
    states, words, cons = encode_chains(sym, tabs, cg)
    lens = np.array([len(w) for w in words], dtype=np.int64).reshape(n_tiles, S)
    if (lens // CHUNK > (0xFF if S >= 8 else 0xFFFF)).any():
        raise TileAnsError("chain longer than the chunk count field")
    ngr = chain_group_counts(n_groups, S, n_tiles)
    steps = cg.shape[1]
    rank = request_ranks(lens, ngr, cons.reshape(n_tiles, S, steps))
    offsets, stream = build_stream(words, lens.reshape(-1), rank, S)
    n_ch = n_tiles * S
    n_blocks = -(-n_ch // BLOCK_CHAINS)
    hdr = HEADER.pack(MAGIC, VERSION, dtype_tag & 0xFF, E, P, S, len(dims), mask, TILE_LOG2,
                      n_bytes, n_tiles, n_blocks, len(stream), 0)
    flat = lens.reshape(-1)
    full = (flat // CHUNK).astype("<u1" if S >= 8 else "<u2")
    tails = np.zeros(2 * (-(-n_ch // 2)), dtype=np.int64)
    tails[:n_ch] = flat % CHUNK
    nib = (tails[0::2] | (tails[1::2] << 4)).astype("<u1")
    tables = b"".join(F[p].astype("<u2").tobytes() for p in range(len(F)) if not (mask >> p) & 1)
    return b"".join([hdr, np.array(dims, dtype="<u8").tobytes(), tables, offsets.astype("<u4").tobytes(),
                     full.tobytes(), nib.tobytes(), states.astype("<u4").tobytes(), stream.astype("<u2").tobytes()])


class Blob:
    def __init__(self, **kw):
        self.__dict__.update(kw)


def parse(buf: bytes) -> Blob:
    if len(buf) < HEADER.size:
        raise TileAnsError("blob truncated")
    (magic, ver, tag, E, p, S, ndim, mask, tl, n_bytes, n_tiles, n_blocks, n_words, z) = HEADER.unpack_from(buf, 0)
    if magic != MAGIC or ver != VERSION or p != P or tl != TILE_LOG2 or z != 0:
        raise TileAnsError("bad header")
    if E not in ELEM_SIZES or S not in (1, 2, 4, 8, 16, 32, 64) or not (1 <= ndim <= 8) or mask >> n_contexts(E):
        raise TileAnsError("bad header fields")
    off = HEADER.size
    if len(buf) < off + 8 * ndim:
        raise TileAnsError("blob truncated")
    dims = tuple(int(d) for d in np.frombuffer(buf, "<u8", ndim, off))
    off += 8 * ndim
    if any(d < 1 for d in dims) or n_bytes != E * int(np.prod(dims, dtype=object)):
        raise TileAnsError("bad shape")
    n_groups = -(-n_bytes // 8)
    if n_tiles != max(1, -(-n_groups // TILE_GROUPS)):
        raise TileAnsError("bad tile count")
    n_ch = n_tiles * S
    if n_blocks != -(-n_ch // BLOCK_CHAINS):
        raise TileAnsError("bad block count")
    nc = n_contexts(E)
    n_coded = sum(1 for q in range(nc) if not (mask >> q) & 1)
    fw = 1 if S >= 8 else 2
    n_nib = -(-n_ch // 2)
    need = off + 512 * n_coded + 4 * n_blocks + fw * n_ch + n_nib + 4 * n_ch + 2 * n_words
    if len(buf) != need:
        raise TileAnsError("blob size mismatch")
    F = np.zeros((nc, 256), dtype=np.int64)
    for q in range(nc):
        if (mask >> q) & 1:
            F[q] = M // 256
        else:
            F[q] = np.frombuffer(buf, "<u2", 256, off)
            off += 512
            if int(F[q].sum()) != M:
                raise TileAnsError("table does not sum to 2048")
    offs = np.frombuffer(buf, "<u4", n_blocks, off).copy(); off += 4 * n_blocks
    full = np.frombuffer(buf, "<u1" if fw == 1 else "<u2", n_ch, off).astype(np.int64); off += fw * n_ch
    nib = np.frombuffer(buf, "<u1", n_nib, off).astype(np.int64); off += n_nib
    st = np.frombuffer(buf, "<u4", n_ch, off).copy(); off += 4 * n_ch
    stream = np.frombuffer(buf, "<u2", n_words, off).copy()
    tails = np.stack([nib & 15, nib >> 4], axis=1).reshape(-1)[:n_ch]
    if (tails >= CHUNK).any() or (n_ch % 2 and (nib[-1] >> 4) != 0):
        raise TileAnsError("bad tail length")
    lens = CHUNK * full + tails
    size = block_geometry(lens, S)[3]
    if n_words != CHUNK * int(size.sum()):
        raise TileAnsError("chain lengths do not cover the stream")
    if not np.array_equal(offs.astype(np.int64), np.concatenate([[0], np.cumsum(size)[:-1]])):
        raise TileAnsError("block offsets inconsistent")
    if (st < L).any():
        raise TileAnsError("state below L")
    return Blob(dtype_tag=tag, E=E, S=S, dims=dims, mask=mask, n_bytes=n_bytes, n_tiles=n_tiles,
                tables=Tables(F), block_offsets=offs, chain_lens=lens.astype(np.uint16), states=st, stream=stream)


def decode(buf, tiles=None):
    """Decode a TileANS blob: (bytes uint8[n_bytes], info).  ``tiles`` restricts
    decoding to some tiles (the other bytes stay zero)."""
    b = parse(buf)
    n_groups = -(-b.n_bytes // 8)
    n_tiles, cg = chain_layout(n_groups, b.S)
    S = b.S
    ngr = chain_group_counts(n_groups, S, n_tiles)
    keep = np.ones(n_tiles, dtype=bool)
    if tiles is not None:
        keep[:] = False
        keep[np.asarray(list(tiles), dtype=np.int64)] = True
    ngr = np.where(keep[:, None], ngr, 0)
    lens = np.where(keep[:, None], b.chain_lens.astype(np.int64).reshape(n_tiles, S), 0)
    sched = TileSchedule(lens, ngr)
    reader = ChunkReader(b, sched)
    x = b.states.astype(np.uint64).copy()
    out = np.zeros((n_groups, 8), dtype=np.uint8)
    F, CUM, S2I = b.tables.F, b.tables.CUM, b.tables.SLOT2ID
    sched.prime()
    for g in range(cg.shape[1]):
        act = (g < ngr).reshape(-1)
        if sched.serves(g):
            sched.service(g)
        idx = np.nonzero(act)[0]
        if idx.size == 0:
            continue
        q0 = reader.q.copy()
        for i in range(8):
            ctx = i % n_contexts(b.E)
            slot = (x[idx] & np.uint64(M - 1)).astype(np.int64)
            v = S2I[ctx, slot]
            f = F[ctx, v].astype(np.uint64)
            x[idx] = f * (x[idx] >> np.uint64(P)) + slot.astype(np.uint64) - CUM[ctx, v].astype(np.uint64)
            low = idx[x[idx] < L]
            if low.size:
                x[low] = (x[low] << np.uint64(16)) | reader.take(low)
            out[cg[idx, g], i] = v
        sched.consume(act.reshape(n_tiles, S), (reader.q - q0).reshape(n_tiles, S))
    active = keep.repeat(S) & (ngr.reshape(-1) > 0)
    info = dict(final_state_ok=bool((x[active] == L).all()), reads_in_bounds=not bool(reader.overrun.any()),
                S=S, E=b.E, dims=b.dims, mask=b.mask)
    return out.reshape(-1)[:b.n_bytes].copy(), info
