"""Stream layout of blob v3: where every chain's words sit (oracle).

[ABS] / [SUM] say only that the coordinates are rANS-coded in independently
decodable tiles.  How the words sit in memory is this project's format,
chosen so that a GPU wave fetches them with contiguous loads:

* every chain's words (decoding order) are cut into chunks of 8 words; a
  chain has nfull = len // 8 full chunks and a tail of len % 8 words;
* a block (64 consecutive chains) stores [the main area of each of its tiles,
  in tile order] [the tails of its chains, chain order, word after word]
  [zeros up to a multiple of 8 words]; blocks follow each other;
* a tile's main area holds its chains' full chunks in request order: the
  order in which the reference reader below asks for them.  Chains take their
  turn in chain order within a site; a sync site repeats rounds until no chain
  wants more.  Blobs without escape symbols:

      prime                      sync until ahead >= 17
      group g (g even)           sync until ahead >= 17, then one round in which
                                 a chain asks if ahead <= 24

  blobs with escape symbols (header flag), every group served:

      prime                      sync until ahead >= 24
      group g (every g)          sync until ahead >= 24, then one round in which
                                 a chain asks if ahead <= 24

  where ahead = words fetched - words consumed (the tail counts as one
  request).  A chain asks only while it has unfetched words and only at groups
  it decodes (g < its group count).

Why these numbers: a group consumes at most 8 words without escapes (one per
symbol) and at most 24 with them (two more per escape for up to 28 raw bits).
The reader's words from a site's last round arrive only at the next site, so
a chain may read only what the sync rounds fetched: 17 covers the two
escape-free groups until the next site, 24 the one group of a blob with
escapes.  A chain never holds more than 32 words ahead (the reader's ring).

Pins (tests): hand-worked schedules for small consumption patterns; every
word fetched by a sync round before it is read, and never more than 32 words
ahead, on random patterns; encoder/decoder round trips.
"""
from __future__ import annotations

import numpy as np

CHUNK = 8            # words per chunk
BLOCK = 64           # chains per block
RING = 32            # words a chain may hold ahead
AHEAD_GROUP = 17     # two escape-free groups consume <= 16
AHEAD_ESC = 24       # one group with escapes consumes <= 24
ASYNC_MAX = RING - CHUNK


class TileSchedule:
    """The reference reader for all tiles at once (arrays shaped (n_tiles, S)).

    ``rank[t, j, n]`` receives the position (in chunks from the tile's start) of
    chain j's full chunk n, in the order requested.  ``esc`` selects the
    schedule of blobs with escape symbols.  ``landed`` counts the words of the
    sync rounds (and of earlier sites): the words a chain may read.
    """

    def __init__(self, lens: np.ndarray, ngr: np.ndarray, esc: bool = False):
        self.n = np.asarray(lens, dtype=np.int64)
        self.ngr = np.asarray(ngr, dtype=np.int64)
        self.esc = bool(esc)
        self.ahead = AHEAD_ESC if esc else AHEAD_GROUP
        T, S = self.n.shape
        self.F = np.zeros((T, S), dtype=np.int64)
        self.landed = np.zeros((T, S), dtype=np.int64)
        self.q = np.zeros((T, S), dtype=np.int64)
        self.ctr = np.zeros(T, dtype=np.int64)
        nfull = int((self.n // CHUNK).max()) if self.n.size else 0
        self.rank = np.full((T, S, max(nfull, 1)), -1, dtype=np.int64)

    def _round(self, want):
        """One round: every wanting chain takes its next chunk, in chain order."""
        full = want & (self.n - self.F >= CHUNK)
        order = np.cumsum(full, axis=1) - 1
        t_idx, j_idx = np.nonzero(full)
        self.rank[t_idx, j_idx, self.F[t_idx, j_idx] // CHUNK] = self.ctr[t_idx] + order[t_idx, j_idx]
        self.ctr += full.sum(axis=1)
        self.F = np.where(full, self.F + CHUNK, np.where(want, self.n, self.F))
        assert (self.F - self.q <= RING).all(), "a chain would hold more than the ring"

    def _sync(self, cand, ahead):
        while True:
            want = cand & (self.F - self.q < ahead) & (self.F < self.n)
            if not want.any():
                break
            self._round(want)
        self.landed = self.F.copy()

    def prime(self):
        self._sync(np.ones_like(self.n, dtype=bool), self.ahead)

    def serves(self, g: int) -> bool:
        """Whether group g begins with a service site."""
        return self.esc or g % 2 == 0

    def service(self, g: int):
        act = g < self.ngr
        self._sync(act, self.ahead)
        self._round(act & (self.F - self.q <= ASYNC_MAX) & (self.F < self.n))

    def consume(self, act, words):
        self.q = np.where(act, self.q + words, self.q)


def request_ranks(lens, ngr, cons, esc=False):
    """Run the whole schedule for known per-group consumption.

    lens, ngr: (T, S); cons: (T, S, steps) words consumed by each chain's group g;
    esc: the blob holds escape symbols.  Returns rank (T, S, max full chunks).
    """
    sch = TileSchedule(lens, ngr, esc)
    sch.prime()
    steps = cons.shape[2]
    for g in range(steps):
        act = g < sch.ngr
        if sch.serves(g):
            sch.service(g)
        sch.consume(act, cons[:, :, g])
        assert (sch.q <= sch.landed).all(), "a word was read before a sync round fetched it"
    assert (sch.F == sch.n).all()
    return sch.rank


def block_geometry(lens, S: int):
    """Word positions of every chain's pieces, relative to its block's start.

    lens: (n_chains,).  Returns (nfull, main_start, tail_pos, block_chunks):
    main_start = start of the chain's tile main area, tail_pos = start of its
    tail, both in words from the block start; block_chunks = size of each block
    in chunks.
    """
    lens = np.asarray(lens, dtype=np.int64)
    n_ch = len(lens)
    nfull = lens // CHUNK
    tail = lens % CHUNK
    nb = -(-n_ch // BLOCK)
    main_start = np.zeros(n_ch, dtype=np.int64)
    tail_pos = np.zeros(n_ch, dtype=np.int64)
    block_chunks = np.zeros(nb, dtype=np.int64)
    for b in range(nb):
        c0, c1 = BLOCK * b, min(BLOCK * (b + 1), n_ch)
        tiles_main = CHUNK * nfull[c0:c1].reshape(-1, S).sum(axis=1)
        tstart = np.concatenate([[0], np.cumsum(tiles_main)[:-1]])
        main_start[c0:c1] = np.repeat(tstart, S)
        tails0 = int(tiles_main.sum())
        tail_pos[c0:c1] = tails0 + np.cumsum(tail[c0:c1]) - tail[c0:c1]
        block_chunks[b] = -(-(tails0 + int(tail[c0:c1].sum())) // CHUNK)
    return nfull, main_start, tail_pos, block_chunks


def build_stream(words, lens, rank, S: int):
    """Block areas from per-chain word arrays and the request ranks.

    rank: (n_tiles, S, max full chunks) from the schedule.  Returns
    (block offsets u32 in chunks, stream u16).
    """
    lens = np.asarray(lens, dtype=np.int64)
    nfull, main_start, tail_pos, block_chunks = block_geometry(lens, S)
    offsets = np.concatenate([[0], np.cumsum(block_chunks)[:-1]]).astype(np.int64)
    stream = np.zeros(CHUNK * int(block_chunks.sum()), dtype=np.uint16)
    for c in range(len(lens)):
        base = CHUNK * offsets[c // BLOCK]
        w = words[c]
        t, j = c // S, c % S
        for nn in range(nfull[c]):
            p = base + main_start[c] + CHUNK * rank[t, j, nn]
            stream[p:p + CHUNK] = w[CHUNK * nn:CHUNK * nn + CHUNK]
        r = lens[c] % CHUNK
        if r:
            p = base + tail_pos[c]
            stream[p:p + r] = w[CHUNK * nfull[c]:]
    return offsets.astype(np.uint32), stream
