"""Tile rANS coder (oracle), vectorised across independent chains.

[SUM]: the final coordinates are coded with rANS in independently decodable
tiles; [ABS]: "entropy-coded in independently decodable tiles".  Parameters
(pages silent; ours): 32-bit state x in [L, 2^32) with L = 2^16, 16-bit
words, M = 2^P slots per table (P = 10 or 11, ``model.precision``).  Reference: J. Duda, "Asymmetric numeral
systems" (arXiv 1311.2540), range variant.

Decoding one symbol of table T:
    slot = x mod M; find s with cum_s <= slot < cum_s + f_s;
    x <- f_s * floor(x / M) + slot - cum_s;  if x < L: x <- x * 2^16 + next word.
Decoding b <= 16 raw bits (bypass):
    r = x mod 2^b;  x <- floor(x / 2^b);      if x < L: x <- x * 2^16 + next word.
Raw fields wider than 16 bits are two bypasses, low 16 bits first.

The encoder runs the chain's operations in reverse from x = L, emitting a word
whenever the next step would leave [L, 2^32); its final state is stored and
the decoder must end at exactly x = L.

Pins (tests): round trip on random tables including escapes and partial
tiles; final state L; code length within the ideal sum of -log2(f/M) plus the
per-chain flush bound.
"""
from __future__ import annotations

import numpy as np

from .model import Model

L = 1 << 16
WORD = 16
OPS_PER_COORD = 3     # symbol + up to two bypasses


def _ops_for_group(sym, g, i):
    """Per-op arrays for coordinate i of the groups g (in decoding order)."""
    ctx = sym["ctx"][g, i]
    ids = sym["id"][g, i]
    rv = sym["rawval"][g, i]
    rb = sym["rawbits"][g, i]
    lo_b = np.minimum(rb, 16)
    hi_b = np.maximum(rb - 16, 0)
    lo_v = rv & 0xFFFF
    hi_v = rv >> 16
    return ctx, ids, lo_b, lo_v, hi_b, hi_v


def encode_chains(sym, model: Model, chain_groups):
    """Encode every chain.

    ``chain_groups`` is an (n_chains, steps) int64 array of global group
    indices in decoding order, -1 where a chain has no more groups.
    Returns (states uint32[n_chains], list of uint16 word arrays in decoding
    order, words (n_chains, steps): how many words the decoder reads while
    decoding each step's group -- the words emitted while encoding it).
    """
    n_ch, steps = chain_groups.shape
    x = np.full(n_ch, L, dtype=np.uint64)
    cap = steps * 8 * OPS_PER_COORD + 1
    buf = np.zeros((n_ch, cap), dtype=np.uint64)
    cnt = np.zeros(n_ch, dtype=np.int64)
    per_step = np.zeros((n_ch, steps), dtype=np.int64)
    F, CUM = model.F, model.CUM
    cur = [0]

    def emit(idx, mask):
        if mask.any():
            sel = idx[mask]
            buf[sel, cnt[sel]] = x[sel] & 0xFFFF
            cnt[sel] += 1
            per_step[sel, cur[0]] += 1
            x[sel] >>= np.uint64(16)

    def bypass(idx, b, v):
        act = b > 0
        if not act.any():
            return
        bb = b.astype(np.uint64)
        lim = np.left_shift(np.uint64(1), np.uint64(32) - bb)
        emit(idx, act & (x[idx] >= lim))
        xs = x[idx]
        x[idx] = np.where(act, np.left_shift(xs, bb) | v.astype(np.uint64), xs)

    for s in range(steps - 1, -1, -1):
        g = chain_groups[:, s]
        idx = np.nonzero(g >= 0)[0]
        if idx.size == 0:
            continue
        cur[0] = s
        gg = g[idx]
        for i in range(7, -1, -1):
            ctx, ids, lo_b, lo_v, hi_b, hi_v = _ops_for_group(sym, gg, i)
            bypass(idx, hi_b, hi_v)
            bypass(idx, lo_b, lo_v)
            f = F[ctx, ids].astype(np.uint64)
            cum = CUM[ctx, ids].astype(np.uint64)
            assert (f > 0).all()
            # the encoder keeps x below f * (L / M) * 2^16 = f << (32 - P) before a step
            emit(idx, x[idx] >= np.left_shift(f, np.uint64(32 - model.P)))
            xs = x[idx]
            x[idx] = (xs // f) * np.uint64(model.M) + (xs % f) + cum
    states = x.astype(np.uint32)
    assert (x < (1 << 32)).all() and (x >= L).all()
    words = [buf[c, :cnt[c]][::-1].astype(np.uint16) for c in range(n_ch)]
    return states, words, per_step


class WordReader:
    """Per-chain word cursors over chain-contiguous word arrays (the coder's own
    tests; the blob layout has its own reader in ``codec``)."""

    def __init__(self, words):
        self.words = [np.asarray(w, dtype=np.uint16) for w in words]
        self.q = np.zeros(len(words), dtype=np.int64)
        self.overrun = np.zeros(len(words), dtype=bool)

    def word_at(self, c: int, i: int) -> int:
        w = self.words[c]
        return int(w[i]) if 0 <= i < len(w) else -1

    def take(self, idx):
        out = np.zeros(len(idx), dtype=np.uint64)
        for n, c in enumerate(idx):
            v = self.word_at(c, self.q[c])
            if v < 0:
                self.overrun[c] = True
                v = 0
            out[n] = v
            self.q[c] += 1
        return out


class ChainDecoder:
    """Decodes chains group by group (all chains of a step together)."""

    def __init__(self, model: Model, states, n_groups: int):
        self.model = model
        self.k = model.k
        self.K = 1 << model.k
        self.x = np.asarray(states, dtype=np.uint64).copy()
        self.u = np.zeros((n_groups, 8), dtype=np.int64)

    def _symbol(self, x, ctx):
        """One table step: returns (new x before renormalisation, symbol id)."""
        F, CUM, S2I = self.model.F, self.model.CUM, self.model.SLOT2ID
        slot = (x & np.uint64(self.model.M - 1)).astype(np.int64)
        ids = S2I[ctx, slot]
        f = F[ctx, ids].astype(np.uint64)
        cum = CUM[ctx, ids].astype(np.uint64)
        return f * (x >> np.uint64(self.model.P)) + slot.astype(np.uint64) - cum, ids

    def decode_group(self, idx, groups, reader):
        """Decode the next group of chains ``idx`` (global group ids ``groups``)."""
        k, K = self.k, self.K
        x = self.x

        def renorm(sel):
            low = x[sel] < L
            if low.any():
                s2 = sel[low]
                w = reader.take(s2)
                x[s2] = (x[s2] << np.uint64(16)) | w

        def bypass(b):
            r = np.zeros(len(idx), dtype=np.int64)
            act = b > 0
            if act.any():
                sel = idx[act]
                bb = b[act].astype(np.uint64)
                r[act] = (x[sel] & ((np.uint64(1) << bb) - np.uint64(1))).astype(np.int64)
                x[sel] = x[sel] >> bb
                renorm(sel)
            return r

        c = np.zeros(len(idx), dtype=np.int64)
        pi = np.zeros(len(idx), dtype=np.int64)
        urow = np.zeros((len(idx), 8), dtype=np.int64)
        for i in range(8):
            if i == 0:
                ctx = np.zeros(len(idx), dtype=np.int64)
            elif i < 7:
                ctx = 1 + c
            else:
                ctx = 3 + 2 * c + pi
            x[idx], ids = self._symbol(x[idx], ctx)
            renorm(idx)
            if i == 0:
                c = ids >> 9
                sid = ids & 511
            else:
                sid = ids
            msym = sid >> 1
            neg = sid & 1
            big = msym >= K
            e = k + (msym - K) // 4
            top2 = (msym - K) % 4
            nb = np.where(big, e - 2 - (1 if i == 7 else 0), 0)
            lo = bypass(np.minimum(nb, 16))
            hi = bypass(np.maximum(nb - 16, 0))
            raw = lo | (hi << 16)
            if i == 7:
                rho = np.where(c == 0, pi, pi ^ neg)
                raw = np.where(big, (raw << 1) | rho, raw)
            m = np.where(big, (np.int64(1) << np.where(big, e, 0)) | (top2 << np.where(big, e - 2, 0)) | raw, msym)
            u = (2 * m + c) * np.where(neg == 1, -1, 1)
            urow[:, i] = u
            if i < 7:
                pi = pi ^ np.mod(u >> 1, 2)
        self.u[groups] = urow


def decode_chains(model: Model, states, chain_groups, reader, n_groups: int):
    """Decode chain-contiguous words; returns (u int64 (n_groups, 8), final x)."""
    dec = ChainDecoder(model, states, n_groups)
    for s in range(chain_groups.shape[1]):
        g = chain_groups[:, s]
        idx = np.nonzero(g >= 0)[0]
        if idx.size:
            dec.decode_group(idx, g[idx], reader)
    return dec.u, dec.x


def ideal_bits(sym, model: Model) -> float:
    f = model.F[sym["ctx"], sym["id"]].astype(np.float64)
    return float(np.sum(model.P - np.log2(f)) + sym["rawbits"].sum())
