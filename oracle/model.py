"""Conditional probability model of lattice coordinates (oracle).

[ABS]: the compressor "combines row-normalized E8 lattice quantization with a
conditional probability model of lattice coordinates".  The pages give no
detail, so the model below is this project's reading; everything in it is
integer arithmetic.

Symbols.  A group is 8 doubled coordinates u (one E8 point).  Its coset is
c = u_0 mod 2.  Each coordinate becomes a magnitude m = (|u| - c) / 2 and a
sign neg = [u < 0].  Magnitudes below K = 2^k are coded directly
(msym = m); larger ones fall in log-buckets with 4 sub-buckets per octave,
msym = K + 4 (e - k) + ((m >> (e-2)) & 3) with e = floor(log2 m), and the
remaining e - 2 low bits of m travel raw (bypass-coded).  The signed symbol is
sid = 2 msym + neg (c = 0, m = 0 has no sign: sid = 0).

Contexts (7 tables of M = 2^P slots; P = 10 when K <= 32, P = 11 when K >= 64):
  0          FIRST      coordinate 0, joint over (c, sid): id = 512 c + sid
  1 + c      FREE[c]    coordinates 1..6
  3 + 2c + pi  LAST[c][pi] coordinate 7, where pi = parity of sum_{i<7} floor(u_i/2).
E8 forces sum_i floor(u_i/2) to be even, so the last coordinate's
floor(u_7/2) has parity pi: LAST only holds the direct symbols that agree with
it, and for bucket symbols one raw bit fewer is sent (its low bit is implied:
rho = pi for c = 0, rho = pi xor neg for c = 1).

Stored model: coset weights w = Q([n(0), n(1)], M) and per-coset magnitude
frequencies g_c = Q(n_c(msym), M / 2).  FREE[c] gives each sign half of the
magnitude's probability (the zero of coset 0 gets 2 g_0(0)), so signs cost
exactly one bit.  FIRST and LAST are derived from the stored model with Q.

Pins (tests): Q's invariants (sum, floor of one, idempotence), symbol map
bijection over all magnitudes < 2^29, LAST restriction consistent with the
E8 parity of random lattice points, LOG2Q values clear of rounding ties.
"""
from __future__ import annotations

import math
import numpy as np

P_MAX = 11
M_MAX = 1 << P_MAX    # the largest table: 2048 slots
N_CTX = 7
ID_SPACE = 1024       # ids per table (FIRST uses 512 c + sid)
MAX_E = 28            # |u| < 2^30  ->  m < 2^29  ->  e <= 28


def precision(k: int) -> int:
    """Table precision P (M = 2^P slots) for escape threshold K = 2^k: 10 for K <= 32,
    11 for K >= 64.  (This project's reading -- the pages fix no table size.  On
    row-scaled Gaussian weights, 1024 slots cost, counting both the longer code and
    the coarser resolution the rate search then settles on, about 0.005 bit a
    coordinate at K = 16, 0.01 at K = 32, 0.02-0.03 at K = 64 and 0.1 at K = 128;
    the two larger alphabets keep 2048 slots.)"""
    return 11 if k >= 6 else 10


def n_msym(k: int) -> int:
    """Size of the magnitude alphabet for K = 2^k (direct + all log-buckets)."""
    return (1 << k) + 4 * (MAX_E + 1 - k)


# ---------------------------------------------------------------- symbol map
def magnitude_symbol(m: np.ndarray, k: int):
    """m -> (msym, raw, rawbits) for the full (non-LAST) coding."""
    m = np.asarray(m, dtype=np.int64)
    K = 1 << k
    msym = m.copy()
    raw = np.zeros_like(m)
    rb = np.zeros_like(m)
    big = m >= K
    if big.any():
        mb = m[big]
        e = np.floor(np.log2(mb.astype(np.float64))).astype(np.int64)
        # guard the float log against off-by-one at exact powers of two
        e = np.where((np.int64(1) << e) > mb, e - 1, e)
        e = np.where((np.int64(1) << (e + 1)) <= mb, e + 1, e)
        top2 = (mb >> (e - 2)) & 3
        msym[big] = K + 4 * (e - k) + top2
        raw[big] = mb & ((np.int64(1) << (e - 2)) - 1)
        rb[big] = e - 2
    return msym, raw, rb


def magnitude_from_symbol(msym: np.ndarray, raw: np.ndarray, k: int) -> np.ndarray:
    msym = np.asarray(msym, dtype=np.int64)
    raw = np.asarray(raw, dtype=np.int64)
    K = 1 << k
    out = msym.copy()
    big = msym >= K
    e = k + (msym[big] - K) // 4
    top2 = (msym[big] - K) % 4
    out[big] = (np.int64(1) << e) | (top2 << (e - 2)) | raw[big]
    return out


def bucket_exponent(msym, k):
    K = 1 << k
    return k + (np.asarray(msym, dtype=np.int64) - K) // 4


# ---------------------------------------------------------------- frequency quantiser Q
def quantize_freqs(weights, ids, total: int) -> np.ndarray:
    """Q(weights, total): integer frequencies over ``ids`` (ascending) summing to ``total``.

    Present ids (weight > 0) get max(1, floor(w T / W)).  If fewer than two ids
    are present, the smallest absent ids of the list join as present with
    weight 0 (so no symbol ever owns the whole table).  A shortfall is handed
    out +1 at a time by largest remainder w T mod W (ties: smaller id); an
    excess is taken back -1 at a time from the largest frequency above 1
    (ties: smaller id).  With zero total weight the two joined ids split T.
    Returns an array aligned with ``ids``.
    """
    w = np.asarray(weights, dtype=np.int64)
    ids = np.asarray(ids, dtype=np.int64)
    assert w.shape == ids.shape and (np.diff(ids) > 0).all()
    present = w > 0
    if present.sum() < 2:
        for pos in range(len(ids)):
            if not present[pos]:
                present[pos] = True
                if present.sum() >= 2:
                    break
    W = int(w.sum())
    f = np.zeros(len(ids), dtype=np.int64)
    if W == 0:
        pos = np.nonzero(present)[0]
        f[pos[0]] = total // 2
        f[pos[1]] = total - total // 2
        return f
    T = int(total)
    fl = [(int(wi) * T) // W for wi in w]
    rem = [(int(wi) * T) % W for wi in w]
    for p in range(len(ids)):
        if present[p]:
            f[p] = max(1, fl[p])
    d = T - int(f.sum())
    if d > 0:
        order = sorted((p for p in range(len(ids)) if present[p]), key=lambda p: (-rem[p], p))
        for p in order[:d]:
            f[p] += 1
    while d < 0:
        best = -1
        for p in range(len(ids)):
            if present[p] and f[p] > 1 and (best < 0 or f[p] > f[best]):
                best = p
        f[best] -= 1
        d += 1
    assert int(f.sum()) == T
    return f


# ---------------------------------------------------------------- stored model
class Model:
    """Stored model (coset weights + magnitude frequencies) and its 7 derived tables."""

    def __init__(self, k: int, w1: int, g0: np.ndarray, g1: np.ndarray):
        self.k = k
        self.K = 1 << k
        self.nm = n_msym(k)
        self.P = precision(k)
        self.M = 1 << self.P
        self.w = np.array([self.M - w1, w1], dtype=np.int64)
        self.g = [np.zeros(self.nm, dtype=np.int64), np.zeros(self.nm, dtype=np.int64)]
        self.g[0][:len(g0)] = g0
        self.g[1][:len(g1)] = g1
        self._derive()

    # FREE[c](sid)
    def _free(self, c: int) -> np.ndarray:
        f = np.zeros(2 * self.nm, dtype=np.int64)
        g = self.g[c]
        f[0::2] = g
        f[1::2] = g
        if c == 0:
            f[0] = 2 * g[0]
            f[1] = 0
        return f

    def last_alphabet(self, c: int, pi: int) -> np.ndarray:
        """Signed symbols allowed as the last coordinate in context (c, pi)."""
        sid = np.arange(2 * self.nm, dtype=np.int64)
        msym, neg = sid >> 1, sid & 1
        direct = msym < self.K
        if c == 0:
            ok = np.where(direct, (msym & 1) == pi, True)
            ok &= sid != 1
        else:
            ok = np.where(direct, ((msym + neg) & 1) == pi, True)
        return sid[ok]

    def _derive(self):
        F = np.zeros((N_CTX, ID_SPACE), dtype=np.int64)
        free = [self._free(0), self._free(1)]
        F[1, :2 * self.nm] = free[0]
        F[2, :2 * self.nm] = free[1]
        # FIRST: joint over (c, sid)
        ids = []
        wts = []
        for c in (0, 1):
            for sid in range(2 * self.nm):
                if c == 0 and sid == 1:
                    continue
                ids.append(512 * c + sid)
                wts.append(int(self.w[c]) * int(free[c][sid]))
        F[0, ids] = quantize_freqs(wts, ids, self.M)
        # LAST[c][pi]
        for c in (0, 1):
            for pi in (0, 1):
                alph = self.last_alphabet(c, pi)
                F[3 + 2 * c + pi, alph] = quantize_freqs(free[c][alph], alph, self.M)
        self.F = F
        self.CUM = np.zeros_like(F)
        self.CUM[:, 1:] = np.cumsum(F, axis=1)[:, :-1]
        # slot -> id (the plain definition of the rANS symbol lookup)
        self.SLOT2ID = np.zeros((N_CTX, self.M), dtype=np.int64)
        for t in range(N_CTX):
            self.SLOT2ID[t] = np.repeat(np.arange(ID_SPACE), F[t])

    # -- serialisation: LSB-first bit packing -------------------------------
    def to_bytes(self) -> bytes:
        bits = []

        def put(v, n):
            for i in range(n):
                bits.append((int(v) >> i) & 1)

        put(self.w[1], 11)
        for c in (0, 1):
            g = self.g[c]
            nz = np.nonzero(g)[0]
            n_mag = int(nz[-1]) + 1
            put(n_mag, 8)
            for v in g[:n_mag]:
                put(v, 10)
        while len(bits) % 8:
            bits.append(0)
        out = bytearray(len(bits) // 8)
        for i, b in enumerate(bits):
            out[i >> 3] |= b << (i & 7)
        return bytes(out)

    @staticmethod
    def from_bytes(buf: bytes, k: int) -> "Model":
        pos = [0]

        def get(n):
            v = 0
            for i in range(n):
                p = pos[0] + i
                if (p >> 3) >= len(buf):
                    raise ValueError("model truncated")
                v |= ((buf[p >> 3] >> (p & 7)) & 1) << i
            pos[0] += n
            return v

        w1 = get(11)
        gs = []
        for c in (0, 1):
            n_mag = get(8)
            if n_mag > n_msym(k) or n_mag < 1:
                raise ValueError("bad magnitude alphabet size")
            gs.append(np.array([get(10) for _ in range(n_mag)], dtype=np.int64))
        M = 1 << precision(k)
        if not (1 <= w1 <= M - 1):
            raise ValueError("bad coset weight")
        for g in gs:
            if int(g.sum()) != M // 2 or (g > 0).sum() < 2:
                raise ValueError("bad magnitude frequencies")
        if (len(buf) * 8 - pos[0]) >= 8:
            raise ValueError("model has trailing bytes")
        return Model(k, w1, gs[0], gs[1])


def build_model(k: int, coset_counts, mag_counts0, mag_counts1) -> Model:
    nm = n_msym(k)
    M = 1 << precision(k)
    w = quantize_freqs(coset_counts, [0, 1], M)
    g0 = quantize_freqs(mag_counts0[:nm], np.arange(nm), M // 2)
    g1 = quantize_freqs(mag_counts1[:nm], np.arange(nm), M // 2)
    return Model(k, int(w[1]), g0, g1)


# ---------------------------------------------------------------- per-group symbols
def group_symbols(u: np.ndarray, k: int):
    """Symbolise groups of doubled coordinates u (n, 8).

    Returns a dict of (n, 8) arrays in decoding order: ctx (table index), id
    (symbol id in that table), rawval / rawbits (bits sent by bypass after the
    symbol), plus c (n,), msym (n, 8) for counting.
    """
    u = np.asarray(u, dtype=np.int64)
    n = u.shape[0]
    c = np.mod(u[:, 0], 2)
    mag = (np.abs(u) - c[:, None]) // 2
    neg = (u < 0).astype(np.int64)
    msym, raw, rb = magnitude_symbol(mag.reshape(-1), k)
    msym = msym.reshape(n, 8)
    raw = raw.reshape(n, 8)
    rb = rb.reshape(n, 8)
    sid = 2 * msym + neg
    q = u >> 1                                          # floor(u / 2)
    pi = np.mod(q[:, :7].sum(axis=1), 2)
    ctx = np.empty((n, 8), dtype=np.int64)
    ctx[:, 0] = 0
    ctx[:, 1:7] = (1 + c)[:, None]
    ctx[:, 7] = 3 + 2 * c + pi
    ids = sid.copy()
    ids[:, 0] = 512 * c + sid[:, 0]
    rawval = raw.copy()
    rawbits = rb.copy()
    # last coordinate: bucket's low raw bit is implied by the E8 parity
    K = 1 << k
    lastb = msym[:, 7] >= K
    rho = np.where(c == 0, pi, pi ^ neg[:, 7])
    assert (np.mod(q[:, 7], 2) == pi).all(), "E8 parity violated"
    if lastb.any():
        assert ((raw[lastb, 7] & 1) == rho[lastb]).all()
        rawval[lastb, 7] = raw[lastb, 7] >> 1
        rawbits[lastb, 7] = rb[lastb, 7] - 1
    return dict(ctx=ctx, id=ids, rawval=rawval, rawbits=rawbits, c=c, msym=msym, pi=pi)


def count_symbols(sym, nm: int):
    c = sym["c"]
    coset_counts = np.array([(c == 0).sum(), (c == 1).sum()], dtype=np.int64)
    mags = []
    for cc in (0, 1):
        ms = sym["msym"][c == cc].reshape(-1)
        mags.append(np.bincount(ms, minlength=nm).astype(np.int64))
    return coset_counts, mags[0], mags[1]


def choose_k(mags: np.ndarray) -> int:
    """Smallest k in 3..7 with #(m >= 2^k) * 2^20 <= #coordinates (else 7).

    The pages leave the split between directly coded magnitudes and escape
    buckets open; this reading keeps escapes (raw-bit symbols) at most one in
    2^20 coordinates of the sample whenever K = 2^k <= 128 allows it.
    """
    n = mags.size
    for k in range(3, 8):
        if int((mags >= (1 << k)).sum()) * (1 << 20) <= n:
            return k
    return 7


# ---------------------------------------------------------------- cost table
def log2q_table() -> np.ndarray:
    """LOG2Q[f] = floor(2^16 log2 f + 1/2) for f in [1, 2048] (index 0 unused)."""
    t = np.zeros(M_MAX + 1, dtype=np.int64)
    for f in range(1, M_MAX + 1):
        t[f] = int(math.floor(65536.0 * math.log2(f) + 0.5))
    return t


LOG2Q = log2q_table()


def est_bits_q16(sym, model: Model) -> int:
    """Estimated code length in units of 2^-16 bit: sum of (P - log2 f) + raw bits."""
    f = model.F[sym["ctx"], sym["id"]]
    assert (f > 0).all()
    return int((model.P * 65536 - LOG2Q[f]).sum()) + 65536 * int(sym["rawbits"].sum())
