"""Pins for the stream layout's request schedule (oracle.layout): hand-worked
orders, the fetched-before-read invariant on random consumption patterns, and the
block geometry."""
import numpy as np
import pytest

from oracle import layout


def test_hand_worked_two_chains():
    # No escapes.  Chain 0: 40 words, groups of 8; chain 1: 24 words, groups 8, 8, 8, 0, 0.
    # prime:  rounds (0:r0 1:r1) (0:r2 1:r3) (0:r4 1:r5): 24 ahead each, chain 1 complete
    # g0:     sync to 17: nothing; async: 0:r6 (24 <= 24 ahead)
    # g1:     no site (chain 0 reads words 8..15 of what it fetched by g0's sync)
    # g2:     sync to 17: chain 0 has 32 - 16 = 16 < 17 ahead -> 0:r7 (all fetched)
    lens = np.array([[40, 24]])
    ngr = np.array([[5, 3]])
    cons = np.array([[[8, 8, 8, 8, 8], [8, 8, 8, 0, 0]]])
    rank = layout.request_ranks(lens, ngr, cons)
    assert rank[0, 0, :5].tolist() == [0, 2, 4, 6, 7]
    assert rank[0, 1, :3].tolist() == [1, 3, 5]


def test_hand_worked_escape_schedule():
    # A blob with escapes: every group is served, to 24 ahead.
    # Chain 0: 40 words, five groups of 8; chain 1: 64 words, groups of 20, 20, 8, 8, 8.
    # prime:  (0:r0 1:r1) (0:r2 1:r3) (0:r4 1:r5): both 24 ahead
    # g0:     sync: nothing; async 0:r6 1:r7 (both 24 <= 24 ahead); consume 8, 20
    # g1:     sync: chain 1 has 32 - 20 = 12 -> 1:r8 (20) -> 1:r9 (28); async: chain 0
    #         (32 - 8 = 24 ahead) 0:r10 (all fetched); consume 8, 20
    # g2:     sync: chain 1 has 48 - 40 = 8 -> 1:r11 (16) -> 1:r12 (24, all fetched)
    lens = np.array([[40, 64]])
    ngr = np.array([[5, 5]])
    cons = np.array([[[8, 8, 8, 8, 8], [20, 20, 8, 8, 8]]])
    rank = layout.request_ranks(lens, ngr, cons, esc=True)
    assert rank[0, 0, :5].tolist() == [0, 2, 4, 6, 10]
    assert rank[0, 1, :8].tolist() == [1, 3, 5, 7, 8, 9, 11, 12]
    # the same pattern under the escape-free schedule would read words before they land
    with pytest.raises(AssertionError):
        layout.request_ranks(lens, ngr, cons)


def test_hand_worked_tail_and_short_chain():
    # Chain 0: 32 words in groups of 8; chain 1: 20 words in groups of 5 (tail 4).
    # prime: (0:r0 1:r1) (0:r2 1:r3) (0:r4, chain 1 takes its tail: 20 fetched)
    # g0: async 0:r5 (24 <= 24 ahead); nothing else is ever asked for.
    lens = np.array([[32, 20]])
    ngr = np.array([[4, 4]])
    cons = np.array([[[8, 8, 8, 8], [5, 5, 5, 5]]])
    rank = layout.request_ranks(lens, ngr, cons)
    assert rank[0, 0, :4].tolist() == [0, 2, 4, 5]
    assert rank[0, 1, :2].tolist() == [1, 3]


@pytest.mark.parametrize("S,seed,esc", [(1, 0, False), (2, 1, False), (8, 2, False), (64, 4, False),
                                        (1, 5, True), (2, 6, True), (8, 7, True), (8, 3, True), (64, 8, True)])
def test_random_patterns_fetch_before_read(S, seed, esc):
    rng = np.random.default_rng(seed)
    T = 50
    steps = 512 // S
    ngr = np.full((T, S), steps)
    ngr[-1] = rng.integers(0, steps + 1, S)           # a ragged last tile
    live = np.arange(steps) < ngr[..., None]
    cons = rng.integers(0, 9, (T, S, steps))
    if esc:
        # groups with escapes consume up to 24 words; some chains escape in runs
        slow = (rng.random((T, S, steps)) < 0.05) | ((rng.random((T, S, 1)) < 0.1) & (rng.random((T, S, steps)) < 0.7))
        cons = np.where(slow, rng.integers(0, 25, (T, S, steps)), cons)
    cons = np.where(live, cons, 0)
    lens = cons.sum(axis=2)
    # asserts every word read was landed by a sync round and the ring never overfills
    rank = layout.request_ranks(lens, ngr, cons, esc=esc)
    nfull = lens // layout.CHUNK
    for t in range(T):
        got = np.concatenate([rank[t, j, :nfull[t, j]] for j in range(S)])
        assert np.array_equal(np.sort(got), np.arange(nfull[t].sum()))   # a permutation
        for j in range(S):
            assert (np.diff(rank[t, j, :nfull[t, j]]) > 0).all()          # in chain order


def test_schedule_catches_a_planted_overread():
    # the invariant check itself: a 25-word group is more than any group may consume
    # (24 with escapes); the first group's 25th word comes from g0's asynchronous round,
    # which lands only at the next site, so both schedules must refuse the pattern
    lens = np.array([[25]])
    ngr = np.array([[1]])
    cons = np.array([[[25]]])
    for esc in (False, True):
        with pytest.raises(AssertionError):
            layout.request_ranks(lens, ngr, cons, esc=esc)
    layout.request_ranks(np.array([[24]]), ngr, np.array([[[24]]]), esc=True)


def test_block_geometry():
    S = 8
    lens = np.array([17, 8, 0, 31, 5, 16, 9, 2] * 8 + [3, 40, 7, 1, 0, 0, 8, 15], dtype=np.int64)
    nfull, main_start, tail_pos, chunks = layout.block_geometry(lens, S)
    assert nfull.tolist()[:8] == [2, 1, 0, 3, 0, 2, 1, 0]
    per_tile = 8 * np.array([9] * 8 + [7])              # full-chunk words per tile
    assert main_start[:64].tolist() == list(np.repeat(np.cumsum(per_tile[:8]) - per_tile[:8], 8))
    assert main_start[64:].tolist() == [0] * 8
    tails = lens % 8
    assert tail_pos[0] == 8 * 72 and tail_pos[1] == 8 * 72 + 1 and tail_pos[3] == 8 * 72 + 1
    assert chunks.tolist() == [72 + -(-int(tails[:64].sum()) // 8), 7 + -(-int(tails[64:].sum()) // 8)]


# ---- the stream layout inverts: every chain's words come back from the blob

INVERT_CASES = [
    # (rows, cols, target bpp, chains per tile, seed): ragged last tiles, escapes at
    # 8 and 11 bpp, one chain per tile, all 64 chains of a block in one tile
    (256, 256, 3.5, 1, 0),
    (300, 520, 4.0, 8, 1),
    (200, 512, 8.0, 8, 2),
    (120, 512, 11.0, 4, 3),
    (200, 512, 3.0, 64, 4),
    (37, 13, 2.3, 2, 5),
]


@pytest.mark.parametrize("R,C,t,S,seed", INVERT_CASES)
def test_stream_gives_back_every_chains_words(monkeypatch, R, C, t, S, seed):
    """compress() places each chain's words (as encode_chains emitted them, in decoding
    order) at the positions the request schedule assigns; reading the blob by hand --
    blocks from their offsets, tiles' main areas in tile order, full chunk n of chain j
    at 8 * rank[t, j, n], then the tails in chain order, then zero padding -- must give
    every chain's words back exactly."""
    import synth
    import oracle
    from oracle import codec, numerics as nx

    seen = {}
    enc, place = codec.encode_chains, codec.build_stream

    def spy_encode(sym, model, cg):
        states, words, cons = enc(sym, model, cg)
        seen["words"] = [np.array(w, dtype=np.uint16) for w in words]
        seen["cons"] = np.array(cons)
        seen["cg"] = np.array(cg)
        return states, words, cons

    def spy_place(words, lens, rank, S_):
        seen["rank"] = np.array(rank)
        return place(words, lens, rank, S_)

    monkeypatch.setattr(codec, "encode_chains", spy_encode)
    monkeypatch.setattr(codec, "build_stream", spy_place)
    blob = oracle.compress(synth.rowscaled(R, C, seed), nx.DT_BF16, t, chains_per_tile=S)
    b = oracle.parse_blob(blob)
    words, rank = seen["words"], seen["rank"]
    n_ch = b.n_tiles * S
    lens = b.chain_lens.astype(np.int64)
    assert len(words) == n_ch
    assert [len(w) for w in words] == lens.tolist()

    # the ranks are the schedule's for the consumption the encoder recorded
    T_, steps = b.n_tiles, seen["cg"].shape[1]
    ngr = (seen["cg"] >= 0).sum(axis=1).reshape(T_, S)
    assert np.array_equal(layout.request_ranks(lens.reshape(T_, S), ngr, seen["cons"].reshape(T_, S, steps),
                                               esc=bool(b.flags & 1)), rank)

    stream = b.stream
    offs = [int(o) * 8 for o in b.block_offsets] + [len(stream)]
    for blk in range(b.n_blocks):
        c0, c1 = 64 * blk, min(64 * blk + 64, n_ch)
        pos = offs[blk]
        for tile in range(c0 // S, -(-c1 // S)):
            chunks = 0
            for j in range(S):
                c = tile * S + j
                for n in range(int(lens[c]) // 8):
                    p = pos + 8 * int(rank[tile, j, n])
                    assert np.array_equal(stream[p:p + 8], words[c][8 * n:8 * n + 8]), (c, n)
                    chunks += 1
            # the tile's ranks are exactly 0 .. chunks - 1
            got = sorted(int(rank[tile, j, n]) for j in range(S) for n in range(int(lens[tile * S + j]) // 8))
            assert got == list(range(chunks))
            pos += 8 * chunks
        for c in range(c0, c1):
            r = int(lens[c]) % 8
            assert np.array_equal(stream[pos:pos + r], words[c][len(words[c]) - r:]), c
            pos += r
        assert 0 <= offs[blk + 1] - pos < 8
        assert not stream[pos:offs[blk + 1]].any()
