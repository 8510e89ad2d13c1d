"""Pins for the stream layout's request schedule (oracle.layout): hand-worked
orders, the fetched-before-read invariant on random consumption patterns, and the
block geometry."""
import numpy as np
import pytest

from oracle import layout


def test_hand_worked_two_chains():
    # Chain 0: 40 words, five groups of 8, no escapes.
    # Chain 1: 64 words, groups of 20, 20, 8, 8, 8; groups 0 and 1 hold escapes.
    # prime:  rounds (0:r0 1:r1) (0:r2 1:r3) (0:r4 1:r5): both 24 ahead
    # g0:     service: no sync; async 0:r6 1:r7 (both had 24 <= 24 ahead)
    #         chain 1 escapes: 32 ahead >= 24, nothing; consumes 20 -> 12 ahead
    #         after: 1:r8 (20 ahead)
    # g1:     chain 1 escapes: 20 < 24 -> 1:r9 (28); consumes 20 -> 8 ahead
    #         after: 1:r10 (16), 1:r11 (24, all fetched)
    # g2:     service: chain 0 has 32 - 16 = 16 < 17 ahead -> 0:r12 (all fetched)
    lens = np.array([[40, 64]])
    ngr = np.array([[5, 5]])
    cons = np.array([[[8, 8, 8, 8, 8], [20, 20, 8, 8, 8]]])
    slow = np.zeros((1, 2, 5), dtype=bool)
    slow[0, 1, :2] = True
    rank = layout.request_ranks(lens, ngr, cons, slow)
    assert rank[0, 0, :5].tolist() == [0, 2, 4, 6, 12]
    assert rank[0, 1, :8].tolist() == [1, 3, 5, 7, 8, 9, 10, 11]


def test_hand_worked_tail_and_short_chain():
    # Chain 0: 32 words in groups of 8; chain 1: 20 words in groups of 5 (tail 4).
    # prime: (0:r0 1:r1) (0:r2 1:r3) (0:r4, chain 1 takes its tail: 20 fetched)
    # g0: async 0:r5 (24 <= 24 ahead); nothing else is ever asked for.
    lens = np.array([[32, 20]])
    ngr = np.array([[4, 4]])
    cons = np.array([[[8, 8, 8, 8], [5, 5, 5, 5]]])
    rank = layout.request_ranks(lens, ngr, cons, np.zeros((1, 2, 4), dtype=bool))
    assert rank[0, 0, :4].tolist() == [0, 2, 4, 5]
    assert rank[0, 1, :2].tolist() == [1, 3]


@pytest.mark.parametrize("S,seed", [(1, 0), (2, 1), (8, 2), (8, 3), (64, 4)])
def test_random_patterns_fetch_before_read(S, seed):
    rng = np.random.default_rng(seed)
    T = 50
    steps = 512 // S
    ngr = np.full((T, S), steps)
    ngr[-1] = rng.integers(0, steps + 1, S)           # a ragged last tile
    slow = (rng.random((T, S, steps)) < 0.05) & (np.arange(steps) < ngr[..., None])
    cons = np.where(slow, rng.integers(0, 25, (T, S, steps)), rng.integers(0, 9, (T, S, steps)))
    cons = np.where(np.arange(steps) < ngr[..., None], cons, 0)
    lens = cons.sum(axis=2)
    rank = layout.request_ranks(lens, ngr, cons, slow)    # asserts fetched-before-read
    nfull = lens // layout.CHUNK
    for t in range(T):
        got = np.concatenate([rank[t, j, :nfull[t, j]] for j in range(S)])
        assert np.array_equal(np.sort(got), np.arange(nfull[t].sum()))   # a permutation
        for j in range(S):
            assert (np.diff(rank[t, j, :nfull[t, j]]) > 0).all()          # in chain order


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
