"""Pins of the oracle's candidate-block expansion ([Sparse indexer]
关键源码片段, _expand_candidates_kernel).

Nothing here calls the HIP path. Expected values: hand-worked rows
(tests/golden/worked_tokens.json, "candidate_expansion") and, exhaustively
over a tiny domain and on random rows, a restatement in tokens rather than
blocks: the sparse blocks written must cover exactly the tokens of the row's
range [ks, ke) that the candidate blocks cover, and end must count them.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(5656)


def i32(*v):
    return np.array(v, np.int32)


def _tokens_of_candidates(cand, ks, ke, ratio, sbk):
    """Tokens of [ks, ke) inside candidate blocks (ratio*sbk tokens each,
    counted from ks)."""
    width = ratio * sbk
    out = set()
    for c in cand:
        if c < 0:
            continue
        out.update(t for t in range(ks + c * width, ks + (c + 1) * width) if ks <= t < ke)
    return out


def _tokens_of_output(sparse, n_valid, ks, ke, sbk):
    """Tokens of [ks, ke) inside the first n_valid output blocks (the base
    ks // sbk removed, sbk tokens each counted from ks)."""
    base = ks // sbk
    out = set()
    for b in sparse[:n_valid]:
        rel = int(b) - base
        out.update(t for t in range(ks + rel * sbk, ks + (rel + 1) * sbk) if ks <= t < ke)
    return out


def _check_row(cand, ks, ke, ratio, sbk, sparse, end):
    base = ks // sbk
    want = _tokens_of_candidates(cand, ks, ke, ratio, sbk)
    # the kept blocks: each one touches the range, so the count of distinct
    # sparse blocks touched by the candidate tokens is n_valid (unique input)
    blocks = sorted({(t - ks) // sbk for t in want})
    n_valid = len(blocks)
    assert list(sparse[:n_valid]) == [b + base for b in blocks]
    pad = blocks[-1] + base if blocks else base
    assert all(int(v) == pad for v in sparse[n_valid:])
    assert _tokens_of_output(sparse, n_valid, ks, ke, sbk) == want
    assert end == len(want)


def test_worked_rows(golden):
    ce = golden["candidate_expansion"]
    cand = np.array([ce["candidates"]], np.int32)
    for row in ce["rows"]:
        sparse, end = oracle.expand_candidates(cand, i32(row["ks"]), i32(row["ke"]),
                                               row["ratio"], row["sbk"])
        assert sparse[0].tolist() == row["sparse"], row
        assert int(end[0]) == row["end"], row


@pytest.mark.parametrize("ratio,sbk", [(1, 8), (1, 16), (2, 8)])
def test_exhaustive_tiny_domain(ratio, sbk):
    """Every pair of distinct candidates in -1..5 (and -1, -1), every ks in
    0..2*sbk and ke in ks-1..ks+7*sbk: the token restatement holds."""
    pairs = [p for p in itertools.product(range(-1, 6), repeat=2) if p[0] != p[1] or p[0] < 0]
    ks_all = range(0, 2 * sbk + 1, 3)
    n = 0
    for ks in ks_all:
        kes = list(range(max(ks - 1, 0), ks + 7 * sbk + 1, 5))
        rows = [(p, ks, ke) for p in pairs for ke in kes]
        cand = np.array([r[0] for r in rows], np.int32)
        sparse, end = oracle.expand_candidates(cand, np.array([r[1] for r in rows], np.int32),
                                               np.array([r[2] for r in rows], np.int32),
                                               ratio, sbk)
        for i, (p, k0, k1) in enumerate(rows):
            _check_row(p, k0, k1, ratio, sbk, sparse[i], int(end[i]))
            n += 1
    assert n > 1000


@pytest.mark.parametrize("ratio,sbk", [(1, 16), (2, 8), (1, 8)])
def test_random_rows(ratio, sbk):
    rows, k = 200, 64
    ks = RNG.integers(0, 5000, rows).astype(np.int32)
    ke = (ks + RNG.integers(-10, 3000, rows)).astype(np.int32)
    cand = np.empty((rows, k), np.int32)
    for r in range(rows):
        cand[r] = RNG.permutation(k * 3)[:k] - 5   # unique, some negative, some too large
    sparse, end = oracle.expand_candidates(cand, ks, ke, ratio, sbk)
    for r in range(rows):
        _check_row(cand[r].tolist(), int(ks[r]), int(ke[r]), ratio, sbk, sparse[r], int(end[r]))


def test_duplicates_are_kept_and_sorted():
    """The page's kernel sorts without de-duplicating: duplicate candidates
    give duplicate sparse blocks, each counted in n_valid."""
    cand = np.array([[3, 1, 3, 1]], np.int32)
    sparse, end = oracle.expand_candidates(cand, i32(0), i32(64), 1, 16)
    assert sparse[0].tolist() == [1, 1, 3, 3]
    assert int(end[0]) == 3 * 16 + 16


def test_rejects_bad_parameters():
    cand = np.zeros((1, 4), np.int32)
    for ratio, sbk in ((3, 8), (0, 8), (1, 0)):
        with pytest.raises(ValueError):
            oracle.expand_candidates(cand, i32(0), i32(10), ratio, sbk)


def test_rows_at_the_int32_edge():
    """Rows whose range length ke - ks sits at 2^31 - SBK - 1, 2^31 - SBK and
    2^31 - SBK + 1, against hand-worked values. The page's kernel forms
    ke - ks + SBK - 1 in int32; past 2^31 - SBK that sum wraps negative and
    its program keeps no block (all outputs 0, end 0). The expansion here
    takes the range's blocks in exact integers, so those rows keep the
    blocks that cover [ks, ke), as they do below the edge.

    SBK 16, RATIO 1, ks 0, candidates (2^27 - 1, 7, 2^27 - 2, -1):
      ke = 2^31 - 17: max_block = ceil(ke / 16) = 2^27 - 1, so 7 and 2^27 - 2
        are kept; the last starts at token (2^27 - 2) * 16 = 2^31 - 32 and
        holds ke - (2^31 - 32) = 15 tokens of the range: end = 16 + 15 = 31.
      ke = 2^31 - 16: the same blocks; the last block is full: end = 32.
      ke = 2^31 - 15: max_block = 2^27, so 2^27 - 1 is kept too; it starts at
        2^31 - 16 and holds 1 token: end = 2 * 16 + 1 = 33.
    SBK 8, RATIO 2 (candidate c -> sparse blocks 2c, 2c + 1), ks 0,
    candidates (2^27 - 1, 3, -1, 2^27 + 5):
      ke = 2^31 - 8: max_block = 2^28 - 1; kept 6, 7, 2^28 - 2; the last
        starts at 2^31 - 16 and holds 8 tokens: end = 2 * 8 + 8 = 24.
      ke = 2^31 - 7: max_block = 2^28; 2^28 - 1 is kept too, starting at
        2^31 - 8 with 1 token: end = 3 * 8 + 1 = 25.
    """
    b27, b28 = 2 ** 27, 2 ** 28
    cand = np.array([[b27 - 1, 7, b27 - 2, -1]] * 3, np.int32)
    ke = i32(2 ** 31 - 17, 2 ** 31 - 16, 2 ** 31 - 15)
    sparse, end = oracle.expand_candidates(cand, i32(0, 0, 0), ke, 1, 16)
    assert sparse.tolist() == [[7, b27 - 2, b27 - 2, b27 - 2],
                               [7, b27 - 2, b27 - 2, b27 - 2],
                               [7, b27 - 2, b27 - 1, b27 - 1]]
    assert end.tolist() == [31, 32, 33]
    for r in range(3):
        _check_row(cand[r].tolist(), 0, int(ke[r]), 1, 16, sparse[r], int(end[r]))

    cand = np.array([[b27 - 1, 3, -1, b27 + 5]] * 2, np.int32)
    ke = i32(2 ** 31 - 8, 2 ** 31 - 7)
    sparse, end = oracle.expand_candidates(cand, i32(0, 0), ke, 2, 8)
    assert sparse.tolist() == [[6, 7, b28 - 2] + [b28 - 2] * 5,
                               [6, 7, b28 - 2, b28 - 1] + [b28 - 1] * 4]
    assert end.tolist() == [24, 25]
    for r in range(2):
        _check_row(cand[r].tolist(), 0, int(ke[r]), 2, 8, sparse[r], int(end[r]))
