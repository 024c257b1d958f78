"""Pins of the oracle's exact top-K selection.

Rules (SALS on Ascend, QSI top-k: exact, stable descending sort; Day 10·2
sparse top-k: ties go to the lower block index, the last block is always kept,
no padding when there are fewer blocks than k; Quest: sink page kept) are
checked against a brute-force Python sort on tiny inputs with planted ties.
"""
import itertools

import numpy as np
import pytest

import oracle


def brute(scores, L, unit_tokens, k, fh, ft):
    """Reference selection by full sort of (score desc, index asc)."""
    S = 16
    n = -(-L // unit_tokens)
    npg = -(-L // S)
    upu = unit_tokens // S
    if n <= fh + ft + k:
        keep = set(range(n))
    else:
        mid = sorted(range(fh, n - ft), key=lambda u: (-scores[u], u))
        keep = set(range(fh)) | set(range(n - ft, n)) | set(mid[:k])
    pages = [p for u in sorted(keep) for p in range(u * upu, min((u + 1) * upu, npg))]
    return pages


def _run(scores_rows, lens, unit_tokens, k, fh, ft):
    B = len(lens)
    mu = scores_rows.shape[-1]
    max_sel = min((k + fh + ft) * (unit_tokens // 16), -(-max(lens) // 16))
    max_sel = max(max_sel, 1)
    sel, num = oracle.select(scores_rows.reshape(B, 1, mu), np.array(lens), unit_tokens, k, fh, ft,
                             max_sel)
    return sel[:, 0], num[:, 0], max_sel


@pytest.mark.parametrize("unit_tokens", [16, 64])
def test_select_matches_bruteforce_with_ties(unit_tokens):
    rng = np.random.default_rng(1)
    for trial in range(300):
        n_units = int(rng.integers(1, 40))
        L = int(rng.integers((n_units - 1) * unit_tokens + 1, n_units * unit_tokens + 1))
        # few distinct values force exact ties
        vals = rng.choice(np.array([-1.0, 0.0, -0.0, 0.5, 2.0, 2.0000000001]), size=n_units)
        k = int(rng.integers(0, n_units + 3))
        fh = int(rng.integers(0, 3))
        ft = int(rng.integers(0, 3))
        sel, num, max_sel = _run(vals[None], [L], unit_tokens, k, fh, ft)
        want = brute(list(vals), L, unit_tokens, k, fh, ft)
        assert num[0] == len(want)
        assert list(sel[0, :num[0]]) == want
        assert np.all(sel[0, num[0]:] == -1)


def test_select_properties_random():
    rng = np.random.default_rng(2)
    for trial in range(200):
        n = int(rng.integers(3, 300))
        L = n * 16 - int(rng.integers(0, 16))
        s = rng.standard_normal(n)
        s[rng.integers(0, n, 5)] = s[0]  # ties
        k = int(rng.integers(1, 40))
        sel, num, _ = _run(s[None], [L], 16, k, 1, 1)
        got = list(sel[0, :num[0]])
        assert num[0] == min(k + 2, n)
        assert got == sorted(got) and len(set(got)) == len(got)
        assert 0 in got and n - 1 in got
        if n > k + 2:
            chosen = set(got) - {0, n - 1}
            rest = set(range(1, n - 1)) - chosen
            worst = min(chosen, key=lambda u: (s[u], -u))
            for u in rest:  # nothing left out beats something kept
                assert (s[u], -u) < (s[worst], -worst)


def test_negative_zero_ties_positive_zero():
    s = np.array([5.0, 0.0, -0.0, 0.0, -0.0, 5.0])
    sel, num, _ = _run(s[None], [96], 16, 2, 1, 1)
    assert list(sel[0, :num[0]]) == [0, 1, 2, 5]


def test_fewer_units_than_budget_selects_all_without_padding():
    s = np.array([3.0, 1.0, 2.0])
    sel, num, max_sel = _run(s[None], [40], 16, 126, 1, 1)
    assert num[0] == 3 and list(sel[0, :3]) == [0, 1, 2]


def test_sals_blocks_expand_to_pages_and_clip():
    # 5 blocks of 64 tokens; the sequence ends 3 pages into block 4
    L = 4 * 64 + 40
    s = np.array([0.1, 9.0, 0.2, 8.0, 0.0])
    sel, num, _ = _run(s[None], [L], 64, 1, 0, 2)
    # top-1 of blocks {0,1,2} is block 1; tail blocks 3 and 4
    assert list(sel[0, :num[0]]) == [4, 5, 6, 7, 12, 13, 14, 15, 16, 17, 18]


def test_k_zero_keeps_only_forced():
    s = np.arange(10, dtype=np.float64)
    sel, num, _ = _run(s[None], [160], 16, 0, 1, 1)
    assert list(sel[0, :num[0]]) == [0, 9]


def test_batch_rows_are_independent():
    rng = np.random.default_rng(3)
    lens = [16 * 20, 16 * 7 - 5, 1]
    mu = 20
    s = rng.standard_normal((3, mu))
    sel, num, max_sel = _run(s, lens, 16, 4, 1, 1)
    for b in range(3):
        want = brute(list(s[b]), lens[b], 16, 4, 1, 1)
        assert list(sel[b, :num[b]]) == want
