"""The list checker used by the GPU selection tests, on rows built to be near
ties: it accepts the oracle's list and a list that differs only inside the
rounding band, and rejects a wrong list, a tie resolved to the higher index and
malformed rows."""
import numpy as np

import oracle
from tests.selection_check import judge_choice, judge_page_row, judge_token_row

D = 16
U = np.r_[np.ones(8), np.zeros(D - 8)]
DSTAR = D - 1          # the channel whose query-block sum is tiny
TINY = 2.0 ** -20


def _page_case(delta):
    """Query block 39 leans along U; page 5 too, and page 20 copies page 5 with
    one key changed by ``delta`` in channel DSTAR, where the query block sums to
    2^-20: the two scores differ by delta * 2^-20."""
    rng = np.random.default_rng(31)
    L, qb = 128 * 40, 39
    q = rng.standard_normal((1, L, 1, D))
    k = rng.standard_normal((1, L, 1, D))
    q[0, qb * 128:(qb + 1) * 128, 0] += U
    q[0, qb * 128:(qb + 1) * 128, 0, DSTAR] = 0.0
    q[0, qb * 128, 0, DSTAR] = TINY
    k[0, 5 * 128:6 * 128, 0] += 0.5 * U
    k[0, 20 * 128:21 * 128, 0] = k[0, 5 * 128:6 * 128, 0]
    k[0, 20 * 128, 0, DSTAR] += delta
    return q, k, qb


def _row(ids, width):
    r = np.full(width, -1, np.int32)
    r[:len(ids)] = sorted(ids)
    return r, len(ids)


def test_page_near_tie_accepts_both_sides_rejects_wrong():
    q, k, qb = _page_case(delta=1.0)
    idx, cnt, near = oracle.page_select(q, k, top_m=1)
    assert near[0, 0, qb], "the constructed row must be a near tie"
    base = oracle.window_blocks(qb)
    got = list(idx[0, 0, qb, :cnt[0, 0, qb]])
    assert got == sorted(base + [20])          # exact answer: page 20 is higher by 2^-20
    W = idx.shape[-1]
    assert judge_page_row(idx[0, 0, qb], int(cnt[0, 0, qb]), q, k, 0, 0, qb, 1) is None
    alt, n = _row(base + [5], W)               # inside the rounding band: a valid float answer
    assert judge_page_row(alt, n, q, k, 0, 0, qb, 1) is None
    wrong, n = _row(base + [7], W)             # a page far below the boundary
    assert judge_page_row(wrong, n, q, k, 0, 0, qb, 1) is not None
    missing, n = _row(base[1:] + [20, 7], W)   # window block 0 dropped
    assert judge_page_row(missing, n, q, k, 0, 0, qb, 1) is not None
    unsorted = np.array(list(reversed(sorted(base + [20]))) + [-1] * (W - len(base) - 1), np.int32)
    assert judge_page_row(unsorted, len(base) + 1, q, k, 0, 0, qb, 1) is not None
    junk = idx[0, 0, qb].copy()
    junk[-1] = 3                                # padding that is not -1
    assert judge_page_row(junk, int(cnt[0, 0, qb]), q, k, 0, 0, qb, 1) is not None


def test_page_exact_tie_must_go_to_lower_index():
    q, k, qb = _page_case(delta=0.0)
    idx, cnt, _ = oracle.page_select(q, k, top_m=1)
    base = oracle.window_blocks(qb)
    assert list(idx[0, 0, qb, :cnt[0, 0, qb]]) == sorted(base + [5])
    W = idx.shape[-1]
    assert judge_page_row(idx[0, 0, qb], int(cnt[0, 0, qb]), q, k, 0, 0, qb, 1) is None
    hi, n = _row(base + [20], W)
    assert "tie" in judge_page_row(hi, n, q, k, 0, 0, qb, 1)


def _token_case(delta):
    """Query block 29 leans along U; keys P1, P2 lean strongly, J1 less, and J2
    copies J1 with channel DSTAR changed by ``delta`` (query-block sum 2^-20)."""
    rng = np.random.default_rng(32)
    L, qb = 128 * 30, 29
    q = rng.standard_normal((1, L, 1, D))
    k = rng.standard_normal((1, L, 1, D))
    q[0, qb * 128:(qb + 1) * 128, 0] += U
    q[0, qb * 128:(qb + 1) * 128, 0, DSTAR] = 0.0
    q[0, qb * 128, 0, DSTAR] = TINY
    p1, p2, j1, j2 = 5 * 128 + 7, 5 * 128 + 90, 9 * 128 + 1, 9 * 128 + 100
    k[0, p1, 0] += 5 * U
    k[0, p2, 0] += 5 * U
    k[0, j1, 0] += 3 * U
    k[0, j2, 0] = k[0, j1, 0]
    k[0, j2, 0, DSTAR] += delta
    pages = sorted({0, 5, 9} | set(range(23, 30)))
    pidx = np.full((1, 1, 30, 10), -1, np.int32)
    pcnt = np.zeros((1, 1, 30), np.int32)
    pidx[0, 0, qb, :len(pages)] = pages
    pcnt[0, 0, qb] = len(pages)
    return q, k, qb, pidx, pcnt, (p1, p2, j1, j2)


def test_token_near_tie_accepts_both_sides_rejects_wrong():
    q, k, qb, pidx, pcnt, (p1, p2, j1, j2) = _token_case(delta=2.0 ** -6)
    tok, tcnt, near = oracle.token_select(q, k, pidx, pcnt, top_k=3)
    assert near[0, 0, qb], "the constructed row must be a near tie"
    assert list(tok[0, 0, qb, :3]) == [p1, p2, j2]
    pages = pidx[0, 0, qb, :pcnt[0, 0, qb]]
    assert judge_token_row(tok[0, 0, qb], 3, q, k, pages, 0, 0, qb, 3) is None
    assert judge_token_row(np.array([p1, p2, j1], np.int32), 3, q, k, pages, 0, 0, qb, 3) is None
    assert judge_token_row(np.array([p1, p2, j1 + 5], np.int32), 3, q, k, pages, 0, 0, qb, 3) is not None
    assert judge_token_row(np.array([p1, j1, j2], np.int32), 3, q, k, pages, 0, 0, qb, 3) is not None
    inwin = 25 * 128 + 3                        # a token of a window page is no candidate
    assert judge_token_row(np.array([p1, p2, inwin], np.int32), 3, q, k, pages, 0, 0, qb, 3) is not None
    assert judge_token_row(np.array([p1, p2], np.int32), 2, q, k, pages, 0, 0, qb, 3) is not None


def test_token_exact_tie_must_go_to_lower_index():
    q, k, qb, pidx, pcnt, (p1, p2, j1, j2) = _token_case(delta=0.0)
    tok, _, _ = oracle.token_select(q, k, pidx, pcnt, top_k=3)
    assert list(tok[0, 0, qb, :3]) == [p1, p2, j1]
    pages = pidx[0, 0, qb, :pcnt[0, 0, qb]]
    assert "tie" in judge_token_row(np.array([p1, p2, j2], np.int32), 3, q, k, pages, 0, 0, qb, 3)


def test_judge_choice_rules():
    from fractions import Fraction as F
    cands = [1, 2, 3, 4]
    exact = [F(10), F(9), F(9), F(1)]
    band = [0.0, 0.0, 0.0, 0.0]
    assert judge_choice({1, 2}, cands, exact, band, 2) is None
    assert judge_choice({1, 3}, cands, exact, band, 2) is not None     # tie to the higher index
    assert judge_choice({1, 4}, cands, exact, band, 2) is not None     # 9 beats 1
    assert judge_choice({1}, cands, exact, band, 2) is not None        # too few
    assert judge_choice({1, 5}, cands, exact, band, 2) is not None     # not a candidate
    assert judge_choice({1, 4}, cands, exact, [0.0, 0.0, 0.0, 4.0], 2) is not None
    assert judge_choice({1, 4}, cands, exact, [0.0, 4.0, 4.0, 4.0], 2) is None   # inside the band
