"""Judging page and token lists against the oracle.

The lists of page selection and of the second hierarchical stage are decided
by float64 scores.  Where the oracle's own float64 decision is certified (the
margin at the top-M / top-K boundary is beyond rounding), the answer is unique
and a list must match it bit for bit.  On the other ("near") rows several lists
are correct float answers, and a list is accepted when, with the row's exact
rational scores:

* its count is the unique count (window part plus min(M, #candidates) pages,
  or min(K, #candidates) tokens);
* it is strictly ascending and padded with -1;
* a page list holds every block of the window, and its other entries are
  candidates; a token list holds candidates only;
* no unchosen candidate beats a chosen one by more than the two candidates'
  rounding bands;
* among exactly equal scores, every chosen candidate precedes every unchosen
  one (ties go to the lower index).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import oracle
from oracle import DEFAULT_WINDOW


def judge_choice(chosen, cands, exact, band, m):
    """None if the set ``chosen`` is a valid top-``m`` choice among ``cands``
    (exact scores ``exact``, rounding bands ``band``), else the reason."""
    chosen = set(int(c) for c in chosen)
    pos = {c: i for i, c in enumerate(cands)}
    if not chosen <= set(pos):
        return f"not candidates: {sorted(chosen - set(pos))[:5]}"
    if len(chosen) != min(m, len(cands)):
        return f"{len(chosen)} chosen, expected {min(m, len(cands))}"
    if len(chosen) == len(cands) or not chosen:
        return None
    low = min(exact[pos[c]] + Fraction(band[pos[c]]) for c in chosen)
    high = max(exact[pos[d]] - Fraction(band[pos[d]]) for d in cands if d not in chosen)
    if high > low:
        return "an unchosen candidate beats a chosen one beyond the rounding band"
    groups: dict = {}
    for c in cands:
        groups.setdefault(exact[pos[c]], []).append(c)
    for members in groups.values():
        if len(members) < 2:
            continue
        ins = [c for c in members if c in chosen]
        outs = [c for c in members if c not in chosen]
        if ins and outs and max(ins) > min(outs):
            return f"exact tie resolved to the higher index ({max(ins)} chosen, {min(outs)} not)"
    return None


def _listed(row, count):
    """The first ``count`` entries, or the reason the row is malformed."""
    row = np.asarray(row)
    head, tail = row[:count], row[count:]
    if (tail != -1).any():
        return None, "entries past the count are not -1"
    if count > 1 and not (np.diff(head) > 0).all():
        return None, "not strictly ascending"
    return [int(x) for x in head], None


def judge_page_row(row, count, q, k, b, h, qb, top_m, win=DEFAULT_WINDOW):
    """None if ``row`` (count ``count``) is a valid page list for this row."""
    listed, why = _listed(row, count)
    if why:
        return why
    base = oracle.window_blocks(qb, win)
    if not set(base) <= set(listed):
        return "window blocks missing"
    cands, exact, band = oracle.page_scores_exact(q, k, b, h, qb, win)
    if len(listed) != len(base) + min(top_m, len(cands)):
        return f"count {len(listed)}, expected {len(base) + min(top_m, len(cands))}"
    return judge_choice(set(listed) - set(base), cands, exact, band, top_m)


def judge_token_row(row, count, q, k, pages, b, h, qb, top_k, win=DEFAULT_WINDOW):
    """None if ``row`` (count ``count``) is a valid token list for this row,
    whose page list is ``pages``."""
    listed, why = _listed(row, count)
    if why:
        return why
    cands, exact, band = oracle.token_scores_exact(q, k, pages, b, h, qb, win)
    return judge_choice(listed, cands, exact, band, top_k)


def check_page_lists(idx, cnt, q, k, top_m, ridx, rcnt, near, heads=None, win=DEFAULT_WINDOW):
    """GPU page lists idx [B, Hq, nqb, W] / cnt [B, Hq, nqb] (numpy) against the
    oracle's (ridx, rcnt, near): counts everywhere, bit-exact lists on certified
    rows, judged lists on near rows.  Returns the number of near rows judged."""
    B, Hq, nqb, _ = idx.shape
    hs = range(Hq) if heads is None else heads
    judged = 0
    for b in range(B):
        for h in hs:
            assert np.array_equal(cnt[b, h], rcnt[b, h]), f"b {b} head {h}: counts differ"
            ok = ~near[b, h]
            bad = np.argwhere((idx[b, h] != ridx[b, h]).any(-1) & ok).ravel()
            assert len(bad) == 0, f"b {b} head {h}: certified rows {bad[:5].tolist()} differ"
            for qb in np.flatnonzero(near[b, h]):
                why = judge_page_row(idx[b, h, qb], int(cnt[b, h, qb]), q, k, b, h, int(qb), top_m, win)
                assert why is None, f"b {b} head {h} qb {qb}: {why}"
                judged += 1
    return judged


def check_token_lists(tok, tcnt, q, k, pidx, pcnt, top_k, rtok, rtcnt, near, heads=None, win=DEFAULT_WINDOW):
    """GPU token lists tok [B, Hq, nqb, K] / tcnt [B, Hq, nqb] against the
    oracle's second stage run over the same page lists (pidx, pcnt): counts
    everywhere, bit-exact lists on certified rows, judged lists on near rows.
    Returns the number of near rows judged."""
    B, Hq, nqb, _ = tok.shape
    hs = range(Hq) if heads is None else heads
    judged = 0
    for b in range(B):
        for h in hs:
            assert np.array_equal(tcnt[b, h], rtcnt[b, h]), f"b {b} head {h}: token counts differ"
            ok = ~near[b, h]
            bad = np.argwhere((tok[b, h] != rtok[b, h]).any(-1) & ok).ravel()
            assert len(bad) == 0, f"b {b} head {h}: certified rows {bad[:5].tolist()} differ"
            for qb in np.flatnonzero(near[b, h]):
                pages = pidx[b, h, qb, :pcnt[b, h, qb]]
                why = judge_token_row(tok[b, h, qb], int(tcnt[b, h, qb]), q, k, pages, b, h, int(qb), top_k, win)
                assert why is None, f"b {b} head {h} qb {qb}: {why}"
                judged += 1
    return judged
