"""Float64 reference implementation (test infrastructure only; see package doc).

Array conventions (logical layouts; the oracle never looks at strides):

* q     [B, L, Hq, Dqk]   k [B, L, Hkv, Dqk]   v [B, L, Hkv, Dv]
* o     [B, L, Hq, Dv]    lse [B, Hq, L]       (natural log)
* query head h reads kv head  h // (Hq // Hkv).

Readings of the sources that the code below relies on (each is also listed in
the design notes of the repository):

* the window of query block qb is the union of the global blocks
  [0, n_global) and the local blocks [qb - n_local + 1, qb], clipped to
  [0, qb]; blocks are counted once (a 0/1 mask, "LoZA: ZigZag sparse
  attention" page, section 2.1, equation (2));
* inside the query's own block the rule is causal, key j <= query i,
  self included (same page, section 2.2.1);
* the scale is a caller-supplied constant, 1/sqrt(d) by default (same page,
  section 2.1, equation (1));
* rows at or beyond L do not exist and keys at or beyond L are never read.
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction

import numpy as np


@dataclass(frozen=True)
class Window:
    """Block-window geometry: 1 global + 7 local blocks of 128 tokens by default
    (QbitAI report on LongCat LoZA, sparse-window paragraph)."""
    block_size: int = 128
    n_global: int = 1
    n_local: int = 7

    @property
    def width(self) -> int:
        return self.n_global + self.n_local


DEFAULT_WINDOW = Window()


# ---------------------------------------------------------------------------
# block index
# ---------------------------------------------------------------------------

def window_blocks(qb: int, win: Window = DEFAULT_WINDOW) -> list[int]:
    """Ascending, distinct block ids readable from query block ``qb``."""
    glob = set(range(0, min(win.n_global, qb + 1)))
    local = set(range(max(0, qb - win.n_local + 1), qb + 1))
    return sorted(glob | local)


def block_index(n_qblocks: int, win: Window = DEFAULT_WINDOW):
    """idx int32 [n_qblocks, W] (ascending, -1 padded), cnt int32 [n_qblocks]."""
    W = win.width
    idx = np.full((n_qblocks, W), -1, np.int32)
    cnt = np.zeros(n_qblocks, np.int32)
    for qb in range(n_qblocks):
        ids = window_blocks(qb, win)
        idx[qb, :len(ids)] = ids
        cnt[qb] = len(ids)
    return idx, cnt


def block_index_seq(seq_lens, win: Window = DEFAULT_WINDOW):
    """Decode rows: the query of a sequence of length n sits at position n - 1."""
    seq_lens = np.asarray(seq_lens)
    W = win.width
    idx = np.full((len(seq_lens), W), -1, np.int32)
    cnt = np.zeros(len(seq_lens), np.int32)
    for b, n in enumerate(seq_lens):
        ids = window_blocks((int(n) - 1) // win.block_size, win)
        idx[b, :len(ids)] = ids
        cnt[b] = len(ids)
    return idx, cnt


# ---------------------------------------------------------------------------
# masked softmax attention, the plain definition
# ---------------------------------------------------------------------------

def _attend(qr: np.ndarray, kr: np.ndarray, vr: np.ndarray, allowed: np.ndarray, scale: float):
    """Softmax attention of rows ``qr`` [R, D] over keys ``kr`` [N, D] / values
    ``vr`` [N, Dv], restricted to ``allowed`` [R, N]; every row allows >= 1 key.

    s = scale * q.k ; m = max over allowed ; w = exp(s - m) ; o = sum w v / sum w ;
    lse = m + ln(sum w).
    """
    s = scale * (qr @ kr.T)
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=1, keepdims=True)
    o = (w @ vr) / l
    return o, m[:, 0] + np.log(l[:, 0])


def _kv_head(h: int, Hq: int, Hkv: int) -> int:
    return h // (Hq // Hkv)


def ssa_rows(q_rows, row0, k_seq, v_seq, scale, heads, Hq, win: Window = DEFAULT_WINDOW):
    """SSA output for rows ``row0 .. row0+R-1`` of ONE sequence.

    q_rows [R, len(heads), Dqk] are those rows for the query heads ``heads``;
    k_seq [L, Hkv, Dqk] / v_seq [L, Hkv, Dv] hold (at least) every key the rows
    may read.  The rows must lie in a single query block.
    Returns o [R, len(heads), Dv], lse [R, len(heads)].
    """
    q_rows = np.asarray(q_rows, np.float64)
    R = q_rows.shape[0]
    bs = win.block_size
    qb = row0 // bs
    assert (row0 + R - 1) // bs == qb, "rows must share one query block"
    L, Hkv = k_seq.shape[0], k_seq.shape[1]
    pos = np.concatenate([np.arange(t * bs, min((t + 1) * bs, L)) for t in window_blocks(qb, win)])
    rows = row0 + np.arange(R)
    allowed = pos[None, :] <= rows[:, None]
    o = np.empty((R, len(heads), v_seq.shape[2]))
    lse = np.empty((R, len(heads)))
    for n, h in enumerate(heads):
        g = _kv_head(h, Hq, Hkv)
        o[:, n], lse[:, n] = _attend(q_rows[:, n], np.asarray(k_seq[pos, g], np.float64),
                                     np.asarray(v_seq[pos, g], np.float64), allowed, scale)
    return o, lse


def ssa_attention(q, k, v, scale, win: Window = DEFAULT_WINDOW):
    """Full SSA output: o [B, L, Hq, Dv], lse [B, Hq, L]."""
    B, L, Hq, _ = q.shape
    Dv = v.shape[3]
    o = np.empty((B, L, Hq, Dv))
    lse = np.empty((B, Hq, L))
    heads = list(range(Hq))
    bs = win.block_size
    for b in range(B):
        for r0 in range(0, L, bs):
            r1 = min(r0 + bs, L)
            ob, lb = ssa_rows(q[b, r0:r1], r0, k[b], v[b], scale, heads, Hq, win)
            o[b, r0:r1] = ob
            lse[b, :, r0:r1] = lb.T
    return o, lse


def dense_causal_rows(q_rows, row0, k_seq, v_seq, scale, heads, Hq):
    """Causal attention (key j <= query i) for rows row0 .. row0+R-1 of one sequence."""
    q_rows = np.asarray(q_rows, np.float64)
    R = q_rows.shape[0]
    Hkv = k_seq.shape[1]
    end = row0 + R
    allowed = np.arange(end)[None, :] <= (row0 + np.arange(R))[:, None]
    o = np.empty((R, len(heads), v_seq.shape[2]))
    lse = np.empty((R, len(heads)))
    for n, h in enumerate(heads):
        g = _kv_head(h, Hq, Hkv)
        o[:, n], lse[:, n] = _attend(q_rows[:, n], np.asarray(k_seq[:end, g], np.float64),
                                     np.asarray(v_seq[:end, g], np.float64), allowed, scale)
    return o, lse


def dense_causal(q, k, v, scale, chunk: int = 128):
    B, L, Hq, _ = q.shape
    o = np.empty((B, L, Hq, v.shape[3]))
    lse = np.empty((B, Hq, L))
    heads = list(range(Hq))
    for b in range(B):
        for r0 in range(0, L, chunk):
            r1 = min(r0 + chunk, L)
            ob, lb = dense_causal_rows(q[b, r0:r1], r0, k[b], v[b], scale, heads, Hq)
            o[b, r0:r1] = ob
            lse[b, :, r0:r1] = lb.T
    return o, lse


def ssa_backward(q, k, v, do, scale, win: Window = DEFAULT_WINDOW):
    """Gradients of the SSA output with respect to q, k and v.

    For one query block and head, with P = softmax of the masked scaled scores
    (the forward above) and dO the incoming gradient of its output rows:
      dV += P^T dO ;  dP = dO V^T ;  dS = P * (dP - rowsum(P * dP)) ;
      dQ  = scale * dS K ;  dK += scale * dS^T Q
    -- the chain rule through o = P v and the softmax (whose Jacobian is
    diag(p) - p p^T).  Keys are summed over every query block and query head
    that reads them (the window's inverse map; a kv head serves Hq / Hkv query
    heads).  The sparse operator is part of training (LongCat sparse attention
    article, section 4: a custom, deterministic forward and backward).
    Returns dq [B, L, Hq, Dqk], dk [B, L, Hkv, Dqk], dv [B, L, Hkv, Dv].
    """
    B, L, Hq, Dqk = q.shape
    Hkv, Dv = k.shape[2], v.shape[3]
    bs = win.block_size
    dq = np.zeros((B, L, Hq, Dqk))
    dk = np.zeros((B, L, Hkv, Dqk))
    dv = np.zeros((B, L, Hkv, Dv))
    for b in range(B):
        for r0 in range(0, L, bs):
            r1 = min(r0 + bs, L)
            pos = np.concatenate([np.arange(t * bs, min((t + 1) * bs, L)) for t in window_blocks(r0 // bs, win)])
            allowed = pos[None, :] <= np.arange(r0, r1)[:, None]
            for h in range(Hq):
                g = _kv_head(h, Hq, Hkv)
                qr = np.asarray(q[b, r0:r1, h], np.float64)
                kr = np.asarray(k[b, pos, g], np.float64)
                vr = np.asarray(v[b, pos, g], np.float64)
                dor = np.asarray(do[b, r0:r1, h], np.float64)
                s = np.where(allowed, scale * (qr @ kr.T), -np.inf)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                dp = dor @ vr.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, r0:r1, h] = scale * (ds @ kr)
                np.add.at(dk[b, :, g], pos, scale * (ds.T @ qr))
                np.add.at(dv[b, :, g], pos, p.T @ dor)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# decode over a paged cache
# ---------------------------------------------------------------------------

def decode(q, k_pages, v_pages, block_table, seq_lens, scale, win: Window = DEFAULT_WINDOW,
           batches=None):
    """One new query per sequence over a paged cache.

    q [B, Hq, Dqk]; k_pages [P, Hkv, page, Dqk]; v_pages [P, Hkv, page, Dv]
    (page == block size); block_table [B, max_blocks] maps logical block ->
    physical page; seq_lens [B] counts the new token, whose key/value are
    already in the cache, so the query sits at position n - 1.
    Returns o [B, Hq, Dv], lse [B, Hq] (rows of ``batches`` only, if given).
    """
    B, Hq, _ = q.shape
    Hkv = k_pages.shape[1]
    bs = win.block_size
    assert k_pages.shape[2] == bs
    batches = range(B) if batches is None else batches
    o = np.full((B, Hq, v_pages.shape[3]), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b in batches:
        n = int(seq_lens[b])
        blocks = window_blocks((n - 1) // bs, win)
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            ks, vs = [], []
            for t in blocks:
                page = int(block_table[b, t])
                valid = min(bs, n - t * bs)
                ks.append(np.asarray(k_pages[page, g, :valid], np.float64))
                vs.append(np.asarray(v_pages[page, g, :valid], np.float64))
            kr, vr = np.concatenate(ks), np.concatenate(vs)
            qr = np.asarray(q[b, h], np.float64)[None, :]
            ob, lb = _attend(qr, kr, vr, np.ones((1, kr.shape[0]), bool), scale)
            o[b, h], lse[b, h] = ob[0], lb[0]
    return o, lse


def dense_decode(q, k_pages, v_pages, block_table, seq_lens, scale, batches=None):
    """Dense (full causal) attention of one new query per sequence over a paged
    cache: every cached key 0 .. n-1 -- the decode step of the layers LoZA keeps
    dense ("LoZA: ZigZag sparse attention" page, section 2.1, equation (1), with
    the causal rule of section 2.2.1).  Layouts as for ``decode``."""
    B, Hq, _ = q.shape
    Hkv = k_pages.shape[1]
    bs = k_pages.shape[2]
    batches = range(B) if batches is None else batches
    o = np.full((B, Hq, v_pages.shape[3]), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b in batches:
        n = int(seq_lens[b])
        blocks = range((n + bs - 1) // bs)
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            kr = np.concatenate([np.asarray(k_pages[int(block_table[b, t]), g, :min(bs, n - t * bs)], np.float64)
                                 for t in blocks])
            vr = np.concatenate([np.asarray(v_pages[int(block_table[b, t]), g, :min(bs, n - t * bs)], np.float64)
                                 for t in blocks])
            ob, lb = _attend(np.asarray(q[b, h], np.float64)[None, :], kr, vr, np.ones((1, kr.shape[0]), bool), scale)
            o[b, h], lse[b, h] = ob[0], lb[0]
    return o, lse


def chunk_prefill(q, k_pages, v_pages, block_table, seq_lens, scale, win: Window = DEFAULT_WINDOW,
                  batches=None):
    """A chunk of T new queries per sequence over a paged cache (chunked prefill).

    q [B, T, Hq, Dqk] holds the queries at positions n - T .. n - 1 of sequence
    b (n = seq_lens[b], which counts the chunk; the chunk's keys and values are
    already in the cache); k_pages / v_pages / block_table as for ``decode``.
    Each query i reads the window of its own block and keys j <= i: the same
    rule as ``ssa_rows``, with the keys gathered from the pages.
    Returns o [B, T, Hq, Dv], lse [B, Hq, T] (rows of ``batches`` only, if given).
    """
    B, T, Hq, _ = q.shape
    Hkv = k_pages.shape[1]
    bs = win.block_size
    assert k_pages.shape[2] == bs
    batches = range(B) if batches is None else batches
    o = np.full((B, T, Hq, v_pages.shape[3]), np.nan)
    lse = np.full((B, Hq, T), np.nan)
    for b in batches:
        n = int(seq_lens[b])
        q0 = n - T
        for qb in range(q0 // bs, (n - 1) // bs + 1):
            r0, r1 = max(q0, qb * bs), min(n, (qb + 1) * bs)  # the chunk's rows in this block
            blocks = window_blocks(qb, win)
            pos = np.concatenate([np.arange(t * bs, min((t + 1) * bs, n)) for t in blocks])
            allowed = pos[None, :] <= np.arange(r0, r1)[:, None]
            for h in range(Hq):
                g = _kv_head(h, Hq, Hkv)
                kr = np.concatenate([np.asarray(k_pages[int(block_table[b, t]), g, :min(bs, n - t * bs)], np.float64)
                                     for t in blocks])
                vr = np.concatenate([np.asarray(v_pages[int(block_table[b, t]), g, :min(bs, n - t * bs)], np.float64)
                                     for t in blocks])
                ob, lb = _attend(np.asarray(q[b, r0 - q0:r1 - q0, h], np.float64), kr, vr, allowed, scale)
                o[b, r0 - q0:r1 - q0, h] = ob
                lse[b, h, r0 - q0:r1 - q0] = lb
    return o, lse


# ---------------------------------------------------------------------------
# page selection (sink page + local pages + top-M scored pages)
# ---------------------------------------------------------------------------

def block_sums(x, block: int = 128):
    """Per-block sums over the sequence axis: [B, L, H, D] -> [B, nblocks, H, D] (fp64).

    The query-block-mean . page-mean score of the variant ranks pages exactly
    like the sum . sum score (a positive factor per query block), so sums are used.
    """
    x = np.asarray(x, np.float64)
    B, L, H, D = x.shape
    nb = (L + block - 1) // block
    out = np.zeros((B, nb, H, D))
    for t in range(nb):
        out[:, t] = x[:, t * block:min((t + 1) * block, L)].sum(axis=1)
    return out


def _exact_scores(qsum_exact, ksum_exact, cands):
    return [sum(a * b for a, b in zip(qsum_exact, ksum_exact[c])) for c in cands]


def page_select(q, k, win: Window = DEFAULT_WINDOW, top_m: int = 8, heads=None):
    """Block lists for page-selected attention (LongCat sparse attention article,
    section 3: sink + sliding window kept, top-M pages by a coarse page score).

    For query head h and query block qb the list is the window of ``qb`` plus the
    ``top_m`` candidate pages c in [n_global, qb - n_local] with the highest
    score <sum of q over block qb, sum of k over page c> (kv head of h); equal
    scores prefer the lower page.  When there are at most ``top_m`` candidates
    all are taken.  Lists are ascending and padded with -1 to
    W = n_global + n_local + top_m.

    ``heads`` restricts the work to some query heads (other rows stay -1 / 0).

    Returns idx int32 [B, Hq, nqb, W], cnt int32 [B, Hq, nqb] and
    near bool [B, Hq, nqb]: rows whose float64 scores left the top-M boundary
    within rounding error and were therefore re-decided with exact rationals
    (any selection within that error band is an equally valid float answer).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    bs = win.block_size
    nqb = (L + bs - 1) // bs
    W = win.width + top_m
    qs = block_sums(q, bs)
    ks = block_sums(k, bs)
    idx = np.full((B, Hq, nqb, W), -1, np.int32)
    cnt = np.zeros((B, Hq, nqb), np.int32)
    near = np.zeros((B, Hq, nqb), bool)
    for b in range(B):
        for h in (range(Hq) if heads is None else heads):
            g = _kv_head(h, Hq, Hkv)
            for qb in range(nqb):
                base = window_blocks(qb, win)
                c0, c1 = win.n_global, qb - win.n_local + 1   # candidates c0 .. c1-1
                cands = list(range(c0, c1))
                if len(cands) <= top_m:
                    chosen = cands
                elif top_m == 0:
                    chosen = []
                else:
                    a = qs[b, qb, h]
                    kc = ks[b, c0:c1, g]
                    sc = kc @ a
                    err = 1e-9 * (np.abs(kc) @ np.abs(a))
                    # descending score, then ascending page id
                    order = np.lexsort((np.arange(c0, c1), -sc))
                    sm, sn = sc[order[top_m - 1]], sc[order[top_m]]
                    if sm - sn > 2.0 * err.max():
                        chosen = [c0 + int(n) for n in order[:top_m]]
                    else:
                        near[b, h, qb] = True
                        rq = q[b, qb * bs:min((qb + 1) * bs, L), h]
                        qsum_exact = [sum(Fraction(float(x)) for x in rq[:, d]) for d in range(D)]
                        ksum_exact = {}
                        for c in cands:
                            rk = np.asarray(k[b, c * bs:(c + 1) * bs, g])
                            ksum_exact[c] = [sum(Fraction(float(x)) for x in rk[:, d]) for d in range(D)]
                        ex = _exact_scores(qsum_exact, ksum_exact, cands)
                        order = sorted(range(len(cands)), key=lambda n: (-ex[n], cands[n]))
                        chosen = [cands[n] for n in order[:top_m]]
                ids = sorted(set(base) | set(chosen))
                idx[b, h, qb, :len(ids)] = ids
                cnt[b, h, qb] = len(ids)
    return idx, cnt, near


def _exact_block_sum(rows):
    """Exact rational per-channel sum of the rows [n, D] (their float values are
    dyadic, so every partial sum is exact)."""
    rows = np.asarray(rows, np.float64)
    return [sum((Fraction(float(x)) for x in rows[:, d]), Fraction(0)) for d in range(rows.shape[1])]


def page_scores_exact(q, k, b, h, qb, win: Window = DEFAULT_WINDOW):
    """The first-stage scores of one row (batch b, query head h, query block qb)
    as exact rationals, for judging a selection that float rounding may have
    decided differently (LongCat sparse attention article, section 3,
    hierarchical indexing: a coarse score per 128-token page).

    Returns (cands, exact, band): the candidate pages [n_global, qb - n_local],
    their scores <sum of q over block qb, sum of k over page c> as Fractions,
    and per candidate the rounding band 1e-9 * sum |a_d b_d| that
    ``page_select`` certifies its float64 decisions against.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    _, L, Hq, _ = q.shape
    g = _kv_head(h, Hq, k.shape[2])
    bs = win.block_size
    cands = list(range(win.n_global, qb - win.n_local + 1))
    qsum = _exact_block_sum(q[b, qb * bs:min((qb + 1) * bs, L), h])
    af = np.asarray([float(x) for x in qsum])
    exact, band = [], []
    for c in cands:
        ksum = _exact_block_sum(k[b, c * bs:min((c + 1) * bs, L), g])
        exact.append(sum((a * x for a, x in zip(qsum, ksum)), Fraction(0)))
        band.append(1e-9 * float(np.abs(af) @ np.abs(np.asarray([float(x) for x in ksum]))))
    return cands, exact, band


def token_scores_exact(q, k, pages, b, h, qb, win: Window = DEFAULT_WINDOW):
    """The second-stage scores of one row as exact rationals (same section,
    second stage of hierarchical indexing, with the training-free score of
    ``token_select``): candidates are the tokens of the listed ``pages`` that
    lie outside the window of qb; score(j) = <sum of q over block qb, k_j>.

    Returns (cands, exact, band) like ``page_scores_exact``.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    _, L, Hq, _ = q.shape
    g = _kv_head(h, Hq, k.shape[2])
    bs = win.block_size
    inside = set(window_blocks(qb, win))
    pages = sorted({int(c) for c in pages if c >= 0 and int(c) not in inside})
    cands = [j for c in pages for j in range(c * bs, min((c + 1) * bs, L))]
    qsum = _exact_block_sum(q[b, qb * bs:min((qb + 1) * bs, L), h])
    af = np.asarray([float(x) for x in qsum])
    exact = [sum((a * Fraction(float(x)) for a, x in zip(qsum, k[b, j, g])), Fraction(0)) for j in cands]
    band = [1e-9 * float(np.abs(af) @ np.abs(k[b, j, g])) for j in cands]
    return cands, exact, band


def block_list_rows(q_rows, row0, k_seq, v_seq, scale, heads, Hq, lists, block: int = 128):
    """Attention of rows row0.. (one query block, one sequence) over explicit block
    lists: ``lists[n]`` is the list of readable block ids for query head heads[n];
    keys must also satisfy j <= i."""
    q_rows = np.asarray(q_rows, np.float64)
    R = q_rows.shape[0]
    L, Hkv = k_seq.shape[0], k_seq.shape[1]
    rows = row0 + np.arange(R)
    o = np.empty((R, len(heads), v_seq.shape[2]))
    lse = np.empty((R, len(heads)))
    for n, h in enumerate(heads):
        ids = [int(t) for t in lists[n] if t >= 0]
        pos = np.concatenate([np.arange(t * block, min((t + 1) * block, L)) for t in ids])
        allowed = pos[None, :] <= rows[:, None]
        g = _kv_head(h, Hq, Hkv)
        o[:, n], lse[:, n] = _attend(q_rows[:, n], np.asarray(k_seq[pos, g], np.float64),
                                     np.asarray(v_seq[pos, g], np.float64), allowed, scale)
    return o, lse


def block_list_attention(q, k, v, scale, idx, cnt, block: int = 128):
    """Full output of attention over per-(b, h, qb) lists idx [B, Hq, nqb, W]."""
    B, L, Hq, _ = q.shape
    o = np.empty((B, L, Hq, v.shape[3]))
    lse = np.empty((B, Hq, L))
    heads = list(range(Hq))
    for b in range(B):
        for r0 in range(0, L, block):
            r1 = min(r0 + block, L)
            qb = r0 // block
            lists = [idx[b, h, qb, :cnt[b, h, qb]] for h in heads]
            ob, lb = block_list_rows(q[b, r0:r1], r0, k[b], v[b], scale, heads, Hq, lists, block)
            o[b, r0:r1] = ob
            lse[b, :, r0:r1] = lb.T
    return o, lse


# ---------------------------------------------------------------------------
# hierarchical indexing, second stage: single tokens inside the recalled pages
# ---------------------------------------------------------------------------

def token_select(q, k, page_idx, page_cnt, win: Window = DEFAULT_WINDOW, top_k: int = 512, heads=None):
    """Second, fine-grained stage of hierarchical indexing (LongCat sparse
    attention article, section 3, hierarchical indexing: the first stage recalls
    the top-M pages, the second scores every token of those pages and keeps the
    top K).

    The pages leave the fine score to a trained indexer; the training-free
    reading used here scores a token j with the same query-block sum as the
    first stage:  score(j) = <sum of q over block qb, k_j>  (kv head of h).
    Candidates are the tokens of the listed pages that lie outside the window of
    qb (the window's pages are attended whole).  The K highest scores are kept,
    equal scores preferring the lower token; with at most K candidates all are
    kept.  Token lists are ascending and padded with -1 to width K.

    Returns tok int32 [B, Hq, nqb, K], tok_cnt int32 [B, Hq, nqb] and near bool
    [B, Hq, nqb] (rows whose float64 scores left the top-K boundary within
    rounding error and were re-decided with exact rationals).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    bs = win.block_size
    nqb = (L + bs - 1) // bs
    K = top_k
    tok = np.full((B, Hq, nqb, K), -1, np.int32)
    tcnt = np.zeros((B, Hq, nqb), np.int32)
    near = np.zeros((B, Hq, nqb), bool)
    qs = block_sums(q, bs)
    for b in range(B):
        for h in (range(Hq) if heads is None else heads):
            g = _kv_head(h, Hq, Hkv)
            for qb in range(nqb):
                inside = set(window_blocks(qb, win))
                pages = sorted(int(c) for c in page_idx[b, h, qb, :page_cnt[b, h, qb]] if c >= 0 and c not in inside)
                cand = [j for c in pages for j in range(c * bs, min((c + 1) * bs, L))]
                if len(cand) <= K:
                    chosen = cand
                else:
                    a = qs[b, qb, h]
                    kc = k[b, cand, g]
                    sc = kc @ a
                    err = 1e-9 * (np.abs(kc) @ np.abs(a))
                    order = np.lexsort((np.asarray(cand), -sc))  # descending score, then ascending token
                    if K == 0 or sc[order[K - 1]] - sc[order[K]] > 2.0 * err.max():
                        chosen = [cand[int(n)] for n in order[:K]]
                    else:
                        near[b, h, qb] = True
                        rq = q[b, qb * bs:min((qb + 1) * bs, L), h]
                        qsum_exact = [sum(Fraction(float(x)) for x in rq[:, d]) for d in range(D)]
                        ex = [sum(qe * Fraction(float(x)) for qe, x in zip(qsum_exact, k[b, j, g])) for j in cand]
                        order = sorted(range(len(cand)), key=lambda n: (-ex[n], cand[n]))
                        chosen = [cand[n] for n in order[:K]]
                chosen = sorted(chosen)
                tok[b, h, qb, :len(chosen)] = chosen
                tcnt[b, h, qb] = len(chosen)
    return tok, tcnt, near


def token_list_attention(q, k, v, scale, idx, cnt, tok, tok_cnt, block: int = 128, rows=None, heads=None):
    """Attention of each query over the listed blocks (causal, as in
    ``block_list_attention``) together with the listed single tokens of its
    query block; the tokens all precede the block, so no causal rule applies to
    them.  ``rows`` / ``heads`` (optional) restrict the work to some query
    blocks / query heads (other entries of o / lse are left NaN).

    Returns o [B, L, Hq, Dv] and lse [B, Hq, L].
    """
    q = np.asarray(q, np.float64)
    B, L, Hq, _ = q.shape
    Hkv = k.shape[2]
    nqb = (L + block - 1) // block
    o = np.full((B, L, Hq, v.shape[3]), np.nan)
    lse = np.full((B, Hq, L), np.nan)
    for b in range(B):
        for qb in (range(nqb) if rows is None else rows):
            r0, r1 = qb * block, min((qb + 1) * block, L)
            qi = np.arange(r0, r1)
            for h in (range(Hq) if heads is None else heads):
                g = _kv_head(h, Hq, Hkv)
                ids = [int(t) for t in idx[b, h, qb, :cnt[b, h, qb]] if t >= 0]
                pos = [j for t in ids for j in range(t * block, min((t + 1) * block, L))]
                toks = [int(t) for t in tok[b, h, qb, :tok_cnt[b, h, qb]]]
                keys = np.asarray(pos + toks, np.int64)
                allowed = np.concatenate([np.asarray(pos, np.int64)[None, :] <= qi[:, None],
                                          np.ones((r1 - r0, len(toks)), bool)], axis=1)
                oo, ll = _attend(q[b, r0:r1, h], np.asarray(k[b, keys, g], np.float64),
                                 np.asarray(v[b, keys, g], np.float64), allowed, scale)
                o[b, r0:r1, h] = oo
                lse[b, h, r0:r1] = ll
    return o, lse
