"""Pins of the float64 oracle against facts that do not come from the oracle.

* brute force: pure-Python loops over an explicit mask that is built by walking
  back from the query's block (the window described in the QbitAI report on
  LongCat LoZA: one global block plus the seven most recent blocks of 128
  tokens), with math.exp and no max subtraction;
* the dense special case against torch's own scaled_dot_product_attention;
* closed forms: block counts, keys per query, total pairs, lse of a zero query;
* structural outputs: one-hot values per block, constant values, the first row;
* decode of a sequence of length n == row n - 1 of the prefill on the same data;
* a chunk of queries over a paged cache == brute force over the cached sequence;
* dense decode over a paged cache == the last row of the dense causal attention;
* gradients == central finite differences of the forward on tiny inputs, and ==
  torch's autograd through an explicitly masked softmax at the real window;
* page selection re-decided with exact rationals on tiny inputs.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import Window

RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------------------
# independent brute force
# ---------------------------------------------------------------------------

def brute_window_keys(i, bs, n_global, n_local):
    """Keys a query i may read: walk back n_local blocks from its own block, add
    the global blocks, keep causally earlier keys."""
    qb = i // bs
    blocks = []
    t = qb
    while t >= 0 and len(blocks) < n_local:
        blocks.append(t)
        t -= 1
    for g in range(n_global):
        if g <= qb and g not in blocks:
            blocks.append(g)
    return [j for j in range(i + 1) if j // bs in blocks]


def brute_rows(q, k, v, scale, rows, keys_of):
    """Pure-Python attention for the listed rows; no max subtraction (inputs are
    small enough that exp never overflows)."""
    B, L, Hq, D = q.shape
    Hkv, Dv = k.shape[2], v.shape[3]
    out = {}
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in rows:
                keys = keys_of(i)
                w = [math.exp(scale * math.fsum(float(q[b, i, h, c]) * float(k[b, j, g, c]) for c in range(D)))
                     for j in keys]
                den = math.fsum(w)
                o = [math.fsum(w[n] * float(v[b, j, g, c]) for n, j in enumerate(keys)) / den for c in range(Dv)]
                out[(b, h, i)] = (np.array(o), math.log(den))
    return out


@pytest.mark.parametrize("L,bs,ng,nl,Hq,Hkv", [
    (37, 4, 1, 3, 2, 1),   # ragged, GQA 2:1
    (40, 4, 1, 3, 2, 2),
    (29, 4, 2, 2, 1, 1),   # two global blocks
    (17, 8, 1, 7, 1, 1),   # L below the window: dense
])
def test_ssa_bruteforce_small(L, bs, ng, nl, Hq, Hkv):
    D, Dv = 3, 2
    q = RNG.standard_normal((1, L, Hq, D))
    k = RNG.standard_normal((1, L, Hkv, D))
    v = RNG.standard_normal((1, L, Hkv, Dv))
    win = Window(bs, ng, nl)
    o, lse = oracle.ssa_attention(q, k, v, 0.7, win)
    ref = brute_rows(q, k, v, 0.7, range(L), lambda i: brute_window_keys(i, bs, ng, nl))
    for (b, h, i), (ob, lb) in ref.items():
        np.testing.assert_allclose(o[b, i, h], ob, rtol=1e-12, atol=1e-12)
        assert abs(lse[b, h, i] - lb) < 1e-12


def test_ssa_bruteforce_real_geometry():
    """Real window (128-token blocks, 1 + 7) at L = 2304, on rows chosen around
    every block edge that changes the window, and the ragged end."""
    L, D = 2304, 2
    q = RNG.standard_normal((1, L, 1, D))
    k = RNG.standard_normal((1, L, 1, D))
    v = RNG.standard_normal((1, L, 1, D))
    rows = [0, 1, 127, 128, 895, 896, 1023, 1024, 1025, 1151, 1152, 1279, 2047, 2048, 2303]
    o, lse = oracle.ssa_attention(q, k, v, 1 / math.sqrt(D))
    ref = brute_rows(q, k, v, 1 / math.sqrt(D), rows, lambda i: brute_window_keys(i, 128, 1, 7))
    for (b, h, i), (ob, lb) in ref.items():
        np.testing.assert_allclose(o[b, i, h], ob, rtol=1e-11, atol=1e-12)
        assert abs(lse[b, h, i] - lb) < 1e-11


# ---------------------------------------------------------------------------
# library routine: torch's attention on the dense special case and with a mask
# ---------------------------------------------------------------------------

def torch_sdpa(q, k, v, scale, mask=None, causal=False):
    Hq, Hkv = q.shape[2], k.shape[2]
    rep = Hq // Hkv
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(rep, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(rep, dim=1)
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=causal, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("L", [1, 100, 777, 1024])
def test_short_sequences_equal_textbook_causal(L):
    """For L <= 1024 every key before the query lies in the window, so SSA is
    textbook causal attention (and so is the separately written dense oracle)."""
    D = 16
    q = RNG.standard_normal((1, L, 2, D))
    k = RNG.standard_normal((1, L, 2, D))
    v = RNG.standard_normal((1, L, 2, 8))
    ref = torch_sdpa(q, k, v, 0.25, causal=True)
    o_s, _ = oracle.ssa_attention(q, k, v, 0.25)
    o_d, _ = oracle.dense_causal(q, k, v, 0.25)
    np.testing.assert_allclose(o_s, ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(o_d, ref, rtol=1e-10, atol=1e-12)


def test_dense_causal_long_matches_torch():
    L, D = 1500, 8
    q = RNG.standard_normal((1, L, 2, D))
    k = RNG.standard_normal((1, L, 1, D))
    v = RNG.standard_normal((1, L, 1, 4))
    ref = torch_sdpa(q, k, v, 0.3, causal=True)
    o_d, _ = oracle.dense_causal(q, k, v, 0.3)
    np.testing.assert_allclose(o_d, ref, rtol=1e-10, atol=1e-12)


def test_ssa_long_matches_torch_with_walked_mask():
    L, D = 1700, 16
    q = RNG.standard_normal((1, L, 2, D))
    k = RNG.standard_normal((1, L, 2, D))
    v = RNG.standard_normal((1, L, 2, 16))
    mask = np.zeros((L, L), bool)
    for i in range(L):
        mask[i, brute_window_keys(i, 128, 1, 7)] = True
    ref = torch_sdpa(q, k, v, 1 / 4, mask=mask)
    o, _ = oracle.ssa_attention(q, k, v, 1 / 4)
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def nkeys_closed(i):
    """Keys per query for the default window: i + 1 below 1024, else one full
    global block + 6 full local blocks + the causal part of the own block."""
    return i + 1 if i < 1024 else 128 + 6 * 128 + (i % 128) + 1


def pairs_closed(L):
    if L <= 1024:
        return L * (L + 1) // 2
    assert L % 128 == 0
    return 524800 + (1921 * (L - 1024)) // 2


def test_block_index_closed_form():
    idx, cnt = oracle.block_index(300)
    for qb in range(300):
        assert cnt[qb] == min(qb + 1, 8)
        row = list(idx[qb, :cnt[qb]])
        assert row == sorted(set(row))
        assert 0 in row and qb in row
        assert all(x == -1 for x in idx[qb, cnt[qb]:])
        assert max(row) == qb and (qb < 7 or min(r for r in row if r > 0) == qb - 6)


def test_block_index_seq_matches_rows():
    lens = np.array([1, 127, 128, 129, 1024, 1025, 65536, 131072])
    idx, cnt = oracle.block_index_seq(lens)
    ridx, rcnt = oracle.block_index(1024)
    for b, n in enumerate(lens):
        qb = (n - 1) // 128
        assert list(idx[b]) == list(ridx[qb]) and cnt[b] == rcnt[qb]


@pytest.mark.parametrize("L,expect", [(2048, 1508352), (32768, 31014912), (131072, 125435904),
                                      (262144, 251330560), (1024, 524800)])
def test_total_pairs_closed_form(L, expect):
    """Pairs per head from the block index (blocks below the query block are
    full, the own block is causal) equal the closed form; the window never
    exceeds S = 1024 keys (QbitAI report: window fixed at 1024 tokens)."""
    nqb = L // 128
    idx, cnt = oracle.block_index(nqb)
    total = 0
    for qb in range(nqb):
        full = cnt[qb] - 1
        total += 128 * 128 * full + 128 * 129 // 2
        assert 128 * cnt[qb] <= 1024
    assert total == expect == pairs_closed(L)


def test_zero_query_lse_counts_keys_and_onehot_blocks():
    """q = 0 makes every allowed key weigh the same: lse = ln(#keys) and, with
    one-hot values per block, o = (#keys of that block)/(#keys)."""
    L, D = 1408 + 37, 4
    nb = (L + 127) // 128
    q = np.zeros((1, L, 1, D))
    k = RNG.standard_normal((1, L, 1, D))
    v = np.zeros((1, L, 1, nb))
    for j in range(L):
        v[0, j, 0, j // 128] = 1.0
    o, lse = oracle.ssa_attention(q, k, v, 0.1)
    for i in range(L):
        n = nkeys_closed(i)
        assert abs(lse[0, 0, i] - math.log(n)) < 1e-12
        qb = i // 128
        for t in range(nb):
            if t == qb:
                expect = (i % 128) + 1
            elif t == 0 or qb - 6 <= t < qb:
                expect = 128
            else:
                expect = 0
            assert abs(o[0, i, 0, t] - expect / n) < 1e-13


def test_constant_values_and_first_row():
    L = 1300
    q = RNG.standard_normal((1, L, 1, 8))
    k = RNG.standard_normal((1, L, 1, 8))
    v = np.broadcast_to(np.array([1.5, -2.0, 0.25]), (1, L, 1, 3)).copy()
    o, _ = oracle.ssa_attention(q, k, v, 0.5)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-14)  # softmax weights sum to 1
    v2 = RNG.standard_normal((1, L, 1, 3))
    o2, lse2 = oracle.ssa_attention(q, k, v2, 0.5)
    np.testing.assert_allclose(o2[0, 0, 0], v2[0, 0, 0], rtol=0, atol=1e-15)
    assert abs(lse2[0, 0, 0] - 0.5 * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-14


# ---------------------------------------------------------------------------
# decode == last prefill row
# ---------------------------------------------------------------------------

def _paged(k_seq, bs, rng, P_extra=5):
    """Scatter one sequence [L, H, D] into pages [P, H, bs, D] via a random table."""
    L, H, D = k_seq.shape
    nblk = (L + bs - 1) // bs
    P = nblk + P_extra
    perm = rng.permutation(P)[:nblk]
    pages = np.full((P, H, bs, D), np.nan)
    for t in range(nblk):
        rows = k_seq[t * bs:min((t + 1) * bs, L)]
        pages[perm[t], :, :rows.shape[0]] = rows.transpose(1, 0, 2)
    return pages, perm


@pytest.mark.parametrize("n,Hq,Hkv", [(1, 2, 2), (200, 4, 2), (1024, 2, 1), (1025, 2, 2), (2000, 2, 2)])
def test_decode_equals_prefill_last_row(n, Hq, Hkv):
    rng = np.random.default_rng(n)
    D, Dv = 8, 6
    q = rng.standard_normal((1, n, Hq, D))
    k = rng.standard_normal((1, n, Hkv, D))
    v = rng.standard_normal((1, n, Hkv, Dv))
    o_p, lse_p = oracle.ssa_attention(q, k, v, 0.3)
    kp, perm = _paged(k[0], 128, rng)
    vp = np.full((kp.shape[0], Hkv, 128, Dv), np.nan)
    for t in range((n + 127) // 128):
        rows = v[0, t * 128:min((t + 1) * 128, n)]
        vp[perm[t], :, :rows.shape[0]] = rows.transpose(1, 0, 2)
    bt = np.full((1, 16), -1, np.int32)
    bt[0, :len(perm)] = perm
    o_d, lse_d = oracle.decode(q[:, n - 1], kp, vp, bt, np.array([n]), 0.3)
    np.testing.assert_allclose(o_d[0], o_p[0, n - 1], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse_d[0], lse_p[0, :, n - 1], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("n,Hq,Hkv", [(1, 2, 2), (300, 4, 2), (1500, 2, 1)])
def test_dense_decode_equals_dense_last_row(n, Hq, Hkv):
    rng = np.random.default_rng(700 + n)
    D, Dv = 8, 6
    q = rng.standard_normal((1, n, Hq, D))
    k = rng.standard_normal((1, n, Hkv, D))
    v = rng.standard_normal((1, n, Hkv, Dv))
    o_p, lse_p = oracle.dense_causal(q, k, v, 0.3)
    kp, vp, perm = _paged_kv(k[0], v[0], 128, rng)
    bt = np.full((1, 16), -1, np.int32)
    bt[0, :len(perm)] = perm
    o_d, lse_d = oracle.dense_decode(q[:, n - 1], kp, vp, bt, np.array([n]), 0.3)
    np.testing.assert_allclose(o_d[0], o_p[0, n - 1], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse_d[0], lse_p[0, :, n - 1], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# chunked prefill over a paged cache == brute force over the cached sequence
# ---------------------------------------------------------------------------

def _paged_kv(k_seq, v_seq, bs, rng, P_extra=5):
    """Scatter one sequence's keys [n, H, D] and values [n, H, Dv] into NaN-filled
    pages through one random table; returns pages and the table row."""
    kp, perm = _paged(k_seq, bs, rng, P_extra)
    n, H, Dv = v_seq.shape
    vp = np.full((kp.shape[0], H, bs, Dv), np.nan)
    for t in range((n + bs - 1) // bs):
        rows = v_seq[t * bs:min((t + 1) * bs, n)]
        vp[perm[t], :, :rows.shape[0]] = rows.transpose(1, 0, 2)
    return kp, vp, perm


@pytest.mark.parametrize("n,T,bs,ng,nl,Hq,Hkv", [
    (37, 9, 4, 1, 3, 2, 1),    # chunk crosses two blocks, ragged end, GQA 2:1
    (40, 40, 4, 1, 3, 1, 1),   # the whole sequence
    (29, 1, 4, 2, 2, 2, 2),    # one query (a decode step), two global blocks
    (33, 6, 4, 1, 3, 1, 1),    # chunk starts mid-block
])
def test_chunk_prefill_bruteforce_small(n, T, bs, ng, nl, Hq, Hkv):
    rng = np.random.default_rng(1000 + n + T)
    D, Dv = 3, 2
    q = rng.standard_normal((1, n, Hq, D))
    k = rng.standard_normal((1, n, Hkv, D))
    v = rng.standard_normal((1, n, Hkv, Dv))
    win = Window(bs, ng, nl)
    kp, vp, perm = _paged_kv(k[0], v[0], bs, rng)
    bt = np.full((1, len(perm) + 3), -1, np.int32)
    bt[0, :len(perm)] = perm
    o, lse = oracle.chunk_prefill(q[:, n - T:], kp, vp, bt, np.array([n]), 0.7, win)
    ref = brute_rows(q, k, v, 0.7, range(n - T, n), lambda i: brute_window_keys(i, bs, ng, nl))
    for (b, h, i), (ob, lb) in ref.items():
        np.testing.assert_allclose(o[b, i - (n - T), h], ob, rtol=1e-12, atol=1e-12)
        assert abs(lse[b, h, i - (n - T)] - lb) < 1e-12


def test_chunk_prefill_bruteforce_real_geometry():
    """128-token blocks, 1 + 7: a 700-query chunk ending at n = 2304 (it starts
    mid-block and spans six query blocks); rows at every window edge."""
    rng = np.random.default_rng(77)
    n, T, D = 2304, 700, 2
    q = rng.standard_normal((1, n, 1, D))
    k = rng.standard_normal((1, n, 1, D))
    v = rng.standard_normal((1, n, 1, D))
    kp, vp, perm = _paged_kv(k[0], v[0], 128, rng)
    bt = perm[None, :].astype(np.int32)
    o, lse = oracle.chunk_prefill(q[:, n - T:], kp, vp, bt, np.array([n]), 1 / math.sqrt(D))
    rows = [1604, 1605, 1663, 1664, 1791, 1792, 2047, 2048, 2175, 2176, 2303]
    ref = brute_rows(q, k, v, 1 / math.sqrt(D), rows, lambda i: brute_window_keys(i, 128, 1, 7))
    for (b, h, i), (ob, lb) in ref.items():
        np.testing.assert_allclose(o[b, i - (n - T), h], ob, rtol=1e-11, atol=1e-12)
        assert abs(lse[b, h, i - (n - T)] - lb) < 1e-11


# ---------------------------------------------------------------------------
# backward: central finite differences of the (pinned) forward, and torch's
# autograd through an explicitly masked softmax attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("L,bs,ng,nl,Hq,Hkv", [
    (13, 4, 1, 3, 2, 1),   # ragged, GQA 2:1: a kv head sums both query heads
    (16, 4, 2, 2, 1, 1),   # two global blocks
])
def test_backward_finite_differences(L, bs, ng, nl, Hq, Hkv):
    rng = np.random.default_rng(500 + L)
    D, Dv, scale = 3, 2, 0.6
    win = Window(bs, ng, nl)
    q = rng.standard_normal((1, L, Hq, D))
    k = rng.standard_normal((1, L, Hkv, D))
    v = rng.standard_normal((1, L, Hkv, Dv))
    g = rng.standard_normal((1, L, Hq, Dv))  # loss = sum(o * g), so dO = g

    def loss(q_, k_, v_):
        return float((oracle.ssa_attention(q_, k_, v_, scale, win)[0] * g).sum())

    dq, dk, dv = oracle.ssa_backward(q, k, v, g, scale, win)
    eps = 1e-6
    for x, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-7 * max(1.0, abs(fd)), (which, idx, fd, grad[idx])


def test_backward_matches_torch_autograd_walked_mask():
    """Real window at L = 1300 (block 0 read by every query block, local blocks
    by the next 7), GQA 2:1, against torch autograd in float64."""
    L, D, Hq, Hkv = 1300, 8, 2, 1
    rng = np.random.default_rng(901)
    q = rng.standard_normal((1, L, Hq, D))
    k = rng.standard_normal((1, L, Hkv, D))
    v = rng.standard_normal((1, L, Hkv, D))
    g = rng.standard_normal((1, L, Hq, D))
    mask = np.zeros((L, L), bool)
    for i in range(L):
        mask[i, brute_window_keys(i, 128, 1, 7)] = True
    tq, tk, tv = (torch.tensor(x[0], dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    m = torch.tensor(mask)
    out = []
    for h in range(Hq):
        s = (tq[:, h] @ tk[:, 0].T) * 0.3
        p = torch.softmax(s.masked_fill(~m, float("-inf")), dim=-1)
        out.append(p @ tv[:, 0])
    (torch.stack(out, dim=1) * torch.tensor(g[0])).sum().backward()
    dq, dk, dv = oracle.ssa_backward(q, k, v, g, 0.3)
    np.testing.assert_allclose(dq[0], tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk[0], tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv[0], tv.grad.numpy(), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# page selection
# ---------------------------------------------------------------------------

def test_page_select_short_is_dense():
    """With at most top_m candidates every earlier page is kept: L <= 2048 is dense."""
    L = 2048 + 50
    q = RNG.standard_normal((1, L, 2, 8))
    k = RNG.standard_normal((1, L, 1, 8))
    idx, cnt, near = oracle.page_select(q, k, top_m=8)
    for qb in range(16):
        for h in range(2):
            assert list(idx[0, h, qb, :cnt[0, h, qb]]) == list(range(qb + 1))
    assert cnt[0, 0, 16] == 16 and not near.any()


def test_page_select_bruteforce_exact_tiny():
    """Tiny geometry (block 4, 1 global, 2 local, top 2): every row re-decided by
    enumerating the candidates with exact rational scores."""
    bs, ng, nl, M = 4, 1, 2, 2
    win = Window(bs, ng, nl)
    L, D = 53, 3
    q = np.round(RNG.standard_normal((1, L, 2, D)) * 8) / 8
    k = np.round(RNG.standard_normal((1, L, 1, D)) * 8) / 8
    idx, cnt, _ = oracle.page_select(q, k, win, top_m=M)
    for h in range(2):
        for qb in range((L + bs - 1) // bs):
            rows = range(qb * bs, min((qb + 1) * bs, L))
            qsum = [sum(Fraction(float(q[0, i, h, c])) for i in rows) for c in range(D)]
            base = set(range(max(0, qb - nl + 1), qb + 1)) | ({0} if qb >= 0 else set())
            cands = [c for c in range(1, qb + 1) if c not in base]
            score = {c: sum(qsum[d] * sum(Fraction(float(k[0, j, 0, d])) for j in range(c * bs, (c + 1) * bs))
                            for d in range(D)) for c in cands}
            best = sorted(cands, key=lambda c: (-score[c], c))[:M]
            want = sorted(base | set(best))
            assert list(idx[0, h, qb, :cnt[0, h, qb]]) == want


def test_page_select_planted_and_ties():
    """A page whose keys share a direction with the query block is selected; an
    exact duplicate of the best page loses the tie to the lower index."""
    rng = np.random.default_rng(7)
    L, D = 128 * 40, 16
    q = rng.standard_normal((1, L, 1, D))
    k = rng.standard_normal((1, L, 1, D))
    u = rng.standard_normal(D)
    qb = 39
    q[0, qb * 128:(qb + 1) * 128, 0] += u
    k[0, 5 * 128:6 * 128, 0] += u            # planted page 5
    k[0, 20 * 128:21 * 128, 0] = k[0, 5 * 128:6 * 128, 0]   # exact duplicate at 20
    idx, cnt, near = oracle.page_select(q, k, top_m=1)
    row = list(idx[0, 0, qb, :cnt[0, 0, qb]])
    assert 5 in row and 20 not in row
    idx2, cnt2, _ = oracle.page_select(q, k, top_m=2)
    row2 = list(idx2[0, 0, qb, :cnt2[0, 0, qb]])
    assert 5 in row2 and 20 in row2


def test_block_list_attention_with_window_lists_is_ssa():
    L = 1600
    q = RNG.standard_normal((1, L, 2, 8))
    k = RNG.standard_normal((1, L, 2, 8))
    v = RNG.standard_normal((1, L, 2, 8))
    idx, cnt = oracle.block_index((L + 127) // 128)
    nqb = idx.shape[0]
    idx4 = np.broadcast_to(idx[None, None], (1, 2, nqb, 8))
    cnt3 = np.broadcast_to(cnt[None, None], (1, 2, nqb))
    o1, l1 = oracle.block_list_attention(q, k, v, 0.2, idx4, cnt3)
    o2, l2 = oracle.ssa_attention(q, k, v, 0.2)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# hierarchical indexing, second stage (tokens inside the recalled pages)
# ---------------------------------------------------------------------------

def _tiny_token_case(seed=11, L=61, D=3, Hq=2):
    rng = np.random.default_rng(seed)
    q = np.round(rng.standard_normal((1, L, Hq, D)) * 8) / 8
    k = np.round(rng.standard_normal((1, L, 1, D)) * 8) / 8
    v = rng.standard_normal((1, L, 1, 2))
    return q, k, v


def _token_select_matches_brute(seed=11, before_select=None):
    """Tiny geometry (block 4, 1 global, 2 local, top 2 pages, top 3 tokens): every
    row re-decided by enumerating the candidate tokens with exact rational scores."""
    win, M, K = Window(4, 1, 2), 2, 3
    q, k, _ = _tiny_token_case(seed)
    L, D = q.shape[1], q.shape[3]
    pidx, pcnt, _ = oracle.page_select(q, k, win, top_m=M)
    if before_select:
        before_select()
    tok, tcnt, _ = oracle.token_select(q, k, pidx, pcnt, win, top_k=K)
    ok = True
    for h in range(2):
        for qb in range((L + 3) // 4):
            inside = set(range(max(0, qb - 1), qb + 1)) | {0}
            pages = [int(c) for c in pidx[0, h, qb, :pcnt[0, h, qb]] if c not in inside]
            cand = [j for c in pages for j in range(4 * c, min(4 * c + 4, L))]
            rows = range(4 * qb, min(4 * qb + 4, L))
            qsum = [sum(Fraction(float(q[0, i, h, d])) for i in rows) for d in range(D)]
            score = {j: sum(qsum[d] * Fraction(float(k[0, j, 0, d])) for d in range(D)) for j in cand}
            want = sorted(sorted(cand, key=lambda j: (-score[j], j))[:K])
            ok &= list(tok[0, h, qb, :tcnt[0, h, qb]]) == want
            ok &= bool((tok[0, h, qb, tcnt[0, h, qb]:] == -1).all())
    return ok


def test_token_select_bruteforce_exact_tiny():
    assert _token_select_matches_brute(11) and _token_select_matches_brute(21)


def test_token_select_planted_mistake_is_caught(monkeypatch):
    """Window pages wrongly counted as candidates (the global block dropped from
    the window the second stage excludes) must fail the brute-force pin."""
    import oracle.ssa as S
    good_wb = S.window_blocks
    assert _token_select_matches_brute(11)
    no_global = lambda qb, win=S.DEFAULT_WINDOW: good_wb(qb, Window(win.block_size, 0, win.n_local))
    assert not _token_select_matches_brute(11, lambda: monkeypatch.setattr(S, "window_blocks", no_global))


def test_token_select_keeping_every_candidate_is_page_attention():
    """With K at least the recalled pages' token count, window blocks + tokens is
    the same key set as the page list: the attention outputs agree to rounding."""
    rng = np.random.default_rng(12)
    L, Hq = 128 * 20 + 37, 2
    q = rng.standard_normal((1, L, Hq, 8))
    k = rng.standard_normal((1, L, 1, 8))
    v = rng.standard_normal((1, L, 1, 8))
    pidx, pcnt, _ = oracle.page_select(q, k, top_m=3)
    tok, tcnt, _ = oracle.token_select(q, k, pidx, pcnt, top_k=3 * 128)
    widx, wcnt = oracle.block_index((L + 127) // 128)
    nqb = widx.shape[0]
    widx4 = np.broadcast_to(widx[None, None], (1, Hq, nqb, 8))
    wcnt3 = np.broadcast_to(wcnt[None, None], (1, Hq, nqb))
    o1, l1 = oracle.token_list_attention(q, k, v, 0.3, widx4, wcnt3, tok, tcnt)
    o2, l2 = oracle.block_list_attention(q, k, v, 0.3, pidx, pcnt)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-13)
    # rows 16.. keep 3 pages = 384 tokens; shorter rows keep what they have
    assert tcnt[0, 0, 19] == 384 and tcnt[0, 0, 8] == 128 and tcnt[0, 0, 7] == 0


def test_token_select_planted_and_ties():
    """Keys sharing a direction with the query block are selected; an exact
    duplicate of the best key loses the tie to the lower token."""
    rng = np.random.default_rng(13)
    L, D = 128 * 30, 16
    q = rng.standard_normal((1, L, 1, D))
    k = rng.standard_normal((1, L, 1, D))
    u = rng.standard_normal(D) * 3
    qb = 29
    q[0, qb * 128:(qb + 1) * 128, 0] += u
    planted = [5 * 128 + 7, 5 * 128 + 90, 9 * 128 + 1]
    for j in planted:
        k[0, j, 0] += u
    qsum = q[0, qb * 128:(qb + 1) * 128, 0].sum(axis=0)
    weakest = min(planted, key=lambda j: k[0, j, 0] @ qsum)
    k[0, 9 * 128 + 100, 0] = k[0, weakest, 0]          # exact duplicate of the weakest planted key
    pidx = np.full((1, 1, 30, 10), -1, np.int32)
    pcnt = np.zeros((1, 1, 30), np.int32)
    row = sorted({0, 5, 9} | set(range(23, 30)))
    pidx[0, 0, qb, :len(row)] = row
    pcnt[0, 0, qb] = len(row)
    tok, tcnt, _ = oracle.token_select(q, k, pidx, pcnt, top_k=3)
    assert list(tok[0, 0, qb, :3]) == planted
    tok4, _, _ = oracle.token_select(q, k, pidx, pcnt, top_k=4)
    assert list(tok4[0, 0, qb, :4]) == sorted(planted + [9 * 128 + 100])


def test_token_list_attention_bruteforce_tiny():
    """Explicit per-query key sets (listed blocks causally, plus the tokens) with a
    pure-Python softmax."""
    win, M, K = Window(4, 1, 2), 2, 3
    q, k, v = _tiny_token_case(seed=14)
    L = q.shape[1]
    pidx, pcnt, _ = oracle.page_select(q, k, win, top_m=M)
    tok, tcnt, _ = oracle.token_select(q, k, pidx, pcnt, win, top_k=K)
    nqb = (L + 3) // 4
    widx = np.full((1, 2, nqb, 3), -1, np.int32)
    wcnt = np.zeros((1, 2, nqb), np.int32)
    for qb in range(nqb):
        w = oracle.window_blocks(qb, win)
        widx[0, :, qb, :len(w)] = w
        wcnt[0, :, qb] = len(w)
    o, lse = oracle.token_list_attention(q, k, v, 0.7, widx, wcnt, tok, tcnt, block=4)
    for h in range(2):
        for i in range(L):
            qb = i // 4
            keys = [j for t in oracle.window_blocks(qb, win) for j in range(4 * t, min(4 * t + 4, L)) if j <= i]
            keys += [int(j) for j in tok[0, h, qb, :tcnt[0, h, qb]]]
            s = [0.7 * sum(float(q[0, i, h, d]) * float(k[0, j, 0, d]) for d in range(3)) for j in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            ref = [sum(wi * float(v[0, j, 0, c]) for wi, j in zip(w, keys)) / sum(w) for c in range(2)]
            assert np.allclose(o[0, i, h], ref, rtol=1e-12, atol=1e-13)
            assert abs(lse[0, h, i] - (m + math.log(sum(w)))) < 1e-12


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# ---------------------------------------------------------------------------

def _ssa_vs_brute(win=Window(4, 1, 3)):
    L = 33
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, L, 2, 3))
    k = rng.standard_normal((1, L, 1, 3))
    v = rng.standard_normal((1, L, 1, 2))
    o, lse = oracle.ssa_attention(q, k, v, 0.7, win)
    ref = brute_rows(q, k, v, 0.7, range(L),
                     lambda i: brute_window_keys(i, win.block_size, win.n_global, win.n_local))
    return max(max(np.abs(o[b, i, h] - ob).max(), abs(lse[b, h, i] - lb)) for (b, h, i), (ob, lb) in ref.items())


def test_planted_mistakes_are_caught(monkeypatch):
    import oracle.ssa as S
    assert _ssa_vs_brute() < 1e-12
    good_wb = S.window_blocks
    good_attend = S._attend

    # one local block too many
    monkeypatch.setattr(S, "window_blocks", lambda qb, win=S.DEFAULT_WINDOW:
                        good_wb(qb, Window(win.block_size, win.n_global, win.n_local + 1)))
    assert _ssa_vs_brute() > 1e-3
    monkeypatch.setattr(S, "window_blocks", good_wb)

    # global block dropped
    monkeypatch.setattr(S, "window_blocks", lambda qb, win=S.DEFAULT_WINDOW:
                        good_wb(qb, Window(win.block_size, 0, win.n_local)))
    assert _ssa_vs_brute() > 1e-3
    monkeypatch.setattr(S, "window_blocks", good_wb)

    # sign of the scores flipped
    monkeypatch.setattr(S, "_attend", lambda qr, kr, vr, al, sc: good_attend(qr, kr, vr, al, -sc))
    assert _ssa_vs_brute() > 1e-3

    # keys used in place of values (wrong operand)
    monkeypatch.setattr(S, "_attend", lambda qr, kr, vr, al, sc: good_attend(qr, kr, kr[:, :vr.shape[1]], al, sc))
    assert _ssa_vs_brute() > 1e-3

    # scale applied twice
    monkeypatch.setattr(S, "_attend", lambda qr, kr, vr, al, sc: good_attend(qr, kr, vr, al, sc * sc))
    assert _ssa_vs_brute() > 1e-3

    # the max dropped from lse
    def no_max(qr, kr, vr, al, sc):
        o, lse = good_attend(qr, kr, vr, al, sc)
        s = np.where(al, sc * (qr @ kr.T), -np.inf)
        return o, lse - s.max(axis=1)
    monkeypatch.setattr(S, "_attend", no_max)
    assert _ssa_vs_brute() > 1e-3
    monkeypatch.setattr(S, "_attend", good_attend)
    assert _ssa_vs_brute() < 1e-12


# ---------------------------------------------------------------------------
# the shared generator rounds like torch
# ---------------------------------------------------------------------------

def test_generator_rounding_matches_torch():
    import synth
    x = np.random.default_rng(0).standard_normal(100000, dtype=np.float32) * 3
    bits = synth.f32_to_bf16_bits(x)
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, tb)
    back = synth.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_window_facts_from_the_pages():
    """The oracle's default window reproduces the page-stated geometry: blocks of
    128 tokens, 1 global + 7 local, at most S = 1024 keys per query."""
    import os
    facts = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "window_facts.txt")):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            facts[k] = int(v)
    w = oracle.DEFAULT_WINDOW
    assert (w.block_size, w.n_global, w.n_local) == (facts["block_size"], facts["n_global"], facts["n_local"])
    L = 4096
    q = np.zeros((1, L, 1, 2))
    k = RNG.standard_normal((1, L, 1, 2))
    v = np.ones((1, L, 1, 1))
    _, lse = oracle.ssa_attention(q, k, v, 1.0)
    nkeys = np.exp(lse[0, 0])
    assert abs(nkeys.max() - facts["window_tokens"]) < 1e-6
    assert abs(nkeys[facts["window_tokens"] - 1] - facts["window_tokens"]) < 1e-6
