"""GPU parity: the second stage of hierarchical indexing (token lists, bit-exact)
and attention over window blocks plus the listed tokens."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import bits_to_dev, check_close, gen, say, to_f64
from tests.selection_check import check_page_lists, check_token_lists

pytestmark = pytest.mark.gpu


def check_pages(pidx, pcnt, qh, kh, M, heads=None):
    """The GPU page lists against the oracle's first stage (bit-exact where
    certified, judged on near ties); returns them as numpy arrays."""
    gp, gc = pidx.cpu().numpy(), pcnt.cpu().numpy()
    ridx, rcnt, pnear = oracle.page_select(qh, kh, top_m=M, heads=heads)
    judged = check_page_lists(gp, gc, qh, kh, M, ridx, rcnt, pnear, heads=heads)
    say(f"page lists: {judged} near-tie rows judged")
    return gp, gc


def compare_tokens(tok, tcnt, qh, kh, gp, gc, K, heads=None):
    """The GPU token lists against the oracle's second stage run over the same
    (validated) page lists: bit-exact where certified, judged on near ties."""
    rtok, rtcnt, near = oracle.token_select(qh, kh, gp, gc, top_k=K, heads=heads)
    judged = check_token_lists(tok.cpu().numpy(), tcnt.cpu().numpy(), qh, kh, gp, gc, K, rtok, rtcnt, near,
                               heads=heads)
    say(f"token lists: {judged} near-tie rows judged")
    return int(near.sum())


def select_both(lib, q, k, qh, kh, M, K, heads=None):
    """GPU page + token selection, both checked against the oracle."""
    from long_context_block_ssa_amd import page_select_workspace_size
    ws = torch.empty((page_select_workspace_size(q, k) + 256,), dtype=torch.uint8, device=q.device)
    pidx, pcnt = lib.page_select(q, k, top_m=M, workspace=ws)
    tok, tcnt = lib.token_select(q, k, pidx, pcnt, ws, top_m=M, top_k=K)
    torch.cuda.synchronize()
    gp, gc = check_pages(pidx, pcnt, qh, kh, M, heads)
    compare_tokens(tok, tcnt, qh, kh, gp, gc, K, heads)
    return tok, tcnt


@pytest.mark.parametrize("L,Hq,Hkv,D,M,K", [
    (128 * 40 + 17, 2, 1, 128, 8, 512),
    (128 * 40 + 17, 2, 1, 128, 8, 100),
    (128 * 33, 2, 2, 64, 4, 300),
    (128 * 30, 1, 1, 128, 8, 1024),   # every candidate kept
    (128 * 30, 1, 1, 128, 8, 0),      # no tokens
    (128 * 36, 2, 2, 128, 32, 1000),  # up to 28 recalled pages, 3584 candidates
])
def test_token_select_small(lib, L, Hq, Hkv, D, M, K):
    qh, q = gen(61, synth.Q, 1, L, Hq, D)
    kh, k = gen(61, synth.K, 1, L, Hkv, D)
    say(f"token_select L={L} Hq={Hq} Hkv={Hkv} D={D} M={M} K={K}")
    select_both(lib, q, k, qh, kh, M, K)


def test_token_select_many_pages(lib):
    """More pages per head than the bucket kernel counts in LDS at once
    (4096): the buckets are built over several page segments."""
    L, D, M, K = 128 * 4100 + 5, 64, 4, 256
    qh, q = gen(63, synth.Q, 1, L, 1, D)
    kh, k = gen(63, synth.K, 1, L, 1, D)
    say(f"token_select L={L} (4101 query blocks) D={D} M={M} K={K}")
    select_both(lib, q, k, qh, kh, M, K)


def test_token_select_planted_and_ties(lib):
    """Keys planted along the query block's direction are the ones kept; an exact
    duplicate of the weakest planted key loses the tie to the lower token."""
    L, D = 128 * 30, 128
    qh = synth.bf16_bits_to_f32(synth.seq_tensor(62, synth.Q, 1, L, 1, D)).copy()
    kh = synth.bf16_bits_to_f32(synth.seq_tensor(62, synth.K, 1, L, 1, D)).copy()
    qb = 29
    u = np.zeros(D, np.float32)
    u[:32] = 1.0
    qh[0, qb * 128:(qb + 1) * 128, 0] += u
    # page 5 carries the whole page a little along u (so the page stage recalls
    # it); three of its keys much more
    kh[0, 5 * 128:6 * 128, 0] += 0.25 * u
    planted = [5 * 128 + 7, 5 * 128 + 90, 5 * 128 + 100]
    for j in planted:
        kh[0, j, 0] += 2 * u
    qbits, kbits = synth.f32_to_bf16_bits(qh), synth.f32_to_bf16_bits(kh)
    qh, kh = synth.bf16_bits_to_f32(qbits), synth.bf16_bits_to_f32(kbits)
    qsum = qh[0, qb * 128:(qb + 1) * 128, 0].astype(np.float64).sum(axis=0)
    weakest = min(planted, key=lambda j: kh[0, j, 0].astype(np.float64) @ qsum)
    dup = 5 * 128 + 120
    kbits[0, dup, 0] = kbits[0, weakest, 0]
    kh = synth.bf16_bits_to_f32(kbits)
    q, k = bits_to_dev(qbits), bits_to_dev(kbits)
    for K, want in [(3, planted), (4, sorted(planted + [dup]))]:
        say(f"token_select planted K={K}")
        tok, tcnt = select_both(lib, q, k, qh, kh, 8, K)
        assert tok[0, 0, qb, :K].cpu().tolist() == want


@pytest.mark.parametrize("L,Hq,Hkv,K,out", [
    (128 * 24 + 33, 2, 1, 300, torch.bfloat16),
    (128 * 24 + 33, 2, 1, 0, torch.bfloat16),
    (128 * 20, 2, 2, 1024, torch.float32),
    (128 * 19 + 5, 1, 1, 32, torch.bfloat16),
])
def test_hi_attention_small(lib, L, Hq, Hkv, K, out):
    D = 128
    qh, q = gen(63, synth.Q, 1, L, Hq, D)
    kh, k = gen(63, synth.K, 1, L, Hkv, D)
    vh, v = gen(63, synth.V, 1, L, Hkv, D)
    say(f"hi_attention L={L} Hq={Hq} Hkv={Hkv} K={K} out={out}")
    o, lse, tok, tcnt, pidx, pcnt = lib.hi_attention(q, k, v, top_m=8, top_k=K, out_dtype=out, with_lse=True,
                                                     with_pages=True)
    torch.cuda.synchronize()
    gp, gc = check_pages(pidx, pcnt, qh, kh, 8)
    compare_tokens(tok, tcnt, qh, kh, gp, gc, K)
    nqb = (L + 127) // 128
    widx, wcnt = oracle.block_index(nqb)
    w4 = np.broadcast_to(widx[None, None], (1, Hq, nqb, widx.shape[1]))
    c3 = np.broadcast_to(wcnt[None, None], (1, Hq, nqb))
    # attention over the GPU's own (validated) token lists
    ro, rl = oracle.token_list_attention(qh, kh, vh, 1 / math.sqrt(D), w4, c3, tok.cpu().numpy(), tcnt.cpu().numpy())
    check_close(to_f64(o), ro, "hi attention o")
    check_close(to_f64(lse), rl, "hi attention lse")


def test_hi_keep_all_matches_page_attention(lib):
    """K = M * 128 keeps every recalled token: the same key set as the page list."""
    L, H, D = 128 * 26, 2, 128
    _, q = gen(64, synth.Q, 1, L, H, D)
    _, k = gen(64, synth.K, 1, L, H, D)
    _, v = gen(64, synth.V, 1, L, H, D)
    say("hi keep-all vs page attention")
    o1, l1, _, _ = lib.hi_attention(q, k, v, top_m=8, top_k=1024, out_dtype=torch.float32, with_lse=True)
    o2, l2, _, _ = lib.page_attention(q, k, v, top_m=8, out_dtype=torch.float32, with_lse=True)
    torch.cuda.synchronize()
    check_close(to_f64(o1), to_f64(o2), "keep-all o")
    check_close(to_f64(l1), to_f64(l2), "keep-all lse")


def test_prefill_tokens_invalid_rows(lib):
    """Token rows that are not ascending, reach into the query block or repeat a
    listed block make exactly their query block's rows NaN."""
    L, H, D = 128 * 20, 1, 128
    qh, q = gen(65, synth.Q, 1, L, H, D)
    kh, k = gen(65, synth.K, 1, L, H, D)
    vh, v = gen(65, synth.V, 1, L, H, D)
    nqb = L // 128
    K = 64
    widx, wcnt = lib.block_index(nqb)
    rng = np.random.default_rng(66)
    tok = np.full((1, H, nqb, K), -1, np.int32)
    tcnt = np.zeros((1, H, nqb), np.int32)
    for qb in range(9, nqb):  # valid rows: ascending tokens of pages 1 .. qb-7
        cand = np.arange(128, (qb - 6) * 128)
        pick = np.sort(rng.choice(cand, size=40, replace=False))
        tok[0, 0, qb, :40] = pick
        tcnt[0, 0, qb] = 40
    broken = {12: "descending", 15: "inside the query block", 17: "in a listed block"}
    tok[0, 0, 12, [3, 4]] = tok[0, 0, 12, [4, 3]]
    tok[0, 0, 15, 39] = 15 * 128 + 3
    tok[0, 0, 17, 0] = 5
    say("prefill_tokens invalid rows")
    td, cd = torch.from_numpy(tok).cuda(), torch.from_numpy(tcnt).cuda()
    o, lse = lib.prefill_tokens(q, k, v, lib.lists_from_index(widx, wcnt), lib.token_lists(td, cd),
                                out_dtype=torch.float32, with_lse=True)
    torch.cuda.synchronize()
    o, lse = to_f64(o), to_f64(lse)
    for qb in broken:
        assert np.isnan(o[0, qb * 128:(qb + 1) * 128]).all() and np.isnan(lse[0, :, qb * 128:(qb + 1) * 128]).all()
    good = [qb for qb in range(nqb) if qb not in broken]
    rows = np.concatenate([np.arange(qb * 128, (qb + 1) * 128) for qb in good])
    wi, wc = oracle.block_index(nqb)
    w4 = np.broadcast_to(wi[None, None], (1, H, nqb, wi.shape[1]))
    c3 = np.broadcast_to(wc[None, None], (1, H, nqb))
    ro, rl = oracle.token_list_attention(qh, kh, vh, 1 / math.sqrt(D), w4, c3, tok, tcnt, rows=good)
    check_close(o[0, rows], ro[0, rows], "valid rows o")
    check_close(lse[0, :, rows], rl[0, :, rows], "valid rows lse")


def test_hi_cfg5_full(lib):
    """L = 131072, H = 16, d = 128, M = 8, K = 512: page and token lists of all
    16 heads checked (bit-exact where certified, judged on near ties);
    attention over the GPU's lists checked on sampled query blocks (and every
    near-tie block) of every head."""
    L, H, D, M, K = 131072, 16, 128, 8, 512
    say("cfg5 inputs")
    qh, q = gen(5, synth.Q, 1, L, H, D)
    kh, k = gen(5, synth.K, 1, L, H, D)
    vh, v = gen(5, synth.V, 1, L, H, D)
    q = q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    k = k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    v = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    say("cfg5 hierarchical attention full size")
    o, lse, tok, tcnt, pidx, pcnt = lib.hi_attention(q, k, v, top_m=M, top_k=K, with_lse=True, with_pages=True)
    torch.cuda.synchronize()
    gp, gc = check_pages(pidx, pcnt, qh, kh, M)
    rtok, rtcnt, near = oracle.token_select(qh, kh, gp, gc, top_k=K)
    gt, gtc = tok.cpu().numpy(), tcnt.cpu().numpy()
    judged = check_token_lists(gt, gtc, qh, kh, gp, gc, K, rtok, rtcnt, near)
    say(f"cfg5 token lists: {judged} near-tie rows judged")
    nqb = L // 128
    wi, wc = oracle.block_index(nqb)
    w4 = np.broadcast_to(wi[None, None], (1, H, nqb, wi.shape[1]))
    c3 = np.broadcast_to(wc[None, None], (1, H, nqb))
    sample = sorted({3, 15, 16, 17, 500, 1023} | set(int(x) for x in np.flatnonzero(near[0].any(0))))
    ro, rl = oracle.token_list_attention(qh, kh, vh, 1 / math.sqrt(D), w4, c3, gt, gtc, rows=sample)
    for qb in sample:
        rows = slice(qb * 128, (qb + 1) * 128)
        check_close(to_f64(o[0, rows]), ro[0, rows], f"cfg5 qb={qb}")
        check_close(to_f64(lse[0][:, rows]), rl[0][:, rows], f"cfg5 lse qb={qb}")


def test_cli_index_shared_by_a_layer_pair(lib):
    """Cross-layer index reuse: the owner layer's page and token lists, computed
    once from its q and k, drive the next layer's attention over that layer's
    own q, k and v."""
    L, H, D, M, K = 128 * 22 + 9, 2, 128, 8, 256
    qh1, q1 = gen(67, synth.Q, 1, L, H, D)
    kh1, k1 = gen(67, synth.K, 1, L, H, D)
    qh2, q2 = gen(68, synth.Q, 1, L, H, D)
    kh2, k2 = gen(68, synth.K, 1, L, H, D)
    vh2, v2 = gen(68, synth.V, 1, L, H, D)
    from long_context_block_ssa_amd import page_select_workspace_size
    say("CLI: lists of layer 1, attention of layer 2")
    ws = torch.empty((page_select_workspace_size(q1, k1) + 256,), dtype=torch.uint8, device=q1.device)
    pidx, pcnt = lib.page_select(q1, k1, top_m=M, workspace=ws)
    tok, tcnt = lib.token_select(q1, k1, pidx, pcnt, ws, top_m=M, top_k=K)
    nqb = (L + 127) // 128
    widx, wcnt = lib.block_index(nqb)
    o2, l2 = lib.prefill_tokens(q2, k2, v2, lib.lists_from_index(widx, wcnt), lib.token_lists(tok, tcnt),
                                with_lse=True)
    op, lp = lib.prefill(q2, k2, v2, lib.lists_per_head(pidx, pcnt), with_lse=True)
    torch.cuda.synchronize()
    gp, gc = check_pages(pidx, pcnt, qh1, kh1, M)
    compare_tokens(tok, tcnt, qh1, kh1, gp, gc, K)
    rtok, rtcnt = tok.cpu().numpy(), tcnt.cpu().numpy()
    ridx, rcnt = gp, gc
    wi, wc = oracle.block_index(nqb)
    w4 = np.broadcast_to(wi[None, None], (1, H, nqb, wi.shape[1]))
    c3 = np.broadcast_to(wc[None, None], (1, H, nqb))
    ro, rl = oracle.token_list_attention(qh2, kh2, vh2, 1 / math.sqrt(D), w4, c3, rtok, rtcnt)
    check_close(to_f64(o2), ro, "layer 2 over layer 1's tokens: o")
    check_close(to_f64(l2), rl, "layer 2 over layer 1's tokens: lse")
    rpo, rpl = oracle.block_list_attention(qh2, kh2, vh2, 1 / math.sqrt(D), ridx, rcnt)
    check_close(to_f64(op), rpo, "layer 2 over layer 1's pages: o")
    check_close(to_f64(lp), rpl, "layer 2 over layer 1's pages: lse")
