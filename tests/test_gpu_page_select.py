"""GPU parity: page selection (bit-exact lists) and attention over the lists."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import check_close, gen, say, to_f64
from tests.selection_check import check_page_lists

pytestmark = pytest.mark.gpu


def compare_lists(idx, cnt, qh, kh, top_m, ridx, rcnt, near, heads=None):
    """Bit-exact on every row the oracle certified; a near-tie row (float scores
    within rounding of the top-M boundary) is judged against its exact rational
    scores.  Returns the GPU lists as numpy arrays."""
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    judged = check_page_lists(gi, gc, qh, kh, top_m, ridx, rcnt, near, heads=heads)
    say(f"page lists: {judged} near-tie rows judged")
    return gi, gc


@pytest.mark.parametrize("L,Hq,Hkv,D,M", [(128 * 40 + 17, 2, 1, 128, 8), (128 * 33, 2, 2, 64, 4),
                                          (128 * 20, 1, 1, 128, 0), (2048, 2, 2, 128, 8),
                                          # several 128-page chunks; M = 1 and M = 8 take the DPP
                                          # bar of a row's first chunk, M = 9, 16, 32 the bitonic one
                                          (128 * 300 + 5, 2, 1, 128, 1), (128 * 300 + 5, 2, 1, 128, 9),
                                          (128 * 300, 2, 2, 128, 16), (128 * 300, 1, 1, 64, 32)])
def test_page_select_small(lib, L, Hq, Hkv, D, M):
    qh, q = gen(51, synth.Q, 1, L, Hq, D)
    kh, k = gen(51, synth.K, 1, L, Hkv, D)
    say(f"page_select L={L} Hq={Hq} Hkv={Hkv} D={D} M={M}")
    idx, cnt = lib.page_select(q, k, top_m=M)
    torch.cuda.synchronize()
    ridx, rcnt, near = oracle.page_select(qh, kh, top_m=M)
    compare_lists(idx, cnt, qh, kh, M, ridx, rcnt, near)


@pytest.mark.parametrize("L,Hq,Hkv,D,M", [(128 * 40 + 17, 2, 1, 128, 8), (128 * 33, 2, 2, 64, 4)])
def test_page_select_phases_equal_one_call(lib, L, Hq, Hkv, D, M):
    """ssa_page_block_sums then ssa_page_select_top on one workspace give the
    lists of one ssa_page_select call bit for bit (the same kernels)."""
    qh, q = gen(53, synth.Q, 1, L, Hq, D)
    kh, k = gen(53, synth.K, 1, L, Hkv, D)
    say(f"page phases L={L} Hq={Hq} Hkv={Hkv} D={D} M={M}")
    idx, cnt = lib.page_select(q, k, top_m=M)
    ws = torch.full((lib.page_select_workspace_size(q, k) + 256,), 0xFF, dtype=torch.uint8, device="cuda")
    lib.page_block_sums(q, k, ws)
    idx2, cnt2 = lib.page_select_top(q, k, ws, top_m=M)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2)
    ridx, rcnt, near = oracle.page_select(qh, kh, top_m=M)
    compare_lists(idx2, cnt2, qh, kh, M, ridx, rcnt, near)


def test_page_select_planted_and_tie(lib):
    """A planted page is selected; an exact duplicate loses the tie to the
    lower page; both are taken when M = 2."""
    L, D = 128 * 40, 128
    qh = synth.bf16_bits_to_f32(synth.seq_tensor(7, synth.Q, 1, L, 1, D)).copy()
    kh = synth.bf16_bits_to_f32(synth.seq_tensor(7, synth.K, 1, L, 1, D)).copy()
    qb = 39
    qh[0, qb * 128:(qb + 1) * 128, 0] += 1.0
    kh[0, 5 * 128:6 * 128, 0] += 1.0
    kh[0, 20 * 128:21 * 128, 0] = kh[0, 5 * 128:6 * 128, 0]
    qbits = synth.f32_to_bf16_bits(qh)
    kbits = synth.f32_to_bf16_bits(kh)
    qh, kh = synth.bf16_bits_to_f32(qbits), synth.bf16_bits_to_f32(kbits)
    from tests.gpu_util import bits_to_dev
    q, k = bits_to_dev(qbits), bits_to_dev(kbits)
    for M, want in [(1, {5}), (2, {5, 20})]:
        say(f"page_select planted M={M}")
        idx, cnt = lib.page_select(q, k, top_m=M)
        torch.cuda.synchronize()
        row = set(idx[0, 0, qb, :cnt[0, 0, qb]].cpu().tolist())
        assert want <= row and (M == 2 or 20 not in row)
        ridx, rcnt, near = oracle.page_select(qh, kh, top_m=M)
        compare_lists(idx, cnt, qh, kh, M, ridx, rcnt, near)


def test_page_attention_small(lib):
    L, Hq, Hkv, D = 128 * 24 + 33, 2, 1, 128
    qh, q = gen(52, synth.Q, 1, L, Hq, D)
    kh, k = gen(52, synth.K, 1, L, Hkv, D)
    vh, v = gen(52, synth.V, 1, L, Hkv, D)
    say("page attention small")
    o, lse, idx, cnt = lib.page_attention(q, k, v, top_m=8, with_lse=True)
    torch.cuda.synchronize()
    ridx, rcnt, near = oracle.page_select(qh, kh, top_m=8)
    gi, gc = compare_lists(idx, cnt, qh, kh, 8, ridx, rcnt, near)
    # the attention over the GPU's own (validated) lists
    ro, rl = oracle.block_list_attention(qh, kh, vh, 1 / math.sqrt(D), gi, gc)
    check_close(to_f64(o), ro, "page attention o")
    check_close(to_f64(lse), rl, "page attention lse")


def test_page_select_cfg5_full(lib):
    """L = 131072, H = 16, d = 128, M = 8: the lists of all 16 heads checked
    (bit-exact where certified, judged on near ties); attention over the GPU's
    lists checked on sampled query blocks of every head."""
    L, H, D = 131072, 16, 128
    say("cfg5 inputs")
    qh, q = gen(5, synth.Q, 1, L, H, D)
    kh, k = gen(5, synth.K, 1, L, H, D)
    vh, v = gen(5, synth.V, 1, L, H, D)
    q = q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    k = k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    v = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    say("cfg5 page attention full size")
    o, lse, idx, cnt = lib.page_attention(q, k, v, top_m=8, with_lse=True)
    torch.cuda.synchronize()
    ridx, rcnt, near = oracle.page_select(qh, kh, top_m=8)
    say(f"cfg5 near rows: {int(near.sum())}")
    gi, gc = compare_lists(idx, cnt, qh, kh, 8, ridx, rcnt, near)
    heads = list(range(H))
    sample = sorted({3, 15, 16, 17, 500, 1023} | set(int(x) for x in np.flatnonzero(near[0].any(0))))
    for qb in sample:
        rows = slice(qb * 128, (qb + 1) * 128)
        lists = [gi[0, h, qb, :gc[0, h, qb]] for h in heads]
        ro, rl = oracle.block_list_rows(qh[0, rows], qb * 128, kh[0], vh[0], 1 / math.sqrt(D), heads, H, lists)
        check_close(to_f64(o[0, rows]), ro, f"cfg5 qb={qb}")
        check_close(to_f64(lse[0][:, rows]).T, rl, f"cfg5 lse qb={qb}")
