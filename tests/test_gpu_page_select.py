"""GPU parity: page selection (bit-exact lists) and attention over the lists."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import check_close, gen, say, to_f64

pytestmark = pytest.mark.gpu


def compare_lists(idx, cnt, ridx, rcnt, near, heads=None, q=None, k=None):
    """Bit-exact on every row the oracle certified; on near-tie rows (float
    scores within rounding of the top-M boundary) accept any list whose
    fixed part matches and whose count matches."""
    idx = idx.cpu().numpy()
    cnt = cnt.cpu().numpy()
    hs = range(idx.shape[1]) if heads is None else heads
    mism = 0
    for h in hs:
        ok = ~near[:, h]
        if not np.array_equal(cnt[:, h][ok], rcnt[:, h][ok]) or not np.array_equal(idx[:, h][ok], ridx[:, h][ok]):
            bad = np.argwhere((idx[:, h] != ridx[:, h]).any(-1) & ok)
            mism += len(bad)
            say(f"head {h}: mismatching rows {bad[:5].ravel().tolist()}")
        assert np.array_equal(cnt[:, h], rcnt[:, h])
    assert mism == 0
    return int(near.sum())


@pytest.mark.parametrize("L,Hq,Hkv,D,M", [(128 * 40 + 17, 2, 1, 128, 8), (128 * 33, 2, 2, 64, 4),
                                          (128 * 20, 1, 1, 128, 0), (2048, 2, 2, 128, 8)])
def test_page_select_small(lib, L, Hq, Hkv, D, M):
    qh, q = gen(51, synth.Q, 1, L, Hq, D)
    kh, k = gen(51, synth.K, 1, L, Hkv, D)
    say(f"page_select L={L} Hq={Hq} Hkv={Hkv} D={D} M={M}")
    idx, cnt = lib.page_select(q, k, top_m=M)
    torch.cuda.synchronize()
    ridx, rcnt, near = oracle.page_select(qh, kh, top_m=M)
    compare_lists(idx, cnt, ridx, rcnt, near)


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
        compare_lists(idx, cnt, ridx, rcnt, near)


def test_page_attention_small(lib):
    L, Hq, Hkv, D = 128 * 24 + 33, 2, 1, 128
    qh, q = gen(52, synth.Q, 1, L, Hq, D)
    kh, k = gen(52, synth.K, 1, L, Hkv, D)
    vh, v = gen(52, synth.V, 1, L, Hkv, D)
    say("page attention small")
    o, lse, idx, cnt = lib.page_attention(q, k, v, top_m=8, with_lse=True)
    torch.cuda.synchronize()
    ridx, rcnt, near = oracle.page_select(qh, kh, top_m=8)
    compare_lists(idx, cnt, ridx, rcnt, near)
    ro, rl = oracle.block_list_attention(qh, kh, vh, 1 / math.sqrt(D), ridx, rcnt)
    check_close(to_f64(o), ro, "page attention o")
    check_close(to_f64(lse), rl, "page attention lse")


def test_page_select_cfg5_full(lib):
    """L = 131072, H = 16, d = 128, M = 8: lists of heads 0, 7, 15 bit-exact;
    attention over the lists checked on sampled query blocks."""
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
    heads = [0, 7, 15]
    ridx, rcnt, near = oracle.page_select(qh, kh, top_m=8, heads=heads)
    compare_lists(idx, cnt, ridx, rcnt, near, heads=heads)
    for qb in [3, 15, 16, 17, 500, 1023]:
        rows = slice(qb * 128, (qb + 1) * 128)
        lists = [ridx[0, h, qb, :rcnt[0, h, qb]] for h in heads]
        ro, rl = oracle.block_list_rows(qh[0, rows][:, heads], qb * 128, kh[0], vh[0], 1 / math.sqrt(D), heads, H,
                                        lists)
        check_close(to_f64(o[0, rows][:, heads]), ro, f"cfg5 qb={qb}")
        check_close(to_f64(lse[0, heads][:, rows]).T, rl, f"cfg5 lse qb={qb}")
