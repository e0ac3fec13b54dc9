"""Structural GPU checks that need no oracle: with q = 0 every admitted key gets
the same weight, so with values one-hot in the key's block id the output is
(#admitted keys of that block) / (#admitted keys) and lse = ln(#admitted keys).
This pins window membership (and, for page selection, the tie rule: q = 0
gives every candidate page the score 0, so the lowest pages win) from counts
alone."""
import math

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import gen, say

pytestmark = pytest.mark.gpu


def window_counts(i, blocks):
    """Admitted keys of query i per listed block (causal in the own block)."""
    qb = i // 128
    out = {}
    for t in blocks:
        if t < qb:
            out[t] = 128
        elif t == qb:
            out[t] = i % 128 + 1
    return out


def expected_row(i, blocks, width):
    cnt = window_counts(i, blocks)
    n = sum(cnt.values())
    want = np.zeros(width)
    for t, c in cnt.items():
        want[t % width] += c / n
    return want, n


def ssa_blocks(qb):
    return sorted({0} | set(range(max(0, qb - 6), qb + 1)))


def onehot_rows(L, width, device="cuda"):
    """[L, width] bf16 rows, row j one-hot at (j // 128) mod width."""
    v = torch.zeros((L, width), dtype=torch.bfloat16, device=device)
    v[torch.arange(L, device=device), (torch.arange(L, device=device) // 128) % width] = 1.0
    return v


def test_structural_onehot_latent_prefill(lib):
    """576-wide latent shared by 16 heads, values = its first 512 channels."""
    B, L, H, DQK, DV = 1, 128 * 20 + 57, 16, 576, 512
    q = torch.zeros((B, L, H, DQK), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((B, L, 1, DQK), dtype=torch.bfloat16, device="cuda")
    c[0, :, 0, :DV] = onehot_rows(L, DV)
    c[0, :, 0, DV:] = torch.from_numpy(
        synth.bf16_bits_to_f32(synth.seq_tensor(81, synth.LATENT, 1, L, 1, DQK - DV, "bf16", 1 / 24))[0, :, 0]).cuda()
    say("structural one-hot prefill, 576/512 latent")
    o, lse = lib.ssa(q, c, c[..., :DV], scale=1 / 24, out_dtype=torch.float32, with_lse=True)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    for i in range(L):
        want, n = expected_row(i, ssa_blocks(i // 128), DV)
        assert np.abs(lse[0, :, i] - math.log(n)).max() < 1e-5, i
        assert np.abs(o[0, i] - want[None]).max() < 1e-5, i


def test_structural_onehot_latent_decode(lib):
    """576/512 decode: window pages hold one-hot latents, every other page and
    every slot at or past the sequence end holds NaN."""
    H, DQK, DV = 128, 576, 512
    lens = np.asarray([1, 129, 1500, 4000, 70001, 131072], np.int32)
    bt, P = synth.decode_block_table(82, lens, 128)
    pool = torch.full((P, 1, 128, DQK), float("nan"), dtype=torch.bfloat16, device="cuda")
    for b, n in enumerate(lens):
        qb = (int(n) - 1) // 128
        for t in ssa_blocks(qb):
            page = torch.zeros((128, DQK), dtype=torch.bfloat16)
            page[:, t % DV] = 1.0
            page[:, DV:] = 0.5
            valid = min(128, int(n) - t * 128)
            page[valid:] = float("nan")
            pool[int(bt[b, t]), 0] = page.cuda()
    q = torch.zeros((len(lens), H, DQK), dtype=torch.bfloat16, device="cuda")
    say("structural one-hot decode, 576/512 latent")
    o, lse = lib.decode(q, pool, pool[..., :DV], torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(),
                        scale=1 / 24, with_lse=True)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    for b, n in enumerate(lens):
        i = int(n) - 1
        want, nk = expected_row(i, ssa_blocks(i // 128), DV)
        assert np.abs(lse[b] - math.log(nk)).max() < 1e-5, b
        # bf16 output: one-hot shares are k/nk, rounded to 8 significant bits
        assert np.abs(o[b] - want[None]).max() <= 2.0 ** -8 * want.max() + 1e-7, b


def test_structural_onehot_page_attention(lib):
    """Page selection with q = 0: every candidate scores 0, ties go to the lower
    page, so query block qb >= 16 keeps pages 1..8 beside its window; attention
    over those lists then weighs every admitted key equally."""
    B, L, Hq, Hkv, D, M = 1, 128 * 40 + 33, 2, 1, 128, 8
    q = torch.zeros((B, L, Hq, D), dtype=torch.bfloat16, device="cuda")
    _, k = gen(83, synth.K, B, L, Hkv, D)
    v = onehot_rows(L, D).reshape(B, L, Hkv, D).contiguous()
    say("structural one-hot page attention")
    o, lse, idx, cnt = lib.page_attention(q, k, v, top_m=M, out_dtype=torch.float32, with_lse=True)
    torch.cuda.synchronize()
    o, lse, idx, cnt = o.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    nqb = (L + 127) // 128
    for qb in range(nqb):
        cands = list(range(1, qb - 6))
        blocks = sorted(set(ssa_blocks(qb)) | set(cands[:M]))
        for h in range(Hq):
            assert list(idx[0, h, qb, :cnt[0, h, qb]]) == blocks, (qb, h)
            assert (idx[0, h, qb, cnt[0, h, qb]:] == -1).all()
        for i in range(qb * 128, min((qb + 1) * 128, L)):
            want, n = expected_row(i, blocks, D)
            assert np.abs(lse[0, :, i] - math.log(n)).max() < 1e-5, i
            assert np.abs(o[0, i] - want[None]).max() < 1e-5, i
