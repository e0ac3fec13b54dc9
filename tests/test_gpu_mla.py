"""GPU parity at the latent-shared (MLA-like) shape: 576-wide keys shared by
all query heads, values = the first 512 channels.  Inputs are N(0,1)/24
(1/sqrt(576)), so outputs are ~1e-3 and the absolute 1e-2 bound is weak; each
check also requires max error / max |reference| <= 1e-2."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import bits_to_dev, check_close, say, to_f64
from tests.test_gpu_decode import build_case, run_and_check

pytestmark = pytest.mark.gpu

DQK, DV = 576, 512
MUL = 1.0 / 24.0
SCALE = 1.0 / 24.0


def mla_inputs(seed, B, L, Hq, shared=True):
    qb = synth.seq_tensor(seed, synth.Q, B, L, Hq, DQK, "bf16", MUL)
    cb = synth.seq_tensor(seed, synth.LATENT, B, L, 1, DQK, "bf16", MUL)
    q, c = bits_to_dev(qb), bits_to_dev(cb)
    qh, ch = synth.bf16_bits_to_f32(qb), synth.bf16_bits_to_f32(cb)
    if shared:
        return qh, ch, ch[..., :DV], q, c, c[..., :DV]
    vb = synth.seq_tensor(seed, synth.V, B, L, 1, DV, "bf16", MUL)
    return qh, ch, synth.bf16_bits_to_f32(vb), q, c, bits_to_dev(vb)


@pytest.mark.parametrize("L,Hq,shared,out", [(1300, 16, True, None), (129, 16, True, torch.float32),
                                             (1000, 32, False, None), (2304, 16, True, None)])
def test_mla_prefill_small(lib, L, Hq, shared, out):
    qh, kh, vh, q, k, v = mla_inputs(71, 1, L, Hq, shared)
    say(f"mla prefill L={L} Hq={Hq} shared={shared}")
    o, lse = lib.ssa(q, k, v, scale=SCALE, out_dtype=out, with_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.ssa_attention(qh.astype(np.float64), kh, vh, SCALE)
    check_close(to_f64(o), ro, f"mla L={L} o", rel=True)
    check_close(to_f64(lse), rl, f"mla L={L} lse")


@pytest.mark.parametrize("jump,dense", [(40.0, False), (60.0, False), (100.0, False), (60.0, True)])
def test_mla_prefill_reference_max_rerun(lib, jump, dense):
    """Scores jump by `jump` nats at block 3, far above the reference max the
    576-wide kernel takes from the first keys a row sees.  40: weights up to
    2^58, whose sums pass 2^64; 60: up to 2^87; 100: fp32 overflow on the
    first pass.  In each case the tile is rerun with the exact row maxima, and
    every row must match (the dense layer sees its own block first)."""
    B, L, H = 1, 1024, 2
    g = torch.Generator().manual_seed(int(jump) + 7)
    q = torch.ones((B, L, H, DQK)).bfloat16()
    c = (0.05 * torch.randn((B, L, 1, DQK), generator=g)).bfloat16()
    c[:, 3 * 128:4 * 128] = jump / (DQK * SCALE)  # q.k * scale = jump (up to bf16 rounding)
    c[:, 3 * 128:4 * 128, :, :DV] = torch.randn((128, DV), generator=g).bfloat16()[None, :, None]
    c[:, 3 * 128:4 * 128, :, DV:] = jump / ((DQK - DV) * SCALE)  # only the rope part carries the jump
    say(f"mla reference-max rerun jump={jump} dense={dense}")
    qd, cd = q.cuda(), c.cuda()
    if dense:
        o, lse = lib.dense_causal(qd, cd, cd[..., :DV], scale=SCALE, with_lse=True)
    else:
        o, lse = lib.ssa(qd, cd, cd[..., :DV], scale=SCALE, with_lse=True)
    torch.cuda.synchronize()
    f64 = lambda t: t.float().double().numpy()
    ref = oracle.dense_causal if dense else oracle.ssa_attention
    ro, rl = ref(f64(q), f64(c), f64(c[..., :DV]), SCALE)
    check_close(to_f64(o), ro, f"mla rerun jump={jump} o")
    check_close(to_f64(lse), rl, f"mla rerun jump={jump} lse")


def test_mla_dense_small(lib):
    qh, kh, vh, q, k, v = mla_inputs(72, 1, 700, 16)
    say("mla dense")
    o, _ = lib.dense_causal(q, k, v, scale=SCALE)
    torch.cuda.synchronize()
    ro, _ = oracle.dense_causal(qh.astype(np.float64), kh, vh, SCALE)
    check_close(to_f64(o), ro, "mla dense o", rel=True)


def test_mla_prefill_full_size_sampled(lib):
    """B=1, L=262144, 128 heads x 576/512 (the launch the benchmark times);
    query blocks 0-8, 2047 and 8 seeded random ones, all heads."""
    B, L, H = 1, 262144, 128
    say("mla full-size inputs")
    q = synth.torch_normal_bf16(404, (B, L, H, DQK), MUL)
    c = synth.torch_normal_bf16(405, (B, L, 1, DQK), MUL)
    say("mla full-size prefill")
    o, lse = lib.ssa(q, c, c[..., :DV], scale=SCALE, with_lse=True)
    torch.cuda.synchronize()
    ch = c[0].float().cpu().numpy()
    rng = np.random.default_rng(4)
    qbs = list(range(9)) + [2047] + sorted(rng.choice(np.arange(9, 2047), 8, replace=False).tolist())
    for qb in qbs:
        rows = slice(qb * 128, (qb + 1) * 128)
        qr = q[0, rows].float().cpu().numpy().astype(np.float64)
        ro, rl = oracle.ssa_rows(qr, qb * 128, ch, ch[..., :DV], SCALE, list(range(H)), H)
        check_close(to_f64(o[0, rows]), ro, f"mla full qb={qb}", rel=True)
        check_close(to_f64(lse[0, :, rows]).T, rl, f"mla full lse qb={qb}")
    del q, o, c


@pytest.mark.parametrize("lens,Hq", [([1, 5, 129, 1000, 3000], 32), ([1025, 70000], 16)])
def test_mla_decode_small(lib, lens, Hq):
    dev, host = build_case(81, len(lens), Hq, 1, DQK, lens, mul=MUL, Dv=DV, share_kv=True)
    run_and_check(lib, dev, host, SCALE, f"mla decode {lens}", rel=True, v_view=dev["k"][..., :DV])


def test_mla_decode_separate_v(lib):
    lens = [300, 2000]
    dev, host = build_case(82, len(lens), 16, 1, DQK, lens, mul=MUL, Dv=DV, share_kv=False)
    run_and_check(lib, dev, host, SCALE, "mla decode separate v", rel=True)


def test_mla_decode_full_size(lib):
    """Batch 8 at context 1,048,576 (last block full), 128 heads."""
    lens = [1048576] * 8
    dev, host = build_case(4, 8, 128, 1, DQK, lens, mul=MUL, Dv=DV, share_kv=True)
    run_and_check(lib, dev, host, SCALE, "mla decode 1M", rel=True, v_view=dev["k"][..., :DV])


def test_mla_decode_reused_workspace_and_invalid_rows(lib):
    """A workspace holding NaN bytes from elsewhere, reused by a second call on
    fewer sequences; rows with a bad length or page are NaN, the others match."""
    lens = [500, 1300, 900, 700, 2000]
    dev, host = build_case(83, len(lens), 16, 1, DQK, lens, mul=MUL, Dv=DV, share_kv=True)
    ws = torch.full((lib.decode_workspace_size(len(lens), 16, DQK, DV) + 256,), 0xFF, dtype=torch.uint8,
                    device="cuda")
    vv = dev["k"][..., :DV]
    ro, rl = oracle.decode(host["q"], host["k"], host["k"][..., :DV], host["bt"], host["sl"], SCALE)
    say("mla decode dirty workspace")
    o, lse = lib.decode(dev["q"], dev["k"], vv, dev["bt"], dev["sl"], scale=SCALE, with_lse=True, workspace=ws)
    torch.cuda.synchronize()
    check_close(to_f64(o), ro, "mla dirty workspace o", rel=True)
    check_close(to_f64(lse), rl, "mla dirty workspace lse")
    sl, bt = dev["sl"][:4].clone(), dev["bt"][:4].clone()
    sl[1] = 0
    bt[2, (900 - 1) // 128] = 10 ** 6  # own block of sequence 2 points outside the pool
    sl[3] = bt.shape[1] * 128 + 1
    say("mla decode invalid rows, reused workspace")
    o2, l2 = lib.decode(dev["q"][:4], dev["k"], vv, bt, sl, scale=SCALE, with_lse=True, workspace=ws)
    torch.cuda.synchronize()
    o2n = o2.float().cpu().numpy()
    assert np.isnan(o2n[1:]).all() and np.isnan(l2.cpu().numpy()[1:]).all()
    check_close(to_f64(o2[0:1]), ro[0:1], "mla valid row beside invalid ones", rel=True)
    check_close(to_f64(l2[0:1]), rl[0:1], "mla valid row lse")


@pytest.mark.parametrize("win", [(128, 2, 5), (128, 1, 11)])
def test_mla_decode_other_windows(lib, win):
    """The split kernel's grid and workspace follow the window width."""
    lens = [1, 300, 2500]
    w = oracle.Window(*win)
    dev, host = build_case(84, len(lens), 32, 1, DQK, lens, mul=MUL, Dv=DV, share_kv=True, head=win[1], tail=win[2])
    say(f"mla decode window={win}")
    vv = dev["k"][..., :DV]
    o, lse = lib.decode(dev["q"], dev["k"], vv, dev["bt"], dev["sl"], scale=SCALE, window=lib.Window(*win),
                        with_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(host["q"], host["k"], host["k"][..., :DV], host["bt"], host["sl"], SCALE, w)
    check_close(to_f64(o), ro, f"mla window {win} o", rel=True)
    check_close(to_f64(lse), rl, f"mla window {win} lse")
