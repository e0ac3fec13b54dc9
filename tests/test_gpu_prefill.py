"""GPU parity: block index, SSA prefill and the dense causal layer against the
float64 oracle, through the C ABI (python binding -> libssa.so)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import check_close, gen, say, to_f64

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# block index: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("nqb", [1, 2, 7, 8, 9, 256, 2048, 8192])
@pytest.mark.parametrize("win", [(128, 1, 7), (128, 2, 3), (64, 0, 5), (128, 4, 1)])
def test_block_index_bit_exact(lib, nqb, win):
    say(f"block_index nqb={nqb} win={win}")
    w = lib.Window(*win)
    idx, cnt = lib.block_index(nqb, w)
    torch.cuda.synchronize()
    ridx, rcnt = oracle.block_index(nqb, oracle.Window(*win))
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(cnt.cpu().numpy(), rcnt)


def test_block_index_seq_bit_exact(lib):
    lens = np.array([1, 2, 127, 128, 129, 1023, 1024, 1025, 65536, 65537, 131072, 1048576, 0, -3], np.int32)
    rng = np.random.default_rng(0)
    lens = np.concatenate([lens, rng.integers(1, 2_000_000, 500).astype(np.int32)])
    say(f"block_index_seq B={len(lens)}")
    idx, cnt = lib.block_index_seq(torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    good = lens >= 1
    ridx, rcnt = oracle.block_index_seq(lens[good])
    assert np.array_equal(idx.cpu().numpy()[good], ridx)
    assert np.array_equal(cnt.cpu().numpy()[good], rcnt)
    assert (cnt.cpu().numpy()[~good] == 0).all() and (idx.cpu().numpy()[~good] == -1).all()


# ---------------------------------------------------------------------------
# SSA prefill, full comparison at sizes the oracle finishes in seconds
# ---------------------------------------------------------------------------

CASES = [
    # name, dtype, B, L, Hq, Hkv, D, layout, out
    ("cfg1-f32-2048", "f32", 1, 2048, 1, 1, 64, "blhd", torch.float32),
    ("bf16-d128-ragged", "bf16", 2, 1000, 2, 2, 128, "blhd", None),
    ("bf16-d128-gqa-bhld", "bf16", 1, 2300, 4, 2, 128, "bhld", None),
    ("bf16-d64-ragged", "bf16", 1, 1921, 2, 1, 64, "blhd", None),
    ("bf16-d128-outf32", "bf16", 1, 3072, 2, 2, 128, "bhld", torch.float32),
    ("f32-ragged-gqa", "f32", 2, 1409, 2, 1, 64, "bhld", torch.float32),
    ("bf16-d128-L1", "bf16", 1, 1, 1, 1, 128, "blhd", None),
    ("bf16-d128-L129", "bf16", 1, 129, 1, 1, 128, "blhd", None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ssa_prefill_parity(lib, case):
    name, dt, B, L, Hq, Hkv, D, layout, out = case
    seed = 11
    qh, q = gen(seed, synth.Q, B, L, Hq, D, dt)
    kh, k = gen(seed, synth.K, B, L, Hkv, D, dt)
    vh, v = gen(seed, synth.V, B, L, Hkv, D, dt)
    if layout == "bhld":
        q = q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        k = k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        v = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    scale = 1.0 / math.sqrt(D)
    say(f"ssa_prefill {name}")
    o, lse = lib.ssa(q, k, v, scale=scale, out_dtype=out, with_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.ssa_attention(qh.astype(np.float64), kh, vh, scale)
    check_close(to_f64(o), ro, f"{name} o")
    check_close(to_f64(lse), rl, f"{name} lse")


@pytest.mark.parametrize("win,D", [((128, 0, 5), 128), ((128, 2, 3), 128), ((128, 3, 13), 128),
                                   ((128, 2, 9), 64)])
def test_ssa_prefill_other_windows(lib, win, D):
    """Window geometries other than 1 global + 7 local blocks, through the
    same kernels (list widths 5 to 16)."""
    B, L, H = 1, 128 * 24 + 40, 2
    qh, q = gen(13, synth.Q, B, L, H, D)
    kh, k = gen(13, synth.K, B, L, H, D)
    vh, v = gen(13, synth.V, B, L, H, D)
    say(f"ssa_prefill window={win} D={D}")
    o, lse = lib.ssa(q, k, v, window=lib.Window(*win), with_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.ssa_attention(qh.astype(np.float64), kh, vh, 1 / math.sqrt(D), oracle.Window(*win))
    check_close(to_f64(o), ro, f"window {win} o")
    check_close(to_f64(lse), rl, f"window {win} lse")


@pytest.mark.parametrize("mode", ["dense", "window-2-14"])
def test_f32_prefill_long_lists(lib, mode):
    """fp32 at d = 64 with lists longer than the four waves of a workgroup
    (each wave takes several key blocks before the merge): the dense layer,
    and a 16-block window."""
    B, L, H, D = 1, 128 * 20 + 77, 2, 64
    qh, q = gen(17, synth.Q, B, L, H, D, "f32")
    kh, k = gen(17, synth.K, B, L, H, D, "f32")
    vh, v = gen(17, synth.V, B, L, H, D, "f32")
    say(f"f32 prefill {mode}")
    if mode == "dense":
        o, lse = lib.dense_causal(q, k, v, with_lse=True)
        ro, rl = oracle.dense_causal(qh.astype(np.float64), kh, vh, 1 / math.sqrt(D))
    else:
        o, lse = lib.ssa(q, k, v, window=lib.Window(128, 2, 14), with_lse=True)
        ro, rl = oracle.ssa_attention(qh.astype(np.float64), kh, vh, 1 / math.sqrt(D), oracle.Window(128, 2, 14))
    torch.cuda.synchronize()
    check_close(to_f64(o), ro, f"f32 {mode} o")
    check_close(to_f64(lse), rl, f"f32 {mode} lse")


def test_dense_causal_parity_small(lib):
    B, L, Hq, Hkv, D = 1, 1500, 2, 1, 128
    qh, q = gen(5, synth.Q, B, L, Hq, D)
    kh, k = gen(5, synth.K, B, L, Hkv, D)
    vh, v = gen(5, synth.V, B, L, Hkv, D)
    say("dense_causal small")
    o, lse = lib.dense_causal(q, k, v, with_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_causal(qh.astype(np.float64), kh, vh, 1 / math.sqrt(D))
    check_close(to_f64(o), ro, "dense o")
    check_close(to_f64(lse), rl, "dense lse")


def test_ssa_equals_dense_below_window(lib):
    """L <= 1024: every key is inside the window, so SSA and the dense layer
    compute the same attention."""
    B, L, H, D = 1, 1024, 2, 128
    _, q = gen(9, synth.Q, B, L, H, D)
    _, k = gen(9, synth.K, B, L, H, D)
    _, v = gen(9, synth.V, B, L, H, D)
    say("ssa == dense at L=1024")
    o1, _ = lib.ssa(q, k, v)
    o2, _ = lib.dense_causal(q, k, v)
    torch.cuda.synchronize()
    # same keys, visited in a different order (and rescaled at different
    # moments): equal up to the bf16 rounding of the outputs
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2


def test_structural_onehot_prefill(lib):
    """q = 0 weighs every readable key equally; with V = one-hot(block id) the
    output is (#keys of that block) / (#keys), which pins window membership."""
    B, L, H, D = 1, 128 * 20 + 57, 2, 128
    q = torch.zeros((B, L, H, D), dtype=torch.bfloat16, device="cuda")
    _, k = gen(3, synth.K, B, L, H, D)
    v = torch.zeros((B, L, H, D), dtype=torch.bfloat16, device="cuda")
    blk = torch.arange(L, device="cuda") // 128
    v[0, torch.arange(L, device="cuda"), :, blk % D] = 1.0
    say("structural one-hot prefill")
    o, lse = lib.ssa(q, k, v, out_dtype=torch.float32, with_lse=True)
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    lse = lse.cpu().numpy()
    nb = (L + 127) // 128
    for i in range(L):
        qb = i // 128
        n = i + 1 if i < 1024 else 897 + (i % 128)
        assert abs(lse[0, 0, i] - math.log(n)) < 1e-5
        want = np.zeros(D)
        for t in range(nb):
            if t == qb:
                c = i % 128 + 1
            elif t == 0 or qb - 6 <= t < qb:
                c = 128
            else:
                c = 0
            want[t % D] += c / n
        assert np.abs(o[0, i, 0] - want).max() < 1e-5, i


def test_prefill_nan_outside_window(lib):
    """Keys of blocks outside a query block's window are NaN: the rows of that
    query block must stay finite and match the oracle."""
    B, L, H, D = 1, 128 * 16, 1, 128
    qh, q = gen(4, synth.Q, B, L, H, D)
    kh, k = gen(4, synth.K, B, L, H, D)
    vh, v = gen(4, synth.V, B, L, H, D)
    qb = 15  # window {0, 9..15}: poison blocks 1..8
    k[:, 128:9 * 128] = float("nan")
    v[:, 128:9 * 128] = float("nan")
    say("prefill nan poison")
    o, _ = lib.ssa(q, k, v)
    torch.cuda.synchronize()
    rows = slice(qb * 128, L)
    ro, _ = oracle.ssa_rows(qh[0, rows].astype(np.float64), qb * 128, kh[0], vh[0], 1 / math.sqrt(D), [0], 1)
    check_close(to_f64(o[0, rows]), ro, "nan-poison rows")


@pytest.mark.parametrize("jump", [40.0, 60.0, 100.0])
def test_prefill_reference_max_rerun(lib, jump):
    """Scores jump by `jump` nats at block 3, far above the reference max the
    kernel takes from the first keys it sees (block 0).  40: weights up to
    2^58 -- their sums pass 2^64, so the tile is rerun once tracking the max,
    and kept; 60: weights up to 2^87, rerun again with the true max; 100:
    weights overflow fp32 on the first pass.  Every row must still match."""
    B, L, H, D = 1, 1024, 2, 128
    scale = 1.0 / math.sqrt(D)
    g = torch.Generator().manual_seed(int(jump))
    q = torch.ones((B, L, H, D)).bfloat16()
    k = (0.05 * torch.randn((B, L, H, D), generator=g)).bfloat16()
    k[:, 3 * 128:4 * 128] = jump / (D * scale)  # q.k * scale = jump (up to bf16 rounding)
    v = torch.randn((B, L, H, D), generator=g).bfloat16()
    say(f"prefill reference-max rerun jump={jump}")
    o, lse = lib.ssa(q.cuda(), k.cuda(), v.cuda(), scale=scale, with_lse=True)
    torch.cuda.synchronize()
    f64 = lambda t: t.float().double().numpy()
    ro, rl = oracle.ssa_attention(f64(q), f64(k), f64(v), scale)
    check_close(to_f64(o), ro, f"rerun jump={jump} o")
    check_close(to_f64(lse), rl, f"rerun jump={jump} lse")


def test_prefill_deterministic(lib):
    B, L, H, D = 1, 4096, 4, 128
    _, q = gen(8, synth.Q, B, L, H, D)
    _, k = gen(8, synth.K, B, L, H, D)
    _, v = gen(8, synth.V, B, L, H, D)
    say("determinism")
    o1, l1 = lib.ssa(q, k, v, with_lse=True)
    o2, l2 = lib.ssa(q, k, v, with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------------------
# full size of the prefill workload (B=1, H=16, d=128, L=32768) on sampled rows
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def cfg2(lib):
    B, L, H, D = 1, 32768, 16, 128
    say("cfg2 inputs")
    qh, q = gen(2, synth.Q, B, L, H, D)
    kh, k = gen(2, synth.K, B, L, H, D)
    vh, v = gen(2, synth.V, B, L, H, D)
    # the benchmark's layout: [B, H, L, D] contiguous
    q = q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    k = k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    v = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    return qh, kh, vh, q, k, v


SAMPLE_QB = [0, 1, 6, 7, 8, 100, 201, 255]


def test_cfg2_ssa_sampled(lib, cfg2):
    qh, kh, vh, q, k, v = cfg2
    say("cfg2 ssa prefill full size")
    o, lse = lib.ssa(q, k, v, with_lse=True)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(128)
    for qb in SAMPLE_QB:
        rows = slice(qb * 128, (qb + 1) * 128)
        ro, rl = oracle.ssa_rows(qh[0, rows].astype(np.float64), qb * 128, kh[0], vh[0], scale, list(range(16)), 16)
        check_close(to_f64(o[0, rows]), ro, f"cfg2 ssa qb={qb}")
        check_close(to_f64(lse[0, :, rows]).T, rl, f"cfg2 ssa lse qb={qb}")


def test_cfg2_dense_sampled(lib, cfg2):
    qh, kh, vh, q, k, v = cfg2
    say("cfg2 dense full size")
    o, lse = lib.dense_causal(q, k, v, with_lse=True)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(128)
    for qb in [0, 9, 255]:
        rows = slice(qb * 128, (qb + 1) * 128)
        heads = [0, 7, 15]
        ro, rl = oracle.dense_causal_rows(qh[0, rows][:, heads].astype(np.float64), qb * 128, kh[0], vh[0], scale,
                                          heads, 16)
        check_close(to_f64(o[0, rows][:, heads]), ro, f"cfg2 dense qb={qb}")
        check_close(to_f64(lse[0, heads][:, rows]).T, rl, f"cfg2 dense lse qb={qb}")
