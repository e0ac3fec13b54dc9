"""GPU parity: SSA decode over a paged cache against the float64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import bits_to_dev, check_close, say, to_f64

pytestmark = pytest.mark.gpu


def build_case(seed, B, Hq, Hkv, D, seq_lens, head=1, tail=7, mul=1.0, Dv=None, share_kv=False):
    """Paged cache with finite values only in the first `head` and last `tail`
    logical blocks of every sequence, and only in slots < n; NaN elsewhere.

    Returns device tensors and a compact host copy (only the filled pages) for
    the oracle.
    """
    Dv = D if Dv is None else Dv
    seq_lens = np.asarray(seq_lens, np.int32)
    bt, P = synth.decode_block_table(seed, seq_lens, 128)
    fill = synth.decode_fill_blocks(seq_lens, 128, head, tail)
    kp = torch.full((P, Hkv, 128, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    vp = kp if share_kv else torch.full((P, Hkv, 128, Dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids, kh, vh = [], [], []
    for b, blocks in enumerate(fill):
        n = int(seq_lens[b])
        for t in blocks:
            kb = synth.page_chunk(seed, synth.K, b, t, Hkv, D, "bf16", mul)
            vb = kb[..., :Dv] if share_kv else synth.page_chunk(seed, synth.V, b, t, Hkv, Dv, "bf16", mul)
            valid = min(128, n - t * 128)
            kb = kb.copy()
            vb = vb.copy()
            kb[:, valid:] = 0x7FC0  # bf16 NaN past the sequence end
            vb[:, valid:] = 0x7FC0
            ids.append(int(bt[b, t]))
            kh.append(kb)
            vh.append(vb)
    idx = torch.tensor(ids, dtype=torch.long, device="cuda")
    kp[idx] = bits_to_dev(np.stack(kh)[:, None]).reshape(len(ids), Hkv, 128, D)
    if not share_kv:
        vp[idx] = bits_to_dev(np.stack(vh)[:, None]).reshape(len(ids), Hkv, 128, Dv)
    # compact host pool for the oracle: remap physical ids to 0..len(ids)-1
    remap = {p: i for i, p in enumerate(ids)}
    bt_c = np.full_like(bt, -1)
    for b in range(len(seq_lens)):
        for t in range(bt.shape[1]):
            if bt[b, t] in remap:
                bt_c[b, t] = remap[bt[b, t]]
    k_host = synth.bf16_bits_to_f32(np.stack(kh))
    v_host = synth.bf16_bits_to_f32(np.stack(vh))
    q_bits = synth.decode_query(seed, len(seq_lens), Hq, D, "bf16", mul)
    q = bits_to_dev(q_bits[None]).reshape(len(seq_lens), Hq, D)
    dev = dict(q=q, k=kp, v=vp, bt=torch.from_numpy(bt).cuda(), sl=torch.from_numpy(seq_lens).cuda())
    host = dict(q=synth.bf16_bits_to_f32(q_bits), k=k_host, v=v_host, bt=bt_c, sl=seq_lens)
    return dev, host


def run_and_check(lib, dev, host, scale, name, rel=False, v_view=None):
    say(f"ssa_decode {name}")
    v = dev["v"] if v_view is None else v_view
    o, lse = lib.decode(dev["q"], dev["k"], v, dev["bt"], dev["sl"], scale=scale, with_lse=True)
    torch.cuda.synchronize()
    vh = host["v"] if v_view is None else host["k"][..., :v.shape[3]]
    ro, rl = oracle.decode(host["q"], host["k"], vh, host["bt"], host["sl"], scale)
    check_close(to_f64(o), ro, f"{name} o", rel=rel)
    check_close(to_f64(lse), rl, f"{name} lse")
    return o


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 4, 2), (128, 2, 2), (64, 3, 1), (128, 16, 1), (128, 8, 1), (128, 6, 2),
                                     (128, 15, 3), (128, 16, 2)])
def test_decode_small_nan_poisoned(lib, D, Hq, Hkv):
    lens = [1, 2, 127, 128, 129, 1000, 1024, 1025, 5000, 7777]
    dev, host = build_case(21, len(lens), Hq, Hkv, D, lens)
    run_and_check(lib, dev, host, 1 / math.sqrt(D), f"small D={D} Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("win,D,Hq,Hkv", [((128, 2, 3), 128, 4, 2), ((128, 1, 15), 128, 2, 2),
                                         ((128, 0, 6), 64, 3, 1), ((128, 4, 12), 64, 2, 1),
                                         ((128, 0, 8), 128, 8, 2), ((128, 2, 10), 128, 8, 2)])
def test_decode_other_windows(lib, win, D, Hq, Hkv):
    """Other window geometries; a 16-block window runs the 1024-thread
    instantiation (one wave per block); grouped heads read a window of more
    than 4 blocks in rounds of 4 (12 blocks: 3 rounds)."""
    lens = [1, 130, 700, 2048, 2049, 3001]
    w = oracle.Window(*win)
    dev, host = build_case(23, len(lens), Hq, Hkv, D, lens, head=win[1], tail=win[2])
    say(f"ssa_decode window={win} D={D} Hq={Hq} Hkv={Hkv}")
    o, lse = lib.decode(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], window=lib.Window(*win), with_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(host["q"], host["k"], host["v"], host["bt"], host["sl"], 1 / math.sqrt(D), w)
    check_close(to_f64(o), ro, f"decode window {win} o")
    check_close(to_f64(lse), rl, f"decode window {win} lse")


def test_decode_cfg3_full(lib):
    """Batch 64, 16/16 heads, d = 128, lengths uniform in [65536, 131072]."""
    lens = synth.decode_seq_lens(3, 64, 65536, 131072)
    dev, host = build_case(3, 64, 16, 16, 128, lens)
    run_and_check(lib, dev, host, 1 / math.sqrt(128), "cfg3 full")


@pytest.mark.parametrize("B,Hq,Hkv", [(32, 16, 8), (64, 12, 4)])
def test_decode_gqa_one_workgroup_per_window(lib, B, Hq, Hkv):
    """Grouped heads with B * Hkv >= 256 windows: one workgroup per window with
    all of its query heads (fewer windows split the heads over two)."""
    rng = np.random.default_rng(41)
    lens = [int(x) for x in rng.integers(1, 6000, size=B)]
    dev, host = build_case(41, B, Hq, Hkv, 128, lens)
    run_and_check(lib, dev, host, 1 / math.sqrt(128), f"gqa {Hq}/{Hkv} B={B}")


def test_decode_gqa_cfg3_full(lib):
    """Grouped heads at the decode workload's contexts: batch 64, 16 query heads
    on 2 kv heads (8 per kv head), d = 128, lengths uniform in [65536, 131072]."""
    lens = synth.decode_seq_lens(3, 64, 65536, 131072)
    dev, host = build_case(5, 64, 16, 2, 128, lens)
    run_and_check(lib, dev, host, 1 / math.sqrt(128), "gqa 16/2 full")


def test_decode_equals_prefill_last_row(lib):
    """The decode of a sequence of length n equals row n - 1 of the prefill."""
    D, H = 128, 2
    for n in [1, 300, 1024, 1153, 4000]:
        qh = synth.seq_tensor(31, synth.Q, 1, n, H, D)
        kh = synth.seq_tensor(31, synth.K, 1, n, H, D)
        vh = synth.seq_tensor(31, synth.V, 1, n, H, D)
        q, k, v = bits_to_dev(qh), bits_to_dev(kh), bits_to_dev(vh)
        say(f"decode==prefill n={n}")
        o_p, l_p = lib.ssa(q, k, v, with_lse=True)
        nb = (n + 127) // 128
        perm = np.random.default_rng(n).permutation(nb + 3)[:nb].astype(np.int32)
        kp = torch.full((nb + 3, H, 128, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        vp = torch.full((nb + 3, H, 128, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        for t in range(nb):
            r = slice(t * 128, min((t + 1) * 128, n))
            cnt = r.stop - r.start
            kp[int(perm[t]), :, :cnt] = k[0, r].transpose(0, 1)
            vp[int(perm[t]), :, :cnt] = v[0, r].transpose(0, 1)
        bt = torch.from_numpy(perm[None]).cuda()
        sl = torch.tensor([n], dtype=torch.int32, device="cuda")
        o_d, l_d = lib.decode(q[:, n - 1], kp, vp, bt, sl, with_lse=True)
        torch.cuda.synchronize()
        ro, rl = oracle.ssa_rows(synth.bf16_bits_to_f32(qh[0, n - 1:n]).astype(np.float64), n - 1,
                                 synth.bf16_bits_to_f32(kh[0]), synth.bf16_bits_to_f32(vh[0]),
                                 1 / math.sqrt(D), [0, 1], H)
        check_close(to_f64(o_d), ro, f"decode n={n}")
        check_close(to_f64(o_p[0, n - 1:n]), ro, f"prefill row n-1 n={n}")
        assert (o_d.float() - o_p[0, n - 1].float()).abs().max().item() <= 1e-2
        assert (l_d - l_p[0, :, n - 1]).abs().max().item() <= 1e-3


def test_decode_invalid_rows_are_nan(lib):
    """Lengths outside [1, max_blocks*128] and page ids outside [0, num_pages)
    give NaN rows; the other rows are unaffected."""
    lens = [500, 1300, 900, 700]
    dev, host = build_case(41, 4, 2, 2, 128, lens)
    sl = dev["sl"].clone()
    bt = dev["bt"].clone()
    sl[1] = 0
    bt[2, (900 - 1) // 128] = 10 ** 6   # own block of sequence 2 points outside the pool
    sl[3] = bt.shape[1] * 128 + 1
    say("decode invalid rows")
    o, lse = lib.decode(dev["q"], dev["k"], dev["v"], bt, sl, with_lse=True)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    assert np.isnan(o[1:]).all() and np.isnan(lse.cpu().numpy()[1:]).all()
    ro, _ = oracle.decode(host["q"], host["k"], host["v"], host["bt"], host["sl"], 1 / math.sqrt(128), batches=[0])
    check_close(o[0:1], ro[0:1], "valid row beside invalid ones")


def test_decode_structural_onehot(lib):
    """q = 0 and V = one-hot(logical block id): o = (#keys in block)/(#keys)."""
    D, H = 128, 1
    lens = np.array([1, 129, 1024, 1025, 3000, 70000], np.int32)
    bt, P = synth.decode_block_table(5, lens, 128)
    kp = torch.zeros((P, H, 128, D), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros((P, H, 128, D), dtype=torch.bfloat16, device="cuda")
    for b, n in enumerate(lens):
        for t in range((int(n) + 127) // 128):
            vp[int(bt[b, t]), :, :, t % D] = 1.0
    q = torch.zeros((len(lens), H, D), dtype=torch.bfloat16, device="cuda")
    say("decode structural")
    o, lse = lib.decode(q, kp, vp, torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(), with_lse=True)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    for b, n in enumerate(lens):
        i = int(n) - 1
        qb = i // 128
        nk = i + 1 if i < 1024 else 897 + (i % 128)
        assert abs(float(lse[b, 0]) - math.log(nk)) < 1e-5
        want = np.zeros(D)
        for t in range(qb + 1):
            c = (i % 128 + 1) if t == qb else (128 if (t == 0 or t >= qb - 6) else 0)
            want[t % D] += c / nk
        assert np.abs(o[b, 0] - want).max() <= 2 ** -8, b


# ---------------------------------------------------------------------------
# dense decode (every cached key; the dense layers of a layer stack)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("D,Hq,Hkv", [(128, 4, 2), (64, 2, 2)])
def test_decode_dense_small(lib, D, Hq, Hkv):
    lens = [1, 2, 127, 128, 129, 1000, 2049, 5000]
    dev, host = build_case(31, len(lens), Hq, Hkv, D, lens, head=1, tail=64)  # every block filled
    say(f"ssa_decode_dense D={D} Hq={Hq} Hkv={Hkv}")
    o, lse = lib.decode_dense(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], with_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_decode(host["q"], host["k"], host["v"], host["bt"], host["sl"], 1 / math.sqrt(D))
    check_close(to_f64(o), ro, f"dense decode D={D} o")
    check_close(to_f64(lse), rl, f"dense decode D={D} lse")


def test_decode_dense_bad_rows(lib):
    lens = [300, 0, 900]
    dev, host = build_case(32, 3, 2, 2, 128, [300, 1, 900], head=1, tail=64)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    bt = dev["bt"].clone()
    bt[2, 3] = 10 ** 6  # a page outside the pool in sequence 2
    say("ssa_decode_dense bad rows")
    o, lse = lib.decode_dense(dev["q"], dev["k"], dev["v"], bt, sl, with_lse=True)
    torch.cuda.synchronize()
    og = to_f64(o)
    assert np.isnan(og[1]).all() and np.isnan(og[2]).all() and np.isnan(to_f64(lse)[[1, 2]]).all()
    ro, rl = oracle.dense_decode(host["q"], host["k"], host["v"], host["bt"], np.array(lens), 1 / math.sqrt(128),
                                 batches=[0])
    check_close(og[0], ro[0], "dense decode bad-rows case, row 0")


def test_decode_dense_long_contexts(lib):
    """4 sequences at 60K-130K tokens (every block read: up to 1016 blocks, 64 groups of 16),
    a device-drawn pool; the oracle checks sequence 1 (all 16 heads) on the pages copied back."""
    lens = synth.decode_seq_lens(33, 4, 60000, 130000)
    bt, P = synth.decode_block_table(33, lens, 128)
    g = torch.Generator(device="cuda")
    g.manual_seed(33)
    kp = torch.randn((P, 16, 128, 128), device="cuda", generator=g).to(torch.bfloat16)
    vp = torch.randn((P, 16, 128, 128), device="cuda", generator=g).to(torch.bfloat16)
    q = torch.randn((4, 16, 128), device="cuda", generator=g).to(torch.bfloat16)
    say(f"ssa_decode_dense lens={list(lens)}")
    o, lse = lib.decode_dense(q, kp, vp, torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(), with_lse=True)
    torch.cuda.synchronize()
    b = 1
    nb = (int(lens[b]) + 127) // 128
    pages = torch.from_numpy(bt[b, :nb].astype(np.int64)).cuda()
    kh = kp[pages].float().cpu().numpy()
    vh = vp[pages].float().cpu().numpy()
    bt_c = np.arange(nb, dtype=np.int32)[None]
    ro, rl = oracle.dense_decode(q[b:b + 1].float().cpu().numpy(), kh, vh, bt_c, lens[b:b + 1], 1 / math.sqrt(128))
    check_close(to_f64(o[b:b + 1]), ro, "dense decode long o")
    check_close(to_f64(lse[b:b + 1]), rl, "dense decode long lse")
