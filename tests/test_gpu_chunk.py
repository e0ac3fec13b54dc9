"""GPU parity: chunked prefill over a paged cache (a chunk of T new queries per
sequence, each with the window of its own block) against the float64 oracle,
and against ssa_prefill of the whole sequence."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import bits_to_dev, check_close, say, to_f64

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC0  # bf16 NaN


def build_chunk_case(seed, lens, T, Hq, Hkv, D=128, blocks_of=None, poison_pages=()):
    """Paged cache holding finite values only in the blocks ``blocks_of(b, n)``
    lists (default: every block of the sequence), and only in slots < n; every
    other page and slot is NaN.  The queries are the last T positions of each
    sequence.  Returns device tensors and a compact host copy for the oracle."""
    lens = np.asarray(lens, np.int32)
    B = len(lens)
    bt, P = synth.decode_block_table(seed, lens, 128)
    kp = torch.full((P, Hkv, 128, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    vp = torch.full((P, Hkv, 128, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids, kh, vh = [], [], []
    for b in range(B):
        n = int(lens[b])
        nblk = (n + 127) // 128
        blocks = range(nblk) if blocks_of is None else blocks_of(b, n)
        for t in blocks:
            kb = synth.page_chunk(seed, synth.K, b, t, Hkv, D).copy()
            vb = synth.page_chunk(seed, synth.V, b, t, Hkv, D).copy()
            valid = min(128, n - t * 128)
            kb[:, valid:] = NAN_BITS
            vb[:, valid:] = NAN_BITS
            ids.append(int(bt[b, t]))
            kh.append(kb)
            vh.append(vb)
    idx = torch.tensor(ids, dtype=torch.long, device="cuda")
    kp[idx] = bits_to_dev(np.stack(kh)[:, None]).reshape(len(ids), Hkv, 128, D)
    vp[idx] = bits_to_dev(np.stack(vh)[:, None]).reshape(len(ids), Hkv, 128, D)
    remap = {p: i for i, p in enumerate(ids)}
    bt_c = np.full_like(bt, -1)
    for b in range(B):
        for t in range(bt.shape[1]):
            if bt[b, t] in remap:
                bt_c[b, t] = remap[bt[b, t]]
    q_bits = synth.seq_tensor(seed, synth.Q, B, T, Hq, D)[:, :T]
    bt_dev = bt.copy()
    for b, t in poison_pages:  # out-of-pool page ids
        bt_dev[b, t] = P + 7
    dev = dict(q=bits_to_dev(q_bits), k=kp, v=vp, bt=torch.from_numpy(bt_dev).cuda(),
               sl=torch.from_numpy(lens).cuda())
    host = dict(q=synth.bf16_bits_to_f32(q_bits), k=synth.bf16_bits_to_f32(np.stack(kh)),
                v=synth.bf16_bits_to_f32(np.stack(vh)), bt=bt_c, sl=lens)
    return dev, host


def run_chunk(lib, dev, T, out_dtype=None):
    idx, cnt = lib.block_index(dev["bt"].shape[1])
    return lib.prefill_chunk(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], lib.lists_from_index(idx, cnt),
                             out_dtype=out_dtype, with_lse=True)


@pytest.mark.parametrize("T,lens,Hq,Hkv,out_f32", [
    (1, [1, 2, 127, 128, 129, 1025, 5000], 4, 2, False),      # one query: the decode row
    (100, [100, 128, 300, 1000, 4000], 2, 2, False),           # inside one block or across two
    (300, [300, 1024, 1500, 7777], 4, 1, True),                # 3-4 query blocks, GQA 4:1, fp32 out
    (1024, [1024, 1100, 3000], 2, 2, False),                   # the whole window's span
])
def test_chunk_small_nan_poisoned(lib, T, lens, Hq, Hkv, out_f32):
    name = f"ssa_prefill_chunk T={T} lens={lens} Hq={Hq} Hkv={Hkv} f32={out_f32}"
    say(name)
    dev, host = build_chunk_case(31 + T, lens, T, Hq, Hkv)
    o, lse = run_chunk(lib, dev, T, torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    ro, rl = oracle.chunk_prefill(host["q"], host["k"], host["v"], host["bt"], host["sl"], 1 / math.sqrt(128))
    check_close(to_f64(o), ro, f"{name} o")
    check_close(to_f64(lse), rl, f"{name} lse")


@pytest.mark.parametrize("win,T,lens", [
    ((128, 2, 3), 300, [300, 1100, 2600]),   # two global blocks, three local
    ((128, 0, 6), 200, [200, 900, 1999]),    # no global block
    ((128, 4, 12), 700, [700, 3000]),        # 16-block window
])
def test_chunk_other_windows(lib, win, T, lens):
    name = f"ssa_prefill_chunk window={win} T={T} lens={lens}"
    say(name)
    dev, host = build_chunk_case(71 + T, lens, T, 2, 2)
    idx, cnt = lib.block_index(dev["bt"].shape[1], lib.Window(*win))
    o, lse = lib.prefill_chunk(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], lib.lists_from_index(idx, cnt),
                               with_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.chunk_prefill(host["q"], host["k"], host["v"], host["bt"], host["sl"], 1 / math.sqrt(128),
                                  oracle.Window(*win))
    check_close(to_f64(o), ro, f"{name} o")
    check_close(to_f64(lse), rl, f"{name} lse")


def test_chunk_invalid_rows_are_nan(lib):
    """A sequence shorter than the chunk gets NaN rows; a page outside the pool
    turns the rows of the query blocks whose window lists it into NaN (block 0's
    page: every row of the sequence); the other rows are unaffected."""
    lens = [500, 100, 900, 2000, 700]
    T = 200
    # sequence 2 (rows 700..899): block 6 holds rows 768..899, whose window is
    # blocks 0..6; rows 700..767 (block 5) read blocks 0..5 only
    dev, host = build_chunk_case(44, lens, T, 2, 2, poison_pages=[(2, 6), (4, 0)])
    say("ssa_prefill_chunk invalid rows")
    o, lse = run_chunk(lib, dev, T)
    torch.cuda.synchronize()
    og, lg = to_f64(o), to_f64(lse)
    assert np.isnan(og[1]).all() and np.isnan(lg[1]).all()   # n = 100 < T
    assert np.isnan(og[4]).all() and np.isnan(lg[4]).all()   # block 0 outside the pool
    assert np.isnan(og[2, 68:]).all() and np.isnan(lg[2, :, 68:]).all()
    ro, rl = oracle.chunk_prefill(host["q"], host["k"], host["v"], host["bt"], host["sl"], 1 / math.sqrt(128),
                                  batches=[0, 2, 3])
    check_close(og[2, :68], ro[2, :68], "invalid-rows case, batch 2 rows of block 5 o")
    check_close(lg[2, :, :68], rl[2, :, :68], "invalid-rows case, batch 2 rows of block 5 lse")
    for b in (0, 3):
        check_close(og[b], ro[b], f"invalid-rows case, batch {b} o")
        check_close(lg[b], rl[b], f"invalid-rows case, batch {b} lse")


def test_chunks_equal_whole_prefill(lib):
    """Prefilling a 3000-token sequence as chunks of 1000, 1000, 1000 over the
    paged cache gives bit for bit the rows of one ssa_prefill over the whole
    sequence (same blocks, same stages, same arithmetic)."""
    n, Hq, D = 3000, 2, 128
    seed = 55
    q_bits = synth.seq_tensor(seed, synth.Q, 1, n, Hq, D)[:, :n]
    k_bits = synth.seq_tensor(seed, synth.K, 1, n, Hq, D)[:, :n]
    v_bits = synth.seq_tensor(seed, synth.V, 1, n, Hq, D)[:, :n]
    q, k, v = bits_to_dev(q_bits), bits_to_dev(k_bits), bits_to_dev(v_bits)
    say("ssa_prefill whole sequence")
    whole, whole_lse = lib.ssa(q, k, v, with_lse=True)
    # the same sequence in a paged cache
    nblk = (n + 127) // 128
    perm = np.random.default_rng(seed).permutation(nblk + 3)[:nblk].astype(np.int32)
    kp = torch.full((nblk + 3, Hq, 128, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    vp = kp.clone()
    for t in range(nblk):
        r0, r1 = t * 128, min(n, (t + 1) * 128)
        kp[int(perm[t]), :, :r1 - r0] = k[0, r0:r1].transpose(0, 1)
        vp[int(perm[t]), :, :r1 - r0] = v[0, r0:r1].transpose(0, 1)
    bt = torch.from_numpy(perm[None, :]).cuda()
    idx, cnt = lib.block_index(nblk)
    for c0 in (0, 1000, 2000):
        say(f"ssa_prefill_chunk rows {c0}..{c0 + 999}")
        sl = torch.tensor([c0 + 1000], dtype=torch.int32, device="cuda")
        o, lse = lib.prefill_chunk(q[:, c0:c0 + 1000].contiguous(), kp, vp, bt, sl, lib.lists_from_index(idx, cnt),
                                   with_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o, whole[:, c0:c0 + 1000]), f"chunk {c0}: max diff {(o.float() - whole[:, c0:c0 + 1000].float()).abs().max().item()}"
        assert torch.equal(lse, whole_lse[:, :, c0:c0 + 1000])


def test_chunk_full_size_sampled(lib):
    """The benchmark's chunk shape (T = 2048 new tokens at contexts of 64K-128K,
    16 heads, d = 128) on 4 sequences; the oracle checks every row of two of
    them."""
    lens = synth.decode_seq_lens(6, 4, 65536, 131072)
    T = 2048

    def blocks_of(b, n):
        q0 = n - T
        return sorted({0} | set(range(max(0, q0 // 128 - 6), (n + 127) // 128)))

    dev, host = build_chunk_case(61, lens, T, 16, 16, blocks_of=blocks_of)
    say(f"ssa_prefill_chunk full size lens={list(lens)}")
    o, lse = run_chunk(lib, dev, T)
    torch.cuda.synchronize()
    ro, rl = oracle.chunk_prefill(host["q"], host["k"], host["v"], host["bt"], host["sl"], 1 / math.sqrt(128),
                                  batches=[0, 3])
    og, lg = to_f64(o), to_f64(lse)
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    for b in (0, 3):
        check_close(og[b], ro[b], f"full-size chunk batch {b} o")
        check_close(lg[b], rl[b], f"full-size chunk batch {b} lse")
