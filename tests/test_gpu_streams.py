"""GPU parity on a side stream: entry points that allocate outputs and
temporaries (workspaces, lists) run on a caller-given stream while torch's
current stream keeps allocating and filling fresh tensors.  The temporaries
must belong to the side stream, or the caching allocator could hand their
memory to the current stream's fills while the kernels still use it."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import check_close, gen, say, to_f64
from tests.test_gpu_decode import build_case

pytestmark = pytest.mark.gpu


def _churn(n=24, numel=1 << 22):
    """Allocate, fill and free tensors on the current stream."""
    for i in range(n):
        t = torch.empty((numel,), dtype=torch.float32, device="cuda")
        t.fill_(float(i) + 0.5)
        del t


def test_side_stream_hi_attention_and_decode(lib):
    L, H, D, M, K = 128 * 30 + 11, 2, 128, 8, 300
    qh, q = gen(71, synth.Q, 1, L, H, D)
    kh, k = gen(71, synth.K, 1, L, H, D)
    vh, v = gen(71, synth.V, 1, L, H, D)
    lens = [1, 129, 1500, 4000, 9000]
    dev, host = build_case(72, len(lens), 4, 2, 128, lens)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    say("side stream: hi_attention, decode, dense decode and ssa while the current stream churns")
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        o, lse, tok, tcnt, pidx, pcnt = lib.hi_attention(q, k, v, top_m=M, top_k=K, with_lse=True,
                                                         with_pages=True, stream=side)
        _churn()
        od, ld = lib.decode(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], with_lse=True, stream=side)
        _churn()
        os_, ls_ = lib.ssa(q, k, v, with_lse=True, stream=side)
        _churn()
        outs.append((o, lse, tok, tcnt, pidx, pcnt, od, ld, os_, ls_))
    side.synchronize()
    torch.cuda.synchronize()

    scale = 1 / math.sqrt(D)
    o, lse, tok, tcnt, pidx, pcnt, od, ld, os_, ls_ = outs[0]
    for later in outs[1:]:     # the kernels are deterministic: every repetition agrees bit for bit
        for a, b in zip(outs[0], later):
            assert torch.equal(a, b)
    gp, gc = pidx.cpu().numpy(), pcnt.cpu().numpy()
    ridx, rcnt, pnear = oracle.page_select(qh, kh, top_m=M)
    assert not pnear.any() and np.array_equal(gp, ridx) and np.array_equal(gc, rcnt)
    rtok, rtcnt, near = oracle.token_select(qh, kh, gp, gc, top_k=K)
    assert not near.any()
    assert np.array_equal(tok.cpu().numpy(), rtok) and np.array_equal(tcnt.cpu().numpy(), rtcnt)
    nqb = (L + 127) // 128
    wi, wc = oracle.block_index(nqb)
    w4 = np.broadcast_to(wi[None, None], (1, H, nqb, wi.shape[1]))
    c3 = np.broadcast_to(wc[None, None], (1, H, nqb))
    ro, rl = oracle.token_list_attention(qh, kh, vh, scale, w4, c3, rtok, rtcnt)
    check_close(to_f64(o), ro, "side stream hi o")
    check_close(to_f64(lse), rl, "side stream hi lse")
    rdo, rdl = oracle.decode(host["q"], host["k"], host["v"], host["bt"], host["sl"], 1 / math.sqrt(128))
    check_close(to_f64(od), rdo, "side stream decode o")
    check_close(to_f64(ld), rdl, "side stream decode lse")
    rso, rsl = oracle.ssa_attention(qh, kh, vh, scale)
    check_close(to_f64(os_), rso, "side stream ssa o")
    check_close(to_f64(ls_), rsl, "side stream ssa lse")
