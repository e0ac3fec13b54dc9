"""The allocation-free page selection (ssa_page_select_noalloc, fixed device
scratch) against ssa_page_select with a caller workspace: identical lists on
two calls in a row, the second with a smaller input (the scratch keeps the
first call's sums, and the second must not see them)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import gen, say

pytestmark = pytest.mark.gpu


def _noalloc(lib, q, k, M):
    """Through the C ABI with preallocated outputs."""
    B, L, Hq, _ = q.shape
    nqb = (L + 127) // 128
    idx = torch.full((B, Hq, nqb, 8 + M), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Hq, nqb), -7, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    a = lib._attn_args(q, k, k, q, None, 1.0)
    w = lib.DEFAULT_WINDOW.c()
    rc = lib.load().ssa_page_select_noalloc(ctypes.byref(a), ctypes.byref(w), M, idx.data_ptr(), cnt.data_ptr(),
                                            torch.cuda.current_stream().cuda_stream)
    assert rc == lib.SSA_OK, lib.last_error()
    return idx, cnt


@pytest.mark.parametrize("first,second", [
    ((131072, 16, 16, 128, 8), (128 * 40 + 17, 2, 1, 128, 8)),    # the full 32 MiB, then a small case
    ((128 * 300 + 5, 4, 2, 64, 4), (128 * 33, 2, 2, 64, 4)),
])
def test_page_select_noalloc_matches_workspace_version(lib, first, second):
    for n, (L, Hq, Hkv, D, M) in enumerate((first, second)):
        _, q = gen(91 + n, synth.Q, 1, L, Hq, D)
        _, k = gen(91 + n, synth.K, 1, L, Hkv, D)
        say(f"page_select_noalloc call {n}: L={L} Hq={Hq} Hkv={Hkv} D={D} M={M}")
        idx, cnt = _noalloc(lib, q, k, M)
        ridx, rcnt = lib.page_select(q, k, top_m=M)
        torch.cuda.synchronize()
        assert torch.equal(cnt, rcnt), f"call {n}: counts differ"
        assert torch.equal(idx, ridx), f"call {n}: lists differ"
        assert int(cnt.min()) >= 1
