"""The C-ABI library loads, exports every declared symbol, and rejects invalid
arguments on the host before any HIP call (so these run without a GPU).

No test here makes a call that would pass validation: the device pointers used
are fake, so a valid call would launch a kernel on them.
"""
import ctypes
import os
import re

import pytest

import long_context_block_ssa_amd as ssa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssa.LIB_PATH):
        from long_context_block_ssa_amd import _build
        _build.build(verbose=False)
    return ssa.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "ssa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 9
    assert set(names) == set(ssa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version(lib):
    assert lib.ssa_version() == 10000


def good_args(**over):
    a = ssa.CAttnArgs()
    a.dtype = a.out_dtype = ssa.DTYPE_BF16
    a.B, a.L, a.Hq, a.Hkv, a.Dqk, a.Dv = 1, 256, 2, 2, 128, 128
    a.scale = 0.088
    a.q = a.k = a.v = FAKE
    a.o = FAKE + 4096
    a.lse = None
    for s in ("q_stride", "k_stride", "v_stride", "o_stride"):
        setattr(a, s, (ctypes.c_int64 * 3)(256 * 2 * 128, 2 * 128, 128))
    for key, val in over.items():
        setattr(a, key, val)
    return a


def lists(**over):
    li = ssa.CBlockLists()
    li.idx, li.cnt, li.W, li.n_qblocks = FAKE, FAKE, 8, 2
    for key, val in over.items():
        setattr(li, key, val)
    return li


@pytest.mark.parametrize("over,code,needle", [
    (dict(q=None), ssa.SSA_ERR_INVALID, "non-NULL"),
    (dict(o=FAKE + 2), ssa.SSA_ERR_INVALID, "aligned"),
    (dict(B=0), ssa.SSA_ERR_INVALID, "sizes"),
    (dict(L=-5), ssa.SSA_ERR_INVALID, "sizes"),
    (dict(Hq=3), ssa.SSA_ERR_INVALID, "multiple"),
    (dict(scale=0.0), ssa.SSA_ERR_INVALID, "scale"),
    (dict(scale=float("nan")), ssa.SSA_ERR_INVALID, "scale"),
    (dict(dtype=7), ssa.SSA_ERR_INVALID, "dtype"),
    (dict(Dqk=96, Dv=96), ssa.SSA_ERR_UNSUPPORTED, "no kernel"),
    (dict(dtype=ssa.DTYPE_F32, out_dtype=ssa.DTYPE_BF16, Dqk=64, Dv=64), ssa.SSA_ERR_UNSUPPORTED, "no kernel"),
    (dict(q_stride=(ctypes.c_int64 * 3)(1000, 3, 128)), ssa.SSA_ERR_INVALID, "stride"),
    (dict(k_stride=(ctypes.c_int64 * 3)(-256, 256, 128)), ssa.SSA_ERR_INVALID, "stride"),
])
def test_prefill_and_dense_reject(lib, over, code, needle):
    a = good_args(**over)
    li = lists()
    assert lib.ssa_prefill(ctypes.byref(a), ctypes.byref(li), None) == code
    assert needle in lib.ssa_last_error().decode()
    assert lib.ssa_dense_causal(ctypes.byref(a), None) == code


@pytest.mark.parametrize("over,needle", [
    (dict(idx=None), "non-NULL"),
    (dict(W=0), "W="),
    (dict(W=65), "W="),
    (dict(n_qblocks=1), "rows per head"),
    (dict(idx_sh=-1), "strides"),
])
def test_prefill_rejects_bad_lists(lib, over, needle):
    a = good_args()
    li = lists(**over)
    assert lib.ssa_prefill(ctypes.byref(a), ctypes.byref(li), None) == ssa.SSA_ERR_INVALID
    assert needle in lib.ssa_last_error().decode()
    assert lib.ssa_prefill(ctypes.byref(a), None, None) == ssa.SSA_ERR_INVALID


def test_block_index_rejects(lib):
    w = ssa.CWindow(128, 1, 7)
    assert lib.ssa_block_index(None, 4, FAKE, FAKE, None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_block_index(ctypes.byref(w), 0, FAKE, FAKE, None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_block_index(ctypes.byref(w), 4, None, FAKE, None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_block_index(ctypes.byref(w), 4, FAKE + 2, FAKE, None) == ssa.SSA_ERR_INVALID
    bad = ssa.CWindow(128, 1, 0)
    assert lib.ssa_block_index(ctypes.byref(bad), 4, FAKE, FAKE, None) == ssa.SSA_ERR_INVALID
    wide = ssa.CWindow(128, 30, 40)
    assert lib.ssa_block_index(ctypes.byref(wide), 4, FAKE, FAKE, None) == ssa.SSA_ERR_INVALID
    assert "width" in lib.ssa_last_error().decode()
    assert lib.ssa_block_index_seq(ctypes.byref(w), None, 4, FAKE, FAKE, None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_block_index_seq(ctypes.byref(w), FAKE, 0, FAKE, FAKE, None) == ssa.SSA_ERR_INVALID


def decode_args(**over):
    a = ssa.CDecodeArgs()
    a.dtype = ssa.DTYPE_BF16
    a.B, a.Hq, a.Hkv, a.Dqk, a.Dv = 2, 4, 4, 128, 128
    a.page_size, a.num_pages, a.max_blocks = 128, 10, 5
    a.scale = 0.088
    a.q = a.k_pages = a.v_pages = a.o = FAKE
    a.block_table = a.seq_lens = FAKE
    a.q_stride = (ctypes.c_int64 * 2)(512, 128)
    a.k_stride = (ctypes.c_int64 * 3)(4 * 128 * 128, 128 * 128, 128)
    a.v_stride = (ctypes.c_int64 * 3)(4 * 128 * 128, 128 * 128, 128)
    a.o_stride = (ctypes.c_int64 * 2)(512, 128)
    a.bt_stride = 5
    for key, val in over.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("over,code", [
    (dict(block_table=None), ssa.SSA_ERR_INVALID),
    (dict(seq_lens=None), ssa.SSA_ERR_INVALID),
    (dict(page_size=64), ssa.SSA_ERR_INVALID),
    (dict(Hq=6), ssa.SSA_ERR_INVALID),
    (dict(num_pages=0), ssa.SSA_ERR_INVALID),
    (dict(bt_stride=4), ssa.SSA_ERR_INVALID),
    (dict(scale=-1.0), ssa.SSA_ERR_INVALID),
    (dict(dtype=ssa.DTYPE_F32), ssa.SSA_ERR_UNSUPPORTED),
    (dict(Dqk=576, Dv=512, Hkv=2), ssa.SSA_ERR_UNSUPPORTED),
    (dict(Hq=64, Hkv=2), ssa.SSA_ERR_UNSUPPORTED),
    (dict(k_stride=(ctypes.c_int64 * 3)(4 * 128 * 128, 128 * 128, 100)), ssa.SSA_ERR_INVALID),
    # 127 slots of 2^24 elements: a page's rows span more than 2^31 bytes
    (dict(v_stride=(ctypes.c_int64 * 3)(128 << 24, 128, 1 << 24)), ssa.SSA_ERR_UNSUPPORTED),
])
def test_decode_rejects(lib, over, code):
    a = decode_args(**over)
    w = ssa.CWindow(128, 1, 7)
    assert lib.ssa_decode(ctypes.byref(a), ctypes.byref(w), None) == code
    assert lib.ssa_last_error().decode() != ""


def test_decode_rejects_window(lib):
    a = decode_args()
    assert lib.ssa_decode(ctypes.byref(a), None, None) == ssa.SSA_ERR_INVALID
    w = ssa.CWindow(128, 9, 9)  # 18 waves > 16
    assert lib.ssa_decode(ctypes.byref(a), ctypes.byref(w), None) == ssa.SSA_ERR_INVALID


def mla_decode_args(**over):
    base = dict(B=3, Hq=32, Hkv=1, Dqk=576, Dv=512,
                q_stride=(ctypes.c_int64 * 2)(32 * 576, 576),
                k_stride=(ctypes.c_int64 * 3)(128 * 576, 128 * 576, 576),
                v_stride=(ctypes.c_int64 * 3)(128 * 576, 128 * 576, 576),
                o_stride=(ctypes.c_int64 * 2)(32 * 512, 512))
    base.update(over)
    return decode_args(**base)


def chunk_args(**over):
    a = ssa.CChunkArgs()
    a.dtype = a.out_dtype = ssa.DTYPE_BF16
    a.B, a.T, a.Hq, a.Hkv, a.Dqk, a.Dv = 2, 300, 4, 2, 128, 128
    a.page_size, a.num_pages, a.max_blocks = 128, 40, 16
    a.scale = 0.088
    a.q = a.k_pages = a.v_pages = FAKE
    a.o = FAKE + 4096
    a.block_table = a.seq_lens = FAKE
    a.q_stride = (ctypes.c_int64 * 3)(300 * 4 * 128, 4 * 128, 128)
    a.k_stride = (ctypes.c_int64 * 3)(2 * 128 * 128, 128 * 128, 128)
    a.v_stride = (ctypes.c_int64 * 3)(2 * 128 * 128, 128 * 128, 128)
    a.o_stride = (ctypes.c_int64 * 3)(300 * 4 * 128, 4 * 128, 128)
    a.bt_stride = 16
    for key, val in over.items():
        setattr(a, key, val)
    return a


def chunk_lists(**over):
    ls = ssa.CBlockLists()
    ls.idx, ls.cnt, ls.W, ls.n_qblocks = FAKE, FAKE, 8, 16
    for key, val in over.items():
        setattr(ls, key, val)
    return ls


@pytest.mark.parametrize("over,lover,code", [
    (dict(T=0), {}, ssa.SSA_ERR_INVALID),
    (dict(T=16 * 128 + 1), {}, ssa.SSA_ERR_INVALID),      # longer than any cached sequence
    (dict(page_size=64), {}, ssa.SSA_ERR_INVALID),
    (dict(Hq=5), {}, ssa.SSA_ERR_INVALID),
    (dict(bt_stride=15), {}, ssa.SSA_ERR_INVALID),
    (dict(seq_lens=None), {}, ssa.SSA_ERR_INVALID),
    (dict(scale=float("nan")), {}, ssa.SSA_ERR_INVALID),
    (dict(q=FAKE + 8), {}, ssa.SSA_ERR_INVALID),           # alignment
    ({}, dict(n_qblocks=15), ssa.SSA_ERR_INVALID),          # rows must cover every block of max_blocks
    ({}, dict(W=65), ssa.SSA_ERR_INVALID),
    ({}, dict(idx=None), ssa.SSA_ERR_INVALID),
    (dict(Dqk=64, Dv=64), {}, ssa.SSA_ERR_UNSUPPORTED),
    (dict(dtype=ssa.DTYPE_F32, out_dtype=ssa.DTYPE_F32), {}, ssa.SSA_ERR_UNSUPPORTED),
    (dict(k_stride=(ctypes.c_int64 * 3)(128 << 24, 128, 1 << 24)), {}, ssa.SSA_ERR_UNSUPPORTED),
])
def test_prefill_chunk_rejects(lib, over, lover, code):
    a = chunk_args(**over)
    assert lib.ssa_prefill_chunk(ctypes.byref(a), ctypes.byref(chunk_lists(**lover)), None) == code
    assert lib.ssa_last_error().decode() != ""
    assert lib.ssa_prefill_chunk(None, ctypes.byref(chunk_lists()), None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_prefill_chunk(ctypes.byref(chunk_args()), None, None) == ssa.SSA_ERR_INVALID


def bwd_args(**over):
    a = ssa.CBwdArgs()
    a.dtype = ssa.DTYPE_BF16
    a.grad_dtype = ssa.DTYPE_F32
    a.B, a.L, a.Hq, a.Hkv, a.Dqk, a.Dv = 2, 3000, 4, 2, 128, 128
    a.scale = 0.088
    a.q = a.k = a.v = a.o = a.dout = FAKE
    a.lse = FAKE
    a.dq, a.dk, a.dv = FAKE + 4096, FAKE + 8192, FAKE + 12288
    for n, h in (("q_stride", 4), ("o_stride", 4), ("do_stride", 4), ("dq_stride", 4), ("k_stride", 2), ("v_stride", 2),
                 ("dk_stride", 2), ("dv_stride", 2)):
        setattr(a, n, (ctypes.c_int64 * 3)(3000 * h * 128, h * 128, 128))
    for key, val in over.items():
        setattr(a, key, val)
    return a


def test_backward_workspace_size(lib):
    w = ssa.CWindow(128, 1, 7)
    a = bwd_args()
    nqb = (3000 + 127) // 128
    rec = 2 * 4 * nqb * 4 * 64 * 4
    part = 1 * ((nqb + 6) // 7) * 2 * 2 * 2 * 128 * 128 * 4  # one global block, parts of 7 query blocks
    assert lib.ssa_prefill_backward_workspace_size(ctypes.byref(a), ctypes.byref(w)) == \
        ((rec + 255) // 256 * 256 + part + 255) // 256 * 256
    assert lib.ssa_prefill_backward_workspace_size(None, ctypes.byref(w)) == 0


@pytest.mark.parametrize("over,code", [
    (dict(lse=None), ssa.SSA_ERR_INVALID),
    (dict(dout=None), ssa.SSA_ERR_INVALID),
    (dict(Hq=3), ssa.SSA_ERR_INVALID),
    (dict(scale=0.0), ssa.SSA_ERR_INVALID),
    (dict(dq=FAKE + 8), ssa.SSA_ERR_INVALID),
    (dict(grad_dtype=7), ssa.SSA_ERR_INVALID),
    (dict(Dqk=64, Dv=64), ssa.SSA_ERR_UNSUPPORTED),
    (dict(dtype=ssa.DTYPE_F32), ssa.SSA_ERR_UNSUPPORTED),
    (dict(q_stride=(ctypes.c_int64 * 3)(0, 1 << 26, 128)), ssa.SSA_ERR_UNSUPPORTED),
])
def test_backward_rejects(lib, over, code):
    w = ssa.CWindow(128, 1, 7)
    a = bwd_args(workspace=FAKE, workspace_bytes=1 << 40, **over)
    assert lib.ssa_prefill_backward(ctypes.byref(a), ctypes.byref(w), None) == code
    assert lib.ssa_last_error().decode() != ""


def test_backward_workspace_rules(lib):
    w = ssa.CWindow(128, 1, 7)
    a = bwd_args()
    need = lib.ssa_prefill_backward_workspace_size(ctypes.byref(a), ctypes.byref(w))
    assert lib.ssa_prefill_backward(ctypes.byref(a), ctypes.byref(w), None) == ssa.SSA_ERR_WORKSPACE
    a = bwd_args(workspace=FAKE, workspace_bytes=need - 1)
    assert lib.ssa_prefill_backward(ctypes.byref(a), ctypes.byref(w), None) == ssa.SSA_ERR_WORKSPACE
    a = bwd_args(workspace=FAKE + 16, workspace_bytes=need)
    assert lib.ssa_prefill_backward(ctypes.byref(a), ctypes.byref(w), None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_prefill_backward(ctypes.byref(a), None, None) == ssa.SSA_ERR_INVALID


def test_decode_dense_rules(lib):
    a = decode_args()  # B=2, Hq=4, 128/128, max_blocks 5
    need = lib.ssa_decode_dense_workspace_size(ctypes.byref(a))
    assert need == (2 * 4 * 1 * 130 * 4 + 255) // 256 * 256
    assert lib.ssa_decode_dense_workspace_size(None) == 0
    assert lib.ssa_decode_dense(ctypes.byref(a), None) == ssa.SSA_ERR_WORKSPACE
    a = decode_args(workspace=FAKE + 16, workspace_bytes=need)
    assert lib.ssa_decode_dense(ctypes.byref(a), None) == ssa.SSA_ERR_INVALID
    a = mla_decode_args(workspace=FAKE, workspace_bytes=1 << 30)
    assert lib.ssa_decode_dense(ctypes.byref(a), None) == ssa.SSA_ERR_UNSUPPORTED
    assert "ssa_decode_dense" in lib.ssa_last_error().decode()


def test_decode_workspace_size(lib):
    w = ssa.CWindow(128, 1, 7)
    a = mla_decode_args()
    # fp32 (512 channels + m + l + 2 pad) per (sequence, head, window slot)
    assert lib.ssa_decode_workspace_size(ctypes.byref(a), ctypes.byref(w)) == (3 * 32 * 8 * 516 * 4 + 255) // 256 * 256
    w2 = ssa.CWindow(128, 2, 3)
    assert lib.ssa_decode_workspace_size(ctypes.byref(a), ctypes.byref(w2)) == (3 * 32 * 5 * 516 * 4 + 255) // 256 * 256
    assert lib.ssa_decode_workspace_size(ctypes.byref(decode_args()), ctypes.byref(w)) == 0
    assert lib.ssa_decode_workspace_size(None, ctypes.byref(w)) == 0
    assert ssa.decode_workspace_size(3, 32, 576, 512) == (3 * 32 * 8 * 516 * 4 + 255) // 256 * 256


def test_decode_gqa_workspace(lib):
    """Grouped heads at d = 128 need no workspace at any window width (a
    workgroup reads the whole window in rounds of 4 blocks); only the 576/512
    latent does."""
    a = decode_args(Hq=16, Hkv=2)
    for win in (ssa.CWindow(128, 1, 7), ssa.CWindow(128, 1, 3), ssa.CWindow(128, 2, 10)):
        assert lib.ssa_decode_workspace_size(ctypes.byref(a), ctypes.byref(win)) == 0
    assert ssa.decode_workspace_size(2, 16, 128, 128, Hkv=2) == 0
    assert ssa.decode_workspace_size(2, 16, 576, 512) > 0


def test_decode_mla_workspace_rules(lib):
    w = ssa.CWindow(128, 1, 7)
    a = mla_decode_args()
    need = lib.ssa_decode_workspace_size(ctypes.byref(a), ctypes.byref(w))
    assert lib.ssa_decode(ctypes.byref(a), ctypes.byref(w), None) == ssa.SSA_ERR_WORKSPACE
    a = mla_decode_args(workspace=FAKE, workspace_bytes=need - 1)
    assert lib.ssa_decode(ctypes.byref(a), ctypes.byref(w), None) == ssa.SSA_ERR_WORKSPACE
    assert "workspace" in lib.ssa_last_error().decode()
    a = mla_decode_args(workspace=FAKE + 16, workspace_bytes=need)
    assert lib.ssa_decode(ctypes.byref(a), ctypes.byref(w), None) == ssa.SSA_ERR_INVALID
    a = mla_decode_args(Hq=24, workspace=FAKE, workspace_bytes=1 << 30)  # 16 heads per workgroup
    assert lib.ssa_decode(ctypes.byref(a), ctypes.byref(w), None) == ssa.SSA_ERR_UNSUPPORTED


def test_page_select_rejects(lib):
    a = good_args()
    w = ssa.CWindow(128, 1, 7)
    need = lib.ssa_page_select_workspace_size(ctypes.byref(a), ctypes.byref(w))
    nqb = 2
    assert need == (8 * 1 * 2 * nqb * 128 + 255) // 256 * 256 * 2
    assert lib.ssa_page_select(ctypes.byref(a), ctypes.byref(w), 8, FAKE, FAKE, FAKE, need - 1, None) \
        == ssa.SSA_ERR_WORKSPACE
    assert lib.ssa_page_select(ctypes.byref(a), ctypes.byref(w), 8, FAKE, FAKE, None, need, None) \
        == ssa.SSA_ERR_WORKSPACE
    assert lib.ssa_page_select(ctypes.byref(a), ctypes.byref(w), 33, FAKE, FAKE, FAKE, need, None) \
        == ssa.SSA_ERR_INVALID
    assert lib.ssa_page_select(ctypes.byref(a), ctypes.byref(w), 8, FAKE, FAKE, FAKE + 16, need, None) \
        == ssa.SSA_ERR_INVALID  # workspace alignment
    a2 = good_args(Dqk=576, Dv=512)
    assert lib.ssa_page_select(ctypes.byref(a2), ctypes.byref(w), 8, FAKE, FAKE, FAKE, 1 << 30, None) \
        == ssa.SSA_ERR_UNSUPPORTED


def test_page_phases_reject(lib):
    """ssa_page_block_sums / ssa_page_select_top validate like ssa_page_select
    (the sums phase takes no lists), and nothing is launched on an error."""
    a = good_args()
    w = ssa.CWindow(128, 1, 7)
    need = lib.ssa_page_select_workspace_size(ctypes.byref(a), ctypes.byref(w))
    assert lib.ssa_page_block_sums(ctypes.byref(a), ctypes.byref(w), FAKE, need - 1, None) == ssa.SSA_ERR_WORKSPACE
    assert lib.ssa_page_block_sums(ctypes.byref(a), ctypes.byref(w), None, need, None) == ssa.SSA_ERR_WORKSPACE
    assert lib.ssa_page_block_sums(ctypes.byref(a), ctypes.byref(w), FAKE + 16, need, None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_page_block_sums(None, ctypes.byref(w), FAKE, need, None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_page_block_sums(ctypes.byref(good_args(Dqk=576, Dv=512)), ctypes.byref(w), FAKE, 1 << 30, None) \
        == ssa.SSA_ERR_UNSUPPORTED
    assert lib.ssa_page_select_top(ctypes.byref(a), ctypes.byref(w), 8, FAKE, FAKE, FAKE, need - 1, None) \
        == ssa.SSA_ERR_WORKSPACE
    assert lib.ssa_page_select_top(ctypes.byref(a), ctypes.byref(w), 8, None, FAKE, FAKE, need, None) \
        == ssa.SSA_ERR_INVALID
    assert lib.ssa_page_select_top(ctypes.byref(a), ctypes.byref(w), 33, FAKE, FAKE, FAKE, need, None) \
        == ssa.SSA_ERR_INVALID
    assert "ssa_page_select_top" in lib.ssa_last_error().decode()


def test_page_select_noalloc_rejects(lib):
    """Sizes beyond the fixed 32 MiB scratch are refused before any device call;
    the usual argument checks run first."""
    w = ssa.CWindow(128, 1, 7)
    # B=1, Hq=Hkv=16, L=131072, D=128: exactly 32 MiB of sums -- accepted by the size check
    a = good_args(Hq=16, Hkv=16, L=131072)
    assert lib.ssa_page_select_workspace_size(ctypes.byref(a), ctypes.byref(w)) == 32 << 20
    # one more query block on top: refused
    big = good_args(Hq=16, Hkv=16, L=131072 + 1)
    assert lib.ssa_page_select_noalloc(ctypes.byref(big), ctypes.byref(w), 8, FAKE, FAKE, None) \
        == ssa.SSA_ERR_WORKSPACE
    assert "scratch" in lib.ssa_last_error().decode()
    assert lib.ssa_page_select_noalloc(ctypes.byref(good_args()), ctypes.byref(w), 33, FAKE, FAKE, None) \
        == ssa.SSA_ERR_INVALID
    assert lib.ssa_page_select_noalloc(ctypes.byref(good_args()), ctypes.byref(w), 8, None, FAKE, None) \
        == ssa.SSA_ERR_INVALID
    assert lib.ssa_page_select_noalloc(None, ctypes.byref(w), 8, FAKE, FAKE, None) == ssa.SSA_ERR_INVALID
    a2 = good_args(Dqk=576, Dv=512)
    assert lib.ssa_page_select_noalloc(ctypes.byref(a2), ctypes.byref(w), 8, FAKE, FAKE, None) \
        == ssa.SSA_ERR_UNSUPPORTED


def tokens(**over):
    t = ssa.CTokenLists()
    t.tok, t.cnt, t.K, t.n_qblocks = FAKE, FAKE, 512, 2
    for key, val in over.items():
        setattr(t, key, val)
    return t


@pytest.mark.parametrize("aover,tover,code,needle", [
    (dict(), dict(K=-1), ssa.SSA_ERR_INVALID, "K="),
    (dict(), dict(K=1025), ssa.SSA_ERR_INVALID, "K="),
    (dict(), dict(tok=None), ssa.SSA_ERR_INVALID, "non-NULL"),
    (dict(), dict(cnt=None, K=0), ssa.SSA_ERR_INVALID, "non-NULL"),
    (dict(), dict(cnt=FAKE + 2), ssa.SSA_ERR_INVALID, "aligned"),
    (dict(), dict(n_qblocks=1), ssa.SSA_ERR_INVALID, "rows per head"),
    (dict(), dict(tok_sb=-1), ssa.SSA_ERR_INVALID, "strides"),
    (dict(Dqk=64, Dv=64), dict(), ssa.SSA_ERR_UNSUPPORTED, "Dqk = Dv = 128"),
    (dict(B=0), dict(), ssa.SSA_ERR_INVALID, "sizes"),
])
def test_prefill_tokens_rejects(lib, aover, tover, code, needle):
    a = good_args(**aover)
    assert lib.ssa_prefill_tokens(ctypes.byref(a), ctypes.byref(lists()), ctypes.byref(tokens(**tover)),
                                  None) == code
    assert needle in lib.ssa_last_error().decode()
    assert lib.ssa_prefill_tokens(ctypes.byref(good_args()), ctypes.byref(lists()), None, None) \
        == ssa.SSA_ERR_INVALID
    assert lib.ssa_prefill_tokens(ctypes.byref(good_args()), ctypes.byref(lists(W=0)),
                                  ctypes.byref(tokens()), None) == ssa.SSA_ERR_INVALID


def test_token_select_rejects(lib):
    a = good_args()
    w = ssa.CWindow(128, 1, 7)
    need = lib.ssa_page_select_workspace_size(ctypes.byref(a), ctypes.byref(w))
    tneed = lib.ssa_token_select_workspace_size(ctypes.byref(a), ctypes.byref(w), 8)
    R = 1 * 2 * 2
    r256 = lambda x: (x + 255) // 256 * 256
    assert tneed == 3 * r256(4 * R) + 2 * r256(4 * R * 8) + r256(8 * R * 8 * 128)
    assert lib.ssa_token_select_workspace_size(ctypes.byref(a), ctypes.byref(w), 33) == 0
    assert lib.ssa_token_select_workspace_size(None, ctypes.byref(w), 8) == 0

    def call(a=a, w=w, top_m=8, ws=FAKE, nbytes=need, top_k=512, tok=FAKE, tws=FAKE, tbytes=tneed):
        return lib.ssa_token_select(ctypes.byref(a), ctypes.byref(w) if w is not None else None, top_m, FAKE,
                                    FAKE, ws, nbytes, top_k, tok, FAKE, tws, tbytes, None)
    assert call(tbytes=tneed - 1) == ssa.SSA_ERR_WORKSPACE
    assert call(tws=None) == ssa.SSA_ERR_WORKSPACE
    assert call(tws=FAKE + 16) == ssa.SSA_ERR_INVALID
    assert call(nbytes=need - 1) == ssa.SSA_ERR_WORKSPACE
    assert "workspace" in lib.ssa_last_error().decode()
    assert call(ws=None) == ssa.SSA_ERR_WORKSPACE
    assert call(ws=FAKE + 16) == ssa.SSA_ERR_INVALID
    assert call(top_m=33) == ssa.SSA_ERR_INVALID
    assert call(top_k=-1) == ssa.SSA_ERR_INVALID
    assert call(top_k=1025) == ssa.SSA_ERR_INVALID
    assert call(tok=None) == ssa.SSA_ERR_INVALID
    assert call(tok=FAKE + 1) == ssa.SSA_ERR_INVALID
    assert call(w=None) == ssa.SSA_ERR_INVALID
    assert call(w=ssa.CWindow(64, 1, 7)) == ssa.SSA_ERR_UNSUPPORTED
    assert call(a=good_args(Dqk=576, Dv=512)) == ssa.SSA_ERR_UNSUPPORTED
    assert call(a=good_args(dtype=ssa.DTYPE_F32, out_dtype=ssa.DTYPE_F32, Dqk=64, Dv=64)) == ssa.SSA_ERR_UNSUPPORTED
    assert call(a=good_args(Hq=3)) == ssa.SSA_ERR_INVALID
    assert lib.ssa_token_select(None, ctypes.byref(w), 8, FAKE, FAKE, FAKE, need, 8, FAKE, FAKE, FAKE, tneed, None) \
        == ssa.SSA_ERR_INVALID


def test_error_is_thread_local(lib):
    import threading
    a = good_args(B=0)
    li = lists()
    assert lib.ssa_prefill(ctypes.byref(a), ctypes.byref(li), None) == ssa.SSA_ERR_INVALID
    seen = {}

    def other():
        seen["msg"] = lib.ssa_last_error().decode()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "sizes" in lib.ssa_last_error().decode()
