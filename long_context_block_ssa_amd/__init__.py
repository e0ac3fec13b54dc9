"""Python binding of libssa (block-sparse streaming attention on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libssa.so``; torch supplies device memory and the current
stream.  The C entry points are documented in ``include/ssa.h``; the Python
functions carry the same names without the ``ssa_`` prefix.

Tensors use the logical layouts of the header:
  q [B, L, Hq, Dqk], k [B, L, Hkv, Dqk], v [B, L, Hkv, Dv] (any strides, last dim contiguous)
  decode: q [B, Hq, Dqk], k_pages [P, Hkv, 128, Dqk], v_pages [P, Hkv, 128, Dv]

There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import inspect
import math
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SSA_LIB_PATH selects another build of the same library (the host-sanitized
# one, for the CPU-side checks of the C ABI)
LIB_PATH = os.environ.get("SSA_LIB_PATH") or os.path.join(_PKG, "_lib", "libssa.so")

SSA_OK, SSA_ERR_INVALID, SSA_ERR_UNSUPPORTED, SSA_ERR_DEVICE, SSA_ERR_WORKSPACE = range(5)
DTYPE_F32, DTYPE_BF16 = 0, 1

# every symbol include/ssa.h declares
EXPORTS = (
    "ssa_block_index", "ssa_block_index_seq", "ssa_prefill", "ssa_prefill_tokens", "ssa_dense_causal",
    "ssa_prefill_chunk", "ssa_prefill_backward", "ssa_prefill_backward_workspace_size", "ssa_decode",
    "ssa_decode_dense", "ssa_decode_dense_workspace_size", "ssa_decode_workspace_size", "ssa_page_select",
    "ssa_page_select_workspace_size", "ssa_page_select_noalloc", "ssa_page_block_sums", "ssa_page_select_top",
    "ssa_token_select", "ssa_token_select_workspace_size", "ssa_last_error",
    "ssa_version",
)


class SSAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[ssa error {code}] {msg}")
        self.code = code


# ---------------------------------------------------------------------------
# ctypes mirrors of the header's structs
# ---------------------------------------------------------------------------

class CWindow(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("n_global", ctypes.c_int32), ("n_local", ctypes.c_int32)]


class CAttnArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("L", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Dqk", ctypes.c_int32), ("Dv", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
    ]


class CBlockLists(ctypes.Structure):
    _fields_ = [
        ("idx", ctypes.c_void_p), ("cnt", ctypes.c_void_p),
        ("W", ctypes.c_int32), ("n_qblocks", ctypes.c_int32),
        ("idx_sb", ctypes.c_int64), ("idx_sh", ctypes.c_int64),
        ("cnt_sb", ctypes.c_int64), ("cnt_sh", ctypes.c_int64),
    ]


class CTokenLists(ctypes.Structure):
    _fields_ = [
        ("tok", ctypes.c_void_p), ("cnt", ctypes.c_void_p),
        ("K", ctypes.c_int32), ("n_qblocks", ctypes.c_int32),
        ("tok_sb", ctypes.c_int64), ("tok_sh", ctypes.c_int64),
        ("cnt_sb", ctypes.c_int64), ("cnt_sh", ctypes.c_int64),
    ]


class CDecodeArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Dqk", ctypes.c_int32), ("Dv", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64 * 2), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 2),
        ("bt_stride", ctypes.c_int64),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class CChunkArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Dqk", ctypes.c_int32), ("Dv", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("bt_stride", ctypes.c_int64),
    ]


class CBwdArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("L", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Dqk", ctypes.c_int32), ("Dv", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("dout", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3), ("v_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 3), ("do_stride", ctypes.c_int64 * 3),
        ("dq_stride", ctypes.c_int64 * 3), ("dk_stride", ctypes.c_int64 * 3), ("dv_stride", ctypes.c_int64 * 3),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


@dataclass(frozen=True)
class Window:
    """Window geometry; defaults = 1 global + 7 local blocks of 128 tokens."""
    block_size: int = 128
    n_global: int = 1
    n_local: int = 7

    @property
    def width(self) -> int:
        return self.n_global + self.n_local

    def c(self) -> CWindow:
        return CWindow(self.block_size, self.n_global, self.n_local)


DEFAULT_WINDOW = Window()

_lib = None


def load(path: str = LIB_PATH):
    """Load libssa.so (once).  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libssa.so not found at {path}; build it with "
                          "`python -m long_context_block_ssa_amd._build`")
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.ssa_block_index.argtypes = [ctypes.POINTER(CWindow), i32, vp, vp, vp]
    lib.ssa_block_index_seq.argtypes = [ctypes.POINTER(CWindow), vp, i32, vp, vp, vp]
    lib.ssa_prefill.argtypes = [ctypes.POINTER(CAttnArgs), ctypes.POINTER(CBlockLists), vp]
    lib.ssa_prefill_tokens.argtypes = [ctypes.POINTER(CAttnArgs), ctypes.POINTER(CBlockLists),
                                       ctypes.POINTER(CTokenLists), vp]
    lib.ssa_token_select.argtypes = [ctypes.POINTER(CAttnArgs), ctypes.POINTER(CWindow), i32, vp, vp, vp,
                                     ctypes.c_size_t, i32, vp, vp, vp, ctypes.c_size_t, vp]
    lib.ssa_token_select_workspace_size.argtypes = [ctypes.POINTER(CAttnArgs), ctypes.POINTER(CWindow), i32]
    lib.ssa_token_select_workspace_size.restype = ctypes.c_size_t
    lib.ssa_dense_causal.argtypes = [ctypes.POINTER(CAttnArgs), vp]
    lib.ssa_prefill_chunk.argtypes = [ctypes.POINTER(CChunkArgs), ctypes.POINTER(CBlockLists), vp]
    lib.ssa_prefill_backward.argtypes = [ctypes.POINTER(CBwdArgs), ctypes.POINTER(CWindow), vp]
    lib.ssa_prefill_backward_workspace_size.argtypes = [ctypes.POINTER(CBwdArgs), ctypes.POINTER(CWindow)]
    lib.ssa_prefill_backward_workspace_size.restype = ctypes.c_size_t
    lib.ssa_decode.argtypes = [ctypes.POINTER(CDecodeArgs), ctypes.POINTER(CWindow), vp]
    lib.ssa_decode_dense.argtypes = [ctypes.POINTER(CDecodeArgs), vp]
    lib.ssa_decode_dense_workspace_size.argtypes = [ctypes.POINTER(CDecodeArgs)]
    lib.ssa_decode_dense_workspace_size.restype = ctypes.c_size_t
    lib.ssa_decode_workspace_size.argtypes = [ctypes.POINTER(CDecodeArgs), ctypes.POINTER(CWindow)]
    lib.ssa_decode_workspace_size.restype = ctypes.c_size_t
    lib.ssa_page_select_workspace_size.argtypes = [ctypes.POINTER(CAttnArgs), ctypes.POINTER(CWindow)]
    lib.ssa_page_select_workspace_size.restype = ctypes.c_size_t
    lib.ssa_page_select.argtypes = [ctypes.POINTER(CAttnArgs), ctypes.POINTER(CWindow), i32, vp, vp, vp,
                                    ctypes.c_size_t, vp]
    lib.ssa_page_select_noalloc.argtypes = [ctypes.POINTER(CAttnArgs), ctypes.POINTER(CWindow), i32, vp, vp, vp]
    lib.ssa_page_block_sums.argtypes = [ctypes.POINTER(CAttnArgs), ctypes.POINTER(CWindow), vp, ctypes.c_size_t, vp]
    lib.ssa_page_select_top.argtypes = [ctypes.POINTER(CAttnArgs), ctypes.POINTER(CWindow), i32, vp, vp, vp,
                                        ctypes.c_size_t, vp]
    lib.ssa_last_error.restype = ctypes.c_char_p
    lib.ssa_last_error.argtypes = []
    lib.ssa_version.argtypes = []
    for name in ("ssa_block_index", "ssa_block_index_seq", "ssa_prefill", "ssa_dense_causal", "ssa_prefill_chunk",
                 "ssa_decode", "ssa_page_select", "ssa_page_block_sums", "ssa_page_select_top", "ssa_version"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int):
    if rc != SSA_OK:
        raise SSAError(rc, load().ssa_last_error().decode())


def last_error() -> str:
    return load().ssa_last_error().decode()


def version() -> int:
    return load().ssa_version()


def _on_stream(fn):
    """Run an entry point with ``stream`` (when given) as torch's current stream,
    so that the outputs and temporaries it allocates belong to the stream its
    kernels run on: the caching allocator then hands their memory only to work
    ordered after those kernels."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        stream = sig.bind_partial(*args, **kwargs).arguments.get("stream")
        ctx = torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()
        with ctx:
            return fn(*args, **kwargs)
    return wrapper


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return DTYPE_F32
    if t == torch.bfloat16:
        return DTYPE_BF16
    raise SSAError(SSA_ERR_UNSUPPORTED, f"dtype {t} (need float32 or bfloat16)")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _strides3(t: torch.Tensor, name: str):
    if t.dim() != 4:
        raise SSAError(SSA_ERR_INVALID, f"{name} must be 4-d [B, L, H, D], got {tuple(t.shape)}")
    if t.stride(3) != 1:
        raise SSAError(SSA_ERR_INVALID, f"{name} channel dimension must be contiguous")
    return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def _attn_args(q, k, v, o, lse, scale) -> CAttnArgs:
    B, L, Hq, Dqk = q.shape
    Hkv, Dv = k.shape[2], v.shape[3]
    a = CAttnArgs()
    a.dtype = _dtype_code(q.dtype)
    a.out_dtype = _dtype_code(o.dtype)
    a.B, a.L, a.Hq, a.Hkv, a.Dqk, a.Dv = B, L, Hq, Hkv, Dqk, Dv
    a.scale = float(1.0 / math.sqrt(Dqk) if scale is None else scale)
    a.q, a.k, a.v, a.o, a.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse)
    a.q_stride = _strides3(q, "q")
    a.k_stride = _strides3(k, "k")
    a.v_stride = _strides3(v, "v")
    a.o_stride = _strides3(o, "o")
    return a


def _out(q, v, out_dtype, with_lse):
    B, L, Hq, _ = q.shape
    o = torch.empty((B, L, Hq, v.shape[3]), dtype=out_dtype or q.dtype, device=q.device)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device) if with_lse else None
    return o, lse


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

@_on_stream
def block_index(n_qblocks: int, window: Window = DEFAULT_WINDOW, device="cuda", stream=None):
    """ssa_block_index: (idx int32 [n_qblocks, W], cnt int32 [n_qblocks])."""
    lib = load()
    idx = torch.empty((n_qblocks, window.width), dtype=torch.int32, device=device)
    cnt = torch.empty((n_qblocks,), dtype=torch.int32, device=device)
    w = window.c()
    _check(lib.ssa_block_index(ctypes.byref(w), n_qblocks, _ptr(idx), _ptr(cnt), _stream(stream)))
    return idx, cnt


@_on_stream
def block_index_seq(seq_lens: torch.Tensor, window: Window = DEFAULT_WINDOW, stream=None):
    """ssa_block_index_seq for decode rows (seq_lens int32 [B] on the device)."""
    lib = load()
    B = seq_lens.shape[0]
    idx = torch.empty((B, window.width), dtype=torch.int32, device=seq_lens.device)
    cnt = torch.empty((B,), dtype=torch.int32, device=seq_lens.device)
    w = window.c()
    _check(lib.ssa_block_index_seq(ctypes.byref(w), _ptr(seq_lens), B, _ptr(idx), _ptr(cnt), _stream(stream)))
    return idx, cnt


def lists_from_index(idx: torch.Tensor, cnt: torch.Tensor) -> CBlockLists:
    """Block lists shared by every batch and head (the SSA window).  The struct
    holds raw device pointers: keep idx and cnt alive while it is in use."""
    lists = CBlockLists()
    lists.idx, lists.cnt = _ptr(idx), _ptr(cnt)
    lists.W, lists.n_qblocks = idx.shape[1], idx.shape[0]
    lists.idx_sb = lists.idx_sh = lists.cnt_sb = lists.cnt_sh = 0
    return lists


def lists_per_head(idx: torch.Tensor, cnt: torch.Tensor) -> CBlockLists:
    """Block lists per (batch, query head): idx [B, Hq, nqb, W], cnt [B, Hq, nqb].
    Keep idx and cnt alive while the struct is in use."""
    assert idx.is_contiguous() and cnt.is_contiguous()
    B, H, nqb, W = idx.shape
    lists = CBlockLists()
    lists.idx, lists.cnt = _ptr(idx), _ptr(cnt)
    lists.W, lists.n_qblocks = W, nqb
    lists.idx_sb, lists.idx_sh = H * nqb * W, nqb * W
    lists.cnt_sb, lists.cnt_sh = H * nqb, nqb
    return lists


@_on_stream
def prefill(q, k, v, lists: CBlockLists, scale=None, out=None, out_dtype=None, with_lse=False,
            lse=None, stream=None):
    """ssa_prefill over the given block lists.  Returns (o, lse or None)."""
    lib = load()
    if out is None:
        out, lse2 = _out(q, v, out_dtype, with_lse)
        lse = lse if lse is not None else lse2
    a = _attn_args(q, k, v, out, lse, scale)
    _check(lib.ssa_prefill(ctypes.byref(a), ctypes.byref(lists), _stream(stream)))
    return out, lse


@_on_stream
def ssa(q, k, v, scale=None, window: Window = DEFAULT_WINDOW, out_dtype=None, with_lse=False, stream=None):
    """Block index + SSA prefill, the two calls of the hot path."""
    nqb = (q.shape[1] + window.block_size - 1) // window.block_size
    idx, cnt = block_index(nqb, window, device=q.device, stream=stream)
    return prefill(q, k, v, lists_from_index(idx, cnt), scale=scale, out_dtype=out_dtype,
                   with_lse=with_lse, stream=stream)


@_on_stream
def dense_causal(q, k, v, scale=None, out=None, out_dtype=None, with_lse=False, lse=None, stream=None):
    """ssa_dense_causal: the dense comparison layer."""
    lib = load()
    if out is None:
        out, lse2 = _out(q, v, out_dtype, with_lse)
        lse = lse if lse is not None else lse2
    a = _attn_args(q, k, v, out, lse, scale)
    _check(lib.ssa_dense_causal(ctypes.byref(a), _stream(stream)))
    return out, lse


@_on_stream
def prefill_chunk(q, k_pages, v_pages, block_table, seq_lens, lists: CBlockLists, scale=None, out=None,
                  out_dtype=None, with_lse=False, lse=None, stream=None):
    """ssa_prefill_chunk: q [B, T, Hq, D] = the last T positions of each cached
    sequence (seq_lens counts them).  Returns (o [B, T, Hq, Dv], lse [B, Hq, T] or None)."""
    lib = load()
    B, T, Hq, Dqk = q.shape
    P, Hkv, page, _ = k_pages.shape
    Dv = v_pages.shape[3]
    if out is None:
        out = torch.empty((B, T, Hq, Dv), dtype=out_dtype or q.dtype, device=q.device)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    for t, name in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (out, "o")):
        if t.stride(-1) != 1:
            raise SSAError(SSA_ERR_INVALID, f"{name} channel dimension must be contiguous")
    a = CChunkArgs()
    a.dtype, a.out_dtype = _dtype_code(q.dtype), _dtype_code(out.dtype)
    a.B, a.T, a.Hq, a.Hkv, a.Dqk, a.Dv = B, T, Hq, Hkv, Dqk, Dv
    a.page_size, a.num_pages, a.max_blocks = page, P, block_table.shape[1]
    a.scale = float(1.0 / math.sqrt(Dqk) if scale is None else scale)
    a.q, a.k_pages, a.v_pages = _ptr(q), _ptr(k_pages), _ptr(v_pages)
    a.block_table, a.seq_lens, a.o, a.lse = _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse)
    a.q_stride = (ctypes.c_int64 * 3)(q.stride(0), q.stride(1), q.stride(2))
    a.k_stride = (ctypes.c_int64 * 3)(k_pages.stride(0), k_pages.stride(1), k_pages.stride(2))
    a.v_stride = (ctypes.c_int64 * 3)(v_pages.stride(0), v_pages.stride(1), v_pages.stride(2))
    a.o_stride = (ctypes.c_int64 * 3)(out.stride(0), out.stride(1), out.stride(2))
    a.bt_stride = block_table.stride(0)
    _check(lib.ssa_prefill_chunk(ctypes.byref(a), ctypes.byref(lists), _stream(stream)))
    return out, lse


def _bwd_args(q, k, v, o, dout, lse, dq, dk, dv, scale) -> CBwdArgs:
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        if t.dim() != 4 or t.stride(-1) != 1:
            raise SSAError(SSA_ERR_INVALID, f"{name} must be [B, L, H, D] with a contiguous channel dimension")
    a = CBwdArgs()
    a.dtype, a.grad_dtype = _dtype_code(q.dtype), _dtype_code(dq.dtype)
    a.B, a.L, a.Hq, a.Dqk = q.shape
    a.Hkv, a.Dv = k.shape[2], v.shape[3]
    a.scale = float(1.0 / math.sqrt(a.Dqk) if scale is None else scale)
    a.q, a.k, a.v, a.o, a.dout, a.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse)
    a.dq, a.dk, a.dv = _ptr(dq), _ptr(dk), _ptr(dv)
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", o), ("do_stride", dout),
                    ("dq_stride", dq), ("dk_stride", dk), ("dv_stride", dv)):
        setattr(a, name, (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2)))
    return a


def prefill_backward_workspace_size(q, k, window: Window = DEFAULT_WINDOW) -> int:
    a = CBwdArgs()
    a.B, a.L, a.Hq, _ = q.shape
    a.Hkv = k.shape[2]
    w = window.c()
    return int(load().ssa_prefill_backward_workspace_size(ctypes.byref(a), ctypes.byref(w)))


@_on_stream
def prefill_backward(q, k, v, o, dout, lse, scale=None, window: Window = DEFAULT_WINDOW, grad_dtype=None,
                     dq=None, dk=None, dv=None, workspace=None, stream=None):
    """ssa_prefill_backward: (dq, dk, dv) of the SSA prefill whose output o and
    lse [B, Hq, L] (fp32) the forward returned; dout is the gradient of o."""
    lib = load()
    gd = grad_dtype or q.dtype
    dq = torch.empty(q.shape, dtype=gd, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=gd, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=gd, device=q.device) if dv is None else dv
    a = _bwd_args(q, k, v, o, dout, lse, dq, dk, dv, scale)
    w = window.c()
    need = int(lib.ssa_prefill_backward_workspace_size(ctypes.byref(a), ctypes.byref(w)))
    if workspace is None:
        workspace = torch.empty((need + 256,), dtype=torch.uint8, device=q.device)
    base = workspace.data_ptr()
    off = (-base) % 256
    a.workspace, a.workspace_bytes = base + off, max(workspace.numel() - off, 0)
    _check(lib.ssa_prefill_backward(ctypes.byref(a), ctypes.byref(w), _stream(stream)))
    return dq, dk, dv


def decode_workspace_size(B: int, Hq: int, Dqk: int, Dv: int, window: Window = DEFAULT_WINDOW,
                          Hkv: int | None = None) -> int:
    """ssa_decode_workspace_size: bytes of device workspace ssa_decode needs (0 for most shapes);
    ``Hkv`` defaults to Hq (one query head per kv head)."""
    a = CDecodeArgs()
    a.B, a.Hq, a.Hkv, a.Dqk, a.Dv = B, Hq, Hq if Hkv is None else Hkv, Dqk, Dv
    w = window.c()
    return int(load().ssa_decode_workspace_size(ctypes.byref(a), ctypes.byref(w)))


@_on_stream
def decode(q, k_pages, v_pages, block_table, seq_lens, scale=None, window: Window = DEFAULT_WINDOW,
           out=None, with_lse=False, lse=None, workspace=None, stream=None):
    """ssa_decode over a paged cache.  Returns (o [B, Hq, Dv], lse [B, Hq] or None).

    ``workspace`` (a uint8 device tensor) is allocated here when the shape
    needs one and none is given."""
    lib = load()
    B, Hq, Dqk = q.shape
    P, Hkv, page, _ = k_pages.shape
    Dv = v_pages.shape[3]
    if out is None:
        out = torch.empty((B, Hq, Dv), dtype=q.dtype, device=q.device)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    for t, name in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (out, "o")):
        if t.stride(-1) != 1:
            raise SSAError(SSA_ERR_INVALID, f"{name} channel dimension must be contiguous")
    a = CDecodeArgs()
    a.dtype = _dtype_code(q.dtype)
    a.B, a.Hq, a.Hkv, a.Dqk, a.Dv = B, Hq, Hkv, Dqk, Dv
    a.page_size, a.num_pages, a.max_blocks = page, P, block_table.shape[1]
    a.scale = float(1.0 / math.sqrt(Dqk) if scale is None else scale)
    a.q, a.k_pages, a.v_pages = _ptr(q), _ptr(k_pages), _ptr(v_pages)
    a.block_table, a.seq_lens, a.o, a.lse = _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse)
    a.q_stride = (ctypes.c_int64 * 2)(q.stride(0), q.stride(1))
    a.k_stride = (ctypes.c_int64 * 3)(k_pages.stride(0), k_pages.stride(1), k_pages.stride(2))
    a.v_stride = (ctypes.c_int64 * 3)(v_pages.stride(0), v_pages.stride(1), v_pages.stride(2))
    a.o_stride = (ctypes.c_int64 * 2)(out.stride(0), out.stride(1))
    a.bt_stride = block_table.stride(0)
    w = window.c()
    need = int(lib.ssa_decode_workspace_size(ctypes.byref(a), ctypes.byref(w)))
    if need > 0:
        if workspace is None:
            workspace = torch.empty((need + 256,), dtype=torch.uint8, device=q.device)
        base = workspace.data_ptr()
        off = (-base) % 256
        a.workspace, a.workspace_bytes = base + off, max(workspace.numel() - off, 0)
    _check(lib.ssa_decode(ctypes.byref(a), ctypes.byref(w), _stream(stream)))
    return out, lse


@_on_stream
def decode_dense(q, k_pages, v_pages, block_table, seq_lens, scale=None, out=None, with_lse=False, lse=None,
                 workspace=None, stream=None):
    """ssa_decode_dense: the new query over every cached key.  Returns (o [B, Hq, Dv], lse or None)."""
    lib = load()
    B, Hq, Dqk = q.shape
    P, Hkv, page, _ = k_pages.shape
    Dv = v_pages.shape[3]
    if out is None:
        out = torch.empty((B, Hq, Dv), dtype=q.dtype, device=q.device)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    a = CDecodeArgs()
    a.dtype = _dtype_code(q.dtype)
    a.B, a.Hq, a.Hkv, a.Dqk, a.Dv = B, Hq, Hkv, Dqk, Dv
    a.page_size, a.num_pages, a.max_blocks = page, P, block_table.shape[1]
    a.scale = float(1.0 / math.sqrt(Dqk) if scale is None else scale)
    a.q, a.k_pages, a.v_pages = _ptr(q), _ptr(k_pages), _ptr(v_pages)
    a.block_table, a.seq_lens, a.o, a.lse = _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse)
    a.q_stride = (ctypes.c_int64 * 2)(q.stride(0), q.stride(1))
    a.k_stride = (ctypes.c_int64 * 3)(k_pages.stride(0), k_pages.stride(1), k_pages.stride(2))
    a.v_stride = (ctypes.c_int64 * 3)(v_pages.stride(0), v_pages.stride(1), v_pages.stride(2))
    a.o_stride = (ctypes.c_int64 * 2)(out.stride(0), out.stride(1))
    a.bt_stride = block_table.stride(0)
    need = int(lib.ssa_decode_dense_workspace_size(ctypes.byref(a)))
    if workspace is None:
        workspace = torch.empty((need + 256,), dtype=torch.uint8, device=q.device)
    base = workspace.data_ptr()
    off = (-base) % 256
    a.workspace, a.workspace_bytes = base + off, max(workspace.numel() - off, 0)
    _check(lib.ssa_decode_dense(ctypes.byref(a), _stream(stream)))
    return out, lse


def page_select_workspace_size(q, k, window: Window = DEFAULT_WINDOW) -> int:
    lib = load()
    dummy_o = q  # only shapes are read
    a = _attn_args(q, k, k, dummy_o, None, 1.0)
    w = window.c()
    return int(lib.ssa_page_select_workspace_size(ctypes.byref(a), ctypes.byref(w)))


@_on_stream
def page_select(q, k, top_m: int = 8, window: Window = DEFAULT_WINDOW, workspace=None, stream=None):
    """ssa_page_select: (idx int32 [B, Hq, nqb, W], cnt int32 [B, Hq, nqb])."""
    lib = load()
    B, L, Hq, D = q.shape
    nqb = (L + window.block_size - 1) // window.block_size
    W = window.width + top_m
    idx = torch.empty((B, Hq, nqb, W), dtype=torch.int32, device=q.device)
    cnt = torch.empty((B, Hq, nqb), dtype=torch.int32, device=q.device)
    a = _attn_args(q, k, k, q, None, 1.0)
    w = window.c()
    need = int(lib.ssa_page_select_workspace_size(ctypes.byref(a), ctypes.byref(w)))
    if workspace is None:
        workspace = torch.empty((need + 256,), dtype=torch.uint8, device=q.device)
    base = workspace.data_ptr()
    off = (-base) % 256
    _check(lib.ssa_page_select(ctypes.byref(a), ctypes.byref(w), top_m, _ptr(idx), _ptr(cnt),
                               base + off, workspace.numel() - off, _stream(stream)))
    return idx, cnt


@_on_stream
def page_block_sums(q, k, workspace, window: Window = DEFAULT_WINDOW, stream=None):
    """ssa_page_block_sums: the fp64 block sums of q and k into ``workspace``
    (uint8, at least page_select_workspace_size + 256 bytes); returns it."""
    lib = load()
    a = _attn_args(q, k, k, q, None, 1.0)
    w = window.c()
    base = workspace.data_ptr()
    off = (-base) % 256
    _check(lib.ssa_page_block_sums(ctypes.byref(a), ctypes.byref(w), base + off, workspace.numel() - off,
                                   _stream(stream)))
    return workspace


@_on_stream
def page_select_top(q, k, workspace, top_m: int = 8, window: Window = DEFAULT_WINDOW, stream=None):
    """ssa_page_select_top: (idx, cnt) of ssa_page_select from the block sums
    ``page_block_sums`` left in ``workspace``."""
    lib = load()
    B, L, Hq, D = q.shape
    nqb = (L + window.block_size - 1) // window.block_size
    W = window.width + top_m
    idx = torch.empty((B, Hq, nqb, W), dtype=torch.int32, device=q.device)
    cnt = torch.empty((B, Hq, nqb), dtype=torch.int32, device=q.device)
    a = _attn_args(q, k, k, q, None, 1.0)
    w = window.c()
    base = workspace.data_ptr()
    off = (-base) % 256
    _check(lib.ssa_page_select_top(ctypes.byref(a), ctypes.byref(w), top_m, _ptr(idx), _ptr(cnt), base + off,
                                   workspace.numel() - off, _stream(stream)))
    return idx, cnt


@_on_stream
def page_select_noalloc(q, k, top_m: int = 8, window: Window = DEFAULT_WINDOW, idx=None, cnt=None, stream=None):
    """ssa_page_select_noalloc: page selection with the library's fixed scratch
    (no workspace).  Pass preallocated ``idx`` [B, Hq, nqb, W] / ``cnt``
    [B, Hq, nqb] (int32, contiguous) to allocate nothing here either."""
    lib = load()
    B, L, Hq, D = q.shape
    nqb = (L + window.block_size - 1) // window.block_size
    W = window.width + top_m
    if idx is None:
        idx = torch.empty((B, Hq, nqb, W), dtype=torch.int32, device=q.device)
    if cnt is None:
        cnt = torch.empty((B, Hq, nqb), dtype=torch.int32, device=q.device)
    if tuple(idx.shape) != (B, Hq, nqb, W) or tuple(cnt.shape) != (B, Hq, nqb) or not (
            idx.is_contiguous() and cnt.is_contiguous()):
        raise SSAError(SSA_ERR_INVALID, "idx / cnt must be contiguous [B, Hq, nqb, W] / [B, Hq, nqb]")
    a = _attn_args(q, k, k, q, None, 1.0)
    w = window.c()
    _check(lib.ssa_page_select_noalloc(ctypes.byref(a), ctypes.byref(w), top_m, _ptr(idx), _ptr(cnt),
                                       _stream(stream)))
    return idx, cnt


def _aligned256(workspace):
    base = workspace.data_ptr()
    off = (-base) % 256
    return base + off, workspace.numel() - off


def token_lists(tok: torch.Tensor, tok_cnt: torch.Tensor) -> CTokenLists:
    """Token lists per (batch, query head): tok [B, Hq, nqb, K], tok_cnt [B, Hq, nqb].
    Keep tok and tok_cnt alive while the struct is in use."""
    assert tok.is_contiguous() and tok_cnt.is_contiguous()
    B, H, nqb, K = tok.shape
    t = CTokenLists()
    t.tok, t.cnt = _ptr(tok), _ptr(tok_cnt)
    t.K, t.n_qblocks = K, nqb
    t.tok_sb, t.tok_sh = H * nqb * K, nqb * K
    t.cnt_sb, t.cnt_sh = H * nqb, nqb
    return t


@_on_stream
def prefill_tokens(q, k, v, lists: CBlockLists, tokens: CTokenLists, scale=None, out=None, out_dtype=None,
                   with_lse=False, lse=None, stream=None):
    """ssa_prefill_tokens: attention over the block lists plus the token lists.  Returns (o, lse or None)."""
    lib = load()
    if out is None:
        out, lse2 = _out(q, v, out_dtype, with_lse)
        lse = lse if lse is not None else lse2
    a = _attn_args(q, k, v, out, lse, scale)
    _check(lib.ssa_prefill_tokens(ctypes.byref(a), ctypes.byref(lists), ctypes.byref(tokens), _stream(stream)))
    return out, lse


def token_select_workspace_size(q, k, top_m: int = 8, window: Window = DEFAULT_WINDOW) -> int:
    lib = load()
    a = _attn_args(q, k, k, q, None, 1.0)
    w = window.c()
    return int(lib.ssa_token_select_workspace_size(ctypes.byref(a), ctypes.byref(w), top_m))


@_on_stream
def token_select(q, k, page_idx, page_cnt, page_workspace, top_m: int = 8, top_k: int = 512,
                 window: Window = DEFAULT_WINDOW, workspace=None, stream=None):
    """ssa_token_select after page_select(q, k, top_m, window, workspace=page_workspace):
    (tok int32 [B, Hq, nqb, top_k], tok_cnt int32 [B, Hq, nqb])."""
    lib = load()
    B, L, Hq, _ = q.shape
    nqb = (L + window.block_size - 1) // window.block_size
    tok = torch.empty((B, Hq, nqb, top_k), dtype=torch.int32, device=q.device)
    tcnt = torch.empty((B, Hq, nqb), dtype=torch.int32, device=q.device)
    a = _attn_args(q, k, k, q, None, 1.0)
    w = window.c()
    if workspace is None:
        need = int(lib.ssa_token_select_workspace_size(ctypes.byref(a), ctypes.byref(w), top_m))
        workspace = torch.empty((need + 256,), dtype=torch.uint8, device=q.device)
    pbase, pbytes = _aligned256(page_workspace)
    wbase, wbytes = _aligned256(workspace)
    _check(lib.ssa_token_select(ctypes.byref(a), ctypes.byref(w), top_m, _ptr(page_idx), _ptr(page_cnt), pbase,
                                pbytes, top_k, _ptr(tok), _ptr(tcnt), wbase, wbytes, _stream(stream)))
    return tok, tcnt


@_on_stream
def hi_attention(q, k, v, top_m: int = 8, top_k: int = 512, scale=None, window: Window = DEFAULT_WINDOW,
                 out_dtype=None, with_lse=False, with_pages=False, stream=None):
    """Both stages of hierarchical indexing, then attention over the window blocks
    plus the chosen tokens.  Returns (o, lse, tok, tok_cnt), followed by the
    first stage's (page_idx, page_cnt) when ``with_pages``."""
    B, L, Hq, _ = q.shape
    ws = torch.empty((page_select_workspace_size(q, k, window) + 256,), dtype=torch.uint8, device=q.device)
    pidx, pcnt = page_select(q, k, top_m, window, workspace=ws, stream=stream)
    tok, tcnt = token_select(q, k, pidx, pcnt, ws, top_m, top_k, window, stream=stream)
    nqb = (L + window.block_size - 1) // window.block_size
    widx, wcnt = block_index(nqb, window, device=q.device, stream=stream)
    o, lse = prefill_tokens(q, k, v, lists_from_index(widx, wcnt), token_lists(tok, tcnt), scale=scale,
                            out_dtype=out_dtype, with_lse=with_lse, stream=stream)
    if with_pages:
        return o, lse, tok, tcnt, pidx, pcnt
    return o, lse, tok, tcnt


@_on_stream
def page_attention(q, k, v, top_m: int = 8, scale=None, window: Window = DEFAULT_WINDOW, out_dtype=None,
                   with_lse=False, stream=None):
    """Page selection followed by attention over the per-head lists."""
    idx, cnt = page_select(q, k, top_m, window, stream=stream)
    o, lse = prefill(q, k, v, lists_per_head(idx, cnt), scale=scale, out_dtype=out_dtype,
                     with_lse=with_lse, stream=stream)
    return o, lse, idx, cnt
