"""GPU parity: SSA backward (dq, dk, dv) against the float64 oracle's chain
rule, on the GPU's own bf16 inputs, forward output and lse.

Tolerance for gradients: the kernels multiply P and dS as bf16 MFMA operands
and form delta from the bf16 forward output (each a relative rounding of
2^-9), so the error of a gradient entry scales with the gradients' size; the
check is max |g - g_ref| <= 2^-7 max |g_ref| (4 roundings' worth; at least
1e-5) and mean |g - g_ref| <= 1e-3.  (Rounding only dS to bf16 in float64 already
gives 5.4e-3 on dq for the L = 300 case, whose max |dq| is 3.0.)"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import TOL_MEAN, gen, say, to_f64

pytestmark = pytest.mark.gpu

DOUT = 90  # tensor id of the incoming gradient in the generators


def check_grad(got: np.ndarray, ref: np.ndarray, what: str):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite gradient"
    err = np.abs(got - ref)
    mx, mean, size = float(err.max()), float(err.mean()), float(np.abs(ref).max())
    say(f"{what}: max {mx:.3e} (max|ref| {size:.3e}) mean {mean:.3e}")
    # (an absolute floor of 1e-5 for gradients that vanish exactly, e.g. a row with one key)
    assert mx <= max(2.0 ** -7 * size, 1e-5), f"{what}: max abs err {mx} > 2^-7 * {size}"
    assert mean <= TOL_MEAN, f"{what}: mean abs err {mean}"


def run_case(lib, name, B, L, Hq, Hkv, win=(128, 1, 7), layout="blhd", grad_dtype=None, seed=7):
    say(f"ssa_prefill_backward {name}")
    qh, q = gen(seed, synth.Q, B, L, Hq, 128)
    kh, k = gen(seed, synth.K, B, L, Hkv, 128)
    vh, v = gen(seed, synth.V, B, L, Hkv, 128)
    gh, g = gen(seed, DOUT, B, L, Hq, 128)
    if layout == "bhld":
        q, k, v, g = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v, g))
    w = lib.Window(*win)
    o, lse = lib.ssa(q, k, v, window=w, with_lse=True)
    dq, dk, dv = lib.prefill_backward(q, k, v, o, g, lse, window=w, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.ssa_backward(qh, kh, vh, gh, 1 / math.sqrt(128), oracle.Window(*win))
    for got, ref, what in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        check_grad(to_f64(got), ref, f"{name} {what}")
    return dq, dk, dv


@pytest.mark.parametrize("name,B,L,Hq,Hkv,win,layout,gd", [
    ("L300", 1, 300, 2, 2, (128, 1, 7), "blhd", torch.float32),          # inside the first blocks
    ("L1300-gqa", 1, 1300, 4, 2, (128, 1, 7), "blhd", torch.float32),    # crosses the window; kv heads sum 2 heads
    ("L2100-bhld-bf16", 2, 2100, 2, 2, (128, 1, 7), "bhld", None),      # ragged end, bf16 gradients
    ("L2500-2g3l", 1, 2500, 2, 1, (128, 2, 3), "blhd", torch.float32),   # two global blocks, 3 local
    ("L1", 1, 1, 1, 1, (128, 1, 7), "blhd", torch.float32),
    ("L1700-0g6l", 1, 1700, 2, 2, (128, 0, 6), "blhd", torch.float32),  # no global block: no partials
    ("L1500-1l", 1, 1500, 2, 2, (128, 1, 1), "blhd", torch.float32),    # block 0 and the own block only
    ("L129", 1, 129, 1, 1, (128, 1, 7), "blhd", torch.float32),
])
def test_backward_parity(lib, name, B, L, Hq, Hkv, win, layout, gd):
    run_case(lib, name, B, L, Hq, Hkv, win, layout, gd)


def test_backward_deterministic(lib):
    """Two runs give the same bits (no atomics; the global block's parts are
    summed in a fixed order)."""
    B, L, H = 1, 3000, 2
    _, q = gen(3, synth.Q, B, L, H, 128)
    _, k = gen(3, synth.K, B, L, H, 128)
    _, v = gen(3, synth.V, B, L, H, 128)
    _, g = gen(3, DOUT, B, L, H, 128)
    say("ssa_prefill_backward determinism")
    o, lse = lib.ssa(q, k, v, with_lse=True)
    a = lib.prefill_backward(q, k, v, o, g, lse)
    b = lib.prefill_backward(q, k, v, o, g, lse)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_full_size_two_heads(lib):
    """The prefill workload's shape (B=1, L=32768, 16 heads, d=128, [B, H, L, D]
    layout); the oracle checks every gradient of heads 0 and 11 (heads are
    independent: Hq = Hkv)."""
    B, L, H = 1, 32768, 16
    say("backward full-size inputs")
    qh, q = gen(2, synth.Q, B, L, H, 128)
    kh, k = gen(2, synth.K, B, L, H, 128)
    vh, v = gen(2, synth.V, B, L, H, 128)
    gh, g = gen(2, DOUT, B, L, H, 128)
    q, k, v, g = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v, g))
    say("ssa_prefill_backward full size")
    o, lse = lib.ssa(q, k, v, with_lse=True)
    dq, dk, dv = lib.prefill_backward(q, k, v, o, g, lse, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    heads = [0, 11]
    rq, rk, rv = oracle.ssa_backward(qh[:, :, heads], kh[:, :, heads], vh[:, :, heads], gh[:, :, heads],
                                     1 / math.sqrt(128))
    for got, ref, what in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        check_grad(to_f64(got[:, :, heads]), ref, f"full-size {what}")
