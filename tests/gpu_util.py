"""Helpers for the GPU parity tests: upload generated inputs, compare with the
oracle.  Inputs come from ``synth`` only; expected values from ``oracle`` only."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth

TOL_MAX = 1e-2   # max |o - o_ref| over the checked elements
TOL_MEAN = 1e-3  # mean |o - o_ref|


def say(msg: str):
    """Name the case before each GPU step (flushed, so a fault still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def bits_to_dev(bits: np.ndarray, layout: str = "blhd") -> torch.Tensor:
    """uint16 bf16 bits, logical [B, L, H, D] -> device bf16 tensor (logical
    [B, L, H, D]); layout 'bhld' stores it head-major and returns a permuted view."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    if layout == "bhld":
        return t.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    return t.contiguous().cuda()


def f32_to_dev(x: np.ndarray, layout: str = "blhd") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if layout == "bhld":
        return t.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    return t.contiguous().cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def gen(seed, tid, B, L, H, D, dtype="bf16", mul=1.0):
    """(host values as float32 exactly, device tensor)."""
    x = synth.seq_tensor(seed, tid, B, L, H, D, dtype, mul)
    if dtype == "bf16":
        return synth.bf16_bits_to_f32(x), bits_to_dev(x)
    return x, f32_to_dev(x)


def check_close(got: np.ndarray, ref: np.ndarray, what: str, rel: bool = False):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    say(f"{what}: max {mx:.3e} mean {mean:.3e}")
    assert mx <= TOL_MAX, f"{what}: max abs err {mx}"
    assert mean <= TOL_MEAN, f"{what}: mean abs err {mean}"
    if rel:
        scale = float(np.abs(ref).max())
        assert mx / scale <= 1e-2, f"{what}: max err / max|ref| = {mx / scale}"
    return mx, mean
