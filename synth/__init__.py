"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module only draws numbers and lays them out; it holds none of the attention
arithmetic.  Every draw is reproducible from ``(seed, tensor_id, chunk ids)`` so
that any 128-row chunk of a large tensor can be regenerated on its own (the
oracle checks sampled rows of multi-GB inputs that way).

Recipe (all configurations):

* values are ``numpy.random.default_rng([seed, tensor_id, b, t])`` standard
  normal float32 draws for the chunk of rows ``t*128 .. t*128+127`` of batch
  ``b`` (all heads, all channels), optionally multiplied by a power-free scale
  (``1/24`` for the 576-wide latent shape, applied in float32 before rounding);
* then rounded to bfloat16 with round-to-nearest-even (what ``tensor.to(bf16)``
  does), or kept as float32 for float32 workloads.

The GPU side receives the bf16 bit patterns; the oracle receives the very same
values widened to float64.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 128

# tensor ids
Q, K, V, LATENT, QDEC = 0, 1, 2, 3, 4


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even; returns the uint16 bit patterns.

    Inputs are finite (they are normal draws), so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _chunk_f32(seed: int, tensor_id: int, b: int, t: int, shape, mul: float) -> np.ndarray:
    rng = np.random.default_rng([seed, tensor_id, b, t])
    x = rng.standard_normal(shape, dtype=np.float32)
    if mul != 1.0:
        x = x * np.float32(mul)
    return x


def rows_chunk(seed: int, tensor_id: int, b: int, t: int, H: int, D: int,
               dtype: str = "bf16", mul: float = 1.0) -> np.ndarray:
    """Rows ``t*128 .. t*128+127`` of batch ``b`` for a logical [B, L, H, D] tensor.

    Returns uint16 bf16 bits (dtype 'bf16') or float32 values (dtype 'f32'),
    shape [128, H, D].  Rows past the sequence end are simply ignored by callers.
    """
    x = _chunk_f32(seed, tensor_id, b, t, (CHUNK, H, D), mul)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def seq_tensor(seed: int, tensor_id: int, B: int, L: int, H: int, D: int,
               dtype: str = "bf16", mul: float = 1.0, workers: int = 8) -> np.ndarray:
    """Whole logical [B, L, H, D] tensor (bf16 bits or float32), chunk by chunk.

    Chunks are independent draws, so they are filled by a thread pool; the
    result does not depend on ``workers``.
    """
    nt = (L + CHUNK - 1) // CHUNK
    out = np.empty((B, nt * CHUNK, H, D), np.uint16 if dtype == "bf16" else np.float32)

    def fill(bt):
        b, t = bt
        out[b, t * CHUNK:(t + 1) * CHUNK] = rows_chunk(seed, tensor_id, b, t, H, D, dtype, mul)

    jobs = [(b, t) for b in range(B) for t in range(nt)]
    if workers > 1 and len(jobs) > 8:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, jobs))
    else:
        for j in jobs:
            fill(j)
    return out[:, :L]


def as_f64(x: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """Widen generated values (bf16 bits or float32) to float64, exactly."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


# ----------------------------------------------------------------------------
# decode workload: per-sequence lengths and a paged cache
# ----------------------------------------------------------------------------

def decode_seq_lens(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    """Context lengths (new token included), uniform integers in [lo, hi]."""
    rng = np.random.default_rng([seed, 99])
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def decode_block_table(seed: int, seq_lens: np.ndarray, block: int, rotation: int = 0,
                       max_blocks: int | None = None):
    """A seeded page table emulating a paged allocator.

    Every sequence owns ceil(n/block) pages; the physical ids of all pages of all
    sequences are a seeded permutation of ``0 .. P-1``.  Returns
    ``(block_table int32 [B, max_blocks] padded with -1, num_pages)``.
    """
    nblk = (seq_lens.astype(np.int64) + block - 1) // block
    P = int(nblk.sum())
    if max_blocks is None:
        max_blocks = int(nblk.max())
    rng = np.random.default_rng([seed, 98, rotation])
    perm = rng.permutation(P).astype(np.int32)
    bt = np.full((len(seq_lens), max_blocks), -1, np.int32)
    off = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt, P


def decode_fill_blocks(seq_lens: np.ndarray, block: int, head: int = 1, tail: int = 8):
    """Logical block ids that receive finite values, per sequence.

    The generator fills the first ``head`` and the last ``tail`` logical blocks
    of every sequence with normal draws; every other page (and, in the caller,
    every slot at or after the sequence end) holds NaN, so a read of cache
    memory that the caller did not mean to expose turns the output into NaN.
    """
    out = []
    for n in seq_lens:
        last = (int(n) - 1) // block
        ids = sorted(set(range(min(head, last + 1))) | set(range(max(0, last - tail + 1), last + 1)))
        out.append(ids)
    return out


def page_chunk(seed: int, tensor_id: int, b: int, t: int, H: int, D: int,
               dtype: str = "bf16", mul: float = 1.0) -> np.ndarray:
    """Values of logical block ``t`` of sequence ``b`` in page layout [H, 128, D]."""
    x = _chunk_f32(seed, tensor_id, b, t, (H, CHUNK, D), mul)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def decode_query(seed: int, B: int, H: int, D: int, dtype: str = "bf16", mul: float = 1.0,
                 rotation: int = 0) -> np.ndarray:
    rng = np.random.default_rng([seed, QDEC, rotation])
    x = rng.standard_normal((B, H, D), dtype=np.float32)
    if mul != 1.0:
        x = x * np.float32(mul)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def torch_normal_bf16(seed: int, shape, mul: float = 1.0, device="cuda"):
    """Seeded N(0,1) * mul draws rounded to bf16, generated on the device by
    torch's own (Philox) generator -- for tensors too large to draw on the host
    (the 38 GB query of the 576-wide latent workload).  Checks copy the rows
    they need back to the host, so both sides read identical values."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    step = 1 << 28
    for s0 in range(0, flat.numel(), step):
        n = min(step, flat.numel() - s0)
        x = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
        if mul != 1.0:
            x.mul_(mul)
        flat[s0:s0 + n].copy_(x)
        del x
    return out
