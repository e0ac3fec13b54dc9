#!/usr/bin/env python3
"""Benchmark of the SSA hot path on one MI355X.

One step = one pass over every row of the path on resident synthetic inputs:

  a1  block index            (256 query blocks)
  a2  SSA prefill            B=1, H=16, d=128, L=32768, bf16, layout [B, H, L, D]
                             (and the small fp32 case B=1, H=1, d=64, L=2048, timed too)
  a3  SSA decode             batch 64, H=16/16, d=128, context ~ U[65536, 131072]
                             (and grouped heads: the same batch with 16 query heads on 2 kv heads)
  a4  latent-shared shape    prefill B=1, L=262144, 128 heads x 576/512 (V = first 512
                             channels of the shared latent); decode batch 8 at 1,048,576
  a5  dense causal layer     same tensors as a2 (the comparison layer)
  a6+a7 page selection       L=131072, H=16, d=128, M=8
  a8  page-selected prefill  over those lists
  f1  chunked prefill        16 sequences at context ~ U[65536, 131072], the last 2048
                             tokens of each as one chunk over the paged cache, H=16/16, d=128
  f3  SSA backward           dq, dk, dv of the a2 prefill (its output and lse computed once
                             outside the timed region; dout ~ N(0,1))

The headline value is the SSA prefill throughput (algorithmic TFLOP/s: 4*d per
(query, key) pair the window admits) at the L=32768 workload; the decode GB/s
(algorithmic bytes: every admitted key and value row once, plus q and o) at
the ~128K-context decode workload is reported beside it, each with its
fraction of the MI355X peak (bf16 dense MFMA 2.5 PFLOP/s, HBM 8 TB/s).  Kernel
times come from HIP timing events (no system-scope fence on completion)
recorded on the stream the kernels run on.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
    python bench.py --zigzag     # f4: dense/SSA layer-stack prefill timing at 128K and 256K
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3
PEAK_FP64_TFLOPS = 78.6


class TimingEvent:
    """A HIP event used only for timing, recorded on torch's current stream (the
    stream the library's kernels are launched on).  It is created with
    hipEventDisableSystemFence: a default event performs a system-scope memory
    fence when it completes (cache writeback and invalidation), which puts
    several microseconds between the kernels on either side of it; a timing
    event needs none.  The calls go to the HIP runtime torch has loaded (found
    in the process's memory map), so that its stream handles are valid."""

    FLAGS = 0x20000000  # hipEventDisableSystemFence
    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            with open("/proc/self/maps") as f:
                paths = {line.split()[-1] for line in f if "libamdhip64.so" in line}
            if len(paths) != 1:
                raise RuntimeError(f"expected one loaded HIP runtime, found {sorted(paths)}")
            cls._hip = ctypes.CDLL(paths.pop())
        return cls._hip

    def __init__(self):
        import ctypes
        self._c = ctypes
        hip = self._runtime()
        self.ev = ctypes.c_void_p()
        self._check(hip.hipEventCreateWithFlags(ctypes.byref(self.ev), ctypes.c_uint(self.FLAGS)), "create")

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise RuntimeError(f"hipEvent {what} failed: error {rc}")

    def record(self):
        import torch
        stream = self._c.c_void_p(torch.cuda.current_stream().cuda_stream)
        self._check(self._hip.hipEventRecord(self.ev, stream), "record")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (waits for `end`)."""
        self._check(self._hip.hipEventSynchronize(end.ev), "synchronize")
        ms = self._c.c_float()
        self._check(self._hip.hipEventElapsedTime(self._c.byref(ms), self.ev, end.ev), "elapsed time")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


# ----------------------------------------------------------------------------
# workload sizes and algorithmic work (closed forms of the window)
# ----------------------------------------------------------------------------

W1 = dict(B=1, L=2048, H=1, D=64, seed=1)
W2 = dict(B=1, L=32768, H=16, D=128, seed=2)
W3 = dict(B=64, H=16, D=128, lo=65536, hi=131072, seed=3, Hkv_gqa=2)
W5 = dict(B=1, L=131072, H=16, D=128, M=8, K=512, seed=5)
W4 = dict(L=262144, H=128, DQK=576, DV=512, seed=4, dec_B=8, dec_n=1048576, dec_rot=32)
W6 = dict(B=16, T=2048, H=16, D=128, lo=65536, hi=131072, seed=6)


def keys_ssa(i: int) -> int:
    """Keys a query at position i reads: 1 global + 7 local blocks of 128."""
    return i + 1 if i < 1024 else 128 + 6 * 128 + (i % 128) + 1


def keys_page(i: int, M: int = 8) -> int:
    w = 128 * (8 + M)
    return i + 1 if i < w else w - 128 + (i % 128) + 1


def pairs(L: int, keys) -> int:
    # per 128-row block the count is an arithmetic series; sum exactly
    return sum(keys(i) for i in range(L))


def ssa_flops(L, H, D, B=1):
    return 4 * D * pairs(L, keys_ssa) * H * B


def mla_flops(L, H, DQK, DV, B=1):
    return 2 * (DQK + DV) * pairs(L, keys_ssa) * H * B


def mla_decode_bytes(lens, Hq, DQK, DV):
    # the latent row is read once and serves as key and value
    return sum(keys_ssa(int(n) - 1) for n in lens) * DQK * 2 + len(lens) * Hq * (DQK + DV) * 2


def dense_flops(L, H, D, B=1):
    return 4 * D * (L * (L + 1) // 2) * H * B


def page_flops(L, H, D, M, B=1):
    return 4 * D * pairs(L, lambda i: keys_page(i, M)) * H * B


def hi_tokens(qb: int, M: int, K: int) -> int:
    """Tokens the second hierarchical stage keeps for query block qb: the
    recalled pages outside the window are min(M, qb - 7) (all of them while
    they number at most M), 128 tokens each, of which K at most."""
    return min(K, 128 * min(M, max(qb - 7, 0)))


def hi_flops(L, H, D, M, K, B=1):
    """4d flops per (query, key) pair: the window's keys plus the block's tokens."""
    return 4 * D * (pairs(L, keys_ssa) + sum(128 * hi_tokens(qb, M, K) for qb in range(L // 128))) * H * B


def chunk_flops(lens, T, H, D):
    """4*d per admitted pair over the last T positions of every sequence."""
    return 4 * D * H * sum(keys_ssa(i) for n in lens for i in range(int(n) - T, int(n)))


def bwd_flops(L, H, D, B=1):
    """5 products of 2*d flops per admitted pair: S recomputed, dP, dV, dQ, dK."""
    return 10 * D * pairs(L, keys_ssa) * H * B


def decode_bytes(lens, Hq, Hkv, Dqk, Dv):
    kv = sum(keys_ssa(int(n) - 1) for n in lens) * Hkv * (Dqk + Dv) * 2
    return kv + len(lens) * Hq * (Dqk + Dv) * 2


# ----------------------------------------------------------------------------
# CPU baseline: the float64 oracle on the host cores (runs before any GPU use,
# so the worker pool is forked from a process that holds no HIP state)
# ----------------------------------------------------------------------------

_CPU = {}


def _cpu_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _cpu_task(qb):
    import oracle
    q, k, v = _CPU["q"], _CPU["k"], _CPU["v"]
    H = q.shape[2]
    rows = slice(qb * 128, (qb + 1) * 128)
    oracle.ssa_rows(q[0, rows], qb * 128, k[0], v[0], 1 / math.sqrt(q.shape[3]), list(range(H)), H)
    return qb


def host_cores():
    """Host cores this process may use: its CPU affinity set, capped by the
    cgroup CPU quota and by OMP_NUM_THREADS when those are set (a GPU machine gives
    each GPU a share of its cores and says so there), with the CPU model."""
    n = len(os.sched_getaffinity(0))
    limits = {"affinity": n}
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if quota != "max":
            limits["cgroup_quota"] = max(1, int(int(quota) // int(period)))
    except (OSError, ValueError):
        pass
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        limits["omp_num_threads"] = max(1, int(os.environ["OMP_NUM_THREADS"]))
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return min(limits.values()), model, limits


def cpu_baseline(budget_s: float = 25.0):
    L, H, D, seed = W2["L"], W2["H"], W2["D"], W2["seed"]
    _CPU["q"] = synth.bf16_bits_to_f32(synth.seq_tensor(seed, synth.Q, 1, L, H, D))
    _CPU["k"] = synth.bf16_bits_to_f32(synth.seq_tensor(seed, synth.K, 1, L, H, D))
    _CPU["v"] = synth.bf16_bits_to_f32(synth.seq_tensor(seed, synth.V, 1, L, H, D))
    cores, model, limits = host_cores()
    ctx = mp.get_context("fork")
    nqb = L // 128
    order = list(range(nqb - 1, -1, -1))  # bench order: last query blocks first
    done = []
    passes = 0
    with ctx.Pool(cores, initializer=_cpu_init) as pool:
        pool.map(_cpu_task, order[:cores])  # start the workers
        t0 = time.perf_counter()
        # whole passes over the workload until about `budget_s` seconds of wall
        # time (stopping early inside a pass if one pass is longer than that)
        while time.perf_counter() - t0 < budget_s / 2:
            for qb in pool.imap_unordered(_cpu_task, order, chunksize=1):
                done.append(qb)
                if time.perf_counter() - t0 > budget_s:
                    break
            passes += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        pool.terminate()
    flops = sum(4 * D * sum(keys_ssa(i) for i in range(qb * 128, (qb + 1) * 128)) * H for qb in done)
    _CPU.clear()
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "cpu_model": model,
        "core_limits": limits,
        "kind": "oracle",
        "sample": f"float64 numpy oracle, SSA prefill of the L={L} H={H} d={D} workload: {len(done)} query-block "
                  f"rows x {H} heads ({len(done) / nqb:.2f} passes over its {nqb} query blocks), "
                  f"{dt:.1f} s wall on {cores} processes (one per usable host core, {model})",
        "seconds": dt,
    }


def cpu_rows_baseline():
    """The float64 oracle on a small sample of every other row's workload, one
    process and one BLAS thread, each reported in that row's unit (the work of
    the sample over its wall time).  Inputs are synthetic of the same shapes;
    the 576-wide rows use generator draws instead of the benchmark's
    device-side ones (the values do not change the time)."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except Exception:
        limit = None
    out = {}

    def timed(name, unit, work, sample, fn, min_s=1.0):
        # the sample again and again until at least min_s seconds of wall time
        t0 = time.perf_counter()
        reps = 0
        while True:
            fn()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_s:
                break
        out[name] = {"value": work * reps / dt / (1e12 if unit == "TFLOP/s" else 1e9), "unit": unit, "cores": 1,
                     "kind": "oracle", "sample": f"{sample} (x{reps})", "seconds": dt}

    f64 = lambda bits: synth.bf16_bits_to_f32(bits).astype(np.float64)
    # a3 decode: 4 of the 64 sequences
    B3, H3, D3, s3 = W3["B"], W3["H"], W3["D"], W3["seed"]
    Hkv3g = W3["Hkv_gqa"]
    nd = 16
    lens = synth.decode_seq_lens(s3, B3, W3["lo"], W3["hi"])[:nd]
    fill = synth.decode_fill_blocks(lens, 128, 1, 7)
    bt = np.full((nd, int(lens.max()) // 128 + 1), -1, np.int32)
    kh, vh = [], []
    for b, blocks in enumerate(fill):
        for t in blocks:
            bt[b, t] = len(kh)
            kh.append(synth.page_chunk(s3, synth.K, b, t, H3, D3))
            vh.append(synth.page_chunk(s3, synth.V, b, t, H3, D3))
    kp, vp = f64(np.stack(kh)), f64(np.stack(vh))
    q3 = f64(synth.decode_query(s3, nd, H3, D3))
    timed("a3 ssa_decode", "GB/s", decode_bytes(lens, H3, H3, D3, D3),
          f"{nd} of the 64 sequences of the decode workload",
          lambda: oracle.decode(q3, kp, vp, bt, lens, 1 / math.sqrt(D3)))
    # a2 inputs serve the dense, backward rows (two heads)
    L2, H2, D2, s2 = W2["L"], W2["H"], W2["D"], W2["seed"]
    q2 = f64(synth.seq_tensor(s2, synth.Q, 1, L2, H2, D2)[:, :, :2])
    k2 = f64(synth.seq_tensor(s2, synth.K, 1, L2, H2, D2)[:, :, :2])
    v2 = f64(synth.seq_tensor(s2, synth.V, 1, L2, H2, D2)[:, :, :2])
    qb = L2 // 128 - 1
    timed("a5 dense_causal", "TFLOP/s", 4 * D2 * sum(range(qb * 128 + 1, L2 + 1)) * 2,
          "dense causal rows of the last query block, 2 of the 16 heads",
          lambda: oracle.dense_causal_rows(q2[0, qb * 128:], qb * 128, k2[0], v2[0], 1 / math.sqrt(D2), [0, 1], 2))
    g2 = f64(synth.seq_tensor(s2, 90, 1, L2, H2, D2)[:, :, :1])
    timed("f3 ssa_backward", "TFLOP/s", bwd_flops(L2, 1, D2),
          "whole backward of 1 of the 16 heads of the prefill workload",
          lambda: oracle.ssa_backward(q2[:, :, :1], k2[:, :, :1], v2[:, :, :1], g2, 1 / math.sqrt(D2)))
    # a6-a8 page selection: head 0 of the L=131072 workload
    L5, H5, D5, M5, s5 = W5["L"], W5["H"], W5["D"], W5["M"], W5["seed"]
    q5 = synth.bf16_bits_to_f32(synth.seq_tensor(s5, synth.Q, 1, L5, H5, D5)[:, :, :1])
    k5 = synth.bf16_bits_to_f32(synth.seq_tensor(s5, synth.K, 1, L5, H5, D5)[:, :, :1])
    sel = {}
    timed("a6-a7 page_select", "GB/s", 2 * L5 * D5 * 2, "block sums, scores and top-8 lists of 1 of the 16 heads",
          lambda: sel.update(r=oracle.page_select(q5, k5, top_m=M5)))
    v5 = synth.bf16_bits_to_f32(synth.seq_tensor(s5, synth.V, 1, L5, H5, D5)[:, :, :1])
    idx, cnt = sel["r"][:2]
    qbs = list(range(L5 // 128 - 16, L5 // 128))
    timed("a8 page_prefill", "TFLOP/s", 4 * D5 * sum(keys_page(i, M5) for qb_ in qbs for i in range(qb_ * 128, qb_ * 128 + 128)),
          "rows of the last 16 query blocks, 1 of the 16 heads",
          lambda: [oracle.block_list_rows(q5[0, qb_ * 128:(qb_ + 1) * 128].astype(np.float64), qb_ * 128, k5[0], v5[0],
                                          1 / math.sqrt(D5), [0], 1, [list(idx[0, 0, qb_, :cnt[0, 0, qb_]])])
                   for qb_ in qbs])
    # f2: the second hierarchical stage for head 0, attention of the last 16 query blocks
    K5 = W5["K"]
    tsel = {}
    cand = sum(128 * min(M5, max(qb_ - 7, 0)) for qb_ in range(L5 // 128) if 128 * min(M5, max(qb_ - 7, 0)) > K5)
    timed("f2 token_select", "GFLOP/s", 2 * D5 * cand, "top-512 token lists of every query block of 1 of the 16 heads",
          lambda: tsel.update(r=oracle.token_select(q5, k5, idx, cnt, top_k=K5)))
    tok, tcnt = tsel["r"][:2]
    wi, wc = oracle.block_index(L5 // 128)
    w4 = wi[None, None]
    c3 = wc[None, None]
    q5d = q5.astype(np.float64)
    timed("f2 hi_prefill", "TFLOP/s",
          4 * D5 * sum(keys_ssa(i) + hi_tokens(qb_, M5, K5) for qb_ in qbs for i in range(qb_ * 128, qb_ * 128 + 128)),
          "rows of the last 16 query blocks, 1 of the 16 heads",
          lambda: oracle.token_list_attention(q5d, k5, v5, 1 / math.sqrt(D5), w4, c3, tok, tcnt, rows=qbs))
    # a4: the 576-wide shape (one query block x 16 of the 128 heads; one decode sequence)
    H4, DQ4, DV4 = W4["H"], W4["DQK"], W4["DV"]
    L4s = 2048
    c4 = f64(synth.seq_tensor(W4["seed"], synth.K, 1, L4s, 1, DQ4, mul=1 / 24))
    q4 = f64(synth.seq_tensor(W4["seed"], synth.Q, 1, 128, 16, DQ4, mul=1 / 24))
    timed("a4 mla_prefill", "TFLOP/s", 2 * (DQ4 + DV4) * sum(keys_ssa(i) for i in range(L4s - 128, L4s)) * 16,
          "one query block at position 1920..2047 (a full window), 16 of the 128 heads",
          lambda: oracle.ssa_rows(q4[0], L4s - 128, c4[0], c4[0, :, :, :DV4], 1 / 24, list(range(16)), 16))
    pages = c4[0].reshape(L4s // 128, 128, 1, DQ4).transpose(0, 2, 1, 3)
    q4d = f64(synth.decode_query(W4["seed"], 1, H4, DQ4, mul=1 / 24))
    timed("a4 mla_decode", "GB/s", mla_decode_bytes([L4s], H4, DQ4, DV4), "one sequence of 2048 keys (a full window), 128 heads",
          lambda: oracle.decode(q4d, pages, pages[..., :DV4], np.arange(L4s // 128, dtype=np.int32)[None],
                                np.array([L4s]), 1 / 24))
    # f1: one sequence's 2048-token chunk, 2 of the 16 heads
    B6, T6, H6, D6, s6 = W6["B"], W6["T"], W6["H"], W6["D"], W6["seed"]
    n6 = int(synth.decode_seq_lens(s6, B6, W6["lo"], W6["hi"])[0])
    need = sorted({0} | set(range((n6 - T6) // 128 - 6, (n6 + 127) // 128)))
    bt6 = np.full((1, (n6 + 127) // 128), -1, np.int32)
    kh6, vh6 = [], []
    for t in need:
        bt6[0, t] = len(kh6)
        kh6.append(synth.page_chunk(s6, synth.K, 0, t, H6, D6)[:2])
        vh6.append(synth.page_chunk(s6, synth.V, 0, t, H6, D6)[:2])
    q6 = f64(synth.seq_tensor(s6, synth.Q, 1, T6, H6, D6)[:, :, :2])
    timed("f1 chunk_prefill", "TFLOP/s", chunk_flops([n6], T6, 2, D6), "the 2048-token chunk of 1 of the 16 sequences, 2 of the 16 heads",
          lambda: oracle.chunk_prefill(q6, f64(np.stack(kh6)), f64(np.stack(vh6)), bt6, np.array([n6]), 1 / math.sqrt(D6)))
    if limit is not None:
        limit.unregister() if hasattr(limit, "unregister") else None
    return out


# ----------------------------------------------------------------------------
# GPU part
# ----------------------------------------------------------------------------

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.txt")
KERNEL_SOURCES = {  # row key -> (kernel-name fragments in the trace, source file)
    "ssa_prefill": (("prefill_d128_kernel",), "prefill_d128.hip"),
    "ssa_decode": (("decode_mha_kernel", "128"), "decode.hip"),
    "mla_prefill": (("prefill_wide_kernel", "576"), "prefill_wide.hip"),
    "mla_decode": (("decode_mla_partial_kernel", "true"), "decode_mla.hip"),
    "ssa_decode_gqa": (("decode_gqa_kernel",), "decode_gqa.hip"),
}


def source_sha(fname: str) -> str:
    src = os.path.join(ROOT, "long_context_block_ssa_amd", "csrc", fname)
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def traffic_for(key: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current source of the kernel; else None."""
    try:
        for line in open(TRAFFIC_FILE):
            f = line.split()
            if len(f) >= 4 and f[0] == key and f[2] == source_sha(KERNEL_SOURCES[key][1]):
                return float(f[1])
    except OSError:
        pass
    return None


def write_traffic(fetch_dir: str, write_dir: str, out_path: str):
    """Per-launch HBM bytes from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE,
    KiB per dispatch) of `bench.py --only prefill,decode,mla,copy`, each scaled
    by what the same counter reads for the plain 1 GiB copy (which moves exactly
    1 GiB each way)."""
    import csv
    import glob

    def per_kernel(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
                vals[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"]) * 1024.0
        return vals  # kernel name -> {dispatch: bytes}

    def pick(vals, frags):
        per = [v for k, v in vals.items() if all(f in k for f in frags)]
        if not per:
            return None
        d = per[0]
        return sum(d.values()) / len(d)

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    copy_bytes = float(1 << 30)
    # the calibration copy is the largest copy dispatch of the run
    copy_f = [x for k, v in fetch.items() if "copy" in k.lower() for x in v.values()]
    copy_w = [x for k, v in write.items() if "copy" in k.lower() for x in v.values()]
    fcal = copy_bytes / max(copy_f) if copy_f and max(copy_f) > 0 else 1.0
    wcal = copy_bytes / max(copy_w) if copy_w and max(copy_w) > 0 else 1.0
    run = ("cd /tmp && rocprofv3 --pmc {c} --output-format csv -d <out>/pmc_{c} -o run -- python3 "
           "/root/repo/bench.py --only prefill,decode,mla,copy --steps 2 --warmup 1 --no-cpu-baseline")
    lines = [f"# HBM bytes per launch: FETCH_SIZE * {fcal:.4f} + WRITE_SIZE * {wcal:.4f} (per dispatch, averaged);",
             "# factors = 1 GiB / the counter's reading on a plain 1 GiB device copy (bench.py --only copy).",
             "# commands: " + run.format(c="FETCH_SIZE"),
             "#           " + run.format(c="WRITE_SIZE"),
             "#           python3 bench.py --write-traffic <out>/pmc_FETCH_SIZE <out>/pmc_WRITE_SIZE profiles/traffic.txt",
             "# key bytes_per_launch source_sha fetch_bytes write_bytes"]
    for key, (frags, fname) in KERNEL_SOURCES.items():
        fb, wb = pick(fetch, frags), pick(write, frags)
        if fb is not None and wb is not None:
            fb, wb = fb * fcal, wb * wcal
            lines.append(f"{key} {fb + wb:.0f} {source_sha(fname)} {fb:.0f} {wb:.0f}")
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


# counter groups for the per-kernel summaries: each fits one rocprofv3 pass
# (at most 8 SQ, 2 TA, 2 TD counters)
COUNTER_GROUPS = [
    "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT "
    "SQ_LDS_IDX_ACTIVE",
    "SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_MISC SQ_INST_CYCLES_VMEM "
    "SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_ANY",
    "SQ_WAIT_ANY SQ_ACTIVE_INST_VMEM SQ_INST_CYCLES_VMEM_RD SQ_ACTIVE_INST_SCA SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_SALU "
    "SQ_INSTS_VMEM_RD SQ_ACTIVE_INST_FLAT TA_TA_BUSY_sum TA_ADDR_STALLED_BY_TC_CYCLES_sum",
    "TD_TD_BUSY_sum TD_TC_STALL_sum TA_DATA_STALLED_BY_TC_CYCLES_sum TA_ADDR_STALLED_BY_TD_CYCLES_sum SQ_BUSY_CYCLES",
]


def write_counters(root: str, frags: str, out_path: str, title: str, command: str):
    """Per-kernel summary of the COUNTER_GROUPS passes under ROOT (one
    sub-directory per pass, each a rocprofv3 --pmc --kernel-trace run): the
    counters averaged per dispatch of the kernels whose name holds every
    comma-separated fragment of FRAGS (a fragment 'grid=N' matches the grid
    size in threads instead), and the derived figures of the MI355X's 8 XCDs x
    4 shader engines, 256 CUs and 1024 SIMDs."""
    import csv
    import glob

    want = [f for f in frags.split(",") if f]

    def match(name, grid):
        for f in want:
            if f.startswith("grid="):
                if str(grid) != f[5:]:
                    return False
            elif f not in name:
                return False
        return True

    vals, durs = {}, []
    for f in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        per = {}
        for r in csv.DictReader(open(f)):
            grid = r.get("Grid_Size", r.get("Grid_Size_X", ""))
            if not match(r["Kernel_Name"], grid):
                continue
            per.setdefault(r["Counter_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
            per[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        for c, d in per.items():
            vals[c] = sum(d.values()) / len(d)
    for f in glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if match(r["Kernel_Name"], r.get("Grid_Size_X", "")):
                durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    if not vals:
        raise RuntimeError(f"no counters for kernel fragments {frags} under {root}")
    dur = sorted(durs)[len(durs) // 2] if durs else float("nan")
    v = vals.get
    lines = [f"# {title}", f"# {command}",
             f"# kernel duration under the counters (median over {len(durs)} dispatches): {dur * 1e6:.1f} us",
             f"{'counter':40s} {'per_dispatch':>14s}"]
    lines += [f"{k:40s} {x:14.4g}" for k, x in sorted(vals.items())]
    lines.append("")
    lines.append("derived (MI355X: 8 XCDs x 4 shader engines, 256 CUs, 1024 SIMDs)")
    busy = v("SQ_BUSY_CYCLES")
    if busy and dur == dur:
        clk = busy / 32 / dur
        cyc = dur * clk
        lines.append(f"shader clock       SQ_BUSY_CYCLES / 32 SEs / duration               {clk / 1e9:.2f} GHz")
        if v("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
            lines.append(f"MFMA utilisation   SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles)  "
                         f"{100 * v('SQ_VALU_MFMA_BUSY_CYCLES') / (1024 * cyc):.1f} %")
        for ctr, name in (("TA_TA_BUSY_sum", "TA busy"), ("TD_TD_BUSY_sum", "TD busy")):
            if v(ctr) is not None:
                lines.append(f"{name:18s} {ctr} / (256 CUs x cycles)               {100 * v(ctr) / (256 * cyc):.1f} %")
        if v("TD_TD_BUSY_sum") and v("TD_TC_STALL_sum") is not None:
            lines.append(f"TD stalled on TC   TD_TC_STALL_sum / TD_TD_BUSY_sum                    "
                         f"{100 * v('TD_TC_STALL_sum') / v('TD_TD_BUSY_sum'):.1f} %")
    waves = v("SQ_WAVES")
    if waves:
        parts = [f"{v(c) / waves:.0f} {n}" for c, n in (("SQ_INSTS_MFMA", "MFMA"), ("SQ_INSTS_VALU", "VALU (MFMA included)"),
                                                        ("SQ_INSTS_VALU_TRANS_F32", "trans"), ("SQ_INSTS_SALU", "SALU"),
                                                        ("SQ_INSTS_LDS", "LDS"), ("SQ_INSTS_VMEM_RD", "VMEM reads"))
                 if v(c) is not None]
        lines.append("per wave           " + ", ".join(parts))
    wc = v("SQ_WAVE_CYCLES")
    if wc and v("SQ_ACTIVE_INST_ANY") is not None and v("SQ_WAIT_INST_ANY") is not None and v("SQ_WAIT_ANY") is not None:
        lines.append(f"wave time          issuing {100 * v('SQ_ACTIVE_INST_ANY') / wc:.0f} %, blocked on issue "
                     f"{100 * v('SQ_WAIT_INST_ANY') / wc:.0f} %, waiting (waitcnt/barrier) {100 * v('SQ_WAIT_ANY') / wc:.0f} %"
                     " of SQ_WAVE_CYCLES")
    if v("SQ_LDS_BANK_CONFLICT") is not None and v("SQ_LDS_IDX_ACTIVE"):
        lines.append(f"LDS bank conflicts SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE          "
                     f"{100 * v('SQ_LDS_BANK_CONFLICT') / v('SQ_LDS_IDX_ACTIVE'):.1f} %")
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def short_kernel_name(name: str) -> str:
    """'void ssa::(anonymous namespace)::k<128, 128, false, 2, __bf16>(ssa::P)' -> 'k<128, 128, false, 2, __bf16>'."""
    # the profiler's own demangler prints the leading template arguments <__bf16, true, ...> of the
    # dense-layer instantiation as <bool _Accum, bool, E, ...>
    name = name.replace("<bool _Accum, bool, E", "<__bf16, true")
    n = name.replace("void ", "").replace("ssa::(anonymous namespace)::", "").replace("ssa::", "")
    depth = 0
    for i, ch in enumerate(n):  # cut at the argument list (the first '(' outside template brackets)
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i]
    return n


def write_trace_summary(stats_csv: str, out_path: str, command: str):
    """Short text summary of a rocprofv3 --kernel-trace --stats run: this library's kernels,
    one line per (kernel, workgroup count) -- the same kernel serves rows of different sizes -- with calls and
    average / min / max duration, from the per-dispatch kernel_trace.csv beside kernel_stats.csv."""
    import csv
    import shutil
    import subprocess

    def demangle(n):
        if n.startswith("_Z") and shutil.which("c++filt"):
            # this c++filt predates the mangling of __bf16 (DF16b): spell it as a
            # placeholder class name, then put it back
            out = subprocess.run(["c++filt", n.replace("DF16b", "9BFLOAT16x")], capture_output=True,
                                 text=True).stdout.strip()
            if out and not out.startswith("_Z"):
                return out.replace("BFLOAT16x", "__bf16")
        return n

    trace_csv = stats_csv.replace("kernel_stats.csv", "kernel_trace.csv")
    groups = {}
    for r in csv.DictReader(open(trace_csv)):
        n = demangle(r["Kernel_Name"])
        if "ssa::" not in n:
            continue
        wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
        nwg = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) // max(wg, 1)
        dt = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault((short_kernel_name(n), nwg, wg), []).append(dt)
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))
    w = max([len(k[0]) for k, _ in rows] + [6])
    lines = ["# rocprofv3 kernel-trace summary (this library's kernels; one line per kernel and grid; microseconds)",
             f"# command: {command}",
             f"{'kernel':{w}s} {'workgroups':>10s} {'wg_size':>7s} {'calls':>6s} {'avg_us':>11s} {'min_us':>11s} "
             f"{'max_us':>11s}"]
    lines += [f"{k:{w}s} {nwg:10d} {wg:7d} {len(v):6d} {sum(v) / len(v):11.1f} {min(v):11.1f} {max(v):11.1f}"
              for (k, nwg, wg), v in rows]
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def zigzag(dev, ssa, torch):
    """Layer-stack timing (timing only, synthetic weights): a decoder layer =
    QKV projection, attention, output projection with residual, SwiGLU MLP with
    residual (hidden 2048 = 16 heads x 128, MLP 5632; norms left out), its
    attention either dense causal or SSA.  LoZA keeps half the layers dense
    and makes the other half SSA, alternating (the ZigZag layout, "LoZA:
    ZigZag sparse attention" page / QbitAI report), so a 50/50 stack costs
    (t_dense + t_ssa) per layer pair against 2 t_dense for the all-dense model."""
    H, D, FFN = 16, 128, 5632
    hid = H * D
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    mk = lambda *shape: (torch.randn(*shape, device=dev, generator=g, dtype=torch.float32) * 0.02).to(torch.bfloat16)
    w_qkv, w_o, w_13, w_2 = mk(hid, 3 * hid), mk(hid, hid), mk(hid, 2 * FFN), mk(FFN, hid)
    res = {}
    for L in (131072, 262144):
        x0 = mk(L, hid)
        o = torch.empty((1, L, H, D), dtype=torch.bfloat16, device=dev)
        idx, cnt = ssa.block_index(L // 128, device=dev)
        lists = ssa.lists_from_index(idx, cnt)

        def layer(x, dense):
            qkv = x @ w_qkv
            q, k, v = (qkv[:, i * hid:(i + 1) * hid].view(1, L, H, D) for i in range(3))
            if dense:
                ssa.dense_causal(q, k, v, out=o)
            else:
                ssa.prefill(q, k, v, lists, out=o)
            x = x + o.view(L, hid) @ w_o
            h = x @ w_13
            return x + (torch.nn.functional.silu(h[:, :FFN]) * h[:, FFN:]) @ w_2

        times = {}
        for dense in (False, True):
            layer(x0, dense)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 2
            e0.record()
            for _ in range(reps):
                layer(x0, dense)
            e1.record()
            torch.cuda.synchronize()
            times["dense" if dense else "ssa"] = e0.elapsed_time(e1) / reps
        td, ts = times["dense"], times["ssa"]
        res[f"L{L}"] = {"dense_layer_ms": td, "ssa_layer_ms": ts, "layer_ratio": td / ts,
                        "zigzag_50_50_prefill_speedup": 2 * td / (td + ts)}
        print(f"[zigzag] L={L}: dense layer {td:.1f} ms, SSA layer {ts:.2f} ms, "
              f"50/50 stack vs all-dense: {2 * td / (td + ts):.2f}x", flush=True)
        del x0, o
        torch.cuda.empty_cache()
    # decode side: the a3 batch (64 sequences at ~U[64K, 128K]) one token per sequence; the
    # dense layer reads every cached key (ssa_decode_dense), the SSA layer its window
    # (ssa_decode); the cache contents do not change the time (left uninitialised)
    B3 = W3["B"]
    lens = synth.decode_seq_lens(W3["seed"], B3, W3["lo"], W3["hi"])
    bt, P = synth.decode_block_table(W3["seed"], lens, 128)
    kp = torch.empty((P, H, 128, D), dtype=torch.bfloat16, device=dev)
    vp = torch.empty_like(kp)
    btd, sl = torch.from_numpy(bt).to(dev), torch.from_numpy(lens).to(dev)
    od = torch.empty((B3, H, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((ssa.decode_workspace_size(B3, H, D, D) + 256,), dtype=torch.uint8, device=dev)
    x0 = mk(B3, hid)

    def dlayer(x, dense):
        qkv = x @ w_qkv
        q = qkv[:, :hid].view(B3, H, D)
        if dense:
            ssa.decode_dense(q, kp, vp, btd, sl, out=od)
        else:
            ssa.decode(q, kp, vp, btd, sl, out=od)
        x = x + od.view(B3, hid) @ w_o
        h = x @ w_13
        return x + (torch.nn.functional.silu(h[:, :FFN]) * h[:, FFN:]) @ w_2

    dt = {}
    for dense in (False, True):
        dlayer(x0, dense)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            dlayer(x0, dense)
        e1.record()
        torch.cuda.synchronize()
        dt["dense" if dense else "ssa"] = e0.elapsed_time(e1) / reps
    td, ts = dt["dense"], dt["ssa"]
    dec = {"batch": B3, "mean_context": float(np.mean(lens)), "dense_layer_ms": td, "ssa_layer_ms": ts,
           "layer_ratio": td / ts, "zigzag_50_50_decode_speedup": 2 * td / (td + ts)}
    print(f"[zigzag] decode batch {B3} at mean context {np.mean(lens):.0f}: dense layer {td:.3f} ms, "
          f"SSA layer {ts:.3f} ms, 50/50 stack vs all-dense: {2 * td / (td + ts):.2f}x", flush=True)
    print(json.dumps({"zigzag_prefill": res, "zigzag_decode": dec,
                      "layer": {"hidden": hid, "heads": H, "head_dim": D, "mlp": FFN, "dtype": "bf16",
                                "weights": "synthetic N(0, 0.02^2)"}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotations", type=int, default=2, help="independent decode page sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=25.0)
    ap.add_argument("--only", default="", help="comma list of rows to run (prefill,decode,dense,page,mla,chunk,bwd,hi); "
                    "for profiling one kernel -- the JSON line is printed only for a full run")
    ap.add_argument("--write-traffic", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"),
                    help="summarise two rocprofv3 --pmc runs into a traffic file and exit")
    ap.add_argument("--write-counters", nargs=5, metavar=("PMC_ROOT", "KERNEL_FRAGMENTS", "OUT", "TITLE", "COMMAND"),
                    help="summarise the COUNTER_GROUPS rocprofv3 passes for one kernel into a text file and exit")
    ap.add_argument("--counter-groups", action="store_true", help="print the counter groups, one per line, and exit")
    ap.add_argument("--zigzag", action="store_true", help="f4: dense/SSA layer-stack prefill timing and exit")
    ap.add_argument("--trace-summary", nargs=3, metavar=("KERNEL_STATS_CSV", "OUT", "COMMAND"),
                    help="summarise a rocprofv3 --kernel-trace --stats run into a short text file and exit")
    args = ap.parse_args()
    if args.trace_summary:
        write_trace_summary(*args.trace_summary)
        return
    if args.counter_groups:
        print("\n".join(COUNTER_GROUPS))
        return
    if args.write_counters:
        write_counters(*args.write_counters)
        return
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only; --gpus {args.gpus} is not supported "
              "(every row of the path fits one MI355X)", file=sys.stderr)
        sys.exit(2)

    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_budget)
    if cpu:
        print(f"[bench] cpu baseline: {cpu['value']:.4f} TFLOP/s ({cpu['sample']})", flush=True)
    cpu_rows = None if args.no_cpu_baseline else cpu_rows_baseline()
    if cpu_rows:
        for name, r in cpu_rows.items():
            print(f"[bench] cpu baseline {name:20s} {r['value']:10.4f} {r['unit']:8s} ({r['seconds']:.1f} s: {r['sample']})",
                  flush=True)

    import torch
    import long_context_block_ssa_amd as ssa

    ssa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.zigzag:
        zigzag(dev, ssa, torch)
        return

    def up(bits, head_major=True):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
        if head_major:  # [B, H, L, D] in memory, logical [B, L, H, D] view
            return t.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)
        return t.to(dev)

    only = set(x for x in args.only.split(",") if x)
    run = {name: (not only) or (name in only) for name in ("prefill", "decode", "dense", "page", "mla", "chunk", "bwd",
                                                          "hi")}
    run["page"] = run["page"] or run["hi"]  # the token stage starts from the page lists
    run["copy"] = "copy" in only  # calibration copy for the traffic counters, only on request

    print("[bench] generating inputs", flush=True)
    # a2 / a5 inputs
    L2, H2, D2, s2 = W2["L"], W2["H"], W2["D"], W2["seed"]
    nqb2 = L2 // 128
    if run["prefill"] or run["dense"] or run["bwd"]:
        q2, k2, v2 = (up(synth.seq_tensor(s2, t, 1, L2, H2, D2)) for t in (synth.Q, synth.K, synth.V))
        o2 = torch.empty((1, H2, L2, D2), dtype=torch.bfloat16, device=dev).permute(0, 2, 1, 3)
        od = torch.empty_like(o2)
    # a2 fp32 inputs (the small case: one head, d = 64, L = 2048)
    L1, H1, D1, s1 = W1["L"], W1["H"], W1["D"], W1["seed"]
    if run["prefill"]:
        q1, k1, v1 = (torch.from_numpy(np.ascontiguousarray(synth.seq_tensor(s1, t, 1, L1, H1, D1, "f32"))).to(dev)
                      for t in (synth.Q, synth.K, synth.V))
        o1 = torch.empty_like(q1)
        win1 = ssa.block_index(L1 // 128, device=dev)
        lists1 = ssa.lists_from_index(*win1)
    # a3 inputs: one paged pool, several independent (q, table) sets
    B3, H3, D3, s3 = W3["B"], W3["H"], W3["D"], W3["seed"]
    Hkv3g = W3["Hkv_gqa"]
    lens = synth.decode_seq_lens(s3, B3, W3["lo"], W3["hi"])
    if run["decode"]:
        tables = []
        P = None
        for r in range(args.rotations):
            bt, P = synth.decode_block_table(s3, lens, 128, rotation=r)
            tables.append(bt)
        kp = torch.full((P, H3, 128, D3), float("nan"), dtype=torch.bfloat16, device=dev)
        vp = torch.full((P, H3, 128, D3), float("nan"), dtype=torch.bfloat16, device=dev)
        fill = synth.decode_fill_blocks(lens, 128, 1, 7)
        for r, bt in enumerate(tables):
            ids, kh, vh = [], [], []
            for b, blocks in enumerate(fill):
                for t in blocks:
                    ids.append(int(bt[b, t]))
                    kh.append(synth.page_chunk(s3 + 100 * r, synth.K, b, t, H3, D3))
                    vh.append(synth.page_chunk(s3 + 100 * r, synth.V, b, t, H3, D3))
            idx_t = torch.tensor(ids, dtype=torch.long, device=dev)
            kp[idx_t] = up(np.stack(kh), head_major=False)
            vp[idx_t] = up(np.stack(vh), head_major=False)
        q3 = [up(synth.decode_query(s3, B3, H3, D3, rotation=r)[None], head_major=False)[0]
              for r in range(args.rotations)]
        bts = [torch.from_numpy(bt).to(dev) for bt in tables]
        sl3 = torch.from_numpy(lens).to(dev)
        o3 = torch.empty((B3, H3, D3), dtype=torch.bfloat16, device=dev)
        # grouped heads: the same 16 query heads on the first Hkv3g kv heads of the pool
        kp3g, vp3g = kp[:, :Hkv3g], vp[:, :Hkv3g]
        o3g = torch.empty((B3, H3, D3), dtype=torch.bfloat16, device=dev)
    # a6-a8 inputs
    if run["page"]:
        L5, H5, D5, M5, s5 = W5["L"], W5["H"], W5["D"], W5["M"], W5["seed"]
        q5, k5, v5 = (up(synth.seq_tensor(s5, t, 1, L5, H5, D5)) for t in (synth.Q, synth.K, synth.V))
        o5 = torch.empty((1, H5, L5, D5), dtype=torch.bfloat16, device=dev).permute(0, 2, 1, 3)
        nqb5 = L5 // 128
        idx5 = torch.empty((1, H5, nqb5, 8 + M5), dtype=torch.int32, device=dev)
        cnt5 = torch.empty((1, H5, nqb5), dtype=torch.int32, device=dev)
        ws5 = torch.empty((ssa.page_select_workspace_size(q5, k5) + 256,), dtype=torch.uint8, device=dev)
    if run["hi"]:  # f2: the window's blocks plus K tokens of the recalled pages
        K5 = W5["K"]
        win5 = ssa.block_index(nqb5, device=dev)  # held: the lists point into these tensors
        lists5w = ssa.lists_from_index(*win5)
        wst5 = torch.empty((ssa.token_select_workspace_size(q5, k5, M5) + 256,), dtype=torch.uint8, device=dev)
        o5h = torch.empty((1, H5, L5, D5), dtype=torch.bfloat16, device=dev).permute(0, 2, 1, 3)
    # a4 inputs: values N(0,1)/24, drawn on the device (the query is 38.6 GB)
    if run["mla"]:
        L4, H4, DQ4, DV4, s4 = W4["L"], W4["H"], W4["DQK"], W4["DV"], W4["seed"]
        q4 = synth.torch_normal_bf16(1000 * s4 + 1, (1, L4, H4, DQ4), 1 / 24, device=dev)
        c4 = synth.torch_normal_bf16(1000 * s4 + 2, (1, L4, 1, DQ4), 1 / 24, device=dev)
        o4 = torch.empty((1, L4, H4, DV4), dtype=torch.bfloat16, device=dev)
        B4d, n4d, R4 = W4["dec_B"], W4["dec_n"], W4["dec_rot"]
        lens4 = np.full(B4d, n4d, np.int32)
        nb4 = n4d // 128
        # R4 tables over one pool; each table's window pages are distinct from the others'
        P4 = B4d * nb4
        pool4 = torch.full((P4, 1, 128, DQ4), float("nan"), dtype=torch.bfloat16, device=dev)
        tables4 = []
        for r in range(R4):
            bt4, _ = synth.decode_block_table(s4, lens4, 128, rotation=r)
            tables4.append(bt4)
        win_ids = sorted({int(bt[b, t]) for bt in tables4 for b in range(B4d) for t in [0] + list(range(nb4 - 7, nb4))})
        pool4[torch.tensor(win_ids, dtype=torch.long, device=dev)] = synth.torch_normal_bf16(
            1000 * s4 + 3, (len(win_ids), 1, 128, DQ4), 1 / 24, device=dev)
        q4d = [synth.torch_normal_bf16(1000 * s4 + 10 + r, (B4d, H4, DQ4), 1 / 24, device=dev) for r in range(R4)]
        bts4 = [torch.from_numpy(bt).to(dev) for bt in tables4]
        sl4 = torch.from_numpy(lens4).to(dev)
        o4d = torch.empty((B4d, H4, DV4), dtype=torch.bfloat16, device=dev)
        ws4 = torch.empty((ssa.decode_workspace_size(B4d, H4, DQ4, DV4) + 256,), dtype=torch.uint8, device=dev)
    # f1 inputs: a compact pool holding only the pages the chunks read (block 0
    # and the blocks from 6 before the chunk's first block to the end)
    if run["chunk"]:
        B6, T6, H6, D6, s6 = W6["B"], W6["T"], W6["H"], W6["D"], W6["seed"]
        lens6 = synth.decode_seq_lens(s6, B6, W6["lo"], W6["hi"])
        nblk6 = (lens6 + 127) // 128
        bt6 = np.full((B6, int(nblk6.max())), -1, np.int32)
        kh, vh = [], []
        for b in range(B6):
            need = sorted({0} | set(range(max(0, (int(lens6[b]) - T6) // 128 - 6), int(nblk6[b]))))
            for t in need:
                bt6[b, t] = len(kh)
                kh.append(synth.page_chunk(s6, synth.K, b, t, H6, D6))
                vh.append(synth.page_chunk(s6, synth.V, b, t, H6, D6))
        kp6, vp6 = up(np.stack(kh), head_major=False), up(np.stack(vh), head_major=False)
        q6 = up(synth.seq_tensor(s6, synth.Q, B6, T6, H6, D6), head_major=False)
        o6 = torch.empty((B6, T6, H6, D6), dtype=torch.bfloat16, device=dev)
        bt6d, sl6 = torch.from_numpy(bt6).to(dev), torch.from_numpy(lens6).to(dev)
        idx6, cnt6 = ssa.block_index(bt6.shape[1], device=dev)
        lists6 = ssa.lists_from_index(idx6, cnt6)
    # f3 inputs: the a2 forward's output and lse, an incoming gradient
    if run["bwd"]:
        win2 = ssa.block_index(nqb2, device=dev)
        lists2 = ssa.lists_from_index(*win2)
        ob, lseb = ssa.prefill(q2, k2, v2, lists2, with_lse=True)
        gb = up(synth.seq_tensor(s2, 90, 1, L2, H2, D2))
        dqb, dkb, dvb = (torch.empty((1, H2, L2, D2), dtype=torch.bfloat16, device=dev).permute(0, 2, 1, 3)
                         for _ in range(3))
        wsb = torch.empty((ssa.prefill_backward_workspace_size(q2, k2) + 256,), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    rows = ["a1 block_index", "a2 ssa_prefill", "a3 ssa_decode", "a5 dense_causal", "a6 page_sums", "a7 page_top_m",
            "a8 page_prefill", "a4 mla_prefill", "a4 mla_decode", "f1 chunk_prefill", "f3 ssa_backward",
            "f2 token_select", "f2 hi_prefill", "a2 ssa_prefill_f32", "a3 ssa_decode_gqa"]
    nev = len(rows) + 1

    if run["copy"]:
        cp_src = torch.ones((1 << 29,), dtype=torch.bfloat16, device=dev)
        cp_dst = torch.empty_like(cp_src)

    def step(s, ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        idx2, cnt2 = ssa.block_index(nqb2, device=dev)
        mark(1)
        if run["prefill"]:
            ssa.prefill(q2, k2, v2, ssa.lists_from_index(idx2, cnt2), out=o2)
        mark(2)
        r = s % args.rotations
        if run["decode"]:
            ssa.decode(q3[r], kp, vp, bts[r], sl3, out=o3)
        mark(3)
        if run["dense"]:
            ssa.dense_causal(q2, k2, v2, out=od)
        mark(4)
        if run["page"]:  # a6 then a7: ssa_page_select in its two phases, timed apart
            ssa.page_block_sums(q5, k5, ws5)
        mark(5)
        if run["page"]:
            i5, c5 = ssa.page_select_top(q5, k5, ws5, top_m=M5)
        mark(6)
        if run["page"]:
            ssa.prefill(q5, k5, v5, ssa.lists_per_head(i5, c5), out=o5)
        mark(7)
        if run["mla"]:
            win4 = ssa.block_index(L4 // 128, device=dev)
            ssa.prefill(q4, c4, c4[..., :DV4], ssa.lists_from_index(*win4),
                        scale=1 / 24, out=o4)
        mark(8)
        if run["mla"]:
            r4 = s % R4
            ssa.decode(q4d[r4], pool4, pool4[..., :DV4], bts4[r4], sl4, scale=1 / 24, out=o4d, workspace=ws4)
        mark(9)
        if run["chunk"]:
            ssa.prefill_chunk(q6, kp6, vp6, bt6d, sl6, lists6, out=o6)
        mark(10)
        if run["bwd"]:
            ssa.prefill_backward(q2, k2, v2, ob, gb, lseb, dq=dqb, dk=dkb, dv=dvb, workspace=wsb)
        mark(11)
        if run["hi"]:
            t5, tc5 = ssa.token_select(q5, k5, i5, c5, ws5, top_m=M5, top_k=K5, workspace=wst5)
        mark(12)
        if run["hi"]:
            ssa.prefill_tokens(q5, k5, v5, lists5w, ssa.token_lists(t5, tc5), out=o5h)
        mark(13)
        if run["prefill"]:
            ssa.prefill(q1, k1, v1, lists1, out=o1)
        mark(14)
        if run["decode"]:
            ssa.decode(q3[r], kp3g, vp3g, bts[r], sl3, out=o3g)
        mark(15)
        if run["copy"]:
            cp_dst.copy_(cp_src)

    print("[bench] warmup", flush=True)
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    try:
        evs = [[TimingEvent() for _ in range(nev)] for _ in range(args.steps)]
        timing = "HIP timing events (hipEventDisableSystemFence)"
    except (OSError, RuntimeError, AttributeError) as exc:  # keep measuring with torch's events
        print(f"[bench] timing events unavailable ({exc}); torch events instead", flush=True)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
        timing = "torch events"
    print("[bench] timing", flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(s, evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_row = [float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)])) for i in range(len(rows))]
    ms_step = wall * 1e3 / args.steps
    for name, ms in zip(rows, per_row):
        print(f"[bench] {name:22s} {ms * 1e3:10.1f} us", flush=True)

    if only:
        return
    for t, name in ((o1, "ssa f32"), (o2, "ssa"), (o3, "decode"), (o3g, "decode gqa"), (od, "dense"), (o5, "page"), (o4[0, -128:], "mla"),
                    (o4d, "mla decode"), (o6, "chunk"), (dqb, "dq"), (dkb, "dk"), (dvb, "dv"), (o5h, "hi")):
        if not torch.isfinite(t.float()).all():
            raise RuntimeError(f"non-finite {name} output")

    T = dict(zip(rows, per_row))
    T["a6-a7"] = T["a6 page_sums"] + T["a7 page_top_m"]  # one ssa_page_select
    f1 = ssa_flops(L1, H1, D1)
    t1 = T["a2 ssa_prefill_f32"] * 1e-3
    f2 = ssa_flops(L2, H2, D2)
    t2 = T["a2 ssa_prefill"] * 1e-3
    tf2 = f2 / t2 / 1e12
    b3 = decode_bytes(lens, H3, H3, D3, D3)
    t3 = T["a3 ssa_decode"] * 1e-3
    gb3 = b3 / t3 / 1e9
    b3g = decode_bytes(lens, H3, Hkv3g, D3, D3)
    t3g = T["a3 ssa_decode_gqa"] * 1e-3
    gb3g = b3g / t3g / 1e9
    fd = dense_flops(L2, H2, D2)
    f5 = page_flops(L5, H5, D5, M5)
    b5 = 2 * L5 * H5 * D5 * 2
    # block sums: q and k read (bf16), their fp64 sums written; scores: 2*D fp64
    # flops per (query block, candidate page) pair of every head
    b5s = b5 + 2 * H5 * nqb5 * D5 * 8
    f5s = 2 * D5 * H5 * sum(max(qb - 7, 0) for qb in range(nqb5))
    kernels = {
        "ssa_prefill": {"bound": "mfma", "achieved": tf2, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": tf2 / PEAK_BF16_TFLOPS, "traffic": traffic_for("ssa_prefill"),
                        "us": T["a2 ssa_prefill"] * 1e3, "work": f2},
        "ssa_decode": {"bound": "hbm", "achieved": gb3, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                       "frac": gb3 / PEAK_HBM_GBS, "traffic": traffic_for("ssa_decode"),
                       "us": T["a3 ssa_decode"] * 1e3, "work": b3},
        "ssa_decode_gqa": {"bound": "hbm", "achieved": gb3g, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": gb3g / PEAK_HBM_GBS, "traffic": traffic_for("ssa_decode_gqa"),
                           "us": T["a3 ssa_decode_gqa"] * 1e3, "work": b3g, "heads": f"{H3}/{Hkv3g}"},
        "dense_causal": {"bound": "mfma", "achieved": fd / (T["a5 dense_causal"] * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": fd / (T["a5 dense_causal"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                         "us": T["a5 dense_causal"] * 1e3, "work": fd},
        # a6: an HBM scan (q and k read once, fp64 block sums written)
        "page_sums": {"bound": "hbm", "achieved": b5s / (T["a6 page_sums"] * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                      "unit": "GB/s", "frac": b5s / (T["a6 page_sums"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      "us": T["a6 page_sums"] * 1e3, "work": b5s},
        # a7: fp64 scores of every (query block, candidate page) pair, then the top-M lists
        "page_top_m": {"bound": "mfma_fp64", "achieved": f5s / (T["a7 page_top_m"] * 1e-3) / 1e12,
                       "peak": PEAK_FP64_TFLOPS, "unit": "TFLOP/s",
                       "frac": f5s / (T["a7 page_top_m"] * 1e-3) / 1e12 / PEAK_FP64_TFLOPS,
                       "us": T["a7 page_top_m"] * 1e3, "work": f5s},
        "page_select": {"us": T["a6-a7"] * 1e3},
        "page_prefill": {"bound": "mfma", "achieved": f5 / (T["a8 page_prefill"] * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": f5 / (T["a8 page_prefill"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                         "us": T["a8 page_prefill"] * 1e3, "work": f5},
        "block_index": {"us": T["a1 block_index"] * 1e3},
        # the small fp32 case: 16 query blocks cannot fill 256 CUs; its time is
        # the latency of one tile, reported against the fp32 MFMA peak
        "ssa_prefill_f32": {"bound": "latency", "achieved": f1 / t1 / 1e12, "peak": PEAK_FP32_TFLOPS,
                            "unit": "TFLOP/s", "frac": f1 / t1 / 1e12 / PEAK_FP32_TFLOPS, "us": T["a2 ssa_prefill_f32"] * 1e3,
                            "work": f1, "tokens_per_s": L1 / t1},
    }
    f4 = mla_flops(L4, H4, DQ4, DV4)
    b4 = mla_decode_bytes(lens4, H4, DQ4, DV4)
    kernels["mla_prefill"] = {"bound": "mfma", "achieved": f4 / (T["a4 mla_prefill"] * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": f4 / (T["a4 mla_prefill"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                              "traffic": traffic_for("mla_prefill"), "us": T["a4 mla_prefill"] * 1e3, "work": f4}
    kernels["mla_decode"] = {"bound": "hbm", "achieved": b4 / (T["a4 mla_decode"] * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": b4 / (T["a4 mla_decode"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                             "traffic": traffic_for("mla_decode"), "us": T["a4 mla_decode"] * 1e3, "work": b4}
    f6 = chunk_flops(lens6, T6, H6, D6)
    kernels["chunk_prefill"] = {"bound": "mfma", "achieved": f6 / (T["f1 chunk_prefill"] * 1e-3) / 1e12,
                                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                "frac": f6 / (T["f1 chunk_prefill"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                "us": T["f1 chunk_prefill"] * 1e3, "work": f6}
    fb = bwd_flops(L2, H2, D2)
    kernels["ssa_backward"] = {"bound": "mfma", "achieved": fb / (T["f3 ssa_backward"] * 1e-3) / 1e12,
                               "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                               "frac": fb / (T["f3 ssa_backward"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                               "us": T["f3 ssa_backward"] * 1e3, "work": fb}
    fh = hi_flops(L5, H5, D5, M5, K5)
    # the second stage scores every recalled token: D fp64 FMAs on a key row
    # (2D bytes, re-read from cache by neighbouring query blocks) per candidate
    cand5 = H5 * sum(128 * min(M5, max(qb - 7, 0)) for qb in range(nqb5) if 128 * min(M5, max(qb - 7, 0)) > K5)
    kernels["token_select"] = {"us": T["f2 token_select"] * 1e3, "candidates": cand5,
                               "candidate_rows_per_s": cand5 / (T["f2 token_select"] * 1e-3),
                               "fp64_gflops": 2 * D5 * cand5 / (T["f2 token_select"] * 1e-3) / 1e9}
    kernels["hi_prefill"] = {"bound": "mfma", "achieved": fh / (T["f2 hi_prefill"] * 1e-3) / 1e12,
                             "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                             "frac": fh / (T["f2 hi_prefill"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                             "us": T["f2 hi_prefill"] * 1e3, "work": fh}
    out = {
        "metric": "SSA prefill TFLOP/s (frac MFMA peak) + decode GB/s (frac HBM) at 128K ctx",
        "value": tf2,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "SSA prefill B=1 H=16 d=128 L=32768 bf16 (value) + SSA decode batch 64 H=16/16 d=128 "
                        "ctx U[65536,131072] bf16 (decode) + dense causal (same shape) + page selection "
                        "L=131072 H=16 d=128 M=8 + latent-shared 576/512 x 128 heads: prefill L=262144, "
                        "decode batch 8 at 1048576 + chunked prefill of the last 2048 tokens of 16 sequences "
                        "at ctx U[65536,131072] over a paged cache + SSA backward of the prefill workload + "
                        "hierarchical second stage (top-512 tokens of the 8 recalled pages) and attention over "
                        "window + tokens at the page-selection shape",
            "timing": timing,
            "prefill_tokens_per_s": L2 / t2,
            "decode_gbps": gb3,
            "decode_frac_hbm": gb3 / PEAK_HBM_GBS,
            "decode_tokens_per_s": B3 / t3,
            "decode_gqa_gbps": gb3g,
            "decode_gqa_frac_hbm": gb3g / PEAK_HBM_GBS,
            "page_select_index_share": T["a6-a7"] / (T["a6-a7"] + T["a8 page_prefill"]),
            "hi_index_share": (T["a6-a7"] + T["f2 token_select"]) / (T["a6-a7"] + T["f2 token_select"] + T["f2 hi_prefill"]),
        },
        "roofline": kernels["ssa_prefill"],
        "roofline_decode": kernels["ssa_decode"],
        "kernels": kernels,
        "cpu_baseline": cpu,
        "cpu_baseline_rows": cpu_rows,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
