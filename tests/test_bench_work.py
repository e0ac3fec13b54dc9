"""The benchmark's algorithmic work (the numerators of its rooflines), pinned
against independent counts: brute-force window membership on small lengths,
the closed forms of the window's pair totals, and the plain formulas of the
dense and decode cases.  Host logic only; no GPU."""
import subprocess
import sys

import pytest

import bench


def window_keys_brute(i: int, n_global: int = 1, n_local: int = 7, block: int = 128) -> int:
    """Keys j <= i whose block is global or among the n_local blocks ending at i's."""
    qb = i // block
    return sum(1 for j in range(i + 1) if j // block < n_global or qb - n_local < j // block <= qb)


@pytest.mark.parametrize("i", [0, 1, 127, 128, 500, 1023, 1024, 1025, 1151, 1152, 2047, 3000, 5000])
def test_keys_ssa_matches_brute_force(i):
    assert bench.keys_ssa(i) == window_keys_brute(i)


@pytest.mark.parametrize("i", [0, 2047, 2048, 2100, 4095, 6000])
def test_keys_page_matches_window_of_16_blocks(i):
    # the page-selected list holds 1 + 7 + M = 16 blocks once qb >= 16; until then every block
    qb = i // 128
    expect = i + 1 if qb < 16 else 15 * 128 + (i % 128) + 1
    assert bench.keys_page(i, 8) == expect


@pytest.mark.parametrize("L", [128, 1000, 1024, 2048, 32768])
def test_pairs_closed_form(L):
    got = bench.pairs(L, bench.keys_ssa)
    if L <= 1024:
        assert got == L * (L + 1) // 2
    else:
        assert L % 128 == 0
        assert 2 * got == 2 * 524800 + 1921 * (L - 1024)  # 524,800 + 960.5 (L - 1024)


def test_workload_totals():
    # SSA prefill at L = 32768, 16 heads, d = 128: 4 d flops per admitted pair
    assert bench.ssa_flops(32768, 16, 128) == 4 * 128 * 16 * (524800 + 1921 * (32768 - 1024) // 2)
    assert bench.ssa_flops(32768, 16, 128) == 254_074_159_104
    # the dense comparison layer: every causal pair
    assert bench.dense_flops(32768, 16, 128) == 4 * 128 * 16 * 32768 * 32769 // 2 == 4_398_180_728_832
    # page-selected attention over 16-block lists at L = 131072: 4,130,340,864 pairs over 16 heads
    assert bench.page_flops(131072, 16, 128, 8) == 4 * 128 * 4_130_340_864
    # latent-shared prefill: 2 (576 + 512) flops per pair, 128 heads, L = 262144 (~70.0 TFLOP)
    f = bench.mla_flops(262144, 128, 576, 512)
    assert f == 2 * 1088 * 128 * bench.pairs(262144, bench.keys_ssa)
    assert abs(f / 1e12 - 70.0) < 0.05
    # backward: five 2 d products per pair
    assert bench.bwd_flops(32768, 16, 128) * 4 == bench.ssa_flops(32768, 16, 128) * 10


def test_decode_bytes_brute_force():
    lens = [1, 128, 129, 1024, 1025, 70000]
    Hq, Hkv, D = 4, 2, 128
    kv = sum(window_keys_brute(n - 1) for n in lens[:5]) + bench.keys_ssa(70000 - 1)
    assert bench.keys_ssa(70000 - 1) == 896 + (70000 - 1) % 128 + 1
    assert bench.decode_bytes(lens, Hq, Hkv, D, D) == kv * Hkv * 2 * D * 2 + len(lens) * Hq * 2 * D * 2
    # the latent row (576 wide) is read once for key and value
    assert bench.mla_decode_bytes(lens, 128, 576, 512) == kv * 576 * 2 + len(lens) * 128 * 1088 * 2


@pytest.mark.parametrize("qb,expect", [(0, 0), (7, 0), (8, 128), (11, 512), (15, 512), (1000, 512)])
def test_hi_tokens(qb, expect):
    # recalled pages outside the window: min(M, qb - 7); 128 tokens each, at most K
    assert bench.hi_tokens(qb, 8, 512) == expect


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
