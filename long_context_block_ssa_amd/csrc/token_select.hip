// Second stage of hierarchical indexing, gfx950.
//
// The LongCat sparse attention article (section 3, hierarchical indexing)
// selects coarse-to-fine: the first stage recalls the top-M 128-token pages
// of a query block (page_select.hip), the second scores every token of those
// pages and keeps the top K.  The article leaves the token score to a
// trained indexer; here it is the first stage's score taken per token,
//      score(j) = < sum of q over query block qb , k_j >      (fp64),
// so one list serves the 128 queries of the block.  Candidates are the
// tokens of the listed pages that lie outside the window of qb (pages
// n_global .. qb - n_local); the window's pages are read whole by the
// attention anyway.
//
// One workgroup of 4 waves per (b, query head, query block):
//   1. wave 0 turns the page list into the ascending, duplicate-free list of
//      candidate pages (at most 32);
//   2. with at most K candidates every candidate token is kept;
//   3. otherwise each candidate key row is scored by D/8 lanes (16 bytes of
//      bf16 each, so a row is one contiguous read), fp64 products summed in a
//      fixed order (per lane over its 8 channels, then a butterfly across the
//      row's lanes);
//   4. the K-th largest score T is found exactly by a radix select over the
//      order-preserving 64-bit image of the fp64 scores, 8 bits per pass
//      (NaN counts as -inf, -0 as +0);
//   5. every score above T is kept, and of the scores equal to T the needed
//      number with the lowest candidate index (= lowest token); they are
//      written out in candidate order, so the output list is ascending.
#include "common.hpp"

namespace ssa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTsThreads = 256;
constexpr int kTsWaves = kTsThreads / 64;
constexpr int kMaxCandPages = 32;
constexpr int kMaxCand = kMaxCandPages * 128;

// order-preserving map of a score to an unsigned key (larger score -> larger
// key); -0 is folded onto +0 and NaN onto -inf
__device__ __forceinline__ uint64_t order_key(double x) {
  if (x == 0.0) x = 0.0;
  if (x != x) x = -__builtin_inf();
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = __shfl_xor(static_cast<int>(static_cast<uint32_t>(u)), m);
  const int hi = __shfl_xor(static_cast<int>(static_cast<uint32_t>(u >> 32)), m);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo));
}

// exclusive prefix sum of v over the workgroup (every thread calls it)
__device__ __forceinline__ int block_excl_scan(int v, int32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int at = x - v;
  for (int w = 0; w < wave; ++w) at += wsum[w];
  __syncthreads();  // wsum is reused by the next scan
  return at;
}

template <int D>
__global__ __launch_bounds__(kTsThreads) void token_select_kernel(TokenSelectParams p) {
  constexpr int LPR = D / 8;      // lanes per key row
  constexpr int RPW = 64 / LPR;   // rows per wave and load
  constexpr int U = 16;           // loads in flight per lane
  __shared__ uint64_t key[kMaxCand];
  __shared__ uint32_t hist[256];
  __shared__ int32_t pages[kMaxCandPages];
  __shared__ int32_t wsum[kTsWaves];
  __shared__ int32_t s_npg, s_need;
  __shared__ uint64_t s_prefix;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qb = static_cast<int>(blockIdx.x % static_cast<unsigned>(p.nqb));
  const int bh = static_cast<int>(blockIdx.x / static_cast<unsigned>(p.nqb));
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int hk = h / p.group;
  const int64_t row = static_cast<int64_t>(bh) * p.nqb + qb;
  const int32_t* prow = p.pidx + row * p.PW;
  int32_t* trow = p.tok + row * p.K;
  const int K = p.K;

  // ---- 1. candidate pages -------------------------------------------------
  if (wave == 0) {
    const int pc = min(max(p.pcnt[row], 0), p.PW);
    const int c = lane < pc ? prow[lane] : -1;
    bool ok = lane < pc && c >= p.n_global && c <= qb - p.n_local;
    for (int j = 0; j < pc; ++j) {  // a repeated page counts once (its first entry)
      const int cj = __builtin_amdgcn_readlane(c, j);
      if (j < lane && cj == c) ok = false;
    }
    const uint64_t okm = __builtin_amdgcn_ballot_w64(ok);
    int rank = 0;
    for (int j = 0; j < pc; ++j) {
      const int cj = __builtin_amdgcn_readlane(c, j);
      if (((okm >> j) & 1) && cj < c) ++rank;
    }
    if (ok && rank < kMaxCandPages) pages[rank] = c;
    if (lane == 0) s_npg = min(__popcll(okm), kMaxCandPages);
  }
  __syncthreads();
  const int npg = s_npg;
  const int C = npg * 128;

  // ---- 2. at most K candidates: all of them (K = 0: none) -----------------
  if (C <= K || K == 0) {
    for (int e = tid; e < K; e += kTsThreads) trow[e] = e < C ? pages[e >> 7] * 128 + (e & 127) : -1;
    if (tid == 0) p.tcnt[row] = min(C, K);
    return;
  }

  // ---- 3. scores ------------------------------------------------------------
  const double* qs = p.qsum + row * D;
  const int cl = lane % LPR, rl = lane / LPR;
  double qv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qv[i] = qs[cl * 8 + i];
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + b * p.ks_b + hk * p.ks_h + cl * 8;
  constexpr int kChunk = RPW * U;            // rows of one wave's pass (64 or 128)
  constexpr int kStep = kTsWaves * kChunk;
  for (int r0 = wave * kChunk; r0 < C; r0 += kStep) {
    // C is a multiple of 128, so a chunk is wholly inside or outside
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * RPW + rl;
      const int t = pages[r >> 7] * 128 + (r & 127);
      v[u] = *reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(t) * p.ks_l);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      double acc = 0.0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc = __builtin_fma(qv[2 * w], static_cast<double>(__builtin_bit_cast(float, v[u][w] << 16)), acc);
        acc = __builtin_fma(qv[2 * w + 1], static_cast<double>(__builtin_bit_cast(float, v[u][w] & 0xFFFF0000u)), acc);
      }
#pragma unroll
      for (int m = LPR / 2; m > 0; m >>= 1) acc += shfl_xor_f64(acc, m);
      if (cl == 0) key[r0 + u * RPW + rl] = order_key(acc);
    }
  }

  // ---- 4. the K-th largest key T, 8 bits at a time (radix select) ----------
  // invariant: `need` keys are still to be chosen among those whose leading
  // bits equal `prefix`, and at least that many exist
  uint64_t prefix = 0;
  int need = K;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    hist[tid] = 0;  // 256 threads, 256 bins
    __syncthreads();
    for (int r = tid; r < C; r += kTsThreads) {
      const uint64_t kk = key[r];
      if (pass == 0 || (kk >> (shift + 8)) == prefix) atomicAdd(&hist[(kk >> shift) & 255], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // bins in descending order, 4 per lane
      uint32_t c[4], tot = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = hist[255 - 4 * lane - q];
        tot += c[q];
      }
      uint32_t incl = tot;
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      uint32_t run = incl - tot;  // keys in higher bins
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (run < static_cast<uint32_t>(need) && run + c[q] >= static_cast<uint32_t>(need)) {
          s_prefix = (prefix << 8) | static_cast<uint64_t>(255 - 4 * lane - q);
          s_need = need - static_cast<int>(run);
        }
        run += c[q];
      }
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
  }
  // every key above T is chosen, and of the keys equal to T the `need` with
  // the lowest candidate index (= lowest token)
  const uint64_t T = prefix;

  // ---- 5. the chosen tokens in candidate order ------------------------------
  const int per = (C + kTsThreads - 1) / kTsThreads;
  const int e0 = min(tid * per, C), e1 = min(e0 + per, C);
  int eq = 0;
  for (int e = e0; e < e1; ++e) eq += key[e] == T;
  int eq_before = block_excl_scan(eq, wsum);
  int mine = 0;
  for (int e = e0; e < e1; ++e) {
    const uint64_t kk = key[e];
    mine += kk > T || (kk == T && eq_before++ < need);
  }
  int at = block_excl_scan(mine, wsum);
  eq_before -= eq;  // back to the range start
  for (int e = e0; e < e1; ++e) {
    const uint64_t kk = key[e];
    if (kk > T || (kk == T && eq_before++ < need)) trow[at++] = pages[e >> 7] * 128 + (e & 127);
  }
  if (tid == 0) p.tcnt[row] = K;
}

}  // namespace

hipError_t launch_token_select(const TokenSelectParams& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(p.B) * p.Hq * p.nqb));
  if (p.D == 128) return launch_kernel(token_select_kernel<128>, grid, dim3(kTsThreads), 0, stream, p);
  if (p.D == 64) return launch_kernel(token_select_kernel<64>, grid, dim3(kTsThreads), 0, stream, p);
  return hipErrorNotSupported;
}

}  // namespace ssa
