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
// Page-major: a page is recalled by several query blocks (about M of them
// on average), so scoring row by row would gather each recalled page once
// per recalling block.  Instead the work is turned around:
//   0. zero the per-page recall counters;
//   1. rows: one wave per (b, head, query block) turns the page list into
//      the ascending, duplicate-free candidate pages (at most top_m); a row
//      with at most K candidate tokens (or K = 0) is written out here, the
//      others count themselves into their pages' recall counters;
//   2. offsets: one workgroup per (b, head) scans the counters into bucket
//      offsets;
//   3. fill: each open row appends (row, slot) to its pages' buckets (the
//      order inside a bucket is free: every entry has its own output place);
//   4. score: one workgroup per (b, head, page) loads the page's 128 key
//      rows once into registers and multiplies the query-block sums of up to
//      16 recalling rows at a time against them on the fp64 matrix cores
//      (the key rows stay bf16 in registers and are widened per step),
//      writing order-preserving 64-bit keys (NaN counts as -inf, -0 as +0)
//      into each recalling row's slot;
//   5. select: one wave per open row finds the K-th largest key T exactly
//      by a radix select (LDS histograms, 8 bits a pass; once at most 64
//      keys share the leading bits found so far, they are ranked by
//      counting), keeps every key
//      above T and, of the keys equal to T, the needed number with the lowest
//      candidate index (= lowest token), and writes them in candidate order,
//      so the list comes out ascending.
// Each recalled page is read once per query head, instead of once per
// recalling query block.
#include "common.hpp"

namespace ssa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kTsThreads = 256;
constexpr int kTsWaves = kTsThreads / 64;
constexpr int kMaxSlots = 32;
constexpr int kEnt = 16;  // recalling rows staged per round of the score kernel
static_assert(kTsThreads / 16 == kEnt, "the score kernel stages one recalling row per 16 threads");

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

__global__ __launch_bounds__(kTsThreads) void ts_zero_kernel(int32_t* cnt, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kTsThreads + threadIdx.x;
  if (i < n) cnt[i] = 0;
}

// 1. one wave per row (b, h, qb)
__global__ __launch_bounds__(kTsThreads) void ts_rows_kernel(TokenSelectParams p) {
  __shared__ int32_t spg[kTsWaves][kMaxSlots];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t R = static_cast<int64_t>(p.B) * p.Hq * p.nqb;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kTsWaves + wave;
  if (row >= R) return;  // whole waves
  const int qb = static_cast<int>(row % p.nqb);
  const int64_t bh = row / p.nqb;
  const int32_t* prow = p.pidx + row * p.PW;
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
  const int npg = min(static_cast<int>(__popcll(okm)), p.S);  // the lowest S candidate pages
  const bool keep = ok && rank < npg;
  if (keep) {
    spg[wave][rank] = c;
    p.pages[row * p.S + rank] = c;
  }
  const int C = npg * 128, K = p.K;
  if (C <= K || K == 0) {  // every candidate (or none): final here
    int32_t* trow = p.tok + row * K;
    for (int e = lane; e < K; e += 64) trow[e] = e < C ? spg[wave][e >> 7] * 128 + (e & 127) : -1;
    if (lane == 0) {
      p.tcnt[row] = min(C, K);
      p.npg[row] = 0;
    }
    return;
  }
  if (lane == 0) p.npg[row] = npg;
  if (keep) atomicAdd(&p.cnt[bh * p.nqb + c], 1);
}

// 2. one workgroup per (b, h): bucket offsets of its pages; counters reset
// to serve as fill cursors
__global__ __launch_bounds__(kTsThreads) void ts_offsets_kernel(TokenSelectParams p) {
  __shared__ int32_t wsum[kTsWaves];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * p.nqb;
  int32_t* cnt = p.cnt + base;
  int32_t* off = p.off + base;
  const int per = (p.nqb + kTsThreads - 1) / kTsThreads;
  const int c0 = min(static_cast<int>(threadIdx.x) * per, p.nqb), c1 = min(c0 + per, p.nqb);
  int mine = 0;
  for (int c = c0; c < c1; ++c) mine += cnt[c];
  int at = block_excl_scan(mine, wsum);
  for (int c = c0; c < c1; ++c) {
    const int n = cnt[c];
    off[c] = at;
    at += n;
    cnt[c] = 0;
  }
}

// 3. one wave per open row: (row, slot) into the bucket of each of its pages
__global__ __launch_bounds__(kTsThreads) void ts_fill_kernel(TokenSelectParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t R = static_cast<int64_t>(p.B) * p.Hq * p.nqb;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kTsWaves + wave;
  if (row >= R) return;
  const int npg = p.npg[row];
  if (lane >= npg) return;
  const int qb = static_cast<int>(row % p.nqb);
  const int64_t bh = row / p.nqb;
  const int c = p.pages[row * p.S + lane];
  const int64_t pcix = bh * p.nqb + c;
  const int pos = p.off[pcix] + atomicAdd(&p.cnt[pcix], 1);
  p.ent[bh * p.nqb * p.S + pos] = qb * p.S + lane;
}

// 4. one workgroup per (b, h, page): scores = (query-block sums of up to 16
// recalling rows) x (the page's 128 key rows)^T on v_mfma_f64_16x16x4f64.
// Wave w owns rows 32w .. 32w+31 as two 16-row tiles.  Contraction step s
// takes channels (D/4) kk + s for kk = 0..3 (lane l feeds kk = l / 16), so a
// lane's key channels are D/4 contiguous bf16 values, loaded once and
// widened to fp64 per step.  A lane's output register r holds recalling row
// l/16 + 4r and key row l mod 16 of the tile.
template <int D>
__global__ __launch_bounds__(kTsThreads) __attribute__((amdgpu_waves_per_eu(3))) void ts_score_kernel(TokenSelectParams p) {
  constexpr int NS = D / 4;     // contraction steps
  constexpr int QP = D + 2;     // padded LDS row of query-block sums
  __shared__ double qs[kEnt][QP];
  __shared__ int32_t ents[kEnt];
  const int64_t pcix = blockIdx.x;
  const int n = p.cnt[pcix];
  if (n == 0) return;
  const int c = static_cast<int>(pcix % p.nqb);
  const int64_t bh = pcix / p.nqb;
  const int h = static_cast<int>(bh % p.Hq), b = static_cast<int>(bh / p.Hq);
  const int hk = h / p.group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, kk = lane >> 4;
  // B operand: key row 32 wave + 16 t + col, channels NS kk .. NS kk + NS-1
  constexpr int NV = NS / 8;  // 16-byte loads per tile
  u32x4 kr[2][NV];
  {
    const __bf16* kbase = static_cast<const __bf16*>(p.k) + b * p.ks_b + hk * p.ks_h +
                          static_cast<int64_t>(c) * 128 * p.ks_l + NS * kk;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < NV; ++v)
        kr[t][v] = *reinterpret_cast<const u32x4*>(kbase + (32 * wave + 16 * t + col) * p.ks_l + 8 * v);
  }
  const int32_t* eb = p.ent + bh * p.nqb * p.S + p.off[pcix];
  const double* qsb = p.qsum + bh * p.nqb * D;
  uint64_t* kb = p.keys + bh * p.nqb * p.S * 128;
  for (int e0 = 0; e0 < n; e0 += kEnt) {
    const int ne = min(kEnt, n - e0);
    __syncthreads();  // the previous round's reads of qs and ents are done
    if (tid < ne) ents[tid] = eb[e0 + tid];
    __syncthreads();
    {  // thread t stages D/16 channels of entry t/16 (independent loads)
      constexpr int CPT = D / 16;
      const int ee = tid / 16, ch0 = (tid % 16) * CPT;
      if (ee < ne) {
        const double* src = qsb + static_cast<int64_t>(ents[ee] / p.S) * D + ch0;
        double tv[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) tv[j] = src[j];
#pragma unroll
        for (int j = 0; j < CPT; ++j) qs[ee][ch0 + j] = tv[j];
      } else {  // unused A rows: zeros (their outputs are not stored)
#pragma unroll
        for (int j = 0; j < CPT; ++j) qs[ee][ch0 + j] = 0.0;
      }
    }
    __syncthreads();
    f64x4 acc[2] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
    const double* arow = &qs[col][NS * kk];  // A operand: recalling row col (rows >= ne are ignored)
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int st = 8 * v + j;
        const double a = arow[st];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t x = kr[t][v][j >> 1];
          const float kf = __builtin_bit_cast(float, (j & 1) ? (x & 0xFFFF0000u) : (x << 16));
          acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, static_cast<double>(kf), acc[t], 0, 0, 0);
        }
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = kk + 4 * r;
      if (e < ne) {
        const int ev = ents[e];
        uint64_t* dst = kb + (static_cast<int64_t>(ev / p.S) * p.S + ev % p.S) * 128 + 32 * wave + col;
        dst[0] = order_key(acc[0][r]);
        dst[16] = order_key(acc[1][r]);
      }
    }
  }
}

// lanes below this one whose bit is set in b
__device__ __forceinline__ int rank_below(uint64_t b) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b >> 32),
                                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b), 0u)));
}

// 5. one wave per open row, four rows per workgroup; everything stays inside
// the wave (its own LDS regions, ballots and lane shuffles), so no workgroup
// barrier is needed
__global__ __launch_bounds__(kTsThreads) void ts_select_kernel(TokenSelectParams p) {
  extern __shared__ uint64_t lds_keys[];  // per wave: S * 128 keys
  __shared__ uint32_t hist_all[kTsWaves][256];
  __shared__ uint64_t small_all[kTsWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t R = static_cast<int64_t>(p.B) * p.Hq * p.nqb;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kTsWaves + wave;
  if (row >= R) return;  // whole waves
  const int npg = p.npg[row];
  if (npg == 0) return;
  uint64_t* key = lds_keys + static_cast<size_t>(wave) * p.S * 128;
  uint32_t* hist = hist_all[wave];
  uint64_t* small = small_all[wave];
  const int C = npg * 128, K = p.K;
  const uint64_t* src = p.keys + row * p.S * 128;
  for (int r = lane; r < C; r += 64) key[r] = src[r];
  const int cpg = p.pages[row * p.S + (lane < npg ? lane : 0)];  // page of slot `lane`
  __builtin_amdgcn_wave_barrier();

  // the K-th largest key T, 8 bits at a time: `need` keys are still to be
  // chosen among those whose leading `bits` bits equal `prefix`, and at least
  // that many exist
  uint64_t prefix = 0;
  int need = K, bits = 0;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
#pragma unroll
    for (int q = 0; q < 4; ++q) hist[4 * lane + q] = 0;
    __builtin_amdgcn_wave_barrier();
    for (int r = lane; r < C; r += 64) {
      const uint64_t kk = key[r];
      if (pass == 0 || (kk >> (shift + 8)) == prefix) atomicAdd(&hist[(kk >> shift) & 255], 1u);
    }
    __builtin_amdgcn_wave_barrier();
    uint32_t cb[4], tot = 0;  // bins in descending order, 4 per lane
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      cb[q] = hist[255 - 4 * lane - q];
      tot += cb[q];
    }
    uint32_t incl = tot;
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    uint32_t run = incl - tot;  // keys in higher bins
    int fbin = -1, fneed = 0, fleft = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (run < static_cast<uint32_t>(need) && run + cb[q] >= static_cast<uint32_t>(need)) {
        fbin = 255 - 4 * lane - q;
        fneed = need - static_cast<int>(run);
        fleft = static_cast<int>(cb[q]);
      }
      run += cb[q];
    }
    const int sl = static_cast<int>(__builtin_ctzll(__builtin_amdgcn_ballot_w64(fbin >= 0)));  // one lane
    prefix = (prefix << 8) | static_cast<uint64_t>(__builtin_amdgcn_readlane(fbin, sl));
    need = __builtin_amdgcn_readlane(fneed, sl);
    const int left = __builtin_amdgcn_readlane(fleft, sl);
    bits = 8 * (pass + 1);
    __builtin_amdgcn_wave_barrier();  // the histogram is read before the next pass clears it
    if (left <= 64) break;            // few keys left: ranked by counting below
  }
  uint64_t T = prefix;
  if (bits < 64) {
    int m = 0;
    for (int r0 = 0; r0 < C; r0 += 64) {  // C is a multiple of 128
      const uint64_t kk = key[r0 + lane];
      const bool in = (kk >> (64 - bits)) == prefix;
      const uint64_t bl = __builtin_amdgcn_ballot_w64(in);
      if (in) small[m + rank_below(bl)] = kk;
      m += static_cast<int>(__popcll(bl));
    }
    __builtin_amdgcn_wave_barrier();
    const uint64_t mine = lane < m ? small[lane] : 0;
    int gt = 0, ge = 0;
    for (int j = 0; j < m; ++j) {
      const uint64_t o = small[j];
      gt += o > mine;
      ge += o >= mine;
    }
    const int sl = static_cast<int>(
        __builtin_ctzll(__builtin_amdgcn_ballot_w64(lane < m && gt < need && ge >= need)));  // lanes holding T
    T = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mine >> 32), sl)))
         << 32) |
        static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(mine)), sl));
    need -= __builtin_amdgcn_readlane(gt, sl);
  }

  // every key above T, and of those equal to T the first `need` in candidate
  // order; written in candidate order (e = r0 + lane, r0 ascending)
  int32_t* trow = p.tok + row * K;
  int eqc = 0, at = 0;
  for (int r0 = 0; r0 < C; r0 += 64) {
    const int e = r0 + lane;
    const uint64_t kk = key[e];
    const bool eq = kk == T;
    const uint64_t be = __builtin_amdgcn_ballot_w64(eq);
    const bool sel = kk > T || (eq && eqc + rank_below(be) < need);
    const uint64_t bs = __builtin_amdgcn_ballot_w64(sel);
    const int page = __builtin_amdgcn_readlane(cpg, r0 >> 7);  // 64 | 128: one page per r0
    if (sel) trow[at + rank_below(bs)] = page * 128 + (e & 127);
    eqc += static_cast<int>(__popcll(be));
    at += static_cast<int>(__popcll(bs));
  }
  if (lane == 0) p.tcnt[row] = K;
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t token_select_workspace_bytes(int32_t B, int32_t Hq, int32_t nqb, int32_t S) {
  const size_t R = static_cast<size_t>(B) * Hq * nqb;
  return 3 * round256(4 * R) + 2 * round256(4 * R * S) + round256(8 * R * S * 128);
}

hipError_t launch_token_select(const TokenSelectParams& p, hipStream_t stream) {
  if (p.D != 128 && p.D != 64) return hipErrorNotSupported;
  if (p.S < 0 || p.S > kMaxSlots) return hipErrorNotSupported;
  const int64_t R = static_cast<int64_t>(p.B) * p.Hq * p.nqb;
  const unsigned wave_groups = static_cast<unsigned>((R + kTsWaves - 1) / kTsWaves);
  hipError_t e = launch_kernel(ts_zero_kernel, dim3(static_cast<unsigned>((R + kTsThreads - 1) / kTsThreads)),
                               dim3(kTsThreads), 0, stream, p.cnt, R);
  if (e != hipSuccess) return e;
  e = launch_kernel(ts_rows_kernel, dim3(wave_groups), dim3(kTsThreads), 0, stream, p);
  if (e != hipSuccess) return e;
  if (p.K == 0 || p.S == 0) return hipSuccess;  // every row is final
  e = launch_kernel(ts_offsets_kernel, dim3(static_cast<unsigned>(p.B * p.Hq)), dim3(kTsThreads), 0, stream, p);
  if (e != hipSuccess) return e;
  e = launch_kernel(ts_fill_kernel, dim3(wave_groups), dim3(kTsThreads), 0, stream, p);
  if (e != hipSuccess) return e;
  e = p.D == 128 ? launch_kernel(ts_score_kernel<128>, dim3(static_cast<unsigned>(R)), dim3(kTsThreads), 0, stream, p)
                 : launch_kernel(ts_score_kernel<64>, dim3(static_cast<unsigned>(R)), dim3(kTsThreads), 0, stream, p);
  if (e != hipSuccess) return e;
  const size_t lds = sizeof(uint64_t) * 128 * static_cast<size_t>(p.S) * kTsWaves;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(ts_select_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(lds));
  if (e != hipSuccess) return e;
  return launch_kernel(ts_select_kernel, dim3(wave_groups), dim3(kTsThreads), lds, stream, p);
}

}  // namespace ssa
