// Page selection for the page-selected sparse-attention variant, gfx950.
//
// The LongCat sparse attention article (section 3) keeps a sink region and a
// local sliding window as contiguous reads (mechanism 1, streaming-aware
// indexing) and recalls extra 128-token pages by a coarse page score, keeping
// the top M (mechanism 3, hierarchical indexing, first stage).  Here the sink
// is block 0, the window is the SSA window, and the page score is
// <sum of q over the query block, sum of k over the page>, which ranks pages
// exactly like the product of the means.
//
// Two kernels:
//   1. block_sums: one workgroup per (b, head, block) of q and of k; fp64
//      sums of 128 bf16 rows (exact for these inputs, so the order of the
//      additions does not matter).  An HBM scan of q and k with
//      non-temporal loads.
//   2. select: one workgroup per (b, query head, 16 query blocks); fp64
//      scores of the candidate pages [n_global, qb - n_local] on the fp64
//      matrix cores, top-M kept as a sorted per-row list (equal scores ->
//      lower page), then the ascending list global blocks + chosen pages +
//      local blocks, padded with -1.
#include "common.hpp"

namespace ssa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSumThreads = 256;

// grid.x = B*Hq*nqb (q sums) + B*Hkv*nqb (k sums)
template <int D>
__global__ __launch_bounds__(kSumThreads) void block_sums_kernel(PageSelectParams p) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int nrg = kSumThreads / CPR;     // row groups
  constexpr int NR = 128 / nrg;              // rows per thread
  const int64_t nq = static_cast<int64_t>(p.B) * p.Hq * p.nqb;
  int64_t t = blockIdx.x;
  const bool is_q = t < nq;
  if (!is_q) t -= nq;
  const int H = is_q ? p.Hq : p.Hkv;
  const int blk = static_cast<int>(t % p.nqb);
  const int h = static_cast<int>((t / p.nqb) % H);
  const int b = static_cast<int>(t / (static_cast<int64_t>(p.nqb) * H));
  const __bf16* base = static_cast<const __bf16*>(is_q ? p.q : p.k) + b * (is_q ? p.qs_b : p.ks_b) +
                       h * (is_q ? p.qs_h : p.ks_h);
  const int64_t sl = is_q ? p.qs_l : p.ks_l;
  double* out = (is_q ? p.qsum : p.ksum) + t * D;

  const int cc = threadIdx.x % CPR, rg = threadIdx.x / CPR;
  const int nrow = min(128, p.L - blk * 128);  // rows of this block, >= 1
  // all of a thread's rows are loaded at once (a row past the last one reads
  // the last again and is left out of the sum), as non-temporal loads: q and
  // k are read once here
  u32x4 v[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int row = blk * 128 + min(rg + nrg * i, nrow - 1);
    v[i] = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4*)(base + row * sl + cc * 8));
  }
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    // a repeated row adds +0 (unconditionally, so that no load is sunk into a branch)
    const u32x4 x = rg + nrg * i < nrow ? v[i] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc[2 * w] += static_cast<double>(__builtin_bit_cast(float, x[w] << 16));
      acc[2 * w + 1] += static_cast<double>(__builtin_bit_cast(float, x[w] & 0xFFFF0000u));
    }
  }
  // reduce the nrg row groups: tree over LDS, 8 channels per thread
  __shared__ double buf[kSumThreads][8];
#pragma unroll
  for (int e = 0; e < 8; ++e) buf[threadIdx.x][e] = acc[e];
  __syncthreads();
  for (int s = nrg / 2; s > 0; s >>= 1) {
    if (rg < s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) buf[threadIdx.x][e] += buf[threadIdx.x + s * CPR][e];
    }
    __syncthreads();
  }
  if (rg == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[cc * 8 + e] = buf[threadIdx.x][e];
  }
}

// ---------------------------------------------------------------------------
// select: one workgroup of 4 waves per (b, query head, 16 query blocks).
// Scores are a dense product: S[c][qb] = <ksum[c], qsum[qb]> over D
// channels, taken 128 candidate pages at a time on v_mfma_f64_16x16x4_f64
// (16 candidates x 16 query blocks per tile; lane (n, g) feeds candidate /
// query block n and channels 8m + 2g, 8m + 2g + 1 for m = 0 .. D/8-1, so a
// row's 4 lanes read 64 contiguous bytes per load).  Each query block keeps
// a sorted list of its best top_m pages across the lanes of one wave; a
// chunk's candidate enters only if it beats the list's last entry (and, on a
// row's first chunk, is no worse than a lower bound on the chunk's M-th
// best), by an insertion at the rank a ballot gives.  "Beats" is a total order: higher
// score, equal scores -> lower page (a NaN score counts as -inf).
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 256;
constexpr int kRows = 16;     // query blocks per workgroup
constexpr int kChunk = 128;   // candidate pages scored per round
constexpr int kPad = kChunk + 4;

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bool better(double sa, int ca, double sb, int cb) {
  return sa > sb || (sa == sb && ca < cb);
}

__device__ __forceinline__ double read_lane_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(u), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(u >> 32), l);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// (t1, t2): the two largest of the lane's set; merged with the set of the
// lane CTRL's DPP pattern reads from (disjoint from the lane's own at every
// step of a rotate-and-merge all-reduce)
template <int CTRL>
__device__ __forceinline__ void top2_merge(double& t1, double& t2) {
  const uint64_t u1 = __builtin_bit_cast(uint64_t, t1), u2 = __builtin_bit_cast(uint64_t, t2);
  const uint32_t a = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(u1)), CTRL, 0xF, 0xF, false);
  const uint32_t b = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(u1 >> 32)), CTRL, 0xF, 0xF, false);
  const uint32_t c = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(u2)), CTRL, 0xF, 0xF, false);
  const uint32_t d = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(u2 >> 32)), CTRL, 0xF, 0xF, false);
  const double p1 = __builtin_bit_cast(double, (static_cast<uint64_t>(b) << 32) | a);
  const double p2 = __builtin_bit_cast(double, (static_cast<uint64_t>(d) << 32) | c);
  const double n2 = __builtin_fmax(__builtin_fmin(t1, p1), __builtin_fmax(t2, p2));
  t1 = __builtin_fmax(t1, p1);
  t2 = n2;
}

template <int D>
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(4))) void select_kernel(PageSelectParams p) {
  constexpr int NM = D / 8;  // 16-byte loads per operand row share; 2 MFMAs each
  __shared__ double sc[kRows][kPad];

  // heaviest tiles first (a tile's candidates grow with its query blocks),
  // every (b, head) of a tile index side by side, so the long tiles start
  // early and the short ones fill in behind them
  const int tiles = (p.nqb + kRows - 1) / kRows;
  const int tile = tiles - 1 - static_cast<int>(blockIdx.x / (p.B * p.Hq));
  const int h = static_cast<int>(blockIdx.x % p.Hq);
  const int b = static_cast<int>((blockIdx.x / p.Hq) % p.B);
  const int hk = h / p.group;
  const int qb0 = tile * kRows;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;

  auto g_end_of = [&](int qb) { return min(p.n_global, qb + 1); };
  auto l_begin_of = [&](int qb) { return max(g_end_of(qb), qb - p.n_local + 1); };
  const int qb_last = min(qb0 + kRows, p.nqb) - 1;
  const int ce = l_begin_of(qb_last);  // candidates of every row lie in [n_global, ce)

  // B operand: query-block sums of the 16 rows, staged in LDS (rows D + 2
  // doubles apart: the 16 rows of a fragment read start 4 banks apart), read
  // per product; lane (n, g) takes query block qb0 + n
  __shared__ __attribute__((aligned(16))) double qsl[kRows][D + 2];
  for (int i = threadIdx.x; i < kRows * D / 2; i += kSelThreads) {
    const int r = i / (D / 2), c2 = i % (D / 2);
    const int qrow = min(qb0 + r, p.nqb - 1);
    const double* qs = p.qsum + ((static_cast<int64_t>(b) * p.Hq + h) * p.nqb + qrow) * D;
    *reinterpret_cast<f64x2*>(&qsl[r][2 * c2]) = *reinterpret_cast<const f64x2*>(qs + 2 * c2);
  }
  __syncthreads();
  const double* qrow_l = &qsl[n][2 * g];
  const double* kbase = p.ksum + (static_cast<int64_t>(b) * p.Hkv + hk) * p.nqb * D;

  // the rows of this wave: qb0 + wave + 4 rr; list entry i of a row on lane i
  double ls[kRows / 4];
  int li[kRows / 4];
#pragma unroll
  for (int rr = 0; rr < kRows / 4; ++rr) {
    ls[rr] = -__builtin_inf();
    li[rr] = 0x7fffffff;
  }
  const int M = p.top_m;

  // A operand of this wave's next tile: its loads are issued while the
  // previous tile's products run (each register reloaded once its product
  // has read it), so a tile's L2 round trip hides behind the one before
  f64x2 kf[NM];
  auto load_tile = [&](int c0) {
    const double* kr = kbase + static_cast<int64_t>(max(min(c0 + n, ce - 1), 0)) * D;
#pragma unroll
    for (int m = 0; m < NM; ++m) kf[m] = *reinterpret_cast<const f64x2*>(kr + 8 * m + 2 * g);
  };
  load_tile(p.n_global + 16 * wave);
  for (int cc = p.n_global; cc < ce; cc += kChunk) {
    // scores of candidates cc .. cc+255 for the 16 query blocks
    for (int tt = wave; tt < kChunk / 16; tt += 4) {
      const int c0 = cc + tt * 16;
      if (c0 >= ce) break;
      // this wave's next tile: 4 tiles on in this chunk, else its first of the next
      const int nc0 = tt + 4 < kChunk / 16 ? c0 + 64 : cc + kChunk + 16 * wave;
      const double* nkr = kbase + static_cast<int64_t>(max(min(nc0 + n, ce - 1), 0)) * D;
      f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const f64x2 qv = *reinterpret_cast<const f64x2*>(qrow_l + 8 * m);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(kf[m][0], qv[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(kf[m][1], qv[1], acc, 0, 0, 0);
        kf[m] = *reinterpret_cast<const f64x2*>(nkr + 8 * m + 2 * g);
      }
      // lane (n, g), register r holds candidate c0 + g + 4r of query block
      // qb0 + n (the f64 16x16 output puts row lane/16 + 4 r in register r)
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[n][tt * 16 + g + 4 * r] = acc[r];
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < kRows / 4; ++rr) {
      const int qb = qb0 + wave + 4 * rr;
      if (qb >= p.nqb) continue;
      const int c_lo = g_end_of(qb), c_hi = l_begin_of(qb);
      if (c_hi - c_lo <= M) continue;  // every candidate is taken; no ranking
      double ts = read_lane_f64(ls[rr], M - 1);
      int tc = __builtin_amdgcn_readlane(li[rr], M - 1);
      // While the list is not full (a row's first chunk), bound the chunk's
      // M-th best from below: an item worse than that bar is beaten by M
      // items of the chunk and can be skipped.
      double bs = -__builtin_inf();
      int bc = 0x7fffffff;
      if (tc == 0x7fffffff && M <= 8) {
        // Up to 8 kept: each 16-lane row of the wave finds the two best of
        // its lanes' best scores (a rotate-and-merge all-reduce on DPP, no
        // LDS); every row's second best is reached by two distinct
        // candidates, so the lowest of the four is reached by 8 >= M of
        // them and a candidate scoring strictly below it cannot be kept.
        double t1 = -__builtin_inf(), t2 = -__builtin_inf();
#pragma unroll
        for (int k = 0; k < kChunk / 64; ++k) {
          const int c = cc + 64 * k + lane;
          double s = sc[wave + 4 * rr][64 * k + lane];
          if (s != s) s = -__builtin_inf();
          if (c >= c_lo && c < c_hi) t1 = __builtin_fmax(t1, s);
        }
        top2_merge<0x128>(t1, t2);  // row_ror:8
        top2_merge<0x124>(t1, t2);  // row_ror:4
        top2_merge<0x122>(t1, t2);  // row_ror:2
        top2_merge<0x121>(t1, t2);  // row_ror:1
        bs = __builtin_fmin(__builtin_fmin(read_lane_f64(t2, 0), read_lane_f64(t2, 16)),
                            __builtin_fmin(read_lane_f64(t2, 32), read_lane_f64(t2, 48)));
      } else if (tc == 0x7fffffff) {
        // more than 8 kept: the M-th best of the 64 per-lane bests, from a
        // bitonic sort across the lanes
#pragma unroll
        for (int k = 0; k < kChunk / 64; ++k) {
          const int c = cc + 64 * k + lane;
          double s = sc[wave + 4 * rr][64 * k + lane];
          if (s != s) s = -__builtin_inf();
          if (c >= c_lo && c < c_hi && better(s, c, bs, bc)) {
            bs = s;
            bc = c;
          }
        }
        // sort the lane bests, best first: lane i ends with the i-th best
#pragma unroll
        for (int kk = 2; kk <= 64; kk <<= 1)
#pragma unroll
          for (int j = kk >> 1; j > 0; j >>= 1) {
            const uint64_t u = __builtin_bit_cast(uint64_t, bs);
            const uint32_t plo = __shfl_xor(static_cast<uint32_t>(u), j);
            const uint32_t phi = __shfl_xor(static_cast<uint32_t>(u >> 32), j);
            const double ps = __builtin_bit_cast(double, (static_cast<uint64_t>(phi) << 32) | plo);
            const int pc = __shfl_xor(bc, j);
            const bool keep_better = ((lane & kk) == 0) == ((lane & j) == 0);
            if (keep_better ? better(ps, pc, bs, bc) : better(bs, bc, ps, pc)) {
              bs = ps;
              bc = pc;
            }
          }
        const double b_s = read_lane_f64(bs, M - 1);
        const int b_c = __builtin_amdgcn_readlane(bc, M - 1);
        bs = b_s;
        bc = b_c;
      }
#pragma unroll
      for (int k = 0; k < kChunk / 64; ++k) {
        const int c = cc + 64 * k + lane;
        double s = sc[wave + 4 * rr][64 * k + lane];
        if (s != s) s = -__builtin_inf();
        bool q = c >= c_lo && c < c_hi && better(s, c, ts, tc) && !better(bs, bc, s, c);
        uint64_t mask = __builtin_amdgcn_ballot_w64(q);
        while (mask) {
          const int src = __builtin_ctzll(mask);
          mask &= mask - 1;
          const double xs = read_lane_f64(s, src);
          const int xc = cc + 64 * k + src;
          if (!better(xs, xc, ts, tc)) continue;  // the bar rose since the ballot
          // rank of x: list entries that beat it
          const bool above = lane < M && better(ls[rr], li[rr], xs, xc);
          const int pos = __builtin_popcountll(__builtin_amdgcn_ballot_w64(above));
          // entries at or below pos move down by one (a whole-wave DPP shift:
          // lane i receives lane i-1); x takes pos
          const uint64_t u = __builtin_bit_cast(uint64_t, ls[rr]);
          const uint32_t plo = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(u), 0x138, 0xF, 0xF, false);
          const uint32_t phi = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(u >> 32), 0x138, 0xF, 0xF, false);
          const int pc = __builtin_amdgcn_update_dpp(0, li[rr], 0x138, 0xF, 0xF, false);
          if (lane > pos && lane < M) {
            ls[rr] = __builtin_bit_cast(double, (static_cast<uint64_t>(phi) << 32) | plo);
            li[rr] = pc;
          } else if (lane == pos) {
            ls[rr] = xs;
            li[rr] = xc;
          }
          ts = read_lane_f64(ls[rr], M - 1);
          tc = __builtin_amdgcn_readlane(li[rr], M - 1);
        }
      }
    }
    __syncthreads();  // the next chunk overwrites the scores
  }

  // lists: global blocks, chosen pages ascending, local blocks, padding
#pragma unroll
  for (int rr = 0; rr < kRows / 4; ++rr) {
    const int qb = qb0 + wave + 4 * rr;
    if (qb >= p.nqb) continue;
    const int g_end = g_end_of(qb), l_begin = l_begin_of(qb);
    const int ncand = l_begin - g_end;
    const int take = min(ncand, M);
    const int64_t row = (static_cast<int64_t>(b) * p.Hq + h) * p.nqb + qb;
    int32_t* out = p.idx + row * p.W;
    const int nloc = qb - l_begin + 1;
    const int count = g_end + take + nloc;
    for (int pos = lane; pos < p.W; pos += 64) {
      int v = -1;
      if (pos < g_end) v = pos;
      else if (pos >= g_end + take && pos < count) v = l_begin + (pos - g_end - take);
      else if (pos < g_end + take && ncand <= M) v = pos;  // all candidates, already ascending
      if (!(pos >= g_end && pos < g_end + take && ncand > M)) out[pos] = v;
    }
    if (ncand > M) {
      // lane i < take holds chosen page li; its place is its rank by page id
      int rank = 0;
      for (int j = 0; j < take; ++j) rank += __builtin_amdgcn_readlane(li[rr], j) < li[rr];
      if (lane < take) out[g_end + rank] = li[rr];
    }
    if (lane == 0) p.cnt[row] = count;
  }
}

}  // namespace

// Scratch of the allocation-free entry point, for callers that cannot
// allocate device memory (graph capture, serving loops): the fp64 block sums
// of q and k, kPageScratchBytes at most.  Each GPU the library runs on holds
// its own copy until the process ends.  Every call on a GPU shares it and it
// keeps the last call's sums; nothing in it has to start at zero (the sums
// kernel writes every value the select kernel reads), but calls that overlap
// on one GPU race on it.  Host code uses the address looked up below, never
// the array's name.
static __device__ __align__(256) unsigned char scratch[kPageScratchBytes];

hipError_t page_select_scratch(void** ptr) {
  static std::once_flag once[kMaxDevices];
  static void* addr[kMaxDevices];
  static hipError_t status[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [&] {
    void* a = nullptr;
    status[dev] = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    addr[dev] = a;
  });
  if (status[dev] != hipSuccess) return status[dev];
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_page_sums(const PageSelectParams& p, hipStream_t stream) {
  const int64_t nsum = static_cast<int64_t>(p.B) * (p.Hq + p.Hkv) * p.nqb;
  return p.D == 128 ? launch_kernel(block_sums_kernel<128>, dim3(static_cast<unsigned>(nsum)), dim3(kSumThreads), 0, stream, p)
       : p.D == 64  ? launch_kernel(block_sums_kernel<64>, dim3(static_cast<unsigned>(nsum)), dim3(kSumThreads), 0, stream, p)
                    : hipErrorNotSupported;
}

hipError_t launch_page_top(const PageSelectParams& p, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(p.B) * p.Hq * ((p.nqb + kRows - 1) / kRows));
  if (p.D == 128) return launch_kernel(select_kernel<128>, dim3(grid), dim3(kSelThreads), 0, stream, p);
  if (p.D == 64) return launch_kernel(select_kernel<64>, dim3(grid), dim3(kSelThreads), 0, stream, p);
  return hipErrorNotSupported;
}

hipError_t launch_page_select(const PageSelectParams& p, hipStream_t stream) {
  const hipError_t e = launch_page_sums(p, stream);
  return e != hipSuccess ? e : launch_page_top(p, stream);
}

}  // namespace ssa
