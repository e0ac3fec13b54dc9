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
//   1. rows: one wave per (b, head, query block) turns the page list into
//      the ascending, duplicate-free candidate pages (at most top_m); a row
//      with at most K candidate tokens (or K = 0) is written out here;
//   2. buckets: one workgroup per (b, head) counts the open rows' (row,
//      slot) entries per page, scans the counts into bucket offsets and
//      appends every entry to its page's bucket (the order inside a bucket
//      is free: every entry has its own output place);
//   3. score: one workgroup per (b, head, page) loads the page's 128 key
//      rows once into registers (a row per lane, bf16) and takes the dot
//      products with the query-block sums of up to 8 recalling rows at a
//      time as fp64 FMAs on the vector units, the query-block sum reaching
//      every lane through a row broadcast, writing order-preserving 64-bit
//      keys (NaN counts as -inf, -0 as +0) into each recalling row's slot;
//   4. select: one wave per open row finds the K-th largest key T exactly
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
typedef double f64x2 __attribute__((ext_vector_type(2)));

constexpr int kTsThreads = 256;
constexpr int kTsWaves = kTsThreads / 64;
constexpr int kMaxSlots = 32;
constexpr int kRegSlots = 8;  // rows of at most this many pages keep their keys in registers

// order-preserving map of a score to an unsigned key (larger score -> larger
// key); -0 is folded onto +0 and NaN onto -inf
__device__ __forceinline__ uint64_t order_key(double x) {
  if (x == 0.0) x = 0.0;
  if (x != x) x = -__builtin_inf();
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
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

// 1. one wave per row (b, h, qb)
__global__ __launch_bounds__(kTsThreads) void ts_rows_kernel(TokenSelectParams p) {
  __shared__ int32_t spg[kTsWaves][kMaxSlots];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t R = static_cast<int64_t>(p.B) * p.Hq * p.nqb;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kTsWaves + wave;
  if (row >= R) return;  // whole waves
  const int qb = static_cast<int>(row % p.nqb);
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
}

// 2. one workgroup per (b, h) builds the page buckets of its open rows:
// counts the (row, slot) entries per page in LDS, scans the counts into
// bucket offsets (written out with the counts for the score kernel), then
// appends every entry qb * S + slot to its page's bucket through an LDS
// cursor (the order inside a bucket is free: every entry has its own output
// place).  Pages are taken kBkSeg at a time, so any nqb fits the LDS.
constexpr int kBkThreads = 1024;
constexpr int kBkSeg = 4096;

__global__ __launch_bounds__(kBkThreads) void ts_buckets_kernel(TokenSelectParams p) {
  __shared__ int32_t lc[kBkSeg];
  __shared__ int32_t wsum[kBkThreads / 64];
  __shared__ int32_t seg_end;
  const int tid = threadIdx.x;
  const int64_t rbase = static_cast<int64_t>(blockIdx.x) * p.nqb;  // first row (and page) of (b, h)
  const int nent = p.nqb * p.S;
  const int32_t* npg = p.npg + rbase;
  const int32_t* pages = p.pages + rbase * p.S;
  int32_t* ent = p.ent + rbase * p.S;
  int base = 0;  // bucket offset of the segment's first page
  for (int c0 = 0; c0 < p.nqb; c0 += kBkSeg) {
    const int nc = min(kBkSeg, p.nqb - c0);
    for (int c = tid; c < nc; c += kBkThreads) lc[c] = 0;
    __syncthreads();
    for (int i = tid; i < nent; i += kBkThreads) {
      const int qb = i / p.S;
      if (i - qb * p.S < npg[qb]) {
        const int c = pages[i] - c0;
        if (c >= 0 && c < nc) atomicAdd(&lc[c], 1);
      }
    }
    __syncthreads();
    const int per = (nc + kBkThreads - 1) / kBkThreads;  // a run of consecutive pages per thread
    const int a0 = min(tid * per, nc), a1 = min(a0 + per, nc);
    int mine = 0;
    for (int c = a0; c < a1; ++c) mine += lc[c];
    int at = base + block_excl_scan(mine, wsum);
    for (int c = a0; c < a1; ++c) {
      const int n = lc[c];
      p.off[rbase + c0 + c] = at;
      p.cnt[rbase + c0 + c] = n;
      lc[c] = at;  // from here on the page's fill cursor
      at += n;
    }
    if (tid == kBkThreads - 1) seg_end = at;
    __syncthreads();
    for (int i = tid; i < nent; i += kBkThreads) {
      const int qb = i / p.S, slot = i - qb * p.S;
      if (slot < npg[qb]) {
        const int c = pages[i] - c0;
        if (c >= 0 && c < nc) ent[atomicAdd(&lc[c], 1)] = qb * p.S + slot;
      }
    }
    base = seg_end;
    __syncthreads();  // lc and seg_end are reused by the next segment
  }
}

// 3. one workgroup of two waves per (b, h, page): lane l of wave w owns key
// row 64 w + l of the page.  On this chip fp64 FMAs on the vector units run
// at the fp64 matrix rate, so the scores are plain dot products with no
// padding of the recalling rows to a matrix tile (a page is recalled by ~8
// rows on average, half a 16-row tile).  A wave reads its 64 key rows
// coalesced through LDS into registers once (bf16, a row per lane), stages
// the query-block sums of up to 8 recalling rows in LDS (all loads in flight
// together), then widens 16 channels of its key row to fp64 at a time and
// accumulates the 8 dot products side by side; lane j of each 16-lane row
// holds channel j of a query-block sum and the FMA's row broadcast hands it
// to every lane.  Measured at L = 131072, H = 16, M = 8 (same box, same
// inputs): ~235 us against ~330 us for the former 16 x 16 fp64 MFMA tiles;
// the counters show the vector unit ~2/3 busy at a 1.4 GHz clock (fp64 FMAs
// keep the card's clock low), a quarter of its instructions the widening.
constexpr int kScThreads = 128;
constexpr int kScEnt = 8;     // recalling rows per batch, accumulated side by side
constexpr int kScSlice = 16;  // channels of a key row widened to fp64 at a time

// acc += (lane j of this lane's 16-lane row of q) * k[j] for j = 0..15: the
// fp64 FMA takes its first operand through a row broadcast, so 16 lanes
// holding 16 channels of a query-block sum feed every key lane of the row.
// The s_nop covers the wait states a broadcast source needs after a vector
// write of it.
__device__ __forceinline__ void fmac_row_bcast16(double& acc, double q, const double* k) {
  asm volatile(
      "s_nop 1\n"
      "v_fmac_f64_dpp %0, %1, %2 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %0, %1, %3 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %0, %1, %4 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %0, %1, %5 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %0, %1, %6 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %0, %1, %7 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %0, %1, %8 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %0, %1, %9 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %0, %1, %10 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %0, %1, %11 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %0, %1, %12 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %0, %1, %13 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %0, %1, %14 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %0, %1, %15 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %0, %1, %16 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %0, %1, %17 row_newbcast:15 row_mask:0xf bank_mask:0xf"
      : "+v"(acc)
      : "v"(q), "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "v"(k[4]), "v"(k[5]), "v"(k[6]), "v"(k[7]), "v"(k[8]),
        "v"(k[9]), "v"(k[10]), "v"(k[11]), "v"(k[12]), "v"(k[13]), "v"(k[14]), "v"(k[15]));
}

template <int D>
__global__ __launch_bounds__(kScThreads) __attribute__((amdgpu_waves_per_eu(4))) void ts_score_kernel(TokenSelectParams p) {
  constexpr int HD = kScSlice < D ? kScSlice : D;  // channels per slice
  constexpr int QM = HD / 16;                      // query-sum values per lane and slice
  static_assert(HD % 16 == 0 && D % HD == 0, "slices are whole 16-lane rows of channels");
  // per wave: a 128-byte segment of its 64 key rows at a time, then the
  // batch's query-block sums
  constexpr int kUnits = (kScEnt * D * 8 > 64 * 128 ? kScEnt * D * 8 : 64 * 128) / 16;
  __shared__ u32x4 lds[kScThreads / 64][kUnits];
  const int64_t pcix = blockIdx.x;
  const int n = p.cnt[pcix];
  if (n == 0) return;
  const int c = static_cast<int>(pcix % p.nqb);
  const int64_t bh = pcix / p.nqb;
  const int h = static_cast<int>(bh % p.Hq), b = static_cast<int>(bh / p.Hq);
  const int hk = h / p.group;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int key = 64 * wave + lane;
  const __bf16* kpage = static_cast<const __bf16*>(p.k) + b * p.ks_b + hk * p.ks_h +
                        (static_cast<int64_t>(c) * 128 + 64 * wave) * p.ks_l;
  const int32_t* eb = p.ent + bh * p.nqb * p.S + p.off[pcix];
  const double* qsb = p.qsum + bh * p.nqb * D;
  uint64_t* kb = p.keys + bh * p.nqb * p.S * 128;
  double (*wq)[D] = reinterpret_cast<double (*)[D]>(lds[wave]);
  u32x4* wk = lds[wave];  // [64 rows][8 units of 16 bytes], unit u of row r at u ^ (r & 7)
  // the wave's key rows, bf16, into registers (lane = row): each 128-byte
  // segment is read coalesced (8 rows per load) into LDS and read back by
  // rows; the XOR keeps 8 neighbouring lanes on distinct banks
  u32x4 raw[D / 8];
#pragma unroll
  for (int sg = 0; sg < D / 64; ++sg) {
    u32x4 t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * i + (lane >> 3);
      t[i] = *reinterpret_cast<const u32x4*>(kpage + r * p.ks_l + 64 * sg + 8 * (lane & 7));
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * i + (lane >> 3);
      wk[8 * r + ((lane & 7) ^ (r & 7))] = t[i];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < 8; ++u) raw[8 * sg + u] = wk[8 * lane + (u ^ (lane & 7))];
    __builtin_amdgcn_wave_barrier();
  }
  for (int e0 = 0; e0 < n; e0 += kScEnt) {
    const int ne = min(kScEnt, n - e0);
    // lane e < ne holds the batch's recalling row e (qb * S + slot)
    const int my_ev = lane < ne ? eb[e0 + lane] : 0;
    const int my_qo = (my_ev / p.S) * D;
    // the batch's query-block sums into this wave's LDS rows (wave-local:
    // the wave's own LDS accesses complete in order); all kScEnt rows are
    // loaded so that every load is in flight at once (rows past ne load
    // query block 0's sums, unused)
    {
      constexpr int PL = (D + 127) / 128;  // 16-byte loads per lane and row
      f64x2 t[kScEnt][PL];
#pragma unroll
      for (int e = 0; e < kScEnt; ++e) {
        const double* src = qsb + __builtin_amdgcn_readlane(my_qo, e);
#pragma unroll
        for (int i = 0; i < PL; ++i)
          if (2 * lane + 128 * i < D) t[e][i] = *reinterpret_cast<const f64x2*>(src + 2 * lane + 128 * i);
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int e = 0; e < kScEnt; ++e)
#pragma unroll
        for (int i = 0; i < PL; ++i)
          if (2 * lane + 128 * i < D) *reinterpret_cast<f64x2*>(&wq[e][2 * lane + 128 * i]) = t[e][i];
    }
    __builtin_amdgcn_wave_barrier();
    double acc[kScEnt];
#pragma unroll
    for (int e = 0; e < kScEnt; ++e) acc[e] = 0.0;
#pragma unroll
    for (int ps = 0; ps < D / HD; ++ps) {
      // one slice of widened keys live at a time: the empty asm keeps the
      // widening inside the batch loop instead of hoisted (all D channels
      // as fp64 would not fit in registers)
#pragma unroll
      for (int v = 0; v < HD / 8; ++v) asm volatile("" : "+v"(raw[HD / 8 * ps + v]));
      double kf[HD];
#pragma unroll
      for (int v = 0; v < HD / 8; ++v)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t x = raw[HD / 8 * ps + v][w];
          kf[8 * v + 2 * w] = static_cast<double>(__builtin_bit_cast(float, x << 16));
          kf[8 * v + 2 * w + 1] = static_cast<double>(__builtin_bit_cast(float, x & 0xFFFF0000u));
        }
#pragma unroll
      for (int e = 0; e < kScEnt; ++e) {
        if (e < ne) {
#pragma unroll
          for (int m = 0; m < QM; ++m) fmac_row_bcast16(acc[e], wq[e][HD * ps + 16 * m + (lane & 15)], kf + 16 * m);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < kScEnt; ++e)
      if (e < ne) kb[static_cast<int64_t>(__builtin_amdgcn_readlane(my_ev, e)) * 128 + key] = order_key(acc[e]);
  }
}

// lanes below this one whose bit is set in b
__device__ __forceinline__ int rank_below(uint64_t b) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b >> 32),
                                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b), 0u)));
}

// 4. one wave per open row, four rows per workgroup; everything stays inside
// the wave (its own LDS regions, ballots and lane shuffles), so no workgroup
// barrier is needed.  Candidate e = 64 i + lane of a row is lane's i-th key:
// in registers when a row has at most NK * 64 candidates (NK > 0), else in
// the wave's LDS region (NK = 0).
template <int NK>
__global__ __launch_bounds__(kTsThreads) void ts_select_kernel(TokenSelectParams p) {
  constexpr bool kRegs = NK > 0;
  extern __shared__ uint64_t lds_keys[];  // NK = 0: per wave S * 128 keys
  __shared__ uint32_t hist_all[kTsWaves][256];
  __shared__ uint64_t small_all[kTsWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t R = static_cast<int64_t>(p.B) * p.Hq * p.nqb;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kTsWaves + wave;
  if (row >= R) return;  // whole waves
  const int npg = p.npg[row];
  if (npg == 0) return;
  uint32_t* hist = hist_all[wave];
  uint64_t* small = small_all[wave];
  const int C = npg * 128, K = p.K;
  const int NI = C / 64;  // keys per lane (C is a multiple of 128)
  const uint64_t* src = p.keys + row * p.S * 128;
  uint64_t kv[kRegs ? NK : 1];
  uint64_t* key = lds_keys + (kRegs ? 0 : static_cast<size_t>(wave) * p.S * 128);
  if constexpr (kRegs) {
#pragma unroll
    for (int i = 0; i < NK; ++i) kv[i] = i < NI ? src[64 * i + lane] : 0;
  } else {
    // 8 loads of a lane in flight together
    for (int r0 = 0; r0 < C; r0 += 512) {
      uint64_t t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (r0 + 64 * i < C) t[i] = src[r0 + 64 * i + lane];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (r0 + 64 * i < C) key[r0 + 64 * i + lane] = t[i];
    }
  }
  // f(i, key) for every key of the lane, i ascending
  auto each = [&](auto&& f) {
    if constexpr (kRegs) {
#pragma unroll
      for (int i = 0; i < NK; ++i)
        if (i < NI) f(i, kv[i]);
    } else {
      for (int i = 0; i < NI; ++i) f(i, key[64 * i + lane]);
    }
  };
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
    auto count = [&](uint64_t kk) {
      if (pass == 0 || (kk >> (shift + 8)) == prefix) atomicAdd(&hist[(kk >> shift) & 255], 1u);
    };
    if constexpr (kRegs) {
      each([&](int, uint64_t kk) { count(kk); });
    } else {
      for (int r0 = 0; r0 < C; r0 += 512) {  // 8 reads of a lane before their atomics
        uint64_t t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (r0 + 64 * i < C) t[i] = key[r0 + 64 * i + lane];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (r0 + 64 * i < C) count(t[i]);
      }
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
    each([&](int, uint64_t kk) {
      const bool in = (kk >> (64 - bits)) == prefix;
      const uint64_t bl = __builtin_amdgcn_ballot_w64(in);
      if (in) small[m + rank_below(bl)] = kk;
      m += static_cast<int>(__popcll(bl));
    });
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
  // order; written in candidate order (e = 64 i + lane, i ascending)
  int32_t* trow = p.tok + row * K;
  int eqc = 0, at = 0;
  each([&](int i, uint64_t kk) {
    const int e = 64 * i + lane;
    const bool eq = kk == T;
    const uint64_t be = __builtin_amdgcn_ballot_w64(eq);
    const bool sel = kk > T || (eq && eqc + rank_below(be) < need);
    const uint64_t bs = __builtin_amdgcn_ballot_w64(sel);
    const int page = __builtin_amdgcn_readlane(cpg, i >> 1);  // 64 | 128: one page per i
    if (sel) trow[at + rank_below(bs)] = page * 128 + (e & 127);
    eqc += static_cast<int>(__popcll(be));
    at += static_cast<int>(__popcll(bs));
  });
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
  hipError_t e = launch_kernel(ts_rows_kernel, dim3(wave_groups), dim3(kTsThreads), 0, stream, p);
  if (e != hipSuccess) return e;
  if (p.K == 0 || p.S == 0) return hipSuccess;  // every row is final
  e = launch_kernel(ts_buckets_kernel, dim3(static_cast<unsigned>(p.B * p.Hq)), dim3(kBkThreads), 0, stream, p);
  if (e != hipSuccess) return e;
  e = p.D == 128 ? launch_kernel(ts_score_kernel<128>, dim3(static_cast<unsigned>(R)), dim3(kScThreads), 0, stream, p)
                 : launch_kernel(ts_score_kernel<64>, dim3(static_cast<unsigned>(R)), dim3(kScThreads), 0, stream, p);
  if (e != hipSuccess) return e;
  if (p.S <= kRegSlots) return launch_kernel(ts_select_kernel<2 * kRegSlots>, dim3(wave_groups), dim3(kTsThreads), 0, stream, p);
  const size_t lds = sizeof(uint64_t) * 128 * static_cast<size_t>(p.S) * kTsWaves;
  e = raise_lds_limit_once<ts_select_kernel<0>>(static_cast<int>(sizeof(uint64_t) * 128 * kMaxSlots * kTsWaves));
  if (e != hipSuccess) return e;
  return launch_kernel(ts_select_kernel<0>, dim3(wave_groups), dim3(kTsThreads), lds, stream, p);
}

}  // namespace ssa
