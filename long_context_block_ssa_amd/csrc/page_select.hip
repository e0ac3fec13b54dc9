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
//      additions does not matter).  An HBM scan of q and k.
//   2. select: one workgroup per (b, query head, query block); fp64 scores of
//      the candidate pages [n_global, qb - n_local], top-M by repeated
//      arg-max (equal scores -> lower page), then the ascending list
//      global blocks + chosen pages + local blocks, padded with -1.
#include "common.hpp"

namespace ssa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSumThreads = 256;

// grid.x = B*Hq*nqb (q sums) + B*Hkv*nqb (k sums)
__global__ __launch_bounds__(kSumThreads) void block_sums_kernel(PageSelectParams p) {
  const int D = p.D, CPR = D / 8;                  // 16-byte chunks per row
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

  const int cc = threadIdx.x % CPR, rg = threadIdx.x / CPR, nrg = kSumThreads / CPR;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int r = rg; r < 128; r += nrg) {
    const int row = blk * 128 + r;
    if (row >= p.L) break;
    const u32x4 v = *reinterpret_cast<const u32x4*>(base + row * sl + cc * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc[2 * w] += static_cast<double>(__builtin_bit_cast(float, v[w] << 16));
      acc[2 * w + 1] += static_cast<double>(__builtin_bit_cast(float, v[w] & 0xFFFF0000u));
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

constexpr int kSelThreads = 256;

__device__ __forceinline__ bool better(double sa, int ca, double sb, int cb) {
  return sa > sb || (sa == sb && ca < cb);
}

// dynamic LDS: scores[nqb] doubles
__global__ __launch_bounds__(kSelThreads) void select_kernel(PageSelectParams p) {
  extern __shared__ double scores[];
  __shared__ double qs[128];
  __shared__ double red_s[kSelThreads / 64];
  __shared__ int red_c[kSelThreads / 64];
  __shared__ int chosen[32];

  const int t = blockIdx.x;
  const int qb = t % p.nqb;
  const int h = (t / p.nqb) % p.Hq;
  const int b = t / (p.nqb * p.Hq);
  const int hk = h / p.group;
  const int D = p.D;
  int32_t* out = p.idx + static_cast<int64_t>(t) * p.W;

  const int g_end = min(p.n_global, qb + 1);
  const int l_begin = max(g_end, qb - p.n_local + 1);
  // candidate pages [g_end, l_begin)
  const int ncand = l_begin - g_end;
  const int take = min(ncand, p.top_m);

  if (ncand > p.top_m) {
    const double* qrow = p.qsum + static_cast<int64_t>(t) * D;
    for (int d = threadIdx.x; d < D; d += kSelThreads) qs[d] = qrow[d];
    __syncthreads();
    const double* kbase = p.ksum + (static_cast<int64_t>(b) * p.Hkv + hk) * p.nqb * D;
    for (int c = g_end + threadIdx.x; c < l_begin; c += kSelThreads) {
      const double* kr = kbase + static_cast<int64_t>(c) * D;
      double s = 0.0;
      for (int d = 0; d < D; ++d) s = __builtin_fma(qs[d], kr[d], s);
      scores[c] = s;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int r = 0; r < take; ++r) {
      double bs = -__builtin_inf();
      int bc = 0x7fffffff;
      for (int c = g_end + threadIdx.x; c < l_begin; c += kSelThreads) {
        const double s = scores[c];
        if (better(s, c, bs, bc)) {
          bs = s;
          bc = c;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const double os = __shfl_xor(bs, o);
        const int oc = __shfl_xor(bc, o);
        if (better(os, oc, bs, bc)) {
          bs = os;
          bc = oc;
        }
      }
      if (lane == 0) {
        red_s[wave] = bs;
        red_c[wave] = bc;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        double ws = red_s[0];
        int wc = red_c[0];
        for (int w = 1; w < kSelThreads / 64; ++w)
          if (better(red_s[w], red_c[w], ws, wc)) {
            ws = red_s[w];
            wc = red_c[w];
          }
        chosen[r] = wc;
        scores[wc] = -__builtin_inf();  // removed from later rounds
      }
      __syncthreads();
    }
  } else {
    for (int r = threadIdx.x; r < take; r += kSelThreads) chosen[r] = g_end + r;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    // sort the chosen pages (at most 32) ascending
    for (int i = 1; i < take; ++i) {
      const int x = chosen[i];
      int j = i - 1;
      while (j >= 0 && chosen[j] > x) {
        chosen[j + 1] = chosen[j];
        --j;
      }
      chosen[j + 1] = x;
    }
    int s = 0;
    for (int c = 0; c < g_end; ++c) out[s++] = c;
    for (int i = 0; i < take; ++i) out[s++] = chosen[i];
    for (int c = l_begin; c <= qb; ++c) out[s++] = c;
    p.cnt[t] = s;
    for (; s < p.W; ++s) out[s] = -1;
  }
}

}  // namespace

hipError_t launch_page_select(const PageSelectParams& p, hipStream_t stream) {
  const int64_t nsum = static_cast<int64_t>(p.B) * (p.Hq + p.Hkv) * p.nqb;
  hipError_t e = launch_kernel(block_sums_kernel, dim3(static_cast<unsigned>(nsum)), dim3(kSumThreads), 0, stream, p);
  if (e != hipSuccess) return e;
  const size_t lds = sizeof(double) * static_cast<size_t>(p.nqb);
  return launch_kernel(select_kernel, dim3(static_cast<unsigned>(static_cast<int64_t>(p.B) * p.Hq * p.nqb)),
                       dim3(kSelThreads), lds, stream, p);
}

}  // namespace ssa
