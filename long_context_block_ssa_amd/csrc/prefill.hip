// Block-sparse causal attention prefill for gfx950 (CDNA4).
//
// One workgroup computes one 128-query tile (b, h, qb) over the key blocks
// listed for its query block: the SSA window (block 0 + the 7 most recent
// blocks, QbitAI report on LongCat LoZA, sparse-window paragraph), a
// page-selected list, or every block 0..qb for the dense comparison layer.
// Within the listed blocks it is the masked softmax of equation (2) of the
// "LoZA: ZigZag sparse attention" page (section 2.1), with the causal rule
// key <= query in the own block (section 2.2.1), evaluated as an online
// (running-max) softmax -- the max-subtracted form of the CSA/HCA tutorial
// page, section 7.1, applied block by block, which is an exact rewrite.
//
// bf16 path (Dqk = Dv = D in {64, 128}):
//   - 4 waves, 32 queries each.  The wave computes S^T = K Q^T per 16x16 tile
//     with v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = Q^T from
//     registers), so each lane owns one query column and 4 keys of it; the
//     softmax max/sum over keys is a per-lane reduction plus two cross-lane
//     steps.
//   - O^T = V^T P^T on the same instruction: P^T (the B operand) comes
//     straight from the S^T accumulators converted to bf16; V^T (the A
//     operand) is read from an LDS copy of the V block stored transposed with
//     the key order the P^T registers imply.
//   - K and V blocks (128 x D bf16 each) are staged through LDS once per
//     workgroup and read by the 4 waves.
// f32 path (D = 64): the same structure on v_mfma_f32_16x16x4f32, where
//   each instruction contracts over 4 keys so V is read row-major from LDS.
#include "common.hpp"

namespace ssa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 128;   // tokens per block == queries per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = kBlock / kWaves;  // queries per wave (32)
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float wave_max16x4(float x) {
  // lanes l, l^16, l^32, l^48 hold the same query
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum16x4(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Tile order: query blocks from last to first (the dense layer's longest rows
// first), heads fastest.  Consecutive workgroups land on consecutive XCDs, so
// when B*Hq is a multiple of 8 each (b, h) stays on one XCD for every query
// block and its K/V blocks are reused from that XCD's L2.
__device__ __forceinline__ void tile_coords(const PrefillParams& p, int& b, int& h, int& qb) {
  const int bh_count = p.B * p.Hq;
  const int t = blockIdx.x;
  qb = p.nqb - 1 - t / bh_count;
  const int bh = t % bh_count;
  b = bh / p.Hq;
  h = bh % p.Hq;
}

__device__ __forceinline__ int list_count(const PrefillParams& p, int b, int h, int qb) {
  if (p.dense) return qb + 1;
  return min(p.cnt[b * p.cnt_sb + h * p.cnt_sh + qb], p.W);
}
__device__ __forceinline__ int list_entry(const PrefillParams& p, int b, int h, int qb, int s) {
  if (p.dense) return qb - s;  // own block first
  return p.idx[b * p.idx_sb + h * p.idx_sh + static_cast<int64_t>(qb) * p.W + s];
}

template <typename OutT>
__device__ __forceinline__ void store4(OutT* dst, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float* dst, f32x4 v) {
  *reinterpret_cast<f32x4*>(dst) = v;
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* dst, f32x4 v) {
  *reinterpret_cast<bf16x4*>(dst) = __builtin_convertvector(v, bf16x4);
}

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------

template <int D>
struct BfLds {
  static constexpr int KP = D + 8;       // padded K row (bf16 elements)
  static constexpr int VP = kBlock + 8;  // padded V^T row
  __bf16 k[kBlock * KP];
  __bf16 vt[D * VP];
};

template <int D, typename OutT>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillParams p) {
  constexpr int NC = D / 32;  // 32-wide contraction chunks over channels
  constexpr int NJ = D / 16;  // 16-wide output channel tiles
  constexpr int KP = BfLds<D>::KP, VP = BfLds<D>::VP;
  __shared__ BfLds<D> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  int b, h, qb;
  tile_coords(p, b, h, qb);
  const int hk = h / p.group;
  const __bf16* qbase = static_cast<const __bf16*>(p.q) + b * p.qs_b + h * p.qs_h;
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + b * p.ks_b + hk * p.ks_h;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + b * p.vs_b + hk * p.vs_h;

  // Q^T fragments (B operand): lane (r, g) holds query row r of the 16-query
  // tile n, channels 32c + 8g .. +7.
  bf16x8 qf[2][NC];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int row = qb * kBlock + wave * kQW + n * 16 + r;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 v = {0, 0, 0, 0};
      if (row < p.L) v = *reinterpret_cast<const u32x4*>(qbase + row * p.qs_l + c * 32 + g * 8);
      qf[n][c] = __builtin_bit_cast(bf16x8, v);
    }
  }

  float m[2] = {kNegInf, kNegInf};
  float l[2] = {0.f, 0.f};
  f32x4 acc[NJ][2];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nkb = p.nqb;
  const int count = list_count(p, b, h, qb);
  for (int s = 0; s < count; ++s) {
    const int kb = list_entry(p, b, h, qb, s);
    if (kb < 0 || kb > qb || kb >= nkb) continue;  // uniform over the workgroup
    __syncthreads();                                // previous block fully consumed
    // ---- stage K (row-major) ----
    constexpr int KCH = D / 8;  // 16-byte chunks per row
#pragma unroll
    for (int e = tid; e < kBlock * KCH; e += kThreads) {
      const int row = e / KCH, ch = e % KCH;
      const int key = kb * kBlock + row;
      u32x4 v = {0, 0, 0, 0};
      if (key < p.L) v = *reinterpret_cast<const u32x4*>(kbase + key * p.ks_l + ch * 8);
      *reinterpret_cast<u32x4*>(&sm.k[row * KP + ch * 8]) = v;
    }
    // ---- stage V transposed: each item is 8 keys x 8 channels ----
#pragma unroll
    for (int e = tid; e < 16 * KCH; e += kThreads) {
      const int dd = e % KCH, cg = e / KCH;
      const int c = cg >> 2, gg = cg & 3;
      u32x4 rows[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kk = c * 32 + (i < 4 ? 4 * gg + i : 16 + 4 * gg + (i - 4));
        const int key = kb * kBlock + kk;
        rows[i] = u32x4{0, 0, 0, 0};
        if (key < p.L) rows[i] = *reinterpret_cast<const u32x4*>(vbase + key * p.vs_l + dd * 8);
      }
      // rows[i] word w = channels (2w, 2w+1) of key i; out row (channel) 2w+x
      // word q = keys (2q, 2q+1)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x4 lo, hi;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t a0 = rows[2 * q][w], a1 = rows[2 * q + 1][w];
          lo[q] = (a0 & 0xFFFFu) | (a1 << 16);
          hi[q] = (a0 >> 16) | (a1 & 0xFFFF0000u);
        }
        const int ch0 = dd * 8 + 2 * w;
        *reinterpret_cast<u32x4*>(&sm.vt[ch0 * VP + c * 32 + gg * 8]) = lo;
        *reinterpret_cast<u32x4*>(&sm.vt[(ch0 + 1) * VP + c * 32 + gg * 8]) = hi;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T : 8 key tiles x 2 query tiles ----
    f32x4 sc[8][2];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int n = 0; n < 2; ++n) sc[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&sm.k[(t * 16 + r) * KP + c * 32 + g * 8]);
#pragma unroll
        for (int n = 0; n < 2; ++n) sc[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[n][c], sc[t][n], 0, 0, 0);
      }
    }
    // ---- causal mask in the own block ----
    if (kb == qb) {
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int qi = wave * kQW + n * 16 + r;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t * 16 + g * 4 + i > qi) sc[t][n][i] = kNegInf;
      }
    }
    // ---- online softmax ----
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      float mx = kNegInf;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[t][n][i]);
      mx = wave_max16x4(mx);
      const float m_new = fmaxf(m[n], mx);
      const float alpha = __builtin_amdgcn_exp2f((m[n] - m_new) * p.c1);
      const float mc = m_new * p.c1;
      float rs = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][n][i], p.c1, -mc));
          sc[t][n][i] = e;
          rs += e;
        }
      rs = wave_sum16x4(rs);
      l[n] = l[n] * alpha + rs;
      m[n] = m_new;
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j][n] *= alpha;
    }
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8 pf[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const bf16x4 a = __builtin_convertvector(sc[2 * c][n], bf16x4);
        const bf16x4 bq = __builtin_convertvector(sc[2 * c + 1][n], bf16x4);
        pf[n] = bf16x8{a[0], a[1], a[2], a[3], bq[0], bq[1], bq[2], bq[3]};
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&sm.vt[(j * 16 + r) * VP + c * 32 + g * 8]);
#pragma unroll
        for (int n = 0; n < 2; ++n) acc[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[n], acc[j][n], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O = O^T / l, lse = scale*m + ln l ----
  OutT* obase = static_cast<OutT*>(p.o) + b * p.os_b + h * p.os_h;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int row = qb * kBlock + wave * kQW + n * 16 + r;
    if (row >= p.L) continue;
    const float inv = l[n] > 0.f ? 1.f / l[n] : 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) store4<OutT>(obase + row * p.os_l + j * 16 + g * 4, acc[j][n] * inv);
    if (p.lse && g == 0) {
      const float v = l[n] > 0.f ? m[n] * p.scale + __builtin_amdgcn_logf(l[n]) * kLn2 : kNegInf;
      p.lse[(static_cast<int64_t>(b) * p.Hq + h) * p.L + row] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// f32 kernel (D = 64)
// ---------------------------------------------------------------------------

template <int D>
struct F32Lds {
  static constexpr int P = D + 4;
  float k[kBlock * P];
  float v[kBlock * P];
};

template <int D>
__global__ __launch_bounds__(kThreads) void prefill_f32_kernel(PrefillParams p) {
  constexpr int NC = D / 4;
  constexpr int NJ = D / 16;
  constexpr int P = F32Lds<D>::P;
  __shared__ F32Lds<D> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  int b, h, qb;
  tile_coords(p, b, h, qb);
  const int hk = h / p.group;
  const float* qbase = static_cast<const float*>(p.q) + b * p.qs_b + h * p.qs_h;
  const float* kbase = static_cast<const float*>(p.k) + b * p.ks_b + hk * p.ks_h;
  const float* vbase = static_cast<const float*>(p.v) + b * p.vs_b + hk * p.vs_h;

  // B operand of v_mfma_f32_16x16x4f32: lane (r, g) holds Q[row r][4c + g]
  float qf[2][NC];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int row = qb * kBlock + wave * kQW + n * 16 + r;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[n][c] = row < p.L ? qbase[row * p.qs_l + c * 4 + g] : 0.f;
  }
  float m[2] = {kNegInf, kNegInf};
  float l[2] = {0.f, 0.f};
  f32x4 acc[NJ][2];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nkb = p.nqb;
  const int count = list_count(p, b, h, qb);
  for (int s = 0; s < count; ++s) {
    const int kb = list_entry(p, b, h, qb, s);
    if (kb < 0 || kb > qb || kb >= nkb) continue;
    __syncthreads();
    constexpr int CH = D / 4;
#pragma unroll
    for (int e = tid; e < kBlock * CH; e += kThreads) {
      const int row = e / CH, ch = e % CH;
      const int key = kb * kBlock + row;
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (key < p.L) {
        kv = *reinterpret_cast<const f32x4*>(kbase + key * p.ks_l + ch * 4);
        vv = *reinterpret_cast<const f32x4*>(vbase + key * p.vs_l + ch * 4);
      }
      *reinterpret_cast<f32x4*>(&sm.k[row * P + ch * 4]) = kv;
      *reinterpret_cast<f32x4*>(&sm.v[row * P + ch * 4]) = vv;
    }
    __syncthreads();
    f32x4 sc[8][2];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int n = 0; n < 2; ++n) sc[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float kf = sm.k[(t * 16 + r) * P + c * 4 + g];
#pragma unroll
        for (int n = 0; n < 2; ++n) sc[t][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf, qf[n][c], sc[t][n], 0, 0, 0);
      }
    if (kb == qb) {
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int qi = wave * kQW + n * 16 + r;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t * 16 + g * 4 + i > qi) sc[t][n][i] = kNegInf;
      }
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      float mx = kNegInf;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[t][n][i]);
      mx = wave_max16x4(mx);
      const float m_new = fmaxf(m[n], mx);
      const float alpha = __builtin_amdgcn_exp2f((m[n] - m_new) * p.c1);
      const float mc = m_new * p.c1;
      float rs = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][n][i], p.c1, -mc));
          sc[t][n][i] = e;
          rs += e;
        }
      rs = wave_sum16x4(rs);
      l[n] = l[n] * alpha + rs;
      m[n] = m_new;
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j][n] *= alpha;
    }
    // O^T += V^T P^T, 4 keys per instruction: lane group g supplies key
    // t*16 + 4g + i, which is exactly the S^T element it holds.
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const float vf = sm.v[(t * 16 + g * 4 + i) * P + j * 16 + r];
#pragma unroll
          for (int n = 0; n < 2; ++n) acc[j][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf, sc[t][n][i], acc[j][n], 0, 0, 0);
        }
  }
  float* obase = static_cast<float*>(p.o) + b * p.os_b + h * p.os_h;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int row = qb * kBlock + wave * kQW + n * 16 + r;
    if (row >= p.L) continue;
    const float inv = l[n] > 0.f ? 1.f / l[n] : 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) store4<float>(obase + row * p.os_l + j * 16 + g * 4, acc[j][n] * inv);
    if (p.lse && g == 0) {
      const float v = l[n] > 0.f ? m[n] * p.scale + __builtin_amdgcn_logf(l[n]) * kLn2 : kNegInf;
      p.lse[(static_cast<int64_t>(b) * p.Hq + h) * p.L + row] = v;
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int dtype, int dqk, int dv, bool out_f32, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.nqb) * p.B * p.Hq);
  const dim3 block(kThreads);
  if (dtype == 0) {
    if (dqk == 64 && dv == 64) return launch_kernel(prefill_f32_kernel<64>, grid, block, 0, stream, p);
    return hipErrorNotSupported;
  }
  if (dqk == 128 && dv == 128)
    return out_f32 ? launch_kernel(prefill_bf16_kernel<128, float>, grid, block, 0, stream, p)
                   : launch_kernel(prefill_bf16_kernel<128, __bf16>, grid, block, 0, stream, p);
  if (dqk == 64 && dv == 64)
    return out_f32 ? launch_kernel(prefill_bf16_kernel<64, float>, grid, block, 0, stream, p)
                   : launch_kernel(prefill_bf16_kernel<64, __bf16>, grid, block, 0, stream, p);
  return hipErrorNotSupported;
}

}  // namespace ssa
