// Block-sparse causal attention prefill, fp32 path (D = 64), and the entry
// that dispatches every prefill shape.
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
// fp32 kernel: 4 waves, 32 queries each, on v_mfma_f32_16x16x4f32.  The wave
// computes S^T = K Q^T per 16x16 tile (A = K rows from LDS, B = Q^T from
// registers), so each lane owns one query column and 4 keys of it.  Each
// instruction contracts over 4 keys, so for O^T = V^T P^T the S^T elements a
// lane holds are exactly its P^T operand and V is read row-major from LDS.
//
// bf16 shapes: 128/128 runs the kernel of prefill_d128.hip,
// 64/64 and the latent-shared 576/512 the streaming kernel of
// prefill_wide.hip.
#include "common.hpp"

namespace ssa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 128;  // tokens per block == queries per tile
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

__device__ __forceinline__ void store4(float* dst, f32x4 v) { *reinterpret_cast<f32x4*>(dst) = v; }

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
    for (int j = 0; j < NJ; ++j) store4(obase + row * p.os_l + j * 16 + g * 4, acc[j][n] * inv);
    if (p.lse && g == 0) {
      const float v = l[n] > 0.f ? m[n] * p.scale + __builtin_amdgcn_logf(l[n]) * kLn2 : kNegInf;
      p.lse[(static_cast<int64_t>(b) * p.Hq + h) * p.L + row] = v;
    }
  }
}


}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int dtype, int dqk, int dv, bool out_f32, hipStream_t stream) {
  if (dtype == 0) {
    if (dqk != 64 || dv != 64) return hipErrorNotSupported;
    const dim3 grid(static_cast<unsigned>(p.nqb) * p.B * p.Hq);
    return launch_kernel(prefill_f32_kernel<64>, grid, dim3(kThreads), 0, stream, p);
  }
  if (prefill_d128_supports(p, dqk, dv)) return launch_prefill_d128(p, out_f32, stream);
  return launch_prefill_wide(p, dqk, dv, out_f32, stream);
}

}  // namespace ssa
