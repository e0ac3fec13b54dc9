// Block-sparse causal attention prefill for wide heads on gfx950: the
// latent-shared (MLA-like) shape Dqk = 576, Dv = 512, where every query head
// reads one shared latent row per key and the value is its first 512
// channels.  LoZA rewrites LongCat's MLA attention (QbitAI report on LongCat
// LoZA); within the listed key blocks this is the masked softmax of equation
// (2) of the "LoZA: ZigZag sparse attention" page, section 2.1, causal in
// the own block (section 2.2.1), evaluated as an exact online softmax.
//
// One workgroup = one 128-query block of one head: 4 waves x 32 queries,
// one wave per SIMD (the 32 x 512 fp32 output accumulator alone is 256
// registers per lane).  Keys stream in 64-key stages through two LDS slots:
//   - staging uses global_load_lds_dwordx4 (global -> LDS, no registers);
//     rows are padded by one 16-byte unit so that the 16 lanes reading a
//     fragment column hit 16 distinct bank groups;
//   - S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (A = K rows, ds_read_b128);
//   - O^T = V^T P^T: the V^T operand is read from the row-major K/V slab with
//     ds_read_b64_tr_b16, which hands each lane 4 keys of one channel, so the
//     latent is staged once and serves as both K and V;
//   - the running max is refreshed lazily: the accumulator is rescaled only
//     when the max grows by more than 2^8, which is exact because the final
//     normalisation uses the same reference max.
#include "common.hpp"

namespace ssa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define SSA_LDS __attribute__((address_space(3)))
#define SSA_GLB __attribute__((address_space(1)))

constexpr int kBlk = 128;
constexpr int kStageKeys = 64;
constexpr int kNQ = 1;                 // 16-query tiles per wave
constexpr int kRows = 16 * kNQ;        // queries per wave
constexpr int kWWaves = kBlk / kRows;  // waves per workgroup (one query block)
constexpr int kWThreads = kWWaves * 64;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;  // log2 headroom before the accumulator is rescaled

__device__ __forceinline__ float xlane_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float xlane_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
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

// LDS geometry of one stage slot, in 16-byte units.
template <int DQK, int DV, bool SHARED>
struct WideGeom {
  static constexpr int UK = DQK / 8 + 1;  // K row pitch (one pad unit)
  static constexpr int UV = DV / 8 + 1;   // V row pitch when V is staged apart
  static constexpr int KUNITS = kStageKeys * UK;
  static constexpr int VUNITS = SHARED ? 0 : kStageKeys * UV;
  static constexpr int SLOT = KUNITS + VUNITS;  // multiple of 64 units
  static constexpr int NSLOTS = 2 * SLOT * 16 <= 160 * 1024 ? 2 : 1;
  static_assert(KUNITS % 64 == 0 && VUNITS % 64 == 0, "slab = whole 1 KB wave writes");
};

// Stage `rows0 .. rows0+63` of a [L, D] operand into an LDS slab with row
// pitch U units.  The wave issues instruction i for linear units
// [ (w + i*NW) * 64, +64 ); a lane on the pad unit loads unit 0 of its row.
// Keys at or past L are clamped to row L-1 (finite data, masked later).
template <int D, int U>
__device__ __forceinline__ void stage_rows(SSA_LDS u32x4* slab, const __bf16* base, int64_t stride_l, int key0,
                                           int L, int wave, int lane) {
  constexpr int TOTAL = kStageKeys * U / 64;  // wave-instructions for the slab
#pragma unroll 4
  for (int i = wave; i < TOTAL; i += kWWaves) {
    const int pidx = i * 64 + lane;
    const int row = pidx / U, pos = pidx - row * U;
    const int unit = pos < D / 8 ? pos : 0;
    const int key = min(key0 + row, L - 1);
    const __bf16* src = base + static_cast<int64_t>(key) * stride_l + unit * 8;
    __builtin_amdgcn_global_load_lds((const SSA_GLB void*)(src), (SSA_LDS void*)(slab + i * 64), 16, 0, 0);
  }
}

template <int DQK, int DV, bool SHARED, typename OutT>
__global__ __launch_bounds__(kWThreads) __attribute__((amdgpu_waves_per_eu(kWWaves / 4, kWWaves / 4)))
void prefill_wide_kernel(PrefillParams p) {
  using G = WideGeom<DQK, DV, SHARED>;
  constexpr int NC = DQK / 32;  // 32-channel contraction chunks
  constexpr int NJ = DV / 16;   // 16-channel output tiles
  // two distinct LDS objects, so the compiler can tell a read of one slot from
  // the direct-to-LDS writes into the other and keep the prefetch in flight
  __shared__ u32x4 slot_a[G::SLOT];
  __shared__ u32x4 slot_b[G::NSLOTS == 2 ? G::SLOT : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  // tile order: query blocks last to first, then batch, heads fastest, so the
  // workgroups in flight share their key blocks through L2
  const int bh_count = p.B * p.Hq;
  const int qb = p.nqb - 1 - static_cast<int>(blockIdx.x) / bh_count;
  const int bh = static_cast<int>(blockIdx.x) % bh_count;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int hk = h / p.group;
  const __bf16* qbase = static_cast<const __bf16*>(p.q) + b * p.qs_b + h * p.qs_h;
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + b * p.ks_b + hk * p.ks_h;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + b * p.vs_b + hk * p.vs_h;

  // block list of this query block, copied to LDS once: a global read inside
  // the stage loop would make the wait for it also wait for the in-flight
  // direct-to-LDS prefetch (vector-memory counters drain in order)
  __shared__ int32_t blist[64];
  int count;
  if (p.dense) {
    count = qb + 1;
  } else {
    count = min(p.cnt[b * p.cnt_sb + h * p.cnt_sh + qb], p.W);
    const int32_t* list = p.idx + b * p.idx_sb + h * p.idx_sh + static_cast<int64_t>(qb) * p.W;
    if (tid < count) blist[tid] = list[tid];
    __syncthreads();
  }
  auto block_of = [&](int s) -> int {  // -1: skip
    const int kb = p.dense ? qb - s : blist[s];
    return (kb < 0 || kb > qb || kb >= p.nqb) ? -1 : kb;
  };
  const int nst = 2 * count;

  // Q^T fragments (B operand): lane (r, g) holds query row r of tile n,
  // channels 32c + 8g .. +7
  bf16x8 qf[kNQ][NC];
#pragma unroll
  for (int n = 0; n < kNQ; ++n) {
    const int row = qb * kBlk + wave * kRows + n * 16 + r;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 v = {0, 0, 0, 0};
      if (row < p.L) v = *reinterpret_cast<const u32x4*>(qbase + row * p.qs_l + c * 32 + g * 8);
      qf[n][c] = __builtin_bit_cast(bf16x8, v);
    }
  }
  float m[kNQ], l[kNQ];
#pragma unroll
  for (int n = 0; n < kNQ; ++n) {
    m[n] = kNegInf;
    l[n] = 0.f;
  }
  f32x4 acc[NJ][kNQ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int n = 0; n < kNQ; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int NS = G::NSLOTS;
  auto issue = [&](int s, u32x4* slot_generic) {
    const int kb = block_of(s >> 1);
    if (kb < 0) return;
    SSA_LDS u32x4* slot = (SSA_LDS u32x4*)(slot_generic);
    const int key0 = kb * kBlk + (s & 1) * kStageKeys;
    stage_rows<DQK, G::UK>(slot, kbase, p.ks_l, key0, p.L, wave, lane);
    if constexpr (!SHARED) stage_rows<DV, G::UV>(slot + G::KUNITS, vbase, p.vs_l, key0, p.L, wave, lane);
  };

  // one stage: keys (s>>1)*128 + (s&1)*64 .. +63, staged in `cur`
  auto compute = [&](int s, const u32x4* cur) {
    const int kb = block_of(s >> 1);
    const int half = s & 1;
    const bool work = kb >= 0 && !(kb == qb && half * kStageKeys > wave * kRows + kRows - 1);
    if (!work) return;
    const SSA_LDS u32x4* kslab = (const SSA_LDS u32x4*)(cur);
    const SSA_LDS u32x4* vslab = SHARED ? kslab : kslab + G::KUNITS;
    constexpr int UV = SHARED ? G::UK : G::UV;
    f32x4 sc[4][kNQ];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int n = 0; n < kNQ; ++n) sc[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, kslab[(t * 16 + r) * G::UK + c * 4 + g]);
#pragma unroll
        for (int n = 0; n < kNQ; ++n)
          sc[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[n][c], sc[t][n], 0, 0, 0);
      }
    }
    const bool valid_all = (kb + 1) * kBlk <= p.L && kb < qb;
    if (!valid_all) {
#pragma unroll
      for (int n = 0; n < kNQ; ++n) {
        const int qi = wave * kRows + n * 16 + r;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kk = half * kStageKeys + t * 16 + g * 4 + i;
            const bool dead = (kb == qb && kk > qi) || kb * kBlk + kk >= p.L;
            if (dead) sc[t][n][i] = kNegInf;
          }
      }
    }
#pragma unroll
    for (int n = 0; n < kNQ; ++n) {
      float mx = kNegInf;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[t][n][i]);
      mx = xlane_max(mx);
      const float m_new = fmaxf(m[n], mx);
      // lazy refresh of the reference max
      const bool refresh = (m_new - m[n]) * p.c1 > kLazy;
      const float m_use = refresh ? m_new : m[n];
      if (__builtin_amdgcn_ballot_w64(refresh)) {
        const float alpha = __builtin_amdgcn_exp2f((m[n] - m_use) * p.c1);
        l[n] *= alpha;
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[j][n] *= alpha;
      }
      m[n] = m_use;
      const float mc = m_use * p.c1;
      float rs = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][n][i], p.c1, -mc));
          sc[t][n][i] = e;
          rs += e;
        }
      l[n] += xlane_sum(rs);
    }
    // O^T += V^T P^T over two 32-key chunks
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x8 pf[kNQ];
#pragma unroll
      for (int n = 0; n < kNQ; ++n) {
        const bf16x4 a = __builtin_convertvector(sc[2 * c][n], bf16x4);
        const bf16x4 bq = __builtin_convertvector(sc[2 * c + 1][n], bf16x4);
        pf[n] = bf16x8{a[0], a[1], a[2], a[3], bq[0], bq[1], bq[2], bq[3]};
      }
      // transposed reads: lane j of group g points at key c*32 + h2*16 +
      // 4g + j/4, channels 16*jt + 4*(j%4) .. +3; it receives channel
      // 16*jt + j of keys c*32 + h2*16 + 4g .. +3
      const int krow = c * 32 + 4 * g + (r >> 2);
      const int ch_off = 4 * (r & 3);
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) {
        const int ch = jt * 16 + ch_off;
        const SSA_LDS char* base0 = (const SSA_LDS char*)(vslab + krow * UV + (ch >> 3)) + (ch & 7) * 2;
        const SSA_LDS char* base1 = base0 + 16 * UV * 16;
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SSA_LDS bf16x4*)base0);
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SSA_LDS bf16x4*)base1);
        const bf16x8 vf = bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int n = 0; n < kNQ; ++n)
          acc[jt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[n], acc[jt][n], 0, 0, 0);
      }
    }
  };

  if constexpr (NS == 2) {
    if (nst > 0) issue(0, slot_a);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int s = 0; s < nst; s += 2) {
      if (s + 1 < nst) issue(s + 1, slot_b);
      compute(s, slot_a);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (s + 1 >= nst) break;
      if (s + 2 < nst) issue(s + 2, slot_a);
      compute(s + 1, slot_b);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  } else {
    for (int s = 0; s < nst; ++s) {
      issue(s, slot_a);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      compute(s, slot_a);
      __syncthreads();
    }
  }

  OutT* obase = static_cast<OutT*>(p.o) + b * p.os_b + h * p.os_h;
#pragma unroll
  for (int n = 0; n < kNQ; ++n) {
    const int row = qb * kBlk + wave * kRows + n * 16 + r;
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

template <int DQK, int DV, bool SHARED, typename OutT>
hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.nqb) * p.B * p.Hq);
  return launch_kernel(prefill_wide_kernel<DQK, DV, SHARED, OutT>, grid, dim3(kWThreads), 0, stream, p);
}

}  // namespace

hipError_t launch_prefill_wide(const PrefillParams& p, int dqk, int dv, bool out_f32, hipStream_t stream) {
  if (dqk != 576 || dv != 512) return hipErrorNotSupported;
  const bool shared = p.v == p.k && p.vs_b == p.ks_b && p.vs_l == p.ks_l && p.vs_h == p.ks_h;
  if (shared)
    return out_f32 ? launch_one<576, 512, true, float>(p, stream) : launch_one<576, 512, true, __bf16>(p, stream);
  return out_f32 ? launch_one<576, 512, false, float>(p, stream) : launch_one<576, 512, false, __bf16>(p, stream);
}

}  // namespace ssa
