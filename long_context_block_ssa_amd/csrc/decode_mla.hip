// SSA decode at the latent-shared (MLA-like) shape on gfx950: Hq query heads
// share one key/value latent of width 576 per cached token, the value being
// its first 512 channels.  LoZA rewrites LongCat's MLA layers (QbitAI report
// on LongCat LoZA); a decode step reads the window of the new token's block:
// block 0 and the 7 most recent blocks (same report, sparse-window
// paragraph), the last one partial.
//
// Here the per-sequence work is a dense contraction -- (16 heads x 576) by
// (576 x 1024 keys), then (16 heads x 1024) by (1024 x 512) -- so it runs on
// the matrix cores:
//   - one workgroup per (sequence, 16 query heads), 4 waves; wave w takes
//     window slots w, w+4, ...;
//   - each wave streams its blocks in 16-key steps through a private,
//     double-buffered LDS slab filled by global_load_lds_dwordx4;
//   - S^T (16 keys x 16 heads) on v_mfma_f32_16x16x32_bf16; the online
//     softmax keeps one (m, l) per head; O^T += V^T P^T on
//     v_mfma_f32_16x16x16_bf16, whose V^T operand (4 keys of one channel per
//     lane) is one ds_read_b64_tr_b16 from the row-major latent slab;
//   - the 4 wave partials are merged in LDS: M = max m_w,
//     o = sum o_w e^(m_w - M) / sum l_w e^(m_w - M).
#include "common.hpp"

namespace ssa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define SSA_LDS __attribute__((address_space(3)))
#define SSA_GLB __attribute__((address_space(1)))

constexpr int kDqk = 576, kDv = 512;
constexpr int kHeads = 16;     // query heads per workgroup (one MFMA tile)
constexpr int kMWaves = 4;
constexpr int kStep = 16;      // keys per step
constexpr int kUK = kDqk / 8 + 1;                       // K row pitch in 16-byte units (one pad)
constexpr int kUV = kDv / 8 + 1;                        // separate V row pitch
constexpr int kSlabK = (kStep * kUK + 63) / 64 * 64;    // whole 1 KB wave writes
constexpr int kSlabV = (kStep * kUV + 63) / 64 * 64;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float xlane_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float xlane_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// Stage 16 cache rows (keys key0 .. key0+15 of one page) into a slab with row
// pitch U units; lanes past the slab's rows load row 0 (their units are pad).
// Slots at or past the sequence end (key >= kend) are replaced by the last
// valid one: their scores are masked, and a masked zero weight times finite
// data stays zero inside the MFMA (times NaN it would not).
template <int D, int U, int UNITS>
__device__ __forceinline__ void stage16(SSA_LDS u32x4* slab, const __bf16* page_base, int64_t slot_stride, int key0,
                                        int kend, int lane) {
#pragma unroll
  for (int i = 0; i < UNITS / 64; ++i) {
    const int pidx = i * 64 + lane;
    int row = pidx / U, pos = pidx - row * U;
    if (row >= kStep) {
      row = 0;
      pos = 0;
    }
    const int unit = pos < D / 8 ? pos : 0;
    const int key = min(key0 + row, kend - 1);
    const __bf16* src = page_base + static_cast<int64_t>(key) * slot_stride + unit * 8;
    __builtin_amdgcn_global_load_lds((const SSA_GLB void*)(src), (SSA_LDS void*)(slab + i * 64), 16, 0, 0);
  }
}

template <bool SHARED>
__global__ __launch_bounds__(kMWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mla_kernel(DecodeParams p) {
  constexpr int NBUF = SHARED ? 2 : 1;
  constexpr int SLAB = kSlabK + (SHARED ? 0 : kSlabV);
  constexpr int PER_WAVE = NBUF * SLAB;  // units
  constexpr int NC = kDqk / 32;
  constexpr int NJ = kDv / 16;
  extern __shared__ u32x4 lds_dyn[];
  SSA_LDS u32x4* lds = (SSA_LDS u32x4*)(lds_dyn);
  __shared__ int bad;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  // sequence fastest: consecutive workgroups go to consecutive XCDs, so with
  // B a multiple of 8 every head group of a sequence runs on one XCD and the
  // sequence's latent pages are fetched into that XCD's L2 once
  const int b = blockIdx.x % p.B, h0 = (blockIdx.x / p.B) * kHeads;
  const int n = p.seq_lens[b];
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();

  const bool len_ok = n >= 1 && n <= p.max_blocks * 128;
  int qb = 0, g_end = 0, l_begin = 0, cntw = 0;
  if (len_ok) {
    qb = (n - 1) / 128;
    g_end = min(p.n_global, qb + 1);
    l_begin = max(g_end, qb - p.n_local + 1);
    cntw = g_end + (qb - l_begin + 1);
  } else if (threadIdx.x == 0) {
    bad = 1;
  }
  // window pages, validated and kept in LDS: no global reads inside the step
  // loop, whose waits would also drain the direct-to-LDS prefetch
  __shared__ int32_t pages[16];
  if (static_cast<int>(threadIdx.x) < cntw) {
    const int slot = threadIdx.x;
    const int blk = slot < g_end ? slot : l_begin + (slot - g_end);
    const int page = p.block_table[b * p.bt_stride + blk];
    pages[slot] = page;
    if (page < 0 || page >= p.num_pages) bad = 1;
  }
  __syncthreads();
  const bool all_bad = bad != 0;

  // Q^T fragments (B operand): lane (r, g) = head h0 + r, channels 32c + 8g .. +7
  bf16x8 qf[NC];
  const __bf16* qrow = static_cast<const __bf16*>(p.q) + b * p.qs_b + (h0 + r) * p.qs_h;
#pragma unroll
  for (int c = 0; c < NC; ++c) qf[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + c * 32 + g * 8));

  float m = kNegInf, l = 0.f;
  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  SSA_LDS u32x4* mine = lds + wave * PER_WAVE;
  // the steps of this wave: slots wave, wave+4, ...; 8 steps of 16 keys each
  int nsteps = 0;
  for (int slot = wave; slot < cntw; slot += kMWaves) nsteps += 8;
  if (all_bad) nsteps = 0;
  auto step_src = [&](int st, const __bf16*& kpg, const __bf16*& vpg, int& key0, int& valid) {
    const int slot = wave + (st >> 3) * kMWaves;
    const int blk = slot < g_end ? slot : l_begin + (slot - g_end);
    const int page = pages[slot];
    kpg = static_cast<const __bf16*>(p.k) + static_cast<int64_t>(page) * p.ks_p;
    vpg = static_cast<const __bf16*>(p.v) + static_cast<int64_t>(page) * p.vs_p;
    key0 = (st & 7) * kStep;
    valid = min(128, n - blk * 128) - key0;  // keys of this step that exist (may be <= 0)
  };
  auto issue = [&](int st) {
    const __bf16 *kpg, *vpg;
    int key0, valid;
    step_src(st, kpg, vpg, key0, valid);
    if (valid <= 0) return;
    SSA_LDS u32x4* slab = mine + (st % NBUF) * SLAB;
    stage16<kDqk, kUK, kSlabK>(slab, kpg, p.ks_s, key0, key0 + valid, lane);
    if constexpr (!SHARED) stage16<kDv, kUV, kSlabV>(slab + kSlabK, vpg, p.vs_s, key0, key0 + valid, lane);
  };

  if (NBUF == 2 && nsteps > 0) issue(0);
  for (int st = 0; st < nsteps; ++st) {
    if (NBUF == 2) {
      if (st + 1 < nsteps) issue(st + 1);
    } else {
      issue(st);
    }
    __builtin_amdgcn_s_waitcnt(0);
    const __bf16 *kpg, *vpg;
    int key0, valid;
    step_src(st, kpg, vpg, key0, valid);
    if (valid <= 0) continue;
    const SSA_LDS u32x4* kslab = mine + (st % NBUF) * SLAB;
    const SSA_LDS u32x4* vslab = SHARED ? kslab : kslab + kSlabK;
    constexpr int UV = SHARED ? kUK : kUV;
    // S^T (16 keys x 16 heads)
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bf16x8 kf = __builtin_bit_cast(bf16x8, kslab[r * kUK + c * 4 + g]);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], sc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (g * 4 + i >= valid) sc[i] = kNegInf;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = xlane_max(mx);
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f((m - m_new) * p.c1);
    const float mc = m_new * p.c1;
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], p.c1, -mc));
      rs += sc[i];
    }
    l = l * alpha + xlane_sum(rs);
    m = m_new;
    const bf16x4 pb = __builtin_convertvector(sc, bf16x4);
    // O^T (512 x 16 heads) += V^T (512 x 16 keys) P^T (16 keys x 16 heads)
    const int krow = 4 * g + (r >> 2);
    const int ch_off = 4 * (r & 3);
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
      acc[jt] *= alpha;
      const int ch = jt * 16 + ch_off;
      const SSA_LDS char* a = (const SSA_LDS char*)(vslab + krow * UV + (ch >> 3)) + (ch & 7) * 2;
      const bf16x4 vf = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SSA_LDS bf16x4*)a);
      acc[jt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vf), __builtin_bit_cast(s16x4, pb),
                                                           acc[jt], 0, 0, 0);
    }
  }

  // merge the wave partials: each wave writes o^T [16 heads][512], m, l
  __syncthreads();  // every wave is done with its slabs
  float* part = (float*)(lds_dyn);  // reuse the staging memory
  constexpr int PSTRIDE = kHeads * kDv + 2 * kHeads;
  float* mine_p = part + wave * PSTRIDE;
#pragma unroll
  for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
    for (int i = 0; i < 4; ++i) mine_p[r * kDv + jt * 16 + g * 4 + i] = acc[jt][i];
  if (g == 0) {
    mine_p[kHeads * kDv + r] = m;
    mine_p[kHeads * kDv + kHeads + r] = l;
  }
  __syncthreads();
  const float nan = __builtin_nanf("");
  for (int e = threadIdx.x; e < kHeads * kDv; e += blockDim.x) {
    const int hh = e / kDv, d = e % kDv;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kMWaves; ++w) M = fmaxf(M, part[w * PSTRIDE + kHeads * kDv + hh]);
    float o = 0.f, ls = 0.f;
#pragma unroll
    for (int w = 0; w < kMWaves; ++w) {
      const float mw = part[w * PSTRIDE + kHeads * kDv + hh];
      const float sc = mw == kNegInf ? 0.f : __builtin_amdgcn_exp2f((mw - M) * p.c1);
      o = __builtin_fmaf(part[w * PSTRIDE + hh * kDv + d], sc, o);
      ls = __builtin_fmaf(part[w * PSTRIDE + kHeads * kDv + kHeads + hh], sc, ls);
    }
    __bf16* op = static_cast<__bf16*>(p.o) + b * p.os_b + (h0 + hh) * p.os_h;
    op[d] = static_cast<__bf16>(all_bad ? nan : o / ls);
    if (d == 0 && p.lse)
      p.lse[static_cast<int64_t>(b) * p.Hq + h0 + hh] = all_bad ? nan : M * p.scale + __builtin_amdgcn_logf(ls) * kLn2;
  }
}

template <bool SHARED>
hipError_t launch_mla(const DecodeParams& p, hipStream_t stream) {
  constexpr int NBUF = SHARED ? 2 : 1;
  constexpr int SLAB = kSlabK + (SHARED ? 0 : kSlabV);
  const size_t stage_bytes = sizeof(u32x4) * kMWaves * NBUF * SLAB;
  const size_t part_bytes = sizeof(float) * kMWaves * (kHeads * kDv + 2 * kHeads);
  const size_t lds = stage_bytes > part_bytes ? stage_bytes : part_bytes;
  auto kern = decode_mla_kernel<SHARED>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>(p.B) * (p.Hq / kHeads));
  return launch_kernel(kern, grid, dim3(kMWaves * 64), lds, stream, p);
}

}  // namespace

hipError_t launch_decode_mla(const DecodeParams& p, hipStream_t stream) {
  if (p.Hkv != 1 || p.Hq % kHeads != 0) return hipErrorNotSupported;
  const bool shared = p.v == p.k && p.vs_p == p.ks_p && p.vs_s == p.ks_s;
  return shared ? launch_mla<true>(p, stream) : launch_mla<false>(p, stream);
}

}  // namespace ssa
