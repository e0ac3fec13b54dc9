// SSA decode at the latent-shared (MLA-like) shape on gfx950: Hq query heads
// share one key/value latent of width 576 per cached token, the value being
// its first 512 channels.  LoZA rewrites LongCat's MLA layers (QbitAI report
// on LongCat LoZA); a decode step reads the window of the new token's block:
// block 0 and the 7 most recent blocks (same report, sparse-window
// paragraph), the last one partial.
//
// The per-sequence work is a dense contraction -- (16 heads x 576) by
// (576 x 1024 keys), then (16 heads x 1024) by (1024 x 512) -- on the matrix
// cores.  A sequence's window is only ~1 MB and one CU moves only ~50-100
// GB/s from memory, so the window is spread over all CUs and the pieces are
// merged afterwards:
//   - partial kernel: one workgroup per (sequence, 16 or 32 query heads,
//     window block); its 8 waves split the channels: wave w owns value
//     channels 64w .. 64w+63 and, for the scores, those plus 8 of the 64 rope
//     channels.  A wave loads its share of all 8 16-key steps of the block
//     into registers at once (16 keys x 72 channels per step), so the whole
//     block is in flight from the start;
//   - partial S^T (16 keys x 16 heads) over the wave's channels on
//     v_mfma_f32_16x16x32_bf16 (+ one 16x16x16 for the rope channels),
//     straight from the loaded registers; the 8 partials go through LDS and
//     wave w sums those of step w in a fixed order, so the scores do not
//     depend on which wave sums them; a block holds only 128 keys, so the
//     softmax is exact in two passes (block max, then P) with no rescale;
//   - the wave's value tile goes to a wave-private LDS tile from which
//     ds_read_b64_tr_b16 hands the V^T operand (4 keys of one channel per
//     lane) of O^T += V^T P^T on v_mfma_f32_16x16x16_bf16;
//   - each wave writes its 64 channels of the block's (o, m, l) per head, in
//     fp32, to the workspace: no merge of output tiles inside the workgroup;
//   - merge kernel: one workgroup per (sequence, head) combines the blocks:
//     M = max m_t, o = sum o_t e^(m_t - M) / sum l_t e^(m_t - M), the exact
//     merge of max-subtracted softmax pieces (CSA/HCA tutorial page, section
//     7.1).  The kernel boundary orders the partials' writes before the
//     merge's reads on every XCD.
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
constexpr int kHeads = 16;             // query heads per workgroup (one MFMA tile)
constexpr int kMWaves = 8;             // channel eighths
constexpr int kStep = 16;              // keys per step
constexpr int kSteps = 128 / kStep;    // steps per block
constexpr int kWaveCh = kDv / kMWaves;                 // 64 value channels per wave
constexpr int kRopeCh = (kDqk - kDv) / kMWaves;        // 8 rope channels per wave
constexpr int kGroups = kWaveCh / 32;                  // 32-channel groups per wave
constexpr int kMaxW = 16;              // window slots the merge kernel handles
constexpr int kPart = kDv + 4;         // workspace floats per (sequence, head, window slot): o, m, l, pad
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.6931471805599453f;

// Value tile layout (unit = 16 bytes = 8 channels of one key): unit u of key
// row r sits in 1 KB group u/4 at position 4r + ((u mod 4) ^ swz(r)).  The
// 16-byte writes of one group are one contiguous 1 KB, and the swizzle puts
// the 8-byte transposed reads of lanes 0-31 on distinct banks.
__device__ __forceinline__ int swz(int row) { return ((row >> 2) & 1) << 1; }

__device__ __forceinline__ float xlane_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float xlane_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// Workgroup barrier for LDS traffic only.  __syncthreads() would also wait
// for every outstanding global load, i.e. for the prefetched steps.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The window of a decode row of length n: cntw slots, slot t holding block
// block(t); cntw = 0 for a length outside [1, max_blocks * 128].
struct DecodeWindow {
  int cntw = 0, g_end = 0, l_begin = 0;
  __device__ DecodeWindow(const DecodeParams& p, int n) {
    if (n >= 1 && n <= p.max_blocks * 128) {
      const int qb = (n - 1) / 128;
      g_end = min(p.n_global, qb + 1);
      l_begin = max(g_end, qb - p.n_local + 1);
      cntw = g_end + (qb - l_begin + 1);
    }
  }
  __device__ int block(int t) const { return t < g_end ? t : l_begin + (t - g_end); }
};

// Global-memory vector load (a flat load would also count against the LDS
// wait counter and make every LDS barrier wait for the prefetched steps).
template <typename T>
__device__ __forceinline__ T ldg(const __bf16* ptr) {
  return *(const SSA_GLB T*)(ptr);
}
// the latent block, read as a non-temporal stream (its other head groups
// read it at about the same time)
template <typename T>
__device__ __forceinline__ T ldg_nt(const __bf16* ptr) {
  return __builtin_nontemporal_load((const SSA_GLB T*)(ptr));
}

// Partial kernel: grid (B * W * Hq/(16 HG)), 8 waves.  Each wave owns 64
// value channels and 8 of the 64 rope channels, and applies them to HG tiles
// of 16 heads, so a workgroup serves 16 HG heads from one read of the block.
// SHARED: the value is the first 512 channels of the latent row (one load
// serves both).
//
// A block holds only 128 keys = 8 steps of 16, so the softmax takes two
// exact passes instead of an online rescale, and its vector work is split by
// step rather than repeated in every wave:
//   1. each wave computes the partial S^T of all 8 steps over its channels;
//   2. wave w sums the 8 partials of step w (a fixed order, so every step's
//      scores are the same whoever sums them), masks them and publishes the
//      step's max per head;
//   3. wave w forms P of step w against the block max and publishes it (bf16)
//      with its share of the row sum;
//   4. every wave reads P of all steps and accumulates O^T = V^T P^T over its
//      64 channels.
// No accumulator is ever rescaled.
template <bool SHARED, int HG>
__global__ __launch_bounds__(kMWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_mla_partial_kernel(DecodeParams p) {
  static_assert(kSteps == kMWaves, "one step per wave in the softmax");
  constexpr int NJ = kWaveCh / 16;  // 16-channel output tiles per wave
  // dynamic LDS: partial scores sx [kSteps][HG][kMWaves][64] f32x4, value
  // tiles [kMWaves][kGroups * 64] u32x4, P pb [kSteps][HG][64] bf16x4, step
  // maxima mx [kSteps][HG][16] and row-sum parts ls [kSteps][HG][16] floats
  extern __shared__ f32x4 lds_dyn[];
  f32x4* sx = lds_dyn;
  SSA_LDS u32x4* vtile = (SSA_LDS u32x4*)(sx + kSteps * HG * kMWaves * 64);
  bf16x4* pbuf = reinterpret_cast<bf16x4*>(sx + kSteps * HG * kMWaves * 64 + kMWaves * kGroups * 64);
  float* mxs = reinterpret_cast<float*>(pbuf + kSteps * HG * 64);
  float* lsp = mxs + kSteps * HG * kHeads;

  const int W = p.n_global + p.n_local;
  // sequence fastest, then window slot, then head group: consecutive
  // workgroups go to consecutive XCDs, so with B a multiple of 8 every
  // workgroup of a sequence runs on one XCD and its latent pages are fetched
  // into that XCD's L2 once for all head groups
  const int b = blockIdx.x % p.B;
  const int slot = (blockIdx.x / p.B) % W;
  const int h0 = (blockIdx.x / (p.B * W)) * (kHeads * HG);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int ch0 = wave * kWaveCh;                 // this wave's value channels
  const int rope0 = kDv + wave * kRopeCh + 4 * (g & 1);  // lanes g < 2 carry the rope slice

  // query fragments (B operand: lane (r, g) = head h0 + 16t + r, k-slice g),
  // issued before the window lookup they do not depend on; the rope operand
  // has k-slices 0, 1 only (8 channels), slices 2, 3 are zero
  bf16x8 qf[HG][kGroups];
  bf16x4 qr[HG];
#pragma unroll
  for (int t = 0; t < HG; ++t) {
    const __bf16* qrow = static_cast<const __bf16*>(p.q) + b * p.qs_b + (h0 + kHeads * t + r) * p.qs_h;
#pragma unroll
    for (int j = 0; j < kGroups; ++j) qf[t][j] = ldg<bf16x8>(qrow + ch0 + 32 * j + 8 * g);
    qr[t] = ldg<bf16x4>(qrow + rope0);
    if (g >= 2) qr[t] = bf16x4{};
  }

  const int n = p.seq_lens[b];
  const DecodeWindow win(p, n);
  // the partials of head h0 + hh for this slot start at out + hh * W * kPart
  float* out = p.work + ((static_cast<int64_t>(b) * p.Hq + h0) * W + slot) * kPart;
  // slots past the window are never read; a page outside the pool marks the
  // slot with l = NaN, which the merge kernel turns into a NaN row
  if (slot >= win.cntw) return;
  const int blk = win.block(slot);
  const int page = p.block_table[b * p.bt_stride + blk];
  if (page < 0 || page >= p.num_pages) {
    if (threadIdx.x < kHeads * HG) out[static_cast<int64_t>(threadIdx.x) * W * kPart + kDv + 1] = __builtin_nanf("");
    return;
  }
  const int valid = min(128, n - blk * 128);  // keys of this block that exist, >= 1

  // key rows (A operand: lane (r, g) = key r of the step, k-slice g), all 8
  // steps at once.  Keys at or past `valid` are replaced by the last valid
  // one: their scores are masked, and a masked zero weight times finite data
  // stays zero inside the MFMA (times NaN it would not).
  const __bf16* kpg = static_cast<const __bf16*>(p.k) + static_cast<int64_t>(page) * p.ks_p;
  const __bf16* vpg = static_cast<const __bf16*>(p.v) + static_cast<int64_t>(page) * p.vs_p;
  bf16x8 kc[kSteps][kGroups];
  bf16x4 kr[kSteps];
  bf16x8 vc[SHARED ? 1 : kSteps][kGroups];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int key = min(s * kStep + r, valid - 1);
    const __bf16* krow = kpg + static_cast<int64_t>(key) * p.ks_s;
#pragma unroll
    for (int j = 0; j < kGroups; ++j) kc[s][j] = ldg_nt<bf16x8>(krow + ch0 + 32 * j + 8 * g);
    kr[s] = ldg_nt<bf16x4>(krow + rope0);
    if constexpr (!SHARED) {
      const __bf16* vrow = vpg + static_cast<int64_t>(key) * p.vs_s;
#pragma unroll
      for (int j = 0; j < kGroups; ++j) vc[SHARED ? 0 : s][j] = ldg_nt<bf16x8>(vrow + ch0 + 32 * j + 8 * g);
    }
  }

  // 1. partial S^T of every step over this wave's channels.  The rope
  // product has its own accumulator: a 16x16x16 MFMA that takes a 16x16x32
  // result as its accumulator input a few instructions later has read a
  // stale last register, so chains stay within one opcode.
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const bf16x4 ks = g >= 2 ? bf16x4{} : kr[s];
#pragma unroll
    for (int t = 0; t < HG; ++t) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kGroups; ++j) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc[s][j], qf[t][j], a, 0, 0, 0);
      const f32x4 rope = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
          __builtin_bit_cast(s16x4, ks), __builtin_bit_cast(s16x4, qr[t]), f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      sx[((s * HG + t) * kMWaves + wave) * 64 + lane] = a + rope;
    }
  }
  lds_barrier();

  // 2. step `wave`: full scores (the 8 partials in a fixed order), mask, max
  const int s_own = wave;
  const int kv = valid - s_own * kStep;  // keys of the step that exist (>= 1 for step 0)
  f32x4 so[HG];
#pragma unroll
  for (int t = 0; t < HG; ++t) {
    f32x4 v = sx[((s_own * HG + t) * kMWaves + 0) * 64 + lane];
#pragma unroll
    for (int w = 1; w < kMWaves; ++w) v += sx[((s_own * HG + t) * kMWaves + w) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (g * 4 + i >= kv) v[i] = kNegInf;
    so[t] = v;
    const float mx = xlane_max(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
    if (g == 0) mxs[(s_own * HG + t) * kHeads + r] = mx;
  }
  lds_barrier();

  // 3. block max per head, P of step `wave`, its share of the row sum
  float m[HG];
#pragma unroll
  for (int t = 0; t < HG; ++t) {
    float M = kNegInf;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) M = fmaxf(M, mxs[(s * HG + t) * kHeads + r]);
    m[t] = M;  // finite: key 0 of step 0 exists
    const float mc = M * p.c1;
    f32x4 e;
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(so[t][i], p.c1, -mc));
      rs += e[i];
    }
    rs = xlane_sum(rs);
    pbuf[(s_own * HG + t) * 64 + lane] = __builtin_convertvector(e, bf16x4);
    if (g == 0) lsp[(s_own * HG + t) * kHeads + r] = rs;
  }
  lds_barrier();

  // 4. O^T (64 channels x 16 heads) += V^T (64 x 16 keys) P^T (16 keys x 16 heads)
  float l[HG];
#pragma unroll
  for (int t = 0; t < HG; ++t) {
    float v = 0.f;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) v += lsp[(s * HG + t) * kHeads + r];
    l[t] = v;
  }
  f32x4 acc[HG][NJ];
#pragma unroll
  for (int t = 0; t < HG; ++t)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  SSA_LDS u32x4* vt = vtile + wave * kGroups * 64;
  const int wpos = 4 * r + (g ^ swz(r));
  // transposed read of output tile jt: key row 4g + r/4, channels
  // 16jt + 4(r mod 4) .. +3; the tr read then hands lane (r, g) channel
  // 16jt + r of keys 4g .. 4g+3
  const int vrow = 4 * g + (r >> 2);
  const int vpos = ((r >> 1) & 1) ^ swz(vrow);  // position for even jt; odd jt: ^ 2
  const SSA_LDS char* vrd = (const SSA_LDS char*)(vt) + vrow * 64 + (r & 1) * 8;
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    // value tile of step s (LDS is in order within a wave: the previous
    // step's reads of the tile are done before these writes land)
#pragma unroll
    for (int j = 0; j < kGroups; ++j)
      vt[j * 64 + wpos] = __builtin_bit_cast(u32x4, SHARED ? kc[s][j] : vc[SHARED ? 0 : s][j]);
    bf16x4 pb[HG];
#pragma unroll
    for (int t = 0; t < HG; ++t) pb[t] = pbuf[(s * HG + t) * 64 + lane];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
      const SSA_LDS char* a = vrd + (jt >> 1) * 1024 + (vpos ^ ((jt & 1) << 1)) * 16;
      const bf16x4 vf = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SSA_LDS bf16x4*)(a));
#pragma unroll
      for (int t = 0; t < HG; ++t)
        acc[t][jt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vf),
                                                                __builtin_bit_cast(s16x4, pb[t]), acc[t][jt], 0, 0, 0);
    }
  }

  // this wave's 64 channels of the block's (o, m, l)
#pragma unroll
  for (int t = 0; t < HG; ++t) {
    float* oh = out + static_cast<int64_t>(kHeads * t + r) * W * kPart;
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) *reinterpret_cast<f32x4*>(oh + ch0 + jt * 16 + 4 * g) = acc[t][jt];
    if (wave == 0 && g == 0) {
      oh[kDv] = m[t];
      oh[kDv + 1] = l[t];
    }
  }
}

// Merge kernel: one 64-lane workgroup per (sequence, head), 8 channels a
// lane.  The partials of all W slots are loaded together with the sequence
// length (slots past the window hold stale data and are ignored), so the
// kernel waits for memory once.  Workgroup order: sequence fastest, the same
// XCD assignment as the partial kernel's.
__global__ __launch_bounds__(64) void decode_mla_merge_kernel(DecodeParams p) {
  const int W = p.n_global + p.n_local;
  const int b = blockIdx.x % p.B, h = blockIdx.x / p.B;
  const float* base = p.work + (static_cast<int64_t>(b) * p.Hq + h) * W * kPart;
  const int c0 = threadIdx.x * 8;
  float mt[kMaxW], lt[kMaxW];
  f32x4 oa[kMaxW], ob[kMaxW];
#pragma unroll
  for (int t = 0; t < kMaxW; ++t) {
    if (t < W) {
      const float* pt = base + t * kPart;
      mt[t] = pt[kDv];
      lt[t] = pt[kDv + 1];
      oa[t] = *reinterpret_cast<const f32x4*>(pt + c0);
      ob[t] = *reinterpret_cast<const f32x4*>(pt + c0 + 4);
    }
  }
  const int n = p.seq_lens[b];
  const DecodeWindow win(p, n);
  bool bad = win.cntw == 0;
  float M = kNegInf;
#pragma unroll
  for (int t = 0; t < kMaxW; ++t)
    if (t < win.cntw) {
      M = fmaxf(M, mt[t]);
      bad |= __builtin_isnan(lt[t]);  // a page outside the pool
    }
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
  float ls = 0.f;
#pragma unroll
  for (int t = 0; t < kMaxW; ++t) {
    if (t < win.cntw) {  // every slot of a valid row holds a key: m_t is finite
      const float s = __builtin_amdgcn_exp2f((mt[t] - M) * p.c1);
      ls = __builtin_fmaf(lt[t], s, ls);
      o0 += oa[t] * s;
      o1 += ob[t] * s;
    }
  }
  const float nan = __builtin_nanf("");
  const float inv = 1.f / ls;
  bf16x8 ov;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ov[i] = static_cast<__bf16>(bad ? nan : o0[i] * inv);
    ov[4 + i] = static_cast<__bf16>(bad ? nan : o1[i] * inv);
  }
  __bf16* op = static_cast<__bf16*>(p.o) + b * p.os_b + h * p.os_h + c0;
  *reinterpret_cast<bf16x8*>(op) = ov;
  if (threadIdx.x == 0 && p.lse)
    p.lse[static_cast<int64_t>(b) * p.Hq + h] = bad ? nan : M * p.scale + __builtin_amdgcn_logf(ls) * kLn2;
}

template <bool SHARED, int HG>
hipError_t launch_mla(const DecodeParams& p, hipStream_t stream) {
  const unsigned W = static_cast<unsigned>(p.n_global + p.n_local);
  const dim3 grid(static_cast<unsigned>(p.B) * W * static_cast<unsigned>(p.Hq / (kHeads * HG)));
  const size_t lds = sizeof(f32x4) * kSteps * HG * kMWaves * 64 + sizeof(u32x4) * kMWaves * kGroups * 64 +
                     sizeof(bf16x4) * kSteps * HG * 64 + 2 * sizeof(float) * kSteps * HG * kHeads;
  constexpr auto kern = decode_mla_partial_kernel<SHARED, HG>;
  hipError_t e = raise_lds_limit_once<kern>(static_cast<int>(lds));
  if (e != hipSuccess) return e;
  e = launch_kernel(kern, grid, dim3(kMWaves * 64), lds, stream, p);
  if (e != hipSuccess) return e;
  return launch_kernel(decode_mla_merge_kernel, dim3(static_cast<unsigned>(p.B) * p.Hq), dim3(64), 0, stream, p);
}

}  // namespace

size_t decode_mla_workspace_bytes(int32_t B, int32_t Hq, int32_t W) {
  return sizeof(float) * static_cast<size_t>(B) * Hq * W * kPart;
}

hipError_t launch_decode_mla(const DecodeParams& p, hipStream_t stream) {
  if (p.Hkv != 1 || p.Hq % kHeads != 0 || !p.work || p.n_global + p.n_local > kMaxW) return hipErrorNotSupported;
  const bool shared = p.v == p.k && p.vs_p == p.ks_p && p.vs_s == p.ks_s;
#ifndef SSA_MLA_HG
#define SSA_MLA_HG 2
#endif
  if (SSA_MLA_HG == 2 && p.Hq % (2 * kHeads) == 0)
    return shared ? launch_mla<true, 2>(p, stream) : launch_mla<false, 2>(p, stream);
  return shared ? launch_mla<true, 1>(p, stream) : launch_mla<false, 1>(p, stream);
}

}  // namespace ssa
