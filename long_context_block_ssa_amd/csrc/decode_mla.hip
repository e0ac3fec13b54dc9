// SSA decode at the latent-shared (MLA-like) shape on gfx950: Hq query heads
// share one key/value latent of width 576 per cached token, the value being
// its first 512 channels.  LoZA rewrites LongCat's MLA layers (QbitAI report
// on LongCat LoZA); a decode step reads the window of the new token's block:
// block 0 and the 7 most recent blocks (same report, sparse-window
// paragraph), the last one partial.
//
// The per-sequence work is a dense contraction -- (16 heads x 576) by
// (576 x 1024 keys), then (16 heads x 1024) by (1024 x 512) -- on the matrix
// cores.  A sequence's window is only ~1 MB and one CU stages at most
// ~50-100 GB/s into LDS, so the window is spread over all CUs and the pieces
// are merged afterwards:
//   - partial kernel: one workgroup per (sequence, 16 query heads, window
//     block), 4 waves; each wave takes two 16-key steps of the block through
//     its own LDS slab filled by global_load_lds_dwordx4;
//   - S^T (16 keys x 16 heads) on v_mfma_f32_16x16x32_bf16; the online
//     softmax keeps one (m, l) per head; O^T += V^T P^T on
//     v_mfma_f32_16x16x16_bf16, whose V^T operand (4 keys of one channel per
//     lane) is one ds_read_b64_tr_b16 from the row-major latent slab;
//   - the 4 wave partials are merged in LDS and the block's (o, m, l) per
//     head is written, in fp32, to the workspace;
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
constexpr int kHeads = 16;     // query heads per workgroup (one MFMA tile)
constexpr int kMWaves = 4;
constexpr int kStep = 16;      // keys per step
constexpr int kStepsPerWave = 128 / kStep / kMWaves;    // 2: a wave's share of one block
// Slab layout (unit = 16 bytes = 8 channels): DMA instruction i of a step
// fills units 64i .. 64i+63 with channel units 4i .. 4i+3 of the step's 16
// keys -- key row at 4 units apiece, unit u of the group stored at position
// u ^ swz(row).  One lane pointer plus an immediate offset per instruction
// addresses every load, the K fragment reads of one instruction group are one
// contiguous 1 KB, and the swizzle puts the transposed V reads of lanes 0-31
// on distinct banks.
constexpr int kGK = kDqk / 32;  // 18 instruction groups per K step
constexpr int kGV = kDv / 32;   // 16 per separate V step
__device__ __forceinline__ int swz(int row) { return ((row >> 2) & 1) << 1; }
constexpr int kPart = kDv + 4;  // workspace floats per (sequence, head, window slot): o, m, l, pad
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

// Stage keys key0 .. key0+15 of one page (NG groups of 32 channels).  Keys
// at or past the block's valid count kend are replaced by the last valid
// one: their scores are masked, and a masked zero weight times finite data
// stays zero inside the MFMA (times NaN it would not).
template <int NG>
__device__ __forceinline__ void stage16(SSA_LDS u32x4* slab, const __bf16* page_base, int64_t slot_stride, int key0,
                                        int kend, int lane) {
  const int row = lane >> 2;
  const int u = (lane & 3) ^ swz(row);
  const int key = min(key0 + row, kend - 1);
  const __bf16* src = page_base + static_cast<int64_t>(key) * slot_stride + u * 8;
#pragma unroll
  for (int i = 0; i < NG; ++i)
    __builtin_amdgcn_global_load_lds((const SSA_GLB void*)(src + i * 32), (SSA_LDS void*)(slab + i * 64), 16, 0, 0);
}

template <bool SHARED>
__global__ __launch_bounds__(kMWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_mla_partial_kernel(DecodeParams p) {
  constexpr int SLAB = 64 * (kGK + (SHARED ? 0 : kGV));
  constexpr int NC = kDqk / 32;
  constexpr int NJ = kDv / 16;
  extern __shared__ u32x4 lds_dyn[];
  SSA_LDS u32x4* lds = (SSA_LDS u32x4*)(lds_dyn);
  __shared__ float wm[kMWaves][kHeads], wl[kMWaves][kHeads], wsc[kMWaves][kHeads];

  const int W = p.n_global + p.n_local;
  // sequence fastest, then window slot, then head group: consecutive
  // workgroups go to consecutive XCDs, so with B a multiple of 8 every
  // workgroup of a sequence runs on one XCD and its latent pages are fetched
  // into that XCD's L2 once for all head groups
  const int b = blockIdx.x % p.B;
  const int slot = (blockIdx.x / p.B) % W;
  const int h0 = (blockIdx.x / (p.B * W)) * kHeads;
  const int n = p.seq_lens[b];
  const DecodeWindow win(p, n);
  // slots past the window write nothing; an invalid page leaves the slot
  // unwritten too, and the merge kernel turns the whole row into NaN
  if (slot >= win.cntw) return;
  const int blk = win.block(slot);
  const int page = p.block_table[b * p.bt_stride + blk];
  if (page < 0 || page >= p.num_pages) return;
  const int valid = min(128, n - blk * 128);  // keys of this block that exist, >= 1

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;

  // Q^T fragments (B operand): lane (r, g) = head h0 + r, channels 32c + 8g .. +7
  bf16x8 qf[NC];
  const __bf16* qrow = static_cast<const __bf16*>(p.q) + b * p.qs_b + (h0 + r) * p.qs_h;
#pragma unroll
  for (int c = 0; c < NC; ++c) qf[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + c * 32 + g * 8));

  float m = kNegInf, l = 0.f;
  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const __bf16* kpg = static_cast<const __bf16*>(p.k) + static_cast<int64_t>(page) * p.ks_p;
  const __bf16* vpg = static_cast<const __bf16*>(p.v) + static_cast<int64_t>(page) * p.vs_p;
  SSA_LDS u32x4* kslab = lds + wave * SLAB;
  const SSA_LDS u32x4* vslab = SHARED ? kslab : kslab + 64 * kGK;
  // lane (r, g) reads K row r, unit 4c + g; and for V^T row 4g + r/4,
  // channels 16jt + 4(r mod 4) .. +3 (ds_read_b64_tr_b16 then hands each lane
  // 4 keys of one channel)
  const int kfrag = r * 4 + (g ^ swz(r));
  const int vrow = 4 * g + (r >> 2);
  const int vunit = ((r >> 1) & 1) ^ swz(vrow);  // position within the group for even jt; odd jt: ^ 2
  const SSA_LDS char* vbase = (const SSA_LDS char*)(vslab + vrow * 4) + (r & 1) * 8;
  for (int st = 0; st < kStepsPerWave; ++st) {
    const int key0 = (wave + st * kMWaves) * kStep;  // first key of the step within the block
    const int kv = valid - key0;                      // keys of the step that exist
    if (kv <= 0) break;
    stage16<kGK>(kslab, kpg, p.ks_s, key0, valid, lane);
    if constexpr (!SHARED) stage16<kGV>(kslab + 64 * kGK, vpg, p.vs_s, key0, valid, lane);
    __builtin_amdgcn_s_waitcnt(0);
    // S^T (16 keys x 16 heads)
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bf16x8 kf = __builtin_bit_cast(bf16x8, kslab[c * 64 + kfrag]);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], sc, 0, 0, 0);
      if (c % 6 == 5) __builtin_amdgcn_sched_barrier(0);  // at most 6 key fragments in flight
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (g * 4 + i >= kv) sc[i] = kNegInf;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = xlane_max(mx);
    const float m_new = fmaxf(m, mx);  // finite: key0 < valid, so key 0 of the step is unmasked
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
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
      acc[jt] *= alpha;
      const SSA_LDS char* a = vbase + (jt >> 1) * 1024 + (vunit ^ ((jt & 1) << 1)) * 16;
      const bf16x4 vf = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SSA_LDS bf16x4*)a);
      acc[jt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vf), __builtin_bit_cast(s16x4, pb),
                                                           acc[jt], 0, 0, 0);
      // at most 8 transposed reads in flight: hoisting all 32 would not fit
      // beside the accumulator and the query fragments
      if (jt % 8 == 7) __builtin_amdgcn_sched_barrier(0);
    }
    // the next step restages this slab: the reads of this one must be done
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  }

  // merge the 4 wave partials of the block: per-head scales first, then the
  // channels in two halves of 256 through the (now idle) staging memory
  if (g == 0) {
    wm[wave][r] = m;
    wl[wave][r] = l;
  }
  __syncthreads();  // also: every wave is done with its slab
  float* out = p.work + ((static_cast<int64_t>(b) * p.Hq + h0) * W + slot) * kPart;  // head h0 + hh at + hh * W * kPart
  if (threadIdx.x < kHeads) {
    const int hh = threadIdx.x;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kMWaves; ++w) M = fmaxf(M, wm[w][hh]);
    float ls = 0.f;
#pragma unroll
    for (int w = 0; w < kMWaves; ++w) {
      const float s = wm[w][hh] == kNegInf ? 0.f : __builtin_amdgcn_exp2f((wm[w][hh] - M) * p.c1);
      wsc[w][hh] = s;
      ls = __builtin_fmaf(wl[w][hh], s, ls);
    }
    out[static_cast<int64_t>(hh) * W * kPart + kDv] = M;
    out[static_cast<int64_t>(hh) * W * kPart + kDv + 1] = ls;
  }
  float* part = (float*)(lds_dyn);
  constexpr int HALF = kDv / 2;
  constexpr int ROW = HALF + 4;  // padded head row: the 16-byte writes of lanes r = 0..15 hit distinct banks
  float* mine = part + wave * kHeads * ROW;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int jt = 0; jt < NJ / 2; ++jt)
      *reinterpret_cast<f32x4*>(mine + r * ROW + jt * 16 + g * 4) = acc[hf * (NJ / 2) + jt];
    __syncthreads();
    for (int e = threadIdx.x; e < kHeads * HALF / 4; e += kMWaves * 64) {
      const int hh = e / (HALF / 4), d = (e % (HALF / 4)) * 4;
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kMWaves; ++w) o += *reinterpret_cast<const f32x4*>(part + (w * kHeads + hh) * ROW + d) * wsc[w][hh];
      *reinterpret_cast<f32x4*>(out + static_cast<int64_t>(hh) * W * kPart + hf * HALF + d) = o;
    }
    if (hf == 0) __syncthreads();  // the second half overwrites the first
  }
}

// Merge kernel: one 64-lane workgroup per (sequence, head), 8 channels a lane.
__global__ __launch_bounds__(64) void decode_mla_merge_kernel(DecodeParams p) {
  const int W = p.n_global + p.n_local;
  const int b = blockIdx.x / p.Hq, h = blockIdx.x % p.Hq;
  const int n = p.seq_lens[b];
  const DecodeWindow win(p, n);
  bool bad = win.cntw == 0;
  for (int t = 0; t < win.cntw; ++t) {
    const int page = p.block_table[b * p.bt_stride + win.block(t)];
    bad |= page < 0 || page >= p.num_pages;
  }
  const float* base = p.work + (static_cast<int64_t>(b) * p.Hq + h) * W * kPart;
  float M = kNegInf;
  if (!bad)
    for (int t = 0; t < win.cntw; ++t) M = fmaxf(M, base[t * kPart + kDv]);
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
  float ls = 0.f;
  const int c0 = threadIdx.x * 8;
  if (!bad)
    for (int t = 0; t < win.cntw; ++t) {
      const float* pt = base + t * kPart;
      const float s = __builtin_amdgcn_exp2f((pt[kDv] - M) * p.c1);  // every slot holds a key: m_t is finite
      ls = __builtin_fmaf(pt[kDv + 1], s, ls);
      o0 += *reinterpret_cast<const f32x4*>(pt + c0) * s;
      o1 += *reinterpret_cast<const f32x4*>(pt + c0 + 4) * s;
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

template <bool SHARED>
hipError_t launch_mla(const DecodeParams& p, hipStream_t stream) {
  constexpr int SLAB = 64 * (kGK + (SHARED ? 0 : kGV));
  const size_t stage_bytes = sizeof(u32x4) * kMWaves * SLAB;
  const size_t part_bytes = sizeof(float) * kMWaves * kHeads * (kDv / 2 + 4);
  const size_t lds = stage_bytes > part_bytes ? stage_bytes : part_bytes;
  auto kern = decode_mla_partial_kernel<SHARED>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const unsigned W = static_cast<unsigned>(p.n_global + p.n_local);
  const dim3 grid(static_cast<unsigned>(p.B) * W * static_cast<unsigned>(p.Hq / kHeads));
  e = launch_kernel(kern, grid, dim3(kMWaves * 64), lds, stream, p);
  if (e != hipSuccess) return e;
  return launch_kernel(decode_mla_merge_kernel, dim3(static_cast<unsigned>(p.B) * p.Hq), dim3(64), 0, stream, p);
}

}  // namespace

size_t decode_mla_workspace_bytes(int32_t B, int32_t Hq, int32_t W) {
  return sizeof(float) * static_cast<size_t>(B) * Hq * W * kPart;
}

hipError_t launch_decode_mla(const DecodeParams& p, hipStream_t stream) {
  if (p.Hkv != 1 || p.Hq % kHeads != 0 || !p.work) return hipErrorNotSupported;
  const bool shared = p.v == p.k && p.vs_p == p.ks_p && p.vs_s == p.ks_s;
  return shared ? launch_mla<true>(p, stream) : launch_mla<false>(p, stream);
}

}  // namespace ssa
