// SSA decode over a paged KV cache, gfx950.
//
// A decode step reads, for the query at position n - 1, the window of its
// block qb = (n - 1) / 128: block 0 and the blocks qb - 6 .. qb (QbitAI report
// on LongCat LoZA, sparse-window paragraph); the last block holds
// (n - 1) mod 128 + 1 valid keys.  Long-context decode is bound by reading the
// cache (LongCat sparse attention article, section 1), and contiguous reads
// coalesce (its section 3, mechanism 1), so the kernel is organised around
// streaming whole 128-token pages with 16-byte loads:
//
//   - one workgroup per (sequence, kv head), one wave per window block;
//   - a wave streams its page's K and V rows (each row = D/8 lanes x 16 B),
//     computes the scores with a DPP row reduction, and keeps a partial
//     softmax state (m, l, o[D]) -- an exact rewrite of the max-subtracted
//     softmax of the CSA/HCA tutorial page, section 7.1;
//   - the per-block partials are merged in LDS: M = max m_w,
//     o = sum o_w e^(m_w - M) / sum l_w e^(m_w - M).
#include "common.hpp"

namespace ssa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.6931471805599453f;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the CPR lanes that hold one key row (CPR = 16: a DPP row; CPR = 8:
// half a row).  Every lane of the group ends with the full sum.
template <int CPR>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (CPR == 16) {
    x += dpp<0x128>(x);  // row_ror:8
    x += dpp<0x124>(x);  // row_ror:4
  } else {
    static_assert(CPR == 8, "8 or 16 lanes per key row");
    x += dpp<0x141>(x);  // row_half_mirror
  }
  x += dpp<0x4E>(x);  // quad_perm [2,3,0,1]
  x += dpp<0xB1>(x);  // quad_perm [1,0,3,2]
  return x;
}

// Reduction over the key groups of a wave (lanes with equal lane % CPR).
template <int CPR>
__device__ __forceinline__ float across_keys_max(float x) {
#pragma unroll
  for (int s = CPR; s < 64; s <<= 1) x = fmaxf(x, __shfl_xor(x, s));
  return x;
}
template <int CPR>
__device__ __forceinline__ float across_keys_sum(float x) {
#pragma unroll
  for (int s = CPR; s < 64; s <<= 1) x += __shfl_xor(x, s);
  return x;
}

__device__ __forceinline__ void bf16x8_to_f32(const u32x4 v, float* f) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[2 * w] = __builtin_bit_cast(float, v[w] << 16);
    f[2 * w + 1] = __builtin_bit_cast(float, v[w] & 0xFFFF0000u);
  }
}

constexpr int kMaxWaves = 16;
constexpr int kSub = 16;    // keys per sub-pass
constexpr int kDepth = 1;   // sub-passes of loads in flight ahead of the one scored
constexpr int kPage = 128;  // keys per cache page

__device__ __forceinline__ float dot8_bf16(const float* q, const u32x4 k) {
  float kf[8];
  bf16x8_to_f32(k, kf);
  float d = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) d = __builtin_fmaf(q[e], kf[e], d);
  return d;
}

__device__ __forceinline__ u32x4 ldg16(const __bf16* p) {
  return *(const __attribute__((address_space(1))) u32x4*)(p);
}
// 16 bytes at a wave-uniform base plus a per-lane 32-bit byte offset (one
// offset register per load instead of a 64-bit address), as a non-temporal
// load: every cache byte is read once per step, and streaming it past the
// caches' normal replacement measured ~12% faster on the batch-64 workload
// (~6.2 against ~5.4 TB/s)
__device__ __forceinline__ u32x4 ldg_stream(const char* base, uint32_t off) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4*)(base + off));
}

// One workgroup per (sequence, kv head), one wave per window block.  A wave
// streams its page in sub-passes of kSub keys -- 16-byte loads, D/8 lanes per
// key row, so a wave reads 4 (D = 128) or 8 (D = 64) whole rows per
// instruction -- with the next sub-pass's loads in flight while one is
// scored.  The loads are unconditional: a key past the block's valid ones
// reads the last valid row again (a cache hit) and its score is masked, so
// the compiler counts the loads in flight exactly instead of draining them
// at every branch.  MAXT: the largest workgroup the instantiation serves; at
// most 128 registers per wave, so two 8-wave workgroups share a CU.
// DENSE: every cached block, in groups of nwaves blocks: workgroup
// (split, sequence, kv head) reads blocks split*nwaves + wave and writes its
// merged (o unnormalised, m, l) per query head to p.work; a merge kernel
// combines the groups.
template <int D, int MAXT, bool DENSE = false>
__global__ __launch_bounds__(MAXT) __attribute__((amdgpu_waves_per_eu(4))) void decode_mha_kernel(DecodeParams p) {
  constexpr int CPR = D / 8;      // lanes per key row (16 B each)
  constexpr int KPI = 64 / CPR;   // keys per wave-wide load
  constexpr int NI = kSub / KPI;  // loads per sub-pass and operand
  constexpr int NS = kPage / kSub;
  constexpr int NB = kDepth + 1;  // sub-pass buffers
  __shared__ float part[kMaxWaves][D + 2];
  __shared__ int bad;

  const int lane = threadIdx.x & 63, nwaves = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kr = lane / CPR, cc = lane % CPR;
  const int hk = blockIdx.x % p.Hkv;
  const int b = DENSE ? (blockIdx.x / p.Hkv) % p.B : blockIdx.x / p.Hkv;
  const int split = DENSE ? blockIdx.x / (p.Hkv * p.B) : 0;
  const int n = p.seq_lens[b];
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();

  // window slot of this wave (same rule as the block-index builder)
  int blk = -1;
  const bool len_ok = n >= 1 && n <= p.max_blocks * kPage;
  if (len_ok) {
    if constexpr (DENSE) {
      const int cand = split * nwaves + wave;
      if (cand < (n + kPage - 1) / kPage) blk = cand;
    } else {
      const int qb = (n - 1) / kPage;
      const int g_end = min(p.n_global, qb + 1);
      const int l_begin = max(g_end, qb - p.n_local + 1);
      const int cntw = g_end + (qb - l_begin + 1);
      if (wave < cntw) blk = wave < g_end ? wave : l_begin + (wave - g_end);
    }
  } else if (threadIdx.x == 0) {
    bad = 1;
  }
  int page = -1, valid = 0;  // this wave's keys [0, valid) of the page
  if (blk >= 0) {
    page = __builtin_amdgcn_readfirstlane(p.block_table[b * p.bt_stride + blk]);
    if (page < 0 || page >= p.num_pages) {
      if (lane == 0) bad = 1;
      blk = -1;
    } else {
      valid = min(kPage, n - blk * kPage);
    }
  }
  __syncthreads();
  const bool all_bad = bad != 0;

  // wave-uniform page bases; per-lane byte offsets (rows of a page are < 2^31 bytes apart)
  const char* kp = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.k) + static_cast<int64_t>(page) * p.ks_p + hk * p.ks_h);
  const char* vp = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.v) + static_cast<int64_t>(page) * p.vs_p + hk * p.vs_h);
  const uint32_t kstride = static_cast<uint32_t>(p.ks_s) * 2u, vstride = static_cast<uint32_t>(p.vs_s) * 2u;

  for (int hq = hk * p.group; hq < (hk + 1) * p.group; ++hq) {
    float m = kNegInf, l = 0.f;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    if (!all_bad && blk >= 0) {
      float qv[8];
      bf16x8_to_f32(ldg16(static_cast<const __bf16*>(p.q) + b * p.qs_b + hq * p.qs_h + cc * 8), qv);
      u32x4 kv[NB][NI], vv[NB][NI];
      // byte offsets of this lane's row kr and of the last valid row; row
      // r + c is read at min(r + c, last) (the clamp commutes with the
      // positive stride).  The empty asm makes each sub-pass start from an
      // opaque copy, so its offsets are formed just before its loads rather
      // than all up front.
      uint32_t kb = kr * kstride, vb = kr * vstride;  // row kr + S * kSub
      const uint32_t klast = (valid - 1) * kstride, vlast = (valid - 1) * vstride;
#define SSA_DECODE_LOAD(S)                                                   \
  {                                                                          \
    asm volatile("" : "+v"(kb), "+v"(vb));                                   \
    _Pragma("unroll") for (int i = 0; i < NI; ++i)                           \
      kv[(S) % NB][i] = ldg_stream(kp, min(kb + i * KPI * kstride, klast) + cc * 16); \
    _Pragma("unroll") for (int i = 0; i < NI; ++i)                           \
      vv[(S) % NB][i] = ldg_stream(vp, min(vb + i * KPI * vstride, vlast) + cc * 16); \
    kb += kSub * kstride;                                                    \
    vb += kSub * vstride;                                                    \
  }
#pragma unroll
      for (int s = 0; s < kDepth; ++s) SSA_DECODE_LOAD(s);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s + kDepth < NS) SSA_DECODE_LOAD(s + kDepth < NS ? s + kDepth : 0);
        if (s * kSub < valid) {  // wave-uniform: sub-passes wholly past the valid keys are skipped
          // key of lane group kr (opaque, so the masks are formed here and
          // not hoisted out of the head loop into a register per key)
          int k0 = kr + s * kSub;
          asm volatile("" : "+v"(k0));
          float sc[NI];
          float mx = kNegInf;
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            const float d = group_sum<CPR>(dot8_bf16(qv, kv[s % NB][i]));
            sc[i] = (k0 + i * KPI < valid) ? d : kNegInf;
            mx = fmaxf(mx, sc[i]);
          }
          mx = across_keys_max<CPR>(mx);
          const float m_new = fmaxf(m, mx);  // finite: key 0 is valid
          const float alpha = __builtin_amdgcn_exp2f((m - m_new) * p.c1);
          const float mc = m_new * p.c1;
          l *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] *= alpha;
          float ps_sum = 0.f;
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], p.c1, -mc));
            ps_sum += pe;
            float vf[8];
            bf16x8_to_f32(vv[s % NB][i], vf);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf(pe, vf[e], o[e]);
          }
          // every lane of a key group holds the same pe: count each key once
          l += across_keys_sum<CPR>(ps_sum);
          m = m_new;
        }
      }
#undef SSA_DECODE_LOAD
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = across_keys_sum<CPR>(o[e]);
    }
    if (kr == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) part[wave][cc * 8 + e] = o[e];
    }
    if (lane == 0) {
      part[wave][D] = m;
      part[wave][D + 1] = l;
    }
    __syncthreads();
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
      float M = kNegInf;
      for (int w = 0; w < nwaves; ++w) M = fmaxf(M, part[w][D]);
      float acc = 0.f, lsum = 0.f;
      for (int w = 0; w < nwaves; ++w) {
        const float sc = part[w][D] == kNegInf ? 0.f : __builtin_amdgcn_exp2f((part[w][D] - M) * p.c1);
        acc = __builtin_fmaf(part[w][d], sc, acc);
        lsum = __builtin_fmaf(part[w][D + 1], sc, lsum);
      }
      const float nan = __builtin_nanf("");
      if constexpr (DENSE) {
        // this group's piece: o relative to M, then M and l (l = NaN marks a bad row)
        float* w = p.work + ((static_cast<int64_t>(b) * p.Hq + hq) * p.nsplit + split) * (D + 2);
        w[d] = acc;
        if (d == 0) {
          w[D] = M;
          w[D + 1] = all_bad ? nan : lsum;
        }
      } else {
        const float out = all_bad ? nan : acc / lsum;
        __bf16* op = static_cast<__bf16*>(p.o) + b * p.os_b + hq * p.os_h;
        op[d] = static_cast<__bf16>(out);
        if (d == 0 && p.lse)
          p.lse[static_cast<int64_t>(b) * p.Hq + hq] = all_bad ? nan : M * p.scale + __builtin_amdgcn_logf(lsum) * kLn2;
      }
    }
    __syncthreads();
  }
}

// Decode merge (the dense decode's block groups): one wave per (sequence,
// query head) combines the pieces, M = max m_s, o = sum o_s e^(m_s - M) / sum l_s e^(m_s - M)
// (the exact merge of max-subtracted softmax pieces, CSA/HCA tutorial page,
// section 7.1); a NaN l in any group makes the row NaN.
template <int D>
__global__ __launch_bounds__(64) void decode_dense_merge_kernel(DecodeParams p) {
  const int b = blockIdx.x / p.Hq, hq = blockIdx.x % p.Hq, lane = threadIdx.x;
  const float* w = p.work + (static_cast<int64_t>(b) * p.Hq + hq) * p.nsplit * (D + 2);
  float M = kNegInf;
  bool bad = false;
  for (int s = 0; s < p.nsplit; ++s) {
    M = fmaxf(M, w[s * (D + 2) + D]);
    bad |= __builtin_isnan(w[s * (D + 2) + D + 1]);
  }
  constexpr int PER = D / 64;
  float acc[PER], lsum = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int s = 0; s < p.nsplit; ++s) {
    const float ms = w[s * (D + 2) + D];
    if (ms == kNegInf) continue;  // a group with no key
    const float sc = __builtin_amdgcn_exp2f((ms - M) * p.c1);
    lsum = __builtin_fmaf(w[s * (D + 2) + D + 1], sc, lsum);
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = __builtin_fmaf(w[s * (D + 2) + lane + 64 * i], sc, acc[i]);
  }
  const float nan = __builtin_nanf("");
  __bf16* op = static_cast<__bf16*>(p.o) + b * p.os_b + hq * p.os_h;
#pragma unroll
  for (int i = 0; i < PER; ++i) op[lane + 64 * i] = static_cast<__bf16>(bad ? nan : acc[i] / lsum);
  if (lane == 0 && p.lse)
    p.lse[static_cast<int64_t>(b) * p.Hq + hq] = bad ? nan : M * p.scale + __builtin_amdgcn_logf(lsum) * kLn2;
}

}  // namespace

constexpr int kDenseGroup = 16;  // blocks per dense-decode workgroup (16 waves)

size_t decode_dense_workspace_bytes(int32_t B, int32_t Hq, int32_t max_blocks, int32_t d) {
  const int64_t nsplit = (static_cast<int64_t>(max_blocks) + kDenseGroup - 1) / kDenseGroup;
  return static_cast<size_t>(static_cast<int64_t>(B) * Hq * nsplit * (d + 2) * sizeof(float));
}

hipError_t launch_decode_merge(const DecodeParams& p, int d, hipStream_t stream) {
  const dim3 mgrid(static_cast<unsigned>(p.B) * p.Hq);
  return d == 128 ? launch_kernel(decode_dense_merge_kernel<128>, mgrid, dim3(64), 0, stream, p)
       : d == 64  ? launch_kernel(decode_dense_merge_kernel<64>, mgrid, dim3(64), 0, stream, p)
                  : hipErrorNotSupported;
}

hipError_t launch_decode_dense(const DecodeParams& p, int d, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.nsplit) * p.B * p.Hkv);
  const dim3 block(64 * kDenseGroup);
  hipError_t e = d == 128 ? launch_kernel(decode_mha_kernel<128, 1024, true>, grid, block, 0, stream, p)
               : d == 64  ? launch_kernel(decode_mha_kernel<64, 1024, true>, grid, block, 0, stream, p)
                          : hipErrorNotSupported;
  if (e != hipSuccess) return e;
  return launch_decode_merge(p, d, stream);
}

hipError_t launch_decode(const DecodeParams& p, int dqk, int dv, hipStream_t stream) {
  if (dqk == 576 && dv == 512) return launch_decode_mla(p, stream);
  if (decode_gqa_supports(p, dqk, dv)) return launch_decode_gqa(p, stream);
  const int width = p.n_global + p.n_local;  // validated <= 16
  const dim3 grid(static_cast<unsigned>(p.B) * p.Hkv);
  const dim3 block(64 * width);
  const bool small = block.x <= 512;
  if (dqk == 128 && dv == 128)
    return small ? launch_kernel(decode_mha_kernel<128, 512>, grid, block, 0, stream, p)
                 : launch_kernel(decode_mha_kernel<128, 1024>, grid, block, 0, stream, p);
  if (dqk == 64 && dv == 64)
    return small ? launch_kernel(decode_mha_kernel<64, 512>, grid, block, 0, stream, p)
                 : launch_kernel(decode_mha_kernel<64, 1024>, grid, block, 0, stream, p);
  return hipErrorNotSupported;
}

}  // namespace ssa
