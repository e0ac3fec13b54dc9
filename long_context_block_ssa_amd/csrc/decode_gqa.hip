// SSA decode with grouped query heads (g = Hq / Hkv query heads per kv head,
// 2 <= g <= 16), d = 128, on gfx950.
//
// The step reads the window of the new token's block: block 0 and the 7 most
// recent blocks, the last one partial (QbitAI report on LongCat LoZA,
// sparse-window paragraph).  Decode is bound by reading the cache (LongCat
// sparse attention article, section 1), so every K/V row is read once for all
// g query heads of its kv head, the per-head work goes to the matrix cores,
// and every load of a step is in flight at once:
//   - a (sequence, kv head) window is served by one workgroup of 8 waves, or
//     by two, each with half the query heads, when the windows are fewer
//     than the compute units; per round wave w takes 64 keys (one half of
//     one block) and issues all its K and V loads (32 KB) before it computes
//     anything;
//   - loads read whole rows (4 rows of 256 bytes an instruction: ~13%
//     faster than 16 rows of 64 bytes); each step's K and V rows go to two
//     wave-private LDS tiles;
//   - S^T (16 keys x 16 heads, heads past g are zero) = K Q^T on
//     v_mfma_f32_16x16x32_bf16, its A operand read from the K tile (lane
//     r + 16G: key r of the step, channels 32c + 8G .. +7) and the query
//     fragments as the B operand;
//   - with all 64 keys' scores at hand the wave's softmax is exact in two
//     passes (max, then weights): no accumulator is rescaled;
//   - ds_read_b64_tr_b16 hands, from the V tile, the V^T operand of
//     O^T += V^T P^T on v_mfma_f32_16x16x16_bf16; P^T is the score tile
//     itself, so no weight moves between lanes;
//   - a window wider than 4 blocks is read in rounds of 4 blocks by the same
//     workgroup; a wave's rounds share its running max (the accumulator
//     rescales when it grows), so no partials leave the workgroup and no
//     merge kernel runs;
//   - the 8 waves' (o, m, l) per head are merged in LDS: M = max m_w,
//     o = sum o_w e^(m_w - M) / sum l_w e^(m_w - M), the exact merge of
//     max-subtracted softmax pieces (CSA/HCA tutorial page, section 7.1), in a
//     fixed wave order.
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

constexpr int kD = 128;
constexpr int kStep = 16;            // keys per step
constexpr int kTile = kStep * kD / 8;  // 16-byte units of a step's V tile (4 KB)
constexpr int kPartF = kD + 2;       // floats per (wave, head) partial: o, m, l
constexpr int kWaves = 8;            // waves per workgroup
constexpr int kKeysPerWave = 64;     // half a block
constexpr int kStepsPerWave = kKeysPerWave / kStep;
constexpr int kSlotsPerRound = kWaves * kKeysPerWave / 128;  // window slots per round of a workgroup
constexpr int kMaxW = 16;            // window widths served
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
__device__ __forceinline__ T ldg(const __bf16* ptr) {
  return *(const SSA_GLB T*)(ptr);
}
// cache rows are read once per step: a non-temporal stream
template <typename T>
__device__ __forceinline__ T ldg_nt(const __bf16* ptr) {
  return __builtin_nontemporal_load((const SSA_GLB T*)(ptr));
}
__device__ __forceinline__ float xlane_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float xlane_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// K and V tiles: 16-byte unit u (channels 8u .. 8u+7) of key row k of the
// step at position 16k + (u ^ k): the fragment reads (16 rows, one unit) and
// the transposed reads of one instruction (rows 4G + j/4, units
// 2jt + (j mod 4)/2) then spread over the banks.
__device__ __forceinline__ int vpos(int k, int u) { return 16 * k + (u ^ k); }

// grid B * Hkv * head_splits (kv head fastest, then head split), 8 waves; a
// workgroup serves heads [hs * gh, hs * gh + gh) of its kv head (gh =
// ceil(g / head_splits)) over every window slot, 4 slots a round: in round t
// wave w takes slot 4t + w/2.  Dynamic LDS: 8 partials of 16 heads (the V and K
// tiles, 64 KB, reuse it).
constexpr int kMaxRounds = kMaxW / kSlotsPerRound;
constexpr int kChipCUs = 256;  // compute units of an MI355X

__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_gqa_kernel(DecodeParams p) {
  extern __shared__ u32x4 lds_dyn[];
  __shared__ int bad;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, G = lane >> 4;
  const int hk = blockIdx.x % p.Hkv;
  const int b = (blockIdx.x / p.Hkv) % p.B;
  const int hs = blockIdx.x / (p.Hkv * p.B);
  const int g = p.group;
  const int gh = (g + p.head_splits - 1) / p.head_splits;
  const int h0 = hs * gh;
  const int ng = min(gh, g - h0);  // heads of this workgroup (>= 1)
  const bool mine_h = r < ng;
  const int h = hk * g + h0 + r;  // this lane's query head (none for r >= ng)
  const int key0 = kKeysPerWave * (wave & 1);  // its first key in a block

  // query fragments (B operand of S^T = K Q^T): head h, channels 32c + 8G ..
  bf16x8 qf[4];
  {
    const __bf16* qrow = static_cast<const __bf16*>(p.q) + b * p.qs_b + static_cast<int64_t>(mine_h ? h : hk * g) * p.qs_h;
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = mine_h ? ldg<bf16x8>(qrow + 32 * c + 8 * G) : bf16x8{};
  }

  // the wave's block of every round (the block-index builder's rule); a
  // length outside the cache or a page outside the pool makes the row NaN
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  const int n = p.seq_lens[b];
  const int width = p.n_global + p.n_local;
  const int rounds = (width + kSlotsPerRound - 1) / kSlotsPerRound;
  int valid[kMaxRounds];  // keys of the wave's block that exist, per round
  int page[kMaxRounds];
#pragma unroll
  for (int t = 0; t < kMaxRounds; ++t) {
    valid[t] = 0;
    page[t] = -1;
  }
  if (n >= 1 && n <= p.max_blocks * 128) {
    const int qb = (n - 1) / 128;
    const int g_end = min(p.n_global, qb + 1);
    const int l_begin = max(g_end, qb - p.n_local + 1);
    const int cntw = g_end + (qb - l_begin + 1);
#pragma unroll
    for (int t = 0; t < kMaxRounds; ++t) {
      const int slot = kSlotsPerRound * t + wave / 2;
      if (t < rounds && slot < cntw) {
        const int blk = slot < g_end ? slot : l_begin + (slot - g_end);
        const int pg = __builtin_amdgcn_readfirstlane(p.block_table[b * p.bt_stride + blk]);
        if (pg < 0 || pg >= p.num_pages) {
          if (lane == 0) bad = 1;
        } else {
          page[t] = pg;
          valid[t] = min(128, n - blk * 128);
        }
      }
    }
  } else if (threadIdx.x == 0) {
    bad = 1;
  }
  __syncthreads();
  const bool all_bad = bad != 0;

  float m = kNegInf, l = 0.f;  // head r: the wave's running max, this lane's share of the row sum
  f32x4 acc[kD / 16];          // O^T tile jt: channels 16jt + 4G .. +3 of head r
#pragma unroll
  for (int jt = 0; jt < kD / 16; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t = 0; t < rounds; ++t) {
    int vld = 0, pgt = 0;
#pragma unroll
    for (int u = 0; u < kMaxRounds; ++u)
      if (u == t) {
        vld = valid[u];
        pgt = page[u];
      }
    if (all_bad || key0 >= vld) continue;  // wave-uniform
    const __bf16* kpg = static_cast<const __bf16*>(p.k) + static_cast<int64_t>(pgt) * p.ks_p + hk * p.ks_h;
    const __bf16* vpg = static_cast<const __bf16*>(p.v) + static_cast<int64_t>(pgt) * p.vs_p + hk * p.vs_h;
    // every K and V row of the wave's 64 keys, all in flight at once: load i
    // of step s gives lane (lrow, lu) unit lu (channels 8lu .. 8lu+7) of key
    // key0 + 16s + 4i + lrow (the last valid key for keys past `vld`: finite
    // data whose scores are masked)
    bf16x8 kb[kStepsPerWave][4], vb[kStepsPerWave][4];
    const int lrow = lane >> 4, lu = lane & 15;
#pragma unroll
    for (int s = 0; s < kStepsPerWave; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = min(key0 + s * kStep + 4 * i + lrow, vld - 1);
        kb[s][i] = ldg_nt<bf16x8>(kpg + static_cast<int64_t>(key) * p.ks_s + 8 * lu);
      }
#pragma unroll
    for (int s = 0; s < kStepsPerWave; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = min(key0 + s * kStep + 4 * i + lrow, vld - 1);
        vb[s][i] = ldg_nt<bf16x8>(vpg + static_cast<int64_t>(key) * p.vs_s + 8 * lu);
      }
    // keep every load above this point (the scheduler would otherwise sink
    // the later steps' loads to their uses and expose their latency)
    __builtin_amdgcn_sched_barrier(0);
    // S^T of every step: lane (r, G) gets keys key0 + 16s + 4G + i of head r
    f32x4 sc[kStepsPerWave];
    float mx = kNegInf;
#pragma unroll
    for (int s = 0; s < kStepsPerWave; ++s) {
      // the step's K rows into the wave's K tile, then the A operand from it
      // (LDS is in order within a wave)
      SSA_LDS u32x4* kt = (SSA_LDS u32x4*)(lds_dyn) + (kWaves + wave) * kTile;
#pragma unroll
      for (int i = 0; i < 4; ++i) kt[vpos(4 * i + lrow, lu)] = __builtin_bit_cast(u32x4, kb[s][i]);
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kt[vpos(r, 4 * c + G)]), qf[c], a, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (key0 + s * kStep + 4 * G + i >= vld) a[i] = kNegInf;
      sc[s] = a;
      mx = fmaxf(mx, fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])));
    }
    // the running max over the rounds (finite once a round has keys): the
    // earlier rounds' weights and output rescale to it
    const float mnew = fmaxf(m, xlane_max(mx));
    if (m != kNegInf && mnew != m) {
      const float alpha = __builtin_amdgcn_exp2f((m - mnew) * p.c1);
      l *= alpha;
#pragma unroll
      for (int jt = 0; jt < kD / 16; ++jt) acc[jt] *= alpha;
    }
    m = mnew;
    const float mc = m * p.c1;
    SSA_LDS u32x4* vt = (SSA_LDS u32x4*)(lds_dyn) + wave * kTile;
    // transposed read of O^T tile jt: lane j = r of group G reads key row
    // 4G + j/4, channels 16jt + 4(j mod 4) .. +3 (unit 2jt + (j mod 4)/2,
    // half j mod 2); the read hands lane (r, G) channel 16jt + r of keys
    // 4G .. 4G+3
    const int trow = 4 * G + (r >> 2);
    const SSA_LDS char* vrd = (const SSA_LDS char*)(vt) + (r & 1) * 8;
#pragma unroll
    for (int s = 0; s < kStepsPerWave; ++s) {
      f32x4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[s][i], p.c1, -mc));
      l += (e[0] + e[1]) + (e[2] + e[3]);
      // the step's V rows into the wave's tile (LDS is in order within a
      // wave: the previous step's reads are done before these writes land)
#pragma unroll
      for (int i = 0; i < 4; ++i) vt[vpos(4 * i + lrow, lu)] = __builtin_bit_cast(u32x4, vb[s][i]);
      const bf16x4 pb = __builtin_convertvector(e, bf16x4);
#pragma unroll
      for (int jt = 0; jt < kD / 16; ++jt) {
        const int u = 2 * jt + ((r & 3) >> 1);
        const bf16x4 vf = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SSA_LDS bf16x4*)(vrd + vpos(trow, u) * 16));
        acc[jt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vf),
                                                            __builtin_bit_cast(s16x4, pb), acc[jt], 0, 0, 0);
      }
    }
  }

  // ---- merge the 8 waves per head ------------------------------------------
  // partial of (wave w, head hh): o[kD], m, l at part + (w * 16 + hh) * kPartF
  // (it reuses the V tiles' LDS once every wave is past its last step)
  float* part = reinterpret_cast<float*>(lds_dyn);
  const float lt = xlane_sum(l);
  __syncthreads();
  if (mine_h) {
    float* mine = part + (wave * 16 + r) * kPartF;
#pragma unroll
    for (int jt = 0; jt < kD / 16; ++jt) *reinterpret_cast<f32x4*>(mine + 16 * jt + 4 * G) = acc[jt];
    if (G == 0) {
      mine[kD] = m;  // -inf for a wave without keys: skipped below
      mine[kD + 1] = lt;
    }
  }
  __syncthreads();
  const float nan = __builtin_nanf("");
  for (int i = threadIdx.x; i < ng * kD; i += kWaves * 64) {
    const int hh = i / kD, d = i % kD;
    float M = kNegInf;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, part[(w * 16 + hh) * kPartF + kD]);
    float o = 0.f, lsum = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      const float* pw = part + (w * 16 + hh) * kPartF;
      if (pw[kD] == kNegInf) continue;
      const float sc = __builtin_amdgcn_exp2f((pw[kD] - M) * p.c1);
      o = __builtin_fmaf(pw[d], sc, o);
      lsum = __builtin_fmaf(pw[kD + 1], sc, lsum);
    }
    const int hq = hk * g + h0 + hh;
    __bf16* op = static_cast<__bf16*>(p.o) + b * p.os_b + hq * p.os_h;
    op[d] = static_cast<__bf16>(all_bad ? nan : o / lsum);
    if (d == 0 && p.lse)
      p.lse[static_cast<int64_t>(b) * p.Hq + hq] = all_bad ? nan : M * p.scale + __builtin_amdgcn_logf(lsum) * kLn2;
  }
}

}  // namespace

bool decode_gqa_supports(const DecodeParams& p, int dqk, int dv) {
  return dqk == kD && dv == kD && p.group >= 2 && p.group <= 16 && p.n_global + p.n_local <= kMaxW;
}

hipError_t launch_decode_gqa(const DecodeParams& p, hipStream_t stream) {
  const size_t lds = sizeof(float) * kPartF * 16 * kWaves;  // >= 2 * kWaves tiles (64 KB)
  static_assert(sizeof(float) * kPartF * 16 * kWaves >= sizeof(u32x4) * kTile * 2 * kWaves, "tiles fit");
  hipError_t e = raise_lds_limit_once<decode_gqa_kernel>(static_cast<int>(lds));
  if (e != hipSuccess) return e;
  // fewer (sequence, kv head) windows than compute units: two workgroups per
  // window, each with half the query heads (both read the window; the second
  // read mostly hits L2)
  DecodeParams q = p;
  q.head_splits = p.B * p.Hkv < kChipCUs ? 2 : 1;
  return launch_kernel(decode_gqa_kernel, dim3(static_cast<unsigned>(q.B) * q.Hkv * q.head_splits), dim3(kWaves * 64),
                       lds, stream, q);
}

}  // namespace ssa
