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
// bf16 kernel: two neighbouring query blocks per workgroup
// ---------------------------------------------------------------------------
//
// Neighbouring query blocks read almost the same key blocks (SSA: 7 of 8), so
// a workgroup of 8 waves takes the pair (2p, 2p+1): waves 0-3 own the 128
// queries of block 2p ("A"), waves 4-7 those of block 2p+1 ("B"), 32 queries
// per wave, two waves per SIMD.  Keys are streamed in stages of 64 (half a
// block) through a ring of 4 LDS slots: a stage carries one half-block read
// by both groups, or two half-blocks (one only A reads, one only B reads)
// that are staged side by side.  The next stage is prefetched into registers
// while the current one is computed, so one barrier per stage suffices
// (consecutive stages use disjoint slot pairs).

constexpr int kPairWaves = 8;
constexpr int kPairThreads = kPairWaves * 64;
constexpr int kHalf = 64;  // keys per stage
constexpr int kMaxStages = 4 * 64;

template <int D>
struct PairLds {
  // 16-byte units so that every fragment access is a single ds_read_b128.
  // Rows are padded by one unit: with 64 LDS banks the 16 lanes that read
  // one fragment column then hit 16 distinct 16-byte bank groups.
  static constexpr int KR = D / 8 + 1;      // K row: D channels + pad (units)
  static constexpr int VR = kHalf / 8 + 1;  // V^T row: 64 keys + pad (units)
  u32x4 k[4][kHalf * KR];
  u32x4 vt[4][D * VR];
  int32_t stage[kMaxStages];  // (A half id + 1) | (B half id + 1) << 16; 0 = none
  int32_t lists[3][64];       // A-only, B-only, shared block ids (list mode)
  int32_t nstages;
};

template <int D>
struct StageRegs {
  static constexpr int KN = (kHalf * D / 8 + kPairThreads - 1) / kPairThreads;  // K 16-byte chunks per thread
  static constexpr int VN = (4 * D + kPairThreads - 1) / kPairThreads;          // V 2-key x 8-channel items
  u32x4 k[KN];
  u32x4 v[VN][2];
};

// Global -> registers: half-block `hid` (= 2 * block + half) of K and V.
// K: thread e takes 16 bytes (row e / (D/8), chunk e % (D/8)).
// V: thread e takes 2 consecutive keys (pair kp = e % 32) x 8 channels
// (chunk dd = e / 32): two 16-byte row pieces.
template <int D>
__device__ __forceinline__ void load_half(const __bf16* kbase, const __bf16* vbase, int64_t ks_l, int64_t vs_l,
                                          int L, int hid, int tid, StageRegs<D>& rg) {
  constexpr int CH = D / 8;
  const int row0 = (hid >> 1) * kBlock + (hid & 1) * kHalf;
#pragma unroll
  for (int i = 0; i < StageRegs<D>::KN; ++i) {
    const int e = tid + i * kPairThreads;
    rg.k[i] = u32x4{0, 0, 0, 0};
    if (e < kHalf * CH) {
      const int key = row0 + e / CH;
      if (key < L) rg.k[i] = *reinterpret_cast<const u32x4*>(kbase + key * ks_l + (e % CH) * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < StageRegs<D>::VN; ++i) {
    const int e = tid + i * kPairThreads;
#pragma unroll
    for (int j = 0; j < 2; ++j) rg.v[i][j] = u32x4{0, 0, 0, 0};
    if (e < 4 * D) {
      const int kp = e & 31, dd = e >> 5;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int key = row0 + kp * 2 + j;
        if (key < L) rg.v[i][j] = *reinterpret_cast<const u32x4*>(vbase + key * vs_l + dd * 8);
      }
    }
  }
}

// Registers -> LDS slot.  K keeps its row-major layout; V is written
// transposed (channel rows) with the key order of the P^T registers: within
// each 32-key chunk c, lane group g holds keys c*32 + {4g..4g+3, 16+4g..16+4g+3},
// stored contiguously at c*32 + 8g.  The 32 lanes of one channel chunk write
// one contiguous 128-byte run of a V^T row.
template <int D>
__device__ __forceinline__ void store_half(PairLds<D>& sm, int slot, int tid, const StageRegs<D>& rg) {
  constexpr int CH = D / 8;
  constexpr int KR = PairLds<D>::KR, VR = PairLds<D>::VR;
#pragma unroll
  for (int i = 0; i < StageRegs<D>::KN; ++i) {
    const int e = tid + i * kPairThreads;
    if (e < kHalf * CH) sm.k[slot][(e / CH) * KR + (e % CH)] = rg.k[i];
  }
  uint32_t* vt1 = reinterpret_cast<uint32_t*>(sm.vt[slot]);
#pragma unroll
  for (int i = 0; i < StageRegs<D>::VN; ++i) {
    const int e = tid + i * kPairThreads;
    if (e < 4 * D) {
      const int kp = e & 31, dd = e >> 5;
      const int kq = kp >> 1, c = kq >> 3, w = kq & 7;
      const int pos = c * 32 + (w & 3) * 8 + (w >> 2) * 4 + (kp & 1) * 2;  // in keys; 2 keys = one u32
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t r0 = rg.v[i][0][x], r1 = rg.v[i][1][x];
        const int ch = dd * 8 + 2 * x;
        vt1[ch * (4 * VR) + pos / 2] = (r0 & 0xFFFFu) | (r1 << 16);
        vt1[(ch + 1) * (4 * VR) + pos / 2] = (r0 >> 16) | (r1 & 0xFFFF0000u);
      }
    }
  }
}

// Stage s of the pair: half ids read by group A and group B (-1: none).
template <int D>
__device__ __forceinline__ void get_stage(const PrefillParams& p, const PairLds<D>& sm, int qa, bool has_b, int s,
                                          int& ha, int& hb) {
  if (p.dense) {
    if (has_b && s < 2) {
      ha = -1;
      hb = 2 * (qa + 1) + s;
      return;
    }
    const int h = s - (has_b ? 2 : 0);
    ha = h;
    hb = has_b ? h : -1;
    return;
  }
  const int e = sm.stage[s];
  ha = (e & 0xFFFF) - 1;
  hb = (e >> 16) - 1;
}

// Build the stage table from the two block lists (wave 0; list mode only):
// pairs of (A-only, B-only) blocks first, then unpaired leftovers, then the
// blocks both read; each block gives two half-block stages.
template <int D>
__device__ void build_stages(const PrefillParams& p, PairLds<D>& sm, int b, int h, int qa, bool has_b, int lane) {
  const int nkb = p.nqb;
  auto read_list = [&](int q, int& ent) -> bool {
    const int cnt = min(p.cnt[b * p.cnt_sb + h * p.cnt_sh + q], p.W);
    ent = -1;
    if (lane < cnt) ent = p.idx[b * p.idx_sb + h * p.idx_sh + static_cast<int64_t>(q) * p.W + lane];
    return ent >= 0 && ent <= q && ent < nkb;
  };
  int ea, eb = -1;
  const bool va = read_list(qa, ea);
  bool vb = false;
  if (has_b) vb = read_list(qa + 1, eb);
  // membership tests through LDS
  sm.lists[0][lane] = va ? ea : -1;
  sm.lists[1][lane] = vb ? eb : -1;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  bool a_in_b = false, b_in_a = false;
  for (int j = 0; j < 64; ++j) {
    const int xa = sm.lists[0][j], xb = sm.lists[1][j];
    a_in_b |= va && xb == ea;
    b_in_a |= vb && xa == eb;
  }
  const uint64_t m_ao = __ballot(va && !a_in_b);
  const uint64_t m_bo = __ballot(vb && !b_in_a);
  const uint64_t m_sh = __ballot(va && a_in_b);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int n_ao = __popcll(m_ao), n_bo = __popcll(m_bo), n_sh = __popcll(m_sh);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (va && !a_in_b) sm.lists[0][__popcll(m_ao & below)] = ea;
  if (vb && !b_in_a) sm.lists[1][__popcll(m_bo & below)] = eb;
  if (va && a_in_b) sm.lists[2][__popcll(m_sh & below)] = ea;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int np = min(n_ao, n_bo);
  // block-level entries: k < np: pair; then A leftovers, B leftovers, shared
  const int nblk = np + (n_ao - np) + (n_bo - np) + n_sh;
  for (int k = lane; k < nblk; k += 64) {
    int ba, bb;
    if (k < np) {
      ba = sm.lists[0][k];
      bb = sm.lists[1][k];
    } else if (k < n_ao) {
      ba = sm.lists[0][k];
      bb = -1;
    } else if (k < n_ao + (n_bo - np)) {
      ba = -1;
      bb = sm.lists[1][np + (k - n_ao)];
    } else {
      ba = bb = sm.lists[2][k - n_ao - (n_bo - np)];
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int xa = ba < 0 ? 0 : 2 * ba + half + 1;
      const int xb = bb < 0 ? 0 : 2 * bb + half + 1;
      sm.stage[2 * k + half] = xa | (xb << 16);
    }
  }
  if (lane == 0) sm.nstages = 2 * nblk;
}

template <int D, typename OutT>
__global__ __launch_bounds__(kPairThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_pair_kernel(PrefillParams p) {
  constexpr int NC = D / 32;  // 32-wide contraction chunks over channels
  constexpr int NJ = D / 16;  // 16-wide output channel tiles
  constexpr int KR = PairLds<D>::KR, VR = PairLds<D>::VR;
  __shared__ PairLds<D> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int grp = wave >> 2, wq = wave & 3;  // group (0 = A, 1 = B), wave within group

  // pair coordinates: last pairs first, heads fastest (XCD-friendly, see tile_coords)
  const int npairs = (p.nqb + 1) / 2;
  const int bh_count = p.B * p.Hq;
  const int pr = npairs - 1 - static_cast<int>(blockIdx.x) / bh_count;
  const int bh = static_cast<int>(blockIdx.x) % bh_count;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int qa = 2 * pr;
  const bool has_b = qa + 1 < p.nqb;
  const int my_qb = qa + grp;
  const bool active = grp == 0 || has_b;
  const int hk = h / p.group;
  const __bf16* qbase = static_cast<const __bf16*>(p.q) + b * p.qs_b + h * p.qs_h;
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + b * p.ks_b + hk * p.ks_h;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + b * p.vs_b + hk * p.vs_h;

  int nst;
  if (p.dense) {
    nst = 2 * (qa + 1) + (has_b ? 2 : 0);
  } else {
    if (wave == 0) build_stages<D>(p, sm, b, h, qa, has_b, lane);
    __syncthreads();
    nst = sm.nstages;
  }

  // Q^T fragments (B operand): lane (r, g) holds query row r of 16-query tile
  // n, channels 32c + 8g .. +7.
  bf16x8 qf[2][NC];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int row = my_qb * kBlock + wq * kQW + n * 16 + r;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 v = {0, 0, 0, 0};
      if (active && row < p.L) v = *reinterpret_cast<const u32x4*>(qbase + row * p.qs_l + c * 32 + g * 8);
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

  // prologue: stage 0 into slots 0/1
  StageRegs<D> ra, rb;
  if (nst > 0) {
    int ha, hb;
    get_stage<D>(p, sm, qa, has_b, 0, ha, hb);
    const int h0 = ha >= 0 ? ha : hb;
    load_half<D>(kbase, vbase, p.ks_l, p.vs_l, p.L, h0, tid, ra);
    const bool two = ha >= 0 && hb >= 0 && ha != hb;
    if (two) load_half<D>(kbase, vbase, p.ks_l, p.vs_l, p.L, hb, tid, rb);
    store_half<D>(sm, 0, tid, ra);
    if (two) store_half<D>(sm, 1, tid, rb);
  }
  __syncthreads();

  for (int s = 0; s < nst; ++s) {
    int ha, hb;
    get_stage<D>(p, sm, qa, has_b, s, ha, hb);
    const bool two = ha >= 0 && hb >= 0 && ha != hb;
    const int base = 2 * (s & 1);
    // prefetch stage s+1
    int na = -1, nb = -1;
    bool ntwo = false;
    if (s + 1 < nst) {
      get_stage<D>(p, sm, qa, has_b, s + 1, na, nb);
      ntwo = na >= 0 && nb >= 0 && na != nb;
      load_half<D>(kbase, vbase, p.ks_l, p.vs_l, p.L, na >= 0 ? na : nb, tid, ra);
      if (ntwo) load_half<D>(kbase, vbase, p.ks_l, p.vs_l, p.L, nb, tid, rb);
    }

    const int hid = grp == 0 ? ha : hb;
    const int slot = base + ((grp == 1 && two) ? 1 : 0);
    const int kb = hid >> 1, half = hid & 1;
    // skip when nothing to do, or when the whole half lies above this wave's
    // queries in the diagonal block (every key masked)
    const bool work = active && hid >= 0 && !(kb == my_qb && half * kHalf > wq * kQW + kQW - 1);
    if (work) {
      f32x4 sc[4][2];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int n = 0; n < 2; ++n) sc[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8 kf = __builtin_bit_cast(bf16x8, sm.k[slot][(t * 16 + r) * KR + c * 4 + g]);
#pragma unroll
          for (int n = 0; n < 2; ++n)
            sc[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[n][c], sc[t][n], 0, 0, 0);
        }
      }
      if (kb == my_qb) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int qi = wq * kQW + n * 16 + r;
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (half * kHalf + t * 16 + g * 4 + i > qi) sc[t][n][i] = kNegInf;
        }
      }
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        float mx = kNegInf;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[t][n][i]);
        mx = wave_max16x4(mx);
        const float m_new = fmaxf(m[n], mx);
        const float alpha = __builtin_amdgcn_exp2f((m[n] - m_new) * p.c1);
        const float mc = m_new * p.c1;
        float rs = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t)
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
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 pf[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const bf16x4 a = __builtin_convertvector(sc[2 * c][n], bf16x4);
          const bf16x4 bq = __builtin_convertvector(sc[2 * c + 1][n], bf16x4);
          pf[n] = bf16x8{a[0], a[1], a[2], a[3], bq[0], bq[1], bq[2], bq[3]};
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const bf16x8 vf = __builtin_bit_cast(bf16x8, sm.vt[slot][(j * 16 + r) * VR + c * 4 + g]);
#pragma unroll
          for (int n = 0; n < 2; ++n)
            acc[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[n], acc[j][n], 0, 0, 0);
        }
      }
    }

    if (s + 1 < nst) {
      const int nbase = 2 * ((s + 1) & 1);
      store_half<D>(sm, nbase, tid, ra);
      if (ntwo) store_half<D>(sm, nbase + 1, tid, rb);
    }
    __syncthreads();
  }

  if (!active) return;
  OutT* obase = static_cast<OutT*>(p.o) + b * p.os_b + h * p.os_h;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int row = my_qb * kBlock + wq * kQW + n * 16 + r;
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
  if (dqk == 576 && dv == 512) return launch_prefill_wide(p, dqk, dv, out_f32, stream);
  const dim3 pgrid(static_cast<unsigned>((p.nqb + 1) / 2) * p.B * p.Hq);
  const dim3 pblock(kPairThreads);
  if (dqk == 128 && dv == 128)
    return out_f32 ? launch_kernel(prefill_bf16_pair_kernel<128, float>, pgrid, pblock, 0, stream, p)
                   : launch_kernel(prefill_bf16_pair_kernel<128, __bf16>, pgrid, pblock, 0, stream, p);
  if (dqk == 64 && dv == 64)
    return out_f32 ? launch_kernel(prefill_bf16_pair_kernel<64, float>, pgrid, pblock, 0, stream, p)
                   : launch_kernel(prefill_bf16_pair_kernel<64, __bf16>, pgrid, pblock, 0, stream, p);
  return hipErrorNotSupported;
}

}  // namespace ssa
