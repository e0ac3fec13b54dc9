// Block-sparse causal attention prefill in bf16 on gfx950: the streaming
// kernel for Dqk = Dv = 64 and for the latent-shared
// (MLA-like) shape Dqk = 576, Dv = 512, where every query head reads one
// shared latent row per key and the value is its first 512 channels (LoZA
// rewrites LongCat's MLA attention, QbitAI report on LongCat LoZA).  Within
// the listed key blocks (SSA window, page-selected list, or all blocks for
// the dense layer) this is the masked softmax of equation (2) of the "LoZA:
// ZigZag sparse attention" page, section 2.1, causal in the own block
// (section 2.2.1), evaluated as an exact online softmax.
//
// One workgroup = one 128-query block of one head, 16*NQ queries per wave.
// d = 64: NQ = 2, 4 waves, two workgroups (two waves per SIMD) per CU.  The
// latent-shared 576/512 shape: NQ = 2, 4 waves, one wave per SIMD (the
// 32 x 512 fp32 accumulator fills the 256 AGPRs, Q^T 144 VGPRs), since 16
// queries per wave left each byte read from LDS feeding too few MFMA flops;
// with V staged apart it keeps NQ = 1 (8 waves).  Keys stream in 64-key
// stages through two LDS slots:
//   - staging uses global_load_lds_dwordx4 (global -> LDS, no registers);
//     d = 64 rows are padded by one 16-byte unit so that the 16 lanes
//     reading a fragment column hit 16 distinct bank groups; the 576-wide
//     latent has its own layout (value rows of one wave-instruction each,
//     XOR-swizzled, and a rope tail: see lswz), which also spreads the
//     transposed V reads;
//   - S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (A = K rows, ds_read_b128;
//     B = Q^T held in registers), so each lane owns one query column; at
//     576 a stage runs as two 32-key calls to keep the score tile small;
//   - O^T = V^T P^T: P^T comes from the S^T accumulators converted to bf16;
//     the V^T operand is read from the row-major V slab with
//     ds_read_b64_tr_b16, which hands each lane 4 keys of one channel, so the
//     latent is staged once and serves as both K and V;
//   - d = 64: the running max is refreshed lazily: the accumulator is
//     rescaled only when the max grows by more than 2^8, which is exact
//     because the final normalisation uses the same reference max;
//   - 576: a fixed reference max per row (the max of the wave's first call),
//     never raised, so the accumulator is never rescaled; a row sum above
//     2^64 (or inf / NaN) makes the workgroup rerun the tile, first for the
//     exact row maxima, then with them as the reference.
#include <type_traits>

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

// Layout of the 576-wide latent in a stage slot, in 16-byte units: the 512
// value channels (units 0..63) of key row k as one 1 KB row at k * 64, unit u
// at u ^ lswz(k), lswz(k) = 2 (k mod 8) + (k / 8) mod 2: a bijection on k mod
// 16, so the 16 rows of a fragment read fall on distinct bank groups of the
// 64 banks, and lswz(k) / 2 is one on k mod 8, so the 8 rows x 2 units that
// 32 lanes of a transposed read cover do too (LDS serves 256 bytes a cycle;
// the permutation 4 (k mod 4) + (k / 4) mod 4 left those 2-way conflicted;
// measured, conflict cycles fell from 48% to 32% of the LDS-active cycles
// with the kernel time unchanged); the 64 rope
// channels (units 64..71) in a tail after the 64 rows, 8 units per key, unit
// u of row k at kLatMain + 8 k + ((u - 64) ^ tswz(k)), tswz(k) = (k / 2) mod 8.
// Rows are whole wave-instructions of the direct-to-LDS staging, so a row's
// source address is uniform and a lane's offset within it takes one of a few
// values (no per-stage address arithmetic).
constexpr int kLatMain = 64 * 64;           // units of the 64 value rows
constexpr int kLatUnits = kLatMain + 64 * 8;  // plus the rope tail
__device__ __forceinline__ int lswz(int row) { return 2 * (row & 7) + ((row >> 3) & 1); }
__device__ __forceinline__ int tswz(int row) { return (row >> 1) & 7; }
// unit index of logical unit u (0..71) of staged row `row`
__device__ __forceinline__ int lat_unit(int row, int u) {
  return u < 64 ? row * 64 + (u ^ lswz(row)) : kLatMain + row * 8 + ((u - 64) ^ tswz(row));
}

// LDS geometry of one stage slot, in 16-byte units.
template <int DQK, int DV, bool SHARED>
struct WideGeom {
  static constexpr bool KSW = DQK == 576;  // the latent layout above instead of rows padded by one unit
  static constexpr int UK = KSW ? 64 : DQK / 8 + 1;  // K row pitch (the value rows of the latent)
  static constexpr int UV = DV / 8 + 1;   // V row pitch when V is staged apart
  static constexpr int KUNITS = KSW ? kLatUnits : kStageKeys * UK;
  static constexpr int VUNITS = SHARED ? 0 : kStageKeys * UV;
  static constexpr int SLOT = KUNITS + VUNITS;  // multiple of 64 units
  static constexpr int NSLOTS = 2 * SLOT * 16 <= 160 * 1024 ? 2 : 1;
  // 576/512 with the latent shared by K and V: 32 queries per wave take a
  // 256-register accumulator and 144 registers of Q^T, so one wave per SIMD;
  // each 64-key stage then runs as two 32-key halves (SUBS) to keep the score
  // tile small
  static constexpr int SUBS = KSW ? 2 : 1;
  static_assert(KUNITS % 64 == 0 && VUNITS % 64 == 0, "slab = whole 1 KB wave writes");
};

// Stages rows key0 .. key0+63 of a [L, D] operand into an LDS slab with row
// pitch U units (one 16-byte unit per lane per wave-instruction: the wave
// issues instructions i = wave, wave + NW, ... for linear units
// [i*64, i*64+64)).  A lane's (row, unit) is the same for every stage; with
// CACHE its element offset row*stride + unit*8 is kept in registers, else it
// is recomputed per stage (the 512-wide accumulator leaves no registers).  A
// lane on a row's pad unit loads unit 0 of its row.  Keys at or past L are
// clamped to row L-1 (finite data, masked later).
template <int D, int U, int NW, bool CACHE>
struct Stager {
  static constexpr int TOTAL = kStageKeys * U / 64;  // wave-instructions per slab
  static constexpr int PER = (TOTAL + NW - 1) / NW;  // per wave
  int32_t off[CACHE ? PER : 1];

  __device__ __forceinline__ static void place(int i, int lane, int& row, int& unit) {
    const int pidx = i * 64 + lane;
    row = pidx / U;
    const int pos = pidx - row * U;
    unit = pos < D / 8 ? pos : 0;
  }
  __device__ __forceinline__ void init(int64_t stride_l, int wave, int lane) {
    if constexpr (CACHE) {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        int row, unit;
        place(wave + j * NW, lane, row, unit);
        off[j] = static_cast<int32_t>(row * stride_l) + unit * 8;
      }
    }
  }
  __device__ __forceinline__ void issue(SSA_LDS u32x4* slab, const __bf16* base, int64_t stride_l, int key0, int L,
                                        int wave, int lane) const {
    const bool ragged = key0 + kStageKeys > L;  // uniform: only the last block of a ragged L
    if (CACHE && !ragged) {
      const __bf16* row0 = base + static_cast<int64_t>(key0) * stride_l;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = wave + j * NW;
        if (i < TOTAL)
          __builtin_amdgcn_global_load_lds((const SSA_GLB void*)(row0 + off[CACHE ? j : 0]),
                                           (SSA_LDS void*)(slab + i * 64), 16, 0, 0);
      }
      return;
    }
#pragma unroll 4
    for (int i = wave; i < TOTAL; i += NW) {
      int row, unit;
      place(i, lane, row, unit);
      const int key = min(key0 + row, L - 1);
      const __bf16* src = base + static_cast<int64_t>(key) * stride_l + unit * 8;
      __builtin_amdgcn_global_load_lds((const SSA_GLB void*)(src), (SSA_LDS void*)(slab + i * 64), 16, 0, 0);
    }
  }
};

// Stages latent rows key0 .. key0+63 (576 channels) in the layout above:
// the wave issues value rows wave, wave + NW, ... (a row per instruction, its
// source row uniform, the lane's byte offset (lane ^ lswz(row)) * 16) and
// tail instructions wave, wave + NW, ... (8 rows of 8 units each).  Keys at
// or past L are clamped to row L-1 (finite data, masked later).
template <int NW>
struct LatentStager {
  static constexpr int NT = 8 / NW;  // tail instructions per wave
  __device__ __forceinline__ void init(int64_t, int, int) {}
  __device__ __forceinline__ void issue(SSA_LDS u32x4* slab, const __bf16* base, int64_t stride_l, int key0, int L,
                                        int wave, int lane) const {
    const bool ragged = key0 + kStageKeys > L;  // uniform: only the last block of a ragged L
    const char* b = reinterpret_cast<const char*>(base);
    const int64_t sb = stride_l * 2;
    // The wave's row offset and the lane index made opaque here, so that
    // nothing derived from them is computed once and kept live across the
    // stage loop (the slot pointer itself stays transparent: the compiler
    // must see which of the two LDS objects an in-flight load writes, or it
    // waits for the loads before every LDS read):
    // the compiler otherwise held the 18 x 2 row addresses (M0) and the lane
    // offsets in registers, spilled them, and each reload's vmcnt(0) also
    // waited for the loads just issued.  Per load this costs one scalar add
    // (M0), one XOR and one shift.
    int w64 = wave * 64;  // the wave's first row, in units (opaque; the slot keeps its identity)
    asm volatile("" : "+s"(w64));
    int ln = lane;
    asm volatile("" : "+v"(ln));
    if (!ragged) {
      const char* rp = b + (key0 + wave) * sb;
#pragma unroll
      for (int j = 0; j < kStageKeys / NW; ++j) {
        const int row = wave + NW * j;
        const uint32_t off = static_cast<uint32_t>(ln ^ lswz(row)) * 16;
        __builtin_amdgcn_global_load_lds((const SSA_GLB void*)(rp + off), (SSA_LDS void*)(slab + w64 + NW * 64 * j),
                                         16, 0, 0);
        rp += NW * sb;
        asm volatile("" : "+s"(rp));  // stepped in place, not 16 precomputed row addresses
      }
    } else {
#pragma unroll 1
      for (int j = 0; j < kStageKeys / NW; ++j) {
        const int row = wave + NW * j;
        const char* src = b + min(key0 + row, L - 1) * sb;  // uniform
        const uint32_t off = static_cast<uint32_t>(ln ^ lswz(row)) * 16;
        __builtin_amdgcn_global_load_lds((const SSA_GLB void*)(src + off), (SSA_LDS void*)(slab + row * 64), 16, 0,
                                         0);
      }
    }
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      const int t = wave + NW * m;
      const int row = 8 * t + (ln >> 3);
      const int key = ragged ? min(key0 + row, L - 1) : key0 + row;
      const uint32_t uoff = static_cast<uint32_t>(64 + ((ln & 7) ^ tswz(row))) * 16;
      __builtin_amdgcn_global_load_lds((const SSA_GLB void*)(b + key * sb + uoff),
                                       (SSA_LDS void*)(slab + kLatMain + t * 64), 16, 0, 0);
    }
  }
};

// waves per SIMD: one for the 576-wide kernel with 32 queries per wave, else two
constexpr int wide_wpe(int dqk, int nq) { return dqk == 576 && nq == 2 ? 1 : 2; }

// NQ = 16-query tiles per wave; the workgroup's 128 / (16 NQ) waves cover one
// query block.  Two waves per SIMD: one 8-wave workgroup (NQ = 1) or two
// independent 4-wave workgroups (NQ = 2) per CU.  DENSE: every block
// 0 .. qb, own block first (the dense comparison layer); else the block list.
template <int DQK, int DV, bool SHARED, int NQ, bool DENSE, typename OutT>
__global__ __launch_bounds__(kBlk / (16 * NQ) * 64)
__attribute__((amdgpu_waves_per_eu(wide_wpe(DQK, NQ), wide_wpe(DQK, NQ))))
void prefill_wide_kernel(PrefillParams p) {
  using G = WideGeom<DQK, DV, SHARED>;
  constexpr int kNQ = NQ;
  constexpr int kRows = 16 * NQ;
  constexpr int kWWaves = kBlk / kRows;
  constexpr int NC = DQK / 32;  // 32-channel contraction chunks
  constexpr int NJ = DV / 16;   // 16-channel output tiles
  // two distinct LDS objects, so the compiler can tell a read of one slot from
  // the direct-to-LDS writes into the other and keep the prefetch in flight
  __shared__ u32x4 slot_a[G::SLOT];
  __shared__ u32x4 slot_b[G::NSLOTS == 2 ? G::SLOT : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps wave-level branches scalar
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
  if constexpr (DENSE) {
    count = qb + 1;
  } else {
    count = min(p.cnt[b * p.cnt_sb + h * p.cnt_sh + qb], p.W);
    const int32_t* list = p.idx + b * p.idx_sb + h * p.idx_sh + static_cast<int64_t>(qb) * p.W;
    if (tid < count) blist[tid] = list[tid];
    __syncthreads();
  }
  auto block_of = [&](int s) -> int {  // -1: skip
    // the list entry is the same in every lane: say so, so that everything
    // derived from it (addresses, masks, branches) stays scalar
    const int kb = DENSE ? qb - s : __builtin_amdgcn_readfirstlane(blist[s]);
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
  std::conditional_t<G::KSW, LatentStager<kWWaves>, Stager<DQK, G::UK, kWWaves, (kNQ >= 2)>> kst;
  kst.init(p.ks_l, wave, lane);
  // per-lane unit indices of the latent fragment reads: value chunk c (units
  // 4c .. 4c+3) of row 16 T + r at kb4[c mod 4] + 16 (c / 4) + 1024 T, rope
  // chunk c' of that row at tb2[c'] + 128 T
  int kb4[4], tb2[2];
#pragma unroll
  for (int b4 = 0; b4 < 4; ++b4) kb4[b4] = r * 64 + ((4 * b4 + g) ^ lswz(r));
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) tb2[c2] = kLatMain + r * 8 + ((4 * c2 + g) ^ tswz(r));
  Stager<DV, G::UV, kWWaves, (kNQ >= 2)> vst;
  if constexpr (!SHARED) vst.init(p.vs_l, wave, lane);
  auto issue = [&](int s, u32x4* slot_generic) {
    const int kb = block_of(s >> 1);
    if (kb < 0) return;
    SSA_LDS u32x4* slot = (SSA_LDS u32x4*)(slot_generic);
    const int key0 = kb * kBlk + (s & 1) * kStageKeys;
    kst.issue(slot, kbase, p.ks_l, key0, p.L, wave, lane);
    if constexpr (!SHARED) vst.issue(slot + G::KUNITS, vbase, p.vs_l, key0, p.L, wave, lane);
  };

  // one call: keys (s>>1)*128 + (s&1)*64 + sub*16*KT .. +16*KT-1 of the
  // stage staged in `cur` (KT 16-key tiles; SUBS calls per stage)
  constexpr int SUBS = kNQ >= 2 ? G::SUBS : 1;
  constexpr int KT = 4 / SUBS;
  constexpr int NCH = KT / 2;  // 32-key chunks of the output product
  // FIXREF: each row's reference max is the max of the first call that admits
  // one of its keys, and is never raised (no accumulator rescale, which would
  // take the 256 accumulator registers through the vector unit); else the
  // lazy refresh below
  constexpr bool FIXREF = G::KSW;
  bool ref_set = false;  // wave-uniform: the first call of the first pass has run
  // MODE 0: the first pass; 1: row maxima only; 2: the final pass of a rerun
  auto compute = [&](auto mode_c, int s, const u32x4* cur, int sub) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_c)::value;
    const int kb = block_of(s >> 1);
    const int half = s & 1;
    const int key_lo = half * kStageKeys + sub * 16 * KT;  // first key of the call within its block
    const bool work = kb >= 0 && !(kb == qb && key_lo > wave * kRows + kRows - 1);
    if (!work) return;
    const SSA_LDS u32x4* kslab = (const SSA_LDS u32x4*)(cur);
    const SSA_LDS u32x4* vslab = SHARED ? kslab : kslab + G::KUNITS;
    constexpr int UV = SHARED ? G::UK : G::UV;
    constexpr bool VSW = SHARED && G::KSW;  // V read from the swizzled latent slab
    // K fragment: chunk c (32 channels) of rows 16 rt + (lane mod 16)
    auto kfrag = [&](int rt, int c) -> bf16x8 {
      if constexpr (G::KSW)
        return __builtin_bit_cast(bf16x8, c < 16 ? kslab[kb4[c & 3] + 16 * (c >> 2) + 1024 * rt]
                                                 : kslab[tb2[c - 16] + 128 * rt]);
      else
        return __builtin_bit_cast(bf16x8, kslab[(rt * 16 + r) * G::UK + c * 4 + g]);
    };
    f32x4 sc[KT][kNQ];
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int n = 0; n < kNQ; ++n) sc[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kNQ >= 2) {
      // K fragments are read KD channel chunks ahead of their MFMAs so that the
      // LDS latency is covered by the MFMAs of the chunks in between
      // at 576 two chunks of read-ahead with V two steps ahead measured ~2.5%
      // faster than one and four
      constexpr int KD = G::KSW ? 2 : 1;
      bf16x8 kf[KD + 1][KT];
      auto load_k = [&](int c) {
  #pragma unroll
        for (int t = 0; t < KT; ++t)
          kf[c % (KD + 1)][t] = kfrag(sub * KT + t, c);
      };
  #pragma unroll
      for (int c = 0; c < KD && c < NC; ++c) load_k(c);
  #pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c + KD < NC) load_k(c + KD);
  #pragma unroll
        for (int t = 0; t < KT; ++t)
  #pragma unroll
          for (int n = 0; n < kNQ; ++n)
            sc[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c % (KD + 1)][t], qf[n][c], sc[t][n], 0, 0, 0);
      }
      // keep that order: first reads, then per chunk its MFMAs after the next reads
  #pragma unroll
      for (int c = 0; c < KD && c < NC; ++c) __builtin_amdgcn_sched_group_barrier(0x100, KT, 0);
  #pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c + KD < NC) __builtin_amdgcn_sched_group_barrier(0x100, KT, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, KT * kNQ, 0);
      }
    } else {
      // the 512-wide accumulator leaves no registers for read-ahead here
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8 kf1 = kfrag(t, c);
#pragma unroll
          for (int n = 0; n < kNQ; ++n)
            sc[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf1, qf[n][c], sc[t][n], 0, 0, 0);
        }
      }
    }
    const bool valid_all = (kb + 1) * kBlk <= p.L && kb < qb;
    if (!valid_all) {
#pragma unroll
      for (int n = 0; n < kNQ; ++n) {
        const int qi = wave * kRows + n * 16 + r;
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kk = key_lo + t * 16 + g * 4 + i;
            const bool dead = (kb == qb && kk > qi) || kb * kBlk + kk >= p.L;
            if (dead) sc[t][n][i] = kNegInf;
          }
      }
    }
    auto row_max = [&](int n) {
      float mx = kNegInf;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[t][n][i]);
      return xlane_max(mx);
    };
    if constexpr (FIXREF) {
#pragma unroll
      for (int n = 0; n < kNQ; ++n) {
        if constexpr (MODE == 1) {
          m[n] = fmaxf(m[n], row_max(n));
        } else {
          // the reference: the row max of the wave's first call (which
          // admits key 0 of its block, so every row of the wave has one
          // unless the list is invalid; a row left at -inf weighs its scores
          // against 0, and any overflow that causes is caught by the rerun)
          if constexpr (MODE == 0)
            if (!ref_set) m[n] = row_max(n);
          const float mc = m[n] == kNegInf ? 0.f : m[n] * p.c1;
          float rs = 0.f;
#pragma unroll
          for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][n][i], p.c1, -mc));
              sc[t][n][i] = e;
              rs += e;
            }
          l[n] += rs;  // this lane's part of the row sum, reduced across lanes at the end
        }
      }
      if constexpr (MODE == 0) ref_set = true;
      if constexpr (MODE == 1) return;
    } else {
#pragma unroll
    for (int n = 0; n < kNQ; ++n) {
      const float mx = row_max(n);
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
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][n][i], p.c1, -mc));
          sc[t][n][i] = e;
          rs += e;
        }
      l[n] += xlane_sum(rs);
    }
    }
    // O^T += V^T P^T over two 32-key chunks.  Step st = c * NJ + jt: the
    // V^T fragment of (chunk c, channel tile jt) is two transposed reads --
    // lane j of group g points at key c*32 + h2*16 + 4g + j/4, channels
    // 16*jt + 4*(j%4) .. +3, and receives channel 16*jt + j of keys
    // c*32 + h2*16 + 4g .. +3 -- issued VD steps ahead of its MFMAs.
    if constexpr (kNQ >= 2) {
      constexpr int VD = G::KSW ? 2 : 4;
      constexpr int NSTEP = NCH * NJ;
      bf16x8 vfr[VD + 1];
      auto load_v = [&](int st) {
        const int c = st / NJ, jt = st % NJ;
        const int krow = (sub * NCH + c) * 32 + 4 * g + (r >> 2);
        const int ch = jt * 16 + 4 * (r & 3);
        const int vu = VSW ? 16 * (jt >> 3) + ((2 * (jt & 7) + ((r & 3) >> 1)) ^ lswz(krow)) : (ch >> 3);
        const SSA_LDS char* base0 = (const SSA_LDS char*)(vslab + krow * UV + vu) + (ch & 7) * 2;
        const SSA_LDS char* base1 = base0 + 16 * UV * 16;
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SSA_LDS bf16x4*)base0);
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SSA_LDS bf16x4*)base1);
        vfr[st % (VD + 1)] = bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      };
      bf16x8 pf[NCH][kNQ];
  #pragma unroll
      for (int c = 0; c < NCH; ++c)
  #pragma unroll
        for (int n = 0; n < kNQ; ++n) {
          const bf16x4 a = __builtin_convertvector(sc[2 * c][n], bf16x4);
          const bf16x4 bq = __builtin_convertvector(sc[2 * c + 1][n], bf16x4);
          pf[c][n] = bf16x8{a[0], a[1], a[2], a[3], bq[0], bq[1], bq[2], bq[3]};
        }
  #pragma unroll
      for (int st = 0; st < VD && st < NSTEP; ++st) load_v(st);
  #pragma unroll
      for (int st = 0; st < NSTEP; ++st) {
        if (st + VD < NSTEP) load_v(st + VD);
        const int c = st / NJ, jt = st % NJ;
  #pragma unroll
        for (int n = 0; n < kNQ; ++n)
          acc[jt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfr[st % (VD + 1)], pf[c][n], acc[jt][n], 0, 0, 0);
      }
  #pragma unroll
      for (int st = 0; st < VD && st < NSTEP; ++st) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
  #pragma unroll
      for (int st = 0; st < NSTEP; ++st) {
        if (st + VD < NSTEP) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, kNQ, 1);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 pf1[kNQ];
#pragma unroll
        for (int n = 0; n < kNQ; ++n) {
          const bf16x4 a = __builtin_convertvector(sc[2 * c][n], bf16x4);
          const bf16x4 bq = __builtin_convertvector(sc[2 * c + 1][n], bf16x4);
          pf1[n] = bf16x8{a[0], a[1], a[2], a[3], bq[0], bq[1], bq[2], bq[3]};
        }
        const int krow = c * 32 + 4 * g + (r >> 2);
        const int ch_off = 4 * (r & 3);
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
          const int ch = jt * 16 + ch_off;
          // unit 2jt + (r mod 4)/2 of row krow, its four low bits XOR lswz(krow)
          // (krow mod 16 = 4g + r/4 whatever the chunk): a per-lane unit for
          // each jt mod 8 plus an immediate 16 (jt / 8)
          const int vu = VSW ? 16 * (jt >> 3) + ((2 * (jt & 7) + ((r & 3) >> 1)) ^ lswz(krow)) : (ch >> 3);
          const SSA_LDS char* base0 = (const SSA_LDS char*)(vslab + krow * UV + vu) + (ch & 7) * 2;
          const SSA_LDS char* base1 = base0 + 16 * UV * 16;  // rows krow + 16: the same swizzle
          const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SSA_LDS bf16x4*)base0);
          const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SSA_LDS bf16x4*)base1);
          const bf16x8 vf = bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
          for (int n = 0; n < kNQ; ++n)
            acc[jt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf1[n], acc[jt][n], 0, 0, 0);
        }
      }
    }
  };

  auto run = [&](auto mode_c) __attribute__((always_inline)) {
    if constexpr (NS == 2) {
      if (nst > 0) issue(0, slot_a);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      for (int s = 0; s < nst; s += 2) {
        if (s + 1 < nst) issue(s + 1, slot_b);
#pragma unroll
        for (int sub = 0; sub < SUBS; ++sub) compute(mode_c, s, slot_a, sub);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (s + 1 >= nst) break;
        if (s + 2 < nst) issue(s + 2, slot_a);
#pragma unroll
        for (int sub = 0; sub < SUBS; ++sub) compute(mode_c, s + 1, slot_b, sub);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    } else {
      for (int s = 0; s < nst; ++s) {
        issue(s, slot_a);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        compute(mode_c, s, slot_a, 0);
        __syncthreads();
      }
    }
  };
  run(std::integral_constant<int, 0>{});
  if constexpr (FIXREF) {
#pragma unroll
    for (int n = 0; n < kNQ; ++n) l[n] = xlane_sum(l[n]);
    // a weight above 2^64 (sums and outputs could then approach the fp32
    // range) shows as a row sum above 2^64, inf or NaN: then the whole
    // workgroup reruns the tile, first for the exact row maxima, then with
    // them as the reference (weights <= 1)
    bool bad = false;
#pragma unroll
    for (int n = 0; n < kNQ; ++n) bad |= !(l[n] <= 0x1p64f);
    if (__syncthreads_or(bad)) {
#pragma unroll
      for (int n = 0; n < kNQ; ++n) {
        m[n] = kNegInf;
        l[n] = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      run(std::integral_constant<int, 1>{});
      run(std::integral_constant<int, 2>{});
#pragma unroll
      for (int n = 0; n < kNQ; ++n) l[n] = xlane_sum(l[n]);
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

template <int DQK, int DV, bool SHARED, int NQ, bool DENSE, typename OutT>
hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.nqb) * p.B * p.Hq);
  return launch_kernel(prefill_wide_kernel<DQK, DV, SHARED, NQ, DENSE, OutT>, grid, dim3(kBlk / (16 * NQ) * 64), 0,
                       stream, p);
}

template <int DQK, int DV, bool SHARED, int NQ>
hipError_t launch_mode(const PrefillParams& p, bool out_f32, hipStream_t stream) {
  if (p.dense)
    return out_f32 ? launch_one<DQK, DV, SHARED, NQ, true, float>(p, stream)
                   : launch_one<DQK, DV, SHARED, NQ, true, __bf16>(p, stream);
  return out_f32 ? launch_one<DQK, DV, SHARED, NQ, false, float>(p, stream)
                 : launch_one<DQK, DV, SHARED, NQ, false, __bf16>(p, stream);
}

// NQS / NQA: 16-query tiles per wave with K and V shared / apart
template <int DQK, int DV, int NQS, int NQA>
hipError_t launch_dims(const PrefillParams& p, bool shared, bool out_f32, hipStream_t stream) {
  return shared ? launch_mode<DQK, DV, true, NQS>(p, out_f32, stream)
                : launch_mode<DQK, DV, false, NQA>(p, out_f32, stream);
}

}  // namespace

hipError_t launch_prefill_wide(const PrefillParams& p, int dqk, int dv, bool out_f32, hipStream_t stream) {
  const bool shared = p.v == p.k && p.vs_b == p.ks_b && p.vs_l == p.ks_l && p.vs_h == p.ks_h;
  if (dqk == 576 && dv == 512) return launch_dims<576, 512, 2, 1>(p, shared, out_f32, stream);
  if (dqk == 64 && dv == 64) return launch_dims<64, 64, 2, 2>(p, shared, out_f32, stream);
  return hipErrorNotSupported;
}

}  // namespace ssa
