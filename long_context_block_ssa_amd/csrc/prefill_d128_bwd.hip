// SSA backward on gfx950, bf16, Dqk = Dv = 128: the gradients of the
// block-sparse causal attention with respect to q, k and v.  The sparse
// operator needs a custom, deterministic backward for training (LongCat
// sparse attention article, section 4); LoZA converts its layers in
// mid-training (QbitAI report on LongCat LoZA).  With P the softmax of the
// masked scaled scores, recomputed from the forward's lse, and dO the
// incoming gradient of the output, the chain rule through o = P v and the
// softmax gives
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - delta),   delta_i = sum_c dO_ic O_ic,
//   dQ = scale dS K,   dK = scale dS^T Q.
//
// Kernels (one stream, in this order):
//   - dq: one workgroup per (query block, b, head), laid out like the
//     forward: the window's K and V stream through the LDS ring, S^T = K Q^T
//     and dP^T = V dO^T on 32x32x16 MFMAs with Q and dO in registers (one
//     query per lane), dQ^T += K^T dS^T with K^T read transposed
//     (ds_read_b64_tr_b16).  First it writes its rows' records: per (b,
//     head, 32-row stage) 64 floats, the stage's lse * log2(e), then its
//     -delta (rows past L: 0);
//   - dkdv: one workgroup per (key block, b, kv head) for the local blocks
//     and per (global block, part of its readers, b, kv head): each wave
//     keeps its 32 keys' K and V rows in registers, and the query stages
//     that read the key block -- the window's inverse map: the next n_local
//     query blocks, or every later block for a global block -- stream their
//     Q and dO rows and records through the ring, for every query head of
//     the kv head.  S = Q K^T and dP = dO V^T put one key per lane, so P and
//     dS are directly the B operands of dV^T += dO^T P and dK^T += Q^T dS
//     (dO^T and Q^T read transposed);
//   - reduce: a global block's partials summed in part order.
// No atomics: the result is bitwise deterministic.
#include "attn_d128.hpp"

#include <algorithm>

namespace ssa {
namespace {

using namespace d128;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRec = 64;               // floats per stage record
constexpr int kRingBytes = kSlots * kSlotBytes;  // 64 KB of Q/dO (or K/V) slabs
constexpr int kRecRegion = 1024;       // per wave and slot: the record, then 3 copies of it
constexpr int kDkdvLds = kRingBytes + kSlots * kWaves * kRecRegion;  // 80 KB

// vmcnt(5 k) alone: all but this wave's loads of the last k stages have
// landed (5 loads a stage: 4 row slabs and the record)
__device__ __forceinline__ void wait_stages5(int k) {
  if (k >= 2)
    __builtin_amdgcn_s_waitcnt(0x0F7A);
  else if (k == 1)
    __builtin_amdgcn_s_waitcnt(0x0F75);
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// the stage record's lse*log2(e) and -delta of the 16 query rows a lane holds
// (rows 8j + 4h .. +3 for j = 0..3): 8 reads at the wave's record region
template <int SLOT>
__device__ __forceinline__ void lds_read_rec(uint32_t a, f32x4 (&ls)[4], f32x4 (&dl)[4]) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:%9\n"
      "ds_read_b128 %1, %8 offset:%10\n"
      "ds_read_b128 %2, %8 offset:%11\n"
      "ds_read_b128 %3, %8 offset:%12\n"
      "ds_read_b128 %4, %8 offset:%13\n"
      "ds_read_b128 %5, %8 offset:%14\n"
      "ds_read_b128 %6, %8 offset:%15\n"
      "ds_read_b128 %7, %8 offset:%16\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(ls[0]), "=&v"(ls[1]), "=&v"(ls[2]), "=&v"(ls[3]), "=&v"(dl[0]), "=&v"(dl[1]), "=&v"(dl[2]),
        "=&v"(dl[3])
      : "v"(a), "i"(SLOT * kWaves * kRecRegion), "i"(SLOT * kWaves * kRecRegion + 32),
        "i"(SLOT * kWaves * kRecRegion + 64), "i"(SLOT * kWaves * kRecRegion + 96),
        "i"(SLOT * kWaves * kRecRegion + 128), "i"(SLOT * kWaves * kRecRegion + 160),
        "i"(SLOT * kWaves * kRecRegion + 192), "i"(SLOT * kWaves * kRecRegion + 224)
      : "memory");
}

#define SSA_DMA(src, dst) \
  __builtin_amdgcn_global_load_lds((const SSA_GLB void*)(src), (SSA_LDS void*)(dst), 16, 0, 0)

// ---------------------------------------------------------------------------
// dq: one workgroup per (query block, b, head), 4 waves x 32 queries
// ---------------------------------------------------------------------------
template <typename GradT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(BwdParams p) {
  __shared__ u32x4 ring[kRingBytes / 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h32 = lane >> 5, c32 = lane & 31;
  const int bh_count = p.B * p.Hq;
  const int qb = p.nqb - 1 - static_cast<int>(blockIdx.x) / bh_count;
  const int bh = static_cast<int>(blockIdx.x) % bh_count;
  const int b = bh / p.Hq, h = bh % p.Hq, hk = h / p.group;
  const int qoff = wave * 32;
  const int L = p.L;

  const __bf16* qbase = static_cast<const __bf16*>(p.q) + b * p.qs_b + h * p.qs_h;
  const __bf16* dobase = static_cast<const __bf16*>(p.dout) + b * p.dos_b + h * p.dos_h;
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + b * p.ks_b + hk * p.ks_h;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + b * p.vs_b + hk * p.vs_h;

  // the window of qb in ascending order, entry i on lane i
  const int g_end = min(p.n_global, qb + 1);
  const int l_begin = max(g_end, qb - p.n_local + 1);
  const int nblk = g_end + qb - l_begin + 1;
  const int blane = lane < g_end ? lane : (lane < nblk ? l_begin + lane - g_end : -1);
  const int nst = nblk * (kBlk / kSK);
  auto stage_block = [&](int s) -> int { return s < nst ? __builtin_amdgcn_readlane(blane, s >> 2) : -1; };

  // staging (the forward's): slab instruction j covers rows 4j .. 4j+3; wave
  // w issues j = w and j = w + 4 of the K slab and of the V slab
  const int drow = 4 * wave + (lane >> 4);
  const int dunit = (lane & 15) ^ swz(drow);
  const uint32_t koff = static_cast<uint32_t>(drow * p.ks_l + dunit * 8);
  const uint32_t voff = static_cast<uint32_t>(drow * p.vs_l + dunit * 8);
  const int64_t k16 = 16 * p.ks_l, v16 = 16 * p.vs_l;
  const uint32_t ring0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((SSA_LDS u32x4*)(ring)));
  // row fragment c (A operand): row c32, logical unit 2c + h32
  uint32_t faddr[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) faddr[c] = ring0 + (c32 * kUnits + ((2 * c + h32) ^ swz(c32))) * 16;
  // transposed fragment (dim tile dt, read e) of a slab: lane i of 16-lane
  // group g points at row 8e + 4(g/2) + i/4 (+16 for the second 16 rows),
  // channels 32dt + 16(g%2) + 4(i%4) .. +3
  uint32_t taddr[2][4];
  {
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int row = 8 * e + 4 * (g >> 1) + (i >> 2);
        const int ch = 32 * dt + 16 * (g & 1) + 4 * (i & 3);
        taddr[e][dt] = ring0 + (row * kUnits + ((ch >> 3) ^ swz(row))) * 16 + (ch & 7) * 2;
      }
  }

  // this lane's query column: Q and dO rows (B operands), lse and delta
  const int row = qb * kBlk + qoff + c32;
  bf16x8 qf[8], dof[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    u32x4 a = {0, 0, 0, 0}, d = {0, 0, 0, 0};
    if (row < L) {
      a = *reinterpret_cast<const u32x4*>(qbase + static_cast<int64_t>(row) * p.qs_l + c * 16 + h32 * 8);
      d = *reinterpret_cast<const u32x4*>(dobase + static_cast<int64_t>(row) * p.dos_l + c * 16 + h32 * 8);
    }
    qf[c] = __builtin_bit_cast(bf16x8, a);
    dof[c] = __builtin_bit_cast(bf16x8, d);
  }
  // the row's record: lse * log2 e and -delta, delta = rowsum(dO * O) (this
  // lane's 64 channels, then its partner's 32 lanes away); written for the
  // dk/dv kernel, whose dP MFMAs start from -delta (rows past L: zeros; a row
  // that admitted no key, lse = -inf, must give P = 0)
  float lse2 = 0.f, delta = 0.f;
  {
    float part = 0.f;
    if (row < L) {
      const __bf16* orow = static_cast<const __bf16*>(p.o) + b * p.os_b + h * p.os_h + static_cast<int64_t>(row) * p.os_l;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const u32x4 ov = *reinterpret_cast<const u32x4*>(orow + c * 16 + h32 * 8);
        const u32x4 dv = __builtin_bit_cast(u32x4, dof[c]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          part = __builtin_fmaf(__builtin_bit_cast(float, ov[w] << 16), __builtin_bit_cast(float, dv[w] << 16), part);
          part = __builtin_fmaf(__builtin_bit_cast(float, ov[w] & 0xFFFF0000u), __builtin_bit_cast(float, dv[w] & 0xFFFF0000u),
                                part);
        }
      }
      const float l = p.lse[static_cast<int64_t>(bh) * L + row];
      lse2 = l == -__builtin_inff() ? __builtin_inff() : l * kLog2e;
    }
    delta = part + __shfl_xor(part, 32);
    if (h32 == 0) {
      float* rec = p.rec + (static_cast<int64_t>(bh) * (p.nqb * 4) + row / kSK) * kRec;
      rec[row % kSK] = lse2;
      rec[kSK + row % kSK] = -delta;
    }
  }
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

  // stages are issued in order with QTR = s mod 4 known: a block's first K
  // and V rows are found at its quarter 0 and stepped by 32 rows after that
  const __bf16 *iss_k = kbase, *iss_v = vbase;
  int iss_key0 = 0;
  const int64_t k32 = kSK * p.ks_l, v32 = kSK * p.vs_l;
  auto issue = [&](auto qtr_tag, int s, int slot) {
    constexpr int QTR = decltype(qtr_tag)::value;
    if constexpr (QTR == 0) {
      const int kb = max(stage_block(s), 0);  // past the end: rows of block 0 nobody reads
      iss_key0 = kb * kBlk;
      iss_k = kbase + static_cast<int64_t>(iss_key0) * p.ks_l;
      iss_v = vbase + static_cast<int64_t>(iss_key0) * p.vs_l;
    } else {
      iss_key0 += kSK;
      iss_k += k32;
      iss_v += v32;
    }
    SSA_LDS u32x4* kd = (SSA_LDS u32x4*)(ring) + slot * (kSlotBytes / 16) + wave * 64;
    SSA_LDS u32x4* vd = kd + kSlab;
    if (iss_key0 + kSK <= L) {
      SSA_DMA(iss_k + koff, kd);
      SSA_DMA(iss_k + koff + k16, kd + 256);
      SSA_DMA(iss_v + voff, vd);
      SSA_DMA(iss_v + voff + v16, vd + 256);
    } else {
      const int64_t r0 = min(drow, L - 1 - iss_key0), r1 = min(drow + 16, L - 1 - iss_key0);
      SSA_DMA(iss_k + r0 * p.ks_l + dunit * 8, kd);
      SSA_DMA(iss_k + r1 * p.ks_l + dunit * 8, kd + 256);
      SSA_DMA(iss_v + r0 * p.vs_l + dunit * 8, vd);
      SSA_DMA(iss_v + r1 * p.vs_l + dunit * 8, vd + 256);
    }
  };

  auto stage = [&](auto slot_tag, auto steady_tag, int s, int ns, int nslot) {
    constexpr int SLOT = decltype(slot_tag)::value;
    constexpr bool STEADY = decltype(steady_tag)::value;  // ns < nst is known
    constexpr int OFF = SLOT * kSlotBytes;
    const int kb = stage_block(s);
    const int sub = s & 3;
    const int key0 = kb * kBlk + sub * kSK;
    const bool need = kb >= 0 && key0 < L && !(kb == qb && sub * kSK > qoff + 31);
    if (STEADY || ns < nst) issue(std::integral_constant<int, (SLOT + kSlots - 1) % kSlots>{}, ns, nslot);
    if (!need) return;
    f32x16 sc, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = dp[i] = 0.f;
    {
      u32x4 kraw[8];
      lds_read_k8<OFF>(faddr, kraw);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kraw[c]), qf[c], sc, 0, 0, 0);
    }
    {
      u32x4 vraw[8];
      lds_read_k8<OFF + kSlab * 16>(faddr, vraw);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vraw[c]), dof[c], dp, 0, 0, 0);
    }
    u32x2 kt[16];
    lds_read_vt16<OFF>(taddr, kt);  // K^T of the stage
    if (kb == qb || key0 + kSK > L) {
      const int lim = min(row, L - 1) - key0 - 4 * h32;  // last valid key offset
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) > lim) sc[i] = kNegInf;
    }
    // P^T = exp(scale s - lse), dS^T = P^T (dP^T - delta)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], p.c1, -lse2));
      dp[i] = pe * (dp[i] - delta);
    }
    bf16x8 df[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x4 a = __builtin_convertvector((f32x4){dp[8 * c], dp[8 * c + 1], dp[8 * c + 2], dp[8 * c + 3]}, bf16x4);
      const bf16x4 bq =
          __builtin_convertvector((f32x4){dp[8 * c + 4], dp[8 * c + 5], dp[8 * c + 6], dp[8 * c + 7]}, bf16x4);
      df[c] = bf16x8{a[0], a[1], a[2], a[3], bq[0], bq[1], bq[2], bq[3]};
    }
    // dQ^T += K^T dS^T: chunk c = keys 16c .. 16c+15 in the dS^T register order
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x4 t0 = __builtin_bit_cast(bf16x4, kt[c * 4 + dt]);
        const bf16x4 t1 = __builtin_bit_cast(bf16x4, kt[8 + c * 4 + dt]);
        const bf16x8 tf = bf16x8{t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf, df[c], acc[dt], 0, 0, 0);
      }
  };

  auto settle = [&](int s) {
    const int last = max(kSlots - 2, min(s + kSlots - 1, nst - 1));  // last stage issued
    wait_stages(last - (s + 1));
    stage_barrier();
  };

  for_each_stage<kSlots - 1>([&](auto i) { issue(i, decltype(i)::value, decltype(i)::value); });
  wait_stages(kSlots - 2);
  stage_barrier();
  const int nst_pad = (nst + kSlots - 1) & ~(kSlots - 1);
  int s0 = 0;
  // steady groups: every stage exists and issues the stage kSlots-1 ahead
  for (; s0 + 2 * kSlots - 2 < nst; s0 += kSlots) {
#define SSA_STAGE(k)                                                                                        \
  {                                                                                                         \
    const int s = s0 + (k);                                                                                 \
    stage(std::integral_constant<int, (k)>{}, std::true_type{}, s, s + kSlots - 1, ((k) + kSlots - 1) % kSlots); \
    wait_stages(kSlots - 2);                                                                              \
    stage_barrier();                                                                                        \
  }
    SSA_STAGE(0)
    SSA_STAGE(1)
    SSA_STAGE(2)
    SSA_STAGE(3)
#undef SSA_STAGE
  }
  for (; s0 < nst_pad; s0 += kSlots) {
#define SSA_STAGE(k)                                                                                        \
  {                                                                                                         \
    const int s = s0 + (k);                                                                                 \
    if (s < nst) stage(std::integral_constant<int, (k)>{}, std::false_type{}, s, s + kSlots - 1, ((k) + kSlots - 1) % kSlots); \
    settle(s);                                                                                              \
  }
    SSA_STAGE(0)
    SSA_STAGE(1)
    SSA_STAGE(2)
    SSA_STAGE(3)
#undef SSA_STAGE
  }

  if (row >= L) return;
  GradT* dqb = static_cast<GradT*>(p.dq) + b * p.dqs_b + h * p.dqs_h + static_cast<int64_t>(row) * p.dqs_l;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 v = {acc[dt][4 * k], acc[dt][4 * k + 1], acc[dt][4 * k + 2], acc[dt][4 * k + 3]};
      store4<GradT>(dqb + 32 * dt + 8 * k + 4 * h32, v * p.scale);
    }
}

// ---------------------------------------------------------------------------
// dk, dv: one workgroup per (key block[, part], b, kv head), 4 waves x 32 keys.
// The grid holds the global blocks' parts first (n_part_items workgroups,
// fp32 partials), then the local blocks, so one launch keeps every CU busy.
// ---------------------------------------------------------------------------
template <typename GradT>
__global__ __launch_bounds__(kWaves * 64) void bwd_dkdv_kernel(BwdParams p, int n_part_items) {
  extern __shared__ u32x4 ring[];  // kDkdvLds bytes: the slab ring, then the record regions

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h32 = lane >> 5, c32 = lane & 31;
  const int bh_count = p.B * p.Hkv;
  const int bh = static_cast<int>(blockIdx.x) % bh_count;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const int L = p.L;
  // the key block and the query blocks [q_begin, q_end) that read it
  const bool partial = static_cast<int>(blockIdx.x) < n_part_items;
  int kb, part = 0, q_begin, q_end;
  if (partial) {
    const int rest = static_cast<int>(blockIdx.x) / bh_count;
    part = rest % p.nparts;
    kb = rest / p.nparts;
    q_begin = kb + part * p.n_local;
    q_end = min(q_begin + p.n_local, p.nqb);
    if (q_begin >= q_end) return;  // a part past the last query block
  } else {
    kb = p.n_global + (static_cast<int>(blockIdx.x) - n_part_items) / bh_count;
    q_begin = kb;
    q_end = min(kb + p.n_local, p.nqb);
  }
  const int nq = q_end - q_begin;
  const int nst = p.group * nq * (kBlk / kSK);  // (query head of the group, query block, quarter)
  const int key = kb * kBlk + wave * 32 + c32;  // this lane's key (B-operand column)
  const bool wave_keys = kb * kBlk + wave * 32 < L;

  // K and V rows of this lane's key (B operands of S = Q K^T and dP = dO V^T)
  bf16x8 kf[8], vf[8];
  {
    const __bf16* kr = static_cast<const __bf16*>(p.k) + b * p.ks_b + hk * p.ks_h + static_cast<int64_t>(key) * p.ks_l;
    const __bf16* vr = static_cast<const __bf16*>(p.v) + b * p.vs_b + hk * p.vs_h + static_cast<int64_t>(key) * p.vs_l;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      u32x4 a = {0, 0, 0, 0}, d = {0, 0, 0, 0};
      if (key < L) {
        a = *reinterpret_cast<const u32x4*>(kr + c * 16 + h32 * 8);
        d = *reinterpret_cast<const u32x4*>(vr + c * 16 + h32 * 8);
      }
      kf[c] = __builtin_bit_cast(bf16x8, a);
      vf[c] = __builtin_bit_cast(bf16x8, d);
    }
  }

  // stage -> (query head of the group, first query row): the rows of a head's
  // stages run from q_begin*128 to q_end*128 in steps of 32 and the heads
  // follow in order, so two cursors (the stage being computed, the stage
  // being loaded) walk them with an add
  struct Cursor {
    int gi, q0;
  };
  const int row_begin = q_begin * kBlk, row_end = q_end * kBlk;
  auto advance = [&](Cursor& cu) -> bool {  // true when the head changes
    cu.q0 += kSK;
    if (cu.q0 != row_end) return false;
    cu.q0 = row_begin;
    ++cu.gi;
    return true;
  };
  Cursor cur_c = {0, row_begin}, iss_c = {0, row_begin};

  const int drow = 4 * wave + (lane >> 4);
  const int dunit = (lane & 15) ^ swz(drow);
  const uint32_t qoffs = static_cast<uint32_t>(drow * p.qs_l + dunit * 8);
  const uint32_t dooffs = static_cast<uint32_t>(drow * p.dos_l + dunit * 8);
  const int64_t q16 = 16 * p.qs_l, do16 = 16 * p.dos_l;
  const uint32_t ring0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((SSA_LDS u32x4*)(ring)));
  uint32_t faddr[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) faddr[c] = ring0 + (c32 * kUnits + ((2 * c + h32) ^ swz(c32))) * 16;
  uint32_t taddr[2][4];
  {
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int row = 8 * e + 4 * (g >> 1) + (i >> 2);
        const int ch = 32 * dt + 16 * (g & 1) + 4 * (i & 3);
        taddr[e][dt] = ring0 + (row * kUnits + ((ch >> 3) ^ swz(row))) * 16 + (ch & 7) * 2;
      }
  }
  // this wave's record region of slot 0; the rows of lane half h32 start 16 h32 bytes in
  const uint32_t raddr = ring0 + kRingBytes + wave * kRecRegion + 16 * h32;

  f32x16 dka[4], dva[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dka[dt][i] = dva[dt][i] = 0.f;

  // the loaded stage's Q and dO row pointers and its record, moved with iss_c
  const __bf16 *iss_q, *iss_d;
  const float* iss_r;
  auto point = [&]() {  // past the last head (never loaded): the first head's rows
    const int hq = hk * p.group + (iss_c.gi >= p.group ? 0 : iss_c.gi);
    const int q0 = iss_c.q0;
    iss_q = static_cast<const __bf16*>(p.q) + b * p.qs_b + hq * p.qs_h + static_cast<int64_t>(q0) * p.qs_l;
    iss_d = static_cast<const __bf16*>(p.dout) + b * p.dos_b + hq * p.dos_h + static_cast<int64_t>(q0) * p.dos_l;
    static_assert(kSK == 32, "a record per 32 query rows");
    iss_r = p.rec + (static_cast<int64_t>(b * p.Hq + hq) * (p.nqb * 4) + (q0 >> 5)) * kRec;
  };
  point();
  const int64_t qstep = static_cast<int64_t>(kSK) * p.qs_l, dstep = static_cast<int64_t>(kSK) * p.dos_l;

  auto issue = [&](int slot) {  // the stage under iss_c, which then moves on
    const int q0 = iss_c.q0;
    SSA_LDS u32x4* qd = (SSA_LDS u32x4*)(ring) + slot * (kSlotBytes / 16) + wave * 64;
    SSA_LDS u32x4* dd = qd + kSlab;
    SSA_LDS u32x4* rd = (SSA_LDS u32x4*)(ring) + (kRingBytes + (slot * kWaves + wave) * kRecRegion) / 16;
    if (q0 + kSK <= L) {
      SSA_DMA(iss_q + qoffs, qd);
      SSA_DMA(iss_q + qoffs + q16, qd + 256);
      SSA_DMA(iss_d + dooffs, dd);
      SSA_DMA(iss_d + dooffs + do16, dd + 256);
    } else {
      // rows at or past L repeat row L-1 (finite, masked later)
      const int64_t r0 = min(drow, L - 1 - q0), r1 = min(drow + 16, L - 1 - q0);
      SSA_DMA(iss_q + r0 * p.qs_l + dunit * 8, qd);
      SSA_DMA(iss_q + r1 * p.qs_l + dunit * 8, qd + 256);
      SSA_DMA(iss_d + r0 * p.dos_l + dunit * 8, dd);
      SSA_DMA(iss_d + r1 * p.dos_l + dunit * 8, dd + 256);
    }
    // the record: 16 lanes cover its 256 bytes, the other lanes repeat them
    SSA_DMA(iss_r + (lane & 15) * 4, rd);
    if (advance(iss_c)) {
      point();
    } else {
      iss_q += qstep;
      iss_d += dstep;
      iss_r += kRec;
    }
  };

  auto stage = [&](auto slot_tag, auto steady_tag, int s, int ns, int nslot) {
    constexpr int SLOT = decltype(slot_tag)::value;
    constexpr bool STEADY = decltype(steady_tag)::value;  // ns < nst is known
    constexpr int OFF = SLOT * kSlotBytes;
    const int q0 = cur_c.q0, qb = q0 >> 7;
    advance(cur_c);
    // nothing to do: no query of the stage reaches this wave's keys, or they do not exist
    const bool need = q0 < L && wave_keys && !(qb == kb && q0 + kSK - 1 < kb * kBlk + wave * 32);
    if (STEADY || ns < nst) issue(nslot);
    if (!need) return;
    // S = Q K^T and dP - delta = dO V^T - delta: 32 queries x this wave's 32
    // keys, one key per lane (the dP MFMAs start from the record's -delta)
    f32x16 sc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = 0.f;
    {
      u32x4 qr[8];
      lds_read_k8<OFF>(faddr, qr);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qr[c]), kf[c], sc, 0, 0, 0);
    }
    f32x4 ls[4], dl[4];
    lds_read_rec<SLOT>(raddr, ls, dl);
    f32x16 dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) dp[i] = dl[i >> 2][i & 3];
    {
      u32x4 dr[8];
      lds_read_k8<OFF + kSlab * 16>(faddr, dr);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, dr[c]), vf[c], dp, 0, 0, 0);
    }
    // register i holds query q0 + 8(i/4) + 4 h32 + (i%4): it must not precede the key and must exist
    if (qb == kb || q0 + kSK > L) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = q0 + 8 * (i >> 2) + 4 * h32 + (i & 3);
        if (qi < key || qi >= L) sc[i] = kNegInf;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sc[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], p.c1, -ls[i >> 2][i & 3]));  // P
      dp[i] = sc[i] * dp[i];                                                             // dS
    }
    bf16x8 pf[2], df[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x4 a = __builtin_convertvector((f32x4){sc[8 * c], sc[8 * c + 1], sc[8 * c + 2], sc[8 * c + 3]}, bf16x4);
      const bf16x4 a2 =
          __builtin_convertvector((f32x4){sc[8 * c + 4], sc[8 * c + 5], sc[8 * c + 6], sc[8 * c + 7]}, bf16x4);
      pf[c] = bf16x8{a[0], a[1], a[2], a[3], a2[0], a2[1], a2[2], a2[3]};
      const bf16x4 d = __builtin_convertvector((f32x4){dp[8 * c], dp[8 * c + 1], dp[8 * c + 2], dp[8 * c + 3]}, bf16x4);
      const bf16x4 d2 =
          __builtin_convertvector((f32x4){dp[8 * c + 4], dp[8 * c + 5], dp[8 * c + 6], dp[8 * c + 7]}, bf16x4);
      df[c] = bf16x8{d[0], d[1], d[2], d[3], d2[0], d2[1], d2[2], d2[3]};
    }
    // dV^T += dO^T P, then dK^T += Q^T dS: chunk c = queries 16c .. 16c+15 in the register order
    {
      u32x2 t[16];
      lds_read_vt16<OFF + kSlab * 16>(taddr, t);  // dO^T
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x4 t0 = __builtin_bit_cast(bf16x4, t[c * 4 + dt]);
          const bf16x4 t1 = __builtin_bit_cast(bf16x4, t[8 + c * 4 + dt]);
          const bf16x8 tf = bf16x8{t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
          dva[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf, pf[c], dva[dt], 0, 0, 0);
        }
    }
    {
      u32x2 t[16];
      lds_read_vt16<OFF>(taddr, t);  // Q^T
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x4 t0 = __builtin_bit_cast(bf16x4, t[c * 4 + dt]);
          const bf16x4 t1 = __builtin_bit_cast(bf16x4, t[8 + c * 4 + dt]);
          const bf16x8 tf = bf16x8{t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
          dka[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf, df[c], dka[dt], 0, 0, 0);
        }
    }
  };

  auto settle = [&](int s) {
    const int last = max(kSlots - 2, min(s + kSlots - 1, nst - 1));
    wait_stages5(last - (s + 1));
    stage_barrier();
  };

#pragma unroll
  for (int i = 0; i < kSlots - 1; ++i) {
    static_assert(kSlots - 1 <= kBlk / kSK, "the prologue's stages exist (nst >= 4)");
    issue(i);
  }
  wait_stages5(kSlots - 2);
  stage_barrier();
  const int nst_pad = (nst + kSlots - 1) & ~(kSlots - 1);
  int s0 = 0;
  // steady groups: every stage exists and issues the stage kSlots-1 ahead
  for (; s0 + 2 * kSlots - 2 < nst; s0 += kSlots) {
#define SSA_STAGE(k)                                                                                        \
  {                                                                                                         \
    const int s = s0 + (k);                                                                                 \
    stage(std::integral_constant<int, (k)>{}, std::true_type{}, s, s + kSlots - 1, ((k) + kSlots - 1) % kSlots); \
    wait_stages5(kSlots - 2);                                                                              \
    stage_barrier();                                                                                        \
  }
    SSA_STAGE(0)
    SSA_STAGE(1)
    SSA_STAGE(2)
    SSA_STAGE(3)
#undef SSA_STAGE
  }
  for (; s0 < nst_pad; s0 += kSlots) {
#define SSA_STAGE(k)                                                                                        \
  {                                                                                                         \
    const int s = s0 + (k);                                                                                 \
    if (s < nst) stage(std::integral_constant<int, (k)>{}, std::false_type{}, s, s + kSlots - 1, ((k) + kSlots - 1) % kSlots); \
    settle(s);                                                                                              \
  }
    SSA_STAGE(0)
    SSA_STAGE(1)
    SSA_STAGE(2)
    SSA_STAGE(3)
#undef SSA_STAGE
  }

  if (key >= L) return;
  // accumulators: lane = key, register i of tile dt = channel 32dt + 8(i/4) + 4 h32 + (i%4)
  if (partial) {
    float* out = p.part + ((((static_cast<int64_t>(kb) * p.nparts + part) * p.B + b) * p.Hkv + hk) * 2) * kBlk * kD +
                 static_cast<int64_t>(key - kb * kBlk) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 vk = {dka[dt][4 * k], dka[dt][4 * k + 1], dka[dt][4 * k + 2], dka[dt][4 * k + 3]};
        const f32x4 vv = {dva[dt][4 * k], dva[dt][4 * k + 1], dva[dt][4 * k + 2], dva[dt][4 * k + 3]};
        *reinterpret_cast<f32x4*>(out + 32 * dt + 8 * k + 4 * h32) = vk * p.scale;
        *reinterpret_cast<f32x4*>(out + kBlk * kD + 32 * dt + 8 * k + 4 * h32) = vv;
      }
  } else {
    GradT* dkr = static_cast<GradT*>(p.dk) + b * p.dks_b + hk * p.dks_h + static_cast<int64_t>(key) * p.dks_l;
    GradT* dvr = static_cast<GradT*>(p.dv) + b * p.dvs_b + hk * p.dvs_h + static_cast<int64_t>(key) * p.dvs_l;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 vk = {dka[dt][4 * k], dka[dt][4 * k + 1], dka[dt][4 * k + 2], dka[dt][4 * k + 3]};
        const f32x4 vv = {dva[dt][4 * k], dva[dt][4 * k + 1], dva[dt][4 * k + 2], dva[dt][4 * k + 3]};
        store4<GradT>(dkr + 32 * dt + 8 * k + 4 * h32, vk * p.scale);
        store4<GradT>(dvr + 32 * dt + 8 * k + 4 * h32, vv);
      }
  }
}

// ---------------------------------------------------------------------------
// reduce: dk / dv of the global blocks = the sum of their parts, in order;
// one thread per (global block, b, kv head, dk|dv, key row, 4 channels)
// ---------------------------------------------------------------------------
template <typename GradT>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdParams p, int n_glob) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int quad = static_cast<int>(gid % 32);
  const int r = static_cast<int>((gid / 32) % kBlk);
  const int which = static_cast<int>((gid / (32 * kBlk)) % 2);
  const int64_t rest = gid / (64 * kBlk);
  const int bh = static_cast<int>(rest % (p.B * p.Hkv));
  const int kb = static_cast<int>(rest / (p.B * p.Hkv));
  if (kb >= n_glob) return;
  const int key = kb * kBlk + r;
  if (key >= p.L) return;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const int np = min(p.nparts, (p.nqb - kb + p.n_local - 1) / p.n_local);  // parts that have readers
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int part = 0; part < np; ++part) {
    const float* src = p.part + ((((static_cast<int64_t>(kb) * p.nparts + part) * p.B + b) * p.Hkv + hk) * 2 + which) *
                                    kBlk * kD +
                       r * kD + quad * 4;
    s += *reinterpret_cast<const f32x4*>(src);
  }
  GradT* dst = which == 0 ? static_cast<GradT*>(p.dk) + b * p.dks_b + hk * p.dks_h + static_cast<int64_t>(key) * p.dks_l
                          : static_cast<GradT*>(p.dv) + b * p.dvs_b + hk * p.dvs_h + static_cast<int64_t>(key) * p.dvs_l;
  store4<GradT>(dst + quad * 4, s);
}

#undef SSA_DMA

template <typename GradT>
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  hipError_t e = launch_kernel(bwd_dq_kernel<GradT>, dim3(static_cast<unsigned>(p.nqb) * p.B * p.Hq),
                               dim3(kWaves * 64), 0, stream, p);
  if (e != hipSuccess) return e;
  const int n_glob = min(p.n_global, p.nqb);
  const unsigned bh = static_cast<unsigned>(p.B) * p.Hkv;
  const int n_part_items = n_glob * p.nparts * static_cast<int>(bh);
  const unsigned items = static_cast<unsigned>(n_part_items) + static_cast<unsigned>(p.nqb - n_glob) * bh;
  e = raise_lds_limit_once<bwd_dkdv_kernel<GradT>>(kDkdvLds);
  if (e != hipSuccess) return e;
  e = launch_kernel(bwd_dkdv_kernel<GradT>, dim3(items), dim3(kWaves * 64), kDkdvLds, stream, p, n_part_items);
  if (e != hipSuccess) return e;
  if (n_glob > 0) {
    const int64_t threads = static_cast<int64_t>(n_glob) * bh * 2 * kBlk * 32;
    e = launch_kernel(bwd_reduce_kernel<GradT>, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0,
                      stream, p, n_glob);
  }
  return e;
}

}  // namespace

size_t prefill_backward_workspace_bytes(int32_t B, int32_t L, int32_t Hq, int32_t Hkv, int32_t n_global,
                                        int32_t n_local) {
  const int64_t nqb = (static_cast<int64_t>(L) + kBlk - 1) / kBlk;
  const int64_t rec = static_cast<int64_t>(B) * Hq * nqb * 4 * kRec * sizeof(float);
  const int64_t n_glob = std::min<int64_t>(n_global, nqb);
  const int64_t nparts = (nqb + n_local - 1) / n_local;
  const int64_t part = n_glob * nparts * B * Hkv * 2 * kBlk * kD * static_cast<int64_t>(sizeof(float));
  return static_cast<size_t>((rec + 255) / 256 * 256 + part);
}

hipError_t launch_prefill_backward_d128(const BwdParams& p, bool grad_f32, hipStream_t stream) {
  return grad_f32 ? launch_bwd<float>(p, stream) : launch_bwd<__bf16>(p, stream);
}

}  // namespace ssa
