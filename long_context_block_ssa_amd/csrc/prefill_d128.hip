// Block-sparse causal attention prefill, bf16, Dqk = Dv = 128, on gfx950.
//
// Within the key blocks listed for a query block (the SSA window: block 0 +
// the 7 most recent blocks, QbitAI report on LongCat LoZA; a page-selected
// list; or all blocks 0..qb for the dense layer) this is the masked softmax of
// equation (2) of the "LoZA: ZigZag sparse attention" page (section 2.1),
// causal in the own block (section 2.2.1), evaluated as an exact online
// softmax.
//
// Layout of the work:
//   - one workgroup = one 128-query block of one head: 4 waves of 32 queries,
//     two workgroups per CU, so each SIMD interleaves two waves;
//   - keys stream in 32-key stages through a 4-slot LDS ring filled with
//     global_load_lds_dwordx4 (global -> LDS, no registers), 3 stages in
//     flight, one barrier per stage; a stage's K fragments and V^T
//     fragments are read from LDS in one batch with one wait;
//   - S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16: each lane
//     owns one query column of the 32 x 32 tile and 16 of its keys, so the
//     row max needs one cross-lane swap (v_permlane32_swap) and the row sum
//     none until the end; P^T is the score accumulator converted to bf16;
//     V^T is read with ds_read_b64_tr_b16 in the key order the P^T registers
//     imply;
//   - rows are stored in LDS with the 16-byte units of row r XOR-permuted by
//     f(r) = 4 (r mod 4) + (r / 4 mod 4): the fragment reads (16 rows, one
//     unit) and the transposed reads (4 rows, 4 units) hit distinct banks,
//     and a 32-row slab is exactly 8 wave-wide DMA writes, two per wave;
//   - no rescaling inside the loop: a query column's reference max is the max
//     of the first stage that has a key for it (its accumulator and sum are
//     still zero then) and stays fixed, so later weights exp(s - ref) may
//     exceed 1.  The first pass computes no max once every column has its
//     reference; a weight above 2^64 (whose sums and outputs could approach
//     the fp32 range) then shows as a partial row sum above 2^64, inf or
//     NaN.  If any column of the workgroup shows one, the tile runs again
//     tracking the true max, and once more with it as the reference if it
//     ended more than 2^64 above the first.  Any fixed reference gives the
//     same normalised result, so this is exact.
//
// TOKENS: after the listed blocks come single tokens of the query block's
// token list (the second stage of hierarchical indexing), 32 per stage.  The
// list is copied to LDS once; each token stage's rows are gathered by the
// same direct-to-LDS loads, one row address per lane, and need no causal
// mask (every listed token precedes the block).
#include "attn_d128.hpp"

namespace ssa {
namespace {

using namespace d128;

constexpr float kHeadroom = 64.f;  // log2 growth of the max over the reference before a rerun
constexpr int kMaxTok = 1024;      // token-list capacity (TOKENS)

// the two token-list entries a lane stages in a token stage (rows e and e+16
// of the stage), read from the LDS copy of the list in an asm block that
// waits for them (see lds_read_k8 for why slot-area reads are not left to
// the compiler)
__device__ __forceinline__ void lds_read_tok2(uint32_t a, int& t0, int& t1) {
  asm volatile(
      "ds_read_b32 %0, %2\n"
      "ds_read_b32 %1, %2 offset:64\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(t0), "=&v"(t1)
      : "v"(a)
      : "memory");
}

// PAGED: chunked prefill over a paged cache.  The workgroup's tile is query
// block q0/128 + tile of the chunk q0 .. n-1 (q0 = n - T); a key block lives
// in page block_table[b][block]; queries and outputs are indexed by position
// - q0.  Everything else is the kernel above with L = n.
template <bool PAGED, bool TOKENS>
using KernelParams = std::conditional_t<PAGED, ChunkParams, std::conditional_t<TOKENS, TokenParams, PrefillParams>>;

template <typename OutT, bool DENSE, bool PAGED, bool TOKENS = false>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_d128_kernel(KernelParams<PAGED, TOKENS> p) {
  static_assert(!(DENSE && PAGED), "no dense layer over a paged cache");
  static_assert(!(TOKENS && (DENSE || PAGED)), "token lists go with block lists over a plain sequence");
  __shared__ u32x4 ring[kSlots * kSlotBytes / 16];
  extern __shared__ int32_t tokl[];  // TOKENS: the row's token list, padded to whole stages

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h32 = lane >> 5;  // which half of the 32-lane column pair
  const int c32 = lane & 31;
  // tile order: query blocks last to first (the dense layer's longest rows
  // first), then batch, heads fastest
  const int bh_count = p.B * p.Hq;
  const int tile = p.nqb - 1 - static_cast<int>(blockIdx.x) / bh_count;
  const int bh = static_cast<int>(blockIdx.x) % bh_count;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int hk = h / p.group;
  const int qoff = wave * 32;  // this wave's first query inside the block

  // a row that cannot be computed (a chunk without a valid sequence or page,
  // an invalid token list): NaN output and lse, stored as bit patterns (this
  // file is compiled without NaN semantics)
  auto nan_row = [&](int t) {
    if constexpr (PAGED || TOKENS) {
      OutT* obase = static_cast<OutT*>(p.o) + b * p.os_b + h * p.os_h;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          OutT* dst = obase + t * p.os_l + 32 * dt + 8 * k + 4 * h32;
          if constexpr (sizeof(OutT) == 4)
            *reinterpret_cast<u32x4*>(dst) = u32x4{0x7FC00000u, 0x7FC00000u, 0x7FC00000u, 0x7FC00000u};
          else
            *reinterpret_cast<u32x2*>(dst) = u32x2{0x7FC07FC0u, 0x7FC07FC0u};
        }
      if (p.lse && h32 == 0) {
        int64_t rows = p.L;
        if constexpr (PAGED) rows = p.T;
        reinterpret_cast<uint32_t*>(p.lse)[(static_cast<int64_t>(b) * p.Hq + h) * rows + t] = 0x7FC00000u;
      }
    }
  };
  int L = p.L, q0 = 0, qb = tile, nkb = p.nqb;  // keys [0, L); first query q0; key blocks [0, nkb)
  if constexpr (PAGED) {
    const int n = p.seq_lens[b];
    if (n < p.T || n > p.max_len) {  // no valid chunk: NaN rows tile*128 .. of this (b, h)
      const int t = tile * kBlk + qoff + c32;
      if (t < p.T) nan_row(t);
      return;
    }
    L = n;
    q0 = n - p.T;
    qb = q0 / kBlk + tile;
    nkb = (n + kBlk - 1) / kBlk;
    if (qb >= nkb) return;  // past the chunk's last block
  }

  const __bf16* qbase = static_cast<const __bf16*>(p.q) + b * p.qs_b + h * p.qs_h;
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + (PAGED ? 0 : b * p.ks_b) + hk * p.ks_h;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + (PAGED ? 0 : b * p.vs_b) + hk * p.vs_h;

  // ---- the block list, read once into registers (entry i on lane i of
  // every wave, fetched with readlane): a global read inside the stage loop
  // would make its wait also wait for the in-flight direct-to-LDS loads ----
  int nblk, blane = -1;
  if constexpr (DENSE) {
    nblk = qb + 1;  // own block first, then down to 0
  } else {
    nblk = min(p.cnt[b * p.cnt_sb + h * p.cnt_sh + qb], p.W);
    const int32_t* list = p.idx + b * p.idx_sb + h * p.idx_sh + static_cast<int64_t>(qb) * p.W;
    const int kb = lane < nblk ? list[lane] : -1;
    blane = (kb < 0 || kb > qb || kb >= nkb) ? -1 : kb;
  }
  // PAGED: page of list entry i on lane i (block 0's page for a skipped
  // entry, which stages rows nobody reads); a listed page or block 0's page
  // outside the pool makes every row of the tile NaN
  int plane = 0, page0 = 0;
  if constexpr (PAGED) {
    const int32_t* bt = p.block_table + b * p.bt_stride;
    page0 = bt[0];
    plane = blane >= 0 ? bt[blane] : page0;
    const bool bad = plane < 0 || plane >= p.num_pages || page0 < 0 || page0 >= p.num_pages;
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
      const int row = qb * kBlk + qoff + c32;
      if (row >= q0 && row < L) nan_row(row - q0);
      return;
    }
  }
  // TOKENS: the token list of the row, checked and copied to LDS.  Entries
  // must be ascending, precede the query block and lie outside every listed
  // block; otherwise every row of the tile is NaN.  Entries past the count up
  // to the end of its last stage repeat the last token (staged, masked).
  int ntok = 0;
  if constexpr (TOKENS) {
    ntok = min(max(p.tcnt[b * p.tcnt_sb + h * p.tcnt_sh + qb], 0), p.K);
    const int32_t* tl = p.tok + b * p.tok_sb + h * p.tok_sh + static_cast<int64_t>(qb) * p.K;
    const int npad = (ntok + kSK - 1) & ~(kSK - 1);
    bool bad = false;
#pragma unroll
    for (int j = 0; j < kMaxTok / (kWaves * 64); ++j) {
      const int e = tid + kWaves * 64 * j;
      if (e < ntok) {
        const int t = tl[e];
        const int prev = e > 0 ? tl[e - 1] : -1;
        bad |= t <= prev || t >= qb * kBlk;
        for (int i = 0; i < nblk; ++i) bad |= __builtin_amdgcn_readlane(blane, i) == (t >> 7);
        tokl[e] = t;
      } else if (e < npad) {
        tokl[e] = tl[ntok - 1];
      }
    }
    if (__syncthreads_or(bad)) {
      const int row = qb * kBlk + qoff + c32;
      if (row < L) nan_row(row);
      return;
    }
  }
  const int nbs = nblk * (kBlk / kSK);  // block stages; token stages follow
  const int nst = nbs + (ntok + kSK - 1) / kSK;
  // block of stage s; -1 for a skipped list entry, a token stage and stages
  // past the end
  auto stage_block = [&](int s) -> int {
    if (s >= nbs) return -1;
    if constexpr (DENSE) return qb - (s >> 2);
    return __builtin_amdgcn_readlane(blane, s >> 2);
  };

  // ---- per-lane constants -----------------------------------------------
  // DMA: slab instruction j covers rows 4j .. 4j+3 (row 4j + lane/16; the lane
  // on physical unit lane%16 loads logical unit (lane%16) ^ f(row)); wave w
  // issues j = w and j = w + 4 of the K slab and of the V slab, whose rows
  // (16 apart) share f
  const int drow = 4 * wave + (lane >> 4);
  const int dunit = (lane & 15) ^ swz(drow);
  const uint32_t koff = static_cast<uint32_t>(drow * p.ks_l + dunit * 8);
  const uint32_t voff = static_cast<uint32_t>(drow * p.vs_l + dunit * 8);
  const int64_t k16 = 16 * p.ks_l, v16 = 16 * p.vs_l;
  const uint32_t ring0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((SSA_LDS u32x4*)(ring)));
  const uint32_t tok0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((SSA_LDS int32_t*)(tokl))) + 4 * drow;
  // K fragment c (A operand): row c32, logical unit 2c + h32
  uint32_t kaddr[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) kaddr[c] = ring0 + (c32 * kUnits + ((2 * c + h32) ^ swz(c32))) * 16;
  // V^T fragment (dim tile dt, read e): lane i of 16-lane group g points at
  // key 8e + 4(g/2) + i/4 (+ 16 for the second 16-key chunk), channels
  // 32dt + 16(g%2) + 4(i%4) .. +3
  uint32_t vaddr[2][4];
  {
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int row = 8 * e + 4 * (g >> 1) + (i >> 2);
        const int ch = 32 * dt + 16 * (g & 1) + 4 * (i & 3);
        vaddr[e][dt] = ring0 + (kSlab + row * kUnits + ((ch >> 3) ^ swz(row))) * 16 + (ch & 7) * 2;
      }
  }

  // ---- queries (B operand of S^T = K Q^T) -------------------------------
  bf16x8 qf[8];
  {
    const int row = qb * kBlk + qoff + c32;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      u32x4 v = {0, 0, 0, 0};
      if (row >= q0 && row < L) v = *reinterpret_cast<const u32x4*>(qbase + (row - q0) * p.qs_l + c * 16 + h32 * 8);
      qf[c] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // m: reference max of this lane's query column (raw score units),
  // mt: true max so far
  float m = kNegInf, mt = kNegInf, l;
  bool track = false;  // track the true max mt (reruns only)
  f32x16 acc[4];

  // ---- staging: this wave's four loads of stage s into ring slot `slot` ---
  // Stages are issued in order and QTR = s mod 4 is known where they are
  // issued, so (non-paged) the first row of a block's K and V is found once,
  // at its quarter 0, and stepped by 32 rows for the other three.
  const __bf16 *iss_k = kbase, *iss_v = vbase;
  int iss_key0 = 0;
  const int64_t k32 = kSK * p.ks_l, v32 = kSK * p.vs_l;
  auto issue = [&](auto qtr_tag, int s, int slot) {
    constexpr int QTR = decltype(qtr_tag)::value;
    SSA_LDS u32x4* kd = (SSA_LDS u32x4*)(ring) + slot * (kSlotBytes / 16) + wave * 64;
    SSA_LDS u32x4* vd = kd + kSlab;
#define SSA_DMA(src, dst) \
  __builtin_amdgcn_global_load_lds((const SSA_GLB void*)(src), (SSA_LDS void*)(dst), 16, 0, 0)
    if constexpr (PAGED) {
      // block kb lives in its page: the stage takes rows 32 QTR .. 32 QTR + 31 of it
      const int sb = stage_block(s);
      // iss_key0: the stage's first key; iss_k, iss_v: its first row in the page
      if constexpr (QTR == 0) {
        const int kb = max(sb, 0);  // skipped entries stage block 0 (unused)
        const int pg = sb >= 0 ? __builtin_amdgcn_readlane(plane, s >> 2) : page0;
        iss_key0 = kb * kBlk;
        iss_k = kbase + static_cast<int64_t>(pg) * p.ks_b;
        iss_v = vbase + static_cast<int64_t>(pg) * p.vs_b;
      } else {
        iss_key0 += kSK;
        iss_k += k32;
        iss_v += v32;
      }
      if (iss_key0 + kSK <= L) {
        SSA_DMA(iss_k + koff, kd);
        SSA_DMA(iss_k + koff + k16, kd + 256);
        SSA_DMA(iss_v + voff, vd);
        SSA_DMA(iss_v + voff + v16, vd + 256);
      } else {
        // the sequence's last block: rows at or past n repeat row n-1
        const int last = L - 1 - iss_key0;
        const int64_t ra = min(drow, last), rb = min(drow + 16, last);
        SSA_DMA(iss_k + ra * p.ks_l + dunit * 8, kd);
        SSA_DMA(iss_k + rb * p.ks_l + dunit * 8, kd + 256);
        SSA_DMA(iss_v + ra * p.vs_l + dunit * 8, vd);
        SSA_DMA(iss_v + rb * p.vs_l + dunit * 8, vd + 256);
      }
    } else {
      if constexpr (TOKENS) {
        if (s >= nbs && s < nst) {  // a token stage: rows are list entries 32(s - nbs) ..
          int ta, tb;
          lds_read_tok2(tok0 + 4 * kSK * (s - nbs), ta, tb);
          SSA_DMA(kbase + static_cast<int64_t>(ta) * p.ks_l + dunit * 8, kd);
          SSA_DMA(kbase + static_cast<int64_t>(tb) * p.ks_l + dunit * 8, kd + 256);
          SSA_DMA(vbase + static_cast<int64_t>(ta) * p.vs_l + dunit * 8, vd);
          SSA_DMA(vbase + static_cast<int64_t>(tb) * p.vs_l + dunit * 8, vd + 256);
          return;
        }
      }
      if constexpr (QTR == 0 || DENSE) {  // (the dense layer: no registers to spare)
        const int kb = max(stage_block(s), 0);  // skipped entries stage block 0 (unused)
        iss_key0 = kb * kBlk + QTR * kSK;
        iss_k = kbase + static_cast<int64_t>(iss_key0) * p.ks_l;
        iss_v = vbase + static_cast<int64_t>(iss_key0) * p.vs_l;
      } else {
        iss_key0 += kSK;
        iss_k += k32;
        iss_v += v32;
      }
      if (iss_key0 + kSK <= p.L) {
        SSA_DMA(iss_k + koff, kd);
        SSA_DMA(iss_k + koff + k16, kd + 256);
        SSA_DMA(iss_v + voff, vd);
        SSA_DMA(iss_v + voff + v16, vd + 256);
      } else {
        // last block of a ragged L: rows at or past L repeat row L-1 (finite, masked later)
        const int64_t r0 = min(drow, p.L - 1 - iss_key0), r1 = min(drow + 16, p.L - 1 - iss_key0);
        SSA_DMA(iss_k + r0 * p.ks_l + dunit * 8, kd);
        SSA_DMA(iss_k + r1 * p.ks_l + dunit * 8, kd + 256);
        SSA_DMA(iss_v + r0 * p.vs_l + dunit * 8, vd);
        SSA_DMA(iss_v + r1 * p.vs_l + dunit * 8, vd + 256);
      }
    }
#undef SSA_DMA
  };

  int cur_kb = -1;  // the block of the stage being computed
  // ---- one stage: keys of stage s in ring slot SLOT; first this wave's
  // loads of stage ns (if any) into slot nslot ------------------------------
  auto stage = [&](auto slot_tag, auto steady_tag, int s, int ns, int nslot) {
    constexpr int SLOT = decltype(slot_tag)::value;
    constexpr bool STEADY = decltype(steady_tag)::value;  // ns < nst is known
    constexpr int OFF = SLOT * kSlotBytes;
    const bool tst = TOKENS && s >= nbs;  // a token stage
    // stages come in order with s mod 4 = SLOT: a block's list entry is read at its first quarter
    if constexpr (SLOT == 0) cur_kb = stage_block(s);
    const int kb = cur_kb;
    constexpr int sub = SLOT;
    const int key0 = kb * kBlk + sub * kSK;
    const bool need = tst || (kb >= 0 && key0 < L && !(kb == qb && sub * kSK > qoff + 31));
    if (STEADY || ns < nst) issue(std::integral_constant<int, (SLOT + kSlots - 1) % kSlots>{}, ns, nslot);
    if (!need) return;
    // S^T = K Q^T: 32 keys x 32 queries
    f32x16 sc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = 0.f;
    // K and V^T of the stage in one batch of LDS reads
    u32x2 vraw[16];
    {
      u32x4 kraw[8];
      lds_read_kv<OFF>(kaddr, vaddr, kraw, vraw);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kraw[c]), qf[c], sc, 0, 0, 0);
    }
    // token stage: entries at or past the count
    if (tst) {
      const int lim = ntok - 1 - (s - nbs) * kSK - 4 * h32;  // last valid entry offset
      if ((s - nbs + 1) * kSK > ntok) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i >> 2) + (i & 3) > lim) sc[i] = kNegInf;
      }
    } else if (kb == qb || key0 + kSK > L) {  // own block: key > query; keys at or past L
      const int qi = qb * kBlk + qoff + c32;
      const int lim = min(qi, L - 1) - key0 - 4 * h32;  // last valid key offset
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) > lim) sc[i] = kNegInf;
    }
    // softmax with a fixed reference max.  The column max is needed only
    // until every column of the wave has its reference, or when the true max
    // is tracked (a rerun)
    if (track || __builtin_amdgcn_ballot_w64(m == kNegInf) != 0) {
      float a8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) a8[i] = fmaxf(sc[i], sc[i + 8]);
#pragma unroll
      for (int i = 0; i < 4; ++i) a8[i] = fmaxf(a8[i], a8[i + 4]);
      const float mx = pair_max(fmaxf(fmaxf(a8[0], a8[1]), fmaxf(a8[2], a8[3])));
      mt = fmaxf(mt, mx);
      if (m == kNegInf) m = mx;  // first keys of this column: nothing to rescale
    }
    // a column with no key seen yet keeps m = -inf: its scores are all -inf
    const float mc = m == kNegInf ? 0.f : m * p.c1;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], p.c1, -mc));
    float r8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r8[i] = sc[i] + sc[i + 8];
#pragma unroll
    for (int i = 0; i < 4; ++i) r8[i] += r8[i + 4];
    l += (r8[0] + r8[1]) + (r8[2] + r8[3]);
    bf16x8 pf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x4 a = __builtin_convertvector((f32x4){sc[8 * c], sc[8 * c + 1], sc[8 * c + 2], sc[8 * c + 3]}, bf16x4);
      const bf16x4 bq =
          __builtin_convertvector((f32x4){sc[8 * c + 4], sc[8 * c + 5], sc[8 * c + 6], sc[8 * c + 7]}, bf16x4);
      pf[c] = bf16x8{a[0], a[1], a[2], a[3], bq[0], bq[1], bq[2], bq[3]};
    }
    // O^T += V^T P^T: chunk c = keys 16c .. 16c+15 in the P^T register order
    const u32x2* v0raw = vraw;      // [c * 4 + dt]: reads e = 0
    const u32x2* v1raw = vraw + 8;  // and e = 1
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x4 v0 = __builtin_bit_cast(bf16x4, v0raw[c * 4 + dt]);
        const bf16x4 v1 = __builtin_bit_cast(bf16x4, v1raw[c * 4 + dt]);
        const bf16x8 vf = bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[c], acc[dt], 0, 0, 0);
      }
  };

  // stage s + 1 must have landed (this wave's loads), then every wave's
  auto settle = [&](int s) {
    const int last = max(kSlots - 2, min(s + kSlots - 1, nst - 1));  // last stage issued
    wait_stages(last - (s + 1));
    stage_barrier();
  };

  for (int pass = 0; pass < 3; ++pass) {
    track = pass > 0;
    l = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
    // prologue: stages 0 .. 2 in flight.  They are issued whether or not they
    // exist (a stage past the end stages rows of block 0 into a slot nobody
    // reads), so the number of loads behind the queries is fixed and the
    // compiler's wait for them is exact.
    for_each_stage<kSlots - 1>([&](auto i) { issue(i, decltype(i)::value, decltype(i)::value); });
    wait_stages(kSlots - 2);  // stage 0
    stage_barrier();
    // Whole groups of 4 stages, so that the loop is left only at its end;
    // stages past the end only take the barrier.
    const int nst_pad = (nst + kSlots - 1) & ~(kSlots - 1);
    int s0 = 0;
    // steady groups: every stage exists and issues the stage kSlots-1 ahead,
    // so the wait before the next stage is always "kSlots-2 stages still in
    // flight" (no runtime choice of the wait, no existence tests)
    for (; s0 + 2 * kSlots - 2 < nst; s0 += kSlots) {
#define SSA_STAGE(k)                                                                          \
  {                                                                                           \
    const int s = s0 + (k);                                                                   \
    stage(std::integral_constant<int, (k)>{}, std::true_type{}, s, s + kSlots - 1, ((k) + kSlots - 1) % kSlots); \
    wait_stages(kSlots - 2);                                                                  \
    stage_barrier();                                                                          \
  }
      SSA_STAGE(0)
      SSA_STAGE(1)
      SSA_STAGE(2)
      SSA_STAGE(3)
#undef SSA_STAGE
    }
    for (; s0 < nst_pad; s0 += kSlots) {
#define SSA_STAGE(k)                                                                 \
  {                                                                                  \
    const int s = s0 + (k);                                                          \
    if (s < nst) stage(std::integral_constant<int, (k)>{}, std::false_type{}, s, s + kSlots - 1, ((k) + kSlots - 1) % kSlots); \
    settle(s);                                                                       \
  }
      SSA_STAGE(0)
      SSA_STAGE(1)
      SSA_STAGE(2)
      SSA_STAGE(3)
#undef SSA_STAGE
    }
    // the max grew too far above the reference somewhere in the workgroup:
    // run the tile again with the true max as the reference
    // pass 0 does not know the true max: a weight above 2^64 shows as a
    // partial row sum above 2^64 (or inf / NaN), and then pass 1 runs the
    // tile again tracking the max; if that max grew too far above the
    // reference, pass 2 uses it as the reference
    const bool far = pass == 0 ? !(l <= 18446744073709551616.f) : (mt - m) * p.c1 > kHeadroom;
    if (pass == 2) break;
    // workgroup vote through the (now idle) ring: every load has landed and
    // every wave is past the last barrier
    int* vote = reinterpret_cast<int*>(ring);
    if (tid == 0) *vote = 0;
    __syncthreads();
    if (far) *vote = 1;
    __syncthreads();
    const bool any = *vote != 0;
    __syncthreads();  // every wave has read the vote before the ring is refilled
    if (!any) break;
    if (pass == 0) {
      m = kNegInf;
      mt = kNegInf;
    } else {
      m = mt;
    }
  }

  // ---- output ------------------------------------------------------------
  OutT* obase = static_cast<OutT*>(p.o) + b * p.os_b + h * p.os_h;
  const float lt = pair_sum(l);
  const int row = qb * kBlk + qoff + c32;
  if (row < q0 || row >= L) return;
  const int t = row - q0;  // output row (the position itself unless PAGED)
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 v = {acc[dt][4 * k], acc[dt][4 * k + 1], acc[dt][4 * k + 2], acc[dt][4 * k + 3]};
      store4<OutT>(obase + t * p.os_l + 32 * dt + 8 * k + 4 * h32, v * inv);
    }
  if (p.lse && h32 == 0) {
    const float v = lt > 0.f ? m * p.scale + __builtin_amdgcn_logf(lt) * kLn2 : kNegInf;
    int64_t rows = p.L;  // lse row length: L, or the chunk length T
    if constexpr (PAGED) rows = p.T;
    p.lse[(static_cast<int64_t>(b) * p.Hq + h) * rows + t] = v;
  }
}

template <typename OutT, bool DENSE, bool PAGED = false>
hipError_t launch_d128(const KernelParams<PAGED, false>& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.nqb) * p.B * p.Hq);
  return launch_kernel(prefill_d128_kernel<OutT, DENSE, PAGED>, grid, dim3(kWaves * 64), 0, stream, p);
}

template <typename OutT>
hipError_t launch_d128_tokens(const TokenParams& p, hipStream_t stream) {
  constexpr auto kern = prefill_d128_kernel<OutT, false, false, true>;
  const size_t lds = sizeof(int32_t) * ((p.K + kSK - 1) & ~(kSK - 1));
  hipError_t e = raise_lds_limit_once<kern>(static_cast<int>(sizeof(int32_t) * kMaxTok));
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>(p.nqb) * p.B * p.Hq);
  return launch_kernel(kern, grid, dim3(kWaves * 64), lds, stream, p);
}

}  // namespace

bool prefill_d128_supports(const PrefillParams& p, int dqk, int dv) {
  return dqk == kD && dv == kD && (p.dense || p.W <= kMaxW);
}

hipError_t launch_prefill_d128(const PrefillParams& p, bool out_f32, hipStream_t stream) {
  if (p.dense) return out_f32 ? launch_d128<float, true>(p, stream) : launch_d128<__bf16, true>(p, stream);
  return out_f32 ? launch_d128<float, false>(p, stream) : launch_d128<__bf16, false>(p, stream);
}

hipError_t launch_prefill_tokens_d128(const TokenParams& p, bool out_f32, hipStream_t stream) {
  if (p.W > kMaxW || p.K < 0 || p.K > kMaxTok) return hipErrorNotSupported;
  return out_f32 ? launch_d128_tokens<float>(p, stream) : launch_d128_tokens<__bf16>(p, stream);
}

hipError_t launch_prefill_chunk_d128(const ChunkParams& p, bool out_f32, hipStream_t stream) {
  if (p.W > kMaxW) return hipErrorNotSupported;
  return out_f32 ? launch_d128<float, false, true>(p, stream) : launch_d128<__bf16, false, true>(p, stream);
}

}  // namespace ssa
