// Block-sparse causal attention prefill, fp32 path (D = 64), and the entry
// that dispatches every prefill shape.
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
// fp32 kernel: 16 queries per workgroup of 4 waves on v_mfma_f32_16x16x4f32,
// the waves splitting the key blocks.  A wave computes S^T = K Q^T per 16x16
// tile (A = K rows from LDS, B = Q^T from registers), so each lane owns one
// query column and 4 keys of it.  Each instruction contracts over 4 keys, so
// for O^T = V^T P^T the S^T elements a lane holds are exactly its P^T operand
// and V is read row-major from LDS.
//
// bf16 shapes: 128/128 runs the kernel of prefill_d128.hip,
// 64/64 and the latent-shared 576/512 the streaming kernel of
// prefill_wide.hip.
#include "common.hpp"

namespace ssa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 128;  // tokens per block == queries per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
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

__device__ __forceinline__ int list_count(const PrefillParams& p, int b, int h, int qb) {
  if (p.dense) return qb + 1;
  return min(p.cnt[b * p.cnt_sb + h * p.cnt_sh + qb], p.W);
}
__device__ __forceinline__ int list_entry(const PrefillParams& p, int b, int h, int qb, int s) {
  if (p.dense) return qb - s;  // own block first
  return p.idx[b * p.idx_sb + h * p.idx_sh + static_cast<int64_t>(qb) * p.W + s];
}


// ---------------------------------------------------------------------------
// f32 kernel (D = 64): one workgroup of 4 waves per 16 queries of a query
// block; the waves split the block's listed key blocks (entry s to wave
// s mod 4), each runs an online softmax over its blocks in 32-key chunks
// staged through its own LDS buffer (the next chunk's rows loaded into
// registers while the current one multiplies), and the four (o, m, l)
// pieces per query are merged exactly in LDS at the end.  Eight workgroups
// per query block instead of one: the small fp32 case (a few query blocks)
// spreads over 32x more SIMDs.
// ---------------------------------------------------------------------------
constexpr int kF32Queries = 16;  // queries per workgroup (one 16-wide MFMA tile)
constexpr int kF32Chunk = 32;    // keys per chunk

template <int D>
struct F32Stage {
  static constexpr int P = D + 4;  // padded row (floats)
  float k[kF32Chunk * P];
  float v[kF32Chunk * P];
};

template <int D>
__global__ __launch_bounds__(kThreads) void prefill_f32_kernel(PrefillParams p) {
  constexpr int NC = D / 4;   // contraction steps of 4 channels
  constexpr int NJ = D / 16;  // output tiles of 16 channels
  constexpr int P = F32Stage<D>::P;
  constexpr int UPR = D / 4;                    // 16-byte units per row
  constexpr int LPU = kF32Chunk * UPR / 64;     // units per lane and chunk (K or V)
  constexpr int GROUPS = kBlock / kF32Queries;  // workgroups per query block
  __shared__ F32Stage<D> st[kWaves];
  static_assert(sizeof(F32Stage<D>) * kWaves >= sizeof(float) * kWaves * (D * kF32Queries + 2 * kF32Queries),
                "the merge reuses the staging buffers");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  // tile order: query blocks from last to first, then the 16-query group,
  // heads fastest
  const int bh_count = p.B * p.Hq;
  const int t = blockIdx.x;
  const int qb = p.nqb - 1 - t / (bh_count * GROUPS);
  const int grp = (t / bh_count) % GROUPS;
  const int bh = t % bh_count;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int hk = h / p.group;
  const int q0 = qb * kBlock + grp * kF32Queries;  // first query of the tile
  const float* qbase = static_cast<const float*>(p.q) + b * p.qs_b + h * p.qs_h;
  const float* kbase = static_cast<const float*>(p.k) + b * p.ks_b + hk * p.ks_h;
  const float* vbase = static_cast<const float*>(p.v) + b * p.vs_b + hk * p.vs_h;
  F32Stage<D>& sm = st[wave];

  // B operand of v_mfma_f32_16x16x4f32: lane (r, g) holds Q[query r][4c + g]
  float qf[NC];
  {
    const int row = q0 + r;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = row < p.L ? qbase[row * p.qs_l + c * 4 + g] : 0.f;
  }
  float m = kNegInf, l = 0.f;  // query r: running max, this lane's share of the row sum
  f32x4 acc[NJ];               // O^T tile j: channels 16j + 4g .. +3 of query r
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this wave's chunks: entries s = wave, wave + 4, ..., 4 chunks of 32 keys
  // per block; chunks wholly past the tile's last query are left out
  const int nkb = p.nqb;
  const int count = list_count(p, b, h, qb);
  const int last_q = min(q0 + kF32Queries, p.L) - 1;
  auto chunk_key0 = [&](int i, int& key0) -> bool {  // i-th chunk of the wave (entry-major)
    const int s = wave + 4 * (i >> 2);
    if (s >= count) return false;
    const int kb = list_entry(p, b, h, qb, s);
    key0 = -1;
    if (kb < 0 || kb > qb || kb >= nkb) return true;  // entry skipped
    const int k0 = kb * kBlock + (i & 3) * kF32Chunk;
    if (k0 > last_q || k0 >= p.L) return true;        // no key of the chunk is visible
    key0 = k0;
    return true;
  };
  f32x4 kr[LPU], vr[LPU];
  auto load_chunk = [&](int key0) {
#pragma unroll
    for (int u = 0; u < LPU; ++u) {
      const int e = u * 64 + lane, row = e / UPR, ch = (e % UPR) * 4;
      const int key = min(key0 + row, p.L - 1);  // rows past L: finite data, masked below
      kr[u] = *reinterpret_cast<const f32x4*>(kbase + key * p.ks_l + ch);
      vr[u] = *reinterpret_cast<const f32x4*>(vbase + key * p.vs_l + ch);
    }
  };
  int cur = -1, i = 0;
  // first chunk with keys
  for (;; ++i) {
    int k0;
    if (!chunk_key0(i, k0)) break;
    if (k0 >= 0) {
      cur = k0;
      break;
    }
  }
  if (cur >= 0) load_chunk(cur);
  while (cur >= 0) {
    // the chunk's rows into the wave's buffer (the wave's LDS accesses are in order)
#pragma unroll
    for (int u = 0; u < LPU; ++u) {
      const int e = u * 64 + lane, row = e / UPR, ch = (e % UPR) * 4;
      *reinterpret_cast<f32x4*>(&sm.k[row * P + ch]) = kr[u];
      *reinterpret_cast<f32x4*>(&sm.v[row * P + ch]) = vr[u];
    }
    // next chunk with keys, its rows in flight during this one's products
    int nxt = -1;
    for (++i;; ++i) {
      int k0;
      if (!chunk_key0(i, k0)) break;
      if (k0 >= 0) {
        nxt = k0;
        break;
      }
    }
    if (nxt >= 0) load_chunk(nxt);
    // S^T = K Q^T: 2 tiles of 16 keys; lane (r, g) holds keys 16tt + 4g + i of query r
    f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        sc[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.k[(tt * 16 + r) * P + c * 4 + g], qf[c], sc[tt], 0, 0, 0);
    // causal rule and the end of the sequence
    const int qi = q0 + r;
    float mx = kNegInf;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = cur + tt * 16 + 4 * g + e;
        if (key > qi || key >= p.L) sc[tt][e] = kNegInf;
        mx = fmaxf(mx, sc[tt][e]);
      }
    mx = wave_max16x4(mx);
    // a query with no visible key so far keeps m = -inf and weights 0 (no
    // branch: the products below run for the whole wave)
    const float m_new = fmaxf(m, mx);
    const float alpha = m == kNegInf ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * p.c1);
    const float mc = m_new == kNegInf ? 0.f : m_new * p.c1;
    float rs = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float w = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[tt][e], p.c1, -mc));
        sc[tt][e] = w;
        rs += w;
      }
    l = l * alpha + rs;
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] *= alpha;
    m = m_new;
    // O^T += V^T P^T, 4 keys per instruction: lane group g supplies key
    // 16tt + 4g + e, which is exactly the S^T element it holds
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.v[(tt * 16 + g * 4 + e) * P + j * 16 + r], sc[tt][e],
                                                        acc[j], 0, 0, 0);
    cur = nxt;
  }

  // ---- merge the 4 waves' pieces per query ---------------------------------
  // piece of wave w: O^T [D][16] at part + w * (D + 2) * 16, then m[16], l[16]
  const float lt = wave_sum16x4(l);
  __syncthreads();  // every wave is done with its staging buffer
  float* part = reinterpret_cast<float*>(st);
  float* mine = part + wave * (D * kF32Queries + 2 * kF32Queries);
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) mine[(j * 16 + 4 * g + e) * kF32Queries + r] = acc[j][e];
  if (g == 0) {
    mine[D * kF32Queries + r] = m;
    mine[D * kF32Queries + kF32Queries + r] = lt;
  }
  __syncthreads();
  float* obase = static_cast<float*>(p.o) + b * p.os_b + h * p.os_h;
  for (int o_i = tid; o_i < D * kF32Queries; o_i += kThreads) {
    const int qq = o_i / D, d = o_i % D;  // consecutive threads: consecutive channels of one query
    const int row = q0 + qq;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, part[w * (D * kF32Queries + 2 * kF32Queries) + D * kF32Queries + qq]);
    float o = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* pw = part + w * (D * kF32Queries + 2 * kF32Queries);
      const float mw = pw[D * kF32Queries + qq];
      if (mw == kNegInf) continue;
      const float sc = __builtin_amdgcn_exp2f((mw - M) * p.c1);
      o = __builtin_fmaf(pw[d * kF32Queries + qq], sc, o);
      lsum = __builtin_fmaf(pw[D * kF32Queries + kF32Queries + qq], sc, lsum);
    }
    if (row >= p.L) continue;
    obase[row * p.os_l + d] = lsum > 0.f ? o / lsum : 0.f;
    if (p.lse && d == 0)
      p.lse[(static_cast<int64_t>(b) * p.Hq + h) * p.L + row] =
          lsum > 0.f ? M * p.scale + __builtin_amdgcn_logf(lsum) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int dtype, int dqk, int dv, bool out_f32, hipStream_t stream) {
  if (dtype == 0) {
    if (dqk != 64 || dv != 64) return hipErrorNotSupported;
    const dim3 grid(static_cast<unsigned>(p.nqb) * p.B * p.Hq * (kBlock / kF32Queries));
    return launch_kernel(prefill_f32_kernel<64>, grid, dim3(kThreads), 0, stream, p);
  }
  if (prefill_d128_supports(p, dqk, dv)) return launch_prefill_d128(p, out_f32, stream);
  return launch_prefill_wide(p, dqk, dv, out_f32, stream);
}

}  // namespace ssa
