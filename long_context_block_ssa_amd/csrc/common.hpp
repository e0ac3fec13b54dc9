// Internal declarations shared by the C-ABI layer and the gfx950 kernels.
// Nothing here is part of the public interface (include/ssa.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <tuple>
#include <type_traits>
#include <utility>

namespace ssa {

// Launch through hipLaunchKernel so that the launch's own status is returned
// (hipGetLastError would also report errors left over by unrelated calls).
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                         Args&&... args) {
  std::tuple<KArgs...> held(std::forward<Args>(args)...);
  return std::apply(
      [&](auto&... a) {
        void* ptrs[] = {static_cast<void*>(&a)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs, shmem, stream);
      },
      held);
}

// Raise the dynamic-LDS limit of kernel KERN to `bytes` (the largest any call
// may pass) once per device.  The limit is a process-wide attribute of the
// function: setting it on every call with that call's own size would let one
// host thread lower it between another thread's set and launch.
constexpr int kMaxDevices = 64;
template <auto KERN>
hipError_t raise_lds_limit_once(int bytes) {
  static std::once_flag once[kMaxDevices];
  static hipError_t status[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [&] {
    status[dev] = hipFuncSetAttribute(reinterpret_cast<const void*>(KERN),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  });
  return status[dev];
}

// ---------------------------------------------------------------------------
// launch parameter blocks (plain structs passed by value to kernels)
// ---------------------------------------------------------------------------

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t qs_b, qs_l, qs_h;
  int64_t ks_b, ks_l, ks_h;
  int64_t vs_b, vs_l, vs_h;
  int64_t os_b, os_l, os_h;
  int32_t B, L, Hq, Hkv, group;  // group = Hq / Hkv
  int32_t nqb;                   // ceil(L / 128)
  float c1;                      // scale * log2(e): exp(scale*s) == exp2(c1*s)
  float scale;
  // block lists; dense != 0 means "every block 0 .. qb" and the list is unused
  const int32_t* idx;
  const int32_t* cnt;
  int32_t W;
  int32_t dense;
  int64_t idx_sb, idx_sh, cnt_sb, cnt_sh;
};

// Chunked prefill over a paged cache: the k/v strides (ks_b, ks_h, ks_l) are
// (page, head, slot); nqb counts query-block tiles per (b, h); the chunk of
// sequence b is positions seq_lens[b] - T .. seq_lens[b] - 1; L is unused.
struct ChunkParams : PrefillParams {
  const int32_t* block_table;
  const int32_t* seq_lens;
  int64_t bt_stride;
  int32_t T, num_pages, max_len;
};

// Attention over listed key blocks plus listed single tokens of each query
// block (the second stage of hierarchical indexing): row (b, h, qb) of the
// token list is tok[b*tok_sb + h*tok_sh + qb*K + e], e < tcnt[b*tcnt_sb +
// h*tcnt_sh + qb].
struct TokenParams : PrefillParams {
  const int32_t* tok;
  const int32_t* tcnt;
  int32_t K;
  int64_t tok_sb, tok_sh, tcnt_sb, tcnt_sh;
};

// Second stage of hierarchical indexing: page lists as page selection writes
// them (contiguous [B, Hq, nqb, PW] and [B, Hq, nqb]), the fp64 query-block
// sums of page selection, token lists out (contiguous [B, Hq, nqb, K] and
// [B, Hq, nqb]).  Workspace (R = B*Hq*nqb rows, S = slots per row = top_m):
// per (b, h, page) recall counts and bucket offsets, per row the candidate
// pages, the buckets (which rows recalled a page, and in which slot), and per
// row S*128 score keys.
struct TokenSelectParams {
  const void* k;
  int64_t ks_b, ks_l, ks_h;
  const double* qsum;  // [B, Hq, nqb, D]
  const int32_t* pidx;
  const int32_t* pcnt;
  int32_t PW, S;
  int32_t B, Hq, Hkv, group, D, nqb;
  int32_t n_global, n_local, K;
  int32_t* tok;
  int32_t* tcnt;
  int32_t* cnt;    // [R] recalls of page (b, h, c)
  int32_t* off;    // [R] bucket start of page (b, h, c) inside the (b, h) region of ent
  int32_t* npg;    // [R] candidate pages of row (b, h, qb); 0 once the row is final
  int32_t* pages;  // [R, S] ascending candidate pages
  int32_t* ent;    // [B*Hq, nqb*S] bucket entries qb*S + slot
  uint64_t* keys;  // [R, S*128] order-preserving score keys
};
size_t token_select_workspace_bytes(int32_t B, int32_t Hq, int32_t nqb, int32_t S);

// SSA backward, bf16, Dqk = Dv = 128.  lse is the forward's natural-log sum
// of exponentials [B, Hq, L]; the workspace holds, per (b, query head, stage
// of 32 queries), a 64-float record: lse * log2(e) of the 32 rows, then
// delta = rowsum(dout * o) of the 32 rows (rows past L: 0), and after the
// records the fp32 partial dk / dv of the global blocks.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int64_t qs_b, qs_l, qs_h;
  int64_t ks_b, ks_l, ks_h;
  int64_t vs_b, vs_l, vs_h;
  int64_t os_b, os_l, os_h;
  int64_t dos_b, dos_l, dos_h;
  int64_t dqs_b, dqs_l, dqs_h;
  int64_t dks_b, dks_l, dks_h;
  int64_t dvs_b, dvs_l, dvs_h;
  int32_t B, L, Hq, Hkv, group;
  int32_t nqb;               // ceil(L / 128)
  int32_t n_global, n_local; // the window
  int32_t nparts;            // query-block parts of global block 0 (ceil(nqb / n_local))
  float c1;                  // scale * log2(e)
  float scale;
  float* rec;                // [B, Hq, nqb * 4, 64] stage records
  float* part;               // [n_global, nparts, B, Hkv, 2, 128, 128] global-block partials
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int64_t qs_b, qs_h;
  int64_t ks_p, ks_h, ks_s;
  int64_t vs_p, vs_h, vs_s;
  int64_t os_b, os_h;
  int64_t bt_stride;
  int32_t B, Hq, Hkv, group;
  int32_t num_pages, max_blocks;
  int32_t n_global, n_local;
  float c1;
  float scale;
  float* work;  // Dqk = 576, and dense decode: per-(sequence, head, slot) partials
  int32_t nsplit;  // dense decode: block groups per sequence (the partials' slots)
  int32_t head_splits;  // grouped heads: workgroups per (sequence, kv head), each a share of the query heads
};

struct PageSelectParams {
  const void* q;
  const void* k;
  int64_t qs_b, qs_l, qs_h;
  int64_t ks_b, ks_l, ks_h;
  int32_t B, L, Hq, Hkv, group, D;
  int32_t nqb;
  int32_t n_global, n_local, top_m, W;
  double* qsum;  // [B, Hq, nqb, D]
  double* ksum;  // [B, Hkv, nqb, D]
  int32_t* idx;  // [B, Hq, nqb, W]
  int32_t* cnt;  // [B, Hq, nqb]
};

// ---------------------------------------------------------------------------
// launchers (defined in the .hip files); each returns a hipError_t
// ---------------------------------------------------------------------------

hipError_t launch_block_index(int32_t block_size, int32_t n_global, int32_t n_local, int32_t rows,
                              const int32_t* seq_lens, int32_t* idx, int32_t* cnt,
                              hipStream_t stream);

// dtype: 0 f32, 1 bf16; out_f32: output element type
hipError_t launch_prefill(const PrefillParams& p, int dtype, int dqk, int dv, bool out_f32,
                          hipStream_t stream);

// Dqk = 576, Dv = 512 (latent-shared heads); called by launch_prefill
hipError_t launch_prefill_wide(const PrefillParams& p, int dqk, int dv, bool out_f32, hipStream_t stream);
// bf16, Dqk = Dv = 128: 32 queries per wave, two waves per SIMD
bool prefill_d128_supports(const PrefillParams& p, int dqk, int dv);
hipError_t launch_prefill_d128(const PrefillParams& p, bool out_f32, hipStream_t stream);
// chunked prefill over a paged cache, bf16, Dqk = Dv = 128
hipError_t launch_prefill_tokens_d128(const TokenParams& p, bool out_f32, hipStream_t stream);
hipError_t launch_token_select(const TokenSelectParams& p, hipStream_t stream);
hipError_t launch_prefill_chunk_d128(const ChunkParams& p, bool out_f32, hipStream_t stream);

// SSA backward (bf16, d = 128): delta / records, dq, dk and dv of the local
// blocks, the global blocks' partials and their reduction
hipError_t launch_prefill_backward_d128(const BwdParams& p, bool grad_f32, hipStream_t stream);
size_t prefill_backward_workspace_bytes(int32_t B, int32_t L, int32_t Hq, int32_t Hkv, int32_t n_global,
                                        int32_t n_local);

hipError_t launch_decode(const DecodeParams& p, int dqk, int dv, hipStream_t stream);
// d = 128 with 2..16 query heads per kv head: each K/V row read once for
// all heads of its kv head (of a workgroup's share of them), a window of any
// width in one workgroup, no workspace.
bool decode_gqa_supports(const DecodeParams& p, int dqk, int dv);
hipError_t launch_decode_gqa(const DecodeParams& p, hipStream_t stream);
// merge p.nsplit pieces (o relative to m, m, l) per (sequence, head) of p.work (dense decode)
hipError_t launch_decode_merge(const DecodeParams& p, int d, hipStream_t stream);

// Dense decode (every cached key), MHA/GQA d = 64/128: nsplit groups of 16
// blocks per (sequence, kv head), partials in p.work, then a merge
hipError_t launch_decode_dense(const DecodeParams& p, int d, hipStream_t stream);
size_t decode_dense_workspace_bytes(int32_t B, int32_t Hq, int32_t max_blocks, int32_t d);

// Dqk = 576, Dv = 512 with one kv head; called by launch_decode.  Needs
// p.work of decode_mla_workspace_bytes(B, Hq, n_global + n_local) bytes.
hipError_t launch_decode_mla(const DecodeParams& p, hipStream_t stream);
size_t decode_mla_workspace_bytes(int32_t B, int32_t Hq, int32_t W);

hipError_t launch_page_select(const PageSelectParams& p, hipStream_t stream);
// its two phases: the fp64 block sums into p.qsum / p.ksum, then the scores
// and top-M lists from them
hipError_t launch_page_sums(const PageSelectParams& p, hipStream_t stream);
hipError_t launch_page_top(const PageSelectParams& p, hipStream_t stream);

// The fixed device scratch of the allocation-free page selection (the fp64
// block sums of q and k): its size, and its address on the current device
// (looked up once per device).
constexpr size_t kPageScratchBytes = size_t{32} << 20;
hipError_t page_select_scratch(void** ptr);

}  // namespace ssa
