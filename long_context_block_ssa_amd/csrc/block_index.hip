// Block-index builder: the window of every query block.
//
// Row qb may read the global blocks [0, n_global) and the local blocks
// [qb - n_local + 1, qb] (its own block included), clipped to [0, qb] and
// counted once -- 1 global + 7 local blocks of 128 tokens by default (QbitAI
// report on LongCat LoZA, sparse-window paragraph).  One thread writes one row,
// ascending, padded with -1.  Integer work only; negligible next to attention.
#include "common.hpp"

namespace ssa {
namespace {

__global__ void block_index_kernel(int32_t block_size, int32_t n_global, int32_t n_local, int32_t rows,
                                   const int32_t* __restrict__ seq_lens, int32_t* __restrict__ idx,
                                   int32_t* __restrict__ cnt) {
  const int32_t r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const int32_t W = n_global + n_local;
  int32_t* out = idx + static_cast<int64_t>(r) * W;
  int32_t qb;
  if (seq_lens) {
    const int32_t n = seq_lens[r];
    if (n < 1) {
      for (int32_t s = 0; s < W; ++s) out[s] = -1;
      cnt[r] = 0;
      return;
    }
    qb = (n - 1) / block_size;
  } else {
    qb = r;
  }
  // global part: [0, min(n_global, qb + 1)); local part starts where the
  // global part ends or at qb - n_local + 1, whichever is larger
  const int32_t g_end = min(n_global, qb + 1);
  const int32_t l_begin = max(g_end, qb - n_local + 1);
  int32_t s = 0;
  for (int32_t t = 0; t < g_end; ++t) out[s++] = t;
  for (int32_t t = l_begin; t <= qb; ++t) out[s++] = t;
  cnt[r] = s;
  for (; s < W; ++s) out[s] = -1;
}

}  // namespace

hipError_t launch_block_index(int32_t block_size, int32_t n_global, int32_t n_local, int32_t rows,
                              const int32_t* seq_lens, int32_t* idx, int32_t* cnt, hipStream_t stream) {
  const int threads = 256;
  const int blocks = (rows + threads - 1) / threads;
  return launch_kernel(block_index_kernel, dim3(blocks), dim3(threads), 0, stream, block_size, n_global, n_local,
                       rows, seq_lens, idx, cnt);
}

}  // namespace ssa
