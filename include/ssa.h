/*
 * ssa.h -- C ABI of libssa, block-sparse streaming attention (SSA) on MI355X (gfx950).
 *
 * SSA is the sparse attention of LongCat's LoZA: every query reads a fixed
 * window of 128-token key blocks -- one global block (block 0) and the seven
 * most recent blocks, its own block included and causally masked -- so the
 * cost per query is bounded by S = 1024 keys (QbitAI report on LongCat LoZA,
 * the paragraphs on the O(L*S) cost and on the 1024-token sparse window).
 * Within the window it is ordinary softmax attention restricted by a 0/1 mask
 * ("LoZA: ZigZag sparse attention" page, section 2.1, equations (1)-(2)).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensor pointers are DEVICE pointers on the caller's current HIP
 *    device; every size is in elements unless it says bytes.
 *  - The caller allocates and owns every buffer.  The library allocates no
 *    device memory and keeps no state besides a thread-local error string.
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL is the null stream) and never synchronises the host.
 *  - Arguments are validated on the host before anything is enqueued; on a
 *    validation failure nothing is launched.  Device-side contents (block
 *    lists, page tables, sequence lengths) cannot be checked on the host; the
 *    kernels treat out-of-range entries as documented per call and never read
 *    or write outside the buffers described here.
 *  - Return value: an ssa_status.  ssa_last_error() describes the last failure
 *    of the calling thread.  The library never aborts, throws or prints.
 *  - Results are bitwise deterministic for identical inputs and launch
 *    arguments: no floating-point atomics are used.
 */
#ifndef SSA_H_
#define SSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSA_VERSION 10000 /* 1.0.0 */

typedef enum ssa_status {
  SSA_OK = 0,
  SSA_ERR_INVALID = 1,     /* a null pointer, a bad size, stride or alignment */
  SSA_ERR_UNSUPPORTED = 2, /* a valid request the library has no kernel for */
  SSA_ERR_DEVICE = 3,      /* the HIP runtime refused a launch               */
  SSA_ERR_WORKSPACE = 4    /* workspace missing or too small                 */
} ssa_status;

typedef enum ssa_dtype { SSA_DTYPE_F32 = 0, SSA_DTYPE_BF16 = 1 } ssa_dtype;

/* Window geometry.  The defaults {128, 1, 7} are the ones of the QbitAI report
 * on LoZA (1 global + 7 local blocks of 128 tokens).  Global blocks are
 * [0, n_global); local blocks are [qb - n_local + 1, qb], the query's own
 * block qb included; the union is clipped to [0, qb] and counted once. */
typedef struct ssa_window {
  int32_t block_size; /* tokens per block; the attention kernels need 128     */
  int32_t n_global;   /* >= 0                                                */
  int32_t n_local;    /* >= 1 (the own block is always local)                 */
} ssa_window;

/* Dense attention operands, logical shapes
 *   q [B, L, Hq, Dqk], k [B, L, Hkv, Dqk], v [B, L, Hkv, Dv] -> o [B, L, Hq, Dv]
 * stored with arbitrary element strides for (batch, position, head) and a
 * contiguous channel dimension.  Query head h reads kv head h / (Hq / Hkv).
 * Requirements: base pointers 16-byte aligned; every stride times the element
 * size a multiple of 16 bytes.  v may alias k (the latent-shared layout uses
 * v = the first Dv channels of k); o must not overlap any input.
 * lse, when not NULL, receives the natural-log sum of exponentials of the
 * scaled scores, fp32, contiguous [B, Hq, L].
 * Supported (dtype, Dqk, Dv): (F32, 64, 64), (BF16, 64, 64), (BF16, 128, 128),
 * (BF16, 576, 512).  out_dtype is BF16 or F32 for BF16 inputs, F32 for F32.
 * scale multiplies q.k before the softmax; it must be finite and > 0
 * (1/sqrt(Dqk) is the usual choice, section 2.1 of the ZigZag page). */
typedef struct ssa_attn_args {
  int32_t dtype;     /* ssa_dtype of q, k, v */
  int32_t out_dtype; /* ssa_dtype of o       */
  int32_t B, L, Hq, Hkv, Dqk, Dv;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_stride[3]; /* (b, l, h) element strides */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
} ssa_attn_args;

/* Per-query-block lists of readable key blocks, as written by
 * ssa_block_index (one list shared by every batch and head: strides 0) or by
 * ssa_page_select (one list per batch and query head).
 *   row (b, h, qb):  idx[b*idx_sb + h*idx_sh + qb*W + s], s < cnt[b*cnt_sb + h*cnt_sh + qb]
 * Entries must be distinct.  An entry < 0, > qb or >= ceil(L/128) is skipped;
 * the own block qb is causally masked (key j <= query i).  A row whose list
 * admits no key produces o = 0 and lse = -inf. */
typedef struct ssa_block_lists {
  const int32_t* idx;
  const int32_t* cnt;
  int32_t W;         /* list capacity, 1 .. 64        */
  int32_t n_qblocks; /* rows per (b, h); >= ceil(L/128) */
  int64_t idx_sb, idx_sh;
  int64_t cnt_sb, cnt_sh;
} ssa_block_lists;

/* Per-query-block lists of single key tokens, as written by ssa_token_select
 * (one list per batch and query head):
 *   row (b, h, qb):  tok[b*tok_sb + h*tok_sh + qb*K + e], e < cnt[b*cnt_sb + h*cnt_sh + qb]
 * (a count below 0 reads as 0, above K as K).  A row's entries must be
 * strictly ascending, below qb*128 (every token precedes its query block, so
 * no causal rule applies to them) and outside every block of the row's block
 * list; a row that breaks this makes every output row of its query block NaN
 * (lse NaN). */
typedef struct ssa_token_lists {
  const int32_t* tok;
  const int32_t* cnt;
  int32_t K;         /* list capacity, 0 .. 1024          */
  int32_t n_qblocks; /* rows per (b, h); >= ceil(L/128)   */
  int64_t tok_sb, tok_sh;
  int64_t cnt_sb, cnt_sh;
} ssa_token_lists;

/* Paged decode operands.  One new query per sequence:
 *   q [B, Hq, Dqk]  -> o [B, Hq, Dv]   (strides for (b, h); channels contiguous)
 *   k_pages [num_pages, Hkv, page_size, Dqk], v_pages [num_pages, Hkv, page_size, Dv]
 *     (strides for (page, head, slot); channels contiguous; v may alias k)
 *   block_table [B, max_blocks] int32: logical block t of sequence b lives in
 *     page block_table[b*bt_stride + t]  (bt_stride >= max_blocks when B > 1)
 *   seq_lens [B] int32: context length INCLUDING the new token, whose key and
 *     value are already in the cache; the query sits at position n - 1.
 * A sequence whose length is outside [1, max_blocks*page_size], or whose
 * window names a page outside [0, num_pages), gets an all-NaN output row (and
 * lse = NaN) and nothing out of range is read.
 * Supported (dtype, Dqk, Dv): (BF16, 64, 64), (BF16, 128, 128) with
 * Hq/Hkv <= 16 and a page's rows within 2^31 bytes of the page base
 * (2 * (127 * slot stride + D) <= 2^31 - 1, else SSA_ERR_UNSUPPORTED), and
 * (BF16, 576, 512) with Hkv == 1 and Hq a multiple of 16.
 * The (576, 512) shape splits every window over its blocks, and (128, 128)
 * with 2 <= Hq/Hkv <= 16 and a window wider than 4 blocks splits it over
 * groups of 4 blocks; both keep fp32 partials in a caller-owned device
 * workspace of at least ssa_decode_workspace_size bytes, 256-byte aligned
 * (SSA_ERR_WORKSPACE if it is missing or short); the other shapes ignore both
 * fields. */
typedef struct ssa_decode_args {
  int32_t dtype; /* of q, k_pages, v_pages and o: BF16 */
  int32_t B, Hq, Hkv, Dqk, Dv;
  int32_t page_size; /* == the window's block_size == 128 */
  int32_t num_pages, max_blocks;
  float scale;
  const void* q;
  const void* k_pages;
  const void* v_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* lse; /* optional, contiguous [B, Hq] */
  int64_t q_stride[2];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[2];
  int64_t bt_stride;
  void* workspace;        /* device scratch, contents on entry ignored */
  size_t workspace_bytes; /* its size */
} ssa_decode_args;

/* ---------------------------------------------------------------------------
 * ssa_block_index -- the window of every query block (QbitAI report on LoZA,
 * sparse-window paragraph).  Writes idx [n_qblocks, W] with W = n_global +
 * n_local: the readable block ids of row qb in ascending order, padded with
 * -1; and cnt [n_qblocks] = their number (min(qb + 1, W) for the defaults).
 * Exact integer output.  n_qblocks >= 1; W <= 64.
 * ------------------------------------------------------------------------- */
int ssa_block_index(const ssa_window* win, int32_t n_qblocks, int32_t* idx, int32_t* cnt,
                    void* stream);

/* Same rule for decode rows: row b uses qb = (seq_lens[b] - 1) / block_size.
 * A length < 1 yields cnt = 0 and a row of -1. */
int ssa_block_index_seq(const ssa_window* win, const int32_t* seq_lens, int32_t B, int32_t* idx,
                        int32_t* cnt, void* stream);

/* ---------------------------------------------------------------------------
 * ssa_prefill -- block-sparse causal attention of every query over the key
 * blocks its row lists (SSA: the lists of ssa_block_index; the page-selected
 * variant: the lists of ssa_page_select).  Within the listed blocks the
 * result is the masked softmax of equation (2) of the ZigZag page, section
 * 2.1.  bf16 inputs are multiplied on the matrix cores with fp32
 * accumulation; the softmax runs in fp32.
 * ------------------------------------------------------------------------- */
int ssa_prefill(const ssa_attn_args* a, const ssa_block_lists* lists, void* stream);

/* ---------------------------------------------------------------------------
 * ssa_prefill_tokens -- ssa_prefill over the row's block list together with
 * the row's single tokens (LongCat sparse attention article, section 3,
 * hierarchical indexing: after the coarse page stage a fine stage keeps the
 * best tokens inside the recalled pages; with the window's blocks as the
 * block list and the lists of ssa_token_select as the tokens this is the
 * attention of that variant).  The keys of query i in block qb are the keys
 * j <= i of its listed blocks plus its block's listed tokens; the softmax is
 * the masked softmax of equation (2) of the ZigZag page, section 2.1.
 * Supported: BF16 with Dqk = Dv = 128 (else SSA_ERR_UNSUPPORTED); output BF16
 * or F32; lse optional.  tokens->cnt must be non-NULL, tokens->tok too when
 * K > 0.
 * ------------------------------------------------------------------------- */
int ssa_prefill_tokens(const ssa_attn_args* a, const ssa_block_lists* lists, const ssa_token_lists* tokens,
                       void* stream);

/* ssa_dense_causal -- the comparison layer: plain causal attention, key j <=
 * query i (equation (1) of the ZigZag page with the causal rule of its
 * section 2.2.1), same kernel family as ssa_prefill. */
int ssa_dense_causal(const ssa_attn_args* a, void* stream);

/* ---------------------------------------------------------------------------
 * ssa_decode -- one decode step of SSA over a paged cache: the query at
 * position n - 1 reads the window of its block (block 0 and the 7 most recent
 * blocks, the last one holding (n - 1) mod 128 + 1 valid keys) -- the fixed
 * 1024-token window of the sparse layers (QbitAI report on LongCat LoZA, the
 * paragraph on streaming sparse attention: 1 global + 7 local blocks of 128
 * tokens), with the masked softmax of equation (2) of the "LoZA: ZigZag
 * sparse attention" page (section 2.1).  Decoding at long context is bound by
 * reading the cache (LongCat sparse attention article, section 1), so each
 * window block is read once, as whole contiguous pages.  The window is
 * split over its blocks and the per-block softmax partials are merged exactly
 * (max-subtracted pieces rescaled to the common maximum): inside one kernel
 * for the 64- and 128-wide heads, through the workspace and a second kernel
 * for the 576/512 latent.  Two calls that share a workspace must be ordered
 * (same stream); the workspace may be reused as soon as the call's work on
 * the stream is done.
 * ------------------------------------------------------------------------- */
int ssa_decode(const ssa_decode_args* a, const ssa_window* win, void* stream);

/* Bytes of workspace ssa_decode needs for these sizes and window, rounded up
 * to a multiple of 256: B * Hq * (n_global + n_local) * 2064 for Dqk = 576,
 * Dv = 512; otherwise 0.  Reads only B, Hq, Dqk, Dv and the window; 0 for
 * NULL arguments. */
size_t ssa_decode_workspace_size(const ssa_decode_args* a, const ssa_window* win);

/* ---------------------------------------------------------------------------
 * ssa_prefill_backward -- gradients of the SSA prefill output with respect to
 * q, k and v, for training: LoZA converts layers in mid-training (QbitAI
 * report on LongCat LoZA), and the sparse operator needs its own
 * deterministic backward (LongCat sparse attention article, section 4).
 * With P the masked softmax of the forward (recomputed from its lse) and dO
 * the incoming gradient of o:
 *   dV = P^T dO,  dP = dO V^T,  dS = P (dP - rowsum(dO * O)),
 *   dQ = scale dS K,  dK = scale dS^T Q,
 * summed over every query block and query head that reads a key (the
 * window's inverse map).  Bitwise deterministic (no atomics).
 *
 * Operands (logical [B, L, H, D], strides for (b, l, h), channels contiguous):
 *   q, k, v: the forward's inputs; o: its output; dout: the gradient of o
 *   (same shape and strides rules as o); lse: the forward's lse, fp32,
 *   contiguous [B, Hq, L] (ssa_prefill with lse != NULL);
 *   dq, dk, dv: written in grad_dtype, shaped like q, k, v (no overlap with
 *   any input).
 * The window is the one the forward used (block_size 128).  workspace: device
 * memory of at least ssa_prefill_backward_workspace_size bytes, 256-byte
 * aligned, contents on entry ignored.
 * Supported: dtype BF16 (q, k, v, o, dout), Dqk = Dv = 128, grad_dtype BF16 or
 * F32, Hq a multiple of Hkv, window width <= 64.
 * ------------------------------------------------------------------------- */
typedef struct ssa_bwd_args {
  int32_t dtype;      /* of q, k, v, o, dout: BF16 */
  int32_t grad_dtype; /* of dq, dk, dv: BF16 or F32 */
  int32_t B, L, Hq, Hkv, Dqk, Dv;
  float scale; /* the forward's */
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3], do_stride[3];
  int64_t dq_stride[3], dk_stride[3], dv_stride[3];
  void* workspace;
  size_t workspace_bytes;
} ssa_bwd_args;

int ssa_prefill_backward(const ssa_bwd_args* a, const ssa_window* win, void* stream);

/* Bytes of workspace ssa_prefill_backward needs: per (b, query head, 32
 * rows) 256 bytes of lse / delta records, plus fp32 partial dk, dv of the
 * global blocks (128 KB per global block, batch, kv head and group of
 * n_local query blocks that reads it).  0 for NULL arguments. */
size_t ssa_prefill_backward_workspace_size(const ssa_bwd_args* a, const ssa_window* win);

/* ---------------------------------------------------------------------------
 * ssa_prefill_chunk -- chunked prefill over a paged cache: T new queries per
 * sequence, at positions n_b - T .. n_b - 1, each reading the key blocks its
 * row lists (row = the query's absolute block, position / 128) and keys
 * j <= i.  With the lists of ssa_block_index this is the SSA window of the
 * QbitAI report on LongCat LoZA applied to a cached sequence, so a long
 * prompt can be prefilled in pieces (each piece's keys and values are
 * appended to the cache first) with the same result as one ssa_prefill over
 * the whole prompt.  Within the listed blocks the result is the masked
 * softmax of equation (2) of the ZigZag page, section 2.1.
 *
 * Operands:
 *   q [B, T, Hq, Dqk] -> o [B, T, Hq, Dv]  (strides for (b, t, h); channels
 *     contiguous; o must not overlap any input)
 *   k_pages, v_pages, block_table, bt_stride, num_pages, max_blocks,
 *     page_size: as in ssa_decode_args (v may alias k)
 *   seq_lens [B] int32: n_b, the cached length INCLUDING the chunk, whose keys
 *     and values are already in the cache; query t sits at position n_b - T + t
 *   lists: as for ssa_prefill, with n_qblocks >= max_blocks rows per (b, h),
 *     indexed by absolute query block; entries < 0, > the row's block or past
 *     the sequence are skipped
 *   lse, when not NULL: fp32, contiguous [B, Hq, T]
 * A sequence whose n_b lies outside [T, max_blocks * page_size] gets all-NaN
 * output rows (and lse = NaN); so do the chunk's rows in a query block whose
 * list names a block mapped to a page outside [0, num_pages), or in any block
 * of a sequence whose block 0 is.  Nothing out of range is read.
 * Supported: dtype BF16 with Dqk = Dv = 128, out_dtype BF16 or F32,
 * page_size 128, Hq a multiple of Hkv, list width W <= 64; a page's rows
 * within 2^31 bytes of its base.
 * ------------------------------------------------------------------------- */
typedef struct ssa_chunk_args {
  int32_t dtype;     /* of q, k_pages, v_pages: BF16 */
  int32_t out_dtype; /* of o: BF16 or F32        */
  int32_t B, T, Hq, Hkv, Dqk, Dv;
  int32_t page_size; /* 128 */
  int32_t num_pages, max_blocks;
  float scale;
  const void* q;
  const void* k_pages;
  const void* v_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  int64_t q_stride[3]; /* (b, t, h) element strides       */
  int64_t k_stride[3]; /* (page, head, slot)              */
  int64_t v_stride[3];
  int64_t o_stride[3]; /* (b, t, h)                       */
  int64_t bt_stride;   /* >= max_blocks when B > 1        */
} ssa_chunk_args;

int ssa_prefill_chunk(const ssa_chunk_args* a, const ssa_block_lists* lists, void* stream);

/* ---------------------------------------------------------------------------
 * ssa_decode_dense -- the decode step of a dense layer over the same paged
 * cache: the new query reads every cached key 0 .. n-1 (softmax attention of
 * equation (1) of the ZigZag page with the causal rule of its section 2.2.1).
 * LoZA keeps half of its layers dense (QbitAI report on LongCat LoZA), so a
 * layer stack alternates this with ssa_decode.  Operands and the handling of
 * bad lengths and pages as for ssa_decode (every block of the sequence is
 * read, so any page of it outside the pool makes the row NaN).  Workspace: at
 * least ssa_decode_dense_workspace_size bytes, 256-byte aligned (per
 * sequence, query head and group of 16 blocks, an fp32 piece of D + 2
 * values, merged exactly by a second kernel).
 * Supported (dtype, Dqk, Dv): (BF16, 64, 64), (BF16, 128, 128), Hq/Hkv <= 16.
 * ------------------------------------------------------------------------- */
int ssa_decode_dense(const ssa_decode_args* a, void* stream);

/* B * Hq * ceil(max_blocks / 16) * (Dv + 2) * 4 bytes, rounded up to 256; 0
 * for NULL arguments or unsupported shapes. */
size_t ssa_decode_dense_workspace_size(const ssa_decode_args* a);

/* ---------------------------------------------------------------------------
 * ssa_page_select -- block lists for the page-selected variant (LongCat
 * sparse attention article, section 3: streaming-aware indexing keeps the
 * sink and the local window; hierarchical indexing scores 128-token pages
 * coarsely and keeps the top M).  For batch b, query head h and query block
 * qb the list is the window of qb plus the top_m pages c in
 * [n_global, qb - n_local] with the highest score
 *      < sum of q over block qb , sum of k over page c >      (kv head of h)
 * ranked in fp64 from exact fp64 block sums; equal scores prefer the lower
 * page; with at most top_m candidates all are kept.  Output lists are
 * ascending, padded with -1:
 *   idx [B, Hq, nqb, W] with W = n_global + n_local + top_m,  cnt [B, Hq, nqb]
 * (contiguous), ready for ssa_prefill with idx_sb = Hq*nqb*W, idx_sh = nqb*W,
 * cnt_sb = Hq*nqb, cnt_sh = nqb.  Uses a.q, a.k, their strides, a.dtype
 * (BF16), B, L, Hq, Hkv, Dqk (64 or 128).  0 <= top_m <= 32.  The workspace
 * holds the fp64 block sums; its size comes from
 * ssa_page_select_workspace_size and it needs 256-byte alignment.
 * ------------------------------------------------------------------------- */
size_t ssa_page_select_workspace_size(const ssa_attn_args* a, const ssa_window* win);
int ssa_page_select(const ssa_attn_args* a, const ssa_window* win, int32_t top_m, int32_t* idx,
                    int32_t* cnt, void* workspace, size_t workspace_bytes, void* stream);

/* ssa_page_block_sums, ssa_page_select_top -- ssa_page_select in its two
 * phases, for callers that reuse the block sums (the second stage of
 * hierarchical indexing, ssa_token_select, reads them from the same
 * workspace) or time the phases apart.  ssa_page_block_sums writes the fp64
 * block sums of q and k (the coarse page representations of the LongCat
 * sparse attention article, section 3) into the workspace; it uses the same
 * fields as ssa_page_select and neither lists nor top_m.  ssa_page_select_top
 * then scores and ranks exactly as ssa_page_select from the sums already in
 * the workspace (it only reads it) and writes idx and cnt.  Arguments,
 * workspace size and alignment, and errors as ssa_page_select; the pair gives
 * the same lists bit for bit as one ssa_page_select call on the same
 * stream. */
int ssa_page_block_sums(const ssa_attn_args* a, const ssa_window* win, void* workspace, size_t workspace_bytes,
                        void* stream);
int ssa_page_select_top(const ssa_attn_args* a, const ssa_window* win, int32_t top_m, int32_t* idx,
                        int32_t* cnt, const void* workspace, size_t workspace_bytes, void* stream);

/* ssa_page_select_noalloc -- ssa_page_select for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the fp64 block sums go to a fixed scratch array
 * inside the library instead of a caller workspace.  Same arguments, lists
 * and errors as ssa_page_select, minus the workspace; the kernels are the
 * same.  Limit: ssa_page_select_workspace_size(a, win) must not exceed
 * 32 MiB (33554432 bytes; e.g. B = 1, Hq = Hkv = 16, L = 131072, Dqk = 128),
 * else SSA_ERR_WORKSPACE and nothing is launched.  The call allocates
 * nothing: each GPU the library runs on holds one copy of the scratch from
 * its first use until the process ends (SSA_ERR_DEVICE if its address cannot
 * be looked up).  Every call on a GPU shares that copy, so calls that overlap
 * on one GPU (other streams, other host threads) race and must be ordered by
 * the caller; calls in one stream are ordered.  Nothing in the scratch needs
 * to start at zero. */
int ssa_page_select_noalloc(const ssa_attn_args* a, const ssa_window* win, int32_t top_m, int32_t* idx,
                            int32_t* cnt, void* stream);

/* ---------------------------------------------------------------------------
 * ssa_token_select -- the fine stage of hierarchical indexing (LongCat sparse
 * attention article, section 3: inside the top-M recalled pages every token
 * is scored and the top K are kept).  The article leaves the token score to
 * a trained indexer; this library scores token j for query block qb with the
 * page stage's query-block sum:
 *      < sum of q over block qb , k_j >      (kv head of h, fp64)
 * Candidates are the tokens of the pages c of row (b, h, qb) of page_idx /
 * page_cnt with n_global <= c <= qb - n_local (the pages outside the window;
 * a repeated page counts once; at most the top_m lowest such pages).  The
 * top_k highest scores are kept, equal scores preferring the lower token;
 * with at most top_k candidates all are kept.  Output lists are ascending,
 * padded with -1:  tok [B, Hq, nqb, top_k],  tok_cnt [B, Hq, nqb]
 * (contiguous), ready for ssa_prefill_tokens with tok_sb = Hq*nqb*top_k,
 * tok_sh = nqb*top_k, cnt_sb = Hq*nqb, cnt_sh = nqb.
 * page_idx / page_cnt are the contiguous lists ssa_page_select wrote with the
 * same a, win and top_m, and page_workspace is the workspace of that call
 * (it holds the fp64 query-block sums), ordered before this call on the
 * stream.  Uses a.k, its strides, a.dtype (BF16), B, L, Hq, Hkv, Dqk (64 or
 * 128).  0 <= top_m <= 32; 0 <= top_k <= 1024 (tok may be NULL when
 * top_k = 0; tok_cnt is then all 0).  The work runs page by page (each
 * recalled page is read once per query head and scored for every query block
 * that recalled it), through a caller-owned device workspace of at least
 * ssa_token_select_workspace_size bytes, 256-byte aligned (B*Hq*nqb*(12 +
 * 8*top_m + 1024*top_m) bytes, about 134 MB at B = 1, Hq = 16, L = 131072,
 * top_m = 8); SSA_ERR_WORKSPACE if it is missing or short.
 * ------------------------------------------------------------------------- */
size_t ssa_token_select_workspace_size(const ssa_attn_args* a, const ssa_window* win, int32_t top_m);
int ssa_token_select(const ssa_attn_args* a, const ssa_window* win, int32_t top_m, const int32_t* page_idx,
                     const int32_t* page_cnt, const void* page_workspace, size_t page_workspace_bytes,
                     int32_t top_k, int32_t* tok, int32_t* tok_cnt, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Text of the calling thread's last error ("" if none).  Valid until the
 * thread's next failing call. */
const char* ssa_last_error(void);

/* SSA_VERSION of the library. */
int ssa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSA_H_ */
