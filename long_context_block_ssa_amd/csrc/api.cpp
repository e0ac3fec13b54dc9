// C-ABI layer of libssa: host-side validation, dispatch and error reporting.
// Every check here runs before anything is enqueued; see include/ssa.h for the
// contract of each entry point.
#include "ssa.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "common.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SSA_OK;
  return fail(SSA_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t elem_size(int dtype) { return dtype == SSA_DTYPE_F32 ? 4 : 2; }

bool valid_window(const ssa_window* w, const char* who, int max_width) {
  if (!w) {
    fail(SSA_ERR_INVALID, "%s: window is NULL", who);
    return false;
  }
  if (w->block_size < 1 || w->n_global < 0 || w->n_local < 1) {
    fail(SSA_ERR_INVALID, "%s: window {%d, %d, %d}: need block_size >= 1, n_global >= 0, n_local >= 1",
         who, w->block_size, w->n_global, w->n_local);
    return false;
  }
  if (w->n_global + w->n_local > max_width) {
    fail(SSA_ERR_INVALID, "%s: window width %d exceeds %d", who, w->n_global + w->n_local, max_width);
    return false;
  }
  return true;
}

// strides (b, l, h) of a [B, L, H, D] operand: non-negative, 16-byte multiples
bool valid_strides(const int64_t s[3], size_t es, const char* who, const char* name) {
  for (int i = 0; i < 3; ++i) {
    if (s[i] < 0 || (static_cast<uint64_t>(s[i]) * es) % 16 != 0) {
      fail(SSA_ERR_INVALID, "%s: %s stride[%d] = %lld: must be >= 0 and a multiple of 16 bytes", who,
           name, i, static_cast<long long>(s[i]));
      return false;
    }
  }
  return true;
}

// Shared validation of dense-operand arguments.  Returns SSA_OK or the error.
int check_attn(const ssa_attn_args* a, const char* who) {
  if (!a) return fail(SSA_ERR_INVALID, "%s: args is NULL", who);
  if (a->dtype != SSA_DTYPE_F32 && a->dtype != SSA_DTYPE_BF16)
    return fail(SSA_ERR_INVALID, "%s: dtype %d is not an ssa_dtype", who, a->dtype);
  if (a->out_dtype != SSA_DTYPE_F32 && a->out_dtype != SSA_DTYPE_BF16)
    return fail(SSA_ERR_INVALID, "%s: out_dtype %d is not an ssa_dtype", who, a->out_dtype);
  if (a->B < 1 || a->L < 1 || a->Hq < 1 || a->Hkv < 1 || a->Dqk < 1 || a->Dv < 1)
    return fail(SSA_ERR_INVALID, "%s: sizes B=%d L=%d Hq=%d Hkv=%d Dqk=%d Dv=%d must be >= 1", who, a->B,
                a->L, a->Hq, a->Hkv, a->Dqk, a->Dv);
  if (a->Hq % a->Hkv != 0)
    return fail(SSA_ERR_INVALID, "%s: Hq=%d is not a multiple of Hkv=%d", who, a->Hq, a->Hkv);
  if (!(std::isfinite(a->scale) && a->scale > 0.f))
    return fail(SSA_ERR_INVALID, "%s: scale %g must be finite and > 0", who, static_cast<double>(a->scale));
  if (!a->q || !a->k || !a->v || !a->o) return fail(SSA_ERR_INVALID, "%s: q, k, v and o must be non-NULL", who);
  if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->o, 16))
    return fail(SSA_ERR_INVALID, "%s: q, k, v and o must be 16-byte aligned", who);
  if (a->lse && !aligned(a->lse, 4)) return fail(SSA_ERR_INVALID, "%s: lse must be 4-byte aligned", who);
  const size_t es = elem_size(a->dtype), eo = elem_size(a->out_dtype);
  if (!valid_strides(a->q_stride, es, who, "q") || !valid_strides(a->k_stride, es, who, "k") ||
      !valid_strides(a->v_stride, es, who, "v") || !valid_strides(a->o_stride, eo, who, "o"))
    return SSA_ERR_INVALID;
  // supported kernels
  const bool f32_64 = a->dtype == SSA_DTYPE_F32 && a->Dqk == 64 && a->Dv == 64 && a->out_dtype == SSA_DTYPE_F32;
  const bool bf_64 = a->dtype == SSA_DTYPE_BF16 && a->Dqk == 64 && a->Dv == 64;
  const bool bf_128 = a->dtype == SSA_DTYPE_BF16 && a->Dqk == 128 && a->Dv == 128;
  const bool bf_mla = a->dtype == SSA_DTYPE_BF16 && a->Dqk == 576 && a->Dv == 512;
  if (!(f32_64 || bf_64 || bf_128 || bf_mla))
    return fail(SSA_ERR_UNSUPPORTED, "%s: no kernel for dtype=%d out_dtype=%d Dqk=%d Dv=%d", who, a->dtype,
                a->out_dtype, a->Dqk, a->Dv);
  return SSA_OK;
}

ssa::PrefillParams make_prefill(const ssa_attn_args* a) {
  ssa::PrefillParams p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.lse = a->lse;
  p.qs_b = a->q_stride[0];
  p.qs_l = a->q_stride[1];
  p.qs_h = a->q_stride[2];
  p.ks_b = a->k_stride[0];
  p.ks_l = a->k_stride[1];
  p.ks_h = a->k_stride[2];
  p.vs_b = a->v_stride[0];
  p.vs_l = a->v_stride[1];
  p.vs_h = a->v_stride[2];
  p.os_b = a->o_stride[0];
  p.os_l = a->o_stride[1];
  p.os_h = a->o_stride[2];
  p.B = a->B;
  p.L = a->L;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.group = a->Hq / a->Hkv;
  p.nqb = static_cast<int32_t>(ceil_div(a->L, 128));
  p.scale = a->scale;
  p.c1 = static_cast<float>(static_cast<double>(a->scale) * 1.4426950408889634);
  return p;
}

int check_lists(const ssa_attn_args* a, const ssa_block_lists* lists, const char* who) {
  if (!lists) return fail(SSA_ERR_INVALID, "%s: lists is NULL", who);
  if (!lists->idx || !lists->cnt) return fail(SSA_ERR_INVALID, "%s: lists idx/cnt must be non-NULL", who);
  if (!aligned(lists->idx, 4) || !aligned(lists->cnt, 4))
    return fail(SSA_ERR_INVALID, "%s: lists idx/cnt must be 4-byte aligned", who);
  if (lists->W < 1 || lists->W > 64) return fail(SSA_ERR_INVALID, "%s: list width W=%d not in [1, 64]", who, lists->W);
  const int64_t nqb = ceil_div(a->L, 128);
  if (lists->n_qblocks < nqb)
    return fail(SSA_ERR_INVALID, "%s: lists hold %d rows per head, L=%d needs %lld", who, lists->n_qblocks, a->L,
                static_cast<long long>(nqb));
  if (lists->idx_sb < 0 || lists->idx_sh < 0 || lists->cnt_sb < 0 || lists->cnt_sh < 0)
    return fail(SSA_ERR_INVALID, "%s: list strides must be >= 0", who);
  return SSA_OK;
}

void set_lists(ssa::PrefillParams& p, const ssa_block_lists* lists) {
  p.idx = lists->idx;
  p.cnt = lists->cnt;
  p.W = lists->W;
  p.dense = 0;
  p.idx_sb = lists->idx_sb;
  p.idx_sh = lists->idx_sh;
  p.cnt_sb = lists->cnt_sb;
  p.cnt_sh = lists->cnt_sh;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* ssa_last_error(void) { return g_last_error.c_str(); }

int ssa_version(void) { return SSA_VERSION; }

int ssa_block_index(const ssa_window* win, int32_t n_qblocks, int32_t* idx, int32_t* cnt, void* stream) {
  const char* who = "ssa_block_index";
  if (!valid_window(win, who, 64)) return SSA_ERR_INVALID;
  if (n_qblocks < 1) return fail(SSA_ERR_INVALID, "%s: n_qblocks=%d must be >= 1", who, n_qblocks);
  if (!idx || !cnt) return fail(SSA_ERR_INVALID, "%s: idx and cnt must be non-NULL", who);
  if (!aligned(idx, 4) || !aligned(cnt, 4)) return fail(SSA_ERR_INVALID, "%s: idx/cnt must be 4-byte aligned", who);
  return device_status(ssa::launch_block_index(win->block_size, win->n_global, win->n_local, n_qblocks, nullptr,
                                               idx, cnt, as_stream(stream)),
                       who);
}

int ssa_block_index_seq(const ssa_window* win, const int32_t* seq_lens, int32_t B, int32_t* idx, int32_t* cnt,
                        void* stream) {
  const char* who = "ssa_block_index_seq";
  if (!valid_window(win, who, 64)) return SSA_ERR_INVALID;
  if (B < 1) return fail(SSA_ERR_INVALID, "%s: B=%d must be >= 1", who, B);
  if (!seq_lens || !idx || !cnt) return fail(SSA_ERR_INVALID, "%s: seq_lens, idx and cnt must be non-NULL", who);
  if (!aligned(seq_lens, 4) || !aligned(idx, 4) || !aligned(cnt, 4))
    return fail(SSA_ERR_INVALID, "%s: seq_lens/idx/cnt must be 4-byte aligned", who);
  return device_status(ssa::launch_block_index(win->block_size, win->n_global, win->n_local, B, seq_lens, idx, cnt,
                                               as_stream(stream)),
                       who);
}

int ssa_prefill(const ssa_attn_args* a, const ssa_block_lists* lists, void* stream) {
  const char* who = "ssa_prefill";
  int rc = check_attn(a, who);
  if (rc != SSA_OK) return rc;
  rc = check_lists(a, lists, who);
  if (rc != SSA_OK) return rc;
  ssa::PrefillParams p = make_prefill(a);
  set_lists(p, lists);
  hipError_t e = ssa::launch_prefill(p, a->dtype, a->Dqk, a->Dv, a->out_dtype == SSA_DTYPE_F32, as_stream(stream));
  if (e == hipErrorNotSupported) return fail(SSA_ERR_UNSUPPORTED, "%s: the library has no kernel for Dqk=%d Dv=%d", who, a->Dqk, a->Dv);
  return device_status(e, who);
}

int ssa_prefill_tokens(const ssa_attn_args* a, const ssa_block_lists* lists, const ssa_token_lists* tokens,
                       void* stream) {
  const char* who = "ssa_prefill_tokens";
  int rc = check_attn(a, who);
  if (rc != SSA_OK) return rc;
  rc = check_lists(a, lists, who);
  if (rc != SSA_OK) return rc;
  if (!tokens) return fail(SSA_ERR_INVALID, "%s: tokens is NULL", who);
  if (!(a->dtype == SSA_DTYPE_BF16 && a->Dqk == 128 && a->Dv == 128))
    return fail(SSA_ERR_UNSUPPORTED, "%s: token lists need BF16 with Dqk = Dv = 128 (got dtype=%d Dqk=%d Dv=%d)", who,
                a->dtype, a->Dqk, a->Dv);
  if (tokens->K < 0 || tokens->K > 1024)
    return fail(SSA_ERR_INVALID, "%s: token list width K=%d not in [0, 1024]", who, tokens->K);
  if ((tokens->K > 0 && !tokens->tok) || !tokens->cnt)
    return fail(SSA_ERR_INVALID, "%s: tokens cnt (and tok when K > 0) must be non-NULL", who);
  if (!aligned(tokens->tok, 4) || !aligned(tokens->cnt, 4))
    return fail(SSA_ERR_INVALID, "%s: tokens tok/cnt must be 4-byte aligned", who);
  const int64_t nqb = ceil_div(a->L, 128);
  if (tokens->n_qblocks < nqb)
    return fail(SSA_ERR_INVALID, "%s: token lists hold %d rows per head, L=%d needs %lld", who, tokens->n_qblocks,
                a->L, static_cast<long long>(nqb));
  if (tokens->tok_sb < 0 || tokens->tok_sh < 0 || tokens->cnt_sb < 0 || tokens->cnt_sh < 0)
    return fail(SSA_ERR_INVALID, "%s: token list strides must be >= 0", who);
  ssa::TokenParams p{};
  static_cast<ssa::PrefillParams&>(p) = make_prefill(a);
  set_lists(p, lists);
  p.tok = tokens->tok;
  p.tcnt = tokens->cnt;
  p.K = tokens->K;
  p.tok_sb = tokens->tok_sb;
  p.tok_sh = tokens->tok_sh;
  p.tcnt_sb = tokens->cnt_sb;
  p.tcnt_sh = tokens->cnt_sh;
  hipError_t e = ssa::launch_prefill_tokens_d128(p, a->out_dtype == SSA_DTYPE_F32, as_stream(stream));
  if (e == hipErrorNotSupported) return fail(SSA_ERR_UNSUPPORTED, "%s: list width W=%d exceeds the kernel's 64", who, lists->W);
  return device_status(e, who);
}

int ssa_dense_causal(const ssa_attn_args* a, void* stream) {
  const char* who = "ssa_dense_causal";
  int rc = check_attn(a, who);
  if (rc != SSA_OK) return rc;
  ssa::PrefillParams p = make_prefill(a);
  p.dense = 1;
  p.W = 0;
  hipError_t e = ssa::launch_prefill(p, a->dtype, a->Dqk, a->Dv, a->out_dtype == SSA_DTYPE_F32, as_stream(stream));
  if (e == hipErrorNotSupported) return fail(SSA_ERR_UNSUPPORTED, "%s: the library has no kernel for Dqk=%d Dv=%d", who, a->Dqk, a->Dv);
  return device_status(e, who);
}

size_t ssa_prefill_backward_workspace_size(const ssa_bwd_args* a, const ssa_window* win) {
  if (!a || !win || a->B < 1 || a->L < 1 || a->Hq < 1 || a->Hkv < 1 || win->n_global < 0 || win->n_local < 1)
    return 0;
  return (ssa::prefill_backward_workspace_bytes(a->B, a->L, a->Hq, a->Hkv, win->n_global, win->n_local) + 255) / 256 *
         256;
}

int ssa_prefill_backward(const ssa_bwd_args* a, const ssa_window* win, void* stream) {
  const char* who = "ssa_prefill_backward";
  if (!a) return fail(SSA_ERR_INVALID, "%s: args is NULL", who);
  if (!valid_window(win, who, 64)) return SSA_ERR_INVALID;
  if (a->dtype != SSA_DTYPE_F32 && a->dtype != SSA_DTYPE_BF16)
    return fail(SSA_ERR_INVALID, "%s: dtype %d is not an ssa_dtype", who, a->dtype);
  if (a->grad_dtype != SSA_DTYPE_F32 && a->grad_dtype != SSA_DTYPE_BF16)
    return fail(SSA_ERR_INVALID, "%s: grad_dtype %d is not an ssa_dtype", who, a->grad_dtype);
  if (a->B < 1 || a->L < 1 || a->Hq < 1 || a->Hkv < 1 || a->Dqk < 1 || a->Dv < 1)
    return fail(SSA_ERR_INVALID, "%s: sizes B=%d L=%d Hq=%d Hkv=%d Dqk=%d Dv=%d must be >= 1", who, a->B, a->L,
                a->Hq, a->Hkv, a->Dqk, a->Dv);
  if (a->Hq % a->Hkv != 0) return fail(SSA_ERR_INVALID, "%s: Hq=%d is not a multiple of Hkv=%d", who, a->Hq, a->Hkv);
  if (!(std::isfinite(a->scale) && a->scale > 0.f))
    return fail(SSA_ERR_INVALID, "%s: scale %g must be finite and > 0", who, static_cast<double>(a->scale));
  if (!a->q || !a->k || !a->v || !a->o || !a->dout || !a->lse || !a->dq || !a->dk || !a->dv)
    return fail(SSA_ERR_INVALID, "%s: q, k, v, o, dout, lse, dq, dk and dv must be non-NULL", who);
  const void* p16[] = {a->q, a->k, a->v, a->o, a->dout, a->dq, a->dk, a->dv};
  for (const void* ptr : p16)
    if (!aligned(ptr, 16)) return fail(SSA_ERR_INVALID, "%s: tensor pointers must be 16-byte aligned", who);
  if (!aligned(a->lse, 4)) return fail(SSA_ERR_INVALID, "%s: lse must be 4-byte aligned", who);
  const size_t es = elem_size(a->dtype), eg = elem_size(a->grad_dtype);
  if (!valid_strides(a->q_stride, es, who, "q") || !valid_strides(a->k_stride, es, who, "k") ||
      !valid_strides(a->v_stride, es, who, "v") || !valid_strides(a->o_stride, es, who, "o") ||
      !valid_strides(a->do_stride, es, who, "dout") || !valid_strides(a->dq_stride, eg, who, "dq") ||
      !valid_strides(a->dk_stride, eg, who, "dk") || !valid_strides(a->dv_stride, eg, who, "dv"))
    return SSA_ERR_INVALID;
  if (win->block_size != 128) return fail(SSA_ERR_UNSUPPORTED, "%s: block_size must be 128", who);
  if (!(a->dtype == SSA_DTYPE_BF16 && a->Dqk == 128 && a->Dv == 128))
    return fail(SSA_ERR_UNSUPPORTED, "%s: no kernel for dtype=%d Dqk=%d Dv=%d (BF16, 128, 128 only)", who, a->dtype,
                a->Dqk, a->Dv);
  // the row strides of q, k, v and dout enter 32-bit staging offsets (16 rows)
  const int64_t* rs[] = {&a->q_stride[1], &a->k_stride[1], &a->v_stride[1], &a->do_stride[1]};
  for (const int64_t* r : rs)
    if (*r >= (int64_t{1} << 26))
      return fail(SSA_ERR_UNSUPPORTED, "%s: row stride %lld must be below 2^26 elements", who,
                  static_cast<long long>(*r));
  const size_t need = ssa_prefill_backward_workspace_size(a, win);
  if (!a->workspace || a->workspace_bytes < need)
    return fail(SSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                a->workspace ? a->workspace_bytes : static_cast<size_t>(0));
  if (!aligned(a->workspace, 256)) return fail(SSA_ERR_INVALID, "%s: workspace must be 256-byte aligned", who);
  ssa::BwdParams p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.dout = a->dout;
  p.lse = a->lse;
  p.dq = a->dq;
  p.dk = a->dk;
  p.dv = a->dv;
  const int64_t* src[] = {a->q_stride, a->k_stride, a->v_stride, a->o_stride, a->do_stride,
                          a->dq_stride, a->dk_stride, a->dv_stride};
  int64_t* dst[][3] = {{&p.qs_b, &p.qs_l, &p.qs_h},    {&p.ks_b, &p.ks_l, &p.ks_h},    {&p.vs_b, &p.vs_l, &p.vs_h},
                       {&p.os_b, &p.os_l, &p.os_h},    {&p.dos_b, &p.dos_l, &p.dos_h}, {&p.dqs_b, &p.dqs_l, &p.dqs_h},
                       {&p.dks_b, &p.dks_l, &p.dks_h}, {&p.dvs_b, &p.dvs_l, &p.dvs_h}};
  for (int t = 0; t < 8; ++t)
    for (int i = 0; i < 3; ++i) *dst[t][i] = src[t][i];
  p.B = a->B;
  p.L = a->L;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.group = a->Hq / a->Hkv;
  p.nqb = static_cast<int32_t>(ceil_div(a->L, 128));
  p.n_global = win->n_global;
  p.n_local = win->n_local;
  p.nparts = static_cast<int32_t>(ceil_div(p.nqb, win->n_local));
  p.scale = a->scale;
  p.c1 = static_cast<float>(static_cast<double>(a->scale) * 1.4426950408889634);
  const int64_t rec_bytes = static_cast<int64_t>(a->B) * a->Hq * p.nqb * 4 * 64 * 4;
  p.rec = static_cast<float*>(a->workspace);
  p.part = reinterpret_cast<float*>(static_cast<char*>(a->workspace) + (rec_bytes + 255) / 256 * 256);
  return device_status(ssa::launch_prefill_backward_d128(p, a->grad_dtype == SSA_DTYPE_F32, as_stream(stream)), who);
}

int ssa_prefill_chunk(const ssa_chunk_args* a, const ssa_block_lists* lists, void* stream) {
  const char* who = "ssa_prefill_chunk";
  if (!a) return fail(SSA_ERR_INVALID, "%s: args is NULL", who);
  if (a->dtype != SSA_DTYPE_F32 && a->dtype != SSA_DTYPE_BF16)
    return fail(SSA_ERR_INVALID, "%s: dtype %d is not an ssa_dtype", who, a->dtype);
  if (a->out_dtype != SSA_DTYPE_F32 && a->out_dtype != SSA_DTYPE_BF16)
    return fail(SSA_ERR_INVALID, "%s: out_dtype %d is not an ssa_dtype", who, a->out_dtype);
  if (a->B < 1 || a->T < 1 || a->Hq < 1 || a->Hkv < 1 || a->Dqk < 1 || a->Dv < 1 || a->num_pages < 1 ||
      a->max_blocks < 1)
    return fail(SSA_ERR_INVALID, "%s: sizes B=%d T=%d Hq=%d Hkv=%d Dqk=%d Dv=%d num_pages=%d max_blocks=%d must be >= 1",
                who, a->B, a->T, a->Hq, a->Hkv, a->Dqk, a->Dv, a->num_pages, a->max_blocks);
  if (a->Hq % a->Hkv != 0) return fail(SSA_ERR_INVALID, "%s: Hq=%d is not a multiple of Hkv=%d", who, a->Hq, a->Hkv);
  if (a->page_size != 128) return fail(SSA_ERR_INVALID, "%s: page_size=%d must be 128", who, a->page_size);
  if (static_cast<int64_t>(a->max_blocks) * 128 > INT32_MAX)
    return fail(SSA_ERR_INVALID, "%s: max_blocks=%d is too large", who, a->max_blocks);
  if (a->T > a->max_blocks * 128)
    return fail(SSA_ERR_INVALID, "%s: T=%d exceeds max_blocks * 128", who, a->T);
  if (!(std::isfinite(a->scale) && a->scale > 0.f))
    return fail(SSA_ERR_INVALID, "%s: scale %g must be finite and > 0", who, static_cast<double>(a->scale));
  if (!a->q || !a->k_pages || !a->v_pages || !a->block_table || !a->seq_lens || !a->o)
    return fail(SSA_ERR_INVALID, "%s: q, k_pages, v_pages, block_table, seq_lens and o must be non-NULL", who);
  if (!aligned(a->q, 16) || !aligned(a->k_pages, 16) || !aligned(a->v_pages, 16) || !aligned(a->o, 16))
    return fail(SSA_ERR_INVALID, "%s: q, k_pages, v_pages and o must be 16-byte aligned", who);
  if (!aligned(a->block_table, 4) || !aligned(a->seq_lens, 4) || (a->lse && !aligned(a->lse, 4)))
    return fail(SSA_ERR_INVALID, "%s: block_table, seq_lens and lse must be 4-byte aligned", who);
  const size_t es = elem_size(a->dtype), eo = elem_size(a->out_dtype);
  if (!valid_strides(a->q_stride, es, who, "q") || !valid_strides(a->k_stride, es, who, "k") ||
      !valid_strides(a->v_stride, es, who, "v") || !valid_strides(a->o_stride, eo, who, "o"))
    return SSA_ERR_INVALID;
  if (a->B > 1 && a->bt_stride < a->max_blocks)
    return fail(SSA_ERR_INVALID, "%s: bt_stride=%lld < max_blocks=%d", who, static_cast<long long>(a->bt_stride),
                a->max_blocks);
  if (!lists) return fail(SSA_ERR_INVALID, "%s: lists is NULL", who);
  if (!lists->idx || !lists->cnt) return fail(SSA_ERR_INVALID, "%s: lists idx/cnt must be non-NULL", who);
  if (!aligned(lists->idx, 4) || !aligned(lists->cnt, 4))
    return fail(SSA_ERR_INVALID, "%s: lists idx/cnt must be 4-byte aligned", who);
  if (lists->W < 1 || lists->W > 64) return fail(SSA_ERR_INVALID, "%s: list width W=%d not in [1, 64]", who, lists->W);
  if (lists->n_qblocks < a->max_blocks)
    return fail(SSA_ERR_INVALID, "%s: lists hold %d rows per head, max_blocks=%d needs as many", who,
                lists->n_qblocks, a->max_blocks);
  if (lists->idx_sb < 0 || lists->idx_sh < 0 || lists->cnt_sb < 0 || lists->cnt_sh < 0)
    return fail(SSA_ERR_INVALID, "%s: list strides must be >= 0", who);
  if (!(a->dtype == SSA_DTYPE_BF16 && a->Dqk == 128 && a->Dv == 128))
    return fail(SSA_ERR_UNSUPPORTED, "%s: no kernel for dtype=%d Dqk=%d Dv=%d (BF16, 128, 128 only)", who, a->dtype,
                a->Dqk, a->Dv);
  // rows of a page are addressed with 32-bit offsets from the page base
  const int64_t row_span = 2 * (127 * std::max(a->k_stride[2], a->v_stride[2]) + a->Dqk);
  if (row_span > INT32_MAX)
    return fail(SSA_ERR_UNSUPPORTED, "%s: slot strides (%lld, %lld) put a page's rows beyond 2^31 bytes", who,
                static_cast<long long>(a->k_stride[2]), static_cast<long long>(a->v_stride[2]));
  ssa::ChunkParams p{};
  p.q = a->q;
  p.k = a->k_pages;
  p.v = a->v_pages;
  p.o = a->o;
  p.lse = a->lse;
  p.qs_b = a->q_stride[0];
  p.qs_l = a->q_stride[1];
  p.qs_h = a->q_stride[2];
  p.ks_b = a->k_stride[0];
  p.ks_h = a->k_stride[1];
  p.ks_l = a->k_stride[2];
  p.vs_b = a->v_stride[0];
  p.vs_h = a->v_stride[1];
  p.vs_l = a->v_stride[2];
  p.os_b = a->o_stride[0];
  p.os_l = a->o_stride[1];
  p.os_h = a->o_stride[2];
  p.B = a->B;
  p.L = 0;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.group = a->Hq / a->Hkv;
  p.nqb = static_cast<int32_t>(ceil_div(a->T, 128) + 1);  // query-block tiles a chunk can touch
  p.scale = a->scale;
  p.c1 = static_cast<float>(static_cast<double>(a->scale) * 1.4426950408889634);
  p.idx = lists->idx;
  p.cnt = lists->cnt;
  p.W = lists->W;
  p.dense = 0;
  p.idx_sb = lists->idx_sb;
  p.idx_sh = lists->idx_sh;
  p.cnt_sb = lists->cnt_sb;
  p.cnt_sh = lists->cnt_sh;
  p.block_table = a->block_table;
  p.seq_lens = a->seq_lens;
  p.bt_stride = a->bt_stride;
  p.T = a->T;
  p.num_pages = a->num_pages;
  p.max_len = a->max_blocks * 128;
  return device_status(ssa::launch_prefill_chunk_d128(p, a->out_dtype == SSA_DTYPE_F32, as_stream(stream)), who);
}

size_t ssa_decode_workspace_size(const ssa_decode_args* a, const ssa_window* win) {
  if (!a || !win || a->B < 1 || a->Hq < 1 || win->n_global < 0 || win->n_local < 0) return 0;
  const int width = win->n_global + win->n_local;
  if (a->Dqk == 576 && a->Dv == 512) return (ssa::decode_mla_workspace_bytes(a->B, a->Hq, width) + 255) / 256 * 256;
  return 0;
}

size_t ssa_decode_dense_workspace_size(const ssa_decode_args* a) {
  if (!a || a->B < 1 || a->Hq < 1 || a->max_blocks < 1) return 0;
  if (!((a->Dqk == 64 && a->Dv == 64) || (a->Dqk == 128 && a->Dv == 128))) return 0;
  return (ssa::decode_dense_workspace_bytes(a->B, a->Hq, a->max_blocks, a->Dqk) + 255) / 256 * 256;
}

// ssa_decode and ssa_decode_dense: shared validation and launch.  dense: every
// cached block, through the workspace (the window is unused)
static int decode_impl(const ssa_decode_args* a, const ssa_window* win, void* stream, bool dense) {
  const char* who = dense ? "ssa_decode_dense" : "ssa_decode";
  const ssa_window dense_win{128, 0, 1};
  if (dense) win = &dense_win;
  if (!a) return fail(SSA_ERR_INVALID, "%s: args is NULL", who);
  if (!valid_window(win, who, 16)) return SSA_ERR_INVALID;
  if (a->dtype != SSA_DTYPE_BF16) return fail(SSA_ERR_UNSUPPORTED, "%s: only BF16 caches are supported", who);
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->Dqk < 1 || a->Dv < 1 || a->num_pages < 1 || a->max_blocks < 1)
    return fail(SSA_ERR_INVALID, "%s: sizes B=%d Hq=%d Hkv=%d Dqk=%d Dv=%d num_pages=%d max_blocks=%d must be >= 1",
                who, a->B, a->Hq, a->Hkv, a->Dqk, a->Dv, a->num_pages, a->max_blocks);
  if (a->Hq % a->Hkv != 0) return fail(SSA_ERR_INVALID, "%s: Hq=%d is not a multiple of Hkv=%d", who, a->Hq, a->Hkv);
  if (a->page_size != win->block_size)
    return fail(SSA_ERR_INVALID, "%s: page_size=%d differs from the window block_size=%d", who, a->page_size,
                win->block_size);
  if (!(std::isfinite(a->scale) && a->scale > 0.f))
    return fail(SSA_ERR_INVALID, "%s: scale %g must be finite and > 0", who, static_cast<double>(a->scale));
  if (!a->q || !a->k_pages || !a->v_pages || !a->block_table || !a->seq_lens || !a->o)
    return fail(SSA_ERR_INVALID, "%s: q, k_pages, v_pages, block_table, seq_lens and o must be non-NULL", who);
  if (!aligned(a->q, 16) || !aligned(a->k_pages, 16) || !aligned(a->v_pages, 16) || !aligned(a->o, 16))
    return fail(SSA_ERR_INVALID, "%s: q, k_pages, v_pages and o must be 16-byte aligned", who);
  if (!aligned(a->block_table, 4) || !aligned(a->seq_lens, 4) || (a->lse && !aligned(a->lse, 4)))
    return fail(SSA_ERR_INVALID, "%s: block_table, seq_lens and lse must be 4-byte aligned", who);
  const int64_t* ss[4] = {a->q_stride, a->k_stride, a->v_stride, a->o_stride};
  const int ns[4] = {2, 3, 3, 2};
  for (int t = 0; t < 4; ++t)
    for (int i = 0; i < ns[t]; ++i)
      if (ss[t][i] < 0 || (ss[t][i] * 2) % 16 != 0)
        return fail(SSA_ERR_INVALID, "%s: stride %lld of operand %d must be >= 0 and a multiple of 16 bytes", who,
                    static_cast<long long>(ss[t][i]), t);
  if (a->B > 1 && a->bt_stride < a->max_blocks)
    return fail(SSA_ERR_INVALID, "%s: bt_stride=%lld < max_blocks=%d", who, static_cast<long long>(a->bt_stride),
                a->max_blocks);
  const bool mha = (a->Dqk == 64 && a->Dv == 64) || (a->Dqk == 128 && a->Dv == 128);
  const bool mla = a->Dqk == 576 && a->Dv == 512 && a->Hkv == 1 && a->Hq % 16 == 0;
  if (!(mha && a->Hq / a->Hkv <= 16) && !(mla && !dense))
    return fail(SSA_ERR_UNSUPPORTED, "%s: no kernel for Dqk=%d Dv=%d Hq=%d Hkv=%d", who, a->Dqk, a->Dv, a->Hq,
                a->Hkv);
  if (win->block_size != 128) return fail(SSA_ERR_UNSUPPORTED, "%s: block_size must be 128", who);
  // the 64/128-wide kernel addresses a page's rows with 32-bit byte offsets
  const int64_t row_span =
      2 * (static_cast<int64_t>(win->block_size - 1) * std::max(a->k_stride[2], a->v_stride[2]) + a->Dqk);
  if (mha && row_span > INT32_MAX)
    return fail(SSA_ERR_UNSUPPORTED, "%s: slot strides (%lld, %lld) put a page's rows beyond 2^31 bytes", who,
                static_cast<long long>(a->k_stride[2]), static_cast<long long>(a->v_stride[2]));
  const size_t need = dense ? ssa_decode_dense_workspace_size(a) : ssa_decode_workspace_size(a, win);
  if (need > 0) {
    if (!a->workspace || a->workspace_bytes < need)
      return fail(SSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                  a->workspace ? a->workspace_bytes : static_cast<size_t>(0));
    if (!aligned(a->workspace, 256)) return fail(SSA_ERR_INVALID, "%s: workspace must be 256-byte aligned", who);
  }
  ssa::DecodeParams p{};
  p.q = a->q;
  p.k = a->k_pages;
  p.v = a->v_pages;
  p.o = a->o;
  p.lse = a->lse;
  p.block_table = a->block_table;
  p.seq_lens = a->seq_lens;
  p.qs_b = a->q_stride[0];
  p.qs_h = a->q_stride[1];
  p.ks_p = a->k_stride[0];
  p.ks_h = a->k_stride[1];
  p.ks_s = a->k_stride[2];
  p.vs_p = a->v_stride[0];
  p.vs_h = a->v_stride[1];
  p.vs_s = a->v_stride[2];
  p.os_b = a->o_stride[0];
  p.os_h = a->o_stride[1];
  p.bt_stride = a->bt_stride;
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.group = a->Hq / a->Hkv;
  p.num_pages = a->num_pages;
  p.max_blocks = a->max_blocks;
  p.n_global = win->n_global;
  p.n_local = win->n_local;
  p.scale = a->scale;
  p.c1 = static_cast<float>(static_cast<double>(a->scale) * 1.4426950408889634);
  p.work = need > 0 ? static_cast<float*>(a->workspace) : nullptr;
  p.nsplit = static_cast<int32_t>(ceil_div(a->max_blocks, 16));
  hipError_t e = dense ? ssa::launch_decode_dense(p, a->Dqk, as_stream(stream))
                       : ssa::launch_decode(p, a->Dqk, a->Dv, as_stream(stream));
  if (e == hipErrorNotSupported) return fail(SSA_ERR_UNSUPPORTED, "%s: the library has no kernel for Dqk=%d Dv=%d", who, a->Dqk, a->Dv);
  return device_status(e, who);
}

int ssa_decode(const ssa_decode_args* a, const ssa_window* win, void* stream) {
  return decode_impl(a, win, stream, false);
}

int ssa_decode_dense(const ssa_decode_args* a, void* stream) { return decode_impl(a, nullptr, stream, true); }

size_t ssa_page_select_workspace_size(const ssa_attn_args* a, const ssa_window* win) {
  if (!a || !win || a->B < 1 || a->L < 1 || a->Hq < 1 || a->Hkv < 1 || a->Dqk < 1 || win->block_size < 1) return 0;
  const size_t nqb = static_cast<size_t>(ceil_div(a->L, win->block_size));
  auto round256 = [](size_t x) { return (x + 255) / 256 * 256; };
  return round256(sizeof(double) * a->B * a->Hq * nqb * a->Dqk) +
         round256(sizeof(double) * a->B * a->Hkv * nqb * a->Dqk);
}

}  // extern "C"

namespace {

// Validation shared by the page-selection entry points; fills everything of
// `p` but the workspace pointers.  lists = false: the block-sums phase, which
// writes no lists (idx and cnt unused).
int page_select_params(const ssa_attn_args* a, const ssa_window* win, int32_t top_m, int32_t* idx, int32_t* cnt,
                       const char* who, ssa::PageSelectParams& p, bool lists = true) {
  if (!a) return fail(SSA_ERR_INVALID, "%s: args is NULL", who);
  if (!valid_window(win, who, 64)) return SSA_ERR_INVALID;
  if (a->dtype != SSA_DTYPE_BF16) return fail(SSA_ERR_UNSUPPORTED, "%s: only BF16 q/k are supported", who);
  if (a->B < 1 || a->L < 1 || a->Hq < 1 || a->Hkv < 1)
    return fail(SSA_ERR_INVALID, "%s: sizes B=%d L=%d Hq=%d Hkv=%d must be >= 1", who, a->B, a->L, a->Hq, a->Hkv);
  if (a->Hq % a->Hkv != 0) return fail(SSA_ERR_INVALID, "%s: Hq=%d is not a multiple of Hkv=%d", who, a->Hq, a->Hkv);
  if (a->Dqk != 64 && a->Dqk != 128) return fail(SSA_ERR_UNSUPPORTED, "%s: Dqk=%d (need 64 or 128)", who, a->Dqk);
  if (top_m < 0 || top_m > 32) return fail(SSA_ERR_INVALID, "%s: top_m=%d not in [0, 32]", who, top_m);
  if (win->n_global + win->n_local + top_m > 64)
    return fail(SSA_ERR_INVALID, "%s: list width %d exceeds 64", who, win->n_global + win->n_local + top_m);
  if (win->block_size != 128) return fail(SSA_ERR_UNSUPPORTED, "%s: block_size must be 128", who);
  if (ceil_div(a->L, 128) > 16384) return fail(SSA_ERR_UNSUPPORTED, "%s: L=%d exceeds 16384 blocks", who, a->L);
  if (!a->q || !a->k) return fail(SSA_ERR_INVALID, "%s: q and k must be non-NULL", who);
  if (lists && (!idx || !cnt)) return fail(SSA_ERR_INVALID, "%s: idx and cnt must be non-NULL", who);
  if (!aligned(a->q, 16) || !aligned(a->k, 16) || (lists && (!aligned(idx, 4) || !aligned(cnt, 4))))
    return fail(SSA_ERR_INVALID, "%s: q/k must be 16-byte and idx/cnt 4-byte aligned", who);
  if (!valid_strides(a->q_stride, 2, who, "q") || !valid_strides(a->k_stride, 2, who, "k")) return SSA_ERR_INVALID;
  p = ssa::PageSelectParams{};
  p.q = a->q;
  p.k = a->k;
  p.qs_b = a->q_stride[0];
  p.qs_l = a->q_stride[1];
  p.qs_h = a->q_stride[2];
  p.ks_b = a->k_stride[0];
  p.ks_l = a->k_stride[1];
  p.ks_h = a->k_stride[2];
  p.B = a->B;
  p.L = a->L;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.group = a->Hq / a->Hkv;
  p.D = a->Dqk;
  p.nqb = static_cast<int32_t>(ceil_div(a->L, 128));
  p.n_global = win->n_global;
  p.n_local = win->n_local;
  p.top_m = top_m;
  p.W = win->n_global + win->n_local + top_m;
  p.idx = idx;
  p.cnt = cnt;
  return SSA_OK;
}

// the q sums, then the k sums, each from a 256-byte boundary
void page_select_workspace(ssa::PageSelectParams& p, void* ws) {
  const size_t qbytes = (sizeof(double) * p.B * p.Hq * p.nqb * p.D + 255) / 256 * 256;
  p.qsum = static_cast<double*>(ws);
  p.ksum = reinterpret_cast<double*>(static_cast<char*>(ws) + qbytes);
}

}  // namespace

extern "C" {

int ssa_page_select(const ssa_attn_args* a, const ssa_window* win, int32_t top_m, int32_t* idx, int32_t* cnt,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "ssa_page_select";
  ssa::PageSelectParams p;
  if (const int rc = page_select_params(a, win, top_m, idx, cnt, who, p); rc != SSA_OK) return rc;
  const size_t need = ssa_page_select_workspace_size(a, win);
  if (!workspace || workspace_bytes < need)
    return fail(SSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  if (!aligned(workspace, 256)) return fail(SSA_ERR_INVALID, "%s: workspace must be 256-byte aligned", who);
  page_select_workspace(p, workspace);
  return device_status(ssa::launch_page_select(p, as_stream(stream)), who);
}

// the workspace checks of the page-selection entry points
static int page_workspace_ok(const ssa_attn_args* a, const ssa_window* win, const void* workspace,
                             size_t workspace_bytes, const char* who) {
  const size_t need = ssa_page_select_workspace_size(a, win);
  if (!workspace || workspace_bytes < need)
    return fail(SSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  if (!aligned(workspace, 256)) return fail(SSA_ERR_INVALID, "%s: workspace must be 256-byte aligned", who);
  return SSA_OK;
}

int ssa_page_block_sums(const ssa_attn_args* a, const ssa_window* win, void* workspace, size_t workspace_bytes,
                        void* stream) {
  const char* who = "ssa_page_block_sums";
  ssa::PageSelectParams p;
  if (const int rc = page_select_params(a, win, 0, nullptr, nullptr, who, p, false); rc != SSA_OK) return rc;
  if (const int rc = page_workspace_ok(a, win, workspace, workspace_bytes, who); rc != SSA_OK) return rc;
  page_select_workspace(p, workspace);
  return device_status(ssa::launch_page_sums(p, as_stream(stream)), who);
}

int ssa_page_select_top(const ssa_attn_args* a, const ssa_window* win, int32_t top_m, int32_t* idx, int32_t* cnt,
                        const void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "ssa_page_select_top";
  ssa::PageSelectParams p;
  if (const int rc = page_select_params(a, win, top_m, idx, cnt, who, p); rc != SSA_OK) return rc;
  if (const int rc = page_workspace_ok(a, win, workspace, workspace_bytes, who); rc != SSA_OK) return rc;
  page_select_workspace(p, const_cast<void*>(workspace));  // read only by the select kernel
  return device_status(ssa::launch_page_top(p, as_stream(stream)), who);
}

int ssa_page_select_noalloc(const ssa_attn_args* a, const ssa_window* win, int32_t top_m, int32_t* idx,
                            int32_t* cnt, void* stream) {
  const char* who = "ssa_page_select_noalloc";
  ssa::PageSelectParams p;
  if (const int rc = page_select_params(a, win, top_m, idx, cnt, who, p); rc != SSA_OK) return rc;
  const size_t need = ssa_page_select_workspace_size(a, win);
  if (need > ssa::kPageScratchBytes)
    return fail(SSA_ERR_WORKSPACE, "%s: these sizes need %zu bytes of scratch; the fixed scratch holds %zu", who,
                need, ssa::kPageScratchBytes);
  void* scratch = nullptr;
  if (const hipError_t e = ssa::page_select_scratch(&scratch); e != hipSuccess)
    return fail(SSA_ERR_DEVICE, "%s: the fixed scratch has no device address: %s", who, hipGetErrorString(e));
  page_select_workspace(p, scratch);
  return device_status(ssa::launch_page_select(p, as_stream(stream)), who);
}

size_t ssa_token_select_workspace_size(const ssa_attn_args* a, const ssa_window* win, int32_t top_m) {
  if (!a || !win || a->B < 1 || a->L < 1 || a->Hq < 1 || win->block_size < 1 || top_m < 0 || top_m > 32) return 0;
  return ssa::token_select_workspace_bytes(a->B, a->Hq, static_cast<int32_t>(ceil_div(a->L, win->block_size)), top_m);
}

int ssa_token_select(const ssa_attn_args* a, const ssa_window* win, int32_t top_m, const int32_t* page_idx,
                     const int32_t* page_cnt, const void* page_workspace, size_t page_workspace_bytes,
                     int32_t top_k, int32_t* tok, int32_t* tok_cnt, void* workspace, size_t workspace_bytes,
                     void* stream) {
  const char* who = "ssa_token_select";
  if (!a) return fail(SSA_ERR_INVALID, "%s: args is NULL", who);
  if (!valid_window(win, who, 64)) return SSA_ERR_INVALID;
  if (a->dtype != SSA_DTYPE_BF16) return fail(SSA_ERR_UNSUPPORTED, "%s: only BF16 k is supported", who);
  if (a->B < 1 || a->L < 1 || a->Hq < 1 || a->Hkv < 1)
    return fail(SSA_ERR_INVALID, "%s: sizes B=%d L=%d Hq=%d Hkv=%d must be >= 1", who, a->B, a->L, a->Hq, a->Hkv);
  if (a->Hq % a->Hkv != 0) return fail(SSA_ERR_INVALID, "%s: Hq=%d is not a multiple of Hkv=%d", who, a->Hq, a->Hkv);
  if (a->Dqk != 64 && a->Dqk != 128) return fail(SSA_ERR_UNSUPPORTED, "%s: Dqk=%d (need 64 or 128)", who, a->Dqk);
  if (top_m < 0 || top_m > 32) return fail(SSA_ERR_INVALID, "%s: top_m=%d not in [0, 32]", who, top_m);
  if (win->n_global + win->n_local + top_m > 64)
    return fail(SSA_ERR_INVALID, "%s: page list width %d exceeds 64", who, win->n_global + win->n_local + top_m);
  if (top_k < 0 || top_k > 1024) return fail(SSA_ERR_INVALID, "%s: top_k=%d not in [0, 1024]", who, top_k);
  if (win->block_size != 128) return fail(SSA_ERR_UNSUPPORTED, "%s: block_size must be 128", who);
  if (ceil_div(a->L, 128) > 16384) return fail(SSA_ERR_UNSUPPORTED, "%s: L=%d exceeds 16384 blocks", who, a->L);
  if (static_cast<int64_t>(a->B) * a->Hq * ceil_div(a->L, 128) > (int64_t{1} << 31) - 1)
    return fail(SSA_ERR_UNSUPPORTED, "%s: B*Hq*ceil(L/128) exceeds 2^31 - 1 rows", who);
  if (!a->k || !page_idx || !page_cnt || (top_k > 0 && !tok) || !tok_cnt)
    return fail(SSA_ERR_INVALID, "%s: k, page_idx, page_cnt, tok_cnt (and tok when top_k > 0) must be non-NULL", who);
  if (!aligned(a->k, 16) || !aligned(page_idx, 4) || !aligned(page_cnt, 4) || !aligned(tok, 4) || !aligned(tok_cnt, 4))
    return fail(SSA_ERR_INVALID, "%s: k must be 16-byte and the lists 4-byte aligned", who);
  if (!valid_strides(a->k_stride, 2, who, "k")) return SSA_ERR_INVALID;
  const size_t pneed = ssa_page_select_workspace_size(a, win);
  if (!page_workspace || page_workspace_bytes < pneed)
    return fail(SSA_ERR_WORKSPACE, "%s: the page selection workspace of %zu bytes is needed, %zu given", who, pneed,
                page_workspace ? page_workspace_bytes : static_cast<size_t>(0));
  if (!aligned(page_workspace, 256)) return fail(SSA_ERR_INVALID, "%s: page_workspace must be 256-byte aligned", who);
  const size_t need = ssa_token_select_workspace_size(a, win, top_m);
  if (!workspace || workspace_bytes < need)
    return fail(SSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  if (!aligned(workspace, 256)) return fail(SSA_ERR_INVALID, "%s: workspace must be 256-byte aligned", who);
  ssa::TokenSelectParams p{};
  p.k = a->k;
  p.ks_b = a->k_stride[0];
  p.ks_l = a->k_stride[1];
  p.ks_h = a->k_stride[2];
  p.qsum = static_cast<const double*>(page_workspace);
  p.pidx = page_idx;
  p.pcnt = page_cnt;
  p.PW = win->n_global + win->n_local + top_m;
  p.S = top_m;
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.group = a->Hq / a->Hkv;
  p.D = a->Dqk;
  p.nqb = static_cast<int32_t>(ceil_div(a->L, 128));
  p.n_global = win->n_global;
  p.n_local = win->n_local;
  p.K = top_k;
  p.tok = tok;
  p.tcnt = tok_cnt;
  const size_t R = static_cast<size_t>(a->B) * a->Hq * p.nqb;
  auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
  char* w = static_cast<char*>(workspace);
  p.cnt = reinterpret_cast<int32_t*>(w);
  w += r256(4 * R);
  p.off = reinterpret_cast<int32_t*>(w);
  w += r256(4 * R);
  p.npg = reinterpret_cast<int32_t*>(w);
  w += r256(4 * R);
  p.pages = reinterpret_cast<int32_t*>(w);
  w += r256(4 * R * top_m);
  p.ent = reinterpret_cast<int32_t*>(w);
  w += r256(4 * R * top_m);
  p.keys = reinterpret_cast<uint64_t*>(w);
  return device_status(ssa::launch_token_select(p, as_stream(stream)), who);
}

}  // extern "C"
