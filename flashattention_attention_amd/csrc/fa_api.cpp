// C-ABI entry points of libfa.so: argument validation (before any HIP call)
// and dispatch to the gfx950 kernel launchers. See include/fa.h for the
// contract of each entry point.
#include "../../include/fa.h"

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>

#include "fa_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return FA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool head_dim_supported(int d) { return d == 64 || d == 128 || d == 256; }
bool prefill_head_dim_supported(int d) { return head_dim_supported(d) || d == 512; }

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr float kLog2e = 1.4426950408889634f;

// Query/key/output side of a prefill call.
int check_attn(const char* fn, const void* q, int64_t q_sb, int64_t q_ss, int64_t q_sh,
               const void* k, int64_t k_sb, int64_t k_ss, int64_t k_sh, const float* o,
               int64_t o_sb, int64_t o_ss, int64_t o_sh, const float* lse,
               const float* row_sum, int batch, int seqlen_q, int seqlen_kv, int n_heads_q,
               int n_heads_kv, int head_dim, int dtype, float softmax_scale,
               int out_unnormalized) {
  if (!q || !k || !o || !lse)
    return fail(FA_ERR_INVALID_ARG, "%s: q, k, v, o and lse must be non-null", fn);
  if (out_unnormalized && !row_sum)
    return fail(FA_ERR_INVALID_ARG, "%s: row_sum is required with out_unnormalized", fn);
  if (batch < 1 || seqlen_q < 1 || n_heads_q < 1 || n_heads_kv < 1)
    return fail(FA_ERR_INVALID_ARG, "%s: batch, seqlen_q and head counts must be >= 1", fn);
  if (seqlen_kv < seqlen_q)
    return fail(FA_ERR_INVALID_ARG, "%s: seqlen_kv (%d) < seqlen_q (%d)", fn, seqlen_kv,
                seqlen_q);
  if (n_heads_q % n_heads_kv != 0)
    return fail(FA_ERR_INVALID_ARG, "%s: n_heads_q (%d) %% n_heads_kv (%d) != 0", fn, n_heads_q,
                n_heads_kv);
  if (!prefill_head_dim_supported(head_dim))
    return fail(FA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128, 256, 512}", fn, head_dim);
  if (dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "%s: dtype %d is not FA_F16 or FA_BF16", fn, dtype);
  if (!isfinite(softmax_scale) || !(softmax_scale > 0.0f))
    return fail(FA_ERR_INVALID_ARG, "%s: softmax_scale must be finite and > 0", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(o))
    return fail(FA_ERR_INVALID_ARG, "%s: q, k, v, o must be 16-byte aligned", fn);
  const int64_t hs[6] = {q_sb, q_ss, q_sh, k_sb, k_ss, k_sh};
  for (int i = 0; i < 6; ++i)
    if (hs[i] < 0 || hs[i] % 8 != 0)
      return fail(FA_ERR_INVALID_ARG,
                  "%s: q/k/v strides must be non-negative multiples of 8 elements", fn);
  if (o_sb < 0 || o_ss < 0 || o_sh < 0 || o_sb % 4 || o_ss % 4 || o_sh % 4)
    return fail(FA_ERR_INVALID_ARG, "%s: o strides must be non-negative multiples of 4 elements",
                fn);
  if (seqlen_kv > (1 << 30) || batch > 65535 || n_heads_kv > 65535)
    return fail(FA_ERR_UNSUPPORTED, "%s: seqlen_kv above 2^30 or batch / KV heads above 65535",
                fn);
  if ((int64_t)batch * n_heads_q * (((int64_t)seqlen_q + 127) / 128) > (1 << 30))
    return fail(FA_ERR_UNSUPPORTED, "%s: grid too large (seqlen_q, heads or batch)", fn);
  if (k_ss > (int64_t)(1 << 23))
    return fail(FA_ERR_UNSUPPORTED, "%s: k sequence stride above 2^23 elements", fn);
  return FA_OK;
}

// Length mask and sliding window of a prefill call.
int check_masks(const char* fn, const int32_t* kv_lens, int window, const float* sink_logits) {
  if (window < 0) return fail(FA_ERR_INVALID_ARG, "%s: window (%d) must be >= 0", fn, window);
  if (kv_lens && ((uintptr_t)kv_lens & 3u))
    return fail(FA_ERR_INVALID_ARG, "%s: kv_lens must be 4-byte aligned", fn);
  if (sink_logits && ((uintptr_t)sink_logits & 3u))
    return fail(FA_ERR_INVALID_ARG, "%s: sink_logits must be 4-byte aligned", fn);
  return FA_OK;
}

// Value side of a prefill call (the tensor repacked into the workspace).
int check_pack(const char* fn, const void* v, int64_t v_sb, int64_t v_ss, int64_t v_sh) {
  if (!v) return fail(FA_ERR_INVALID_ARG, "%s: q, k, v, o and lse must be non-null", fn);
  if (!aligned16(v)) return fail(FA_ERR_INVALID_ARG, "%s: q, k, v, o must be 16-byte aligned", fn);
  const int64_t hs[3] = {v_sb, v_ss, v_sh};
  for (int i = 0; i < 3; ++i)
    if (hs[i] < 0 || hs[i] % 8 != 0)
      return fail(FA_ERR_INVALID_ARG,
                  "%s: q/k/v strides must be non-negative multiples of 8 elements", fn);
  return FA_OK;
}

int check_workspace(const char* fn, const void* workspace, uint64_t workspace_bytes, int batch,
                    int seqlen_kv, int n_heads_kv, int head_dim) {
  const uint64_t need = fa::prefill_workspace_bytes(batch, seqlen_kv, n_heads_kv, head_dim);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(FA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned and hold %llu bytes",
                fn, (unsigned long long)need);
  return FA_OK;
}

fa::PrefillArgs prefill_args(const void* q, int64_t q_sb, int64_t q_ss, int64_t q_sh,
                             const void* k, int64_t k_sb, int64_t k_ss, int64_t k_sh,
                             const void* v, int64_t v_sb, int64_t v_ss, int64_t v_sh, float* o,
                             int64_t o_sb, int64_t o_ss, int64_t o_sh, float* lse,
                             float* row_sum, int batch, int seqlen_q, int seqlen_kv,
                             int n_heads_q, int n_heads_kv, int causal, float softmax_scale,
                             const int32_t* kv_lens, int window, const float* sink_logits) {
  fa::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.row_sum = row_sum;
  a.q_sb = q_sb; a.q_ss = q_ss; a.q_sh = q_sh;
  a.k_sb = k_sb; a.k_ss = k_ss; a.k_sh = k_sh;
  a.v_sb = v_sb; a.v_ss = v_ss; a.v_sh = v_sh;
  a.o_sb = o_sb; a.o_ss = o_ss; a.o_sh = o_sh;
  a.batch = batch; a.seqlen_q = seqlen_q; a.seqlen_kv = seqlen_kv;
  a.n_heads_q = n_heads_q; a.n_heads_kv = n_heads_kv;
  a.causal = causal ? 1 : 0;
  a.scale_log2 = softmax_scale * kLog2e;
  a.kv_lens = kv_lens;
  a.window = window;
  a.sink_logits = sink_logits;
  return a;
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_UNKNOWN_STATUS";
  }
}

const char* fa_last_error(void) { return g_err; }

int fa_prefill_fwd(const void* q, int64_t q_sb, int64_t q_ss, int64_t q_sh,
                   const void* k, int64_t k_sb, int64_t k_ss, int64_t k_sh,
                   const void* v, int64_t v_sb, int64_t v_ss, int64_t v_sh,
                   float* o, int64_t o_sb, int64_t o_ss, int64_t o_sh,
                   float* lse, float* row_sum,
                   int batch, int seqlen_q, int seqlen_kv, int n_heads_q, int n_heads_kv,
                   int head_dim, int dtype, int causal, float softmax_scale,
                   int out_unnormalized, const int32_t* kv_lens, int window,
                   const float* sink_logits, void* workspace, uint64_t workspace_bytes,
                   void* stream) {
  const char* fn = "fa_prefill_fwd";
  int st = check_attn(fn, q, q_sb, q_ss, q_sh, k, k_sb, k_ss, k_sh, o, o_sb, o_ss, o_sh, lse,
                      row_sum, batch, seqlen_q, seqlen_kv, n_heads_q, n_heads_kv, head_dim, dtype,
                      softmax_scale, out_unnormalized);
  if (st == FA_OK) st = check_masks(fn, kv_lens, window, sink_logits);
  if (st == FA_OK) st = check_pack(fn, v, v_sb, v_ss, v_sh);
  // fp16 at head_dim <= 128: one launch reading V's rows, no workspace
  const bool rows = fa::prefill_reads_v_rows(head_dim, dtype == FA_BF16);
  if (st == FA_OK && !rows)
    st = check_workspace(fn, workspace, workspace_bytes, batch, seqlen_kv, n_heads_kv, head_dim);
  if (st == FA_OK && rows && v_ss > (int64_t)(1 << 23))
    st = fail(FA_ERR_UNSUPPORTED, "%s: v sequence stride above 2^23 elements", fn);
  if (st != FA_OK) return st;
  const fa::PrefillArgs a =
      prefill_args(q, q_sb, q_ss, q_sh, k, k_sb, k_ss, k_sh, v, v_sb, v_ss, v_sh, o, o_sb, o_ss,
                   o_sh, lse, row_sum, batch, seqlen_q, seqlen_kv, n_heads_q, n_heads_kv, causal,
                   softmax_scale, kv_lens, window, sink_logits);
  if (rows)
    return hip_status(fa::launch_prefill_attn_vrow(a, head_dim, out_unnormalized != 0,
                                                   (hipStream_t)stream),
                      "fa_prefill_fwd attention launch");
  const fa::VtArgs w{workspace, (size_t)workspace_bytes};
  const hipError_t e =
      fa::launch_prefill_pack(a, w, head_dim, dtype == FA_BF16, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "fa_prefill_fwd V repack launch");
  return hip_status(fa::launch_prefill_attn(a, w, head_dim, dtype == FA_BF16,
                                            out_unnormalized != 0, (hipStream_t)stream),
                    "fa_prefill_fwd attention launch");
}

int fa_prefill_pack_v(const void* v, int64_t v_sb, int64_t v_ss, int64_t v_sh, int batch,
                      int seqlen_kv, int n_heads_kv, int head_dim, int dtype, void* workspace,
                      uint64_t workspace_bytes, void* stream) {
  const char* fn = "fa_prefill_pack_v";
  if (batch < 1 || seqlen_kv < 1 || n_heads_kv < 1)
    return fail(FA_ERR_INVALID_ARG, "%s: batch, seqlen_kv and n_heads_kv must be >= 1", fn);
  if (!prefill_head_dim_supported(head_dim))
    return fail(FA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128, 256, 512}", fn, head_dim);
  if (dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "%s: dtype %d is not FA_F16 or FA_BF16", fn, dtype);
  if (seqlen_kv > (1 << 30) || batch > 65535 || n_heads_kv > 65535)
    return fail(FA_ERR_UNSUPPORTED, "%s: seqlen_kv above 2^30 or batch / heads above 65535", fn);
  int st = check_pack(fn, v, v_sb, v_ss, v_sh);
  if (st == FA_OK)
    st = check_workspace(fn, workspace, workspace_bytes, batch, seqlen_kv, n_heads_kv, head_dim);
  if (st != FA_OK) return st;
  fa::PrefillArgs a{};
  a.v = v; a.v_sb = v_sb; a.v_ss = v_ss; a.v_sh = v_sh;
  a.batch = batch; a.seqlen_kv = seqlen_kv; a.n_heads_kv = n_heads_kv;
  const fa::VtArgs w{workspace, (size_t)workspace_bytes};
  return hip_status(fa::launch_prefill_pack(a, w, head_dim, dtype == FA_BF16, (hipStream_t)stream),
                    "fa_prefill_pack_v launch");
}

int fa_prefill_fwd_packed(const void* q, int64_t q_sb, int64_t q_ss, int64_t q_sh,
                          const void* k, int64_t k_sb, int64_t k_ss, int64_t k_sh,
                          float* o, int64_t o_sb, int64_t o_ss, int64_t o_sh,
                          float* lse, float* row_sum,
                          int batch, int seqlen_q, int seqlen_kv, int n_heads_q, int n_heads_kv,
                          int head_dim, int dtype, int causal, float softmax_scale,
                          int out_unnormalized, const int32_t* kv_lens, int window,
                          const float* sink_logits, const void* workspace,
                          uint64_t workspace_bytes, void* stream) {
  const char* fn = "fa_prefill_fwd_packed";
  int st = check_attn(fn, q, q_sb, q_ss, q_sh, k, k_sb, k_ss, k_sh, o, o_sb, o_ss, o_sh, lse,
                      row_sum, batch, seqlen_q, seqlen_kv, n_heads_q, n_heads_kv, head_dim, dtype,
                      softmax_scale, out_unnormalized);
  if (st == FA_OK) st = check_masks(fn, kv_lens, window, sink_logits);
  if (st == FA_OK)
    st = check_workspace(fn, workspace, workspace_bytes, batch, seqlen_kv, n_heads_kv, head_dim);
  if (st != FA_OK) return st;
  const fa::PrefillArgs a =
      prefill_args(q, q_sb, q_ss, q_sh, k, k_sb, k_ss, k_sh, nullptr, 0, 0, 0, o, o_sb, o_ss,
                   o_sh, lse, row_sum, batch, seqlen_q, seqlen_kv, n_heads_q, n_heads_kv, causal,
                   softmax_scale, kv_lens, window, sink_logits);
  const fa::VtArgs w{const_cast<void*>(workspace), (size_t)workspace_bytes};
  return hip_status(fa::launch_prefill_attn(a, w, head_dim, dtype == FA_BF16,
                                            out_unnormalized != 0, (hipStream_t)stream),
                    "fa_prefill_fwd_packed launch");
}

int fa_prefill_fwd_packed_split(const void* q, int64_t q_sb, int64_t q_ss, int64_t q_sh,
                                const void* k, int64_t k_sb, int64_t k_ss, int64_t k_sh,
                                float* o, int64_t o_sb, int64_t o_ss, int64_t o_sh,
                                float* lse, float* row_sum,
                                int batch, int seqlen_q, int seqlen_kv, int n_heads_q,
                                int n_heads_kv, int head_dim, int dtype, int causal,
                                float softmax_scale, int out_unnormalized, const int32_t* kv_lens,
                                int window, const float* sink_logits, const void* workspace,
                                uint64_t workspace_bytes, void* split_workspace,
                                uint64_t split_workspace_bytes, void* stream) {
  const char* fn = "fa_prefill_fwd_packed_split";
  int st = check_attn(fn, q, q_sb, q_ss, q_sh, k, k_sb, k_ss, k_sh, o, o_sb, o_ss, o_sh, lse,
                      row_sum, batch, seqlen_q, seqlen_kv, n_heads_q, n_heads_kv, head_dim, dtype,
                      softmax_scale, out_unnormalized);
  if (st == FA_OK) st = check_masks(fn, kv_lens, window, sink_logits);
  if (st == FA_OK)
    st = check_workspace(fn, workspace, workspace_bytes, batch, seqlen_kv, n_heads_kv, head_dim);
  if (st != FA_OK) return st;
  const fa::SplitLayout L = fa::prefill_split_layout(batch, seqlen_q, n_heads_q, head_dim);
  if (!split_workspace || split_workspace_bytes < L.total || ((uintptr_t)split_workspace & 255u))
    return fail(FA_ERR_INVALID_ARG,
                "%s: split workspace must be 256-byte aligned and hold %llu bytes", fn,
                (unsigned long long)L.total);
  const fa::PrefillArgs a =
      prefill_args(q, q_sb, q_ss, q_sh, k, k_sb, k_ss, k_sh, nullptr, 0, 0, 0, o, o_sb, o_ss,
                   o_sh, lse, row_sum, batch, seqlen_q, seqlen_kv, n_heads_q, n_heads_kv, causal,
                   softmax_scale, kv_lens, window, sink_logits);
  const fa::VtArgs w{const_cast<void*>(workspace), (size_t)workspace_bytes};
  fa::SplitPlan sp{};
  if (!out_unnormalized && !row_sum)
    sp.n_units = fa::prefill_split_units(batch, seqlen_q, seqlen_kv, n_heads_q, n_heads_kv,
                                         head_dim, causal, window, sp.units);
  if (sp.n_units == 0)
    return hip_status(fa::launch_prefill_attn(a, w, head_dim, dtype == FA_BF16,
                                              out_unnormalized != 0, (hipStream_t)stream),
                      "fa_prefill_fwd_packed_split launch");
  char* ws = (char*)split_workspace;
  sp.cnt = (int*)(ws + L.cnt);
  sp.lse = (float*)(ws + L.lse);
  sp.o = (float*)(ws + L.o);
  return hip_status(fa::launch_prefill_attn_split(a, w, sp, head_dim, dtype == FA_BF16,
                                                  (hipStream_t)stream),
                    "fa_prefill_fwd_packed_split launch");
}

uint64_t fa_prefill_split_workspace_size(int batch, int seqlen_q, int n_heads_q, int head_dim) {
  const size_t t = fa::prefill_split_layout(batch, seqlen_q, n_heads_q, head_dim).total;
  return t == SIZE_MAX ? 0 : t;
}

int fa_prefill_split_units(int batch, int seqlen_q, int seqlen_kv, int n_heads_q, int n_heads_kv,
                           int head_dim, int causal, int window, uint16_t* units, int max_units) {
  if (batch <= 0 || seqlen_q <= 0 || seqlen_kv <= 0 || n_heads_q <= 0 || n_heads_kv <= 0 ||
      n_heads_q % n_heads_kv != 0 || window < 0 || max_units < 0)
    return -fail(FA_ERR_INVALID_ARG, "fa_prefill_split_units: invalid sizes");
  unsigned short tab[fa::kMaxSplitUnits];
  const int n = fa::prefill_split_units(batch, seqlen_q, seqlen_kv, n_heads_q, n_heads_kv,
                                        head_dim, causal, window, tab);
  if (units)
    for (int i = 0; i < n && i < max_units; ++i) units[i] = tab[i];
  return n;
}

int fa_prefill_trio(int batch, int seqlen_q, int seqlen_kv, int n_heads_q, int n_heads_kv,
                    int head_dim, int causal, int window) {
  if (batch <= 0 || seqlen_q <= 0 || seqlen_kv <= 0 || n_heads_q <= 0 || n_heads_kv <= 0 ||
      n_heads_q % n_heads_kv != 0 || window < 0)
    return -fail(FA_ERR_INVALID_ARG, "fa_prefill_trio: invalid sizes");
  return fa::prefill_trio(batch, seqlen_q, seqlen_kv, n_heads_q, n_heads_kv, head_dim, causal,
                          window) ? 1 : 0;
}

int fa_attn_merge(const float* o_a, int64_t oa_sb, int64_t oa_ss, int64_t oa_sh,
                  const float* lse_a, const float* o_b, int64_t ob_sb, int64_t ob_ss,
                  int64_t ob_sh, const float* lse_b, const float* sink_logits, int batch,
                  int seqlen, int n_heads, int head_dim, float* o, int64_t o_sb, int64_t o_ss,
                  int64_t o_sh, float* lse, void* stream) {
  const char* fn = "fa_attn_merge";
  if (!o_a || !lse_a || !o || !lse)
    return fail(FA_ERR_INVALID_ARG, "%s: o_a, lse_a, o and lse must be non-null", fn);
  if (!o_b != !lse_b)
    return fail(FA_ERR_INVALID_ARG, "%s: o_b and lse_b must both be given or both be null", fn);
  if (batch < 1 || seqlen < 1 || n_heads < 1)
    return fail(FA_ERR_INVALID_ARG, "%s: batch, seqlen and n_heads must be >= 1", fn);
  if (!head_dim_supported(head_dim))
    return fail(FA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128, 256}", fn, head_dim);
  if (!aligned16(o_a) || !aligned16(o) || (o_b && !aligned16(o_b)))
    return fail(FA_ERR_INVALID_ARG, "%s: o_a, o_b and o must be 16-byte aligned", fn);
  if (((uintptr_t)lse_a & 3u) || ((uintptr_t)lse & 3u) || ((uintptr_t)lse_b & 3u) ||
      ((uintptr_t)sink_logits & 3u))
    return fail(FA_ERR_INVALID_ARG, "%s: lse and sink arrays must be 4-byte aligned", fn);
  const int64_t st[9] = {oa_sb, oa_ss, oa_sh, ob_sb, ob_ss, ob_sh, o_sb, o_ss, o_sh};
  for (int i = 0; i < 9; ++i)
    if ((i < 3 || i >= 6 || o_b) && (st[i] < 0 || st[i] % 4))
      return fail(FA_ERR_INVALID_ARG, "%s: o strides must be non-negative multiples of 4", fn);
  // one work-item per 16 bytes of O: at most 2^31 of them in the 1-D grid
  if (fa::sat_mul(fa::sat_mul((size_t)batch, (size_t)seqlen),
                  fa::sat_mul((size_t)n_heads, (size_t)(head_dim / 4))) > ((size_t)1 << 31))
    return fail(FA_ERR_UNSUPPORTED, "%s: too many rows", fn);
  fa::BranchMergeArgs a;
  a.o_a = o_a; a.lse_a = lse_a; a.o_b = o_b; a.lse_b = lse_b; a.sink_logits = sink_logits;
  a.o = o; a.lse = lse;
  a.oa_sb = oa_sb; a.oa_ss = oa_ss; a.oa_sh = oa_sh;
  a.ob_sb = ob_sb; a.ob_ss = ob_ss; a.ob_sh = ob_sh;
  a.o_sb = o_sb; a.o_ss = o_ss; a.o_sh = o_sh;
  a.batch = batch; a.seqlen = seqlen; a.n_heads = n_heads;
  return hip_status(fa::launch_branch_merge(a, head_dim, (hipStream_t)stream),
                    "fa_attn_merge launch");
}

uint64_t fa_prefill_workspace_size(int batch, int seqlen_kv, int n_heads_kv, int head_dim) {
  if (batch < 1 || seqlen_kv < 1 || n_heads_kv < 1 || head_dim < 1) return 0;
  const size_t t = fa::prefill_workspace_bytes(batch, seqlen_kv, n_heads_kv, head_dim);
  return t == SIZE_MAX ? 0 : t;
}

// Longest KV length the decode planner accepts (2^30 tokens).
constexpr int kMaxPlanKvLen = 1 << 30;

int fa_decode_plan(const int32_t* kv_lens_host, int batch, int n_heads_q, int n_heads_kv,
                   int head_dim, int num_cus, int* split_len_out, int* max_splits_out) {
  if (!kv_lens_host || !split_len_out || !max_splits_out)
    return fail(FA_ERR_INVALID_ARG, "fa_decode_plan: null pointer argument");
  if (batch < 1 || n_heads_q < 1 || n_heads_kv < 1 || n_heads_q % n_heads_kv != 0 ||
      num_cus < 1)
    return fail(FA_ERR_INVALID_ARG, "fa_decode_plan: bad batch, head counts or num_cus");
  if (!head_dim_supported(head_dim))
    return fail(FA_ERR_UNSUPPORTED, "fa_decode_plan: head_dim %d not in {64, 128, 256}",
                head_dim);
  int max_len = 0;
  for (int b = 0; b < batch; ++b) {
    if (kv_lens_host[b] < 1)
      return fail(FA_ERR_INVALID_ARG, "fa_decode_plan: kv_lens[%d] = %d < 1", b, kv_lens_host[b]);
    if (kv_lens_host[b] > kMaxPlanKvLen)
      return fail(FA_ERR_UNSUPPORTED, "fa_decode_plan: kv_lens[%d] = %d above %d", b,
                  kv_lens_host[b], kMaxPlanKvLen);
    if (kv_lens_host[b] > max_len) max_len = kv_lens_host[b];
  }
  const int g = fa::decode_max_heads_per_wave(n_heads_q / n_heads_kv);
  // split lengths step in whole row blocks of the partial kernel, and in at
  // least 16 keys (the granularity every decode entry point accepts)
  const int bk = std::max(16, fa::decode_block_rows(head_dim, g));
  const int64_t slots = (int64_t)num_cus * fa::decode_waves_per_cu(head_dim);
  const int64_t groups = n_heads_q / g;    // waves per (sequence, split)
  auto waves_of = [&](int64_t sl, int64_t* max_ns) {
    int64_t w = 0, mx = 0;
    for (int b = 0; b < batch; ++b) {
      const int64_t ns = (kv_lens_host[b] + sl - 1) / sl;
      w += ns;
      if (ns > mx) mx = ns;
    }
    if (max_ns) *max_ns = mx;
    return w * groups;
  };
  // Candidates are whole blocks of rows. Two regimes:
  //  * everything fits in one round of resident waves even at one block per
  //    split: latency-bound; minimize the rows a wave streams plus ~0.6 row
  //    per split the merge reads;
  //  * otherwise bandwidth-bound: maximize how full the rounds of resident
  //    waves are (a half-empty last round costs nearly a full one), with a
  //    small charge per extra round; ties go to the shorter split.
  int best = bk;
  double best_score = -1e300;
  const bool latency_bound = waves_of(bk, nullptr) <= slots;
  // Every whole number of blocks up to the longest sequence is a candidate;
  // past ~4096 candidates (lengths above 4096 blocks) they are thinned to
  // multiples of a coarser step, which keeps the plan cheap to compute.
  const int64_t n_cand = ((int64_t)max_len + bk - 1) / bk;
  const int64_t step = (int64_t)bk * ((n_cand + 4095) / 4096);
  for (int64_t sl = bk;; sl += step) {
    int64_t max_ns = 0;
    const int64_t waves = waves_of(sl, &max_ns);
    const int64_t rounds = (waves + slots - 1) / slots;
    const double score = latency_bound
                             ? -((double)sl + 0.6 * (double)max_ns)
                             : (double)waves / (double)(rounds * slots) - 0.04 * (double)rounds;
    if (score > best_score) {
      best_score = score;
      best = (int)sl;
    }
    if (sl >= max_len) break;
  }
  *split_len_out = best;
  *max_splits_out = (int)(((int64_t)max_len + best - 1) / best);
  return ok();
}

}  // extern "C"

namespace {

// Query/cache side of a decode call (shared by the split and fused forms).
int check_decode(const char* fn, const void* q, int64_t q_sb, int64_t q_sh, const void* k_cache,
                 const void* v_cache, int64_t kv_stride_tok, int64_t kv_stride_head,
                 const int64_t* kv_offsets, const int32_t* kv_lens, int batch, int n_heads_q,
                 int n_heads_kv, int head_dim, int dtype, float softmax_scale, int split_len,
                 int max_splits) {
  if (!q || !k_cache || !v_cache || !kv_offsets || !kv_lens)
    return fail(FA_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (batch < 1 || n_heads_q < 1 || n_heads_kv < 1 || n_heads_q % n_heads_kv != 0)
    return fail(FA_ERR_INVALID_ARG, "%s: bad batch or head counts", fn);
  if (!head_dim_supported(head_dim))
    return fail(FA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128, 256}", fn, head_dim);
  if (dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "%s: unsupported dtype %d", fn, dtype);
  if (!isfinite(softmax_scale) || !(softmax_scale > 0.0f))
    return fail(FA_ERR_INVALID_ARG, "%s: softmax_scale must be finite and > 0", fn);
  if (split_len < 16 || split_len % 16 != 0 || max_splits < 1)
    return fail(FA_ERR_INVALID_ARG,
                "%s: split_len must be a positive multiple of 16, max_splits >= 1", fn);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(FA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  if (q_sb < 0 || q_sh < 0 || kv_stride_tok < 0 || kv_stride_head < 0 || q_sb % 8 ||
      q_sh % 8 || kv_stride_tok % 8 || kv_stride_head % 8)
    return fail(FA_ERR_INVALID_ARG, "%s: strides must be non-negative multiples of 8", fn);
  if (max_splits > 2147483647 / 2 || batch > 65535 || n_heads_q > 65535)
    return fail(FA_ERR_UNSUPPORTED, "%s: grid too large", fn);
  // key positions s * split_len + row of the last split are 32-bit on the device
  if ((int64_t)split_len * max_splits > 2147483647 - 65536)
    return fail(FA_ERR_UNSUPPORTED, "%s: split_len * max_splits above the 32-bit key range", fn);
  return FA_OK;
}

fa::DecodeArgs decode_args(const void* q, int64_t q_sb, int64_t q_sh, const void* k_cache,
                           const void* v_cache, int64_t kv_stride_tok, int64_t kv_stride_head,
                           const int64_t* kv_offsets, const int32_t* kv_lens, int batch,
                           int n_heads_q, int n_heads_kv, float softmax_scale, int split_len,
                           int max_splits) {
  fa::DecodeArgs a{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.kv_offsets = kv_offsets; a.kv_lens = kv_lens;
  a.q_sb = q_sb; a.q_sh = q_sh; a.kv_st = kv_stride_tok; a.kv_sh = kv_stride_head;
  a.batch = batch; a.n_heads_q = n_heads_q; a.n_heads_kv = n_heads_kv;
  a.split_len = split_len; a.max_splits = max_splits;
  a.scale_log2 = softmax_scale * kLog2e;
  return a;
}

}  // namespace

extern "C" {

int fa_decode_split_partial(const void* q, int64_t q_sb, int64_t q_sh,
                            const void* k_cache, const void* v_cache,
                            int64_t kv_stride_tok, int64_t kv_stride_head,
                            const int64_t* kv_offsets, const int32_t* kv_lens,
                            int batch, int n_heads_q, int n_heads_kv, int head_dim, int dtype,
                            float softmax_scale, int split_len, int max_splits,
                            float* part_o, float* part_lse, void* stream) {
  const char* fn = "fa_decode_split_partial";
  if (!part_o || !part_lse) return fail(FA_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned16(part_o)) return fail(FA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  const int st = check_decode(fn, q, q_sb, q_sh, k_cache, v_cache, kv_stride_tok,
                              kv_stride_head, kv_offsets, kv_lens, batch, n_heads_q, n_heads_kv,
                              head_dim, dtype, softmax_scale, split_len, max_splits);
  if (st != FA_OK) return st;
  fa::DecodeArgs a = decode_args(q, q_sb, q_sh, k_cache, v_cache, kv_stride_tok, kv_stride_head,
                                 kv_offsets, kv_lens, batch, n_heads_q, n_heads_kv,
                                 softmax_scale, split_len, max_splits);
  a.part_o = part_o; a.part_lse = part_lse;
  return hip_status(fa::launch_decode_partial(a, head_dim, dtype == FA_BF16, (hipStream_t)stream),
                    "fa_decode_split_partial launch");
}

// The single-launch decode on a validated call with its scratch at ws (layout f).
static int launch_fused(const void* q, int64_t q_sb, int64_t q_sh, const void* k_cache,
                        const void* v_cache, int64_t kv_stride_tok, int64_t kv_stride_head,
                        const int64_t* kv_offsets, const int32_t* kv_lens, int batch,
                        int n_heads_q, int n_heads_kv, int head_dim, int dtype,
                        float softmax_scale, int split_len, int max_splits, float* o, float* lse,
                        const fa::FusedLayout& f, char* ws, void* stream, const char* what) {
  fa::DecodeArgs a = decode_args(q, q_sb, q_sh, k_cache, v_cache, kv_stride_tok, kv_stride_head,
                                 kv_offsets, kv_lens, batch, n_heads_q, n_heads_kv,
                                 softmax_scale, split_len, max_splits);
  a.o = o; a.lse = lse;
  a.counters = (int*)(ws + f.counters);
  a.wg_lse = (float*)(ws + f.wg_lse);
  a.wg_o = (float*)(ws + f.wg_o);
  a.max_wg = f.max_wg;
  return hip_status(fa::launch_decode_fused(a, head_dim, dtype == FA_BF16, (hipStream_t)stream),
                    what);
}

int fa_decode_fused(const void* q, int64_t q_sb, int64_t q_sh,
                    const void* k_cache, const void* v_cache,
                    int64_t kv_stride_tok, int64_t kv_stride_head,
                    const int64_t* kv_offsets, const int32_t* kv_lens,
                    int batch, int n_heads_q, int n_heads_kv, int head_dim, int dtype,
                    float softmax_scale, int split_len, int max_splits,
                    float* o, float* lse, void* workspace, uint64_t workspace_bytes,
                    void* stream) {
  const char* fn = "fa_decode_fused";
  if (!o || !lse) return fail(FA_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  const int st = check_decode(fn, q, q_sb, q_sh, k_cache, v_cache, kv_stride_tok,
                              kv_stride_head, kv_offsets, kv_lens, batch, n_heads_q, n_heads_kv,
                              head_dim, dtype, softmax_scale, split_len, max_splits);
  if (st != FA_OK) return st;
  const fa::FusedLayout f =
      fa::decode_fused_layout(batch, n_heads_q, n_heads_kv, head_dim, max_splits);
  if (f.n_counters * (int64_t)sizeof(int) > (int64_t)fa::kFusedCounterBytes)
    return fail(FA_ERR_UNSUPPORTED, "%s: batch * head groups (%lld) above %d", fn,
                (long long)f.n_counters, (int)(fa::kFusedCounterBytes / sizeof(int)));
  if (!workspace || workspace_bytes < f.total || ((uintptr_t)workspace & 255u))
    return fail(FA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned and hold %llu bytes",
                fn, (unsigned long long)f.total);
  return launch_fused(q, q_sb, q_sh, k_cache, v_cache, kv_stride_tok, kv_stride_head, kv_offsets,
                      kv_lens, batch, n_heads_q, n_heads_kv, head_dim, dtype, softmax_scale,
                      split_len, max_splits, o, lse, f, (char*)workspace, stream,
                      "fa_decode_fused launch");
}

int fa_decode_fused_noalloc(const void* q, int64_t q_sb, int64_t q_sh,
                            const void* k_cache, const void* v_cache,
                            int64_t kv_stride_tok, int64_t kv_stride_head,
                            const int64_t* kv_offsets, const int32_t* kv_lens,
                            int batch, int n_heads_q, int n_heads_kv, int head_dim, int dtype,
                            float softmax_scale, int split_len, int max_splits,
                            float* o, float* lse, void* stream) {
  const char* fn = "fa_decode_fused_noalloc";
  if (!o || !lse) return fail(FA_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  const int st = check_decode(fn, q, q_sb, q_sh, k_cache, v_cache, kv_stride_tok,
                              kv_stride_head, kv_offsets, kv_lens, batch, n_heads_q, n_heads_kv,
                              head_dim, dtype, softmax_scale, split_len, max_splits);
  if (st != FA_OK) return st;
  const fa::FusedLayout f =
      fa::decode_fused_layout(batch, n_heads_q, n_heads_kv, head_dim, max_splits);
  if (f.n_counters * (int64_t)sizeof(int) > (int64_t)fa::kFusedCounterBytes)
    return fail(FA_ERR_UNSUPPORTED, "%s: batch * head groups (%lld) above %d", fn,
                (long long)f.n_counters, (int)(fa::kFusedCounterBytes / sizeof(int)));
  if (f.total > fa::kNoAllocScratchBytes)
    return fail(FA_ERR_UNSUPPORTED,
                "%s: this shape needs %llu bytes of scratch, above the library's %llu "
                "(use fa_decode_fused with a caller workspace)", fn,
                (unsigned long long)f.total, (unsigned long long)fa::kNoAllocScratchBytes);
  void* ws = nullptr;
  const hipError_t e = fa::decode_noalloc_scratch(&ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "fa_decode_fused_noalloc scratch set-up");
  return launch_fused(q, q_sb, q_sh, k_cache, v_cache, kv_stride_tok, kv_stride_head, kv_offsets,
                      kv_lens, batch, n_heads_q, n_heads_kv, head_dim, dtype, softmax_scale,
                      split_len, max_splits, o, lse, f, (char*)ws, stream,
                      "fa_decode_fused_noalloc launch");
}

uint64_t fa_decode_fused_workspace_size(int batch, int n_heads_q, int n_heads_kv, int head_dim,
                                        int max_splits) {
  if (batch < 1 || n_heads_q < 1 || n_heads_kv < 1 || n_heads_q % n_heads_kv != 0 ||
      !head_dim_supported(head_dim) || max_splits < 1)
    return 0;
  const size_t t = fa::decode_fused_layout(batch, n_heads_q, n_heads_kv, head_dim, max_splits).total;
  return t == SIZE_MAX ? 0 : t;
}

int fa_decode_fused_waves(int batch, int n_heads_q, int n_heads_kv, int head_dim,
                          int max_splits) {
  if (batch < 1 || n_heads_q < 1 || n_heads_kv < 1 || n_heads_q % n_heads_kv != 0 ||
      !head_dim_supported(head_dim) || max_splits < 1)
    return 0;
  return fa::decode_fused_waves(batch, n_heads_q, n_heads_kv, head_dim, max_splits);
}

int fa_decode_merge_lse(const float* part_o, const float* part_lse, const int32_t* kv_lens,
                        int batch, int n_heads_q, int head_dim, int split_len, int max_splits,
                        float* o, float* lse, void* stream) {
  if (!part_o || !part_lse || !kv_lens || !o || !lse)
    return fail(FA_ERR_INVALID_ARG, "fa_decode_merge_lse: null pointer argument");
  if (batch < 1 || n_heads_q < 1 || split_len < 1 || max_splits < 1)
    return fail(FA_ERR_INVALID_ARG, "fa_decode_merge_lse: sizes must be >= 1");
  if (!head_dim_supported(head_dim))
    return fail(FA_ERR_UNSUPPORTED, "fa_decode_merge_lse: head_dim %d not in {64, 128, 256}",
                head_dim);
  if (batch > 65535 || n_heads_q > 2147483647 / 2)
    return fail(FA_ERR_UNSUPPORTED, "fa_decode_merge_lse: grid too large");
  fa::MergeArgs a;
  a.part_o = part_o; a.part_lse = part_lse; a.kv_lens = kv_lens; a.o = o; a.lse = lse;
  a.batch = batch; a.n_heads_q = n_heads_q; a.split_len = split_len; a.max_splits = max_splits;
  return hip_status(fa::launch_decode_merge(a, head_dim, (hipStream_t)stream),
                    "fa_decode_merge_lse launch");
}

}  // extern "C"
