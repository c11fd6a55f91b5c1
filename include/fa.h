/*
 * fa.h — C ABI of the MI355X (gfx950) exact-attention library libfa.so.
 *
 * The library computes exact scaled-dot-product attention with a tiled online
 * softmax on hand-written gfx950 HIP kernels:
 *
 *   - prefill: causal (or unmasked) GQA forward producing O and the per-row
 *     log-sum-exp;
 *   - decode: one query token per sequence against a KV cache, computed as
 *     split-KV partials followed by a merge of the partials by their LSE.
 *
 * Definitions (all entry points):
 *   s_ij = softmax_scale * sum_d q[i,d] * k[j,d]   for visible keys j
 *   P_ij = exp(s_ij - m_i), m_i = max_j s_ij, l_i = sum_j P_ij (row sum)
 *   O_i  = sum_j P_ij v[j,:] / l_i,   LSE_i = m_i + ln(l_i)   (natural log)
 * Source: "STAGE_D.md — FMHA Kernel Development", section "Kernel Output"
 * (un-normalized output, row sum and LSE; normalization outside the kernel is
 * exact) and sections D3/D4 (a key is masked iff its index exceeds the query
 * position). Query head h reads KV head h / (n_heads_q / n_heads_kv): the
 * KV-head addressing of "60 · r57 — FA KV staging double buffering
 * (REVERTED)", section 2.2, with contiguous head groups.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer owned by the caller. The
 *     library never allocates, frees or synchronizes; it only enqueues
 *     kernels on `stream` (a hipStream_t; NULL means the null stream).
 *   - Half-precision inputs are fp16 or bf16 bit patterns (fa_dtype); all
 *     arithmetic accumulates in fp32; every output is fp32.
 *   - Strides are in ELEMENTS; the innermost (head_dim) stride is always 1.
 *   - Arguments are validated on the host before any HIP call. A rejected
 *     call returns FA_ERR_INVALID_ARG or FA_ERR_UNSUPPORTED, enqueues
 *     nothing, and leaves a description in fa_last_error(). A failed kernel
 *     launch returns FA_ERR_HIP with the HIP error text.
 *   - Results are deterministic: the same inputs and the same plan give the
 *     same bytes on every run (fixed reduction orders; the one atomic, the
 *     arrival counter of fa_decode_fused, only decides which work-group
 *     performs the final merge, not its order).
 *   - Thread-safe: no mutable global state besides the per-thread error text.
 */
#ifndef FA_H
#define FA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,  /* null pointer, bad size/stride/alignment, non-finite scale */
  FA_ERR_UNSUPPORTED = 2,  /* valid request outside the supported set (head_dim, dtype) */
  FA_ERR_HIP = 3           /* a HIP runtime call or kernel launch failed */
} fa_status;

typedef enum { FA_F16 = 0, FA_BF16 = 1 } fa_dtype;

/*
 * fa_prefill_fwd — attention forward over a whole prompt.
 *
 * Source: "STAGE_D.md — FMHA Kernel Development", "Kernel Output" (O, row
 * sum, LSE; external normalization), D3 (per-sequence length mask) and D4
 * (causal mask on the windowed branch); "60 · r57 —
 * FA KV staging double buffering (REVERTED)", sections 1 and 2.2 (grid over
 * query block and head, KV tiles streamed up to the causal bound).
 *
 * Layouts (element strides, innermost dim contiguous):
 *   q  [batch, seqlen_q,  n_heads_q,  head_dim]  half, strides q_sb, q_ss, q_sh
 *   k  [batch, seqlen_kv, n_heads_kv, head_dim]  half, strides k_sb, k_ss, k_sh
 *   v  [batch, seqlen_kv, n_heads_kv, head_dim]  half, strides v_sb, v_ss, v_sh
 *   o  [batch, seqlen_q,  n_heads_q,  head_dim]  fp32, strides o_sb, o_ss, o_sh
 *   lse     [batch, n_heads_q, seqlen_q] fp32, contiguous (natural-log LSE)
 *   row_sum [batch, n_heads_q, seqlen_q] fp32, contiguous, or NULL
 *
 * Query row i sits at position p_i = i + (seqlen_kv - seqlen_q) (bottom-right
 * alignment). Key j is visible to row i when every enabled mask admits it:
 *   causal != 0       j <= p_i                (D4: causal mask)
 *   kv_lens != NULL   j < kv_lens[b]          (D3: per-sequence length mask)
 *   window > 0        j > p_i - window        (sliding window of `window`
 *                                              positions ending at p_i)
 * kv_lens is a DEVICE array [batch] of int32 (4-byte aligned) or NULL (all
 * seqlen_kv keys valid); each value is clamped to [0, seqlen_kv] on the
 * device. window == 0 disables the window; window < 0 is rejected. The masks
 * combine freely (causal == 0 with a window admits every key after
 * p_i - window). A row that sees no key gets o = 0, row_sum = 0 and
 * lse = -inf. Hidden keys that share a key tile (64 keys; 32 at head_dim
 * 256 and 512) with visible ones are read and given weight zero, so K and V must hold
 * finite values there too (V within fp16 range; padding past kv_lens[b]
 * included); tiles with no visible key are skipped.
 *
 * sink_logits: DEVICE array [n_heads_q] of fp32 (4-byte aligned) or NULL. The
 * sink of query head h joins every row's softmax as one more term
 * exp(sink_logits[h]) with no value row (D5/D5d: the sink merge folded into
 * the epilogue), so lse = ln(sum_j exp(s_ij) + exp(sink)), o is normalized by
 * that sum, and in un-normalized mode o and row_sum refer to
 * m_i = max(max_j s_ij, sink). A row with no key then gets o = 0,
 * lse = sink (row_sum = 1 in un-normalized mode).
 *
 * out_unnormalized == 0: o = normalized output; row_sum (optional) = l_i.
 * out_unnormalized != 0: o = sum_j P_ij v[j,:] with P_ij = exp(s_ij - m_i)
 *   (m_i the row's true max), row_sum = l_i (required); the caller normalizes
 *   o / row_sum.
 *
 * workspace: caller-owned device scratch of at least
 * fa_prefill_workspace_size(batch, seqlen_kv, n_heads_kv, head_dim) bytes,
 * 256-byte aligned. For bf16 inputs, and fp16 inputs at head_dim 256 and 512,
 * the call first repacks V into it (fp16, transposed per key tile), then runs
 * the attention kernel; its contents are undefined afterwards and it must not
 * be shared by calls that overlap in time. fp16 inputs at head_dim 64 and 128
 * take one launch that reads V's rows in place (transposing loads from LDS):
 * workspace and workspace_bytes are then ignored and may be NULL and 0, and
 * v stride_s must be at most 2^23 elements, as k's.
 *
 * Supported set: head_dim in {64, 128, 256, 512} (512: "STAGE_D.md", D1.4,
 * with the Q.K^T contraction split over a pair of waves); dtype FA_F16 or
 * FA_BF16; n_heads_q % n_heads_kv == 0; 1 <= seqlen_q <= seqlen_kv <= 2^30;
 * 1 <= batch, n_heads_kv <= 65535 with batch * n_heads_q * ceil(seqlen_q / 128)
 * <= 2^30;
 * softmax_scale finite and > 0; q/k/v/o base pointers 16-byte aligned; q/k/v
 * stride_s, stride_h and stride_b multiples of 8, o strides multiples of 4;
 * k stride_s at most 2^23 elements.
 * V values of bf16 inputs are taken to fp16 for the P.V contraction (exact in
 * fp16's normal range; |v| >= 65520 overflows and is outside the contract).
 * The inputs are read, never written; o/lse/row_sum are written in full.
 */
int fa_prefill_fwd(const void* q, int64_t q_sb, int64_t q_ss, int64_t q_sh,
                   const void* k, int64_t k_sb, int64_t k_ss, int64_t k_sh,
                   const void* v, int64_t v_sb, int64_t v_ss, int64_t v_sh,
                   float* o, int64_t o_sb, int64_t o_ss, int64_t o_sh,
                   float* lse, float* row_sum,
                   int batch, int seqlen_q, int seqlen_kv, int n_heads_q, int n_heads_kv,
                   int head_dim, int dtype, int causal, float softmax_scale,
                   int out_unnormalized, const int32_t* kv_lens, int window,
                   const float* sink_logits, void* workspace, uint64_t workspace_bytes,
                   void* stream);

/*
 * fa_prefill_pack_v / fa_prefill_fwd_packed — fa_prefill_fwd in its two
 * launches, for callers that attend several query sets to one V (a cached
 * prefix) or that time the attention kernel on its own.
 *
 * Source: as fa_prefill_fwd; the V^T tile layout is the operand order of the
 * P.V product of "STAGE_D.md — FMHA Kernel Development", "Kernel Output".
 *
 * fa_prefill_pack_v writes V (layout and strides as in fa_prefill_fwd) into
 * `workspace` as fp16 V^T tiles; nothing else is read or written.
 * fa_prefill_fwd_packed then takes the same arguments as fa_prefill_fwd minus
 * v and its strides, and reads V from a workspace that a completed or
 * earlier-enqueued fa_prefill_pack_v call filled for the same batch,
 * seqlen_kv, n_heads_kv and head_dim (dtype of q/k may differ from the packed
 * V's). The workspace is only read by fa_prefill_fwd_packed, so any number of
 * calls may share one packed workspace; a pack into it must not overlap them
 * in time. Using a workspace that was not filled this way gives unspecified
 * (finite or not) outputs but no out-of-bounds access. Validation and errors
 * as in fa_prefill_fwd; fa_prefill_pack_v checks only its own arguments.
 */
int fa_prefill_pack_v(const void* v, int64_t v_sb, int64_t v_ss, int64_t v_sh, int batch,
                      int seqlen_kv, int n_heads_kv, int head_dim, int dtype, void* workspace,
                      uint64_t workspace_bytes, void* stream);

int fa_prefill_fwd_packed(const void* q, int64_t q_sb, int64_t q_ss, int64_t q_sh,
                          const void* k, int64_t k_sb, int64_t k_ss, int64_t k_sh,
                          float* o, int64_t o_sb, int64_t o_ss, int64_t o_sh,
                          float* lse, float* row_sum,
                          int batch, int seqlen_q, int seqlen_kv, int n_heads_q, int n_heads_kv,
                          int head_dim, int dtype, int causal, float softmax_scale,
                          int out_unnormalized, const int32_t* kv_lens, int window,
                          const float* sink_logits, const void* workspace,
                          uint64_t workspace_bytes, void* stream);

/*
 * fa_prefill_fwd_packed_split — fa_prefill_fwd_packed with the key range of
 * the longest query blocks split over two work-groups.
 *
 * Source: as fa_prefill_fwd_packed; "66 · D2 ...", section 1 (splitting the
 * KV range of one query into parts whose partial results are merged, with
 * the partition a fixed function of the shape) and "STAGE_D.md ...", D5 and
 * D5c (partials carry an LSE and are merged inside the one launch).
 *
 * Same arguments, checks and results as fa_prefill_fwd_packed, plus
 * split_workspace: caller-owned device scratch of at least
 * fa_prefill_split_workspace_size(batch, seqlen_q, n_heads_q, head_dim)
 * bytes, 256-byte aligned, zero-filled before its first use. Its first 64
 * KiB hold the arrival counters (one per 128-row query block of every batch
 * entry and query head) at the same place for every shape, and every call
 * leaves the counters it uses at zero again, so one fill serves any number
 * of later calls, of any shapes the buffer is large enough for. The rest
 * holds partial results, written before they are read within each call.
 * Shapes with more than 16384 query blocks (batch * n_heads_q *
 * ceil(seqlen_q / 128)) run unsplit. Calls that overlap in time must not
 * share the buffer.
 *
 * Under causal masks (and windows) the 128-row query blocks see different
 * numbers of key tiles, and a launch cannot end before its longest block
 * does. The host plans, from the shape alone, which blocks to split
 * (fa_prefill_split_units): a split block's tiles go to two work-groups,
 * each stores its normalized partial O and LSE in split_workspace, and the
 * second to finish merges the two (max-shifted weights, first half always
 * the left operand), so results are the same bytes on every run. The
 * partition of the key range changes the float summation order: results
 * differ from fa_prefill_fwd_packed's within the same tolerances, not
 * bitwise. With out_unnormalized != 0, a row_sum output, head_dim 256 or
 * 512, or a shape the planner does not split, the call runs
 * fa_prefill_fwd_packed's kernel unchanged (split_workspace is then
 * checked but not touched).
 */
int fa_prefill_fwd_packed_split(const void* q, int64_t q_sb, int64_t q_ss, int64_t q_sh,
                                const void* k, int64_t k_sb, int64_t k_ss, int64_t k_sh,
                                float* o, int64_t o_sb, int64_t o_ss, int64_t o_sh,
                                float* lse, float* row_sum,
                                int batch, int seqlen_q, int seqlen_kv, int n_heads_q,
                                int n_heads_kv, int head_dim, int dtype, int causal,
                                float softmax_scale, int out_unnormalized, const int32_t* kv_lens,
                                int window, const float* sink_logits, const void* workspace,
                                uint64_t workspace_bytes, void* split_workspace,
                                uint64_t split_workspace_bytes, void* stream);

/*
 * fa_prefill_split_workspace_size — bytes of split_workspace
 * fa_prefill_fwd_packed_split needs: 64 KiB of arrival counters, then for
 * every 128-row query block of every (batch entry, query head) two halves of
 * partial results (128 x head_dim fp32 O and 128 fp32 LSE each), i.e. about
 * 65536 + 2 * batch * n_heads_q * ceil(seqlen_q / 128) * 128 * (head_dim + 1) * 4.
 * Returns 0 for non-positive sizes. Host only; never fails otherwise.
 */
uint64_t fa_prefill_split_workspace_size(int batch, int seqlen_q, int n_heads_q, int head_dim);

/*
 * fa_prefill_split_units — the work order fa_prefill_fwd_packed_split uses
 * for a shape (host only; for inspection and tests).
 *
 * Source: as fa_prefill_fwd_packed_split.
 *
 * The plan counts each query block's key tiles at full lengths (kv_lens are
 * device data; they change only the balance, never the results), models the
 * launch as list scheduling of work-groups, longest first, on two
 * work-groups per compute unit of 256 (a half costs 6 tile times beyond its
 * tiles: its own prologue, storing its partial and the merge), and picks
 * the split threshold that minimizes the modeled end time. A launch whose
 * unsplit end is modeled under 1.5x the average slot's work is not split
 * (a work-group alone on its compute unit runs faster than the model
 * assumes, so such tails cost less than the split), nor is a plan that
 * gains under 5 %. In practice: long prompts over few heads split, prompts
 * over many heads (or batches) do not.
 * Returns the number of units (0: the call runs unsplit) and writes up to
 * max_units of them to units (may be NULL), longest first; unit =
 * query block | kind << 14 with kind 0 = the whole block, 1 = the first
 * half of its key tiles (floor(n / 2) of n), 2 = the second half. Every block
 * appears either whole or as both halves. Returns -FA_ERR_INVALID_ARG (a
 * negative count) for non-positive sizes, bad head counts, window < 0 or
 * max_units < 0; head dims other than 64 and 128, and shapes with more than
 * 16384 query blocks (the arrival counters' capacity), get 0.
 */
int fa_prefill_split_units(int batch, int seqlen_q, int seqlen_kv, int n_heads_q, int n_heads_kv,
                           int head_dim, int causal, int window, uint16_t* units, int max_units);

/*
 * fa_prefill_trio — whether the attention launch of fa_prefill_fwd_packed
 * (and of fa_prefill_fwd where it repacks V: bf16 inputs) runs three
 * work-groups per compute unit for a shape (host only; for inspection and
 * tests). Results are the same attention either way, within rounding.
 *
 * Source: "60 · r57 — FA KV staging double buffering (REVERTED)", section 1
 * (the grid over query blocks and heads); "STAGE_D.md — FMHA Kernel
 * Development", D3/D4 (the sliding-window branch, whose blocks all see about
 * the same number of keys).
 *
 * The three-per-CU form (32-key tiles, no software pipeline; head_dim 128,
 * an odd number of query heads per KV head) is chosen when the grid's
 * 128-row blocks carry about equal numbers of key tiles (the longest at most
 * 1.25x the mean, counted at full lengths) and there are more blocks than
 * two per compute unit hold (512) but no more than three do (768).
 * Returns 1 (three per CU) or 0 (two); -FA_ERR_INVALID_ARG for
 * non-positive sizes, bad head counts or window < 0.
 */
int fa_prefill_trio(int batch, int seqlen_q, int seqlen_kv, int n_heads_q, int n_heads_kv,
                    int head_dim, int causal, int window);

/*
 * fa_attn_merge — merge two attention passes over disjoint key sets, and an
 * optional per-head sink, through their LSEs.
 *
 * Source: "STAGE_D.md — FMHA Kernel Development", D5 (a sliding-window pass
 * and a sink merged by LSE; D5b does it after the kernels, as here). The
 * formula is not printed on the pages; the max-shifted form is used, with the
 * sink as a pass whose O is 0 and whose LSE is sink_logits[h]:
 *   M = max(lse_a, lse_b, sink), w_x = exp(lse_x - M),
 *   o = (w_a o_a + w_b o_b) / (w_a + w_b + w_sink), lse = M + ln(w_a + w_b + w_sink);
 * rows where every term is -inf get o = 0, lse = -inf. For passes over
 * disjoint key sets this is the attention over their union.
 *
 * Layouts (fp32, element strides, head_dim contiguous): o_a, o_b, o
 * [batch, seqlen, n_heads, head_dim] (16-byte aligned, strides multiples of
 * 4); lse_a, lse_b, lse [batch, n_heads, seqlen] contiguous (the layout
 * fa_prefill_fwd writes; decode outputs are the case seqlen = 1);
 * sink_logits [n_heads]. o_b and lse_b may both be NULL (one pass, e.g. with
 * a sink), sink_logits may be NULL. o may be o_a and lse may be lse_a (in
 * place); no other overlap is allowed. All device memory.
 */
int fa_attn_merge(const float* o_a, int64_t oa_sb, int64_t oa_ss, int64_t oa_sh,
                  const float* lse_a, const float* o_b, int64_t ob_sb, int64_t ob_ss,
                  int64_t ob_sh, const float* lse_b, const float* sink_logits, int batch,
                  int seqlen, int n_heads, int head_dim, float* o, int64_t o_sb, int64_t o_ss,
                  int64_t o_sh, float* lse, void* stream);

/*
 * fa_prefill_workspace_size — bytes of workspace fa_prefill_fwd needs
 * (batch * n_heads_kv * ceil(seqlen_kv / T) * head_dim * T * 2, with tiles of
 * T = 64 keys, 32 at head_dim 256 and 512). Returns 0 for non-positive sizes. Host
 * only; never fails otherwise.
 */
uint64_t fa_prefill_workspace_size(int batch, int seqlen_kv, int n_heads_kv, int head_dim);

/*
 * fa_decode_plan — deterministic split plan for split-KV decode (host only).
 *
 * Source: "66 · D2: explicit K+V register staging (LANDED, +2.0% @1641) and
 * the cp.async negative result", section 1 (decode splits the KV length into
 * ranges; the split count is part of the float summation order, so it must
 * be a fixed function of the shape).
 *
 * kv_lens_host: HOST array [batch] of sequence lengths (each >= 1). Chooses
 * split_len (keys per split, a whole number of the partial kernel's row
 * blocks, so a multiple of 16) to minimize a cost model of the partial and
 * merge kernels: the work items (sequence, group of query heads, split) run
 * in rounds of num_cus * (resident waves per CU), and each round lasts as long
 * as its longest split. max_splits_out = ceil(max(kv_lens) / split_len). The
 * result is a pure function of the arguments (lengths beyond 4096 row blocks
 * are planned over a thinned set of about 4096 candidate split lengths).
 * Returns FA_ERR_INVALID_ARG for null pointers, lengths < 1 or bad head
 * counts, FA_ERR_UNSUPPORTED for an unsupported head_dim or a length above
 * 2^30 tokens.
 */
int fa_decode_plan(const int32_t* kv_lens_host, int batch, int n_heads_q, int n_heads_kv,
                   int head_dim, int num_cus, int* split_len_out, int* max_splits_out);

/*
 * fa_decode_split_partial — per-split partial attention for one query token.
 *
 * Source: "66 · D2 ...", sections 1 and 3.2 (each split [lo, hi) runs the
 * online softmax over its KV rows with the K and V row loads issued ahead of
 * the softmax dependency chain) and "STAGE_D.md ...", section D5 (partials
 * carry an LSE so they can be merged).
 *
 * Layouts:
 *   q        [batch, n_heads_q, head_dim] half, strides q_sb, q_sh
 *   k_cache, v_cache: packed token-major caches; token t of sequence b, KV
 *            head hk, element d at ((kv_offsets[b] + t) * kv_stride_tok +
 *            hk * kv_stride_head + d)
 *   kv_offsets [batch] int64, kv_lens [batch] int32 (device arrays, each
 *            length >= 1)
 *   part_o   [batch, n_heads_q, max_splits, head_dim] fp32, contiguous
 *   part_lse [batch, n_heads_q, max_splits] fp32, contiguous
 *
 * Split s of sequence b covers keys [s*split_len, min(L_b, (s+1)*split_len));
 * for s < ceil(L_b / split_len) it writes the normalized partial output O_s
 * and its natural-log LSE_s. Splits at or past ceil(L_b / split_len) are
 * empty: they are neither read nor written (their contents stay undefined).
 * The caller guarantees ceil(L_b / split_len) <= max_splits (the merge writes
 * NaN for any sequence that breaks this, and for L_b < 1).
 *
 * Supported set: head_dim in {64, 128, 256}; dtype FA_F16 or FA_BF16;
 * n_heads_q % n_heads_kv == 0; split_len a positive multiple of 16;
 * max_splits >= 1; pointers to half data 16-byte aligned, strides multiples
 * of 8.
 */
int fa_decode_split_partial(const void* q, int64_t q_sb, int64_t q_sh,
                            const void* k_cache, const void* v_cache,
                            int64_t kv_stride_tok, int64_t kv_stride_head,
                            const int64_t* kv_offsets, const int32_t* kv_lens,
                            int batch, int n_heads_q, int n_heads_kv, int head_dim, int dtype,
                            float softmax_scale, int split_len, int max_splits,
                            float* part_o, float* part_lse, void* stream);

/*
 * fa_decode_merge_lse — merge split partials into the decode output.
 *
 * Source: "STAGE_D.md ...", section D5 (merging attention passes through
 * their LSE) and "66 · D2 ...", section 5.2 (the combine step after the split
 * partials). The merge formula is not printed on the pages; the max-shifted
 * form is used: M = max_s LSE_s, w_s = exp(LSE_s - M),
 * O = sum_s w_s O_s / sum_s w_s, LSE = M + ln(sum_s w_s).
 *
 * Reads only the first ceil(L_b / split_len) partials of sequence b.
 * Layouts: part_o/part_lse as written by fa_decode_split_partial; o [batch,
 * n_heads_q, head_dim] fp32 contiguous; lse [batch, n_heads_q] fp32. A
 * sequence with L_b < 1 or ceil(L_b / split_len) > max_splits gets NaN in o
 * and lse.
 */
int fa_decode_merge_lse(const float* part_o, const float* part_lse, const int32_t* kv_lens,
                        int batch, int n_heads_q, int head_dim, int split_len, int max_splits,
                        float* o, float* lse, void* stream);

/*
 * fa_decode_fused — split-KV decode in one launch (partials and their merge).
 *
 * Source: as fa_decode_split_partial and fa_decode_merge_lse; "STAGE_D.md —
 * FMHA Kernel Development", D5c (fuse the passes into one kernel launch).
 *
 * Computes what fa_decode_split_partial followed by fa_decode_merge_lse
 * computes (same arguments, same split partition, o and lse as written by the
 * merge), in one kernel: each work-group of W = fa_decode_fused_waves(batch,
 * n_heads_q, n_heads_kv, head_dim, max_splits) waves (4 when the call has more
 * than 16 splits and fits in one round of resident waves, else 1)
 * takes W consecutive splits of one sequence and merges them on chip; when
 * one work-group covers every split of a sequence its merge is the output,
 * otherwise the last work-group of the sequence to finish merges the
 * work-group partials (in index order, so the result is a fixed function of
 * split_len and max_splits and repeated runs are byte-identical; the summation
 * order differs from the two-launch form, which agrees to rounding).
 *
 * workspace: caller-owned device memory of at least
 * fa_decode_fused_workspace_size(batch, n_heads_q, n_heads_kv, head_dim,
 * max_splits) bytes, 256-byte aligned, ZERO-FILLED before its first use. Its
 * first 64 KiB hold arrival counters (one per sequence and group of query
 * heads served together, at most 16384 per call: larger batches return
 * FA_ERR_UNSUPPORTED) and every call returns them to zero when it completes,
 * so one workspace serves any sequence of calls, of any shapes it is large
 * enough for. Calls that overlap in time must not share a workspace. A
 * sequence with
 * L_b < 1 or ceil(L_b / split_len) > max_splits gets NaN in o and lse.
 * Validation and supported set as in fa_decode_split_partial.
 */
int fa_decode_fused(const void* q, int64_t q_sb, int64_t q_sh,
                    const void* k_cache, const void* v_cache,
                    int64_t kv_stride_tok, int64_t kv_stride_head,
                    const int64_t* kv_offsets, const int32_t* kv_lens,
                    int batch, int n_heads_q, int n_heads_kv, int head_dim, int dtype,
                    float softmax_scale, int split_len, int max_splits,
                    float* o, float* lse, void* workspace, uint64_t workspace_bytes,
                    void* stream);

/*
 * fa_decode_fused_noalloc — fa_decode_fused without a caller workspace.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments (minus the workspace), checks, kernels and results as
 * fa_decode_fused: the bytes of o and lse equal those fa_decode_fused
 * writes for the same call. The scratch (arrival counters and work-group
 * partials) is a library-owned static device array of
 * FA_DECODE_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, held until the process
 * ends; the call allocates and frees nothing. The first call on a device
 * looks up that device's copy and enqueues one small kernel on `stream` that
 * clears its 64 KiB of counters; every call leaves them at zero again.
 * Shapes whose fa_decode_fused_workspace_size exceeds the array return
 * FA_ERR_UNSUPPORTED (use fa_decode_fused with a caller workspace). All calls
 * on one GPU share its array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must not be issued.
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)
int fa_decode_fused_noalloc(const void* q, int64_t q_sb, int64_t q_sh,
                            const void* k_cache, const void* v_cache,
                            int64_t kv_stride_tok, int64_t kv_stride_head,
                            const int64_t* kv_offsets, const int32_t* kv_lens,
                            int batch, int n_heads_q, int n_heads_kv, int head_dim, int dtype,
                            float softmax_scale, int split_len, int max_splits,
                            float* o, float* lse, void* stream);

/*
 * fa_decode_fused_workspace_size — bytes of workspace fa_decode_fused needs
 * (0 for invalid sizes). fa_decode_fused_waves — splits one work-group of
 * fa_decode_fused merges on chip (0 for invalid sizes). Host only.
 */
uint64_t fa_decode_fused_workspace_size(int batch, int n_heads_q, int n_heads_kv, int head_dim,
                                        int max_splits);
int fa_decode_fused_waves(int batch, int n_heads_q, int n_heads_kv, int head_dim,
                          int max_splits);

/* Static text for a status code. */
const char* fa_status_string(int status);

/* Detail for the last non-OK return on the calling thread ("" if none). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
