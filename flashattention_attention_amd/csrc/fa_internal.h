// Internal declarations shared by the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Byte counts of workspaces: products and sums that saturate at SIZE_MAX
// instead of wrapping, so an absurd shape can never be given a small size.
inline size_t sat_mul(size_t a, size_t b) {
  size_t r;
  return __builtin_mul_overflow(a, b, &r) ? SIZE_MAX : r;
}
inline size_t sat_add(size_t a, size_t b) {
  size_t r;
  return __builtin_add_overflow(a, b, &r) ? SIZE_MAX : r;
}
inline size_t sat_up256(size_t x) { return x > SIZE_MAX - 255 ? SIZE_MAX : (x + 255) & ~(size_t)255; }

// Arguments of one prefill launch (element strides; head_dim stride is 1).
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  float* row_sum;  // may be null in normalized mode
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int batch, seqlen_q, seqlen_kv, n_heads_q, n_heads_kv;
  int causal;
  float scale_log2;        // softmax_scale * log2(e)
  const int32_t* kv_lens;  // device [batch] valid KV length per sequence, or null
  int window;              // > 0: key j visible only if j > q_pos - window
  const float* sink_logits;  // device [n_heads_q] per-head sink logit, or null
  int wg_serial;           // serial work-group order: work-group slots per XCD (0 = off; set by the launcher)
  int wg_rot;              // second round of first-dispatched work-groups rotated (reversed in the serial order): compute units per XCD (0 = off; set by the launcher)
  int unnorm;              // un-normalized O (set by the launcher)
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int64_t* kv_offsets;
  const int32_t* kv_lens;
  float* part_o;
  float* part_lse;
  int64_t q_sb, q_sh;
  int64_t kv_st, kv_sh;
  int batch, n_heads_q, n_heads_kv;
  int split_len, max_splits;
  float scale_log2;
  // single-launch form only
  float* o;          // [batch, n_heads_q, head_dim]
  float* lse;        // [batch, n_heads_q]
  int* counters;     // [batch, n_heads_q / heads_per_wave], zero between calls
  float* wg_o;       // [batch, n_heads_q, max_wg, head_dim]
  float* wg_lse;     // [batch, n_heads_q, max_wg]
  int max_wg;        // work-groups per (sequence, head group)
};

// Merge of two attention passes (and an optional per-head sink) by LSE.
struct BranchMergeArgs {
  const float* o_a;
  const float* lse_a;
  const float* o_b;          // may be null (no second pass)
  const float* lse_b;
  const float* sink_logits;  // may be null
  float* o;
  float* lse;
  int64_t oa_sb, oa_ss, oa_sh, ob_sb, ob_ss, ob_sh, o_sb, o_ss, o_sh;
  int batch, seqlen, n_heads;
};

struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  const int32_t* kv_lens;
  float* o;
  float* lse;
  int batch, n_heads_q, split_len, max_splits;
};

// Caller-provided scratch for the prefill: fp16 V^T tiles.
struct VtArgs {
  void* ws;
  size_t bytes;
};

// Bytes of prefill workspace needed for these sizes.
size_t prefill_workspace_bytes(int batch, int seqlen_kv, int n_heads_kv, int head_dim);

// Key split of the longest query blocks of a prefill (normalized output, head
// dim 64 or 128): the order in which a launch hands out its work units, and
// the caller's scratch for the halves' partial results. A unit is a whole
// 128-row query block or one half of a split block's key tiles; unit entry =
// query block | kind << 14 (kind 0: whole block, 1: first half, 2: second).
constexpr int kMaxSplitUnits = 512;
// The arrival counters sit in a fixed region at the start of the split
// scratch, the same region for every shape: a scratch zero-filled once then
// serves calls of any shape (each call leaves its counters at zero), and one
// call's partial results never land on another shape's counters. A shape
// with more query blocks than counters runs unsplit.
constexpr size_t kSplitCounterBytes = 65536;
constexpr int64_t kSplitCounters = (int64_t)(kSplitCounterBytes / 4);
struct SplitPlan {
  int* cnt;      // [batch * n_heads_q * nqb] arrival counters (fixed region), zero between calls
  float* o;      // [batch * n_heads_q * nqb][2 halves][128 rows * head_dim] partial O
  float* lse;    // [batch * n_heads_q * nqb][2 halves][128 rows] partial LSE (log2 units)
  int n_units;   // 0: no split (one work-group per block, longest first)
  unsigned short units[kMaxSplitUnits];   // longest unit first
};
// Scratch bytes of the split for these sizes, and the offsets of its parts.
struct SplitLayout {
  size_t cnt, lse, o, total;
};
SplitLayout prefill_split_layout(int batch, int seqlen_q, int n_heads_q, int head_dim);
// The work order for one call's shape (kv_lens are not known on the host: full
// lengths are assumed, which affects only the balance). Returns the unit count
// (0: the call runs unsplit) and fills units[0 .. count).
int prefill_split_units(int batch, int seqlen_q, int seqlen_kv, int n_heads_q, int n_heads_kv,
                        int head_dim, int causal, int window, unsigned short* units);

// Launchers: enqueue on `stream`, return the launch's hipError_t.
// Prefill in two launches: V -> fp16 V^T tiles in the workspace (uses a.v and
// its strides), then attention reading the V^T tiles from the workspace.
hipError_t launch_prefill_pack(const PrefillArgs& a, const VtArgs& w, int head_dim, bool bf16,
                               hipStream_t stream);
hipError_t launch_prefill_attn(const PrefillArgs& a, const VtArgs& w, int head_dim, bool bf16,
                               bool unnormalized, hipStream_t stream);
// One launch reading V's rows directly (no V^T workspace): fp16 inputs at
// head_dim 64 or 128, where prefill_reads_v_rows is true.
bool prefill_reads_v_rows(int head_dim, bool bf16);
// Whether the attention launch of the two-launch prefill runs three work-groups
// per compute unit (32-key tiles) for this shape instead of two.
bool prefill_trio(int batch, int seqlen_q, int seqlen_kv, int n_heads_q, int n_heads_kv,
                  int head_dim, int causal, int window);
hipError_t launch_prefill_attn_vrow(const PrefillArgs& a, int head_dim, bool unnormalized,
                                    hipStream_t stream);
// The same with the key split (sp.n_units > 0); head_dim 64 or 128, normalized output.
hipError_t launch_prefill_attn_split(const PrefillArgs& a, const VtArgs& w, const SplitPlan& sp,
                                     int head_dim, bool bf16, hipStream_t stream);
hipError_t launch_decode_partial(const DecodeArgs& a, int head_dim, bool bf16,
                                 hipStream_t stream);
hipError_t launch_decode_merge(const MergeArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_decode_fused(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t stream);
hipError_t launch_branch_merge(const BranchMergeArgs& a, int head_dim, hipStream_t stream);

// Library-owned scratch of the single-launch decode for callers that cannot
// allocate (one static array per GPU; see fa_decode_fused_noalloc in fa.h).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
// Device address of the current device's scratch; the first call on a device
// looks it up and clears its counter region with a kernel on `stream`.
hipError_t decode_noalloc_scratch(void** out, hipStream_t stream);

// Splits (one per wave) merged inside one work-group of the single-launch decode.
int decode_fused_waves(int batch, int n_heads_q, int n_heads_kv, int head_dim, int max_splits);
// Workspace of the single-launch decode, and the offsets of its parts.
constexpr size_t kFusedCounterBytes = 65536;   // room for 16384 arrival counters
struct FusedLayout {
  size_t counters, wg_lse, wg_o, total;
  int64_t n_counters;
  int waves, max_wg;
};
FusedLayout decode_fused_layout(int batch, int n_heads_q, int n_heads_kv, int head_dim,
                                int max_splits);

// Geometry of the decode partial kernel, for the split planner. Heads per wave
// depend on the shape (see the definition); the planner steps split lengths in
// blocks of the widest choice.
constexpr int kDecodeCus = 256;   // compute units of the target GPU
int decode_max_heads_per_wave(int group);
int decode_heads_per_wave(int group, int batch, int n_heads_q, int head_dim, int max_splits);
int decode_block_rows(int head_dim, int heads_per_wave);
int decode_waves_per_cu(int head_dim);

}  // namespace fa
