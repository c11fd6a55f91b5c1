// Merge of two attention passes over disjoint key sets, and of a per-head
// sink logit, through their LSEs ("STAGE_D.md — FMHA Kernel Development",
// D5: a sliding-window pass and a sink combined after the fact).
//
// Pass results are normalized outputs O_x with natural-log LSE_x. The sink
// sigma_h is a pass with O = 0 and LSE = sigma_h. Per row, with
// M = max(LSE_a, LSE_b, sigma_h) and w_x = exp(LSE_x - M):
//   O = (w_a O_a + w_b O_b) / (w_a + w_b + w_sink),  LSE = M + ln(w_a + w_b + w_sink),
// and a row where every term is -inf gets O = 0, LSE = -inf.
//
// Pure streaming work: each output element reads two input elements once,
// so the kernel is bound by HBM bandwidth. One thread owns 4 consecutive
// elements of one row (a 16-byte load per input and a 16-byte store); rows
// are enumerated in the [batch, seq, head] order of the O layout so that the
// threads of a wave cover whole contiguous rows. Each thread reads every input
// of its elements before writing them, so o may alias o_a (and lse lse_a).
#include "fa_internal.h"

namespace fa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ void __launch_bounds__(256)
branch_merge_kernel(BranchMergeArgs a) {
  constexpr int C = D / 4;                       // 16-byte chunks per row
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)a.batch * a.seqlen * a.n_heads;
  if (t >= rows * C) return;
  const int c = (int)(t % C);
  const int64_t r = t / C;                       // ((b * seqlen + s) * n_heads + h)
  const int h = (int)(r % a.n_heads);
  const int64_t bs = r / a.n_heads;
  const int s = (int)(bs % a.seqlen);
  const int b = (int)(bs / a.seqlen);
  const int64_t li = ((int64_t)b * a.n_heads + h) * a.seqlen + s;   // [batch, head, seq]

  const float la = a.lse_a[li];
  const float lb = a.lse_b ? a.lse_b[li] : -INFINITY;
  const float ls = a.sink_logits ? a.sink_logits[h] : -INFINITY;
  const f32x4 oa = *(const f32x4*)(a.o_a + b * a.oa_sb + s * a.oa_ss + h * a.oa_sh + c * 4);
  f32x4 ob = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (a.o_b) ob = *(const f32x4*)(a.o_b + b * a.ob_sb + s * a.ob_ss + h * a.ob_sh + c * 4);

  const float M = fmaxf(fmaxf(la, lb), ls);
  f32x4 out = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float lse = -INFINITY;
  if (M != -INFINITY) {
    const float wa = __expf(la - M), wb = __expf(lb - M), ws = __expf(ls - M);
    const float W = wa + wb + ws;
    const float inv = 1.0f / W;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = (wa * oa[e] + wb * ob[e]) * inv;
    lse = M + __logf(W);
  }
  *(f32x4*)(a.o + b * a.o_sb + s * a.o_ss + h * a.o_sh + c * 4) = out;
  if (c == 0) a.lse[li] = lse;
}

}  // namespace

hipError_t launch_branch_merge(const BranchMergeArgs& a, int head_dim, hipStream_t stream) {
  const int64_t threads = (int64_t)a.batch * a.seqlen * a.n_heads * (head_dim / 4);
  const dim3 grid((unsigned)((threads + 255) / 256));
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((branch_merge_kernel<64>), grid, dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((branch_merge_kernel<128>), grid, dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL((branch_merge_kernel<256>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fa
