// Split-KV decode for gfx950: per-split partial attention and the LSE merge.
//
// Decode reads every K and V row once and does ~4 FLOP per byte, so it is
// bound by HBM bandwidth, not by the matrix cores. The partial kernel is
// therefore plain VALU work arranged for bandwidth:
//
//  * one wave per (sequence, group of query heads sharing a KV head, split);
//    the wave serves all query heads of the group, so each K/V row is read
//    once for the whole group (the head packing of "STAGE_D.md — FMHA Kernel
//    Development", section D2);
//  * a K or V row is spread over 16 lanes (8 lanes at head_dim 64) with 16
//    contiguous bytes per lane, so one load instruction moves 4 whole rows
//    (1 KB) per wave, fully coalesced;
//  * rows are processed in blocks; the loads for block i+1 are issued before
//    the softmax chain of block i runs, so their latency hides under it (the
//    early-issued K and V loads of "66 · D2: explicit K+V register staging
//    (LANDED, +2.0% @1641) and the cp.async negative result", section 2.2);
//  * dot products use v_dot2 over packed halves, lane partial sums are
//    reduced with DPP row permutes, and the online-softmax update is done
//    once per block and head (section 3.2 of the same page gives the per-row
//    form: new max, correction factor, exponential, running sum and output).
//
// Each split emits a normalized partial O_s and its natural-log LSE_s. The
// merge then combines the partials by LSE in a fixed order, so the result is
// deterministic for a given split plan.
#include "fa_internal.h"

namespace fa {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kSlack = 8.0f;   // stale-max tolerance (log2 units)
constexpr float kLn2 = 0.693147180559945309f;

// DPP controls (gfx9 encoding).
constexpr int kQuadXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;    // lane i <- 7-i within each 8
constexpr int kRowMirror = 0x140;        // lane i <- 15-i within each 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over groups of LPK consecutive lanes (LPK = 8 or 16); every lane of the
// group ends with the same bits (each step adds a symmetric pair).
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowHalfMirror>(x);
  if constexpr (LPK == 16) x += dpp<kRowMirror>(x);
  return x;
}

template <bool BF16>
__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
  if constexpr (BF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                  false);
}

template <bool BF16>
__device__ __forceinline__ float half_lo(unsigned w) {
  if constexpr (BF16) return __uint_as_float(w << 16);
  else return (float)__builtin_bit_cast(f16x2, w)[0];
}
template <bool BF16>
__device__ __forceinline__ float half_hi(unsigned w) {
  if constexpr (BF16) return __uint_as_float(w & 0xffff0000u);
  else return (float)__builtin_bit_cast(f16x2, w)[1];
}

// D: head_dim. G: query heads served per wave (a divisor of the GQA group).
template <int D, int G, bool BF16>
__global__ void __launch_bounds__(64)
decode_partial_kernel(DecodeArgs a) {
  constexpr int LPK = D >= 128 ? 16 : 8;   // lanes per K/V row
  constexpr int EPL = D / LPK;             // elements per lane: 8 or 16
  constexpr int W = EPL / 8;               // 16-byte loads per row per lane
  constexpr int KPS = 64 / LPK;            // rows per load step: 4 or 8
  // load steps per block: 16 KB of K+V per block, halved when the wave serves
  // more than 4 heads (their accumulators need the registers)
  constexpr int NB = D == 256 ? (G > 4 ? 2 : 4) : (G > 4 ? 4 : 8);
  constexpr int BK = KPS * NB;             // rows per block

  const int lane = threadIdx.x;
  const int h0 = blockIdx.x * G;   // head groups fastest: the waves reading the
  const int s = blockIdx.y;        // same tokens' rows are dispatched together
  const int b = blockIdx.z;
  const int hk = h0 / (a.n_heads_q / a.n_heads_kv);
  const int L = a.kv_lens[b];
  const int lo = s * a.split_len;
  if (L < 1 || lo >= L) return;          // empty split: nothing read or written
  const int hi = min(L, lo + a.split_len);
  const int slot = lane / LPK;           // which of the KPS rows of a step
  const int c = lane % LPK;              // which EPL-element chunk of the row

  u32x4 qv[G][W];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const unsigned short* qp = (const unsigned short*)a.q + (int64_t)b * a.q_sb +
                               (int64_t)(h0 + g) * a.q_sh + c * EPL;
#pragma unroll
    for (int w = 0; w < W; ++w) qv[g][w] = *(const u32x4*)(qp + w * 8);
  }

  const int64_t row0 = a.kv_offsets[b];
  const unsigned short* kbase =
      (const unsigned short*)a.k + row0 * a.kv_st + (int64_t)hk * a.kv_sh + c * EPL;
  const unsigned short* vbase =
      (const unsigned short*)a.v + row0 * a.kv_st + (int64_t)hk * a.kv_sh + c * EPL;

  // Load one block of rows. Rows past hi repeat row hi-1 (always valid
  // memory); their scores are masked to -inf, so they contribute exactly 0.
  auto load_block = [&](int start, u32x4 (&kd)[NB][W], u32x4 (&vd)[NB][W]) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int64_t key = min(start + j * KPS + slot, hi - 1);
#pragma unroll
      for (int w = 0; w < W; ++w) {
        kd[j][w] = __builtin_nontemporal_load((const u32x4*)(kbase + key * a.kv_st + w * 8));
        vd[j][w] = __builtin_nontemporal_load((const u32x4*)(vbase + key * a.kv_st + w * 8));
      }
    }
  };

  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -1e30f;
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[g][e] = 0.0f;
  }

  auto compute_block = [&](int start, const u32x4 (&kr)[NB][W], const u32x4 (&vr)[NB][W]) {
    // Scores (log2 units) of this lane's rows, one per step and head.
    float sc[NB][G];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const bool ok = start + j * KPS + slot < hi;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w)
#pragma unroll
          for (int e = 0; e < 4; ++e) d = dot2<BF16>(qv[g][w][e], kr[j][w][e], d);
        d = group_sum<LPK>(d);
        sc[j][g] = ok ? d * a.scale_log2 : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      // Block max over the NB*KPS rows: in-lane over the steps, then across the
      // row slots (values are identical inside a slot, so one lane per slot).
      float lm = sc[0][g];
#pragma unroll
      for (int j = 1; j < NB; ++j) lm = fmaxf(lm, sc[j][g]);
      float bm = -INFINITY;
#pragma unroll
      for (int r = 0; r < KPS; ++r)
        bm = fmaxf(bm, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lm), r * LPK)));
      if (bm > m[g] + kSlack) {
        const float corr = __builtin_amdgcn_exp2f(m[g] - bm);
        m[g] = bm;
        l[g] *= corr;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] *= corr;
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const float p = __builtin_amdgcn_exp2f(sc[j][g] - m[g]);
        l[g] += p;
#pragma unroll
        for (int w = 0; w < W; ++w)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[g][w * 8 + 2 * e] = __builtin_fmaf(p, half_lo<BF16>(vr[j][w][e]),
                                                 o[g][w * 8 + 2 * e]);
            o[g][w * 8 + 2 * e + 1] = __builtin_fmaf(p, half_hi<BF16>(vr[j][w][e]),
                                                     o[g][w * 8 + 2 * e + 1]);
          }
      }
    }
  };

  // Two register buffers in turn: while one block is computed the next one is
  // in flight (the loop is unrolled by two so no buffer is ever copied).
  u32x4 ka[NB][W], va[NB][W], kb[NB][W], vb[NB][W];
  load_block(lo, ka, va);
  for (int start = lo; start < hi; start += 2 * BK) {
    if (start + BK < hi) load_block(start + BK, kb, vb);
    compute_block(start, ka, va);
    if (start + BK >= hi) break;
    if (start + 2 * BK < hi) load_block(start + 2 * BK, ka, va);
    compute_block(start + BK, kb, vb);
  }

  // Sum the row slots (m is the same in every lane), then write the partial.
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int x = LPK; x < 64; x *= 2) {
      l[g] += __shfl_xor(l[g], x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] += __shfl_xor(o[g][e], x);
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t pi = ((int64_t)b * a.n_heads_q + h0 + g) * a.max_splits + s;
      float* po = a.part_o + pi * D + c * EPL;
      const float inv = 1.0f / l[g];
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *(f32x4*)(po + e) = f32x4{o[g][e] * inv, o[g][e + 1] * inv, o[g][e + 2] * inv,
                                  o[g][e + 3] * inv};
      if (c == 0) a.part_lse[pi] = (m[g] + __log2f(l[g])) * kLn2;
    }
  }
}

// One wave per (sequence, query head). Split LSEs are read lane-parallel and
// reduced across the wave; the weighted sum of the split outputs runs over
// the splits in index order with the loads of several splits in flight.
template <int D>
__global__ void __launch_bounds__(64)
decode_merge_kernel(MergeArgs a) {
  constexpr int EPL = D / 64;
  constexpr int U = 32;                    // splits in flight per step
  const int lane = threadIdx.x;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t bh = (int64_t)b * a.n_heads_q + h;
  float* out = a.o + bh * D;
  const int L = a.kv_lens[b];
  const int ns = L < 1 ? 0 : (L + a.split_len - 1) / a.split_len;
  if (ns < 1 || ns > a.max_splits) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[lane * EPL + e] = __builtin_nanf("");
    if (lane == 0) a.lse[bh] = __builtin_nanf("");
    return;
  }
  const float* pl = a.part_lse + bh * a.max_splits;
  const float* po = a.part_o + bh * a.max_splits * D + lane * EPL;

  float M = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += 64)
    if (s0 + lane < ns) M = fmaxf(M, pl[s0 + lane]);
#pragma unroll
  for (int x = 1; x < 64; x *= 2) M = fmaxf(M, __shfl_xor(M, x));

  float wsum = 0.0f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const float wl = s0 + lane < ns ? __expf(pl[s0 + lane] - M) : 0.0f;
    wsum += wl;
    const int n = min(64, ns - s0);
    for (int j = 0; j < n; j += U) {
      float v[U][EPL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int sj = s0 + min(j + u, n - 1);
#pragma unroll
        for (int e = 0; e < EPL; ++e) v[u][e] = po[(int64_t)sj * D + e];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (j + u < n) {
          const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j + u));
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(w, v[u][e], acc[e]);
        }
      }
    }
  }
#pragma unroll
  for (int x = 1; x < 64; x *= 2) wsum += __shfl_xor(wsum, x);
  const float inv = 1.0f / wsum;
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[lane * EPL + e] = acc[e] * inv;
  if (lane == 0) a.lse[bh] = M + __logf(wsum);
}

template <int D, bool BF16>
hipError_t launch_partial_d(const DecodeArgs& a, int g, hipStream_t stream) {
  const dim3 grid(a.n_heads_q / g, a.max_splits, a.batch);
  switch (g) {
#define FA_CASE(G) \
  case G: hipLaunchKernelGGL((decode_partial_kernel<D, G, BF16>), grid, dim3(64), 0, stream, a); break;
    FA_CASE(1) FA_CASE(2) FA_CASE(3) FA_CASE(4) FA_CASE(5) FA_CASE(6) FA_CASE(7) FA_CASE(8)
#undef FA_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// Heads served per wave: the largest divisor of the GQA group that is <= 8.
int decode_heads_per_wave(int group) {
  for (int g = 8; g >= 1; --g)
    if (group % g == 0) return g;
  return 1;
}

// Rows per block of the partial kernel and resident waves per compute unit
// (from its register use: 2 waves per SIMD below head_dim 256, else 1).
int decode_block_rows(int head_dim, int g) {
  const int kps = head_dim >= 128 ? 4 : 8;
  const int nb = head_dim == 256 ? (g > 4 ? 2 : 4) : (g > 4 ? 4 : 8);
  return kps * nb;
}
int decode_waves_per_cu(int head_dim) { return head_dim == 256 ? 4 : 8; }

hipError_t launch_decode_partial(const DecodeArgs& a, int head_dim, bool bf16,
                                 hipStream_t stream) {
  const int g = decode_heads_per_wave(a.n_heads_q / a.n_heads_kv);
  switch (head_dim) {
    case 64: return bf16 ? launch_partial_d<64, true>(a, g, stream)
                         : launch_partial_d<64, false>(a, g, stream);
    case 128: return bf16 ? launch_partial_d<128, true>(a, g, stream)
                          : launch_partial_d<128, false>(a, g, stream);
    case 256: return bf16 ? launch_partial_d<256, true>(a, g, stream)
                          : launch_partial_d<256, false>(a, g, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_merge(const MergeArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid(a.n_heads_q, a.batch);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((decode_merge_kernel<64>), grid, dim3(64), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((decode_merge_kernel<128>), grid, dim3(64), 0, stream, a); break;
    case 256: hipLaunchKernelGGL((decode_merge_kernel<256>), grid, dim3(64), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fa
