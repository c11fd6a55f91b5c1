// Causal / unmasked GQA attention forward (prefill) for gfx950.
//
// One workgroup = 4 waves = 128 query rows of one (batch, query head); the
// workgroup streams the K/V tiles of its KV head up to the causal bound and
// keeps an online softmax per row.
//
// Mapping to the CDNA4 matrix cores (v_mfma_f32_32x32x16_{bf16,f16}): every
// wave owns 32 query rows and computes the TRANSPOSED score tile
// S^T = K . Q^T, so the 32 queries run along the MFMA N dimension (one query
// per lane column) and keys along M. With that orientation each lane holds
// 16 keys of a single query row, so the row max and row sum are in-lane
// reductions plus one exchange between the two 32-lane halves, and the
// output O^T = V^T . P^T keeps one query per lane column as well, so the
// per-row rescale is a per-lane scalar. P never leaves registers: the S^T
// accumulator layout is reused as the B operand of the P.V contraction, with
// the V^T A operand read from LDS in the matching key order.
//
// Tiling follows "60 · r57 — FA KV staging double buffering (REVERTED)",
// sections 1 and 2.2 (grid over query block and head; KV tiles streamed to
// the causal bound; tail rows zero-filled), with the softmax in registers of
// its section 1 and the tile-end rescale of its section 2.3. K/V for tile t+1
// are fetched into registers while tile t is computed (the overlap its
// section 2.4 aims for), then written to LDS between two barriers.
//
// Numerics:
//  * scores accumulate in fp32 from exact half products; the softmax scale
//    is applied to the fp32 scores (never folded into a half Q);
//  * exponentials are base 2 on scores pre-multiplied by scale*log2(e);
//  * P enters the P.V contraction as fp16 (round-to-nearest-even), V as fp16
//    (bf16 V is converted; exact for magnitudes in fp16's normal range); a
//    2^7 headroom factor keeps small P values out of fp16's subnormal range
//    and cancels in O / l;
//  * the running max is only moved (and O, l rescaled) once a tile max
//    exceeds it by more than 2^8 — an exact identity, since O and l share
//    the base — and outputs are referred back to the true row max;
//  * the row sum l accumulates the fp32 P values.
#include "fa_internal.h"

#include <limits.h>

namespace fa {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;          // query rows per workgroup
constexpr float kShift = 7.0f;            // log2 of the fp16 headroom factor on P
constexpr float kSlack = 8.0f;            // stale-max tolerance (log2 units)
constexpr float kLn2 = 0.693147180559945309f;

template <bool BF16>
__device__ __forceinline__ f32x16 mfma_qk(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

__device__ __forceinline__ f32x16 mfma_pv(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two fp32 values -> packed fp16 pair, round-to-nearest-even.
__device__ __forceinline__ unsigned pack_f16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
}

// Packed bf16 pair -> packed fp16 pair.
__device__ __forceinline__ unsigned bf16x2_to_f16x2(unsigned w) {
  return pack_f16x2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D, int BN, bool BF16, bool UNNORM>
__global__ void __launch_bounds__(kThreads)
prefill_kernel(PrefillArgs a) {
  constexpr int KSTR = D + 8;              // K tile row stride in LDS (elements)
  constexpr int VSTR = BN + 4;             // V^T tile row stride in LDS (elements)
  constexpr int NKK = D / 16;              // MFMA k-steps of Q.K^T
  constexpr int NKB = BN / 32;             // 32-key blocks per tile
  constexpr int NDB = D / 32;              // 32-row blocks of O^T
  constexpr int NKS = BN / 16;             // MFMA k-steps of P.V
  constexpr int KCH = BN * D / 8;          // 16-byte chunks in a K tile
  constexpr int K_IT = (KCH + kThreads - 1) / kThreads;
  constexpr int VUN = (BN / 4) * (D / 8);  // (4 keys x 8 dims) units in a V tile
  constexpr int V_IT = (VUN + kThreads - 1) / kThreads;

  __shared__ __attribute__((aligned(16))) unsigned short k_lds[BN * KSTR];
  __shared__ __attribute__((aligned(16))) unsigned short vt_lds[D * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = blockIdx.x;
  const int qb = (int)gridDim.y - 1 - (int)blockIdx.y;   // longest causal rows first
  const int b = blockIdx.z;
  const int hk = h / (a.n_heads_q / a.n_heads_kv);
  const int q0 = qb * kBM;
  const int off = a.seqlen_kv - a.seqlen_q;              // bottom-right alignment

  const int n = lane & 31;    // MFMA column = this lane's query within the wave
  const int hh = lane >> 5;   // lane half
  const int qi = q0 + wave * 32 + n;
  const bool q_valid = qi < a.seqlen_q;
  const int qpos = qi + off;

  const unsigned short* kp =
      (const unsigned short*)a.k + (int64_t)b * a.k_sb + (int64_t)hk * a.k_sh;
  const unsigned short* vp =
      (const unsigned short*)a.v + (int64_t)b * a.v_sb + (int64_t)hk * a.v_sh;

  // Q^T operand: 8 consecutive dims of this lane's query per k-step.
  u32x4 qr[NKK];
  {
    const unsigned short* qp = (const unsigned short*)a.q + (int64_t)b * a.q_sb +
                               (int64_t)qi * a.q_ss + (int64_t)h * a.q_sh;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qr[kk] = q_valid ? *(const u32x4*)(qp + kk * 16 + hh * 8) : u32x4{0, 0, 0, 0};
  }

  // KV range: keys up to the largest query position of the block.
  int kv_end = a.seqlen_kv;
  if (a.causal) kv_end = min(a.seqlen_kv, min(q0 + kBM, a.seqlen_q) + off);
  const int ntiles = (kv_end + BN - 1) / BN;
  const int wave_first_qpos = q0 + wave * 32 + off;
  const int wave_last_qpos =
      a.causal ? min(q0 + wave * 32 + 31, a.seqlen_q - 1) + off : INT_MAX;

  u32x4 kreg[K_IT];
  u32x4 vreg[V_IT][4];

  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < K_IT; ++i) {
      const int c = tid + i * kThreads;
      if (KCH % kThreads == 0 || c < KCH) {
        const int row = c / (D / 8), col = (c % (D / 8)) * 8;
        const int key = t0 + row;
        kreg[i] = key < a.seqlen_kv ? *(const u32x4*)(kp + (int64_t)key * a.k_ss + col)
                                    : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < V_IT; ++i) {
      const int u = tid + i * kThreads;
      if (VUN % kThreads == 0 || u < VUN) {
        const int dc = u % (D / 8), kg = u / (D / 8);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = t0 + kg * 4 + r;
          vreg[i][r] = key < a.seqlen_kv
                           ? *(const u32x4*)(vp + (int64_t)key * a.v_ss + dc * 8)
                           : u32x4{0, 0, 0, 0};
        }
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < K_IT; ++i) {
      const int c = tid + i * kThreads;
      if (KCH % kThreads == 0 || c < KCH) {
        const int row = c / (D / 8), col = (c % (D / 8)) * 8;
        *(u32x4*)(k_lds + row * KSTR + col) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < V_IT; ++i) {
      const int u = tid + i * kThreads;
      if (VUN % kThreads == 0 || u < VUN) {
        const int dc = u % (D / 8), kg = u / (D / 8);
        u32x4 w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[r][e] = BF16 ? bf16x2_to_f16x2(vreg[i][r][e]) : vreg[i][r][e];
        }
        // Transpose 4 keys x 8 dims into V^T rows: dim d gets keys kg*4 .. kg*4+3.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u32x2 lo = {__builtin_amdgcn_perm(w[1][e], w[0][e], 0x05040100u),
                      __builtin_amdgcn_perm(w[3][e], w[2][e], 0x05040100u)};
          u32x2 hi = {__builtin_amdgcn_perm(w[1][e], w[0][e], 0x07060302u),
                      __builtin_amdgcn_perm(w[3][e], w[2][e], 0x07060302u)};
          *(u32x2*)(vt_lds + (dc * 8 + 2 * e) * VSTR + kg * 4) = lo;
          *(u32x2*)(vt_lds + (dc * 8 + 2 * e + 1) * VSTR + kg * 4) = hi;
        }
      }
    }
  };

  float m_used = -1e30f;   // base of the exponentials (log2 units)
  float m_true = -1e30f;   // exact running row max (log2 units)
  float l = 0.0f;          // this lane's part of the row sum (relative to m_used - kShift)
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};

  if (ntiles > 0) load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    const int t0 = t * BN;
    __syncthreads();                 // every wave is done reading the previous tile
    store_tile();
    __syncthreads();                 // the tile is complete in LDS
    if (t + 1 < ntiles) load_tile(t0 + BN);
    if (t0 > wave_last_qpos) continue;   // tile entirely above this wave's diagonal

    // S^T = K . Q^T : rows = keys (M), columns = this wave's 32 queries (N).
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const u32x4 ka = *(const u32x4*)(k_lds + (kb * 32 + n) * KSTR + kk * 16 + hh * 8);
        sacc[kb] = mfma_qk<BF16>(ka, qr[kk], sacc[kb]);
      }
    }

    // Accumulator element i of block kb holds key t0 + kb*32 + (i/4)*8 + hh*4 + i%4.
    const bool need_mask =
        (a.causal && t0 + BN - 1 > wave_first_qpos) || (t0 + BN > a.seqlen_kv);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = t0 + kb * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
          const bool vis = key < a.seqlen_kv && (!a.causal || key <= qpos);
          if (!vis) sacc[kb][i] = -INFINITY;
        }
      }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float tmax = mx * a.scale_log2;   // scale > 0: max commutes with the scaling
    m_true = fmaxf(m_true, tmax);
    const bool grow = tmax > m_used + kSlack;
    if (__ballot(grow)) {
      const float nm = grow ? tmax : m_used;
      const float corr = exp2_fast(m_used - nm);
      m_used = nm;
      l *= corr;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= corr;
    }

    // P = 2^(s*scale*log2e - (m_used - kShift)) <= 2^(kSlack + kShift) = 32768.
    const float base = m_used - kShift;
    u32x4 pk[NKS];
    float ls = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = exp2_fast(__builtin_fmaf(sacc[kb][i], a.scale_log2, -base));
        const float p1 = exp2_fast(__builtin_fmaf(sacc[kb][i + 1], a.scale_log2, -base));
        ls += p0;
        ls += p1;
        pk[kb * 2 + (i >> 3)][(i & 7) >> 1] = pack_f16x2(p0, p1);
      }
    }
    l += ls;

    // O^T += V^T . P^T over this tile's keys (key order matches the S^T layout).
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const unsigned short* vr =
            vt_lds + (db * 32 + n) * VSTR + (ks >> 1) * 32 + (ks & 1) * 16 + hh * 4;
        const u32x2 v0 = *(const u32x2*)(vr);
        const u32x2 v1 = *(const u32x2*)(vr + 8);
        const u32x4 va = {v0[0], v0[1], v1[0], v1[1]};
        oacc[db] = mfma_pv(va, pk[ks], oacc[db]);
      }
    }
  }

  l += __shfl_xor(l, 32);
  if (!q_valid) return;

  // Refer the outputs back to the true row max: factor = 2^((m_used - kShift) - m_true).
  const float to_true = exp2_fast(m_used - kShift - m_true);
  const float row_sum = l * to_true;
  float* orow = a.o + (int64_t)b * a.o_sb + (int64_t)qi * a.o_ss + (int64_t)h * a.o_sh;
  const float f = UNNORM ? to_true : 1.0f / l;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 val = {oacc[db][4 * g] * f, oacc[db][4 * g + 1] * f, oacc[db][4 * g + 2] * f,
                         oacc[db][4 * g + 3] * f};
      *(f32x4*)(orow + db * 32 + g * 8 + hh * 4) = val;
    }
  }
  if (hh == 0) {
    const int64_t ri = ((int64_t)b * a.n_heads_q + h) * a.seqlen_q + qi;
    a.lse[ri] = (m_used - kShift + __log2f(l)) * kLn2;
    if (a.row_sum) a.row_sum[ri] = row_sum;
  }
}

template <int D, int BN, bool BF16>
hipError_t launch_d(const PrefillArgs& a, bool unnorm, hipStream_t stream) {
  const dim3 grid(a.n_heads_q, (a.seqlen_q + kBM - 1) / kBM, a.batch);
  if (unnorm)
    hipLaunchKernelGGL((prefill_kernel<D, BN, BF16, true>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, BN, BF16, false>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, bool bf16, bool unnormalized,
                          hipStream_t stream) {
  switch (head_dim) {
    case 64:
      return bf16 ? launch_d<64, 64, true>(a, unnormalized, stream)
                  : launch_d<64, 64, false>(a, unnormalized, stream);
    case 128:
      return bf16 ? launch_d<128, 64, true>(a, unnormalized, stream)
                  : launch_d<128, 64, false>(a, unnormalized, stream);
    case 256:
      return bf16 ? launch_d<256, 32, true>(a, unnormalized, stream)
                  : launch_d<256, 32, false>(a, unnormalized, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fa
