// Split-KV decode for gfx950: per-split partial attention and the LSE merge.
//
// Decode reads every K and V row once and does ~4 FLOP per byte per query
// head it serves, so with few heads per K/V row it is bound by HBM bandwidth,
// not by the matrix cores. The partial kernel is therefore VALU work arranged
// for bandwidth:
//
//  * one wave per (sequence, set of query heads sharing a KV head, split);
//    when the call needs more than one round of resident waves the wave
//    serves up to 8 query heads of the group, so each K/V row is read once
//    for all of them (the head packing of "STAGE_D.md — FMHA Kernel
//    Development", section D2); when it fits in one round, fewer heads per
//    wave shorten each wave's serial chain (decode_heads_per_wave);
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
//    form: new max, correction factor, exponential, running sum and output);
//  * from 2 query heads per wave (head_dim <= 128) the per-head work
//    moves to the matrix cores: Q.K^T and P.V
//    (split_attend_mfma_pv); each K row then serves up to 16 heads in one
//    16x16x32 MFMA, and the exponentials are spread one per (key, head).
//
// Each split emits a normalized partial O_s and its natural-log LSE_s. The
// merge then combines the partials by LSE in a fixed order, so the result is
// deterministic for a given split plan.
#include "fa_internal.h"

#include <climits>
#include <mutex>

// Scratch of the single-launch decode for callers that cannot allocate
// (fa_decode_fused_noalloc): one copy per GPU, held until the process ends.
// In host code this name only stands for the array; its device address is
// looked up per device (decode_noalloc_scratch) and only that address is
// handed to kernels.
static __device__ __align__(256) unsigned char scratch[fa::kNoAllocScratchBytes];

namespace fa {
namespace {

// Zeroes n 32-bit words (the arrival counters of the scratch, once per device).
__global__ void __launch_bounds__(256) zero_words_kernel(int* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

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

constexpr int lanes_per_row(int d) { return d >= 128 ? 16 : 8; }

// Two floats to packed fp16 (round to nearest even).
__device__ __forceinline__ unsigned pack_f16x2(float lo, float hi) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  f32x2v v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
}

// Online softmax of query heads h0 .. h0+G-1 of sequence b over its keys
// [lo, hi) (lo < hi), by one wave. D: head_dim. G: query heads served per wave
// (a divisor of the GQA group). On return every lane holds the split's running
// max m (log2 units), the row sum l and the un-normalized output o relative to
// base m; lane holds output elements c*EPL .. c*EPL+EPL-1 with c = lane % LPK.
template <int D, int G, bool BF16>
__device__ __forceinline__ void split_attend(const DecodeArgs& a, int b, int h0, int lo, int hi,
                                             int lane, float (&m)[G], float (&l)[G],
                                             float (&o)[G][D / lanes_per_row(D)]) {
  constexpr int LPK = lanes_per_row(D);    // lanes per K/V row
  constexpr int EPL = D / LPK;             // elements per lane: 8 or 16
  constexpr int W = EPL / 8;               // 16-byte loads per row per lane
  constexpr int KPS = 64 / LPK;            // rows per load step: 4 or 8
  // load steps per block: 16 KB of K+V per block, halved when the wave serves
  // more than 4 heads (their accumulators need the registers)
  constexpr int NB = D == 256 ? (G > 4 ? 2 : 4) : (G > 4 ? 4 : 8);
  constexpr int BK = KPS * NB;             // rows per block

  const int hk = h0 / (a.n_heads_q / a.n_heads_kv);
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

  // Sum the row slots (m is the same in every lane).
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int x = LPK; x < 64; x *= 2) {
      l[g] += __shfl_xor(l[g], x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] += __shfl_xor(o[g][e], x);
    }
  }
}

// 16x16x32 MFMA on packed halves (A, B: 8 halves per lane; C: 4 floats per lane).
template <bool BF16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// The same split on the matrix cores, for waves that serve several query heads
// (D <= 128). Per 32-key block:
//  * K and V rows are loaded as whole rows (16 lanes x 16 bytes per 256-byte
//    row, like the VALU form): the MFMA operand layout would have each load
//    instruction take 64 bytes from each of 16 rows, which streamed ~10 %
//    slower from HBM. The wave stores both blocks to its LDS area (16-byte
//    chunks XOR-swizzled by row) and reads the operands back from there;
//  * S^T = K . Q^T, 16 keys x 16 heads per v_mfma_f32_16x16x32 (K read as
//    lane l: row l % 16 of a 16-key half, chunk 4*kk + l / 16, i.e. dims
//    32*kk + 8*(l/16) .. +7; Q of head l % 16 for the same dims, zero past
//    the group); lane l receives S for keys 4*(l/16) .. +3 of head l % 16.
//    The block max and the exponentials run in that layout, one per (key,
//    head);
//  * P^T is already the B operand of O^T = V^T . P^T (heads along N): lane l
//    holds P of head l % 16 for keys 4*(l/16) + 0..3 of both 16-key halves,
//    and the MFMA's 32-long contraction takes those 8 keys in that order;
//  * the V^T operand comes from two ds_read_b64_tr_b16, which hand lane l
//    dim 16*db + l % 16 of keys 4*(l/16) + 0..3 and of the same keys 16
//    further;
//  * O^T accumulates in the MFMA's C layout (lane l: dims 16*db + 4*(l/16) +
//    0..3 of head l % 16), so the rescale on a new max is lane-local;
//  * bf16 caches: Q.K^T runs in bf16, and V is converted to fp16 after the
//    transposing reads (exact in fp16's normal range) for the fp16 P.V.
// P enters the MFMA as fp16 with 2^kPShift headroom over the running max (so
// the small weights stay normal); l sums the fp32 weights. At the end O^T goes
// through LDS to the row layout of split_attend's contract.
// lw: this wave's LDS scratch, 2 x 32 x D halves (K block, V block; 256-byte aligned).
constexpr float kPShift = 6.0f;   // P <= 2^(kSlack + kPShift) = 16384 in fp16

// From 2 heads per wave the matrix-core form is the faster one: the VALU
// form's per-head dot products, exponentials and output FMAs grow with the
// heads (batched long decode: 28/4 heads 1.2x, 32/8 heads 1.1x, 24/8 heads
// 1.05x, 16/8 heads 1.03x faster on the matrix cores, fp16 and bf16 alike).
// One head per wave keeps the VALU form: there the calls are latency-bound
// and the LDS round trips of the matrix-core form lengthen a wave's chain.
__host__ __device__ constexpr bool decode_pv_on_mfma(int d, int g, bool /*bf16*/) {
  return d <= 128 && g >= 2;
}

template <int D, int G, bool BF16>
__device__ __forceinline__ void split_attend_mfma_pv(const DecodeArgs& a, int b, int h0, int lo,
                                                     int hi, int lane, char* lw, float (&m)[G],
                                                     float (&l)[G],
                                                     float (&o)[G][D / lanes_per_row(D)]) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static_assert(G >= 1 && G <= 16, "at most 16 heads per wave");
  constexpr int LPK = lanes_per_row(D);    // lanes per row (row layout)
  constexpr int EPL = D / LPK;             // 8: one 16-byte chunk per lane
  static_assert(EPL == 8, "one chunk per lane and row");
  constexpr int KPS = 64 / LPK;            // rows per load step
  constexpr int BK = 32;                   // keys per block
  constexpr int NB = BK / KPS;             // load steps per block
  constexpr int NKK = D / 32;              // Q.K^T k-steps
  constexpr int NDB = D / 16;              // 16-dim blocks of O^T
  constexpr int ROWB = D * 2;              // bytes per row in LDS
  constexpr int BLK = BK * ROWB;           // bytes per block in LDS
  // Chunk swizzles by row r. K: the 16 rows one operand read touches, 4
  // chunks each, fill every chunk position of the bank lines 4 times (the
  // minimum for 1 KB). V: the 16 rows one transpose read touches, 2 chunks
  // each, land on distinct chunk pairs of their bank line (2 passes for 512 B).
  constexpr auto kswz = [](int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };
  constexpr auto vswz = [](int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); };

  const int hk = h0 / (a.n_heads_q / a.n_heads_kv);
  const int slot = lane / LPK;
  const int c = lane % LPK;
  const int n = lane & 15;                 // MFMA column: query head h0 + n
  const int quad = lane >> 4;

  u32x4 qop[NKK];
  {
    const unsigned short* qp = (const unsigned short*)a.q + (int64_t)b * a.q_sb +
                               (int64_t)(h0 + min(n, G - 1)) * a.q_sh + quad * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qop[kk] = n < G ? *(const u32x4*)(qp + kk * 32) : u32x4{0, 0, 0, 0};
  }

  const int64_t row0 = a.kv_offsets[b];
  const int64_t head = row0 * a.kv_st + (int64_t)hk * a.kv_sh + c * EPL;
  const unsigned short* kbase = (const unsigned short*)a.k + head;
  const unsigned short* vbase = (const unsigned short*)a.v + head;

  // LDS byte offsets. Writes: this lane's chunk of load step j (row
  // j*KPS + slot); the swizzles of those rows depend on j only through
  // j's parity for V at D = 128. Reads: K operand of half sb and k-step kk
  // (row 16*sb + n, chunk 4*kk + quad); V^T transpose read of dim block db
  // (row 4*quad + (lane % 16) / 4, dims 16*db + 4*(lane % 4) .. +3).
  const unsigned kl = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)lw;
  const unsigned vl = kl + BLK;
  const unsigned kw_off = kl + (unsigned)(slot * ROWB + ((c ^ kswz(slot)) << 4));
  unsigned vw_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    vw_off[par] = vl + (unsigned)(slot * ROWB + ((c ^ vswz(par * KPS + slot)) << 4));
  // The area is 256-byte aligned and the swizzles only flip the bits that
  // select 64-byte (K) or 32-byte (V) groups of a row, so k-step kk and dim
  // block db are reached from the kk = 0 / db = 0 offsets by an XOR.
  const unsigned kr0 = kl + (unsigned)(n * ROWB + ((quad ^ kswz(n)) << 4));
  unsigned vr0;
  {
    const int j = lane & 15;
    const int r = 4 * quad + (j >> 2);
    vr0 = vl + (unsigned)(r * ROWB + ((((j & 3) >> 1) ^ vswz(r)) << 4) + 8 * (j & 1));
  }

  // One block of K and V rows (rows past hi repeat row hi-1, valid memory;
  // their scores are masked).
  auto load_block = [&](int start, u32x4 (&kd)[NB], u32x4 (&vd)[NB]) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int64_t off = (int64_t)min(start + j * KPS + slot, hi - 1) * a.kv_st;
      kd[j] = __builtin_nontemporal_load((const u32x4*)(kbase + off));
      vd[j] = __builtin_nontemporal_load((const u32x4*)(vbase + off));
    }
  };

  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  typedef float f32x2 __attribute__((ext_vector_type(2)));

  float mc = -1e30f;   // running max (log2 units) of head column n
  float lp = 0.0f;     // this lane's part of head n's row sum (relative to mc - kPShift)
  f32x4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // A block's rows to LDS. (The previous block's operand reads were consumed
  // by its MFMAs, so this wave's LDS operations have drained.)
  auto stage_block = [&](const u32x4 (&kd)[NB], const u32x4 (&vd)[NB]) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      *(lds_u32x4*)(uintptr_t)(kw_off + (unsigned)(j * KPS * ROWB)) = kd[j];
      *(lds_u32x4*)(uintptr_t)(vw_off[(j * KPS / 4) & 1] + (unsigned)(j * KPS * ROWB)) = vd[j];
    }
  };
  auto compute_block = [&](int start) {
    // Every lane's rows have landed before any lane reads them.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    f32x4 s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        s[sb] = mfma16<BF16>(
            *(const lds_u32x4*)(uintptr_t)((kr0 ^ (unsigned)(kk << 6)) + (unsigned)(sb * 16 * ROWB)),
            qop[kk], s[sb]);
    }
    if (start + BK > hi) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (start + sb * 16 + quad * 4 + i >= hi) s[sb][i] = -INFINITY;
    }
    float lm = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    lm = fmaxf(lm, __shfl_xor(lm, 16));
    lm = fmaxf(lm, __shfl_xor(lm, 32));
    const float bm = lm * a.scale_log2;    // the max commutes with the positive scale
    const bool grow = bm > mc + kSlack;
    if (__ballot(grow)) {
      const float nm = grow ? bm : mc;
      const float corr = __builtin_amdgcn_exp2f(mc - nm);
      mc = nm;
      lp *= corr;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[db][i] *= corr;
    }
    const float base = mc - kPShift;
    float p[2][4];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[sb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][i], a.scale_log2, -base));
        lp += p[sb][i];
      }
    const u32x4 pb = u32x4{pack_f16x2(p[0][0], p[0][1]), pack_f16x2(p[0][2], p[0][3]),
                           pack_f16x2(p[1][0], p[1][1]), pack_f16x2(p[1][2], p[1][3])};
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const unsigned vr = vr0 ^ (unsigned)(db << 5);
      const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)vr);
      const s16x4 hi4 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(vr + 16 * ROWB));
      const f32x2 l2 = __builtin_bit_cast(f32x2, lo4), h2 = __builtin_bit_cast(f32x2, hi4);
      u32x4 va = u32x4{__float_as_uint(l2[0]), __float_as_uint(l2[1]),
                       __float_as_uint(h2[0]), __float_as_uint(h2[1])};
      if constexpr (BF16) {
        // bf16 V to fp16 for the fp16 P.V (exact in fp16's normal range)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          va[e] = pack_f16x2(__uint_as_float(va[e] << 16), __uint_as_float(va[e] & 0xffff0000u));
      }
      oacc[db] = mfma16<false>(va, pb, oacc[db]);
    }
  };

  // Two register buffers in turn, two blocks ahead: once a block's rows are in
  // LDS its registers take the block after next, so while a block is computed
  // the next two are in flight. The loads are issued unconditionally (past hi
  // they repeat row hi-1 and go unused): the compiler can then wait for
  // exactly the block it stages instead of for every load in flight.
  u32x4 ka[NB], kb[NB], va[NB], vb[NB];
  load_block(lo, ka, va);
  load_block(lo + BK, kb, vb);
  for (int start = lo;; start += 2 * BK) {
    stage_block(ka, va);
    load_block(start + 2 * BK, ka, va);
    compute_block(start);
    if (start + BK >= hi) break;
    stage_block(kb, vb);
    load_block(start + 3 * BK, kb, vb);
    compute_block(start + BK);
    if (start + 2 * BK >= hi) break;
  }

  // Head n's row sum over the four lane groups; m and l of every head to every lane.
  lp += __shfl_xor(lp, 16);
  lp += __shfl_xor(lp, 32);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mc), g)) - kPShift;
    l[g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lp), g));
  }
  // O^T (C layout) -> [head][dim] fp32 in LDS -> row layout (every slot alike).
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the last block's reads are done
  float* ob = (float*)lw;                                // G x D floats fit in 32 x D halves
  if (n < G) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *(f32x4*)(ob + n * D + db * 16 + quad * 4) = oacc[db];
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const f32x4 x0 = *(const f32x4*)(ob + g * D + c * EPL);
    const f32x4 x1 = *(const f32x4*)(ob + g * D + c * EPL + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[g][e] = x0[e];
      o[g][4 + e] = x1[e];
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the area is reused
}

// LDS floats per wave that split_run needs: the K and V blocks of the
// matrix-core form, else none.
__host__ __device__ constexpr int decode_lds_floats(int d, int g, bool bf16) {
  return decode_pv_on_mfma(d, g, bf16) ? 2 * 32 * d / 2 : 1;
}

// The split of one wave by whichever form serves its (D, G); pw (this wave's
// decode_lds_floats floats of LDS) is used by the matrix-core forms only.
template <int D, int G, bool BF16>
__device__ __forceinline__ void split_run(const DecodeArgs& a, int b, int h0, int lo, int hi,
                                         int lane, float* pw, float (&m)[G], float (&l)[G],
                                         float (&o)[G][D / lanes_per_row(D)]) {
  if constexpr (decode_pv_on_mfma(D, G, BF16))
    split_attend_mfma_pv<D, G, BF16>(a, b, h0, lo, hi, lane, (char*)pw, m, l, o);
  else
    split_attend<D, G, BF16>(a, b, h0, lo, hi, lane, m, l, o);
}

// Launch order of the decode work-groups. A "unit" is one (sequence, split)
// pair with work (or split group, for the fused kernel), numbered densely in
// (sequence, split) order; a "cluster" is the work-groups that read the same
// K/V rows: one unit, one KV head, and the q_per_kv head groups of that KV
// head. Work-group i runs on XCD i % 8, which has its own L2: a cluster's
// work-groups all go to one XCD, so after the first fetch its rows come from
// that L2 (the loads are non-temporal but reach L2), and consecutive clusters,
// KV heads fastest (the same token rows), go to consecutive XCDs. The grid is
// sized for every sequence at the longest one's split count, but the units
// are numbered densely, so every work-group with work comes before every one
// without (those exit at once). Work-groups are dispatched in order, each as
// soon as a slot frees: with the empty ones interleaved among the real ones,
// the real ones landed unevenly on the compute units and some waited behind a
// full one while others sat idle.
struct DecItem {
  int b, hg, y;   // sequence, head group, split (or split group)
  bool valid;
};
__host__ __device__ inline int64_t dec_grid(int batch, int n_heads_kv, int q_per_kv, int ny) {
  const int64_t c = (int64_t)batch * n_heads_kv * ny;
  return 8 * ((c + 7) / 8) * q_per_kv;
}
// Inclusive prefix sum across the wave.
__device__ __forceinline__ int wave_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  return v;
}
// Work-group id's item; units_of(L) is the number of units of a sequence of L
// keys. Every lane of the wave takes part; the result is wave-uniform.
template <typename UnitsOf>
__device__ inline DecItem dec_item(int id, const int* kv_lens, int batch, int n_heads_kv,
                                   int q_per_kv, int lane, UnitsOf units_of) {
  const int x = id & 7, m = id >> 3;
  const int j = m % q_per_kv;
  const int64_t c = (int64_t)(m / q_per_kv) * 8 + x;
  const int hk = (int)(c % n_heads_kv);
  const int64_t r = c / n_heads_kv;          // unit
  DecItem it;
  it.valid = false;
  it.b = it.y = 0;
  it.hg = hk * q_per_kv + j;
  int64_t base = 0;                          // units of the sequences before b0
  for (int b0 = 0; b0 < batch; b0 += 256) {
    int n[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {            // the four loads in flight together
      const int b = b0 + 64 * i + lane;
      n[i] = b < batch ? units_of(kv_lens[b]) : 0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int incl = wave_scan(n[i], lane);
      const uint64_t hit = __ballot(base + incl > r);
      if (hit) {
        const int first = __ffsll((long long)hit) - 1;
        it.b = b0 + 64 * i + first;
        it.y = (int)(r - base - __shfl(incl - n[i], first));
        it.b = __builtin_amdgcn_readfirstlane(it.b);
        it.y = __builtin_amdgcn_readfirstlane(it.y);
        it.valid = true;
        return it;
      }
      base += __shfl(incl, 63);
    }
  }
  return it;
}

// One wave per (sequence, group of G query heads, split): the split's
// normalized partial output and its natural-log LSE.
template <int D, int G, bool BF16>
__global__ void __launch_bounds__(64)
decode_partial_kernel(DecodeArgs a) {
  constexpr int LPK = lanes_per_row(D);
  constexpr int EPL = D / LPK;
  const int lane = threadIdx.x;
  const int qpk = a.n_heads_q / a.n_heads_kv / G;   // head groups per KV head
  const int sl = a.split_len, ms = a.max_splits;
  const DecItem it = dec_item(blockIdx.x, a.kv_lens, a.batch, a.n_heads_kv, qpk, lane,
                              [=](int L) { return L < 1 ? 0 : min((L + sl - 1) / sl, ms); });
  if (!it.valid) return;                 // no unit: nothing read or written
  const int h0 = it.hg * G, s = it.y, b = it.b;
  const int L = a.kv_lens[b];
  const int lo = s * a.split_len;
  const int hi = min(L, lo + a.split_len);
  const int slot = lane / LPK;
  const int c = lane % LPK;
  __shared__ __attribute__((aligned(256))) float pbuf[decode_lds_floats(D, G, BF16)];
  float m[G], l[G], o[G][EPL];
  split_run<D, G, BF16>(a, b, h0, lo, hi, lane, pbuf, m, l, o);
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

// Merge of ns >= 1 normalized partials of one query head by one wave: pl[j]
// is partial j's natural-log LSE, po + j*D its output row. Split LSEs are read
// lane-parallel and reduced across the wave; the weighted sum of the partial
// outputs runs over the partials in index order with the loads of several
// partials in flight. Writes out[0..D) and *lse_out.
template <int D>
__device__ __forceinline__ void merge_head(const float* pl, const float* po_row0, int ns,
                                           int lane, float* out, float* lse_out) {
  constexpr int EPL = D / 64;
  constexpr int U = 32;                    // partials in flight per step
  const float* po = po_row0 + lane * EPL;
  if (ns <= U) {
    // Common case: the LSEs and every partial row are requested together (one
    // memory round trip); same arithmetic, in the same order, as below.
    const float lv = pl[min(lane, ns - 1)];
    float v[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sj = min(u, ns - 1);
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[u][e] = po[(int64_t)sj * D + e];
    }
    float M = lane < ns ? lv : -INFINITY;
#pragma unroll
    for (int x = 1; x < 64; x *= 2) M = fmaxf(M, __shfl_xor(M, x));
    const float wl = lane < ns ? __expf(lv - M) : 0.0f;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < ns) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(w, v[u][e], acc[e]);
      }
    }
    float wsum = wl;
#pragma unroll
    for (int x = 1; x < 64; x *= 2) wsum += __shfl_xor(wsum, x);
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[lane * EPL + e] = acc[e] * inv;
    if (lane == 0) *lse_out = M + __logf(wsum);
    return;
  }
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
  if (lane == 0) *lse_out = M + __logf(wsum);
}

// NaN output row and LSE: the mark of a sequence whose length breaks the plan.
template <int D>
__device__ __forceinline__ void nan_head(int lane, float* out, float* lse_out) {
#pragma unroll
  for (int e = 0; e < D / 64; ++e) out[lane * (D / 64) + e] = __builtin_nanf("");
  if (lane == 0) *lse_out = __builtin_nanf("");
}

// One wave per (sequence, query head).
template <int D>
__global__ void __launch_bounds__(64)
decode_merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t bh = (int64_t)b * a.n_heads_q + h;
  const int L = a.kv_lens[b];
  const int ns = L < 1 ? 0 : (L + a.split_len - 1) / a.split_len;
  if (ns < 1 || ns > a.max_splits)
    nan_head<D>(lane, a.o + bh * D, a.lse + bh);
  else
    merge_head<D>(a.part_lse + bh * a.max_splits, a.part_o + bh * a.max_splits * D, ns, lane,
                  a.o + bh * D, a.lse + bh);
}

// Single-launch decode. A work-group of NW waves takes NW consecutive splits
// of one (sequence, head group); each wave runs its split as above, and the
// work-group merges the NW results through LDS (max-shifted weights, waves in
// split order). When one work-group covers every split of the sequence, that
// merge is the output. Otherwise each work-group stores its merged partial
// and LSE, and the last work-group of the (sequence, head group) to finish
// (an agent-scope counter; no work-group ever waits for another) merges those
// partials in index order and resets the counter to zero. The result is a
// fixed function of the split plan, so repeated runs are byte-identical.
// The one-wave matrix-core P.V form is held to two waves per SIMD (left to
// itself, the allocator moved a few registers to AGPRs and halved it). The
// 4-wave form runs only when the whole call fits in one round of resident
// waves, where occupancy matters less; held to two waves it spills.
template <int D, int G, bool BF16, int NW>
__global__ void __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(decode_pv_on_mfma(D, G, BF16) && NW == 1 ? 2 : 1)))
decode_fused_kernel(DecodeArgs a) {
  constexpr int LPK = lanes_per_row(D);
  constexpr int EPL = D / LPK;
  constexpr int NT = 64 * NW;
  __shared__ float so[NW][G][D];
  __shared__ float sm[NW][G], sl[NW][G];
  __shared__ int is_last;
  __shared__ __attribute__((aligned(256))) float pbuf[NW][decode_lds_floats(D, G, BF16)];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qpk = a.n_heads_q / a.n_heads_kv / G;   // head groups per KV head
  // A sequence with no key or more splits than max_splits has one unit (its
  // work-group writes the NaN mark), else one per group of NW splits.
  const int slen = a.split_len, ms = a.max_splits;
  const DecItem it = dec_item(blockIdx.x, a.kv_lens, a.batch, a.n_heads_kv, qpk, lane,
                              [=](int L) {
                                const int n = L < 1 ? 0 : (L + slen - 1) / slen;
                                return n < 1 || n > ms ? 1 : (n + NW - 1) / NW;
                              });
  if (!it.valid) return;
  const int hg = it.hg, h0 = hg * G, y = it.y, b = it.b;
  const int L = a.kv_lens[b];
  const int ns = L < 1 ? 0 : (L + a.split_len - 1) / a.split_len;
  const bool bad = ns < 1 || ns > a.max_splits;
  const int nwg = bad ? 0 : (ns + NW - 1) / NW;              // work-groups with splits
  const int nvalid = bad ? 0 : min(NW, max(0, ns - y * NW));  // splits of this one
  const bool single = a.max_wg == 1;

  if (wave < nvalid) {
    const int lo = (y * NW + wave) * a.split_len;
    const int hi = min(L, lo + a.split_len);
    float m[G], l[G], o[G][EPL];
    split_run<D, G, BF16>(a, b, h0, lo, hi, lane, pbuf[wave], m, l, o);
    if (lane < LPK) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          *(f32x4*)&so[wave][g][lane * EPL + e] =
              f32x4{o[g][e], o[g][e + 1], o[g][e + 2], o[g][e + 3]};
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        sm[wave][g] = m[g];
        sl[wave][g] = l[g];
      }
    }
  }
  __syncthreads();

  const int64_t bh0 = (int64_t)b * a.n_heads_q + h0;
  if (nvalid > 0) {
    for (int e = tid; e < G * D; e += NT) {
      const int g = e / D, d = e % D;
      float M = sm[0][g];
      for (int w = 1; w < nvalid; ++w) M = fmaxf(M, sm[w][g]);
      float lsum = 0.0f, acc = 0.0f;
      for (int w = 0; w < nvalid; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm[w][g] - M);
        lsum = __builtin_fmaf(f, sl[w][g], lsum);
        acc = __builtin_fmaf(f, so[w][g][d], acc);
      }
      const float out = acc / lsum;                 // every split has a key: lsum >= 1
      const float lse = (M + __log2f(lsum)) * kLn2;
      if (single) {
        a.o[(bh0 + g) * D + d] = out;
        if (d == 0) a.lse[bh0 + g] = lse;
      } else {   // agent-scope stores: written through to memory, seen by every XCD
        __hip_atomic_store(&a.wg_o[((bh0 + g) * a.max_wg + y) * D + d], out, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0)
          __hip_atomic_store(&a.wg_lse[(bh0 + g) * a.max_wg + y], lse, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (single) {
    if (bad)
      for (int e = tid; e < G * D; e += NT) {
        a.o[(bh0 + e / D) * D + e % D] = __builtin_nanf("");
        if (e % D == 0) a.lse[bh0 + e / D] = __builtin_nanf("");
      }
    return;
  }

  // Count this work-group once its partial has reached memory, and let the
  // last one merge. The partial went out as agent-scope stores, so waiting for
  // their completion publishes it; an agent-scope release fence would instead
  // write back the whole L2 of this XCD from every work-group.
  int* counter = a.counters + (int64_t)b * (a.n_heads_q / G) + hg;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    is_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (bad ? 0 : nwg - 1);
  __syncthreads();
  if (!is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // drop stale cached partials

  // Wave w merges heads w, w + NW, ... of the group, all of them at once so
  // that their loads are in flight together (as merge_head does for one).
  constexpr int GH = (G + NW - 1) / NW;          // heads per wave
  constexpr int EPL2 = D / 64;                   // output elements per lane
  constexpr int U = GH * EPL2 <= 64 ? 64 / (GH * EPL2) : 1;   // partial rows in flight
  const float* pl[GH];
  const float* po[GH];
  bool hv[GH];
#pragma unroll
  for (int i = 0; i < GH; ++i) {
    const int g = wave + i * NW;
    hv[i] = g < G;
    const int64_t bh = bh0 + (hv[i] ? g : 0);
    pl[i] = a.wg_lse + bh * a.max_wg;
    po[i] = a.wg_o + bh * a.max_wg * D + lane * EPL2;
    if (bad && hv[i]) nan_head<D>(lane, a.o + bh * D, a.lse + bh);
  }
  if (!bad && nwg <= U) {
    // Common case: every partial row and LSE is requested in one round.
    float v[GH][U][EPL2], lv[GH];
#pragma unroll
    for (int i = 0; i < GH; ++i) {
      lv[i] = pl[i][min(lane, nwg - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < EPL2; ++e) v[i][u][e] = po[i][(int64_t)min(u, nwg - 1) * D + e];
    }
#pragma unroll
    for (int i = 0; i < GH; ++i) {
      if (!hv[i]) continue;
      float M = lane < nwg ? lv[i] : -INFINITY;
#pragma unroll
      for (int x = 1; x < 64; x *= 2) M = fmaxf(M, __shfl_xor(M, x));
      const float wl = lane < nwg ? __expf(lv[i] - M) : 0.0f;
      float acc[EPL2];
#pragma unroll
      for (int e = 0; e < EPL2; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (u < nwg) {
          const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));
#pragma unroll
          for (int e = 0; e < EPL2; ++e) acc[e] = __builtin_fmaf(w, v[i][u][e], acc[e]);
        }
      float wsum = wl;
#pragma unroll
      for (int x = 1; x < 64; x *= 2) wsum += __shfl_xor(wsum, x);
      const int64_t bh = bh0 + wave + i * NW;
      const float inv = 1.0f / wsum;
#pragma unroll
      for (int e = 0; e < EPL2; ++e) a.o[bh * D + lane * EPL2 + e] = acc[e] * inv;
      if (lane == 0) a.lse[bh] = M + __logf(wsum);
    }
  } else if (!bad) {
    float M[GH], wsum[GH], acc[GH][EPL2];
#pragma unroll
    for (int i = 0; i < GH; ++i) {
      M[i] = -INFINITY;
      wsum[i] = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL2; ++e) acc[i][e] = 0.0f;
    }
    for (int j0 = 0; j0 < nwg; j0 += 64)
#pragma unroll
      for (int i = 0; i < GH; ++i)
        if (j0 + lane < nwg) M[i] = fmaxf(M[i], pl[i][j0 + lane]);
#pragma unroll
    for (int i = 0; i < GH; ++i)
#pragma unroll
      for (int x = 1; x < 64; x *= 2) M[i] = fmaxf(M[i], __shfl_xor(M[i], x));
    for (int j0 = 0; j0 < nwg; j0 += 64) {
      float wl[GH];
#pragma unroll
      for (int i = 0; i < GH; ++i) {
        wl[i] = j0 + lane < nwg ? __expf(pl[i][j0 + lane] - M[i]) : 0.0f;
        wsum[i] += wl[i];
      }
      const int n = min(64, nwg - j0);
      for (int j = 0; j < n; j += U) {
        float v[GH][U][EPL2];
#pragma unroll
        for (int i = 0; i < GH; ++i)
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int sj = j0 + min(j + u, n - 1);
#pragma unroll
            for (int e = 0; e < EPL2; ++e) v[i][u][e] = po[i][(int64_t)sj * D + e];
          }
#pragma unroll
        for (int i = 0; i < GH; ++i)
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (j + u < n) {
              const float w =
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl[i]), j + u));
#pragma unroll
              for (int e = 0; e < EPL2; ++e) acc[i][e] = __builtin_fmaf(w, v[i][u][e], acc[i][e]);
            }
      }
    }
#pragma unroll
    for (int i = 0; i < GH; ++i) {
      if (!hv[i]) continue;
#pragma unroll
      for (int x = 1; x < 64; x *= 2) wsum[i] += __shfl_xor(wsum[i], x);
      const int64_t bh = bh0 + wave + i * NW;
      const float inv = 1.0f / wsum[i];
#pragma unroll
      for (int e = 0; e < EPL2; ++e) a.o[bh * D + lane * EPL2 + e] = acc[i][e] * inv;
      if (lane == 0) a.lse[bh] = M[i] + __logf(wsum[i]);
    }
  }
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, bool BF16>
hipError_t launch_partial_d(const DecodeArgs& a, int g, hipStream_t stream) {
  const int64_t n = dec_grid(a.batch, a.n_heads_kv, a.n_heads_q / a.n_heads_kv / g, a.max_splits);
  if (n > INT_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)n);
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

template <int D, bool BF16, int NW>
hipError_t launch_fused_dw(const DecodeArgs& a, int g, hipStream_t stream) {
  const int64_t n = dec_grid(a.batch, a.n_heads_kv, a.n_heads_q / a.n_heads_kv / g, a.max_wg);
  if (n > INT_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)n);
  switch (g) {
#define FA_CASE(G)                                                                           \
  case G:                                                                                    \
    hipLaunchKernelGGL((decode_fused_kernel<D, G, BF16, NW>), grid, dim3(64 * NW), 0, stream, \
                       a);                                                                   \
    break;
    FA_CASE(1) FA_CASE(2) FA_CASE(3) FA_CASE(4) FA_CASE(5) FA_CASE(6) FA_CASE(7) FA_CASE(8)
#undef FA_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_fused_d(const DecodeArgs& a, int g, int nw, hipStream_t stream) {
  switch (nw) {
    case 1: return launch_fused_dw<D, BF16, 1>(a, g, stream);
    case 4: return launch_fused_dw<D, BF16, 4>(a, g, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Work-group size of the single-launch decode. A call that needs more than one
// round of resident waves is bandwidth-bound: one wave per work-group, so no
// compute unit slot waits on a sibling wave's split, and the one merge at the
// end is cheap next to the streaming (4 KV heads, 28 or 32 query heads, 25
// splits of 1296 tokens: 295 / 314 us with one wave against 355 / 371 with
// four). A call that fits in one round and has many short splits is
// latency-bound: groups of 4 merge on chip first, so the last work-group
// merges few partials (28/4 heads, 1641 tokens: 4 waves beat 2 and 8, which
// packs the latency-bound waves onto too few compute units).
int decode_fused_waves(int batch, int n_heads_q, int n_heads_kv, int head_dim, int max_splits) {
  if (max_splits <= 16) return 1;
  const int g = decode_heads_per_wave(n_heads_q / n_heads_kv, batch, n_heads_q, head_dim,
                                      max_splits);
  const size_t slots = (size_t)kDecodeCus * decode_waves_per_cu(head_dim);
  return sat_mul(sat_mul((size_t)batch, (size_t)(n_heads_q / g)), (size_t)max_splits) <= slots
             ? 4 : 1;
}

FusedLayout decode_fused_layout(int batch, int n_heads_q, int n_heads_kv, int head_dim,
                                int max_splits) {
  FusedLayout f{};
  const int g = decode_heads_per_wave(n_heads_q / n_heads_kv, batch, n_heads_q, head_dim,
                                      max_splits);
  f.waves = decode_fused_waves(batch, n_heads_q, n_heads_kv, head_dim, max_splits);
  f.max_wg = (int)(((int64_t)max_splits + f.waves - 1) / f.waves);
  // The counters sit in a fixed region at the start, whatever the shape, so a
  // workspace can serve calls of different shapes: no call's partials ever
  // land where another shape keeps its (zero between calls) counters.
  f.counters = 0;
  f.n_counters = (int64_t)batch * (n_heads_q / g);
  f.wg_lse = kFusedCounterBytes;
  const size_t parts = sat_mul(sat_mul((size_t)batch, (size_t)n_heads_q), (size_t)f.max_wg);
  f.wg_o = sat_add(f.wg_lse, sat_up256(sat_mul(parts, sizeof(float))));
  f.total = sat_add(f.wg_o, sat_up256(sat_mul(parts, (size_t)head_dim * sizeof(float))));
  return f;
}

hipError_t launch_decode_fused(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t stream) {
  const int g = decode_heads_per_wave(a.n_heads_q / a.n_heads_kv, a.batch, a.n_heads_q, head_dim,
                                      a.max_splits);
  const int nw = decode_fused_waves(a.batch, a.n_heads_q, a.n_heads_kv, head_dim, a.max_splits);
  if ((a.max_splits + nw - 1) / nw != a.max_wg) return hipErrorInvalidValue;
  switch (head_dim) {
    case 64: return bf16 ? launch_fused_d<64, true>(a, g, nw, stream)
                         : launch_fused_d<64, false>(a, g, nw, stream);
    case 128: return bf16 ? launch_fused_d<128, true>(a, g, nw, stream)
                          : launch_fused_d<128, false>(a, g, nw, stream);
    case 256: return bf16 ? launch_fused_d<256, true>(a, g, nw, stream)
                          : launch_fused_d<256, false>(a, g, nw, stream);
    default: return hipErrorInvalidValue;
  }
}

// Heads served per wave. Serving several query heads of a KV head from one
// wave reads each K/V row once for all of them, which is what a bandwidth-bound
// decode needs; but when every wave fits in one round of resident waves the
// call is latency-bound, and a wave's serial chain grows with its heads, so the
// fewest heads per wave that keep the whole call within one round win (at 28/4
// heads and 1641 keys: 10.0 us hot with one head per wave against 14.2 with
// seven). A pure function of the shape, so the float results repeat.
int decode_max_heads_per_wave(int group) {
  for (int g = 8; g >= 1; --g)
    if (group % g == 0) return g;
  return 1;
}
int decode_heads_per_wave(int group, int batch, int n_heads_q, int head_dim, int max_splits) {
  const int gmax = decode_max_heads_per_wave(group);
  const int64_t slots = (int64_t)kDecodeCus * decode_waves_per_cu(head_dim);
  for (int g = 1; g < gmax; ++g)
    if (group % g == 0 && (int64_t)batch * (n_heads_q / g) * max_splits <= slots) return g;
  return gmax;
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
  const int g = decode_heads_per_wave(a.n_heads_q / a.n_heads_kv, a.batch, a.n_heads_q, head_dim,
                                      a.max_splits);
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

hipError_t decode_noalloc_scratch(void** out, hipStream_t stream) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static void* addr[kMaxDevices];
  static hipError_t status[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [&] {
    // With this device current: the address of this device's copy of the array.
    void* p = nullptr;
    hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r == hipSuccess && p == nullptr) r = hipErrorInvalidSymbol;
    if (r == hipSuccess) {
      // The array starts zeroed when the code object loads; the counter region
      // is cleared once more here (a kernel, not a memset, so that a first call
      // made under stream capture records an ordinary kernel node), and every
      // call returns its counters to zero.
      constexpr int n = (int)(kFusedCounterBytes / sizeof(int));
      hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, (int*)p, n);
      r = hipGetLastError();
    }
    addr[dev] = p;
    status[dev] = r;
  });
  if (status[dev] != hipSuccess) return status[dev];
  *out = addr[dev];
  return hipSuccess;
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
