// Causal / unmasked GQA attention forward (prefill) for gfx950.
//
// Two launches on the caller's stream:
//
//  1. vt_pack_kernel: V [B, Skv, Hkv, D] (fp16 or bf16) -> fp16 V^T tiles in
//     the caller's workspace, laid out [B][Hkv][tile][D][T keys] (T = 64;
//     32 at head_dim 256 and 512), keys in
//     the order the P.V
//     contraction consumes them, 16-byte chunks XOR-swizzled inside every
//     row, and zero-filled keys past Skv. bf16 V is converted to fp16 here, once, instead of in every
//     work-group that reads the tile (exact for magnitudes in fp16's normal
//     range).
//
//  2. prefill_kernel: one work-group per (query block, query head, batch);
//     2 waves per SIMD. A work-group has 4 waves, each owning 32 query rows
//     (128 per block) and taking whole tiles of keys (64-key tiles up to
//     head_dim 128, 32-key tiles at head_dim 256), and two work-groups share
//     a compute unit (or, when two query heads of a KV head are paired at
//     head_dim <= 128, one work-group of 8 waves; see wg_waves). Head_dim 512
//     has its own kernel (prefill512_kernel) in which the two waves of a pair
//     split the head dimension.
//
// Mapping to the CDNA4 matrix cores (v_mfma_f32_32x32x16_{bf16,f16}): each
// wave computes the TRANSPOSED score tile S^T = K . Q^T (keys along M, its 32
// queries along N, one query per lane column), so the row max and row sum
// are in-lane reductions plus one exchange between the two 32-lane halves,
// and the output O^T = V^T . P^T keeps one query per lane column, so the
// per-row rescale is a per-lane scalar. P stays in registers: the S^T
// accumulator layout is reused as the B operand of the P.V contraction, with
// the V^T A operand read from LDS in the matching key order.
//
// K and V^T tiles move HBM -> LDS with direct global_load_lds_dwordx4 DMA
// (no VGPR staging), into a two-stage LDS ring: the loads for tile t+1 are
// issued before tile t is computed, and a single barrier per tile both
// publishes tile t+1 and releases tile t's stage (the two fence duties of
// the double-buffer scheme in "42 · r39 — q6_K KDR=2 double-buffer
// (LANDED)", section 2.3). K rows are stored with a 16-byte-chunk XOR
// swizzle so the 32-row MFMA operand reads hit distinct banks.
//
// Tiling and streaming follow "60 · r57 — FA KV staging double buffering
// (REVERTED)", sections 1 and 2.2 (grid over query block and head; KV tiles
// up to the causal bound; rows past the end never contribute), with the
// softmax kept in registers (its section 1) and the tile-end rescale of its
// section 2.3.
//
// Numerics:
//  * scores accumulate in fp32 from exact half products; the softmax scale
//    is applied to the fp32 scores (never folded into a half Q);
//  * exponentials are base 2 on scores pre-multiplied by scale*log2(e);
//  * P enters P.V as fp16 (round-to-nearest-even) with a 2^7 headroom
//    factor that keeps small P out of fp16's subnormal range and cancels in
//    O / l; the row sum l accumulates the fp32 P values;
//  * the running max is only moved (and O, l rescaled) once a tile max
//    exceeds it by more than 2^8 — exact, since O and l share the base —
//    and outputs are referred back to the true row max at the end;
//  * normalized output without row sums needs no exact max: there a tile's
//    max is not taken at all, and the base moves (to the row max) only when
//    a lane's sum of the tile's P exceeds 2^15, which bounds each of those P.
#include "fa_internal.h"

#include <limits.h>

#include <algorithm>
#include <functional>
#include <mutex>
#include <queue>
#include <type_traits>
#include <vector>

namespace fa {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef __attribute__((address_space(3))) void* lptr_t;

constexpr float kShift = 7.0f;            // log2 of the fp16 headroom factor on P
constexpr float kSlack = 8.0f;            // stale-max tolerance (log2 units)
constexpr float kSumCap = 32768.0f;       // tile-sum bound of the max-free softmax (2^15)
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.44269504088896341f;

// Work-group geometry per head dim. Every wave owns 32 query rows of one
// query head and takes whole tiles of keys: 64-key tiles up to head_dim 128,
// 32-key tiles at head_dim 256 (a wave cannot hold 64 keys of scores next to
// its Q and O registers there; 32-key tiles also keep the two tile stages at
// 64 KB, so two work-groups share a compute unit) and at head_dim 512.
// Query heads per work-group (hp): at head_dim <= 128, when the query heads
// that share a KV head come in pairs, a work-group serves the same 128 query
// rows of two of them, so every K and V^T tile brought into LDS feeds eight
// waves while the causal extent of a work-group stays that of 128 rows.
// Waves per work-group: 4 per query head (32 rows each) up to head_dim 256;
// head_dim 512 has its own kernel.
__host__ __device__ constexpr int wg_waves(int d, int hp) { return d <= 256 ? 4 * hp : 8; }
__host__ __device__ constexpr int tile_keys(int d) { return d <= 128 ? 64 : 32; }
__host__ __device__ constexpr int block_rows(int d) { return 128; }

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

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// The value of x held by lane (i ^ 32), combined with x by max or add: one
// v_permlane32_swap exchanges the two 32-lane halves of a wave.
__device__ __forceinline__ f32x2 halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float max_halves(float x) {
  const f32x2 v = halves(x);
  return fmaxf(v[0], v[1]);
}
__device__ __forceinline__ float sum_halves(float x) {
  const f32x2 v = halves(x);
  return v[0] + v[1];
}

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane i's bytes land at lds_addr + 16*i; lds_addr must be wave-uniform. Issued
// through inline asm so that the compiler does not order the tile being
// computed behind this prefetch; completion is awaited explicitly (dma_wait)
// before the barrier that publishes the tile.
__device__ __forceinline__ void dma16(const void* gsrc, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

// The same DMA from a wave-uniform base (held in scalar registers) plus a
// 32-bit per-lane byte offset: one vector register per lane instead of a
// 64-bit address, for kernels whose addresses would not stay in registers.
__device__ __forceinline__ void dma16_at(const void* base, unsigned lane_bytes, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(lane_bytes), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// V^T tile layout: BN keys of D head dims in fp16, stored as BN / 32 halves
// of 32 keys, each D rows (head dims) x 64 bytes of 16-byte chunks. Chunk c
// of a half holds its keys 16*(c/2) + 4*(c%2) + {0,1,2,3} and 16*(c/2) + 8 +
// 4*(c%2) + {0,1,2,3}: the key order in which the S^T accumulator hands P to
// the P.V contraction, so one 16-byte read is one MFMA operand. Chunks are
// XOR-swizzled by row so that the rows read together by an MFMA operand load
// fall on distinct banks. A 64-key tile is two 32-key tiles back to back, so
// kernels with 32-key tiles can read either half of it as a tile of their own.
constexpr int kVtRowBytes = 64;   // bytes per V^T row of a 32-key half
template <int BN, int D>
__device__ __forceinline__ int vt_chunk_offset(int d, int c) {
  static_assert(BN == 32 || BN == 64, "tile sizes");
  return (c >> 2) * (D * kVtRowBytes) + d * kVtRowBytes + (((c & 3) ^ ((d >> 2) & 3)) << 4);
}

// ---------------------------------------------------------------------------
// V -> fp16 V^T tiles. One thread transposes 8 keys x 8 dims: the 8 keys of
// one chunk (see vt_chunk_offset) for dims d0 .. d0+7.
// ---------------------------------------------------------------------------
constexpr int kPackThreads = 64;   // one wave per work-group: a few hundred of them fill the chip

template <int D, bool BF16>
__global__ void __launch_bounds__(kPackThreads)
vt_pack_kernel(const unsigned short* __restrict__ v, int64_t v_sb, int64_t v_ss, int64_t v_sh,
               int seqlen_kv, int n_heads_kv, int ntiles, unsigned short* __restrict__ ws) {
  constexpr int BN = tile_keys(D);
  constexpr int NCH = BN / 8;                        // chunks per V^T row
  constexpr int UNITS = NCH * (D / 8);               // (chunk, dim-group) units per tile
  const int u = blockIdx.x * kPackThreads + threadIdx.x;
  const int t = u / UNITS;
  if (t >= ntiles) return;
  const int c = (u % UNITS) % NCH;                   // chunk: its 8 keys
  const int d0 = ((u % UNITS) / NCH) * 8;            // dims d0 .. d0+7
  const int hk = blockIdx.y, b = blockIdx.z;
  const unsigned short* vp = v + (int64_t)b * v_sb + (int64_t)hk * v_sh + d0;
  u32x4 row[8];                                      // row[j] = 8 dims of key j of the chunk
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int key = t * BN + 16 * (c / 2) + 4 * (c % 2) + (j & 3) + 8 * (j >> 2);
    row[j] = key < seqlen_kv ? *(const u32x4*)(vp + (int64_t)key * v_ss) : u32x4{0, 0, 0, 0};
    if (BF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        row[j][e] = pack_f16x2(__uint_as_float(row[j][e] << 16),
                               __uint_as_float(row[j][e] & 0xffff0000u));
    }
  }
  char* out = (char*)(ws + (((int64_t)b * n_heads_kv + hk) * ntiles + t) * (int64_t)(D * BN));
#pragma unroll
  for (int e = 0; e < 4; ++e) {                      // dims d0+2e (lo halves) and d0+2e+1 (hi)
    u32x4 lo, hi;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[j] = __builtin_amdgcn_perm(row[2 * j + 1][e], row[2 * j][e], 0x05040100u);
      hi[j] = __builtin_amdgcn_perm(row[2 * j + 1][e], row[2 * j][e], 0x07060302u);
    }
    *(u32x4*)(out + vt_chunk_offset<BN, D>(d0 + 2 * e, c)) = lo;
    *(u32x4*)(out + vt_chunk_offset<BN, D>(d0 + 2 * e + 1, c)) = hi;
  }
}

// ---------------------------------------------------------------------------
// Work-group order. The dispatcher hands work-group i of a launch to XCD
// i % 8, and each XCD has its own L2. Work-groups are numbered so that (1)
// the query heads that read one KV head (one "group": a batch entry and a KV
// head) stay on as few XCDs as possible, so that group's K/V^T tiles are
// fetched into as few L2s as possible, and (2) on every XCD the longest
// causal blocks start first. With G groups: G a multiple of 8 gives each XCD
// G/8 whole groups; G dividing 8 spreads each group over 8/G XCDs (the
// group's blocks dealt out in longest-first order); any other G falls back
// to a plain longest-first order.
//
// Serial order (with S work-group slots per XCD): for G a multiple of 8 and
// a group's blocks at least S, each XCD takes its G/8 groups one after the
// other, each group's blocks longest first; for G dividing 8 the order above
// already runs one group per XCD. Work-groups started together read their
// K/V^T tiles in step, so the XCD's L2 serves one group's tiles at a time
// instead of interleaving groups that do not fit it together. The causal
// blocks of a round of S work-groups end at different times, so the next
// round starts one by one and (longest first) all of it ends together: every
// second round on an XCD walks its tiles from the last to the first, which
// puts its blocks in step again, reading the same tile at the same time.
// ---------------------------------------------------------------------------
__host__ __device__ inline int wg_count(int groups, int per_group, int nqb) {
  const int m = per_group * nqb;                     // work-groups of one group
  if (groups % 8 == 0 || 8 % groups != 0) return groups * m;
  const int s = 8 / groups;                          // XCDs per group
  return 8 * ((m + s - 1) / s);
}

struct WgItem {
  int b, hk, unit, qb;   // batch entry, KV head, unit of query heads in the group, query block
  bool valid;
  bool rev;              // walk the key tiles from the last to the first
};

// Whether a launch with `slots` work-group slots per XCD uses the serial
// order: more work-groups per XCD than one round of slots, and for G a
// multiple of 8 at least a round per group (host side; the kernel reads the
// slot count from PrefillArgs::wg_serial).
__host__ __device__ inline bool wg_serial_fits(int groups, int per_group, int nqb, int slots) {
  const int64_t per_g = (int64_t)per_group * nqb;
  if (groups % 8 == 0) return groups > 8 && per_g >= slots;
  if (8 % groups == 0) return per_g * groups / 8 > slots;
  return false;
}

// per_group: work units (sets of query heads) per group. serial_slots > 0:
// the serial order for that many work-group slots per XCD.
//
// rot_cus > 0 (two work-groups per compute unit, rot_cus compute units per
// XCD, a grid of at least two such rounds): the first work-groups of a launch
// land in a fixed pattern, position j of an XCD's sequence (id >> 3) on that
// XCD's compute unit j % rot_cus for j < 2 * rot_cus, so a compute unit's two
// first work-groups are positions j and j + rot_cus. In longest-first order
// that pairs the k-th longest block of each half, and the compute units
// holding the two longest pairs finish last while others idle. The second
// half of those positions is rotated by 5/16 of rot_cus (the ids stay a
// permutation of the same set), which decouples the two. In the serial order
// (whose first round is one group's blocks, longest first, followed by whole
// further groups) the second half of the first round is reversed instead, so
// that each compute unit starts with a long and a short block of that group.
__host__ __device__ inline WgItem wg_item(int id, int batch, int n_heads_kv, int per_group,
                                          int nqb, int serial_slots = 0, int rot_cus = 0) {
  if (rot_cus > 0 && serial_slots == 0) {
    const int j = id >> 3;
    if (j >= rot_cus && j < 2 * rot_cus)
      id = ((rot_cus + (j - rot_cus + (rot_cus * 5) / 16) % rot_cus) << 3) | (id & 7);
  }
  const int groups = batch * n_heads_kv;
  int g, u, rank;                                    // rank 0 = longest block
  bool valid = true, rev = false;
  if (serial_slots > 0 && groups % 8 == 0) {
    const int x = id & 7, j0 = id >> 3;
    const int j = rot_cus > 0 && j0 >= rot_cus && j0 < 2 * rot_cus ? 3 * rot_cus - 1 - j0 : j0;
    const int per_g = per_group * nqb;
    const int gi = j / per_g;                        // this XCD's gi-th group
    const int r = j - gi * per_g;
    rank = r / per_group;
    u = r % per_group;
    g = gi * 8 + x;
    rev = ((j / serial_slots) & 1) != 0;
  } else if (groups % 8 == 0) {
    const int x = id & 7, j = id >> 3;
    const int per_level = (groups >> 3) * per_group;
    rank = j / per_level;
    const int r = j - rank * per_level;
    g = (r / per_group) * 8 + x;
    u = r % per_group;
  } else if (8 % groups == 0) {
    const int s = 8 / groups, x = id & 7, j = id >> 3;
    g = x % groups;
    const int i = j * s + x / groups;
    valid = i < per_group * nqb;
    rank = i / per_group;
    u = i % per_group;
    rev = serial_slots > 0 && ((j / serial_slots) & 1) != 0;
  } else {
    const int per_level = groups * per_group;
    rank = id / per_level;
    const int r = id - rank * per_level;
    g = r / per_group;
    u = r % per_group;
  }
  WgItem w;
  w.b = g / n_heads_kv;
  w.hk = g % n_heads_kv;
  w.unit = u;
  w.qb = nqb - 1 - rank;
  w.valid = valid;
  w.rev = rev;
  return w;
}

// ---------------------------------------------------------------------------
// Attention forward.
// ---------------------------------------------------------------------------
// SPLIT: the work-group runs one unit of the key-split work order (sp): a whole
// query block, or the first or second half of a long block's key tiles. A
// half leaves its normalized partial O and LSE in the caller's scratch and the
// second half to finish merges the two (below, after the tile loop).
struct NoSplit {};
template <bool SPLIT> struct SplitArg { using type = NoSplit; };
template <> struct SplitArg<true> { using type = SplitPlan; };

// VROW: V tiles come straight from V's rows by DMA (fp16 only, head_dim <= 128)
// and each P.V operand is assembled from two LDS transpose reads, so no V^T
// pre-pass runs; otherwise they come from the V^T tiles the pre-pass wrote.
// XMAX: the exact running row max is kept, as un-normalized output and row
// sums need (a.unnorm picks the output form); without it the loop skips the
// per-tile max (the sum-checked base above).
// TRIO (head_dim 128, one query head per work-group): three work-groups per
// compute unit instead of two — 32-key tiles, no software pipeline, O staged
// in two halves — for grids of equal-length blocks that overflow one round of
// two per compute unit (see prefill_trio).
template <int D, bool BF16, bool XMAX, int HP, bool SPLIT, bool VROW = false, bool TRIO = false>
__global__ void __launch_bounds__(64 * wg_waves(D, HP))
__attribute__((amdgpu_waves_per_eu(TRIO ? 3 : 2, TRIO ? 3 : 2)))
prefill_kernel(PrefillArgs a, const unsigned short* __restrict__ vt_ws,
               typename SplitArg<SPLIT>::type sp) {
  static_assert(!VROW || (!BF16 && D <= 128), "V rows are read directly for fp16, head_dim <= 128");
  static_assert(!TRIO || (D == 128 && HP == 1 && !SPLIT && !VROW), "three-per-CU form");
  constexpr int kWaves = wg_waves(D, HP);
  constexpr bool PIPE = D <= 128 && !TRIO;   // software-pipelined loop (register budget)
  const bool unnorm = XMAX && a.unnorm != 0;
  constexpr int QG = 4;                      // query groups of 32 rows per head
  static_assert(kWaves == HP * QG, "work-group shape");
  constexpr int kBM = 32 * QG;               // query rows per work-group
  constexpr int BN = TRIO ? 32 : tile_keys(D);   // keys per tile
  constexpr int NKB = BN / 32;               // 32-key MFMA blocks per tile
  constexpr int NKS = BN / 16;               // MFMA k-steps of P.V per tile
  constexpr int NKK = D / 16;                // MFMA k-steps of Q.K^T
  constexpr int NDB = D / 32;                // 32-row blocks of O^T
  constexpr int KROW = D * 2;                // bytes per K row
  constexpr int KT = BN * KROW;              // bytes per K tile
  constexpr int VT = D * BN * 2;             // bytes per V^T tile
  constexpr int STAGE = KT + VT;
  constexpr int CPR = D / 8;                 // 16-byte chunks per K row
  constexpr int RPI = 64 / CPR;              // K rows per 1 KB DMA instruction
  constexpr int SWZ = CPR < 16 ? CPR - 1 : 15;
  // Two query heads per work-group (HP = 2): the second team of four waves
  // runs half a tile behind the first, so the two waves that share a SIMD
  // are in opposite phases (one turns S into P on the VALU while the other's
  // P.V keeps the matrix core busy). The leading team issues all the DMAs.
  // (The fp16 form that reads V rows keeps both teams in step: staggered, it
  // spills. The exact-max form keeps them in step too: staggered, it ran
  // 1-2 % slower.)
  constexpr bool STAG = HP == 2 && D <= 128 && !TRIO && !SPLIT && !VROW && !XMAX;
  constexpr int kDmaWaves = STAG ? QG : kWaves;
  constexpr int K_INSTR = KT / 1024 / kDmaWaves;   // DMA instructions per wave per tile
  constexpr int V_INSTR = VT / 1024 / kDmaWaves;
  static_assert(K_INSTR >= 1 && V_INSTR >= 1, "tile too small for the DMA split");
  // Row swizzle of V rows in LDS (VROW): one transpose read takes 64 bytes
  // (4 chunks) from each of 4 consecutive rows; XOR-ing the chunk index with
  // 4 * (row & 3) (256-byte rows) or 4 * ((row >> 1) & 1) (128-byte rows, two
  // per bank line) puts the four rows on distinct banks.
  constexpr auto vswz = [](int r) { return D == 64 ? 4 * ((r >> 1) & 1) : 4 * (r & 3); };

  // K/V^T tiles (two stages; three V^T stages with staggered teams); after
  // the loop, the per-wave O staging area (32 rows x D / OH fp32 per wave).
  constexpr int OH = D > 128 || TRIO ? 2 : 1;   // O rows staged in OH parts of D / OH dims
  constexpr int DP = D / OH;
  constexpr int OSTG = 32 * DP * 4;
  constexpr int RING = STAG ? 2 * KT + 3 * VT : 2 * STAGE;
  constexpr int LDS_BYTES = kWaves * OSTG > RING ? kWaves * OSTG : RING;
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qw = wave % QG;               // which 32 query rows
  const int hp = wave / QG;               // which query head of the work-group
  const int nqb = (a.seqlen_q + kBM - 1) / kBM;
  const int per_group = a.n_heads_q / a.n_heads_kv;
  int nunits = nqb;
  if constexpr (SPLIT) nunits = sp.n_units;
  const WgItem item = wg_item(blockIdx.x, a.batch, a.n_heads_kv, per_group / HP, nunits, a.wg_serial,
                              a.wg_rot);
  if (!item.valid) return;
  int qb = item.qb, half = -1;   // half: -1 whole block, else which half of its key tiles
  if constexpr (SPLIT) {
    const unsigned e = sp.units[nunits - 1 - item.qb];   // the unit of this rank
    qb = (int)(e & 0x3fffu);
    half = (int)(e >> 14) - 1;
  }
  const int b = item.b, hk = item.hk;
  const int h = hk * per_group + item.unit * HP + hp;   // the launcher picks HP | per_group
  const int q0 = qb * kBM;
  const int off = a.seqlen_kv - a.seqlen_q;              // bottom-right alignment

  const int n = lane & 31;    // MFMA column = this lane's query within the wave
  const int hh = lane >> 5;   // lane half
  const int qi = q0 + qw * 32 + n;
  const bool q_valid = qi < a.seqlen_q;
  const int qpos = qi + off;

  // Q^T operand: 8 consecutive dims of this lane's query per k-step. Loaded
  // after the first tile's DMA is issued so the two latencies overlap; the
  // registers are consumed right away so the compiler waits for them here and
  // not at their first use inside the tile loop (where that wait would also
  // stall on the prefetch DMA of the next tile).
  u32x4 qr[NKK];
  auto load_q = [&]() {
    const unsigned short* qp = (const unsigned short*)a.q + (int64_t)b * a.q_sb +
                               (int64_t)qi * a.q_ss + (int64_t)h * a.q_sh;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qr[kk] = q_valid ? *(const u32x4*)(qp + kk * 16 + hh * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) asm volatile("" ::"v"(qr[kk]));
  };

  // KV range: keys up to the largest query position of the block.
  // Keys this work-group may see: [kv_lo, kv_end). The causal bound and the
  // sequence's valid length cap the end; a sliding window raises the start
  // (for the block's first row). Tiles wholly outside are never touched; the
  // loop below runs over tiles tb .. tb + ntiles - 1.
  const int kv_len = a.kv_lens ? min(max(a.kv_lens[b], 0), a.seqlen_kv) : a.seqlen_kv;
  int kv_end = kv_len;
  if (a.causal) kv_end = min(kv_end, min(q0 + kBM, a.seqlen_q) + off);
  const int kv_lo = a.window > 0 ? max(0, q0 + off - a.window + 1) : 0;
  int tb = kv_lo / BN;
  int ntiles = kv_end > kv_lo ? (kv_end + BN - 1) / BN - tb : 0;
  if (SPLIT && half >= 0) {    // first half: tiles [0, n/2); second: [n/2, n)
    const int n0 = ntiles / 2;
    if (half == 0) {
      ntiles = n0;
    } else {
      tb += n0;
      ntiles -= n0;
    }
  }
  // V^T tiles as the pre-pass wrote them (tile_keys(D) keys each; the TRIO
  // form reads its 32-key tiles as halves of them).
  constexpr int BNP = tile_keys(D);
  constexpr int VTP = D * BNP * 2;
  const int ntiles_all = (a.seqlen_kv + BNP - 1) / BNP;
  const int wave_first_qpos = q0 + qw * 32 + off;
  // Absolute index of the t-th tile the loop visits (the serial order walks
  // every second group's tiles backwards; the online softmax takes the tiles
  // in any order).
  const int tstep = item.rev ? -1 : 1;
  const int tfirst = item.rev ? tb + ntiles - 1 : tb;
  auto tile = [&](int t) { return tfirst + tstep * t; };

  const unsigned short* kp =
      (const unsigned short*)a.k + (int64_t)b * a.k_sb + (int64_t)hk * a.k_sh;
  const char* vtp = (const char*)vt_ws + ((int64_t)b * a.n_heads_kv + hk) * ntiles_all * VTP;
  const unsigned short* vp =
      (const unsigned short*)a.v + (int64_t)b * a.v_sb + (int64_t)hk * a.v_sh;

  const unsigned lds_base = (unsigned)(uintptr_t)(lptr_t)lds;
  // Row addressing of the DMAs of whole tiles: one 64-bit multiply per tile
  // for this wave's first row, then a fixed step per instruction (RPI rows),
  // all in scalar registers.
  const int64_t k_row2 = a.k_ss * 2, v_row2 = a.v_ss * 2;           // bytes per K / V row
  const char* kp_w = (const char*)kp + (int64_t)wave * K_INSTR * RPI * k_row2;
  const char* vp_w = (const char*)vp + (int64_t)wave * V_INSTR * RPI * v_row2;
  const int64_t k_step = (int64_t)RPI * k_row2, v_step = (int64_t)RPI * v_row2;

  // DMA of this wave's share of the K rows / V^T bytes of tile tile(t) to LDS
  // offset dst. DMA instruction j of a wave writes rows R0 .. R0 + RPI - 1 of
  // the tile (R0 = (wave * K_INSTR + j) * RPI, wave-uniform); lane l takes row
  // R0 + l / CPR, logical chunk (l % CPR) ^ (row & SWZ). R0 is a multiple of
  // RPI, so row & SWZ = (R0 & SWZ) ^ ((l / CPR) & SWZ): the lane part of the
  // offset is the same for every j and the row base goes in scalar
  // registers. The lane parts are rebuilt per tile (a few VALU) rather than
  // held across the loop, which has no registers to spare for them. The
  // ragged last tile clamps each lane's row instead (rows past the end repeat
  // the last row; the mask zeroes them).
  auto issue_k = [&](int t, unsigned dst) {
    const int t0 = tile(t) * BN;
    unsigned ln = (unsigned)lane;
    asm volatile("" : "+v"(ln));
    const unsigned lrow = ln / CPR;
    const unsigned lc16 = ((ln % CPR) ^ (lrow & SWZ)) << 4;
    if (t0 + BN <= a.seqlen_kv) {
      const unsigned lrow_b = lrow * (unsigned)a.k_ss * 2u;   // < 2^31 (k_ss <= 2^23)
      const char* rb = kp_w + (int64_t)t0 * k_row2;
#pragma unroll
      for (int j = 0; j < K_INSTR; ++j) {
        const int r0 = (wave * K_INSTR + j) * RPI;
        dma16_at(rb, (lc16 ^ ((unsigned)(r0 & SWZ) << 4)) + lrow_b,
                 lds_base + dst + (wave * K_INSTR + j) * 1024);
        rb += k_step;
      }
    } else {
#pragma unroll
      for (int j = 0; j < K_INSTR; ++j) {
        const int r0 = (wave * K_INSTR + j) * RPI;
        const int key = min(t0 + r0 + (int)lrow, a.seqlen_kv - 1);
        dma16((const char*)(kp + (int64_t)key * a.k_ss) + (lc16 ^ ((unsigned)(r0 & SWZ) << 4)),
              lds_base + dst + (wave * K_INSTR + j) * 1024);
      }
    }
  };
  auto issue_v = [&](int t, unsigned dst) {
    if constexpr (VROW) {
      // V rows as K rows (same tile size, RPI rows per 1 KB DMA instruction);
      // lane p of an instruction stores its row's 16-byte chunk (p % CPR) ^
      // vswz(row) at position p, where vswz spreads the four rows that one
      // transpose read touches over distinct banks. The swizzle depends on the
      // row only through its offset inside the instruction, so the lane part of
      // the address is the same for every instruction of the tile.
      const int t0 = tile(t) * BN;
      unsigned ln = (unsigned)lane;
      asm volatile("" : "+v"(ln));
      const unsigned lrow = ln / CPR;
      const unsigned lc16 = ((ln % CPR) ^ (unsigned)vswz((int)lrow)) << 4;
      if (t0 + BN <= a.seqlen_kv) {
        const unsigned lrow_b = lrow * (unsigned)a.v_ss * 2u;   // < 2^31 (v_ss <= 2^23)
        const char* rb = vp_w + (int64_t)t0 * v_row2;
#pragma unroll
        for (int j = 0; j < V_INSTR; ++j) {
          dma16_at(rb, lc16 + lrow_b, lds_base + dst + (wave * V_INSTR + j) * 1024);
          rb += v_step;
        }
      } else {
#pragma unroll
        for (int j = 0; j < V_INSTR; ++j) {
          const int r0 = (wave * V_INSTR + j) * RPI;
          const int key = min(t0 + r0 + (int)lrow, a.seqlen_kv - 1);   // P = 0 past the end
          dma16((const char*)(vp + (int64_t)key * a.v_ss) + lc16,
                lds_base + dst + (wave * V_INSTR + j) * 1024);
        }
      }
      return;
    }
    unsigned ln = (unsigned)lane;
    asm volatile("" : "+v"(ln));
    if constexpr (TRIO) {
      // 32-key tile t is half t & 1 of 64-key pre-pass tile t / 2 (the halves
      // lie back to back in the same layout as a 32-key tile).
      static_assert(BNP == 64 && BN == 32 && VTP == 2 * VT, "halves of 64-key tiles");
      const int tt = tile(t);
      const char* base = vtp + (int64_t)(tt >> 1) * VTP + (tt & 1) * VT;
#pragma unroll
      for (int j = 0; j < V_INSTR; ++j) {
        const int J = wave * V_INSTR + j;
        dma16_at(base + J * 1024, ln << 4, lds_base + dst + J * 1024);
      }
      return;
    }
    const char* base = vtp + (int64_t)tile(t) * VT;
#pragma unroll
    for (int j = 0; j < V_INSTR; ++j) {
      const int J = wave * V_INSTR + j;
      dma16_at(base + J * 1024, ln << 4, lds_base + dst + J * 1024);
    }
  };

  // Loop-invariant LDS byte offsets of this lane's MFMA operands inside a stage.
  // (The K swizzle repeats every 16 rows, so block kb adds a constant kb*32 rows.)
  // The XOR swizzle touches only the low 4 bits of the chunk index, so k-step
  // kk >= 8 is k-step kk - 8 plus 16 chunks: 8 offsets serve any head dim.
  constexpr int NKO = NKK < 8 ? NKK : 8;
  int ka_off[NKO];
#pragma unroll
  for (int kk = 0; kk < NKO; ++kk) {
    ka_off[kk] = n * KROW + (((2 * kk + hh) ^ (n & SWZ)) << 4);
  }
  int va_off[NKS];   // + db * 32 rows for head-dim block db (the swizzle repeats every 16 rows)
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    va_off[ks] = vt_chunk_offset<BN, D>(n, ks * 2 + hh);
  // VROW: the byte offset, in a V-row stage, of this lane's first transpose read
  // for head-dim block db at k-step 0. Lane j of a 16-lane group g points at
  // the 4 dims m0 + 4 (j % 4) .. + 3 (m0 = 32 db + 16 (g & 1)) of key 4 hh +
  // j / 4: the read then hands lane j dim m0 + j of keys 4 hh + 0..3, and a
  // second read 8 keys further the keys 8 + 4 hh + 0..3, the key order of P.
  int vr_off[NDB];
  if constexpr (VROW) {
    const int g = lane >> 4, j = lane & 15;
    const int key = 4 * hh + (j >> 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int chunk = 4 * db + 2 * (g & 1) + ((j & 3) >> 1);
      vr_off[db] = key * KROW + ((chunk ^ vswz(key)) << 4) + 8 * (j & 1);
    }
  }

  float m_used = -1e30f;   // base of the exponentials (log2 units)
  float m_true = -1e30f;   // exact running row max (log2 units)
  float l = 0.0f;          // this lane's part of the row sum (relative to m_used - kShift)
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};

  // --- the phases of one tile for this wave --------------------------------
  // S^T = K . Q^T : rows = this wave's keys (M, in blocks of 32), columns = its
  // 32 queries (N). Independent accumulators per 32-key block.
  auto qk = [&](const char* kst, f32x16 (&s)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        s[kb] = mfma_qk<BF16>(
            *(const u32x4*)(kst + ka_off[kk % 8] + (kk / 8) * 256 + kb * 32 * KROW), qr[kk], s[kb]);
  };
  // Whether a tile straddles a bound of some row of this wave (causal diagonal,
  // valid length, window edge), i.e. needs the element mask.
  auto needs_mask = [&](int t0) -> bool {
    return (a.causal && t0 + BN - 1 > wave_first_qpos) || (t0 + BN > kv_len) ||
           (a.window > 0 && t0 <= wave_first_qpos + 31 - a.window);
  };
  // The element mask of a tile that straddles a bound.
  // Element i of block kb holds key t0 + kb*32 + (i/4)*8 + hh*4 + i%4.
  auto apply_mask = [&](f32x16 (&s)[NKB], int t0) {
    // visible: lo <= key offset <= hi, offsets relative to t0 + hh*4
    const int hi = min(a.causal ? qpos : INT_MAX, kv_len - 1) - t0 - hh * 4;
    const int lo = a.window > 0 ? qpos - a.window + 1 - t0 - hh * 4 : INT_MIN;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = kb * 32 + (i >> 2) * 8 + (i & 3);
        if (j > hi || j < lo) s[kb][i] = -INFINITY;
      }
  };
  // Row max of a (masked) tile, scaled to log2 units: straight-line VALU code
  // that can be scheduled among MFMAs.
  auto row_max = [&](const f32x16 (&s)[NKB]) -> float {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = (kb == 0 ? 1 : 0); i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = max_halves(mx);
    return mx * a.scale_log2;   // scale > 0: max commutes with the scaling
  };
  // The running max and (rarely) the move of the exponent base; returns the base.
  auto rebase = [&](float tmax) -> float {
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
    return m_used - kShift;
  };
  auto prep = [&](f32x16 (&s)[NKB], int t0) -> float {
    if (needs_mask(t0)) apply_mask(s, t0);
    return rebase(row_max(s));
  };
  // P = 2^(s*scale*log2e - base) <= 2^(kSlack + kShift) = 32768, packed to
  // fp16; returns this lane's sum of the tile's P.
  auto expo = [&](const f32x16 (&s)[NKB], float base, u32x4 (&pk)[NKS]) -> float {
    float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = exp2_fast(__builtin_fmaf(s[kb][i], a.scale_log2, -base));
        const float p1 = exp2_fast(__builtin_fmaf(s[kb][i + 1], a.scale_log2, -base));
        ls[(i >> 1) & 3] += p0 + p1;
        pk[kb * 2 + (i >> 3)][(i & 7) >> 1] = pack_f16x2(p0, p1);
      }
    return (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };
  // Max-free softmax (!XMAX): a lane's tile sum ts bounds each of its P. Above
  // the cap (or not a number: no base yet, it is still at -1e30) the base
  // moves to the row max and the tile is exponentiated again; after that
  // every P <= 2^kShift. Rare after a row's first visible tile.
  auto sum_check = [&](const f32x16 (&s)[NKB], float& base, float& ts, u32x4 (&pk)[NKS]) {
    if (__ballot(!(ts <= kSumCap))) {
      const float nm = fmaxf(m_used, row_max(s));
      const float corr = exp2_fast(m_used - nm);
      m_used = nm;
      l *= corr;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= corr;
      base = m_used - kShift;
      ts = expo(s, base, pk);
    }
  };
  // O^T += V^T . P^T over this wave's keys (key order matches the S^T layout).
  auto pv = [&](const char* vst, const u32x4 (&pk)[NKS]) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        u32x4 va;
        if constexpr (VROW) {
          typedef short s16x4 __attribute__((ext_vector_type(4)));
          typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
          const char* p0 = vst + vr_off[db] + ks * 16 * KROW;   // keys 16 ks + 4 hh + 0..3
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lptr_t)p0);
          const s16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lptr_t)(p0 + 8 * KROW));
          const auto l2 = __builtin_bit_cast(f32x2, lo), h2 = __builtin_bit_cast(f32x2, hi);
          va = u32x4{__float_as_uint(l2[0]), __float_as_uint(l2[1]), __float_as_uint(h2[0]),
                     __float_as_uint(h2[1])};
        } else {
          va = *(const u32x4*)(vst + va_off[ks] + db * 32 * kVtRowBytes);
        }
        oacc[db] = mfma_pv(va, pk[ks], oacc[db]);
      }
  };
  // Every wave computes every tile of the block, including key halves that
  // lie wholly above its queries (they come out as P = 0): all waves meet at
  // each tile's barrier, so skipping them would not shorten the tile, and
  // uniform control flow keeps the pipelined accumulators in place.
  if constexpr (PIPE) {
    // Software pipeline: while the VALU turns S(t) into P(t), the matrix core
    // computes S(t+1). LDS holds two K tiles and two V^T tiles: iteration t
    // reads K(t+1) and V(t) while K(t+2) and V(t+1) arrive.
    constexpr unsigned KST[2] = {0, KT};
    constexpr unsigned VST[2] = {2 * KT, 2 * KT + VT};
    f32x16 sa[NKB], sb[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sa[kb] = sb[kb] = f32x16{};   // row_max reads sb once unused
    // Staggered teams (STAG): the trailing team (hp = 1) meets the leading
    // team's end-of-tile barrier between its exponentials and its P.V, so it
    // runs P.V(t) while the leading team computes S(t+2) and P(t+1). K(t+2)
    // then overwrites K(t) only after both teams' S(t+1) (before that
    // barrier), and V(t) needs a third stage: the trailing team still reads
    // it while V(t+1) arrives and V(t+2) is issued.
    const bool lead = !STAG || hp == 0;
    auto vst_of = [&](int t) -> unsigned { return STAG ? 2 * KT + (t % 3) * VT : VST[t & 1]; };
    if (lead && ntiles > 0) { issue_k(0, KST[0]); issue_v(0, vst_of(0)); }
    if (lead && ntiles > 1) issue_k(1, KST[1]);
    load_q();
    dma_wait();
    __syncthreads();
    if (ntiles > 0) qk(lds + KST[0], sa);
    __syncthreads();   // K(0) is read everywhere before K(2) overwrites it
    float tm = 0.0f;   // row max of the next tile to exponentiate (log2 units)
    float base = m_used - kShift;
    if (ntiles > 0) {
      if (needs_mask(tile(0) * BN)) apply_mask(sa, tile(0) * BN);
      if constexpr (XMAX) tm = row_max(sa);
    }

    auto iter = [&](int t, auto parity, f32x16 (&cur)[NKB], f32x16 (&nxt)[NKB]) {
      constexpr int P = decltype(parity)::value;
      if (lead && t + 2 < ntiles) issue_k(t + 2, KST[P]);
      if constexpr (XMAX) base = rebase(tm);
      u32x4 pk[NKS];
      float ts;
      // S(t+1) = K(t+1).Q^T on the matrix cores while the VALU turns S(t)
      // into P(t). After the last tile the product is computed anyway, from
      // whatever the other K stage holds, and never used: a branch around it
      // would split this block, and the compiler then hoists the scaling FMAs
      // of the exponentials out of it, away from the MFMAs.
      qk(lds + KST[1 - P], nxt);
      ts = expo(cur, base, pk);
      // The packs of P stay among the MFMAs (the compiler would otherwise sink
      // them past the sum check below, whose rare branch rewrites P).
#pragma unroll
      for (int i = 0; i < NKS; ++i) asm volatile("" ::"v"(pk[i]));
      {
        // Interleave the S(t+1) MFMAs with the exponentials of tile t, with
        // each MFMA's LDS operand read issued three MFMAs ahead of it.
        constexpr int NQ = NKB * NKK, AHEAD = 3;
        __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);   // LDS reads
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
          if (i + AHEAD < NQ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);     // six VALU
        }
      }
      if constexpr (!XMAX) sum_check(cur, base, ts, pk);
      l += ts;
      if (STAG && !lead) __syncthreads();   // the trailing team's barrier (see above)
      // V(t+1) goes out here rather than with K(t+2): its stage held V(t-1),
      // long consumed, and issuing it mid-tile spreads the DMA over the tile.
      if (lead && t + 1 < ntiles) issue_v(t + 1, vst_of(t + 1));
      // P.V of tile t with the row max of tile t+1 interleaved (its base moves
      // at the top of the next step, after this P.V, as before); a straddling
      // tile t+1 is masked first. After the last tile the max is unused.
      if (t + 1 < ntiles && needs_mask(tile(t + 1) * BN)) apply_mask(nxt, tile(t + 1) * BN);
      pv(lds + (STAG ? vst_of(t) : VST[P]), pk);
      if constexpr (XMAX) tm = row_max(nxt);
      {
        // P.V: V^T operand reads four MFMAs ahead; the max's VALU among them.
        // (From V rows an operand takes two transposing reads.)
        constexpr int NP = NKS * NDB, AHEAD = 4, RD = VROW ? 2 : 1;
        __builtin_amdgcn_sched_group_barrier(0x100, AHEAD * RD, 1);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          if (i + AHEAD < NP) __builtin_amdgcn_sched_group_barrier(0x100, RD, 1);
          if constexpr (XMAX) __builtin_amdgcn_sched_group_barrier(0x002, 2, 1);
        }
      }
      if (lead) {
        dma_wait();        // this wave's part of K(t+2), V(t+1) has landed
        __syncthreads();   // ... everywhere; K(t+1) and V(t) may be overwritten next
      }
    };
    for (int t = 0; t < ntiles; t += 2) {
      iter(t, std::integral_constant<int, 0>{}, sa, sb);
      if (t + 1 < ntiles) iter(t + 1, std::integral_constant<int, 1>{}, sb, sa);
    }
    // Every wave meets the same number of barriers: two before the loop, one
    // per tile, and (staggered) this one, after which the trailing team's last
    // P.V is done with the LDS that the O staging reuses.
    if constexpr (STAG) __syncthreads();
  } else {
    // Plain double buffer: tile t+1 (K and V^T together) arrives while tile t
    // is computed from the other stage.
    constexpr unsigned ST_[2] = {0, STAGE};
    float lbase = m_used - kShift;   // the base of the max-free softmax
    auto step = [&](int t, auto stage) {
      constexpr int ST = decltype(stage)::value;
      if (t + 1 < ntiles) { issue_k(t + 1, ST_[1 - ST]); issue_v(t + 1, ST_[1 - ST] + KT); }
      f32x16 sc[NKB];
      qk(lds + ST_[ST], sc);
      {
        // Each MFMA's LDS operand read issued two MFMAs ahead of it (the
        // compiler otherwise waits on every read right before its MFMA; more
        // than two ahead costs registers this path does not have).
        constexpr int NQ = NKB * NKK, AHEAD = 2;
        __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 2);
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
          if (i + AHEAD < NQ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
        }
      }
      float base = lbase;
      if constexpr (XMAX) {
        base = prep(sc, tile(t) * BN);
      } else if (needs_mask(tile(t) * BN)) {
        apply_mask(sc, tile(t) * BN);
      }
      u32x4 pk[NKS];
      float ts = expo(sc, base, pk);
      if constexpr (!XMAX) sum_check(sc, lbase, ts, pk);
      l += ts;
      pv(lds + ST_[ST] + KT, pk);
      {
        constexpr int NP = NKS * NDB, AHEAD = 2;
        __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 3);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
          if (i + AHEAD < NP) __builtin_amdgcn_sched_group_barrier(0x100, 1, 3);
        }
      }
      dma_wait();        // this wave's part of tile t+1 has landed
      __syncthreads();   // tile t+1 landed everywhere; stage ST is free for reuse
    };
    if (ntiles > 0) { issue_k(0, ST_[0]); issue_v(0, ST_[0] + KT); }
    load_q();
    dma_wait();
    __syncthreads();
    for (int t = 0; t < ntiles; t += 2) {
      step(t, std::integral_constant<int, 0>{});
      if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{});
    }
  }

  const float lt = sum_halves(l);

  // Refer the outputs back to the true row max: factor = 2^((m_used - kShift) - m_true).
  const float base = m_used - kShift;    // the exponentials (and lt) are relative to 2^base
  float f, lse2, rsum;
  bool merged = false;
  if constexpr (SPLIT) {
    static_assert(!XMAX, "the key split merges normalized halves");
    __shared__ int split_last;
    if (half >= 0) {
      // This half's normalized partial, O_h = oacc / lt and LSE_h = base +
      // log2(lt) in log2 units (O_h = 0 and LSE_h = -inf for a row the half
      // sees no key of). Stored lane-ordered, element e of lane L of a wave at
      // e * 64 + L of the wave's 32 x D area, with agent-scope stores; the
      // second half to finish reads the other one back after the counter.
      const float fp = lt > 0.0f ? 1.0f / lt : 0.0f;
      const float lp = lt > 0.0f ? base + __log2f(lt) : -INFINITY;
      const int64_t blk = ((int64_t)b * a.n_heads_q + h) * nqb + qb;
      float* po = sp.o + ((blk * 2 + half) * kBM + qw * 32) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          __hip_atomic_store(po + (db * 16 + i) * 64 + lane, oacc[db][i] * fp, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      if (hh == 0)
        __hip_atomic_store(sp.lse + (blk * 2 + half) * kBM + qw * 32 + n, lp, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      // Count this half once its partial has reached memory; the second merges.
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0)
        split_last = __hip_atomic_fetch_add(sp.cnt + blk, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) == 1;
      __syncthreads();
      if (!split_last) return;
      // The other half's partial, read with agent-scope loads: an agent-scope
      // acquire fence would invalidate this XCD's whole L2, and with it the
      // K / V^T tiles the other work-groups on the XCD are streaming.
      const float* qo = sp.o + ((blk * 2 + (1 - half)) * kBM + qw * 32) * D;
      const float lo = __hip_atomic_load(sp.lse + (blk * 2 + (1 - half)) * kBM + qw * 32 + n,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // Merge with the first half always as the left operand, so the result
      // does not depend on which half finished last.
      const float la = half == 0 ? lp : lo, lb = half == 0 ? lo : lp;
      const float mm = fmaxf(la, lb);
      const float wa = mm == -INFINITY ? 0.0f : exp2_fast(la - mm);
      const float wb = mm == -INFINITY ? 0.0f : exp2_fast(lb - mm);
      const float ws = wa + wb;     // sum of the row's key terms relative to 2^mm
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float mine = oacc[db][i] * fp;
          const float other = __hip_atomic_load(qo + (db * 16 + i) * 64 + lane,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const float xa = half == 0 ? mine : other, xb = half == 0 ? other : mine;
          oacc[db][i] = wa * xa + wb * xb;
        }
      if (!a.sink_logits) {
        lse2 = ws > 0.0f ? mm + __log2f(ws) : -INFINITY;
        f = ws > 0.0f ? 1.0f / ws : 0.0f;
      } else {
        // the sink as one more term 2^sg, as in the unsplit case below
        const float sg = a.sink_logits[h] * kLog2e;
        const float lns = ws > 0.0f ? mm + __log2f(ws) : -INFINITY;
        const float mx = fmaxf(lns, sg);
        lse2 = mx == -INFINITY ? -INFINITY
                               : mx + __log2f(exp2_fast(lns - mx) + exp2_fast(sg - mx));
        f = ws > 0.0f ? exp2_fast(mm - lse2) : 0.0f;
      }
      rsum = 0.0f;   // the split is not used when row sums are requested
      if (tid == 0) __hip_atomic_store(sp.cnt + blk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      merged = true;
    }
  }
  if (merged) {
    // f and lse2 come from the merge of the two halves above
  } else if (!a.sink_logits) {
    const float to_true = exp2_fast(base - m_true);
    // a row with no visible key (length or window mask) has lt = 0: O = 0, LSE = -inf
    f = unnorm ? to_true : (lt > 0.0f ? 1.0f / lt : 0.0f);
    lse2 = base + __log2f(lt);
    rsum = lt * to_true;
  } else {
    // The sink joins the softmax as one more term 2^sg with no value row. The
    // output's reference max becomes max(m_true, sg); in normalized form the
    // factor is 2^(base - LSE), all in log2 units, so nothing overflows.
    const float sg = a.sink_logits[h] * kLog2e;
    const float lns = lt > 0.0f ? base + __log2f(lt) : -INFINITY;   // log2 of the key terms
    const float mx = fmaxf(lns, sg);
    lse2 = mx == -INFINITY ? -INFINITY   // no key and a sink at -inf
                           : mx + __log2f(exp2_fast(lns - mx) + exp2_fast(sg - mx));
    const float mr = fmaxf(m_true, sg);
    const float to_ref = lt > 0.0f ? exp2_fast(base - mr) : 0.0f;
    f = unnorm ? to_ref : (lt > 0.0f ? exp2_fast(base - lse2) : 0.0f);
    rsum = lt * to_ref + exp2_fast(sg - mr);
  }
  if (hh == 0 && q_valid) {
    const int64_t ri = ((int64_t)b * a.n_heads_q + h) * a.seqlen_q + qi;
    a.lse[ri] = lse2 * kLn2;
    if (XMAX && a.row_sum) a.row_sum[ri] = rsum;   // the launcher picks XMAX for row sums
  }

  // Stage this wave's 32 output rows in LDS ([row][D] fp32, 16-byte chunks
  // XOR-swizzled by row), then store whole rows: one store instruction then
  // writes 64 x 16 contiguous bytes instead of 16-byte pieces of 32 rows.
  // At head_dim 256 the rows go out in two halves of 128 dims, so the staging
  // area stays within the two tile stages (two work-groups per compute unit).
  // The area is this wave's own: its LDS writes and reads stay in order.
  constexpr int CPRO = DP / 4;                             // 16-byte chunks per staged row
  constexpr int OSW = CPRO < 32 ? CPRO - 1 : 31;
  float* stg = (float*)(lds + wave * OSTG);
  const int row_base = q0 + qw * 32;
  float* obase = a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh;
#pragma unroll
  for (int part = 0; part < OH; ++part) {
#pragma unroll
    for (int db = part * (NDB / OH); db < (part + 1) * (NDB / OH); ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int chunk = (db * 32 - part * DP + g * 8 + hh * 4) / 4;
        *(f32x4*)(stg + n * DP + ((chunk ^ (n & OSW)) << 2)) =
            f32x4{oacc[db][4 * g] * f, oacc[db][4 * g + 1] * f, oacc[db][4 * g + 2] * f,
                  oacc[db][4 * g + 3] * f};
      }
#pragma unroll
    for (int it = 0; it < 32 * CPRO / 64; ++it) {
      const int idx = it * 64 + lane;
      const int r = idx / CPRO, c = idx % CPRO;
      const f32x4 val = *(const f32x4*)(stg + r * DP + ((c ^ (r & OSW)) << 2));
      if (row_base + r < a.seqlen_q)
        *(f32x4*)(obase + (int64_t)(row_base + r) * a.o_ss + part * DP + c * 4) = val;
    }
  }
}

// ---------------------------------------------------------------------------
// Attention forward at head_dim 512 ("STAGE_D.md — FMHA Kernel Development",
// D1.4: a 512-wide head overflows the on-chip budget that fits the narrower
// heads; of the page's options this kernel splits the contraction dimension
// of Q.K^T). A wave cannot hold 32 query rows of Q and of the fp32 output at
// 512 dims in its 256 registers, so the two waves of a pair split the head
// dimension: each holds Q and O for 256 dims and computes the partial S^T
// over them, the pair adds the two partials through LDS (a + b = b + a in
// fp32, so both waves hold bitwise the same S), both run the same online
// softmax, and each multiplies P into its half of V. 8 waves = 4 query groups
// of 32 rows x 2 halves; 32-key tiles; LDS: two stages of K (32 KB) and V^T
// (32 KB) plus 32 KB of partial scores, the 160 KB of a compute unit.
// ---------------------------------------------------------------------------
template <bool BF16, bool UNNORM>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill512_kernel(PrefillArgs a, const unsigned short* __restrict__ vt_ws) {
  constexpr int D = 512, DH = 256;           // head dim; dims per wave
  constexpr int QG = 4;                      // query groups of 32 rows
  constexpr int kBM = 32 * QG;               // query rows per work-group
  constexpr int BN = tile_keys(D);           // keys per tile
  static_assert(BN == 32, "one 32-key MFMA block per tile");
  constexpr int NKK = DH / 16;               // MFMA k-steps of the partial Q.K^T
  constexpr int NDB = DH / 32;               // 32-row blocks of this wave's O^T
  constexpr int NKS = BN / 16;               // MFMA k-steps of P.V
  constexpr int KROW = D * 2;                // bytes per K row (one DMA instruction)
  constexpr int KT = BN * KROW;
  constexpr int VT = D * BN * 2;
  constexpr int STAGE = KT + VT;
  constexpr int K_INSTR = BN / 8;            // K rows per wave per tile
  constexpr int V_INSTR = VT / 1024 / 8;
  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE + 8 * 16 * 64 * 4];
  float* xch = (float*)(lds + 2 * STAGE);    // [wave][element/4][lane][4] partial S^T

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qw = wave % QG;                  // which 32 query rows
  const int dh = wave / QG;                  // which half of the head dims
  const int nqb = (a.seqlen_q + kBM - 1) / kBM;
  const int per_group = a.n_heads_q / a.n_heads_kv;
  const WgItem item = wg_item(blockIdx.x, a.batch, a.n_heads_kv, per_group, nqb, a.wg_serial);
  if (!item.valid) return;
  const int qb = item.qb, b = item.b, hk = item.hk;
  const int h = hk * per_group + item.unit;
  const int q0 = qb * kBM;
  const int off = a.seqlen_kv - a.seqlen_q;  // bottom-right alignment

  const int n = lane & 31;    // MFMA column = this lane's query within the wave
  const int hh = lane >> 5;   // lane half
  const int qi = q0 + qw * 32 + n;
  const bool q_valid = qi < a.seqlen_q;
  const int qpos = qi + off;

  u32x4 qr[NKK];              // Q^T operand: this lane's query, this wave's dims
  auto load_q = [&]() {
    const unsigned short* qp = (const unsigned short*)a.q + (int64_t)b * a.q_sb +
                               (int64_t)qi * a.q_ss + (int64_t)h * a.q_sh + dh * DH;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qr[kk] = q_valid ? *(const u32x4*)(qp + kk * 16 + hh * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) asm volatile("" ::"v"(qr[kk]));
  };

  // Keys this work-group may see, as in prefill_kernel: [kv_lo, kv_end).
  const int kv_len = a.kv_lens ? min(max(a.kv_lens[b], 0), a.seqlen_kv) : a.seqlen_kv;
  int kv_end = kv_len;
  if (a.causal) kv_end = min(kv_end, min(q0 + kBM, a.seqlen_q) + off);
  const int kv_lo = a.window > 0 ? max(0, q0 + off - a.window + 1) : 0;
  const int tb = kv_lo / BN;
  const int ntiles = kv_end > kv_lo ? (kv_end + BN - 1) / BN - tb : 0;
  const int ntiles_all = (a.seqlen_kv + BN - 1) / BN;
  const int wave_first_qpos = q0 + qw * 32 + off;
  // Absolute index of the t-th tile visited (backwards in every second round
  // of the serial order).
  const int tstep = item.rev ? -1 : 1;
  const int tfirst = item.rev ? tb + ntiles - 1 : tb;
  auto tile = [&](int t) { return tfirst + tstep * t; };

  const unsigned short* kp =
      (const unsigned short*)a.k + (int64_t)b * a.k_sb + (int64_t)hk * a.k_sh;
  const char* vtp = (const char*)vt_ws + ((int64_t)b * a.n_heads_kv + hk) * ntiles_all * VT;
  const unsigned lds_base = (unsigned)(uintptr_t)(lptr_t)lds;

  // DMA of tile tile(t) into the stage at LDS offset st. K: one 1 KB row per
  // instruction; lane p stores the row's 16-byte chunk p ^ (row & 15) at
  // position p (the swizzle that spreads an operand load over the banks).
  auto issue = [&](int t, unsigned st) {
    const int t0 = tile(t) * BN;
    // Recomputed per tile (one XOR each) rather than held across the loop:
    // the loop has no registers to spare for four offsets.
    unsigned lane16 = (unsigned)lane << 4;
    asm volatile("" : "+v"(lane16));
#pragma unroll
    for (int j = 0; j < K_INSTR; ++j) {
      const int r = wave * K_INSTR + j;
      const int key = min(t0 + r, a.seqlen_kv - 1);   // rows past the end: masked below
      dma16_at(kp + (int64_t)key * a.k_ss, lane16 ^ ((unsigned)(r & 15) << 4),
               lds_base + st + r * KROW);
    }
#pragma unroll
    for (int j = 0; j < V_INSTR; ++j) {
      const int J = wave * V_INSTR + j;
      dma16_at(vtp + (int64_t)tile(t) * VT + J * 1024, (unsigned)lane << 4,
               lds_base + st + KT + J * 1024);
    }
  };

  // Operand offsets: K row n, logical chunk dh*32 + 2*kk + hh (the XOR only
  // touches the low 4 bits of the chunk index, so it is split off per kk % 8).
  int ka8[8];
#pragma unroll
  for (int k8 = 0; k8 < 8; ++k8) ka8[k8] = n * KROW + (((2 * k8 + hh) ^ (n & 15)) << 4);
  int va_off[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) va_off[ks] = dh * DH * kVtRowBytes + vt_chunk_offset<BN, 512>(n, 2 * ks + hh);

  float m_used = -1e30f, m_true = -1e30f, l = 0.0f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};

  // Each MFMA's LDS operand read is issued one MFMA ahead of it (left alone,
  // the compiler waits on every read right before its MFMA; two ahead needs
  // registers this kernel does not have).
  auto qk = [&](const char* kst, f32x16& s) {
    s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      s = mfma_qk<BF16>(*(const u32x4*)(kst + ka8[kk % 8] + (dh * 32 + (kk / 8) * 16) * 16),
                        qr[kk], s);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < NKK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + 1 < NKK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  // Mask, row max and (rarely) the move of the exponent base, as in prefill_kernel.
  auto prep = [&](f32x16& s, int t0) -> float {
    const bool need_mask = (a.causal && t0 + BN - 1 > wave_first_qpos) || (t0 + BN > kv_len) ||
                           (a.window > 0 && t0 <= wave_first_qpos + 31 - a.window);
    if (need_mask) {
      const int hi = min(a.causal ? qpos : INT_MAX, kv_len - 1) - t0 - hh * 4;
      const int lo = a.window > 0 ? qpos - a.window + 1 - t0 - hh * 4 : INT_MIN;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = (i >> 2) * 8 + (i & 3);
        if (j > hi || j < lo) s[i] = -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = max_halves(mx);
    const float tmax = mx * a.scale_log2;
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
    return m_used - kShift;
  };
  auto expo = [&](const f32x16& s, float base, u32x4 (&pk)[NKS]) {
    float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = exp2_fast(__builtin_fmaf(s[i], a.scale_log2, -base));
      const float p1 = exp2_fast(__builtin_fmaf(s[i + 1], a.scale_log2, -base));
      ls[(i >> 1) & 3] += p0 + p1;
      pk[i >> 3][(i & 7) >> 1] = pack_f16x2(p0, p1);
    }
    l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };
  auto pv = [&](const char* vst, const u32x4 (&pk)[NKS]) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = mfma_pv(*(const u32x4*)(vst + va_off[ks] + db * 32 * kVtRowBytes), pk[ks],
                           oacc[db]);
    constexpr int NP = NKS * NDB;
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      if (i + 1 < NP) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
  };

  // Plain double buffer: tile t+1 arrives while tile t is computed. Two
  // barriers per tile: one publishes the partial scores, one publishes tile
  // t+1 and frees tile t's stage (and the score area).
  constexpr unsigned ST_[2] = {0, STAGE};
  auto step = [&](int t, auto stage) {
    constexpr int ST = decltype(stage)::value;
    if (t + 1 < ntiles) issue(t + 1, ST_[1 - ST]);
    f32x16 s;
    qk(lds + ST_[ST], s);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *(f32x4*)(xch + (wave * 4 + c) * 256 + lane * 4) = f32x4{s[4 * c], s[4 * c + 1],
                                                              s[4 * c + 2], s[4 * c + 3]};
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 p = *(const f32x4*)(xch + ((wave ^ 4) * 4 + c) * 256 + lane * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * c + e] += p[e];
    }
    const float base = prep(s, tile(t) * BN);
    u32x4 pk[NKS];
    expo(s, base, pk);
    pv(lds + ST_[ST] + KT, pk);
    dma_wait();
    __syncthreads();
  };
  if (ntiles > 0) issue(0, ST_[0]);
  load_q();
  dma_wait();
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{});
  }

  const float lt = sum_halves(l);
  const float base = m_used - kShift;
  float f, lse2, rsum;
  if (!a.sink_logits) {
    const float to_true = exp2_fast(base - m_true);
    f = UNNORM ? to_true : (lt > 0.0f ? 1.0f / lt : 0.0f);
    lse2 = base + __log2f(lt);
    rsum = lt * to_true;
  } else {
    const float sg = a.sink_logits[h] * kLog2e;
    const float lns = lt > 0.0f ? base + __log2f(lt) : -INFINITY;
    const float mx = fmaxf(lns, sg);
    lse2 = mx == -INFINITY ? -INFINITY
                           : mx + __log2f(exp2_fast(lns - mx) + exp2_fast(sg - mx));
    const float mr = fmaxf(m_true, sg);
    const float to_ref = lt > 0.0f ? exp2_fast(base - mr) : 0.0f;
    f = UNNORM ? to_ref : (lt > 0.0f ? exp2_fast(base - lse2) : 0.0f);
    rsum = lt * to_ref + exp2_fast(sg - mr);
  }
  if (!q_valid) return;
  if (dh == 0 && hh == 0) {
    const int64_t ri = ((int64_t)b * a.n_heads_q + h) * a.seqlen_q + qi;
    a.lse[ri] = lse2 * kLn2;
    if (a.row_sum) a.row_sum[ri] = rsum;
  }
  // O row qi, dims dh*256 + db*32 + g*8 + hh*4 + {0..3}: 16-byte stores.
  float* orow = a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)qi * a.o_ss + dh * DH;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(f32x4*)(orow + db * 32 + g * 8 + hh * 4) =
          f32x4{oacc[db][4 * g] * f, oacc[db][4 * g + 1] * f, oacc[db][4 * g + 2] * f,
                oacc[db][4 * g + 3] * f};
}

template <int D, bool BF16>
hipError_t launch_pack_d(const PrefillArgs& a, const VtArgs& w, hipStream_t stream) {
  constexpr int BN = tile_keys(D);
  const int ntiles = (int)(((int64_t)a.seqlen_kv + BN - 1) / BN);   // seqlen_kv <= 2^30
  const int64_t units = (int64_t)ntiles * (BN / 8) * (D / 8);
  hipLaunchKernelGGL((vt_pack_kernel<D, BF16>),
                     dim3((unsigned)((units + kPackThreads - 1) / kPackThreads), a.n_heads_kv,
                          a.batch),
                     dim3(kPackThreads), 0, stream, (const unsigned short*)a.v, a.v_sb, a.v_ss, a.v_sh,
                     a.seqlen_kv, a.n_heads_kv, ntiles, (unsigned short*)w.ws);
  return hipGetLastError();
}

// wg_item's first-round rotation (or, in the serial order, reversal) for a
// launch of two work-groups per compute unit (32 compute units per XCD): on
// when the grid fills both first rounds.
inline int first_round_rotation(unsigned grid) {
  constexpr int kCusPerXcd = 32;
  return grid >= 2u * kCusPerXcd * 8 ? kCusPerXcd : 0;
}

template <int D, bool BF16>
hipError_t launch_attn_d(const PrefillArgs& a0, const VtArgs& w, bool unnorm, hipStream_t stream) {
  constexpr int BM = block_rows(D);
  const int per_group = a0.n_heads_q / a0.n_heads_kv;
  const int nqb = (a0.seqlen_q + BM - 1) / BM;
  PrefillArgs a = a0;
  // head_dim 256: one group's K/V^T (2 x 512 bytes per key) outgrows an XCD's
  // L2 at a few thousand keys, so its groups run one at a time per XCD.
  constexpr int kSlots = 32 * 2;   // two work-groups per compute unit
  a.wg_serial = D == 256 && wg_serial_fits(a.batch * a.n_heads_kv, per_group, nqb, kSlots) ? kSlots : 0;
  a.unnorm = unnorm;
  const bool xmax = unnorm || a.row_sum;   // the exact row max is kept for these outputs
  const auto go = [&](auto hp_c, auto trio_c) {
    constexpr int HP = decltype(hp_c)::value;
    constexpr bool TRIO = decltype(trio_c)::value;
    const dim3 grid(wg_count(a.batch * a.n_heads_kv, per_group / HP, nqb));
    a.wg_rot = HP == 1 && !TRIO ? first_round_rotation(grid.x) : 0;
    if (xmax)
      hipLaunchKernelGGL((prefill_kernel<D, BF16, true, HP, false, false, TRIO>), grid,
                         dim3(64 * wg_waves(D, HP)), 0, stream, a, (const unsigned short*)w.ws,
                         NoSplit{});
    else
      hipLaunchKernelGGL((prefill_kernel<D, BF16, false, HP, false, false, TRIO>), grid,
                         dim3(64 * wg_waves(D, HP)), 0, stream, a, (const unsigned short*)w.ws,
                         NoSplit{});
  };
  using no = std::false_type;
  if constexpr (D <= 128) {
    if (per_group % 2 == 0) {
      go(std::integral_constant<int, 2>{}, no{});
      return hipGetLastError();
    }
  }
  if constexpr (D == 128) {
    if (prefill_trio(a.batch, a.seqlen_q, a.seqlen_kv, a.n_heads_q, a.n_heads_kv, D, a.causal,
                     a.window)) {
      go(std::integral_constant<int, 1>{}, std::true_type{});
      return hipGetLastError();
    }
  }
  go(std::integral_constant<int, 1>{}, no{});
  return hipGetLastError();
}

// The attention launch reading V's rows directly (fp16, head_dim <= 128).
template <int D>
hipError_t launch_attn_vrow_d(const PrefillArgs& a0, bool unnorm, hipStream_t stream) {
  constexpr int BM = block_rows(D);
  const int per_group = a0.n_heads_q / a0.n_heads_kv;
  const int nqb = (a0.seqlen_q + BM - 1) / BM;
  PrefillArgs a = a0;
  a.unnorm = unnorm;
  const bool xmax = unnorm || a.row_sum;   // the exact row max is kept for these outputs
  const auto go = [&](auto hp_c) {
    constexpr int HP = decltype(hp_c)::value;
    const dim3 grid(wg_count(a.batch * a.n_heads_kv, per_group / HP, nqb));
    a.wg_rot = HP == 1 ? first_round_rotation(grid.x) : 0;
    if (xmax)
      hipLaunchKernelGGL((prefill_kernel<D, false, true, HP, false, true>), grid,
                         dim3(64 * wg_waves(D, HP)), 0, stream, a, nullptr, NoSplit{});
    else
      hipLaunchKernelGGL((prefill_kernel<D, false, false, HP, false, true>), grid,
                         dim3(64 * wg_waves(D, HP)), 0, stream, a, nullptr, NoSplit{});
  };
  if (per_group % 2 == 0)
    go(std::integral_constant<int, 2>{});
  else
    go(std::integral_constant<int, 1>{});
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_split_d(const PrefillArgs& a, const VtArgs& w, const SplitPlan& sp,
                          hipStream_t stream) {
  const int per_group = a.n_heads_q / a.n_heads_kv;
  const auto go = [&](auto hp_c) {
    constexpr int HP = decltype(hp_c)::value;
    const dim3 grid(wg_count(a.batch * a.n_heads_kv, per_group / HP, sp.n_units));
    hipLaunchKernelGGL((prefill_kernel<D, BF16, false, HP, true>), grid,
                       dim3(64 * wg_waves(D, HP)), 0, stream, a, (const unsigned short*)w.ws, sp);
  };
  if constexpr (D <= 128) {
    if (per_group % 2 == 0) {
      go(std::integral_constant<int, 2>{});
      return hipGetLastError();
    }
  }
  go(std::integral_constant<int, 1>{});
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_attn_512(const PrefillArgs& a0, const VtArgs& w, bool unnorm, hipStream_t stream) {
  const int per_group = a0.n_heads_q / a0.n_heads_kv;
  const int nqb = (a0.seqlen_q + 127) / 128;
  PrefillArgs a = a0;
  // One work-group per compute unit; the K/V^T of a group (2 x 1 KB per key)
  // outgrows an XCD's L2 at a few thousand keys.
  constexpr int kSlots = 32;
  a.wg_serial = wg_serial_fits(a.batch * a.n_heads_kv, per_group, nqb, kSlots) ? kSlots : 0;
  const dim3 grid(wg_count(a.batch * a.n_heads_kv, per_group, nqb));
  if (unnorm)
    hipLaunchKernelGGL((prefill512_kernel<BF16, true>), grid, dim3(512), 0, stream, a,
                       (const unsigned short*)w.ws);
  else
    hipLaunchKernelGGL((prefill512_kernel<BF16, false>), grid, dim3(512), 0, stream, a,
                       (const unsigned short*)w.ws);
  return hipGetLastError();
}

}  // namespace

size_t prefill_workspace_bytes(int batch, int seqlen_kv, int n_heads_kv, int head_dim) {
  if (batch <= 0 || seqlen_kv <= 0 || n_heads_kv <= 0 || head_dim <= 0) return 0;
  const size_t bn = tile_keys(head_dim);
  const size_t ntiles = ((size_t)seqlen_kv + bn - 1) / bn;
  return sat_mul(sat_mul(sat_mul((size_t)batch, (size_t)n_heads_kv), sat_mul(ntiles, bn)),
                 (size_t)head_dim * 2);
}

SplitLayout prefill_split_layout(int batch, int seqlen_q, int n_heads_q, int head_dim) {
  SplitLayout L{};
  if (batch <= 0 || seqlen_q <= 0 || n_heads_q <= 0 || head_dim <= 0) return L;
  const size_t blocks =
      sat_mul(sat_mul((size_t)batch, (size_t)n_heads_q), ((size_t)seqlen_q + 127) / 128);
  L.cnt = 0;                      // fixed for every shape (see kSplitCounterBytes)
  L.lse = kSplitCounterBytes;
  L.o = sat_add(L.lse, sat_up256(sat_mul(blocks, 2 * 128 * 4)));
  L.total = sat_add(L.o, sat_mul(sat_mul(blocks, 2 * 128 * 4), (size_t)head_dim));
  return L;
}

namespace {

// End time of handing out the units in list order, `copies` work-groups per
// unit, each to the earliest free of `slots` work-group slots (time in tiles).
double list_makespan(const std::vector<double>& sizes, int64_t copies, int slots) {
  std::priority_queue<double, std::vector<double>, std::greater<double>> q;
  for (int i = 0; i < slots; ++i) q.push(0.0);
  double end = 0.0;
  for (const double u : sizes)
    for (int64_t c = 0; c < copies; ++c) {
      const double t = q.top() + u;
      q.pop();
      q.push(t);
      end = std::max(end, t);
    }
  return end;
}

struct PlanKey {
  int batch, seqlen_q, seqlen_kv, n_heads_q, n_heads_kv, head_dim, causal, window;
  bool operator==(const PlanKey& o) const {
    return batch == o.batch && seqlen_q == o.seqlen_q && seqlen_kv == o.seqlen_kv &&
           n_heads_q == o.n_heads_q && n_heads_kv == o.n_heads_kv && head_dim == o.head_dim &&
           causal == o.causal && window == o.window;
  }
};
struct PlanEntry {
  PlanKey key;
  int n_units;
  std::vector<unsigned short> units;
};

int plan_units(const PlanKey& k, unsigned short* units) {
  const int D = k.head_dim;
  if (D != 64 && D != 128) return 0;
  const int bm = 128, bn = tile_keys(D);
  const int64_t nqb64 = ((int64_t)k.seqlen_q + bm - 1) / bm;
  if (nqb64 <= 0 || nqb64 > 0x3fff || k.seqlen_kv > (1 << 30)) return 0;
  const int nqb = (int)nqb64;
  // one arrival counter per query block of every (batch entry, query head)
  if ((int64_t)k.batch * k.n_heads_q * nqb > kSplitCounters) return 0;
  // key tiles per query block, as the kernel counts them at full lengths
  const int off = k.seqlen_kv - k.seqlen_q;
  std::vector<int> tiles(nqb);
  for (int qb = 0; qb < nqb; ++qb) {
    const int q0 = qb * bm;
    int kv_end = k.seqlen_kv;
    if (k.causal) kv_end = std::min(kv_end, std::min(q0 + bm, k.seqlen_q) + off);
    const int kv_lo = k.window > 0 ? std::max(0, q0 + off - k.window + 1) : 0;
    tiles[qb] = kv_end > kv_lo ? (kv_end + bn - 1) / bn - kv_lo / bn : 0;
  }
  const int per_group = k.n_heads_q / k.n_heads_kv;
  const int hp = (D <= 128 && per_group % 2 == 0) ? 2 : 1;
  const int slots = kDecodeCus * 8 / wg_waves(D, hp);          // two waves per SIMD
  const int64_t copies = (int64_t)k.batch * k.n_heads_kv * (per_group / hp);
  // What a half costs beyond its tiles, in tile times: its own prologue (Q and
  // the first tiles in flight), storing its partial, the counter and the
  // merge. Fitted to measured split / unsplit times of the causal and the
  // windowed 3314-token prompt (the model ignores that a work-group alone on
  // its compute unit runs faster, so it overstates the tail it removes).
  constexpr double kHalfCost = 6.0;

  // Candidate: split every block of more than `thr` tiles; units longest first
  // (a half's length includes its extra cost).
  struct Unit { double size; unsigned short e; };
  const auto build = [&](int thr, std::vector<Unit>& list) {
    list.clear();
    for (int qb = nqb - 1; qb >= 0; --qb) {
      const int n = tiles[qb];
      if (n > thr && n >= 2) {
        list.push_back({n / 2 + kHalfCost, (unsigned short)(qb | 1 << 14)});
        list.push_back({n - n / 2 + kHalfCost, (unsigned short)(qb | 2 << 14)});
      } else {
        list.push_back({(double)n, (unsigned short)qb});
      }
    }
    std::stable_sort(list.begin(), list.end(),
                     [](const Unit& x, const Unit& y) { return x.size > y.size; });
  };
  const auto cost = [&](const std::vector<Unit>& list) {
    std::vector<double> sz;
    sz.reserve(list.size());
    for (const Unit& u : list) sz.push_back(u.size);
    return list_makespan(sz, copies, slots);
  };
  std::vector<Unit> list, best;
  build(INT_MAX, list);
  const double none = cost(list);
  // Only a launch whose longest blocks far outlast the average slot's work is
  // worth splitting: one round of very unequal blocks (few heads, a long
  // prompt). Measured: 8 heads x 8192 tokens gains 12 % (modeled end 2.0x the
  // average); the 28-head 3314-token prompt (1.35x) lost 6 % with its three
  // longest blocks split, since a work-group alone on its compute unit runs
  // ~1.7x faster and the tail costs less than the model says.
  double total = 0.0;
  for (const Unit& u : list) total += u.size;
  if (none < 1.5 * total * copies / slots) return 0;
  double best_cost = none;
  std::vector<int> cands(tiles);
  std::sort(cands.begin(), cands.end());
  cands.erase(std::unique(cands.begin(), cands.end()), cands.end());
  for (const int thr : cands) {
    build(thr, list);
    if ((int)list.size() > kMaxSplitUnits || (int)list.size() == nqb) continue;
    const double c = cost(list);
    if (c < best_cost) {
      best_cost = c;
      best = list;
    }
  }
  if (best.empty() || best_cost > 0.95 * none) return 0;
  for (size_t i = 0; i < best.size(); ++i) units[i] = best[i].e;
  return (int)best.size();
}

}  // namespace

int prefill_split_units(int batch, int seqlen_q, int seqlen_kv, int n_heads_q, int n_heads_kv,
                        int head_dim, int causal, int window, unsigned short* units) {
  if (batch <= 0 || seqlen_q <= 0 || seqlen_kv <= 0 || n_heads_q <= 0 || n_heads_kv <= 0 ||
      n_heads_q % n_heads_kv != 0)
    return 0;
  const PlanKey key{batch, seqlen_q, seqlen_kv, n_heads_q, n_heads_kv, head_dim, causal != 0,
                    window > 0 ? window : 0};
  // The plan is a pure function of the shape; the last few are kept.
  static std::mutex mu;
  static PlanEntry cache[8];
  static int filled = 0, next = 0;
  {
    std::lock_guard<std::mutex> g(mu);
    for (int i = 0; i < filled; ++i)
      if (cache[i].key == key) {
        std::copy(cache[i].units.begin(), cache[i].units.end(), units);
        return cache[i].n_units;
      }
  }
  const int n = plan_units(key, units);
  std::lock_guard<std::mutex> g(mu);
  PlanEntry& e = cache[next];
  e.key = key;
  e.n_units = n;
  e.units.assign(units, units + n);
  next = (next + 1) % 8;
  filled = std::min(filled + 1, 8);
  return n;
}

hipError_t launch_prefill_attn_split(const PrefillArgs& a, const VtArgs& w, const SplitPlan& sp,
                                     int head_dim, bool bf16, hipStream_t stream) {
  switch (head_dim) {
    case 64:
      return bf16 ? launch_split_d<64, true>(a, w, sp, stream)
                  : launch_split_d<64, false>(a, w, sp, stream);
    case 128:
      return bf16 ? launch_split_d<128, true>(a, w, sp, stream)
                  : launch_split_d<128, false>(a, w, sp, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_pack(const PrefillArgs& a, const VtArgs& w, int head_dim, bool bf16,
                               hipStream_t stream) {
  switch (head_dim) {
    case 64: return bf16 ? launch_pack_d<64, true>(a, w, stream) : launch_pack_d<64, false>(a, w, stream);
    case 128: return bf16 ? launch_pack_d<128, true>(a, w, stream) : launch_pack_d<128, false>(a, w, stream);
    case 256: return bf16 ? launch_pack_d<256, true>(a, w, stream) : launch_pack_d<256, false>(a, w, stream);
    case 512: return bf16 ? launch_pack_d<512, true>(a, w, stream) : launch_pack_d<512, false>(a, w, stream);
    default: return hipErrorInvalidValue;
  }
}

bool prefill_reads_v_rows(int head_dim, bool bf16) { return !bf16 && head_dim <= 128; }

bool prefill_trio(int batch, int seqlen_q, int seqlen_kv, int n_heads_q, int n_heads_kv,
                  int head_dim, int causal, int window) {
  // Three work-groups per compute unit pay off when the blocks are of about
  // equal length and the grid overflows one round of two per compute unit
  // (512 slots) but fits one round of three (768): two per compute unit would
  // end with a partly filled second round. Unequal (causal) blocks keep two
  // per compute unit: there the longest blocks set the end, and they run
  // faster with one neighbour than with two.
  constexpr int kCUs = 256, BM = 128, BNP = 64;
  if (head_dim != 128 || n_heads_kv <= 0 || (n_heads_q / n_heads_kv) % 2 == 0) return false;
  const int nqb = (seqlen_q + BM - 1) / BM;
  const int64_t wgs = (int64_t)batch * n_heads_q * nqb;
  if (wgs <= 2 * kCUs || wgs > 3 * kCUs) return false;
  const int off = seqlen_kv - seqlen_q;
  int64_t sum = 0;
  int most = 0;
  for (int qb = 0; qb < nqb; ++qb) {   // key tiles of each block, as the kernel counts them
    const int q0 = qb * BM;
    int kv_end = seqlen_kv;
    if (causal) kv_end = std::min(kv_end, std::min(q0 + BM, seqlen_q) + off);
    const int kv_lo = window > 0 ? std::max(0, q0 + off - window + 1) : 0;
    const int n = kv_end > kv_lo ? (kv_end + BNP - 1) / BNP - kv_lo / BNP : 0;
    sum += n;
    most = std::max(most, n);
  }
  return sum > 0 && 4 * (int64_t)most * nqb <= 5 * sum;   // longest block <= 1.25 x the mean
}

hipError_t launch_prefill_attn_vrow(const PrefillArgs& a, int head_dim, bool unnormalized,
                                    hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_attn_vrow_d<64>(a, unnormalized, stream);
    case 128: return launch_attn_vrow_d<128>(a, unnormalized, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_attn(const PrefillArgs& a, const VtArgs& w, int head_dim, bool bf16,
                               bool unnormalized, hipStream_t stream) {
  switch (head_dim) {
    case 64:
      return bf16 ? launch_attn_d<64, true>(a, w, unnormalized, stream)
                  : launch_attn_d<64, false>(a, w, unnormalized, stream);
    case 128:
      return bf16 ? launch_attn_d<128, true>(a, w, unnormalized, stream)
                  : launch_attn_d<128, false>(a, w, unnormalized, stream);
    case 256:
      return bf16 ? launch_attn_d<256, true>(a, w, unnormalized, stream)
                  : launch_attn_d<256, false>(a, w, unnormalized, stream);
    case 512:
      return bf16 ? launch_attn_512<true>(a, w, unnormalized, stream)
                  : launch_attn_512<false>(a, w, unnormalized, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fa
