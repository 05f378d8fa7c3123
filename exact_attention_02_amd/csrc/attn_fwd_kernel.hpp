// Fused attention forward for gfx950 (CDNA4): device code.
//
// Method (FlashAttention-2 forward; page "Attention Kernel 实现与正确性验证",
// sections 1.1-1.2; page "Triton Cuda Attention", "在线 Softmax 核心算法"; page
// "Flash Attention 与 Kernel 优化", "running softmax 状态", "causal mask",
// "输出与保存状态"): a workgroup keeps its query rows on chip, streams the
// key/value tiles of one kv head through LDS, and per tile
//   S = scale * Q K^T,  m' = max(m, rowmax S),  a = 2^(m - m'),  P = 2^(S - m'),
//   l = a l + rowsum P,  O = a O + P V,  m = m'
// with scores pre-multiplied by log2(e) so every exponential is a native 2^x
// (exp2 form).  After the last tile O /= l and LSE = (m + log2 l) ln 2.
//
// MI355X mapping (not taken from the pages):
//  * Transposed products.  Each wave computes S^T = K Q^T and O^T = V^T P^T
//    with bf16 MFMAs, so a lane owns queries (MFMA columns) and a few keys of
//    each: the row max and row sum are lane-local plus an exchange between
//    the lanes of one column (v_permlane32_swap, v_permlane16_swap), and the
//    rescale factor is a lane scalar.  The S^T accumulator rounded to bf16 is
//    directly the B operand of the PV product.
//  * MFMA size per launch shape.  The wide single-pass shape uses
//    v_mfma_f32_16x16x32_bf16 (a lane owns two queries and 4 keys per 16-key
//    block): on random bf16 data the chip sustains about 12 % more FLOP/s
//    with it than with the 32x32x16 form (a higher clock under the same power
//    limit), and long launches are power-bound.  The other shapes use
//    v_mfma_f32_32x32x16_bf16 (one query, 16 keys per 32-key block): their
//    short, latency-bound launches run faster with it, and the split variant
//    of the wide shape does not fit its registers in the 16x16 form.
//  * Query fragments stay in VGPRs for the whole kernel (B operand of S^T).
//  * K and V tiles go from HBM straight into LDS (buffer_load_dwordx4 with the
//    lds modifier on a buffer resource per tile, no staging registers, lane
//    offsets fixed for the whole loop), each 16-byte chunk of a row
//    XOR-swizzled by the row index.  K fragments are 128-bit LDS reads; V^T
//    fragments come from the LDS transpose read ds_read_b64_tr_b16 on the
//    untransposed V tile, two per MFMA, in the key order the S^T accumulator
//    layout implies.
//  * A ring of P LDS stages for K and for V: after the barrier that opens tile
//    t the loads of tile t+P are issued into the stage tile t-1 used, so P-1
//    tiles are in flight while one is computed; one barrier per tile.
//  * Lazy, optimistic rescaling: the first tile sets the max used in the
//    exponent; later tiles take their exponentials against it without
//    computing their own max, and only when a tile's sum of P exceeds 2^24
//    (some score more than 24 above the max in use, or an overflow; a
//    wave-uniform branch) is that tile's true max taken, the state rescaled
//    and the tile's exponentials recomputed.  The final O = acc / l and LSE
//    use the same max, so the result is exact up to rounding.
//  * GQA/MQA: a workgroup serves one kv head.  Its MFMA columns enumerate
//    (query row, query head) pairs of that kv group, row-major with the G =
//    H_q/H_kv heads fastest, so every K/V tile in LDS serves all G heads and a
//    decode step (one query row) still fills G columns.
//  * Causal: the tile loop ends at the workgroup's last row; only tiles that
//    cross a wave's diagonal (or the ragged end of the keys) run the masked
//    variant.  With fewer query rows than keys the mask is bottom-right
//    aligned: row i sits at key position i + N_kv - N_q.
//  * Split of the key axis (SPLIT): blockIdx also selects one of n_splits
//    contiguous ranges of the workgroup's key tiles, and the workgroup writes
//    a partial result (O normalised by its own l, in bf16, and log2 l + m in
//    fp32) that the merge kernel combines through the log-sum-exps (page
//    "Attention Kernel 实现与正确性验证", section 2.4, split-T with a
//    safe-softmax merge).
//  * Pairs past the end are clamped to the last valid one on load (their
//    outputs are not stored).  Each K/V tile is read through a buffer
//    resource that ends at the head's last key, so key rows past N_kv come
//    back as zeros; their scores are masked.  Loads need no bounds branches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ea02 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct FwdParams {
  const uint16_t* q;  // [B, H_q, N_q, D] bf16
  const uint16_t* k;  // [B, H_kv, N_kv, D] bf16
  const uint16_t* v;  // [B, H_kv, N_kv, D] bf16
  uint16_t* o;        // [B, H_q, N_q, D] bf16 (single pass)
  float* lse;         // [B, H_q, N_q] natural log (single pass)
  uint16_t* o_part;   // [n_splits, B, H_q, N_q, D] bf16 (split pass)
  float* lse_part;    // [n_splits, B, H_q, N_q] log2 units (split pass)
  int B, H_q, H_kv, N_q, N_kv;
  int G;              // H_q / H_kv
  int n_pairs;        // N_q * G: (row, head) pairs per kv head
  int causal_off;     // N_kv - N_q when causal, else 0
  int n_pair_blocks;  // ceil(n_pairs / pairs per workgroup)
  int n_heads_wg;     // B * H_kv
  int n_splits;       // key-axis splits (1 for the single pass)
  float scale_log2;   // max(|sm_scale| * log2(e), FLT_MIN): strictly positive, so
                      // a masked score (-inf) never meets a zero factor
  uint32_t q_sign;    // 0x80008000 when sm_scale < 0 (Q is negated on load), else 0
  int causal;
  // Work stealing between the XCDs (eight-wave single pass; work_item).
  int* steal;         // nine claim counters, zero on entry and on exit; null: static order
  int n_items;        // workgroups of the static order (the grid may hold more)
  int n_static;       // workgroups below this index take their own item (a multiple of 8)
};

// Work stealing.  The hardware hands workgroup i to XCD i mod 8, so in the
// static order XCD x runs items x, x + 8, x + 16, ... (list x, heaviest
// first), and the slowest XCD sets the launch time.  With counters, the
// workgroups from n_static on claim instead: first the next item of their own
// list (steal[x] counts the claims on list x past its static part), else one
// from the list with the most items left.  The grid holds spare workgroups
// for the fast XCDs; a workgroup that finds every list empty does nothing.
// steal[8] counts finished claims, and the last claimer zeroes all nine
// counters, so they are zero again for the next launch on the stream.  Each
// item is computed the same way whoever runs it, so the results do not depend
// on the schedule.  Used by the forward's eight-wave single pass and by both
// backward kernels.
__device__ __forceinline__ int steal_list_len(int n_items, int x) { return (n_items - x + 7) >> 3; }

// Called by all lanes of one wave; returns the claimed item or -1 (uniform).
__device__ __forceinline__ int claim_work_item(int* steal, int n_items, int n_static, int lane) {
  typedef __attribute__((address_space(1))) int global_int;
  global_int* ctr = (global_int*)steal;  // a global-memory pointer (global, not flat, atomics)
  const int n = n_items, own = blockIdx.x & 7, j0 = n_static >> 3;
  int item = -1;
  if (lane == 0) {
    const int k = __hip_atomic_fetch_add(ctr + own, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (j0 + k < steal_list_len(n, own)) item = 8 * (j0 + k) + own;
  }
  item = __shfl(item, 0);
  // A list that looks empty is empty: the counters only grow, so a load can
  // only under-report a claim.  Each failed claim empties its list for good,
  // so eight rounds suffice.
  for (int round = 0; round < 8 && item < 0; ++round) {
    int left = -1, list = lane;
    if (lane < 8)
      left = steal_list_len(n, lane) - j0 - __hip_atomic_load(ctr + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      const int ol = __shfl_xor(left, o), oi = __shfl_xor(list, o);
      if (ol > left || (ol == left && oi < list)) {
        left = ol;
        list = oi;
      }
    }
    left = __shfl(left, 0);
    list = __shfl(list, 0);
    if (left <= 0) break;
    if (lane == 0) {
      const int k = __hip_atomic_fetch_add(ctr + list, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (j0 + k < steal_list_len(n, list)) item = 8 * (j0 + k) + list;
    }
    item = __shfl(item, 0);
  }
  if (lane == 0) {
    // every claim of this workgroup has completed before it counts as done
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const int done = __hip_atomic_fetch_add(ctr + 8, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (int)gridDim.x - n_static - 1)
      for (int c = 0; c < 9; ++c) __hip_atomic_exchange(ctr + c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return item;
}

// The work item of this workgroup: its own index below n_static or without
// counters, else a claimed one (-1: none left).  Every thread of the
// workgroup calls it; `claimed` is a workgroup-shared int.
__device__ __forceinline__ int work_item(int* steal, int n_items, int n_static, int wave, int lane, int& claimed) {
  const int bid = blockIdx.x;
  if (steal == nullptr || bid < n_static) return bid;
  if (wave == 0) {
    const int item = claim_work_item(steal, n_items, n_static, lane);
    if (lane == 0) claimed = item;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(claimed);
}

template <bool V>
struct BoolTag {
  static constexpr bool value = V;
};

// An LDS ring slot known at compile time (the steady-state loop is unrolled
// by the ring depth, so every operand read takes its slot's offset as an
// immediate); the tail passes a plain int.
template <int V>
struct SlotC {
  static constexpr int value = V;
  __device__ constexpr operator int() const { return V; }
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units: P stays <= 2^8
constexpr float kOverflowSum = 16777216.0f;  // 2^24: largest tile sum of P taken without a rescale
constexpr int kBufferFlags = 0x00020000;  // raw buffer resource word 3 for gfx9 (untyped dword access)

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// x in a VGPR whose value the compiler no longer knows: a constant folded
// into it stays out of the LDS instructions' 16-bit offset field, which the
// V ring's base (64 KiB and up in the deepest ring) would overflow.
__device__ __forceinline__ int opaque_vgpr(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Reductions over the lanes that hold one MFMA column (lanes l, l^32 for
// MN = 32; l, l^16, l^32, l^48 for MN = 16).  v_permlane32_swap exchanges
// lanes 32..63 of its first operand with lanes 0..31 of its second,
// v_permlane16_swap the odd 16-lane rows of the first with the even rows of
// the second; with both operands x, the two results hold x of this lane and
// of its partner.
template <int MN>
__device__ __forceinline__ float col_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  if constexpr (MN == 16) {
    auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
  }
  return x;
}
template <int MN>
__device__ __forceinline__ float col_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  if constexpr (MN == 16) {
    auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(t[0]) + __uint_as_float(t[1]);
  }
  return x;
}

// bf16 MFMA of size MN x MN x (512 / MN) with fp32 accumulators: one lane
// holds MN * MN / 64 of them.
template <int MN>
struct MfmaAcc;
template <>
struct MfmaAcc<32> {
  using type = f32x16;
};
template <>
struct MfmaAcc<16> {
  using type = f32x4;
};
template <int MN>
__device__ __forceinline__ typename MfmaAcc<MN>::type mfma_bf16(bf16x8 a, bf16x8 b, typename MfmaAcc<MN>::type c) {
  if constexpr (MN == 32) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Raw buffer resource: 48-bit base, no stride, num_records bytes.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  u32x4 r;
  r[0] = (uint32_t)a;
  r[1] = (uint32_t)(a >> 32) & 0xffffu;
  r[2] = bytes;
  r[3] = (uint32_t)kBufferFlags;
  return r;
}

// 16 bytes per lane from the buffer at byte offset voff straight into LDS at
// lds_addr + 16 * lane.  Written as inline asm so that the compiler does not
// track it: it would otherwise wait for these loads before every later LDS
// read.  The caller waits (s_waitcnt vmcnt(0)) before a barrier instead.
__device__ __forceinline__ void dma_16B(u32x4 rsrc, int voff, uint32_t lds_addr) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}

template <int D, int NW_, int P_, int QB_, int BN_>
struct Cfg {
  static constexpr int BN = BN_;                 // keys per tile (32 or 64)
  static constexpr int NW = NW_;                 // waves per workgroup
  static constexpr int P = P_;                   // LDS stages (tiles of K and of V in flight)
  static constexpr int QB = QB_;                 // 32-query column blocks per wave
  static constexpr int NT = NW * 64;
  static constexpr int QW = 32 * QB;             // query rows per wave
  static constexpr int DC = D / 8;               // 16-byte chunks per row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;       // one K or V tile
  static constexpr int LOADS = TILE_BYTES / 1024;         // 1 KiB load instructions per tile
  static constexpr int LOADS_PER_WAVE = LOADS / NW;
  static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;
  static constexpr int LDS_BYTES = 2 * P * TILE_BYTES;    // K ring then V ring
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
  static_assert(QB == 1, "one 32-pair query block per wave (the only shape built and tested)");
  static_assert(BN == 32 || BN == 64, "key tiles of 32 or 64");
  static_assert(LOADS % NW == 0 && LOADS_PER_WAVE >= 1, "tile loads split evenly over waves");
  static_assert(P >= 2 && LDS_BYTES <= 160 * 1024, "LDS ring fits the 160 KiB of a CU");
  static_assert((P - 1) * 2 * LOADS_PER_WAVE <= 63, "loads in flight fit the 6-bit vmcnt");
};

// 16-byte chunk swizzles of K and V rows in LDS: stored chunk j of row r
// holds chunk j ^ swz(r), so that the MFMA operand reads hit every bank
// group.  K reads: 16 lanes read 16 consecutive keys at one chunk index, so
// swz is a bijection on r mod 16 (within each row parity for D = 64, whose
// rows are half the 64 banks).  V transpose reads: a half wave reads 4 rows x
// 4 adjacent chunks (MN = 32) or 8 rows x 2 adjacent chunks (MN = 16) of
// aligned rows.  For MN = 16 one swizzle serves both (its bits 1.. take 8
// values over 8 aligned rows), so a K load and a V load share an offset.
// At D = 128 rows r and r + 8 also take chunk indices that differ in more
// than bit 0 (the second half of the rows runs the first half's pattern
// reversed): with the plain 2 (r & 7) + (r >> 3) the 128-bit row reads of
// the K tile took two passes each on gfx950 (SQ_LDS_BANK_CONFLICT: 4 cycles
// per read), with this one they take none; the transpose reads stay free of
// conflicts either way.
template <int D>
__device__ __forceinline__ int kv16_swz(int row) {
  if constexpr (D == 128) return (2 * (row & 7) ^ (14 * ((row >> 3) & 1))) | ((row >> 3) & 1);
  else return 2 * ((row >> 1) & 3) + ((row >> 3) & 1);
}
template <int D, int MN>
__device__ __forceinline__ int k_swz(int row) {
  if constexpr (MN == 16) return kv16_swz<D>(row);
  else if constexpr (D == 128) return row & 15;
  else return (row >> 1) & 7;
}
template <int D, int MN>
__device__ __forceinline__ int v_swz(int row) {
  if constexpr (MN == 16) return kv16_swz<D>(row);
  else if constexpr (D == 128) return 4 * (row & 3);
  else return 4 * ((row >> 1) & 1);
}

// QB: 32-pair query blocks per wave.  Only QB = 1 is built and tested: waves
// of 32 (row, head) pairs, two waves per SIMD (256 registers each).  Two
// blocks per wave (one wave per SIMD, each K or V^T fragment feeding twice
// the MFMAs) measured slower.
// MN: MFMA size, 32 (v_mfma_f32_32x32x16_bf16: one 32-query column block per
// wave) or 16 (v_mfma_f32_16x16x32_bf16: two 16-query column blocks).
// SPLIT: write the partial result of one key range (bf16 O, fp32 log2-unit
// LSE) instead of the final output.
template <int D, int NW, int P, int QB, int BN_, int MN, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(QB == 1 ? 2 : 1, QB == 1 ? 2 : 1)))
void attn_fwd_kernel(FwdParams p) {
  using C = Cfg<D, NW, P, QB, BN_>;
  constexpr int BN = C::BN;
  constexpr int KK = 512 / MN;        // contraction length of one MFMA
  constexpr int ACC = MN * MN / 64;   // accumulator registers per lane and MFMA block
  constexpr int QC = C::QW / MN;      // query column blocks per wave
  constexpr int KB = BN / MN;         // key row blocks of S^T per tile
  using AccT = typename MfmaAcc<MN>::type;
  static_assert(MN == 16 || MN == 32, "MFMA 16x16x32 or 32x32x16");
  constexpr int PPW = C::QW * C::NW;  // (row, head) pairs per workgroup
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // MFMA operand and result layout: lane = MN kgrp + col.  An operand lane
  // holds row (A) or column (B) `col` and contraction slots 8 kgrp .. 8 kgrp
  // + 7; a result lane holds column `col` and rows (r / 4) (256 / MN) + 4 kgrp
  // + r % 4 for its accumulator registers r.
  const int kgrp = lane / MN;
  const int col = lane % MN;

  // ---- work decomposition: heaviest pair blocks first (causal), then the
  //      key splits, kv heads fastest.  Item bid of that order; the
  //      eight-wave single pass may claim it instead (work_item).
  int bid = blockIdx.x;
  if constexpr (!SPLIT && NW == 8) {
    __shared__ int claimed;
    bid = work_item(p.steal, p.n_items, p.n_static, wave, lane, claimed);
    if (bid < 0) return;
  }
  const int head_wg = bid % p.n_heads_wg;
  const int rest = bid / p.n_heads_wg;
  const int split = SPLIT ? rest % p.n_splits : 0;
  const int pb = p.n_pair_blocks - 1 - (SPLIT ? rest / p.n_splits : rest);
  const int g = head_wg % p.H_kv;
  const int b = head_wg / p.H_kv;
  const int G = p.G;
  const int last_pair = p.n_pairs - 1;
  const int P0 = pb * PPW;            // first pair of the workgroup
  const int wp0 = P0 + wave * C::QW;  // first pair of this wave
  const int wave_row0 = min(wp0, last_pair) / G;
  const int wg_row_end = min(P0 + PPW - 1, last_pair) / G + 1;
  const int N_kv = p.N_kv;
  const int off = p.causal_off;

  // key tiles of this workgroup: [0, kv_end) of the kv head, of which the
  // split takes a contiguous range of n_tiles tiles starting at key kbase
  const int kv_end = p.causal ? min(wg_row_end + off, N_kv) : N_kv;
  int n_tiles = (kv_end + BN - 1) / BN;
  int kbase = 0;
  if constexpr (SPLIT) {
    const int per = (n_tiles + p.n_splits - 1) / p.n_splits;
    const int t0 = min(split * per, n_tiles);
    n_tiles = min(per, n_tiles - t0);
    kbase = t0 * BN;
  }

  const size_t kv_base = ((size_t)b * p.H_kv + g) * (size_t)N_kv * D;

  // ---- query fragments (B operands of S^T = K Q^T): in column block qc the
  //      lane holds pair wp0 + MN qc + col = (row, head g*G + j), d = KK*ks +
  //      8*kgrp .. +8.  Pairs past the end are clamped to the last one.
  // (b * H_q + h) * N_q + row of column block qc's pair (recomputed where
  // needed rather than kept live through the tile loop)
  auto bhr_of = [&](int qc) {
    const int pc = min(wp0 + MN * qc + col, last_pair);
    const int row = pc / G;
    const int h = g * G + (pc - row * G);
    return ((size_t)b * p.H_q + h) * (size_t)p.N_q + row;
  };
  // query row of column block qc's pair (recomputed on the masked tiles
  // only: a register held across the tile loop costs more)
  auto row_of = [&](int qc) { return min(wp0 + MN * qc + col, last_pair) / G; };
  bf16x8 qf[QC][D / KK];
#pragma unroll
  for (int qc = 0; qc < QC; ++qc) {
    const size_t bhr = bhr_of(qc);
#pragma unroll
    for (int ks = 0; ks < D / KK; ++ks) {
      u32x4 x = *reinterpret_cast<const u32x4*>(p.q + bhr * D + ks * KK + kgrp * 8);
      x ^= p.q_sign;
      qf[qc][ks] = as_bf16x8(x);
    }
  }

  // ---- direct HBM -> LDS tile loads.  Load instruction i of a tile fills
  //      bytes [1024 i, 1024 i + 1024): lane -> (row, stored chunk j), and it
  //      fetches global chunk j ^ swz(row).  LDS holds a ring of P K tiles
  //      then a ring of P V tiles.  Each tile is read through a buffer
  //      resource that starts at the tile's first key and ends at the last
  //      key of the head, so the lane offsets are loop constants and rows
  //      past the last key come back as zeros (their scores are masked).
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)lds;
  int ld_off_k[C::LOADS_PER_WAVE], ld_off_v[C::LOADS_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::LOADS_PER_WAVE; ++i) {
    const int r = (wave * C::LOADS_PER_WAVE + i) * C::ROWS_PER_LOAD + lane / C::DC;
    ld_off_k[i] = r * C::ROW_BYTES + (((lane % C::DC) ^ k_swz<D, MN>(r)) << 4);
    ld_off_v[i] = r * C::ROW_BYTES + (((lane % C::DC) ^ v_swz<D, MN>(r)) << 4);
  }
  const uint16_t* k_head = p.k + kv_base;
  const uint16_t* v_head = p.v + kv_base;
  // one tile of K (ring 0) or V (ring 1) into ring slot `slot`; tile numbers
  // count from the split's first key
  // A load that no phase reads (the ring's fill before the first V tile and
  // past the last tiles) keeps its place in the load count but gets an empty
  // resource: no memory access, zeros into a free slot.
  auto issue_tile = [&](int tile, int slot, const uint16_t* head, int ring, bool live) {
    const int row0 = kbase + tile * BN;
    const u32x4 rsrc = make_rsrc(head + (size_t)row0 * D, live ? (uint32_t)(N_kv - row0) * C::ROW_BYTES : 0u);
#pragma unroll
    for (int i = 0; i < C::LOADS_PER_WAVE; ++i)
      dma_16B(rsrc, ring == 0 ? ld_off_k[i] : ld_off_v[i], lds_base + (ring * P + slot) * C::TILE_BYTES + (wave * C::LOADS_PER_WAVE + i) * 1024);
  };

  // per-lane LDS byte offsets of the MFMA operand reads (tile-relative)
  // K (A operand of S^T, MN keys x KK d): key MN c + col, chunk (KK/8) ks + kgrp.
  // V^T (A operand of O^T, MN d x KK keys): lane row d = MN db + col; its
  //   contraction slots are the keys KK st + 4 kgrp + {0..3} (first transpose
  //   read) and KK st + KK/2 + 4 kgrp + {0..3} (second): in the S^T
  //   accumulator layout exactly the keys whose scores this lane holds in
  //   the 8 consecutive accumulator registers that form P's B operand of
  //   step st.  Each transpose read: lane L of a 16-lane group addresses row
  //   4 kgrp + L/4 (+ KK st, + KK/2), d = d16 + 4 (L & 3) .. +4, and receives
  //   d = d16 + L of the group's four rows (d16: the group's 16 d).
  const int L = lane & 15;
  const int vt_row = 4 * kgrp + (L >> 2);
  // V ring base plus lane offset of each d block (the tile's slot and step
  // are added as immediates)
  int vt_off[D / MN];
#pragma unroll
  for (int db = 0; db < D / MN; ++db) {
    const int d = db * MN + 16 * ((lane >> 4) % (MN / 16)) + 4 * (L & 3);
    const int chunk = (d >> 3) ^ v_swz<D, MN>(vt_row);
    vt_off[db] = opaque_vgpr(P * C::TILE_BYTES + vt_row * C::ROW_BYTES + chunk * 16 + (d & 7) * 2);
  }
  auto k_read = [&](auto slot, int i) {
    const uint8_t* kb = lds + int(slot) * C::TILE_BYTES;
    const int c = i % KB, ks = i / KB;  // consecutive reads alternate key blocks
    const int key = c * MN + col;
    return *reinterpret_cast<const u32x4*>(kb + key * C::ROW_BYTES +
                                           ((((KK / 8) * ks + kgrp) ^ k_swz<D, MN>(key)) << 4));
  };
  auto v_read = [&](auto slot, int i) {
    const uint8_t* vb = lds + int(slot) * C::TILE_BYTES;
    const int st = i / (D / MN), db = i % (D / MN);
    const uint8_t* a0 = vb + vt_off[db] + (KK * st) * C::ROW_BYTES;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + (KK / 2) * C::ROW_BYTES));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  constexpr int NS = KB * (D / KK);         // K fragment reads per tile (each feeds QC MFMAs)
  constexpr int NP = (BN / KK) * (D / MN);  // V^T fragment reads per tile (each feeds QC MFMAs)
  constexpr int NV = KB * ACC;              // scores per lane per column block per tile
  constexpr int EPR = QC * NV / NS;         // exponentials per K fragment read
  static_assert(EPR * NS == QC * NV, "score work splits evenly");
  constexpr int PF = 2;                     // LDS operand prefetch distance

  // ---- running state: per column block, one query per lane
  float m_used[QC], l_run[QC];
  AccT acc[D / MN][QC];
#pragma unroll
  for (int qc = 0; qc < QC; ++qc) {
    m_used[qc] = -INFINITY;  // max used in the exponent (log2-scaled units)
    l_run[qc] = 0.f;         // this lane's partial sum of P over its keys
#pragma unroll
    for (int i = 0; i < D / MN; ++i) acc[i][qc] = AccT{};
  }
  const float sl2 = p.scale_log2;

  using Scores = AccT[KB][QC];
  // S^T = K Q^T of one tile with no other work interleaved (prologue only)
  auto s_tile = [&](auto slot, Scores& s) {
#pragma unroll
    for (int c = 0; c < KB; ++c)
#pragma unroll
      for (int qc = 0; qc < QC; ++qc) s[c][qc] = AccT{};
    u32x4 kx[PF + 1];
#pragma unroll
    for (int i = 0; i < PF; ++i) kx[i] = k_read(slot, i);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + PF < NS) kx[(i + PF) % (PF + 1)] = k_read(slot, i + PF);
      const int c = i % KB, ks = i / KB;
#pragma unroll
      for (int qc = 0; qc < QC; ++qc)
        s[c][qc] = mfma_bf16<MN>(as_bf16x8(kx[i % (PF + 1)]), qf[qc][ks], s[c][qc]);
    }
  };
  // diagonal or ragged tile: element (c, qc, r) holds key kbase + tile*BN +
  // MN c + (r/4)(256/MN) + 4 kgrp + r%4 of column block qc's query; it is
  // visible when that offset minus 4 kgrp is below lim.  Rows grow with the
  // pair index, so the wave's first row decides.
  auto needs_mask = [&](int tile) {
    const int key0 = kbase + tile * BN;
    return (p.causal && key0 + BN - 1 > wave_row0 + off) || key0 + BN > N_kv;
  };
  auto apply_mask = [&](int tile, Scores& s) {
#pragma unroll
    for (int qc = 0; qc < QC; ++qc) {
      const int lim = (p.causal ? min(row_of(qc) + off + 1, N_kv) : N_kv) - kbase - tile * BN - 4 * kgrp;
#pragma unroll
      for (int c = 0; c < KB; ++c)
#pragma unroll
        for (int r = 0; r < ACC; ++r)
          s[c][qc][r] = (c * MN + (r >> 2) * (256 / MN) + (r & 3) < lim) ? s[c][qc][r] : -INFINITY;
    }
  };
  // raise the exponent's max when the tile max exceeds it by more than the
  // slack (wave-uniform branch; rare after the first tile)
  auto update_max = [&](const float* mx_lane) {
#pragma unroll
    for (int qc = 0; qc < QC; ++qc) {
      const float mt = col_max<MN>(mx_lane[qc]) * sl2;  // sl2 > 0: a masked row stays -inf
      if (__builtin_amdgcn_ballot_w64(mt > m_used[qc] + kRescaleSlack)) {
        const float m_new = fmaxf(m_used[qc], mt);
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_used[qc] - m_new);
        l_run[qc] *= alpha;
#pragma unroll
        for (int db = 0; db < D / MN; ++db) acc[db][qc] *= alpha;
        m_used[qc] = m_new;
      }
    }
  };
  auto lane_max = [&](const Scores& s, float* mx) {
#pragma unroll
    for (int qc = 0; qc < QC; ++qc) {
      float m = s[0][qc][0];
#pragma unroll
      for (int c = 0; c < KB; ++c)
#pragma unroll
        for (int r = (c == 0 ? 1 : 0); r < ACC; ++r) m = fmaxf(m, s[c][qc][r]);
      mx[qc] = m;
    }
  };

  // Software pipeline: one phase per tile t, entered with the scores S(t)
  // computed, masked and the max applied:
  //   O += V(t-1) P(t-1)          (HAS_PREV: 32 MFMAs on V^T operand reads)
  //   P(t) = 2^(S(t) sl2 - m)      (the exponentials, spread over both halves)
  //   S(t+1) = K(t+1) Q^T          (HAS_NEXT: 32 MFMAs on K operand reads)
  // so the softmax VALU of a tile runs under the MFMAs of both neighbouring
  // products instead of only the scores of the next tile.  P(t) goes to
  // pcur while P(t-1) is read from pprev (two buffers, alternating by tile
  // parity).  pcur[qc][st] is the B operand of the KK keys of step st:
  // accumulator registers 8 st .. 8 st + 7 of the lane's scores in
  // key-block-major order.
  using PBuf = bf16x8[QC][BN / KK];
  constexpr int NE = QC * NV;  // exponentials per lane and tile
  auto phase = [&](int t, auto ks_next, auto vs_prev, Scores& sc, Scores& sn, PBuf& pcur, PBuf& pprev,
                   auto has_prev_tag, auto has_next_tag) {
    constexpr bool HAS_PREV = decltype(has_prev_tag)::value;
    constexpr bool HAS_NEXT = decltype(has_next_tag)::value;
    // exponentials under the PV half and under the score half
    constexpr int EA = HAS_PREV ? (HAS_NEXT ? NE / 2 : NE) : 0;
    constexpr int EB = HAS_NEXT ? NE - EA : 0;
    static_assert(EA % NP == 0 && EB % NS == 0, "exponentials spread evenly over the operand reads");
    float m_sub[QC], l_t[QC];
#pragma unroll
    for (int qc = 0; qc < QC; ++qc) {
      m_sub[qc] = (m_used[qc] == -INFINITY) ? 0.f : m_used[qc];
      l_t[qc] = 0.f;
    }
    f32x8 pf[QC];
    // exponential number j of this tile: column block j / NV, element e =
    // j % NV (key block e / ACC, register e % ACC), taken against the max in
    // use (no max of this tile is computed here)
    auto p_elem = [&](int j) {
      const int qc = j / NV, e = j % NV;
      const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e / ACC][qc][e % ACC], sl2, -m_sub[qc]));
      pf[qc][e & 7] = pe;
      l_t[qc] += pe;
      if ((e & 7) == 7) {
        pcur[qc][e >> 3] = __builtin_convertvector(pf[qc], bf16x8);
        // packed here: otherwise the compiler carries the eight fp32 values
        // into the next phase and converts them there
        asm volatile("" : "+v"(pcur[qc][e >> 3]));
      }
    };
    if constexpr (HAS_PREV) {
      // O^T += V^T P^T of tile t-1; step st covers keys KK st .. KK st + KK - 1
      bf16x8 vx[PF + 1];
#pragma unroll
      for (int i = 0; i < PF; ++i) vx[i] = v_read(vs_prev, i);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        if (i + PF < NP) vx[(i + PF) % (PF + 1)] = v_read(vs_prev, i + PF);
        const int st = i / (D / MN), db = i % (D / MN);
#pragma unroll
        for (int qc = 0; qc < QC; ++qc)
          acc[db][qc] = mfma_bf16<MN>(vx[i % (PF + 1)], pprev[qc][st], acc[db][qc]);
#pragma unroll
        for (int e = 0; e < EA / NP; ++e) p_elem(i * (EA / NP) + e);
      }
    }
    // keep the halves apart: interleaving them would hold the next tile's
    // score accumulators and the previous tile's P at once
    if constexpr (HAS_PREV && HAS_NEXT) __builtin_amdgcn_sched_barrier(0);
    if constexpr (HAS_NEXT) {
#pragma unroll
      for (int c = 0; c < KB; ++c)
#pragma unroll
        for (int qc = 0; qc < QC; ++qc) sn[c][qc] = AccT{};
      u32x4 kx[PF + 1];
#pragma unroll
      for (int i = 0; i < PF; ++i) kx[i] = k_read(ks_next, i);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (i + PF < NS) kx[(i + PF) % (PF + 1)] = k_read(ks_next, i + PF);
        const int c = i % KB, ks = i / KB;
#pragma unroll
        for (int qc = 0; qc < QC; ++qc)
          sn[c][qc] = mfma_bf16<MN>(as_bf16x8(kx[i % (PF + 1)]), qf[qc][ks], sn[c][qc]);
#pragma unroll
        for (int e = 0; e < EB / NS; ++e) p_elem(EA + i * (EB / NS) + e);
      }
    }
    if constexpr (!HAS_PREV && !HAS_NEXT) {
#pragma unroll
      for (int j = 0; j < NE; ++j) p_elem(j);
    }
    // A tile sum above 2^24 means some score exceeds the max in use by more
    // than 24 (log2 units), or overflowed: take this tile's true max, rescale
    // the state (O already holds every tile before this one) and recompute
    // the tile's exponentials (rare: the first tile sets the max, and scores
    // rarely climb that far above it).
    bool big = false;
#pragma unroll
    for (int qc = 0; qc < QC; ++qc) big |= !(l_t[qc] <= kOverflowSum);
    if (__builtin_amdgcn_ballot_w64(big)) {
      float mx[QC];
      lane_max(sc, mx);
#pragma unroll
      for (int qc = 0; qc < QC; ++qc) {
        const float mt = col_max<MN>(mx[qc]) * sl2;
        const float m_new = fmaxf(m_used[qc], mt);
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_used[qc] - m_new);
        l_run[qc] *= alpha;
#pragma unroll
        for (int db = 0; db < D / MN; ++db) acc[db][qc] *= alpha;
        m_used[qc] = m_new;
        m_sub[qc] = (m_new == -INFINITY) ? 0.f : m_new;
        l_t[qc] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < NE; ++j) p_elem(j);
    }
#pragma unroll
    for (int qc = 0; qc < QC; ++qc) l_run[qc] += l_t[qc];
    // a diagonal or ragged next tile is masked before its exponentials
    if constexpr (HAS_NEXT) {
      if (needs_mask(t + 1)) apply_mask(t + 1, sn);
    }
  };
  // O += V(t) P(t) of the last tile, after every phase
  auto last_pv = [&](auto vs, PBuf& pl) {
    bf16x8 vx[PF + 1];
#pragma unroll
    for (int i = 0; i < PF; ++i) vx[i] = v_read(vs, i);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (i + PF < NP) vx[(i + PF) % (PF + 1)] = v_read(vs, i + PF);
      const int st = i / (D / MN), db = i % (D / MN);
#pragma unroll
      for (int qc = 0; qc < QC; ++qc) acc[db][qc] = mfma_bf16<MN>(vx[i % (PF + 1)], pl[qc][st], acc[db][qc]);
    }
  };

  // Load schedule.  Group j loads K(j) into K slot j % P and V(j-2) into V
  // slot (j-2) % P; the phase of tile t reads K(t+1) and V(t-1), i.e. group
  // t+1.  Groups are issued P-1 ahead: after the barrier that opens the
  // phase of tile t, group t+P goes into the slots that the phase of tile t-1
  // read (K(t), V(t-2)), which every wave has finished.  A group past either
  // end of the sequence still issues its loads, with empty resources, into
  // its (free) slots, so every group is the same number of loads and each
  // wait below is one constant vmcnt.
  auto issue_group = [&](int j) {
    issue_tile(min(j, n_tiles - 1), j % P, k_head, 0, j < n_tiles);
    issue_tile(max(min(j - 2, n_tiles - 1), 0), (j + P - 2) % P, v_head, 1, j >= 2 && j - 2 < n_tiles);
  };
  constexpr int GROUP_LOADS = 2 * C::LOADS_PER_WAVE;
  auto sync_prologue = [&]() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((P - 1) * GROUP_LOADS) : "memory");
    __syncthreads();
  };
  // every load of groups up to the one that the next phase reads has landed
  auto sync_steady = [&]() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((P - 2) * GROUP_LOADS) : "memory");
    __syncthreads();
  };

  if (n_tiles > 0) {
#pragma unroll
    for (int j = 0; j < P; ++j) issue_group(j);
    sync_prologue();
    Scores sa, sb;  // S(t) of even tiles in sa, of odd tiles in sb
    PBuf pa, pb;    // P(t) of even tiles in pa, of odd tiles in pb
    s_tile(SlotC<0>{}, sa);
    if (needs_mask(0)) apply_mask(0, sa);
    {
      float mx[QC];
      lane_max(sa, mx);
      update_max(mx);
    }
    sync_steady();
    issue_group(P);
    if (n_tiles > 1)
      phase(0, SlotC<1>{}, 0, sa, sb, pa, pb, BoolTag<false>{}, BoolTag<true>{});
    else
      phase(0, 0, 0, sa, sb, pa, pb, BoolTag<false>{}, BoolTag<false>{});
    // Steady state from tile 1, unrolled by the ring depth P: tile t = t0 + J
    // with t0 = 1 mod P, so the ring slots of K(t+1) and V(t-1) and the
    // parity of t are compile-time constants (every LDS offset an
    // immediate, the buffers alternate without copies).  Then the last
    // tiles with run-time slots; t is odd there.
    static_assert(P == 2 || P == 4, "ring depths of 2 or 4: even, so the buffers stay in step");
    int t = 1;
    for (; t + P < n_tiles; t += P) {
      sync_steady();
      issue_group(t + P);
      phase(t, SlotC<2 % P>{}, SlotC<0>{}, sb, sa, pb, pa, BoolTag<true>{}, BoolTag<true>{});
      sync_steady();
      issue_group(t + 1 + P);
      phase(t + 1, SlotC<3 % P>{}, SlotC<1>{}, sa, sb, pa, pb, BoolTag<true>{}, BoolTag<true>{});
      if constexpr (P >= 4) {
        sync_steady();
        issue_group(t + 2 + P);
        phase(t + 2, SlotC<0>{}, SlotC<2>{}, sb, sa, pb, pa, BoolTag<true>{}, BoolTag<true>{});
        sync_steady();
        issue_group(t + 3 + P);
        phase(t + 3, SlotC<1>{}, SlotC<3>{}, sa, sb, pa, pb, BoolTag<true>{}, BoolTag<true>{});
      }
    }
    for (; t + 2 < n_tiles; t += 2) {
      sync_steady();
      issue_group(t + P);
      phase(t, (t + 1) % P, (t - 1) % P, sb, sa, pb, pa, BoolTag<true>{}, BoolTag<true>{});
      sync_steady();
      issue_group(t + 1 + P);
      phase(t + 1, (t + 2) % P, t % P, sa, sb, pa, pb, BoolTag<true>{}, BoolTag<true>{});
    }
    if (t + 1 < n_tiles) {
      sync_steady();
      issue_group(t + P);
      phase(t, (t + 1) % P, (t - 1) % P, sb, sa, pb, pa, BoolTag<true>{}, BoolTag<true>{});
      sync_steady();
      issue_group(t + 1 + P);
      phase(t + 1, 0, t % P, sa, sb, pa, pb, BoolTag<true>{}, BoolTag<false>{});
    } else if (t < n_tiles) {
      sync_steady();
      issue_group(t + P);
      phase(t, 0, (t - 1) % P, sb, sa, pb, pa, BoolTag<true>{}, BoolTag<false>{});
    }
    // the last tile's O += V P, once its V tile (group n_tiles + 1) has landed
    sync_steady();
    if ((n_tiles - 1) % 2 == 0)
      last_pv((n_tiles - 1) % P, pa);
    else
      last_pv((n_tiles - 1) % P, pb);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may outlive the workgroup
  }

  // ---- epilogue.  Single pass: O = acc / l (bf16, round to nearest even),
  //      LSE in natural log.  Split pass: fp32 O = acc / l and log2-unit
  //      m + log2 l of this key range; a range with no visible key (l = 0)
  //      gives O = 0 and -inf, the neutral element of the merge.  A lane
  //      holds d = MN db + g4 (256/MN) + 4 kgrp .. +4 of its query in
  //      registers 4 g4 .. 4 g4 + 3 of acc[db].
#pragma unroll
  for (int qc = 0; qc < QC; ++qc) {
    const float l_tot = col_sum<MN>(l_run[qc]);
    if (wp0 + MN * qc + col > last_pair) continue;
    const size_t bhr = bhr_of(qc);
    if constexpr (!SPLIT) {
      const float inv = 1.f / l_tot;
      uint16_t* orow = p.o + bhr * D;
#pragma unroll
      for (int db = 0; db < D / MN; ++db)
#pragma unroll
        for (int g4 = 0; g4 < ACC / 4; ++g4) {
          const f32x4 f = {acc[db][qc][4 * g4 + 0] * inv, acc[db][qc][4 * g4 + 1] * inv,
                           acc[db][qc][4 * g4 + 2] * inv, acc[db][qc][4 * g4 + 3] * inv};
          const bf16x4 bv = __builtin_convertvector(f, bf16x4);
          *reinterpret_cast<u32x2*>(orow + db * MN + g4 * (256 / MN) + 4 * kgrp) = __builtin_bit_cast(u32x2, bv);
        }
      if (kgrp == 0) p.lse[bhr] = (m_used[qc] + __log2f(l_tot)) * kLn2;
    } else {
      const bool seen = l_tot > 0.f;
      const float inv = seen ? 1.f / l_tot : 0.f;
      const size_t slot = (size_t)split * ((size_t)p.B * p.H_q * p.N_q) + bhr;
      uint16_t* orow = p.o_part + slot * D;
#pragma unroll
      for (int db = 0; db < D / MN; ++db)
#pragma unroll
        for (int g4 = 0; g4 < ACC / 4; ++g4) {
          const f32x4 f = {acc[db][qc][4 * g4 + 0] * inv, acc[db][qc][4 * g4 + 1] * inv,
                           acc[db][qc][4 * g4 + 2] * inv, acc[db][qc][4 * g4 + 3] * inv};
          const bf16x4 bv = __builtin_convertvector(f, bf16x4);
          *reinterpret_cast<u32x2*>(orow + db * MN + g4 * (256 / MN) + 4 * kgrp) = __builtin_bit_cast(u32x2, bv);
        }
      if (kgrp == 0) p.lse_part[slot] = seen ? m_used[qc] + __log2f(l_tot) : -INFINITY;
    }
  }
}

// Merge of the split pass (page "Attention Kernel 实现与正确性验证", section
// 2.4: the split-T partial results combined by a safe softmax over their
// log-sum-exps).  Per (b, h, row), with L_s the log2-unit partial LSEs:
//   M = max_s L_s,  w_s = 2^(L_s - M),  O = sum_s w_s O_s / sum_s w_s,
//   LSE = (M + log2 sum_s w_s) ln 2.
// A thread owns 4 consecutive d of one row and every SL-th split ("split
// lane"); it takes its own max over its splits first, then sums its weighted
// partial outputs, and the SL split lanes of the row are combined through LDS
// by the same rule.  SL is chosen per launch so that a thread sees at most a
// few splits: few rows (a decode step) still spread over many threads.  With
// at most KB splits per thread, every partial output loads in the same round
// as the LSEs; with more, a first pass over the LSEs finds the max and a
// second loads four splits at a time.  Both add a thread's splits in the same
// order.
struct MergeParams {
  const uint16_t* o_part;  // [n_splits, rows, D] bf16: each split's O, normalised by its own sum
  const float* lse_part;   // [n_splits, rows] log2 units
  uint16_t* o;            // [rows, D] bf16
  float* lse;             // [rows]
  int64_t rows;           // B * H_q * N_q
  int n_splits;
};

constexpr int kMergeBatch = 4;  // splits whose loads a thread issues together

template <int D, int NT, int KB>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT))) void attn_merge_kernel(MergeParams p) {
  constexpr int TPR = D / 4;  // threads per row and split lane
  constexpr int SL = NT / TPR;
  const int t = threadIdx.x;
  const int c = t % TPR;
  const int j = t / TPR;
  const int64_t row = blockIdx.x;
  const size_t stride = (size_t)p.rows;
  const int n = p.n_splits;
  const float* lse_r = p.lse_part + row;
  const uint16_t* o_r = p.o_part + (size_t)row * D + 4 * c;

  float m = -INFINITY;
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (n <= KB * SL) {
    float l[KB];
    f32x4 x[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int s = min(j + u * SL, n - 1);
      l[u] = j + u * SL < n ? lse_r[s * stride] : -INFINITY;
      x[u] = __builtin_convertvector(__builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(o_r + s * stride * D)), f32x4);
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) m = fmaxf(m, l[u]);
    if (m != -INFINITY) {
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const float w = __builtin_amdgcn_exp2f(l[u] - m);  // 2^-inf = 0
        wsum += w;
        acc += w * x[u];
      }
    }
  } else {
    for (int s0 = j; s0 < n; s0 += kMergeBatch * SL) {
      float l[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const int s = s0 + u * SL;
        l[u] = s < n ? lse_r[s * stride] : -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) m = fmaxf(m, l[u]);
    }
    if (m != -INFINITY) {
      for (int s0 = j; s0 < n; s0 += kMergeBatch * SL) {
        float l[kMergeBatch];
        f32x4 x[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
          const int s = min(s0 + u * SL, n - 1);
          l[u] = s0 + u * SL < n ? lse_r[s * stride] : -INFINITY;
          x[u] = __builtin_convertvector(__builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(o_r + s * stride * D)), f32x4);
        }
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
          const float w = __builtin_amdgcn_exp2f(l[u] - m);  // 2^-inf = 0
          wsum += w;
          acc += w * x[u];
        }
      }
    }
  }
  __shared__ float st_m[SL][TPR], st_w[SL][TPR];
  __shared__ f32x4 st_o[SL][TPR];
  st_m[j][c] = m;
  st_w[j][c] = wsum;
  st_o[j][c] = acc;
  __syncthreads();
  if (j != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < SL; ++k) M = fmaxf(M, st_m[k][c]);
  float tot = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
#pragma unroll
    for (int k = 0; k < SL; ++k) {
      const float f = __builtin_amdgcn_exp2f(st_m[k][c] - M);  // a lane with no split has m = -inf
      tot += f * st_w[k][c];
      o += f * st_o[k][c];
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const bf16x4 bv = __builtin_convertvector(o * inv, bf16x4);
  *reinterpret_cast<u32x2*>(p.o + (size_t)row * D + 4 * c) = __builtin_bit_cast(u32x2, bv);
  if (c == 0) p.lse[row] = tot > 0.f ? (M + __log2f(tot)) * kLn2 : -INFINITY;
}

// Launches the merge over every row, one block per row, in launches of at
// most 2^31 work-items each (a dispatch counts its work-items in 32 bits).
// Each launch takes a contiguous run of rows through offset pointers; m.rows
// stays the stride between splits.
template <int D, int NT, int KB>
hipError_t launch_merge_rows(const MergeParams& m, hipStream_t stream) {
  constexpr int64_t kRowsPerLaunch = (int64_t(1) << 31) / NT;
  for (int64_t r0 = 0; r0 < m.rows; r0 += kRowsPerLaunch) {
    const int64_t n = m.rows - r0 < kRowsPerLaunch ? m.rows - r0 : kRowsPerLaunch;
    MergeParams c = m;
    c.o_part = m.o_part + r0 * D;
    c.lse_part = m.lse_part + r0;
    c.o = m.o + r0 * D;
    c.lse = m.lse + r0;
    hipLaunchKernelGGL((attn_merge_kernel<D, NT, KB>), dim3(static_cast<unsigned>(n)), dim3(NT), 0, stream, c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ea02
