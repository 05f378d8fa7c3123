// Attention backward for gfx950 (CDNA4): device code.
//
// Method (page "Attention Kernel 实现与正确性验证", section 1.1, third trick:
// the backward recomputes the attention from Q, K and the saved row
// statistics instead of storing S; page "Flash Attention 与 Kernel 优化",
// "Autograd 包装与反向传播": rebuild s = q k^T scale, apply the causal mask,
// rebuild p, then dv, dp, ds, dq, dk).  With the forward's log-sum-exp L:
//   P  = exp(scale Q K^T - L)          (masked entries 0)
//   dV = P^T dO,   dP = dO V^T,   Dl = rowsum(dO * O),   dS = P * (dP - Dl)
//   dQ = scale dS K,   dK = scale dS^T Q          (dK, dV summed over the
//                                                  query heads of a kv head)
//
// Three kernels, and a fourth that sums row-range splits; no atomics (the
// result is deterministic for a given split count):
//  * attn_bwd_prep_kernel: Dl = rowsum(dO * O) and L2 = L log2(e) per row.
//  * attn_bwd_dkdv_kernel: a workgroup owns 32 keys per wave of one kv head;
//    K and V of those keys stay in registers while the query rows of every
//    head of the group stream through LDS (each tile is contiguous rows of
//    one head; row tiles from the last down, the group's heads in turn).  When the key blocks alone are too few to
//    fill the device (one kv head, short sequences), a key block's sequence
//    of row tiles is cut into n_kv_splits contiguous ranges, one workgroup
//    each, writing fp32 partial sums; attn_bwd_kv_reduce_kernel adds them in
//    range order (still deterministic).  Products are taken with the rows of the
//    MFMA accumulator being query rows and its columns keys (a lane owns one
//    key): S = Q K^T and dP = dO V^T read Q and dO from LDS as A operands;
//    dV^T = dO^T P and dK^T = Q^T dS read dO^T and Q^T with the LDS transpose
//    read, while P and dS, rounded to bf16, are the B operands exactly as the
//    accumulator holds them (the query order this implies is the order the
//    transpose read returns).
//    With one wave per SIMD nothing hides a wave's own stalls, so the 32-row
//    blocks are software-pipelined: the softmax VALU of block b issues
//    between the MFMAs of block b-1's dV/dK products and block b+1's S/dP
//    products.  Every MFMA is a compiler builtin, so the compiler sees the
//    accumulators' latencies (it places them in AGPRs, next to K and V).
//  * attn_bwd_dq_kernel: the forward's layout (a lane owns one (row, head)
//    pair of a kv group, K/V tiles stream through LDS): S^T = K Q^T,
//    dP^T = V dO^T, dS^T = P^T (dP^T - Dl), dQ^T += K^T dS^T with K^T from the
//    transpose read.
// Tiles read both row-wise (16-byte chunks) and with the transpose read use
// a swizzle that is conflict-free for both patterns (bwd_swz below).
#pragma once

#include "attn_fwd_kernel.hpp"

namespace ea02 {

typedef float f32x2 __attribute__((ext_vector_type(2)));

template <class T>
struct IsSlotC {
  static constexpr bool value = false;
};
template <int V>
struct IsSlotC<SlotC<V>> {
  static constexpr bool value = true;
};

struct BwdParams {
  const uint16_t* q;     // [B, H_q, N_q, D] bf16
  const uint16_t* k;     // [B, H_kv, N_kv, D]
  const uint16_t* v;     // [B, H_kv, N_kv, D]
  const uint16_t* o;     // [B, H_q, N_q, D]  (forward output)
  const uint16_t* dout;  // [B, H_q, N_q, D]
  const float* lse;      // [B, H_q, N_q] natural log (forward)
  uint16_t* dq;          // [B, H_q, N_q, D]
  uint16_t* dk;          // [B, H_kv, N_kv, D]
  uint16_t* dv;          // [B, H_kv, N_kv, D]
  float* lse2;           // [B, H_q, N_q] workspace: L log2(e)
  float* delta;          // [B, H_q, N_q] workspace: rowsum(dO * O)
  float* kv_part;        // [n_kv_splits, 2, B, H_kv, N_kv, D] fp32 workspace (dK scaled, dV)
                         // of the row-range splits; unused when n_kv_splits == 1
  float* q_part;         // [n_q_splits, B, H_q, N_q, D] fp32 workspace (dQ scaled) of the
                         // key-range splits; unused when n_q_splits == 1
  int B, H_q, H_kv, N_q, N_kv;
  int G;                 // H_q / H_kv
  int n_pairs;           // N_q * G
  int causal_off;        // N_kv - N_q when causal, else 0
  int causal;
  int n_heads_wg;        // B * H_kv
  int n_key_blocks;      // dK/dV kernel: ceil(N_kv / keys per workgroup)
  int n_kv_splits;       // dK/dV kernel: workgroups sharing one key block's row tiles
  int n_pair_blocks;     // dQ kernel: ceil(n_pairs / pairs per workgroup)
  int n_q_splits;        // dQ kernel: workgroups sharing one pair block's key tiles
  float scale_log2;      // max(|sm_scale| log2(e), FLT_MIN)
  float grad_scale;      // sm_scale (signed): factor of dQ and dK
  uint32_t k_sign;       // 0x80008000 when sm_scale < 0: K negated in S (dK/dV kernel)
  uint32_t q_sign;       // 0x80008000 when sm_scale < 0: Q negated in S^T (dQ kernel)
  int64_t rows;          // B * H_q * N_q
  // Work stealing between the XCDs (work_item): nine claim counters, zero
  // on entry and on exit, or null for the static order; per kernel, the
  // workgroups of the static order and how many of them keep their item.
  int* steal;
  int kv_items, kv_static;  // dK/dV kernel
  int q_items, q_static;    // dQ kernel
};

// 16-byte chunk swizzle for tiles read both row-wise (16 lanes, 16 rows, one
// chunk: the XOR must be a bijection on 16 (D=128) or, per row parity, 8 (D=64)
// consecutive rows) and with ds_read_b64_tr_b16 (a half wave reads 4 rows x 4
// chunks: the XOR must move those 4 rows into 4 different aligned 4-chunk
// groups (D=128) or row pairs of one parity into different halves (D=64)).
template <int D>
__device__ __forceinline__ int bwd_swz(int row) {
  if constexpr (D == 128) return 4 * (row & 3) + ((row >> 2) & 3);
  else return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
}

// 4 bytes per lane from the buffer at byte offset voff into LDS at lds_addr +
// 4 * lane (inline asm: not tracked by the compiler, see dma_16B).
__device__ __forceinline__ void dma_4B(u32x4 rsrc, int voff, uint32_t lds_addr) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}

// ---------------------------------------------------------------- prep
// One row per D/8 threads (16 bytes each): Dl = sum_d dO * O, L2 = L log2 e.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void attn_bwd_prep_kernel(BwdParams p) {
  constexpr int TPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < p.rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p.o + row * D + 8 * c);
    const u32x4 g = *reinterpret_cast<const u32x4*>(p.dout + row * D + 8 * c);
    const bf16x8 ab = as_bf16x8(a), gb = as_bf16x8(g);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)ab[e] * (float)gb[e];
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, TPR);
  if (row < p.rows && c == 0) {
    p.delta[row] = acc;
    p.lse2[row] = p.lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------- dK, dV
template <int D, int NW, int P, int BP>
struct BwdKvCfg {
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int DC = D / 8;                       // 16-byte chunks per row
  static constexpr int TILE_BYTES = BP * ROW_BYTES;      // Q or dO rows of one tile
  static constexpr int LOADS = TILE_BYTES / 1024;
  static constexpr int LPW = LOADS / NW;                 // 1 KiB loads per wave per tile and tensor
  static constexpr int RPL = 1024 / ROW_BYTES;           // rows per 1 KiB load
  static constexpr int STAT_BYTES = 2 * 4 * 64;          // per wave: L2 and Dl of up to 64 rows
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES + NW * STAT_BYTES;
  static constexpr int LDS_BYTES = P * STAGE_BYTES;
  static constexpr int GROUP_LOADS = 2 * LPW + 2;
  static_assert(BP == 32 || BP == 64, "tiles of 32 or 64 rows");
  static_assert(LOADS % NW == 0 && LPW >= 1, "tile loads split evenly over waves");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS ring fits the 160 KiB of a CU");
  static_assert((P - 1) * GROUP_LOADS <= 63, "loads in flight fit the 6-bit vmcnt");
};

template <int D, int NW, int P, int BP>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(1, 1)))
void attn_bwd_dkdv_kernel(BwdParams p) {
  using C = BwdKvCfg<D, NW, P, BP>;
  constexpr int BK = 32 * NW;   // keys per workgroup
  constexpr int NBLK = BP / 32; // 32-row blocks per tile
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // heaviest key blocks first (causal: block 0 sees every row), kv heads
  // fastest, then the row-range splits of one key block; item bid of that
  // order, possibly claimed from another XCD's list (work_item)
  __shared__ int claimed;
  const int bid = work_item(p.steal, p.kv_items, p.kv_static, wave, lane, claimed);
  if (bid < 0) return;
  const int head_wg = bid % p.n_heads_wg;
  const int rest = bid / p.n_heads_wg;
  const int split = rest % p.n_kv_splits;
  const int kb = rest / p.n_kv_splits;
  const int g = head_wg % p.H_kv;
  const int b = head_wg / p.H_kv;
  const int G = p.G;
  const int N_q = p.N_q, N_kv = p.N_kv;
  const int off = p.causal_off;
  const int k0 = kb * BK;
  const int kw = k0 + 32 * wave;     // first key of this wave
  const int my_key = kw + col;

  // rows before r_start see no key of this block; row tiles of BP (r_start
  // aligned down to a tile, so every key block shares one tile grid; the
  // rows it adds see none of the block's keys and are masked)
  const int r_start = p.causal ? max(0, k0 - off) / BP * BP : 0;
  const int n_rt = (N_q - r_start + BP - 1) / BP;
  const int n_tiles = G * n_rt;
  // this workgroup's contiguous range of the G * n_rt (head, row tile) tiles
  const int t_lo = (int)(((int64_t)n_tiles * split) / p.n_kv_splits);
  const int t_hi = (int)(((int64_t)n_tiles * (split + 1)) / p.n_kv_splits);

  // K and V of this lane's key: B operands of S = Q K^T and dP = dO V^T
  const size_t kv_base = ((size_t)b * p.H_kv + g) * (size_t)N_kv * D;
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const size_t kr = kv_base + (size_t)min(my_key, N_kv - 1) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 x = *reinterpret_cast<const u32x4*>(p.k + kr + ks * 16 + half * 8);
      x ^= p.k_sign;
      kf[ks] = as_bf16x8(x);
      vf[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(p.v + kr + ks * 16 + half * 8));
    }
  }
  // K and V are MFMA B operands only: kept in AGPRs (an MFMA reads them there)
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+a"(kf[ks]), "+a"(vf[ks]));

  // Q, dO, L2 and Dl of the kv group's G heads: [G, N_q, ...] contiguous.
  // Each tile is read through buffer resources that start at its first row
  // and end at the group's last row: the lane offsets are loop constants and
  // rows past the end come back as zeros (rows past N_q of a head read the
  // next head's rows; both kinds are masked).
  const size_t qg_rows = ((size_t)b * p.H_q + (size_t)g * G) * (size_t)N_q;
  const int group_rows = G * N_q;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)lds;
  const int ld_row_in = lane / C::DC;
  const int ld_chunk = lane % C::DC;
  // tile t of the sequence: row tiles from the last one down, the G heads of
  // a row tile in turn.  Workgroups that run at the same time then read the
  // same Q and dO rows at the same time and the L2 serves all but the first
  // (walking up from each block's own first row spread them over thousands
  // of rows: 36 % of the reads went past the L2 at causal N = 32768).
  auto tile_rows = [&](int t, int& hs, int& row0) {
    const int g = t / G;
    hs = t - g * G;
    row0 = r_start + (n_rt - 1 - g) * BP;
  };
  // one tile (Q, dO, and this wave's private copy of L2 and Dl) into stage slot
  int ld_off[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int r = (wave * C::LPW + i) * C::RPL + ld_row_in;
    ld_off[i] = r * C::ROW_BYTES + ((ld_chunk ^ bwd_swz<D>(r)) << 4);
  }
  const int st_off = min(lane, BP - 1) * 4;
  auto issue = [&](int t, int slot) {
    int hs, row0;
    tile_rows(t, hs, row0);
    const int first = hs * N_q + row0;  // first row of the tile in the group
    const size_t at = qg_rows + (size_t)first;
    const uint32_t rows_left = (uint32_t)(group_rows - first);
    const u32x4 q_rsrc = make_rsrc(p.q + at * D, rows_left * C::ROW_BYTES);
    const u32x4 do_rsrc = make_rsrc(p.dout + at * D, rows_left * C::ROW_BYTES);
    const uint32_t st = lds_base + slot * C::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int li = wave * C::LPW + i;
      dma_16B(q_rsrc, ld_off[i], st + li * 1024);
      dma_16B(do_rsrc, ld_off[i], st + C::TILE_BYTES + li * 1024);
    }
    const uint32_t sb = st + 2 * C::TILE_BYTES + wave * C::STAT_BYTES;
    dma_4B(make_rsrc(p.lse2 + at, rows_left * 4), st_off, sb);
    dma_4B(make_rsrc(p.delta + at, rows_left * 4), st_off, sb + 256);
  };


  f32x16 dkT[D / 32], dvT[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dkT[db] = f32x16{};
    dvT[db] = f32x16{};
  }
  const float sl2 = p.scale_log2;

  // Software pipeline over the 32-row blocks b of the workgroup's tiles
  // (block b is rows 32 (b % 2) .. of the range's tile b / 2).  Per block:
  //   A(b): S and dP (D/8 MFMAs on Q and dO rows read from LDS),
  //   E(b): P = 2^(S scale - L2) and dS = P (dP - Dl) (the VALU, one
  //         exponential per element), rounded to bf16,
  //   B(b): dV^T += dO^T P and dK^T += Q^T dS (D/8 MFMAs on transpose reads).
  // Phase b runs B(b-1) and then A(b+1) with the elements of E(b) spread over
  // both, so the softmax VALU of a block issues under the MFMAs of its
  // neighbours: with one wave per SIMD no other wave would hide it.  S and dP
  // of a block are held for one phase, P and dS for the next; even blocks use
  // the first set of registers, odd blocks the second.
  constexpr int PF = 3;          // LDS operand prefetch distance (MFMA pairs)
  constexpr int NPAIR = D / 16;  // MFMA pairs of A (k-steps) and of B ((st, db) pairs)
  constexpr int NEL = 16;        // elements of E per lane and block
  static_assert(NEL % NPAIR == 0, "elements spread evenly over the MFMA pairs");

  // Per-lane LDS byte offsets of the operand reads: set 0 relative to stage
  // 0, set 1 to stage 2 (kept opaque: two stages do not fit the 16-bit
  // immediate of an LDS instruction).  The steady-state loop is unrolled by
  // the ring depth, so a read knows its stage at compile time and takes the
  // rest of its address (stage parity, block, step, tensor) as the immediate.
  // Transpose reads: rows 16 st + 4 half + L/4 (+8 for the second read),
  // d = db*32 + 16 (G16 & 1) + 4 (L & 3); the swizzle of those rows does not
  // depend on st.  Row reads: 16-byte chunk 2 ks + half of row 32 c + col (the
  // swizzle does not depend on c).  Row statistics: this wave's copy, rows
  // 4 half .. of a block.
  const int L16 = lane & 15;
  int tr_off[2][2][D / 32], rr_off[2][NPAIR], stat_off[2];
#pragma unroll
  for (int set = 0; set < 2; ++set) {
    const int base = set * 2 * C::STAGE_BYTES;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int row = 4 * half + (L16 >> 2) + 8 * hi;
        const int d = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (L16 & 3);
        const int o = row * C::ROW_BYTES + (((d >> 3) ^ bwd_swz<D>(row)) << 4) + (d & 7) * 2;
        tr_off[set][hi][db] = set ? opaque_vgpr(base + o) : o;
      }
#pragma unroll
    for (int ks = 0; ks < NPAIR; ++ks) {
      const int o = col * C::ROW_BYTES + (((2 * ks + half) ^ bwd_swz<D>(col)) << 4);
      rr_off[set][ks] = set ? opaque_vgpr(base + o) : o;
    }
    const int o = 2 * C::TILE_BYTES + wave * C::STAT_BYTES + 16 * half;
    stat_off[set] = set ? opaque_vgpr(base + o) : o;
  }
  // offset set and immediate stage offset of a ring slot (SlotC: known at
  // compile time; int: set 0 and a run-time offset)
  auto sset = [&](auto slot) {
    if constexpr (IsSlotC<decltype(slot)>::value) return decltype(slot)::value >> 1;
    else return 0;
  };
  auto sbase = [&](auto slot) {
    if constexpr (IsSlotC<decltype(slot)>::value) return (decltype(slot)::value & 1) * C::STAGE_BYTES;
    else return int(slot) * C::STAGE_BYTES;
  };
  // rows c*32 .. of Q (tensor 0) or dO (tensor 1), transposed: the A operand
  // of step st, d block db
  auto tr_read = [&](auto slot, int tensor, int c, int st, int db) {
    const int imm = sbase(slot) + tensor * C::TILE_BYTES + (c * 32 + 16 * st) * C::ROW_BYTES;
    const uint8_t* a = lds + imm;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + tr_off[sset(slot)][0][db]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + tr_off[sset(slot)][1][db]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // row c*32 + col of Q (tensor 0) or dO (tensor 1), chunk 2 ks + half
  auto row_read = [&](auto slot, int tensor, int c, int ks) {
    const int imm = sbase(slot) + tensor * C::TILE_BYTES + c * 32 * C::ROW_BYTES;
    return as_bf16x8(*reinterpret_cast<const u32x4*>(lds + imm + rr_off[sset(slot)][ks]));
  };

  auto a_part = [&](auto slot, int c, f32x16& s, f32x16& dp, auto&& hook) {
    s = f32x16{};
    dp = f32x16{};
    bf16x8 qx[PF + 1], ox[PF + 1];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      qx[i] = row_read(slot, 0, c, i);
      ox[i] = row_read(slot, 1, c, i);
    }
#pragma unroll
    for (int ks = 0; ks < NPAIR; ++ks) {
      if (ks + PF < NPAIR) {
        qx[(ks + PF) % (PF + 1)] = row_read(slot, 0, c, ks + PF);
        ox[(ks + PF) % (PF + 1)] = row_read(slot, 1, c, ks + PF);
      }
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qx[ks % (PF + 1)], kf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ox[ks % (PF + 1)], vf[ks], dp, 0, 0, 0);
      hook(ks);
    }
  };
  auto b_part = [&](auto slot, int c, const u32x4* pb, const u32x4* dsb, auto&& hook) {
    bf16x8 qx[PF + 1], ox[PF + 1];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      ox[i] = tr_read(slot, 1, c, i / (D / 32), i % (D / 32));
      qx[i] = tr_read(slot, 0, c, i / (D / 32), i % (D / 32));
    }
#pragma unroll
    for (int i = 0; i < NPAIR; ++i) {
      if (i + PF < NPAIR) {
        ox[(i + PF) % (PF + 1)] = tr_read(slot, 1, c, (i + PF) / (D / 32), (i + PF) % (D / 32));
        qx[(i + PF) % (PF + 1)] = tr_read(slot, 0, c, (i + PF) / (D / 32), (i + PF) % (D / 32));
      }
      const int st = i / (D / 32), db = i % (D / 32);
      dvT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ox[i % (PF + 1)], as_bf16x8(pb[st]), dvT[db], 0, 0, 0);
      dkT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qx[i % (PF + 1)], as_bf16x8(dsb[st]), dkT[db], 0, 0, 0);
      hook(i);
    }
  };
  // masked tile (a wave-uniform test): rows that cannot see some key of this
  // wave, or rows past N_q; their scores become -inf, so P and dS are 0
  auto mask_block = [&](int t, int c, f32x16& s) {
    int hs, row0;
    tile_rows(t, hs, row0);
    if ((p.causal && row0 + off < kw + 31) || row0 + BP > N_q) {
      // element r holds query row row0 + c*32 + 8(r/4) + 4 half + r%4
      const int lo_vis = my_key - off - row0 - c * 32 - 4 * half;  // visible: index >= lo_vis
      const int hi_vis = N_q - row0 - c * 32 - 4 * half;           // and index < hi_vis
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int idx = 8 * (r >> 2) + (r & 3);
        if ((p.causal && idx < lo_vis) || idx >= hi_vis) s[r] = -INFINITY;
      }
    }
  };
  // phase of block b: B(b-1) (HAS_PREV) with elements [0, EA) of E(b), then
  // A(b+1) (HAS_NEXT) with the rest
  auto phase = [&](auto has_prev_tag, auto has_next_tag, auto slot_prev, const u32x4* pb_prev, const u32x4* ds_prev,
                   auto slot_cur, int c_cur, const f32x16& s_cur, const f32x16& dp_cur, u32x4* pb_cur,
                   u32x4* ds_cur, auto slot_next, int c_next, f32x16& s_next, f32x16& dp_next) {
    constexpr bool HAS_PREV = decltype(has_prev_tag)::value;
    constexpr bool HAS_NEXT = decltype(has_next_tag)::value;
    constexpr int EA = HAS_PREV ? (HAS_NEXT ? NEL / 2 : NEL) : 0;
    static_assert(EA % NPAIR == 0 && (NEL - EA) % NPAIR == 0, "whole elements per MFMA pair");
    // this lane's rows' L2 and Dl (element r: row 8(r/4) + 4 half + r%4 of
    // the block), read per half of the elements as they are needed
    const uint8_t* stl = lds + sbase(slot_cur) + c_cur * 32 * 4 + stat_off[sset(slot_cur)];
    f32x4 l4[2], d4[2];
    auto read_stats = [&](int h) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        l4[j] = *reinterpret_cast<const f32x4*>(stl + 32 * (2 * h + j));
        d4[j] = *reinterpret_cast<const f32x4*>(stl + 256 + 32 * (2 * h + j));
      }
    };
    // P and dS of elements r-1, r packed to bf16 pairs as soon as both exist
    float pe_odd = 0.f, sf_odd = 0.f;
    auto e_elem = [&](int r) {
      if ((r & 7) == 0) read_stats(r >> 3);
      const int j = (r >> 2) & 1;
      const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r], sl2, -l4[j][r & 3]));
      const float sv = pe * (dp_cur[r] - d4[j][r & 3]);
      if ((r & 1) == 0) {
        pe_odd = pe;
        sf_odd = sv;
      } else {
        const f32x2 pp = {pe_odd, pe}, ss = {sf_odd, sv};
        pb_cur[r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pp, bf16x2));
        ds_cur[r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(ss, bf16x2));
        // packed here, not carried as fp32 into the next phase
        if ((r & 7) == 7) asm volatile("" : "+v"(pb_cur[r >> 3]), "+v"(ds_cur[r >> 3]));
      }
    };
    if constexpr (HAS_PREV)
      b_part(slot_prev, 1 - c_cur, pb_prev, ds_prev, [&](int i) {
#pragma unroll
        for (int e = 0; e < EA / NPAIR; ++e) e_elem(i * (EA / NPAIR) + e);
      });
    if constexpr (HAS_PREV && HAS_NEXT) __builtin_amdgcn_sched_barrier(0);
    if constexpr (HAS_NEXT)
      a_part(slot_next, c_next, s_next, dp_next, [&](int i) {
#pragma unroll
        for (int e = 0; e < (NEL - EA) / NPAIR; ++e) e_elem(EA + i * ((NEL - EA) / NPAIR) + e);
      });
    if constexpr (!HAS_PREV && !HAS_NEXT) {
#pragma unroll
      for (int r = 0; r < NEL; ++r) e_elem(r);
    }
  };
  auto no_hook = [](int) {};

  // Load ring: the i-th tile of the range goes to slot i % P.  The phase of
  // block 2i+1 opens with a barrier after which tile i+1 (read there by
  // A(2i+2)) has landed and tile i-1 (last read by B(2i-1) in the phase
  // before) is no longer read: tile i+P-1 is issued into its slot.  Past the
  // range's end a clamped tile is re-loaded so every wait is one constant
  // vmcnt.
  static_assert(NBLK == 2 && P == 4, "two 32-row blocks per tile; a ring of four tiles");
  const int n_mine = t_hi - t_lo;
  if (n_mine > 0) {
#pragma unroll
    for (int j = 0; j < P - 1; ++j) issue(t_lo + min(j, n_mine - 1), j);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((P - 2) * C::GROUP_LOADS) : "memory");
    __syncthreads();
    f32x16 s0, dp0, s1, dp1;
    u32x4 p0[2], d0[2], p1[2], d1[2];
    auto barrier_issue = [&](int i) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((P - 3) * C::GROUP_LOADS) : "memory");
      __syncthreads();
      issue(t_lo + min(i + P - 1, n_mine - 1), (i + P - 1) % P);
    };
    // both blocks of tile i (0 < i < n_mine - 1), in slot sc; tile i-1 in
    // slot sp, tile i+1 in slot sn
    auto steady_tile = [&](int i, auto sp, auto sc, auto sn) {
      phase(BoolTag<true>{}, BoolTag<true>{}, sp, p1, d1, sc, 0, s0, dp0, p0, d0, sc, 1, s1, dp1);
      mask_block(t_lo + i, 1, s1);
      barrier_issue(i);
      phase(BoolTag<true>{}, BoolTag<true>{}, sc, p0, d0, sc, 1, s1, dp1, p1, d1, sn, 0, s0, dp0);
      mask_block(t_lo + i + 1, 0, s0);
    };
    // tile 0: A(0); block 0 (no B before it); block 1
    a_part(SlotC<0>{}, 0, s0, dp0, no_hook);
    mask_block(t_lo, 0, s0);
    phase(BoolTag<false>{}, BoolTag<true>{}, SlotC<0>{}, nullptr, nullptr, SlotC<0>{}, 0, s0, dp0, p0, d0, SlotC<0>{},
          1, s1, dp1);
    mask_block(t_lo, 1, s1);
    int i = 1;
    if (n_mine > 1) {
      barrier_issue(0);
      phase(BoolTag<true>{}, BoolTag<true>{}, SlotC<0>{}, p0, d0, SlotC<0>{}, 1, s1, dp1, p1, d1, SlotC<1>{}, 0, s0,
            dp0);
      mask_block(t_lo + 1, 0, s0);
      // steady state from tile 1, unrolled by the ring depth: tile i = 1 mod 4
      // sits in slot 1, and every operand read takes its slot as an immediate
      for (; i + 4 < n_mine; i += 4) {
        steady_tile(i, SlotC<0>{}, SlotC<1>{}, SlotC<2>{});
        steady_tile(i + 1, SlotC<1>{}, SlotC<2>{}, SlotC<3>{});
        steady_tile(i + 2, SlotC<2>{}, SlotC<3>{}, SlotC<0>{});
        steady_tile(i + 3, SlotC<3>{}, SlotC<0>{}, SlotC<1>{});
      }
      for (; i + 1 < n_mine; ++i) steady_tile(i, (i + P - 1) % P, i % P, (i + 1) % P);
      // last tile: block 0 as in the steady state
      phase(BoolTag<true>{}, BoolTag<true>{}, (i + P - 1) % P, p1, d1, i % P, 0, s0, dp0, p0, d0, i % P, 1, s1, dp1);
      mask_block(t_lo + i, 1, s1);
    } else {
      i = 0;
    }
    // the last block: no A after it
    barrier_issue(i);
    phase(BoolTag<true>{}, BoolTag<false>{}, i % P, p0, d0, i % P, 1, s1, dp1, p1, d1, 0, 0, s0, dp0);
    b_part(i % P, 1, p1, d1, no_hook);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may outlive the workgroup
  }

  // dK^T, dV^T: the lane holds key my_key, d = db*32 + 8(r/4) + 4 half + r%4.
  // A split writes its fp32 partial sums (a range with no tile writes zeros).
  if (p.n_kv_splits > 1) {
    if (my_key < N_kv) {
      const size_t plane = (size_t)p.n_heads_wg * N_kv * D;
      float* pk = p.kv_part + 2 * (size_t)split * plane + kv_base + (size_t)my_key * D;
      float* pv = pk + plane;
      const float gs = p.grad_scale;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = db * 32 + 8 * g4 + 4 * half;
          f32x4 fk = {dkT[db][4 * g4] * gs, dkT[db][4 * g4 + 1] * gs, dkT[db][4 * g4 + 2] * gs, dkT[db][4 * g4 + 3] * gs};
          f32x4 fv = {dvT[db][4 * g4], dvT[db][4 * g4 + 1], dvT[db][4 * g4 + 2], dvT[db][4 * g4 + 3]};
          *reinterpret_cast<f32x4*>(pk + d0) = fk;
          *reinterpret_cast<f32x4*>(pv + d0) = fv;
        }
    }
  } else if (my_key < N_kv) {
    uint16_t* dkr = p.dk + kv_base + (size_t)my_key * D;
    uint16_t* dvr = p.dv + kv_base + (size_t)my_key * D;
    const float gs = p.grad_scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * half;
        f32x4 fk = {dkT[db][4 * g4] * gs, dkT[db][4 * g4 + 1] * gs, dkT[db][4 * g4 + 2] * gs, dkT[db][4 * g4 + 3] * gs};
        f32x4 fv = {dvT[db][4 * g4], dvT[db][4 * g4 + 1], dvT[db][4 * g4 + 2], dvT[db][4 * g4 + 3]};
        *reinterpret_cast<u32x2*>(dkr + d0) = __builtin_bit_cast(u32x2, __builtin_convertvector(fk, bf16x4));
        *reinterpret_cast<u32x2*>(dvr + d0) = __builtin_bit_cast(u32x2, __builtin_convertvector(fv, bf16x4));
      }
  }
}

// ---------------------------------------------------------------- split sums
// dK, dV = sum over the row-range splits of the partials, in split order;
// 4 elements per thread (16-byte loads), rounded to bf16 when stored.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void attn_bwd_kv_reduce_kernel(BwdParams p) {
  const size_t plane = (size_t)p.n_heads_wg * p.N_kv * D;
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= plane) return;
  f32x4 sk = *reinterpret_cast<const f32x4*>(p.kv_part + i);
  f32x4 sv = *reinterpret_cast<const f32x4*>(p.kv_part + plane + i);
  for (int s = 1; s < p.n_kv_splits; ++s) {
    sk += *reinterpret_cast<const f32x4*>(p.kv_part + 2 * (size_t)s * plane + i);
    sv += *reinterpret_cast<const f32x4*>(p.kv_part + (2 * (size_t)s + 1) * plane + i);
  }
  *reinterpret_cast<u32x2*>(p.dk + i) = __builtin_bit_cast(u32x2, __builtin_convertvector(sk, bf16x4));
  *reinterpret_cast<u32x2*>(p.dv + i) = __builtin_bit_cast(u32x2, __builtin_convertvector(sv, bf16x4));
}

// dQ = sum over the key-range splits of the partials, in split order; 4
// elements per thread, rounded to bf16 when stored.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void attn_bwd_q_reduce_kernel(BwdParams p) {
  const size_t plane = (size_t)p.rows * D;
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= plane) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(p.q_part + i);
  for (int sp = 1; sp < p.n_q_splits; ++sp) s += *reinterpret_cast<const f32x4*>(p.q_part + (size_t)sp * plane + i);
  *reinterpret_cast<u32x2*>(p.dq + i) = __builtin_bit_cast(u32x2, __builtin_convertvector(s, bf16x4));
}

// ---------------------------------------------------------------- dQ
template <int D, int NW, int P, int BN>
struct BwdQCfg {
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int DC = D / 8;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;
  static constexpr int LOADS = TILE_BYTES / 1024;
  static constexpr int LPW = LOADS / NW;
  static constexpr int RPL = 1024 / ROW_BYTES;
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;   // K then V
  static constexpr int LDS_BYTES = P * STAGE_BYTES;
  static constexpr int GROUP_LOADS = 2 * LPW;
  static_assert(BN == 32 || BN == 64, "key tiles of 32 or 64");
  static_assert(LOADS % NW == 0 && LPW >= 1, "tile loads split evenly over waves");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS ring fits the 160 KiB of a CU");
  static_assert((P - 1) * GROUP_LOADS <= 63, "loads in flight fit the 6-bit vmcnt");
};

// Two waves per SIMD: eight waves share one workgroup's LDS ring, or four
// waves with two stages leave room for a second workgroup on the CU; one
// wave's exponentials and dS run while the other's MFMAs issue (the register
// budget, 256 per wave, still holds the 32-pair accumulators without spilling).
// MN: MFMA size as in the forward, 16 (v_mfma_f32_16x16x32_bf16: a lane owns
// two pairs, the long power-bound launches) or 32 (v_mfma_f32_32x32x16_bf16).
// K and V rows use the forward's swizzle for MN = 16 (its 16x16 transpose
// reads cover 8 rows x 2 chunks) and bwd_swz for MN = 32.
template <int D, int MN>
__device__ __forceinline__ int dq_swz(int row) {
  if constexpr (MN == 16) return kv16_swz<D>(row);
  else return bwd_swz<D>(row);
}
template <int D, int NW, int P, int BN, int MN>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu((NW >= 8 || P <= 2) ? 2 : 1, (NW >= 8 || P <= 2) ? 2 : 1)))
void attn_bwd_dq_kernel(BwdParams p) {
  using C = BwdQCfg<D, NW, P, BN>;
  constexpr int PPW = 32 * NW;        // (row, head) pairs per workgroup
  constexpr int KK = 512 / MN;        // contraction length of one MFMA
  constexpr int ACC = MN * MN / 64;   // accumulator registers per lane and MFMA block
  constexpr int QC = 32 / MN;         // pair column blocks per wave
  using AccT = typename MfmaAcc<MN>::type;
  static_assert(MN == 16 || MN == 32, "MFMA 16x16x32 or 32x32x16");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // lane = MN kgrp + col: operand row/column col, contraction slots 8 kgrp ..
  // +7; result column col, rows (r / 4)(256 / MN) + 4 kgrp + r % 4
  const int kgrp = lane / MN;
  const int col = lane % MN;

  // heaviest pair blocks first (causal: the last rows see every key), kv
  // heads fastest, then the key-range splits of one pair block; item bid of
  // that order, possibly claimed from another XCD's list (work_item)
  __shared__ int claimed;
  const int bid = work_item(p.steal, p.q_items, p.q_static, wave, lane, claimed);
  if (bid < 0) return;
  const int head_wg = bid % p.n_heads_wg;
  const int rest = bid / p.n_heads_wg;
  const int qsplit = rest % p.n_q_splits;
  const int pb = p.n_pair_blocks - 1 - rest / p.n_q_splits;
  const int g = head_wg % p.H_kv;
  const int b = head_wg / p.H_kv;
  const int G = p.G;
  const int N_kv = p.N_kv;
  const int off = p.causal_off;
  const int last_pair = p.n_pairs - 1;
  const int P0 = pb * PPW;
  const int wp0 = P0 + wave * 32;
  const int wave_row0 = min(wp0, last_pair) / G;
  const int wg_row_end = min(P0 + PPW - 1, last_pair) / G + 1;
  const int kv_end = p.causal ? min(wg_row_end + off, N_kv) : N_kv;
  const int n_tiles = (kv_end + BN - 1) / BN;
  // this workgroup's contiguous range of those key tiles
  const int t_lo = (int)(((int64_t)n_tiles * qsplit) / p.n_q_splits);
  const int t_hi = (int)(((int64_t)n_tiles * (qsplit + 1)) / p.n_q_splits);
  const int n_mine = t_hi - t_lo;

  // this lane's pairs (one per column block): Q and dO fragments (B
  // operands), L2 and Dl
  auto bhr_of = [&](int qc) {
    const int pc = min(wp0 + MN * qc + col, last_pair);
    const int row = pc / G;
    const int h = g * G + (pc - row * G);
    return ((size_t)b * p.H_q + h) * (size_t)p.N_q + row;
  };
  auto row_of = [&](int qc) { return min(wp0 + MN * qc + col, last_pair) / G; };
  bf16x8 qf[QC][D / KK], df[QC][D / KK];
  float l2[QC], dl[QC];
#pragma unroll
  for (int qc = 0; qc < QC; ++qc) {
    const size_t bhr = bhr_of(qc);
#pragma unroll
    for (int ks = 0; ks < D / KK; ++ks) {
      u32x4 x = *reinterpret_cast<const u32x4*>(p.q + bhr * D + ks * KK + kgrp * 8);
      x ^= p.q_sign;
      qf[qc][ks] = as_bf16x8(x);
      df[qc][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(p.dout + bhr * D + ks * KK + kgrp * 8));
    }
    l2[qc] = p.lse2[bhr];
    dl[qc] = p.delta[bhr];
  }

  // each K/V tile through buffer resources that start at its first key and
  // end at the head's last key: lane offsets are loop constants and keys past
  // the end come back as zeros (masked)
  const size_t kv_base = ((size_t)b * p.H_kv + g) * (size_t)N_kv * D;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)lds;
  const int ld_row_in = lane / C::DC;
  const int ld_chunk = lane % C::DC;
  int ld_off[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int r = (wave * C::LPW + i) * C::RPL + ld_row_in;
    ld_off[i] = r * C::ROW_BYTES + ((ld_chunk ^ dq_swz<D, MN>(r)) << 4);
  }
  auto issue = [&](int t, int slot) {
    const size_t at = kv_base + (size_t)t * BN * D;
    const uint32_t bytes_left = (uint32_t)(N_kv - t * BN) * C::ROW_BYTES;
    const u32x4 k_rsrc = make_rsrc(p.k + at, bytes_left);
    const u32x4 v_rsrc = make_rsrc(p.v + at, bytes_left);
    const uint32_t st = lds_base + slot * C::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int li = wave * C::LPW + i;
      dma_16B(k_rsrc, ld_off[i], st + li * 1024);
      dma_16B(v_rsrc, ld_off[i], st + C::TILE_BYTES + li * 1024);
    }
  };

  // K^T (A operand of dQ^T, MN d x KK keys) from the transpose read: lane
  // row d = MN db + col; contraction slots are the keys KK st + 4 kgrp +
  // {0..3} (first read) and + KK/2 (second), the keys whose dS this lane
  // holds in 8 consecutive accumulator registers.  Lane L of a 16-lane group
  // addresses row 4 kgrp + L/4, d = d16 + 4 (L & 3) .. +4.
  const int L16 = lane & 15;
  int tr_off[2][D / MN];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int db = 0; db < D / MN; ++db) {
      const int row = 4 * kgrp + (L16 >> 2) + (KK / 2) * hi;
      const int d = db * MN + 16 * ((lane >> 4) % (MN / 16)) + 4 * (L16 & 3);
      tr_off[hi][db] = row * C::ROW_BYTES + (((d >> 3) ^ dq_swz<D, MN>(row)) << 4) + (d & 7) * 2;
    }

  AccT dqT[D / MN][QC];
#pragma unroll
  for (int db = 0; db < D / MN; ++db)
#pragma unroll
    for (int qc = 0; qc < QC; ++qc) dqT[db][qc] = AccT{};
  const float sl2 = p.scale_log2;

  auto compute = [&](int t, int slot) {
    const uint8_t* kt = lds + slot * C::STAGE_BYTES;
    const uint8_t* vt = kt + C::TILE_BYTES;
    const int key0 = t * BN;
    const bool masked = (p.causal && key0 + BN - 1 > wave_row0 + off) || key0 + BN > N_kv;
    // dS of the tile in bf16, 8 consecutive accumulator registers per entry
    // (key-block-major), the B operands of dQ^T
    bf16x8 dsb[QC][BN / KK];
    f32x8 sf[QC];
#pragma unroll
    for (int c = 0; c < BN / MN; ++c) {
      AccT s[QC], dp[QC];
#pragma unroll
      for (int qc = 0; qc < QC; ++qc) s[qc] = dp[qc] = AccT{};
      const int key = c * MN + col;
#pragma unroll
      for (int ks = 0; ks < D / KK; ++ks) {
        const int chunk = (((KK / 8) * ks + kgrp) ^ dq_swz<D, MN>(key)) << 4;
        const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + key * C::ROW_BYTES + chunk));
        const bf16x8 va = as_bf16x8(*reinterpret_cast<const u32x4*>(vt + key * C::ROW_BYTES + chunk));
#pragma unroll
        for (int qc = 0; qc < QC; ++qc) {
          s[qc] = mfma_bf16<MN>(ka, qf[qc][ks], s[qc]);
          dp[qc] = mfma_bf16<MN>(va, df[qc][ks], dp[qc]);
        }
      }
#pragma unroll
      for (int qc = 0; qc < QC; ++qc) {
        // masked tiles only (a wave-uniform branch): invisible scores become
        // -inf, so their dS is 0 with no per-element test below.  Element r
        // holds key key0 + MN c + (r/4)(256/MN) + 4 kgrp + r%4.
        if (masked) {
          const int lim = (p.causal ? min(row_of(qc) + off + 1, N_kv) : N_kv) - key0 - 4 * kgrp;
#pragma unroll
          for (int r = 0; r < ACC; ++r)
            if (c * MN + (r >> 2) * (256 / MN) + (r & 3) >= lim) s[qc][r] = -INFINITY;
        }
#pragma unroll
        for (int r = 0; r < ACC; ++r) {
          const int e = c * ACC + r;
          const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qc][r], sl2, -l2[qc]));
          sf[qc][e & 7] = pe * (dp[qc][r] - dl[qc]);
          if ((e & 7) == 7) dsb[qc][e >> 3] = __builtin_convertvector(sf[qc], bf16x8);
        }
      }
    }
    // dQ^T += K^T dS^T; step st covers keys KK st .. KK st + KK - 1
#pragma unroll
    for (int st = 0; st < BN / KK; ++st)
#pragma unroll
      for (int db = 0; db < D / MN; ++db) {
        const uint8_t* a = kt + (KK * st) * C::ROW_BYTES;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + tr_off[0][db]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + tr_off[1][db]));
        const bf16x8 kT = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qc = 0; qc < QC; ++qc) dqT[db][qc] = mfma_bf16<MN>(kT, dsb[qc][st], dqT[db][qc]);
      }
  };

  // load ring over the range: its i-th tile goes to slot i % P
  if (n_mine > 0) {
#pragma unroll
    for (int j = 0; j < P - 1; ++j) issue(t_lo + min(j, n_mine - 1), j);
    for (int i = 0; i < n_mine; ++i) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((P - 2) * C::GROUP_LOADS) : "memory");
      __syncthreads();
      issue(t_lo + min(i + P - 1, n_mine - 1), (i + P - 1) % P);
      compute(t_lo + i, i % P);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // a split writes its fp32 partial (a range with no tile writes zeros);
  // register 4 g4 + j of dqT[db] holds d = MN db + g4 (256/MN) + 4 kgrp + j
  const float gs = p.grad_scale;
#pragma unroll
  for (int qc = 0; qc < QC; ++qc) {
    if (wp0 + MN * qc + col > last_pair) continue;
    const size_t bhr = bhr_of(qc);
#pragma unroll
    for (int db = 0; db < D / MN; ++db)
#pragma unroll
      for (int g4 = 0; g4 < ACC / 4; ++g4) {
        const int d0 = db * MN + g4 * (256 / MN) + 4 * kgrp;
        const f32x4 f = {dqT[db][qc][4 * g4] * gs, dqT[db][qc][4 * g4 + 1] * gs, dqT[db][qc][4 * g4 + 2] * gs,
                         dqT[db][qc][4 * g4 + 3] * gs};
        if (p.n_q_splits > 1)
          *reinterpret_cast<f32x4*>(p.q_part + ((size_t)qsplit * (size_t)p.rows + bhr) * D + d0) = f;
        else
          *reinterpret_cast<u32x2*>(p.dq + bhr * D + d0) = __builtin_bit_cast(u32x2, __builtin_convertvector(f, bf16x4));
      }
  }
}

}  // namespace ea02
