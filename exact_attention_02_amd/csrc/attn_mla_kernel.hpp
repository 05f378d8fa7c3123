// Multi-head latent attention (MLA) decode for gfx950: device code.
//
// Method (page "Attention Kernel 实现与正确性验证", section 2: 2.1 the
// absorption trick, 2.2 the reference with naive and absorbed forms, 2.3 the
// DeepSeek-V3 shapes, 2.4 FlashMLA decode with a split of the cache axis and
// a safe-softmax merge).  With W_uk absorbed into the query, every head
// attends over the same latent cache row kv = [c_kv (512), k_pe (64)]:
//   q_lat = [q_nope W_uk[h], q_pe]                     (mla_absorb_kernel)
//   out_lat = softmax(scale q_lat kv^T) c_kv           (attn_mla_kernel)
//   out = out_lat W_uv[h]^T                            (mla_up_kernel)
//
// attn_mla_kernel: MQA with 576-wide scores and 512-wide values.  A workgroup
// of four waves owns 64 (query token, head) pairs and streams 32-key tiles of
// the latent cache through a 4-stage LDS ring.  Wave w works on pair block
// w & 1 (32 pairs) and half h = w >> 1 of the problem:
//  * scores: k-steps [18 h, 18 h + 18) of S^T = K Q^T (16 dims each); the
//    two halves' fp32 partials meet in LDS and both waves add them (fp32
//    addition is commutative, so both hold the same S^T and take the same
//    online-softmax decisions: lazy rescale, as in the forward kernel);
//  * values: O^T for dims [256 h, 256 h + 256) with O^T += V^T P^T, V^T from
//    the LDS transpose read of the tile's first 512 columns and P^T the
//    bf16-rounded S^T accumulator.
// A wave thus holds 18 query k-steps and 256 value dims: 72 + 128 registers,
// where all 36 k-steps and 512 dims of a pair block in one wave would not fit.
//
// attn_mla16_kernel (below): the same computation with 16 pairs per wave,
// eight waves of two per SIMD and no exchange; the host takes it when the
// batch fills at least an eighth of the CUs before any split.
#pragma once

#include "attn_fwd_kernel.hpp"

namespace ea02 {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kMlaDc = 512;                 // latent (value) width
constexpr int kMlaDr = 64;                  // rotary width
constexpr int kMlaDqk = kMlaDc + kMlaDr;    // score width
constexpr int kMlaRowBytes = kMlaDqk * 2;   // 1152
constexpr int kMlaChunks = kMlaRowBytes / 16;  // 72

struct MlaParams {
  const uint16_t* q;   // [B, H, S, 576] bf16 (absorbed query)
  const uint16_t* kv;  // [B, T, 576] bf16 latent cache
  uint16_t* o;         // [B, H, S, 512] bf16 (single pass)
  float* lse;          // [B, H, S] natural log (single pass)
  uint16_t* o_part;    // [n_splits, B*H*S, 512] bf16 (split pass)
  float* lse_part;     // [n_splits, B*H*S] log2 units (split pass)
  int B, H, S, T;
  int n_pairs;         // S * H
  int causal_off;      // T - S when causal, else 0
  int n_pair_blocks;   // ceil(n_pairs / 64): workgroups per batch element and split
  int n_splits;
  float scale_log2;    // max(|sm_scale| log2 e, FLT_MIN)
  uint32_t q_sign;     // 0x80008000 when sm_scale < 0
  int causal;
};

// Chunk swizzle of a 1152-byte latent row (72 chunks: XOR values below 8 keep
// a chunk inside its aligned group of 8).  Rows 1152 bytes apart alternate
// between two bank halves, so 16 rows read at one chunk need distinct XORs
// per row parity; the transpose read (4 rows x 4 chunks per half wave) needs
// rows r and r+2 in different 4-chunk halves.
__device__ __forceinline__ int mla_swz(int row) { return 4 * ((row >> 1) & 1) + ((row >> 2) & 3); }

// acc *= alpha on an accumulator the MFMAs keep in AGPRs, each element read,
// scaled and written back by inline asm.  Written as plain VALU code, this
// rare rescale makes the compiler keep VGPR copies of all 128 accumulator
// registers and copy them on every tile, whether or not the rescale runs.
// The compiler does not see into the asm for MFMA hazards: the last MFMA
// that wrote acc (the previous tile's P V) is followed by the barrier and the
// whole score chain before this runs, and the two wait states after each
// write cover an MFMA reading it next.
__device__ __forceinline__ void scale_agpr(f32x16& acc, float alpha) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = acc[r];
    float tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1\n\ts_nop 1"
                 : "+a"(x), "=&v"(tmp)
                 : "v"(alpha));
    acc[r] = x;
  }
}

// The sixteen-pair kernel's (pair block, batch element, split).  Workgroup
// ids go round-robin over the 8 XCDs; they are renumbered so that each XCD
// takes a contiguous run of items, pair block fastest, then split: the pair
// blocks of one (batch, split) read the same cache tiles, and the splits of
// one pair block the same queries, through one XCD's L2 (B = 32: 8 % faster
// than the plain order).  The four-wave kernel keeps the plain order: this
// one measured 11 % slower for it at B = 1, T = 16384.
__device__ __forceinline__ int3 mla_item(const MlaParams& p) {
  const int nwg = gridDim.x;
  const int id = (nwg & 7) ? (int)blockIdx.x : (int)(blockIdx.x & 7) * (nwg >> 3) + (int)(blockIdx.x >> 3);
  const int pb = id % p.n_pair_blocks;
  const int r = id / p.n_pair_blocks;
  return int3{pb, r / p.n_splits, r % p.n_splits};
}

template <int P, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void attn_mla_kernel(MlaParams p) {
  constexpr int NW = 4;
  constexpr int BN = 32;
  constexpr int TILE_BYTES = BN * kMlaRowBytes;          // 36 KiB
  constexpr int LOADS = TILE_BYTES / 1024;               // 36
  constexpr int LPW = LOADS / NW;                        // 9
  constexpr int KSH = kMlaDqk / 16 / 2;                  // 18 k-steps per half
  constexpr int NDB = kMlaDc / 32 / 2;                   // 8 value blocks of 32 per half
  constexpr int PPW = 64;                                // pairs per workgroup
  constexpr int PART_BYTES = NW * 64 * 16 * 4;           // S^T partials, 16 KiB
  static_assert(LOADS % NW == 0 && (P - 1) * LPW <= 63, "load groups");
  static_assert(P * TILE_BYTES + PART_BYTES <= 160 * 1024, "LDS fits the 160 KiB of a CU");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[P * TILE_BYTES + PART_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;
  const int pbw = wave & 1;   // pair block of this wave
  const int kh = wave >> 1;   // half of the k-steps and of the value dims

  // pair blocks of one (batch, split) are B * n_splits apart in the grid so
  // that they share an XCD (and its L2) under round-robin dispatch
  const int bid = blockIdx.x;
  const int bs = bid % (p.B * p.n_splits);
  const int pb = bid / (p.B * p.n_splits);
  const int b = bs / p.n_splits;
  const int split = SPLIT ? bs % p.n_splits : 0;
  const int T = p.T;
  const int off = p.causal_off;
  const int last_pair = p.n_pairs - 1;
  const int P0 = pb * PPW;
  const int wp0 = P0 + 32 * pbw;
  const int wave_row0 = min(wp0, last_pair) / p.H;          // first query token of this wave
  const int row_end = min(P0 + PPW - 1, last_pair) / p.H + 1;

  const int kv_end = p.causal ? min(row_end + off, T) : T;
  int n_tiles = (kv_end + BN - 1) / BN;
  int kbase = 0;
  if constexpr (SPLIT) {
    const int per = (n_tiles + p.n_splits - 1) / p.n_splits;
    const int t0 = min(split * per, n_tiles);
    n_tiles = min(per, n_tiles - t0);
    kbase = t0 * BN;
  }

  // this lane's pair and its half of the query k-steps
  const int pair = wp0 + col;
  const bool valid = pair <= last_pair;
  const int pc = min(pair, last_pair);
  const int my_row = pc / p.H;
  const int h = pc - my_row * p.H;
  const size_t bhr = ((size_t)b * p.H + h) * (size_t)p.S + my_row;
  bf16x8 qf[KSH];
#pragma unroll
  for (int i = 0; i < KSH; ++i) {
    u32x4 x = *reinterpret_cast<const u32x4*>(p.q + bhr * kMlaDqk + (kh * KSH + i) * 16 + half * 8);
    x ^= p.q_sign;
    qf[i] = as_bf16x8(x);
  }

  // tile loads: load li moves bytes [1024 li, 1024 li + 1024) of the tile,
  // lane -> (row, stored chunk j) and fetches chunk j ^ swz(row) of that row
  // A load that no tile step reads (past the last tile) keeps its place in
  // the load count but gets an empty resource: no memory access.
  const u32x4 rsrc = make_rsrc(p.kv + (size_t)b * T * kMlaDqk, (uint32_t)((size_t)T * kMlaRowBytes));
  const u32x4 rsrc_none = make_rsrc(p.kv, 0u);
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)lds;
  auto issue = [&](int t, int slot) {
    const u32x4 rs = t < n_tiles ? rsrc : rsrc_none;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int e = (wave * LPW + i) * 64 + lane;
      const int row = e / kMlaChunks;
      const int j = e - row * kMlaChunks;
      const int key = min(kbase + t * BN + row, T - 1);
      dma_16B(rs, key * kMlaRowBytes + ((j ^ mla_swz(row)) << 4),
              lds_base + slot * TILE_BYTES + (wave * LPW + i) * 1024);
    }
  };

  // V^T transpose-read offsets: rows 4 half + L/4 (+8 for the second read),
  // dims 32 db + 16 (G16 & 1) + 4 (L & 3), i.e. chunk 4 db + c_low with
  // c_low = 2 (G16 & 1) + (L & 3) / 2.  With x = swz(row) < 8 the stored chunk
  // is 4 (db ^ (x >> 2)) + (c_low ^ (x & 3)): for even db that is 4 db + 4 e +
  // ..., for odd db 4 db - 4 e + ..., e = x >> 2, so one base per parity of
  // db plus the immediate 64 db gives every block's address.
  const int L16 = lane & 15;
  const int c_low = 2 * ((lane >> 4) & 1) + ((L16 & 3) >> 1);
  const int inner = ((4 * (L16 & 3)) & 7) * 2;
  int tr_base[2][2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const int row = 4 * half + (L16 >> 2) + 8 * hi;
    const int x = mla_swz(row);
    const int base = row * kMlaRowBytes + ((c_low ^ (x & 3)) << 4) + inner;
    tr_base[hi][0] = base + 64 * (x >> 2);
    tr_base[hi][1] = base - 64 * (x >> 2);
  }

  float* part = reinterpret_cast<float*>(lds + P * TILE_BYTES);
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m_used = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;

  auto compute = [&](int t, int slot) {
    const uint8_t* kt = lds + slot * TILE_BYTES;
    // S^T partial: element r holds key 8(r/4) + 4 half + r%4 of the tile
    f32x16 s = f32x16{};
#pragma unroll
    for (int i = 0; i < KSH; ++i) {
      const int chunk = (2 * (kh * KSH + i) + half) ^ mla_swz(col);
      const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + col * kMlaRowBytes + (chunk << 4)));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[i], s, 0, 0, 0);
    }
    // partials as [r4][wave][lane] float4: a wave's 64 lanes store and load
    // 1 KiB contiguous per access (no bank conflicts)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<f32x4*>(part + ((r4 * NW + wave) * 64 + lane) * 4) =
          f32x4{s[4 * r4], s[4 * r4 + 1], s[4 * r4 + 2], s[4 * r4 + 3]};
    __syncthreads();
    const int other = wave ^ 2;  // same pair block, other half
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(part + ((r4 * NW + other) * 64 + lane) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * r4 + e] += x[e];
    }
    const int key0 = kbase + t * BN;
    if ((p.causal && key0 + BN - 1 > wave_row0 + off) || key0 + BN > T) {
      const int lim = (p.causal ? min(my_row + off + 1, T) : T) - key0 - 4 * half;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) >= lim) s[r] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    const float mt = col_max<32>(mx) * sl2;
    if (__builtin_amdgcn_ballot_w64(mt > m_used + kRescaleSlack)) {
      const float m_new = fmaxf(m_used, mt);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_used - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) scale_agpr(acc[db], alpha);
      m_used = m_new;
    }
    const float m_sub = (m_used == -INFINITY) ? 0.f : m_used;
    f32x8 pf;
    bf16x8 pb2[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -m_sub));
      pf[r & 7] = pe;
      l_run += pe;
      if ((r & 7) == 7) pb2[r >> 3] = __builtin_convertvector(pf, bf16x8);
    }
    // O^T += V^T P^T over this half's 256 value dims
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint8_t* a = kt + (16 * st) * kMlaRowBytes + 64 * (kh * NDB + db);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + tr_base[0][db & 1]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + tr_base[1][db & 1]));
        const bf16x8 vT = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vT, pb2[st], acc[db], 0, 0, 0);
      }
  };

  if (n_tiles > 0) {
#pragma unroll
    for (int j = 0; j < P - 1; ++j) issue(j, j);
    for (int t = 0; t < n_tiles; ++t) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((P - 2) * LPW) : "memory");
      __syncthreads();  // tile t landed; every wave is done with tile t-1 and the partials
      issue(t + P - 1, (t + P - 1) % P);
      compute(t, t % P);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  const float l_tot = col_sum<32>(l_run);
  if (!valid) return;
  const int dbase = kh * (kMlaDc / 2);
  if constexpr (!SPLIT) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = p.o + bhr * kMlaDc + dbase;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * half;
        f32x4 f = {acc[db][4 * g4] * inv, acc[db][4 * g4 + 1] * inv, acc[db][4 * g4 + 2] * inv,
                   acc[db][4 * g4 + 3] * inv};
        *reinterpret_cast<u32x2*>(orow + d0) = __builtin_bit_cast(u32x2, __builtin_convertvector(f, bf16x4));
      }
    if (kh == 0 && half == 0) p.lse[bhr] = (m_used + __log2f(l_tot)) * kLn2;
  } else {
    const bool seen = l_tot > 0.f;
    const float inv = seen ? 1.f / l_tot : 0.f;
    const size_t slot = (size_t)split * ((size_t)p.B * p.H * p.S) + bhr;
    uint16_t* orow = p.o_part + slot * kMlaDc + dbase;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * half;
        const f32x4 f = {acc[db][4 * g4] * inv, acc[db][4 * g4 + 1] * inv, acc[db][4 * g4 + 2] * inv,
                         acc[db][4 * g4 + 3] * inv};
        *reinterpret_cast<u32x2*>(orow + d0) = __builtin_bit_cast(u32x2, __builtin_convertvector(f, bf16x4));
      }
    if (kh == 0 && half == 0) p.lse_part[slot] = seen ? m_used + __log2f(l_tot) : -INFINITY;
  }
}

// ------------------------------------------------- sixteen-pair latent core
// attn_mla16_kernel: the same latent attention with v_mfma_f32_16x16x32_bf16
// and no exchange between waves.  A workgroup of eight waves (two per SIMD)
// owns 128 (query token, head) pairs, 16 per wave, and streams 32-key tiles
// through a 4-stage LDS ring.  Each wave holds all 576 score dims of its
// pairs (18 k-steps of 32: 72 registers of queries) and all 512 value dims
// (32 blocks of 16: 128 accumulator registers), so its softmax needs only
// its own S^T and no barrier sits between the score and value products.
// Against the four-wave form it reads twice the LDS operand bytes per MFMA,
// and in exchange a second wave on each SIMD covers the latency of the
// other's chain.
//
// Lane l owns pair 16 w + (l & 15) and k-group g = l >> 4.  S^T for key
// block c (16 keys) is K Q^T with A = 16 key rows at dims 32 ks + 8 g .. +8
// and B = the pair's query at the same dims; the accumulator holds keys
// 16 c + 4 g + r.  P^T's B operand is then this lane's own 8 scores (keys
// 4 g + r and 16 + 4 g + r), and V^T's A operand the two transpose reads of
// rows 4 g + L / 4 and 16 + 4 g + L / 4 (L = l & 15) at dims 16 db + 4 (L & 3).
//
// Swizzle: chunk j of row r is stored at j ^ mla16_swz(r).  With rows 1152
// bytes apart, rows of one parity share a 128-byte bank half, so the 16-row
// K reads need the swizzle to be a bijection on row bits 1..3, the
// transpose reads (a half wave: 8 aligned rows x 2 adjacent chunks) need bits
// 1..2 of it distinct over the 4 rows of a parity, and rows r and r + 8
// take chunks that differ in more than bit 0.
__device__ __forceinline__ int mla16_swz(int row) {
  const int a = (row >> 1) & 7;
  return (2 * (a & 3) ^ (6 * (a >> 2))) | (a >> 2);
}

constexpr int kMla16Pairs = 128;  // (token, head) pairs per workgroup of attn_mla16_kernel

template <int P, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void attn_mla16_kernel(MlaParams p) {
  constexpr int NW = 8;
  constexpr int BN = 32;
  constexpr int TILE_BYTES = BN * kMlaRowBytes;          // 36 KiB
  constexpr int LOADS = TILE_BYTES / 1024;               // 36 loads of 1 KiB per tile
  constexpr int LPW = (LOADS + NW - 1) / NW;             // 5 per wave; the 4 spare ones move nothing
  constexpr int KS = kMlaDqk / 32;                       // 18 score k-steps
  constexpr int NDB = kMlaDc / 16;                       // 32 value blocks
  constexpr int PPW = 16 * NW;                           // pairs per workgroup
  constexpr int JUNK = P * TILE_BYTES;                   // landing area of the spare loads
  static_assert(PPW == kMla16Pairs && (P - 1) * LPW <= 63, "load groups");
  static_assert(JUNK + 1024 <= 160 * 1024, "LDS fits the 160 KiB of a CU");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[JUNK + 1024];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int kg = lane >> 4;

  const int3 item = mla_item(p);
  const int pb = item.x, b = item.y, split = SPLIT ? item.z : 0;
  const int T = p.T;
  const int off = p.causal_off;
  const int last_pair = p.n_pairs - 1;
  const int P0 = pb * PPW;
  const int wp0 = P0 + 16 * wave;
  const int wave_row0 = min(wp0, last_pair) / p.H;
  const int row_end = min(P0 + PPW - 1, last_pair) / p.H + 1;

  const int kv_end = p.causal ? min(row_end + off, T) : T;
  int n_tiles = (kv_end + BN - 1) / BN;
  int kbase = 0;
  if constexpr (SPLIT) {
    const int per = (n_tiles + p.n_splits - 1) / p.n_splits;
    const int t0 = min(split * per, n_tiles);
    n_tiles = min(per, n_tiles - t0);
    kbase = t0 * BN;
  }

  const int pair = wp0 + col;
  const bool valid = pair <= last_pair;
  const int pc = min(pair, last_pair);
  const int my_row = pc / p.H;
  const int h = pc - my_row * p.H;
  const size_t bhr = ((size_t)b * p.H + h) * (size_t)p.S + my_row;
  bf16x8 qf[KS];
#pragma unroll
  for (int i = 0; i < KS; ++i) {
    u32x4 x = *reinterpret_cast<const u32x4*>(p.q + bhr * kMlaDqk + 32 * i + 8 * kg);
    x ^= p.q_sign;
    qf[i] = as_bf16x8(x);
  }

  // Tile loads: load slot gi = LPW wave + i moves bytes [1024 gi, +1024) of
  // the tile (lane -> row, stored chunk j; it fetches chunk j ^ swz(row)).
  // The resource starts at the tile's first key and ends at the cache's last
  // byte, so rows past T read as zeros (they are masked); slots gi >= LOADS
  // and tiles past the last get an empty resource and land in the junk area.
  const uint8_t* kv_b = reinterpret_cast<const uint8_t*>(p.kv + (size_t)b * T * kMlaDqk);
  const u32x4 rsrc_none = make_rsrc(p.kv, 0u);
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)lds;
  int ld_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int e = min((wave * LPW + i) * 64 + lane, LOADS * 64 - 1);
    const int row = e / kMlaChunks;
    const int j = e - row * kMlaChunks;
    ld_off[i] = row * kMlaRowBytes + ((j ^ mla16_swz(row)) << 4);
  }
  auto issue = [&](int t, int slot) {
    const int key0 = kbase + t * BN;
    const u32x4 rs = t < n_tiles ? make_rsrc(kv_b + (size_t)key0 * kMlaRowBytes, (uint32_t)(T - key0) * kMlaRowBytes)
                                 : rsrc_none;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int gi = wave * LPW + i;
      const bool real = gi < LOADS;
      dma_16B(real ? rs : rsrc_none, ld_off[i], lds_base + (real ? slot * TILE_BYTES + gi * 1024 : JUNK));
    }
  };

  // operand offsets inside a tile (the ring slot's base is added per tile)
  const int ksw = mla16_swz(col);
  int k_off[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) k_off[e] = col * kMlaRowBytes + (((4 * e + kg) ^ ksw) << 4);
  const int vrow = 4 * kg + (col >> 2);
  const int vsw = mla16_swz(vrow);
  const int xlow = (col & 3) >> 1;
  int v_off[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v_off[e] = vrow * kMlaRowBytes + (((2 * e + xlow) ^ vsw) << 4) + 8 * (col & 1);

  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{};
  float m_used = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;

  auto compute = [&](int t, int slot) {
    const uint8_t* kt = lds + slot * TILE_BYTES;
    f32x4 s0 = f32x4{}, s1 = f32x4{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint8_t* a = kt + k_off[ks & 1] + 128 * (ks >> 1);
      const bf16x8 k0 = as_bf16x8(*reinterpret_cast<const u32x4*>(a));
      const bf16x8 k1 = as_bf16x8(*reinterpret_cast<const u32x4*>(a + 16 * kMlaRowBytes));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[ks], s1, 0, 0, 0);
    }
    const int key0 = kbase + t * BN;
    if ((p.causal && key0 + BN - 1 > wave_row0 + off) || key0 + BN > T) {
      const int lim = (p.causal ? min(my_row + off + 1, T) : T) - key0 - 4 * kg;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r >= lim) s0[r] = -INFINITY;
        if (16 + r >= lim) s1[r] = -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3]));
    mx = fmaxf(mx, fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
    const float mt = col_max<16>(mx) * sl2;
    if (__builtin_amdgcn_ballot_w64(mt > m_used + kRescaleSlack)) {
      const float m_new = fmaxf(m_used, mt);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_used - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
      m_used = m_new;
    }
    const float m_sub = (m_used == -INFINITY) ? 0.f : m_used;
    f32x8 pf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pf[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], sl2, -m_sub));
      pf[4 + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], sl2, -m_sub));
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) l_run += pf[r];
    const bf16x8 pbf = __builtin_convertvector(pf, bf16x8);
    // O^T += V^T P^T over all 512 value dims
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint8_t* a = kt + v_off[db & 3] + 128 * (db >> 2);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + 16 * kMlaRowBytes));
      const bf16x8 vT = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vT, pbf, acc[db], 0, 0, 0);
    }
  };

  if (n_tiles > 0) {
#pragma unroll
    for (int j = 0; j < P - 1; ++j) issue(j, j);
    for (int t = 0; t < n_tiles; ++t) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((P - 2) * LPW) : "memory");
      __syncthreads();  // tile t landed; every wave is done with tile t-1
      issue(t + P - 1, (t + P - 1) % P);
      compute(t, t % P);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  const float l_tot = col_sum<16>(l_run);
  if (!valid) return;
  const bool seen = l_tot > 0.f;
  const float inv = SPLIT ? (seen ? 1.f / l_tot : 0.f) : 1.f / l_tot;
  uint16_t* orow;
  if constexpr (SPLIT) orow = p.o_part + ((size_t)split * ((size_t)p.B * p.H * p.S) + bhr) * kMlaDc;
  else orow = p.o + bhr * kMlaDc;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const f32x4 f = {acc[db][0] * inv, acc[db][1] * inv, acc[db][2] * inv, acc[db][3] * inv};
    *reinterpret_cast<u32x2*>(orow + 16 * db + 4 * kg) = __builtin_bit_cast(u32x2, __builtin_convertvector(f, bf16x4));
  }
  if (kg == 0) {
    if constexpr (SPLIT)
      p.lse_part[(size_t)split * ((size_t)p.B * p.H * p.S) + bhr] = seen ? m_used + __log2f(l_tot) : -INFINITY;
    else
      p.lse[bhr] = (m_used + __log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------- projections
struct MlaProjParams {
  const uint16_t* x;    // absorb: q_nope [B, H, S, d_n];  up: out_lat [B, H, S, 512]
  const uint16_t* x2;   // absorb: q_pe [B, H, S, 64]
  const uint16_t* w;    // absorb: W_uk [H, d_n, 512];     up: W_uv [H, d_v, 512]
  uint16_t* y;          // absorb: q_lat [B, H, S, 576];   up: out [B, H, S, d_v]
  int B, H, S, d_n;     // d_n: d_nope (absorb) or d_v (up)
  int rows_per_head;    // B * S
};

constexpr int kAbsorbSlice = 128;   // output columns per absorb block
constexpr int kAbsorbMaxK = 256;    // largest d_nope

// LDS of one absorb block for kp = d_nope rounded up to 16: the W_uk slice
// (kp rows of 256 bytes), then 32 staged query rows of kp + 8 values (16
// bytes of padding per row).
__host__ __device__ constexpr int absorb_lds_bytes(int kp) { return kp * 256 + 32 * (kp + 8) * 2; }

// 16-byte chunk swizzle of the staged W_uk slice (rows of 128 values): a
// bijection on 16 rows for 16-byte row access, and the transpose read (4 rows
// x 4 chunks per 16 lanes) lands on 16 different chunk positions.
__device__ __forceinline__ int absorb_swz(int row) { return 4 * (row & 3) + ((row >> 2) & 3); }

// q_lat[r, c] = sum_d q_nope[r, d] W_uk[h, d, c], q_lat[r, 512 + e] = q_pe[r, e].
// A block of four waves owns head h and 128 output columns: it stages that
// slice of W_uk[h] (d_nope rows, zero-padded to a multiple of 16) in LDS once
// and runs every query row of the head past it in blocks of 32.  Wave w
// computes the 32 x 32 block Y^T = W^T X^T for columns 32 w .. +32 with MFMA:
// A = W^T from the LDS transpose read, B = the matching 8 values of d of a
// query row staged in LDS (q_nope rows are only 2-byte aligned).  W_uk is
// read from memory exactly once.  Dynamic LDS: absorb_lds_bytes(kp).
// VEC_X: the query rows are loaded in 16-byte chunks (d_nope a multiple of 8
// and q_nope 16-byte aligned), else value by value.
template <bool VEC_X>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void mla_absorb_kernel(MlaProjParams p) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t absorb_lds[];
  constexpr int n_cs = kMlaDc / kAbsorbSlice;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int h = blockIdx.x / n_cs;
  const int cs = blockIdx.x % n_cs;
  const int dn = p.d_n;
  const int kp = (dn + 15) & ~15;
  const int xstride = kp + 8;
  uint8_t* wsl = absorb_lds;
  uint16_t* xs = reinterpret_cast<uint16_t*>(absorb_lds + kp * 256);
  // row r of head h is (b, s) = (r / S, r % S)
  auto row_index = [&](int r) { return ((size_t)(r / p.S) * p.H + h) * p.S + (r % p.S); };

  // W_uk[h, d, 128 cs .. +128] -> wsl row d, chunk j at (j ^ swz(d)); at most
  // 16 chunks per thread, all loads issued before the stores
  const uint16_t* wh = p.w + (size_t)h * dn * kMlaDc + cs * kAbsorbSlice;
  {
    u32x4 v[kAbsorbMaxK * 16 / 256];
#pragma unroll
    for (int i = 0; i < kAbsorbMaxK * 16 / 256; ++i) {
      const int e = tid + 256 * i, d = e >> 4, j = e & 15;
      v[i] = d < dn ? *reinterpret_cast<const u32x4*>(wh + (size_t)d * kMlaDc + 8 * j) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kAbsorbMaxK * 16 / 256; ++i) {
      const int e = tid + 256 * i, d = e >> 4, j = e & 15;
      if (d < kp) *reinterpret_cast<u32x4*>(wsl + d * 256 + ((j ^ absorb_swz(d)) << 4)) = v[i];
    }
  }
  // transpose-read offsets: d rows 4 half + L/4 (+8 for the second read) of a
  // 16-row step, columns 32 wave + 16 (G16 & 1) + 4 (L & 3)
  const int L16 = lane & 15;
  int tr_off[2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const int row = 4 * half + (L16 >> 2) + 8 * hi;
    const int c = wave * 32 + 16 * ((lane >> 4) & 1) + 4 * (L16 & 3);
    tr_off[hi] = row * 256 + (((c >> 3) ^ absorb_swz(row)) << 4) + (c & 7) * 2;
  }

  for (int r0 = 0; r0 < p.rows_per_head; r0 += 32) {
    __syncthreads();  // the W slice is staged; the previous rows are read
    // 32 query rows, zero past d_nope and past the last row; thread t takes
    // row t / 8 and every 8th 16-byte chunk (VEC_X) or value of it
    if constexpr (VEC_X) {
      const int r = tid >> 3, c0 = tid & 7;
      const int rr = r0 + r;
      const bool live = rr < p.rows_per_head;
      const uint16_t* xr = p.x + (live ? row_index(rr) * dn : 0);
      u32x4 xc[kAbsorbMaxK / 64];
#pragma unroll
      for (int i = 0; i < kAbsorbMaxK / 64; ++i) {
        const int c = c0 + 8 * i;
        xc[i] = (live && 8 * c < dn) ? *reinterpret_cast<const u32x4*>(xr + 8 * c) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < kAbsorbMaxK / 64; ++i) {
        const int c = c0 + 8 * i;
        if (8 * c < kp) *reinterpret_cast<u32x4*>(xs + r * xstride + 8 * c) = xc[i];
      }
    } else {
      const int r = tid >> 3, d0 = tid & 7;
      const int rr = r0 + r;
      const bool live = rr < p.rows_per_head;
      const uint16_t* xr = p.x + (live ? row_index(rr) * dn : 0);
      uint16_t xv[kAbsorbMaxK / 8];
#pragma unroll
      for (int i = 0; i < kAbsorbMaxK / 8; ++i) {
        const int d = d0 + 8 * i;
        xv[i] = (live && d < dn) ? xr[d] : uint16_t(0);
      }
#pragma unroll
      for (int i = 0; i < kAbsorbMaxK / 8; ++i) {
        const int d = d0 + 8 * i;
        if (d < kp) xs[r * xstride + d] = xv[i];
      }
    }
    __syncthreads();
    f32x16 acc = f32x16{};
    for (int ks = 0; ks < kp / 16; ++ks) {
      const uint8_t* a = wsl + (16 * ks) * 256;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + tr_off[0]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + tr_off[1]));
      const bf16x8 wT = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      // the transpose read returns the k-step's rows 4 half .. +4 and 8 + 4
      // half .. +4 (the order of an MFMA accumulator), so B takes the same d
      const u32x2 x0 = *reinterpret_cast<const u32x2*>(xs + col * xstride + 16 * ks + 4 * half);
      const u32x2 x1 = *reinterpret_cast<const u32x2*>(xs + col * xstride + 16 * ks + 8 + 4 * half);
      const bf16x8 xf = as_bf16x8(u32x4{x0[0], x0[1], x1[0], x1[1]});
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wT, xf, acc, 0, 0, 0);
    }
    // element k holds column 32 wave + 8 (k/4) + 4 half + k%4 of row r0 + col
    const int rr = r0 + col;
    if (rr < p.rows_per_head) {
      const size_t row = row_index(rr);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c = cs * kAbsorbSlice + wave * 32 + 8 * g4 + 4 * half;
        const f32x4 f = {acc[4 * g4], acc[4 * g4 + 1], acc[4 * g4 + 2], acc[4 * g4 + 3]};
        *reinterpret_cast<u32x2*>(p.y + row * kMlaDqk + c) = __builtin_bit_cast(u32x2, __builtin_convertvector(f, bf16x4));
      }
    }
    // the rotary part is copied by the first column slice: 32 rows x 8 chunks
    if (cs == 0) {
      const int r = tid >> 3, j = tid & 7;
      if (r0 + r < p.rows_per_head) {
        const size_t row = row_index(r0 + r);
        *reinterpret_cast<u32x4*>(p.y + row * kMlaDqk + kMlaDc + 8 * j) =
            *reinterpret_cast<const u32x4*>(p.x2 + row * kMlaDr + 8 * j);
      }
    }
  }
}

// out[r, v] = sum_c out_lat[r, c] W_uv[h, v, c]: one wave per (head, 32
// values of v, 32 rows of that head) computes the 32 x 32 block with MFMA,
// A = out_lat rows and B^T = W_uv rows, both read as 16-byte fragments
// straight from global memory (their contiguous dimension is c, the
// contraction).  Rows past the head's last one are clamped and not stored.
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64))) void mla_up_kernel(MlaProjParams p) {
  const int lane = threadIdx.x;
  const int half = lane >> 5, col = lane & 31;
  const int n_vb = p.d_n / 32;
  int bid = blockIdx.x;
  const int vb = bid % n_vb;
  bid /= n_vb;
  const int h = bid % p.H;
  const int r0 = (bid / p.H) * 32;
  // A: row r0 + col of head h; B: W_uv[h, 32 vb + col, :]
  const int rr = min(r0 + col, p.rows_per_head - 1);
  const size_t arow = ((size_t)(rr / p.S) * p.H + h) * p.S + (rr % p.S);
  const uint16_t* a = p.x + arow * kMlaDc + half * 8;
  const uint16_t* w = p.w + ((size_t)h * p.d_n + 32 * vb + col) * kMlaDc + half * 8;
  // the 32 k-steps in two halves, each half's 32 loads issued before its
  // MFMAs (about 5 % faster than loads interleaved with the MFMAs)
  f32x16 acc = f32x16{};
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    u32x4 av[16], bv[16];
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      av[ks] = *reinterpret_cast<const u32x4*>(a + (hb * 16 + ks) * 16);
      bv[ks] = *reinterpret_cast<const u32x4*>(w + (hb * 16 + ks) * 16);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[ks]), as_bf16x8(bv[ks]), acc, 0, 0, 0);
  }
  // element r holds row r0 + 8(r/4) + 4 half + r%4 and v = 32 vb + col
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rowi = r0 + 8 * (r >> 2) + 4 * half + (r & 3);
    if (rowi < p.rows_per_head) {
      const size_t orow = ((size_t)(rowi / p.S) * p.H + h) * p.S + (rowi % p.S);
      p.y[orow * p.d_n + 32 * vb + col] = __builtin_bit_cast(uint16_t, (__bf16)acc[r]);
    }
  }
}

}  // namespace ea02
