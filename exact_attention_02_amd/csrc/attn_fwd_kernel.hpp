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
//    with v_mfma_f32_32x32x16_bf16.  In the 32x32 accumulator layout a lane
//    holds one column and 16 rows, so here a lane owns ONE query and 16 keys
//    per 32-key block: the row max and row sum are lane-local plus a single
//    exchange between the two wave halves (v_permlane32_swap), and the per-row
//    rescale factor is a lane scalar.  The S^T accumulator, rounded to bf16,
//    is directly the B operand of the PV product; the key order this implies
//    is absorbed by storing V^T in LDS with keys permuted to match.
//  * Query fragments live in VGPRs for the whole kernel (B operand of S^T).
//  * K tiles are stored [key][d] in LDS with a 16-byte-chunk XOR swizzle;
//    V tiles are transposed on the way in to V^T[d][key'] (also swizzled),
//    so both MFMA A operands are single 128-bit LDS reads.
//  * Tiles are double-buffered: the global loads of tile t+1 are issued
//    before the math of tile t and written to the other LDS buffer after it;
//    one barrier per tile.
//  * GQA/MQA: the waves of a workgroup take different query heads of the same
//    kv group over the same rows, so each K/V tile in LDS serves all of them.
//  * Causal: the tile loop ends at the workgroup's last row; only tiles that
//    cross a wave's diagonal (or the ragged end of the sequence) run the
//    masked variant; tiles wholly above a wave's rows are skipped by it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ea02 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, H_q, H_kv, N;
  int G;              // H_q / H_kv
  int n_row_blocks;   // ceil(N / rows per workgroup)
  int n_head_groups;  // G / heads per workgroup
  int n_heads_wg;     // B * H_kv * n_head_groups: workgroups per row block
  float scale_log2;   // |sm_scale| * log2(e)
  uint32_t q_sign;    // 0x80008000 when sm_scale < 0 (Q is negated on load), else 0
  int causal;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ float wave_half_swap_max(float x) {
  // v_permlane32_swap exchanges lanes 32..63 of the first operand with lanes
  // 0..31 of the second; with both operands = x the two results hold x of
  // this lane and of lane l^32, in some order.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Position of key `key` (0 <= key < BN) inside a V^T row: within every group
// of 16 keys the quads are stored in the order 0,2,1,3, so that the 8 keys a
// lane needs for one PV k-step are contiguous (see the S^T accumulator layout).
__device__ __forceinline__ int vt_pos(int key) {
  const int quad = (key >> 2) & 3;
  const int pq = ((quad & 1) << 1) | (quad >> 1);  // 0,2,1,3
  return (key & ~15) | (pq << 2) | (key & 3);
}

template <int D, int BN, int NW, int HW>
struct Cfg {
  static constexpr int QW = 32;                 // query rows per wave
  static constexpr int NT = NW * 64;            // threads per workgroup
  static constexpr int BM = QW * NW / HW;       // query rows per workgroup
  static constexpr int DC = D / 8;              // 16-byte chunks per K row
  static constexpr int KC = BN * DC / NT;       // K chunks loaded per thread
  static constexpr int VU = (BN / 4) * DC;      // V units (4 keys x 8 d)
  static constexpr int VUT = (VU + NT - 1) / NT;
  static constexpr int VC = BN / 8;             // 16-byte chunks per V^T row
  static constexpr int K_ELEMS = BN * D;        // u16 per K buffer
  static constexpr int V_ELEMS = D * BN;        // u16 per V^T buffer
  static constexpr int LDS_ELEMS = 2 * (K_ELEMS + V_ELEMS);
  static_assert(BN == 64, "key tile of 64");
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
  static_assert((BN * DC) % NT == 0, "K tile split evenly");
};

// XOR swizzles of 16-byte chunk indices (conflict-light 128-bit LDS access).
template <int DC>
__device__ __forceinline__ int k_swz(int key, int chunk) { return chunk ^ (key & (DC - 1)); }
__device__ __forceinline__ int vt_swz(int d, int chunk) { return chunk ^ ((d ^ (d >> 3)) & 7); }

template <int D, int BN, int NW, int HW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(FwdParams p) {
  using C = Cfg<D, BN, NW, HW>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  uint16_t* const k_lds = lds;                       // [2][BN][D]
  uint16_t* const v_lds = lds + 2 * C::K_ELEMS;      // [2][D][BN]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  // ---- work decomposition: heaviest row blocks first (causal), heads fastest
  const int bid = blockIdx.x;
  const int rb = p.n_row_blocks - 1 - bid / p.n_heads_wg;
  int rest = bid % p.n_heads_wg;
  const int hs = rest % p.n_head_groups;
  rest /= p.n_head_groups;
  const int g = rest % p.H_kv;
  const int b = rest / p.H_kv;
  const int hh = wave % HW;
  const int rsub = wave / HW;
  const int h = g * p.G + hs * HW + hh;
  const int R0 = rb * C::BM;
  const int wr0 = R0 + rsub * C::QW;
  const int N = p.N;

  const int kv_end = p.causal ? min(R0 + C::BM, N) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;

  const size_t kv_base = ((size_t)b * p.H_kv + g) * (size_t)N * D;
  const size_t q_base = ((size_t)b * p.H_q + h) * (size_t)N * D;
  const uint16_t* __restrict__ kg = p.k + kv_base;
  const uint16_t* __restrict__ vg = p.v + kv_base;

  // ---- query fragments (B operand of S^T = K Q^T): lane holds query col,
  //      d = 16*ks + 8*half .. +8
  const int my_row = wr0 + col;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (my_row < N) x = *reinterpret_cast<const u32x4*>(p.q + q_base + (size_t)my_row * D + ks * 16 + half * 8);
    x ^= p.q_sign;
    qf[ks] = as_bf16x8(x);
  }

  // ---- tile staging through registers
  u32x4 kreg[C::KC];
  u32x4 vreg[C::VUT][4];

  auto load_tile = [&](int key0) {
#pragma unroll
    for (int i = 0; i < C::KC; ++i) {
      const int c = tid + i * C::NT;
      const int key = c / C::DC, dc = c % C::DC;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key0 + key < N) x = *reinterpret_cast<const u32x4*>(kg + (size_t)(key0 + key) * D + dc * 8);
      kreg[i] = x;
    }
#pragma unroll
    for (int i = 0; i < C::VUT; ++i) {
      const int u = tid + i * C::NT;
      if (u < C::VU) {
        const int dc = u % C::DC, kgp = u / C::DC;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + kgp * 4 + r;
          u32x4 x = {0u, 0u, 0u, 0u};
          if (key < N) x = *reinterpret_cast<const u32x4*>(vg + (size_t)key * D + dc * 8);
          vreg[i][r] = x;
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* kb = k_lds + buf * C::K_ELEMS;
    uint16_t* vb = v_lds + buf * C::V_ELEMS;
#pragma unroll
    for (int i = 0; i < C::KC; ++i) {
      const int c = tid + i * C::NT;
      const int key = c / C::DC, dc = c % C::DC;
      *reinterpret_cast<u32x4*>(kb + key * D + k_swz<C::DC>(key, dc) * 8) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < C::VUT; ++i) {
      const int u = tid + i * C::NT;
      if (u < C::VU) {
        const int dc = u % C::DC, kgp = u / C::DC;
        const int pos = vt_pos(kgp * 4);
        const int chunk = pos >> 3, sub = pos & 7;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // element e of each row: 16-bit lane e of the 128-bit register
          const int w = e >> 1, sh = (e & 1) * 16;
          const uint32_t a0 = (vreg[i][0][w] >> sh) & 0xffffu;
          const uint32_t a1 = (vreg[i][1][w] >> sh) & 0xffffu;
          const uint32_t a2 = (vreg[i][2][w] >> sh) & 0xffffu;
          const uint32_t a3 = (vreg[i][3][w] >> sh) & 0xffffu;
          u32x2 pk = {a0 | (a1 << 16), a2 | (a3 << 16)};
          const int d = dc * 8 + e;
          *reinterpret_cast<u32x2*>(vb + d * BN + vt_swz(d, chunk) * 8 + sub) = pk;
        }
      }
    }
  };

  // ---- running state (one query per lane)
  float m_run = -INFINITY;  // running max, log2-scaled units
  float l_run = 0.f;        // this lane's partial running sum (its 16 keys per block)
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};

  const float sl2 = p.scale_log2;

  auto process_tile = [&](int buf, int key0, bool masked) {
    const uint16_t* kb = k_lds + buf * C::K_ELEMS;
    const uint16_t* vb = v_lds + buf * C::V_ELEMS;
    // S^T[key][query] for the BN/32 key blocks
    f32x16 s[BN / 32];
#pragma unroll
    for (int c = 0; c < BN / 32; ++c) {
      s[c] = f32x16{};
      const int key = c * 32 + col;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 kx = *reinterpret_cast<const u32x4*>(kb + key * D + k_swz<C::DC>(key, 2 * ks + half) * 8);
        s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kx), qf[ks], s[c], 0, 0, 0);
      }
    }
    if (masked) {
#pragma unroll
      for (int c = 0; c < BN / 32; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + c * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool vis = key < N && (!p.causal || key <= my_row);
          s[c][r] = vis ? s[c][r] : -INFINITY;
        }
    }
    // online softmax (exp2 form)
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < BN / 32; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c][r]);
    mx = wave_half_swap_max(mx);
    // (-inf) * 0 would be NaN when sm_scale is 0: keep a fully masked row at -inf
    const float m_new = fmaxf(m_run, mx == -INFINITY ? -INFINITY : mx * sl2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float rs = 0.f;
    bf16x8 pb[BN / 16];
#pragma unroll
    for (int c = 0; c < BN / 32; ++c) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][8 * t + e], sl2, -m_use));
          // a masked score is -inf; with sm_scale = 0 the product above is NaN
          if (masked) pe = (s[c][8 * t + e] == -INFINITY) ? 0.f : pe;
          pf[e] = pe;
          rs += pe;
        }
        pb[2 * c + t] = __builtin_convertvector(pf, bf16x8);
      }
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = db * 32 + col;
#pragma unroll
      for (int st = 0; st < BN / 16; ++st) {
        const int chunk = 2 * st + half;
        const u32x4 vx = *reinterpret_cast<const u32x4*>(vb + d * BN + vt_swz(d, chunk) * 8);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vx), pb[st], acc[db], 0, 0, 0);
      }
    }
  };

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
  }
  for (int t = 0; t < n_tiles; ++t) {
    const int key0 = t * BN;
    const bool more = t + 1 < n_tiles;
    if (more) load_tile(key0 + BN);
    const bool skip = p.causal && key0 > wr0 + C::QW - 1;
    if (!skip) {
      const bool masked = (p.causal && key0 + BN - 1 > wr0) || (key0 + BN > N);
      if (masked) process_tile(t & 1, key0, true);
      else process_tile(t & 1, key0, false);
    }
    if (more) store_tile((t + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l (bf16, round to nearest even), LSE in natural log
  const float l_tot = wave_half_swap_sum(l_run);
  const float inv = 1.f / l_tot;
  if (my_row < N) {
    uint16_t* orow = p.o + q_base + (size_t)my_row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * half;
        typedef float f32x4v __attribute__((ext_vector_type(4)));
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        f32x4v f = {acc[db][4 * g4 + 0] * inv, acc[db][4 * g4 + 1] * inv,
                    acc[db][4 * g4 + 2] * inv, acc[db][4 * g4 + 3] * inv};
        bf16x4 bv = __builtin_convertvector(f, bf16x4);
        *reinterpret_cast<u32x2*>(orow + d0) = __builtin_bit_cast(u32x2, bv);
      }
    if (half == 0) p.lse[((size_t)b * p.H_q + h) * (size_t)N + my_row] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

}  // namespace ea02
