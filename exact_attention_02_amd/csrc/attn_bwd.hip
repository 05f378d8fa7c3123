// C ABI of the attention backward (declared in include/attn.h): argument
// validation and the three kernel launches.  The library allocates nothing,
// keeps no state and never synchronises.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstddef>
#include <algorithm>
#include <cstdint>

#include "../../include/attn.h"
#include "attn_bwd_kernel.hpp"
#include "abi_util.hpp"

namespace {

using ea02::abi::device_cus;
using ea02::abi::overlaps;

using ea02::BwdParams;

// dK/dV: four waves of 32 keys (128 keys per workgroup), 64-row tiles of Q and
// dO, four LDS stages (136 KiB at D=128).  dQ: eight waves of 32 (row, head)
// pairs (256 per workgroup, two waves per SIMD), 64-key tiles of K and V, four
// stages (128 KiB at D=128); for small grids four waves and two stages (64
// KiB, two workgroups per CU), chosen by q_waves.
constexpr int kKvNW = 4, kKvP = 4, kKvBP = 64;
constexpr int kQNW = 8, kQP = 4, kQBN = 64;
constexpr int kQMidNW = 4, kQMidP = 2;

// Row-range splits of the dK/dV kernel: at most this many per key block.
constexpr int64_t kMaxBwdSplits = 64;
// Partial sums of the library's own choice take at most this much workspace.
constexpr int64_t kAutoPartBytes = int64_t(1) << 30;
// Cost model for the library's split choice (MI355X measurements of these
// kernels): about 2 us per row tile of the dK/dV kernel or key tile of the dQ
// kernel; partial sums written, read back and reduced at about 5 bytes/ps (5
// TB/s); about 5 us for the extra launch.
constexpr double kTileUs = 2.0;
constexpr double kPartBytesPerUs = 5.0e6;
constexpr double kLaunchUs = 5.0;

// Keep n splits only if the time taken off the heaviest workgroup (it walks
// tiles_max tiles unsplit, max(share, tiles_max / n) split) exceeds the cost
// of its fp32 partials (part_bytes per split, plus out_bytes of final output).
int64_t worth_splitting(int64_t n, int64_t tiles_max, int64_t share, double part_bytes, double out_bytes) {
  if (n <= 1) return 1;
  const int64_t split_max = std::max<int64_t>(share, (tiles_max + n - 1) / n);
  const double saved = double(std::max<int64_t>(tiles_max - split_max, 0)) * kTileUs;
  const double cost = (2.0 * n * part_bytes + out_bytes) / kPartBytesPerUs + kLaunchUs;
  return saved > cost ? n : 1;
}


struct Shape {
  int64_t B, H_q, H_kv, N_q, N_kv, D;
  int causal;
};

// Size checks shared by attn_bwd and attn_bwd_num_splits (everything up to
// and including SIZE_OVERFLOW); *empty is set when there is nothing to do.
int check_sizes(const Shape& a, int64_t n_splits, float sm_scale, bool* empty) {
  *empty = false;
  if (a.B < 0 || a.H_q < 0 || a.H_kv < 0 || a.N_q < 0 || a.N_kv < 0 || a.D < 0 || n_splits < 0)
    return ATTN_ERR_NEGATIVE_SIZE;
  if (a.H_kv < 1 || a.H_q % a.H_kv != 0) return ATTN_ERR_HEAD_RATIO;
  if (a.D != 64 && a.D != 128) return ATTN_ERR_HEAD_DIM;
  if (a.causal != 0 && a.causal != 1) return ATTN_ERR_CAUSAL_FLAG;
  if (!std::isfinite(sm_scale)) return ATTN_ERR_SCALE;
  if (n_splits > kMaxBwdSplits) return ATTN_ERR_SPLITS;
  if (a.causal && a.N_q > a.N_kv) return ATTN_ERR_CAUSAL_SHAPE;
  const int64_t lim24 = int64_t(1) << 24;
  const int64_t G = a.H_q / a.H_kv;
  // one kv group's Q / dO rows and one kv head's K / V rows take 32-bit byte offsets
  if (a.N_q > lim24 || a.N_kv > lim24 || a.B > lim24 || a.H_q > (int64_t(1) << 16) ||
      a.N_kv * a.D * 2 > (int64_t(1) << 31) || a.N_q * G * a.D * 2 > (int64_t(1) << 31) ||
      a.B * a.H_q * a.N_q > INT32_MAX)
    return ATTN_ERR_SIZE_OVERFLOW;
  const int64_t key_blocks = (a.N_kv + 32 * kKvNW - 1) / (32 * kKvNW);
  // the smaller dQ pair blocks give the larger grid
  const int64_t pair_blocks = (a.N_q * G + 32 * kQMidNW - 1) / (32 * kQMidNW);
  const int64_t splits = n_splits > 1 ? n_splits : 1;
  // every launch within one dispatch's 32-bit work-item count: dK/dV, dQ
  // (two threads per pair in either shape) and the prep kernel (D/8 threads
  // per row)
  const int64_t prep_blocks = (a.B * a.H_q * a.N_q * (a.D / 8) + 255) / 256;
  if (a.B * a.H_kv * key_blocks * splits > ea02::abi::max_launch_blocks(64 * kKvNW) ||
      a.B * a.H_kv * pair_blocks > ea02::abi::max_launch_blocks(64 * kQMidNW) ||
      prep_blocks > ea02::abi::max_launch_blocks(256))
    return ATTN_ERR_SIZE_OVERFLOW;
  if (a.B == 0 || a.H_q == 0 || (a.N_q == 0 && a.N_kv == 0)) *empty = true;
  return ATTN_OK;
}

// Row tiles (BP query rows of one head) that key block kb visits.
int64_t kv_block_tiles(const Shape& a, int64_t kb) {
  const int64_t off = a.causal ? a.N_kv - a.N_q : 0;
  const int64_t r_start = a.causal ? std::max<int64_t>(0, kb * 32 * kKvNW - off) / kKvBP * kKvBP : 0;
  return (a.H_q / a.H_kv) * ((a.N_q - r_start + kKvBP - 1) / kKvBP);
}

// The library's split count: the heaviest key block (causal: block 0, which
// sees every row) is cut into ranges no longer than an even share of all row
// tiles per CU (one dK/dV workgroup runs per CU at a time), at least 4 tiles
// each, capped at kMaxBwdSplits and at 1 GiB of partial sums, and kept only
// when the cost model above says the split pays for its partial sums.  This
// is 1 when the key blocks are many and balanced (long sequences), and above 1
// both for few key blocks (one kv head, short sequences) and for a causal
// grid of about one workgroup per CU, whose time the heaviest block would
// otherwise set.
int64_t choose_kv_splits(const Shape& a) {
  if (a.N_q == 0 || a.N_kv == 0 || a.B == 0 || a.H_q == 0) return 1;
  const int64_t key_blocks = (a.N_kv + 32 * kKvNW - 1) / (32 * kKvNW);
  const int64_t heads = a.B * a.H_kv;
  const int64_t cus = device_cus();
  int64_t total = 0;
  for (int64_t kb = 0; kb < key_blocks; ++kb) total += kv_block_tiles(a, kb);
  total *= heads;
  const int64_t tiles_max = kv_block_tiles(a, 0);
  const int64_t share = std::max<int64_t>((total + cus - 1) / cus, 4);
  int64_t n = (tiles_max + share - 1) / share;
  n = std::min({n, tiles_max, kMaxBwdSplits});
  const int64_t plane2 = 2 * heads * a.N_kv * a.D * 4;
  n = std::min(n, kAutoPartBytes / plane2);
  n = std::min(n, ea02::abi::max_launch_blocks(64 * kKvNW) / (heads * key_blocks));  // one dispatch
  return worth_splitting(n, tiles_max, share, double(plane2), double(plane2) / 2);
}

// Key tiles (kQBN keys) that dQ pair block pb (32 nw pairs) visits.
int64_t q_block_tiles(const Shape& a, int64_t pb, int nw) {
  const int64_t G = a.H_q / a.H_kv;
  const int64_t last = std::min(pb * 32 * nw + 32 * nw - 1, a.N_q * G - 1);
  const int64_t row_end = last / G + 1;
  const int64_t kv_end = a.causal ? std::min(row_end + a.N_kv - a.N_q, a.N_kv) : a.N_kv;
  return (kv_end + kQBN - 1) / kQBN;
}

// The dQ kernel's key-range splits, by the same rule as the dK/dV splits: the
// heaviest pair block (causal: the last rows) is cut into ranges no longer
// than an even share of all key tiles per CU (one dQ workgroup per CU at a
// time), at least 4 tiles each, at most kMaxBwdSplits, at most 1 GiB of
// partial sums, and only when the cost model says it pays.  1 when the pair
// blocks are many and balanced.  nw: waves (32 pairs each) per dQ workgroup.
int64_t choose_q_splits_nw(const Shape& a, int nw) {
  if (a.N_q == 0 || a.N_kv == 0 || a.B == 0 || a.H_q == 0) return 1;
  const int64_t pair_blocks = (a.N_q * (a.H_q / a.H_kv) + 32 * nw - 1) / (32 * nw);
  const int64_t heads = a.B * a.H_kv;
  const int64_t cus = device_cus();
  int64_t total = 0;
  for (int64_t pb = 0; pb < pair_blocks; ++pb) total += q_block_tiles(a, pb, nw);
  total *= heads;
  const int64_t tiles_max = q_block_tiles(a, pair_blocks - 1, nw);
  const int64_t share = std::max<int64_t>((total + cus - 1) / cus, 4);
  int64_t n = (tiles_max + share - 1) / share;
  n = std::min({n, tiles_max, kMaxBwdSplits});
  const int64_t plane = a.B * a.H_q * a.N_q * a.D * 4;
  n = std::min(n, kAutoPartBytes / plane);
  n = std::min(n, ea02::abi::max_launch_blocks(64 * nw) / (heads * pair_blocks));
  return worth_splitting(n, tiles_max, share, double(plane), double(plane) / 2);
}

// Waves per dQ workgroup, by the forward's rule for its four-wave shape: four
// when the eight-wave grid is causal with row blocks of very different
// lengths (N_q > N_kv / 2) and covers less than two rounds of the device, or
// fills less than one round even with its key-range splits; eight otherwise.
// Measured (backward, MI355X): causal GQA-4 B=2 N=1024 130.7 -> 125.7 us, causal
// MHA N=512 63.6 -> 55.7 us; larger or even grids 1-4 % faster with eight.
int q_waves(const Shape& a) {
  const int64_t wgs = a.B * a.H_kv * ((a.N_q * (a.H_q / a.H_kv) + 32 * kQNW - 1) / (32 * kQNW));
  const int64_t cus = device_cus();
  if (a.causal && 2 * a.N_q > a.N_kv && wgs < 2 * cus) return kQMidNW;
  if (wgs * choose_q_splits_nw(a, kQNW) < cus) return kQMidNW;
  return kQNW;
}

int64_t choose_q_splits(const Shape& a) { return choose_q_splits_nw(a, q_waves(a)); }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace: per-row L2 and Dl, then (256-byte aligned) the dK/dV partials
// when split, then the dQ partials when split.  Offsets of the partials are
// returned through kv_off and q_off.
size_t workspace_layout(const Shape& a, int64_t n_kv, int64_t n_q, size_t* kv_off = nullptr,
                        size_t* q_off = nullptr) {
  size_t cur = size_t(a.B) * size_t(a.H_q) * size_t(a.N_q) * 8;
  if (n_kv > 1) {
    cur = align256(cur);
    if (kv_off) *kv_off = cur;
    cur += size_t(n_kv) * 2 * size_t(a.B * a.H_kv * a.N_kv * a.D) * 4;
  }
  if (n_q > 1) {
    cur = align256(cur);
    if (q_off) *q_off = cur;
    cur += size_t(n_q) * size_t(a.B * a.H_q * a.N_q * a.D) * 4;
  }
  return cur;
}

// Prep, dK/dV (+ the sum of its splits), dQ.  With no query rows only the
// dK/dV kernel runs: every key block then has no row tile and writes zeros.
template <int D>
hipError_t launch_all(const BwdParams& p_in, int q_nw, hipStream_t s) {
  hipError_t e;
  // Both kernels balance the XCDs by work stealing when their grids are long
  // enough (work_item); they run one after the other on the stream and share
  // its counters.
  BwdParams p = p_in;
  const int64_t kv_items = int64_t(p.n_heads_wg) * p.n_key_blocks * p.n_kv_splits;
  const int64_t q_items = int64_t(p.n_heads_wg) * p.n_pair_blocks * p.n_q_splits;
  const ea02::abi::StealPlan kv_plan = ea02::abi::plan_steal(s, kv_items, 1);
  const ea02::abi::StealPlan q_plan = p.rows > 0 ? ea02::abi::plan_steal(s, q_items, q_nw == kQMidNW ? 2 : 1)
                                                 : ea02::abi::StealPlan{nullptr, static_cast<int>(q_items), q_items};
  p.steal = kv_plan.counters ? kv_plan.counters : q_plan.counters;
  p.kv_items = static_cast<int>(kv_items);
  p.kv_static = kv_plan.n_static;
  p.q_items = static_cast<int>(q_items);
  p.q_static = q_plan.n_static;
  if (p.rows > 0) {
    const int64_t prep_blocks = (p.rows + (256 / (D / 8)) - 1) / (256 / (D / 8));
    hipLaunchKernelGGL((ea02::attn_bwd_prep_kernel<D>), dim3(static_cast<unsigned>(prep_blocks)), dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((ea02::attn_bwd_dkdv_kernel<D, kKvNW, kKvP, kKvBP>),
                     dim3(static_cast<unsigned>(kv_plan.launch_grid)), dim3(kKvNW * 64), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.n_kv_splits > 1) {
    const int64_t quads = int64_t(p.n_heads_wg) * p.N_kv * D / 4;
    hipLaunchKernelGGL((ea02::attn_bwd_kv_reduce_kernel<D>), dim3(static_cast<unsigned>((quads + 255) / 256)), dim3(256),
                       0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (p.rows > 0) {
    const dim3 grid(static_cast<unsigned>(q_plan.launch_grid));
    if (q_nw == kQMidNW)
      hipLaunchKernelGGL((ea02::attn_bwd_dq_kernel<D, kQMidNW, kQMidP, kQBN, 32>), grid, dim3(kQMidNW * 64), 0, s, p);
    else
      hipLaunchKernelGGL((ea02::attn_bwd_dq_kernel<D, kQNW, kQP, kQBN, 16>), grid, dim3(kQNW * 64), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.n_q_splits > 1) {
      const int64_t quads = p.rows * D / 4;
      hipLaunchKernelGGL((ea02::attn_bwd_q_reduce_kernel<D>), dim3(static_cast<unsigned>((quads + 255) / 256)),
                         dim3(256), 0, s, p);
      e = hipGetLastError();
    }
  }
  return e;
}

}  // namespace

extern "C" int64_t attn_bwd_num_splits(int64_t B, int64_t H_q, int64_t H_kv, int64_t N_q, int64_t N_kv, int64_t D,
                                       int is_causal) {
  const Shape a{B, H_q, H_kv, N_q, N_kv, D, is_causal};
  bool empty = false;
  if (check_sizes(a, 0, 1.f, &empty) != ATTN_OK) return -1;
  if (empty) return 1;
  return choose_kv_splits(a);
}

extern "C" size_t attn_bwd_workspace_size(int64_t B, int64_t H_q, int64_t H_kv, int64_t N_q, int64_t N_kv,
                                          int64_t D, int is_causal, int64_t n_splits) {
  const Shape a{B, H_q, H_kv, N_q, N_kv, D, is_causal};
  bool empty = false;
  if (check_sizes(a, n_splits, 1.f, &empty) != ATTN_OK || empty || N_q == 0 || N_kv == 0) return 0;
  return workspace_layout(a, n_splits, choose_q_splits(a));
}

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H_q, int64_t H_kv,
                        int64_t N_q, int64_t N_kv, int64_t D, float sm_scale, int is_causal, int64_t n_splits,
                        void* workspace, size_t workspace_size, void* stream) {
  const Shape a{B, H_q, H_kv, N_q, N_kv, D, is_causal};
  bool empty = false;
  int st = check_sizes(a, n_splits, sm_scale, &empty);
  if (st != ATTN_OK) return st;
  if (empty) return ATTN_OK;
  if (N_kv == 0) return ATTN_ERR_NO_KEYS;
  // with no query rows q, out, dout, lse and dq are empty and may be NULL
  if (!k || !v || !dk || !dv || (N_q > 0 && (!q || !out || !dout || !lse || !dq))) return ATTN_ERR_NULL_POINTER;
  auto mis16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; };
  if (mis16(q) || mis16(k) || mis16(v) || mis16(out) || mis16(dout) || mis16(dq) || mis16(dk) || mis16(dv) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return ATTN_ERR_ALIGNMENT;
  // no query rows: nothing to split (the key blocks write zeros)
  const int64_t splits = N_q == 0 ? 1 : (n_splits == 0 ? choose_kv_splits(a) : n_splits);
  const int q_nw = q_waves(a);
  const int64_t q_splits = choose_q_splits_nw(a, q_nw);
  size_t kv_off = 0, q_off = 0;
  const size_t need = N_q == 0 ? 0 : workspace_layout(a, splits, q_splits, &kv_off, &q_off);
  if (need > 0 && (!workspace || workspace_size < need || (reinterpret_cast<uintptr_t>(workspace) & 15u)))
    return ATTN_ERR_WORKSPACE;
  const int64_t G = H_q / H_kv;
  const size_t nq = size_t(B * H_q * N_q * D) * 2, nkv = size_t(B * H_kv * N_kv * D) * 2;
  const size_t nl = size_t(B * H_q * N_q) * 4;
  const void* ins[6] = {q, k, v, out, dout, lse};
  const size_t in_n[6] = {nq, nkv, nkv, nq, nq, nl};
  const void* outs[4] = {dq, dk, dv, workspace};
  const size_t out_n[4] = {nq, nkv, nkv, need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return ATTN_ERR_ALIAS;
  }

  BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(out);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.lse2 = static_cast<float*>(workspace);
  p.delta = static_cast<float*>(workspace) + size_t(B * H_q * N_q);
  p.kv_part = splits > 1 ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kv_off) : nullptr;
  p.q_part = q_splits > 1 ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + q_off) : nullptr;
  p.B = static_cast<int>(B);
  p.H_q = static_cast<int>(H_q);
  p.H_kv = static_cast<int>(H_kv);
  p.N_q = static_cast<int>(N_q);
  p.N_kv = static_cast<int>(N_kv);
  p.G = static_cast<int>(G);
  p.n_pairs = static_cast<int>(N_q * G);
  p.causal_off = is_causal ? static_cast<int>(N_kv - N_q) : 0;
  p.causal = is_causal;
  p.n_heads_wg = static_cast<int>(B * H_kv);
  p.n_key_blocks = static_cast<int>((N_kv + 32 * kKvNW - 1) / (32 * kKvNW));
  p.n_kv_splits = static_cast<int>(splits);
  p.n_pair_blocks = static_cast<int>((N_q * G + 32 * q_nw - 1) / (32 * q_nw));
  p.n_q_splits = static_cast<int>(q_splits);
  // as in the forward: a zero scale becomes FLT_MIN in the exponent (uniform
  // weights, no 0 * inf); the gradient factors use the scale as given
  p.scale_log2 = std::fmax(std::fabs(sm_scale) * ea02::kLog2e, FLT_MIN);
  p.grad_scale = sm_scale;
  p.k_sign = (sm_scale < 0.f) ? 0x80008000u : 0u;
  p.q_sign = p.k_sign;
  p.rows = B * H_q * N_q;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err = (D == 128) ? launch_all<128>(p, q_nw, s) : launch_all<64>(p, q_nw, s);
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
