// C ABI of the fused attention forward (declared in include/attn.h):
// argument validation, kernel-shape and split choice, and kernel launches.
// The library allocates nothing and never synchronises.  Its only state is in
// two file-scope device arrays (the static scratch of attn_fwd_splitkv_static
// and the work-stealing counters, which every launch leaves at zero) and, on
// the host, their addresses per device and the counter slot of each stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "../../include/attn.h"
#include "attn_fwd_kernel.hpp"
#include "abi_util.hpp"

namespace {

using ea02::abi::device_cus;
using ea02::abi::overlaps;

using ea02::FwdParams;
using ea02::MergeParams;

// Kernel shapes.  Wide: eight waves of 32 (row, head) pairs share each K/V
// tile (256 pairs per workgroup, 64-key tiles, four LDS stages, 128 KiB LDS,
// one workgroup per CU).  Mid: four such waves (128 pairs, two stages, 64 KiB
// LDS, two workgroups per CU: the same eight waves per CU in workgroups half
// as long), for small grids (pick_shape).  Narrow:
// one wave of 32 pairs (32-key tiles, two stages, 32 KiB LDS at D=128) for kv
// heads with at most kNarrowPairs pairs, e.g. a decode step, where the wide
// shape would leave most waves without a query; five (D=128) or eight (D=64,
// register-bound) fit on a CU, which keeps enough loads in flight for such
// HBM-bound work.
constexpr int kWideNW = 8, kWideP = 4, kWideBN = 64, kWideMN = 16;
constexpr int kMidNW = 4, kMidP = 2, kMidBN = 64, kMidMN = 32;
constexpr int kNarrowNW = 1, kNarrowP = 2, kNarrowBN = 32, kNarrowMN = 32;
constexpr int kNarrowPairs = 64;
constexpr int kMaxSplits = 256;
constexpr int kMaxDevices = 64;


enum class Kind { kWide, kMid, kNarrow };

struct Shape {
  Kind kind;
  int pairs_per_wg;
  int bn;
  int wg_per_cu;
};

constexpr Shape kWideShape{Kind::kWide, 32 * kWideNW, kWideBN, 1};
constexpr Shape kMidShape{Kind::kMid, 32 * kMidNW, kMidBN, 2};

// Key splits for a grid of wgs workgroups of shape sh over n_kv keys: none
// while the unsplit grid already fills every workgroup slot of the device;
// otherwise enough splits for about two workgroups per CU, or one for the
// wide shape (one fits a CU: a second round of workgroups measured slower
// than fewer, longer splits), each split keeping at least 8 key tiles.
int64_t splits_for(const Shape& sh, int64_t wgs, int64_t n_kv) {
  const int64_t cus = device_cus();
  if (wgs <= 0 || wgs >= cus * sh.wg_per_cu) return 1;
  const int64_t tiles = (n_kv + sh.bn - 1) / sh.bn;
  const int64_t target = std::min<int64_t>(2, sh.wg_per_cu) * cus;
  int64_t n = (target + wgs - 1) / wgs;
  n = std::min<int64_t>(n, tiles / 8);
  n = std::min<int64_t>(n, kMaxSplits);
  // the split grid stays within one dispatch
  n = std::min<int64_t>(n, ea02::abi::max_launch_blocks(64 * kWideNW) / wgs);
  return n < 1 ? 1 : n;
}

// Shape of a problem with n_pairs (row, head) pairs per kv head and n_heads =
// B * H_kv kv heads.  The mid shape replaces the wide one in two cases, both
// measured: (1) a causal grid whose row blocks differ widely in length (N_q >
// N_kv / 2, so the first blocks see few keys and the last ones all of them)
// and that the wide shape covers in less than two rounds of the device: half
// as long workgroups balance the CUs (causal GQA-4 B=2 N=1024: 40.0 -> 34.7
// us); (2) a grid that fills less than one round even with the wide shape's
// key splits (more, shorter workgroups).  Grids of even rows (non-causal, or
// a short causal chunk against a long cache) at one round or more, and
// larger grids, run 1-3 % faster with the wide shape's deeper ring.
Shape pick_shape(int64_t n_pairs, int64_t D, int64_t n_heads, int64_t N_q, int64_t N_kv, bool causal) {
  if (n_pairs <= kNarrowPairs) return {Kind::kNarrow, 32 * kNarrowNW, kNarrowBN, D == 128 ? 5 : 8};
  const int64_t cus = device_cus();
  const int64_t wide_wgs = (n_pairs + kWideShape.pairs_per_wg - 1) / kWideShape.pairs_per_wg * n_heads;
  if (causal && 2 * N_q > N_kv && wide_wgs < 2 * cus) return kMidShape;
  if (wide_wgs * splits_for(kWideShape, wide_wgs, N_kv) < cus) return kMidShape;
  return kWideShape;
}

int shape_threads(Kind kind) {
  return 64 * (kind == Kind::kNarrow ? kNarrowNW : kind == Kind::kMid ? kMidNW : kWideNW);
}

template <int D, bool SPLIT>
hipError_t launch_fwd(Kind kind, const FwdParams& p, int grid, hipStream_t stream) {
  if (kind == Kind::kNarrow)
    hipLaunchKernelGGL((ea02::attn_fwd_kernel<D, kNarrowNW, kNarrowP, 1, kNarrowBN, kNarrowMN, SPLIT>), dim3(grid),
                       dim3(kNarrowNW * 64), 0, stream, p);
  else if (kind == Kind::kMid)
    hipLaunchKernelGGL((ea02::attn_fwd_kernel<D, kMidNW, kMidP, 1, kMidBN, kMidMN, SPLIT>), dim3(grid),
                       dim3(kMidNW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((ea02::attn_fwd_kernel<D, kWideNW, kWideP, 1, kWideBN, (SPLIT ? 32 : kWideMN), SPLIT>), dim3(grid),
                       dim3(kWideNW * 64), 0, stream, p);
  return hipGetLastError();
}

// One block per output row; the block's split lanes grow with the split count
// so that each thread merges at most kMergeBatch splits (blocks of 64, 256 or
// 1024 threads), or up to 4 kMergeBatch in the largest block, all loaded in
// one round.
template <int D>
hipError_t launch_merge(const MergeParams& m, hipStream_t stream) {
  constexpr int tpr = D / 4;
  constexpr int kb = ea02::kMergeBatch;
  if (m.n_splits <= kb * (64 / tpr)) return ea02::launch_merge_rows<D, 64, kb>(m, stream);
  if (m.n_splits <= kb * (256 / tpr)) return ea02::launch_merge_rows<D, 256, kb>(m, stream);
  if (m.n_splits <= kb * (1024 / tpr)) return ea02::launch_merge_rows<D, 1024, kb>(m, stream);
  return ea02::launch_merge_rows<D, 1024, 4 * kb>(m, stream);
}

// Arguments shared by both entry points, after validation.
struct Problem {
  const void *q, *k, *v;
  void* out;
  float* lse;
  int64_t B, H_q, H_kv, N_q, N_kv, D;
  float sm_scale;
  int is_causal;
};

Shape problem_shape(const Problem& a) {
  return pick_shape(a.N_q * (a.H_q / a.H_kv), a.D, a.B * a.H_kv, a.N_q, a.N_kv, a.is_causal != 0);
}

// Checks common to both entry points, in the documented order, up to and
// including the empty-work test (*empty set when there is nothing to do).
int check_sizes(const Problem& a, int64_t n_splits, bool* empty) {
  *empty = false;
  if (a.B < 0 || a.H_q < 0 || a.H_kv < 0 || a.N_q < 0 || a.N_kv < 0 || a.D < 0 || n_splits < 0)
    return ATTN_ERR_NEGATIVE_SIZE;
  if (a.H_kv < 1 || a.H_q % a.H_kv != 0) return ATTN_ERR_HEAD_RATIO;
  if (a.D != 64 && a.D != 128) return ATTN_ERR_HEAD_DIM;
  if (a.is_causal != 0 && a.is_causal != 1) return ATTN_ERR_CAUSAL_FLAG;
  if (!std::isfinite(a.sm_scale)) return ATTN_ERR_SCALE;
  if (n_splits > kMaxSplits) return ATTN_ERR_SPLITS;
  if (a.is_causal && a.N_q > a.N_kv) return ATTN_ERR_CAUSAL_SHAPE;
  // K/V rows are addressed with 32-bit byte offsets within one kv head
  const int64_t lim24 = int64_t(1) << 24;
  if (a.N_q > lim24 || a.N_kv > lim24 || a.N_kv * a.D * 2 > (int64_t(1) << 31) || a.B > lim24 ||
      a.H_q > (int64_t(1) << 16) || a.B * a.H_q * a.N_q > INT32_MAX)
    return ATTN_ERR_SIZE_OVERFLOW;
  const int64_t n_pairs = a.N_q * (a.H_q / a.H_kv);
  if (n_pairs > (int64_t(1) << 30)) return ATTN_ERR_SIZE_OVERFLOW;
  const Shape sh = problem_shape(a);
  const int64_t grid = ((n_pairs + sh.pairs_per_wg - 1) / sh.pairs_per_wg) * a.B * a.H_kv *
                       (n_splits > 1 ? n_splits : 1);
  if (grid > ea02::abi::max_launch_blocks(shape_threads(sh.kind))) return ATTN_ERR_SIZE_OVERFLOW;
  if (a.B == 0 || a.H_q == 0 || a.N_q == 0) {
    *empty = true;
    return ATTN_OK;
  }
  if (a.N_kv == 0) return ATTN_ERR_NO_KEYS;
  return ATTN_OK;
}

int check_buffers(const Problem& a) {
  if (!a.q || !a.k || !a.v || !a.out || !a.lse) return ATTN_ERR_NULL_POINTER;
  auto mis16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  if (mis16(a.q) || mis16(a.k) || mis16(a.v) || mis16(a.out) || (reinterpret_cast<uintptr_t>(a.lse) & 3u))
    return ATTN_ERR_ALIGNMENT;
  return ATTN_OK;
}

int check_alias(const Problem& a, const void* ws, size_t ws_used) {
  const size_t nq = size_t(a.B * a.H_q * a.N_q * a.D) * 2, nkv = size_t(a.B * a.H_kv * a.N_kv * a.D) * 2;
  const size_t nl = size_t(a.B * a.H_q * a.N_q) * 4;
  const void* ins[3] = {a.q, a.k, a.v};
  const size_t in_n[3] = {nq, nkv, nkv};
  for (int i = 0; i < 3; ++i)
    if (overlaps(a.out, nq, ins[i], in_n[i]) || overlaps(a.lse, nl, ins[i], in_n[i]) ||
        overlaps(ws, ws_used, ins[i], in_n[i]))
      return ATTN_ERR_ALIAS;
  if (overlaps(a.out, nq, a.lse, nl) || overlaps(ws, ws_used, a.out, nq) || overlaps(ws, ws_used, a.lse, nl))
    return ATTN_ERR_ALIAS;
  return ATTN_OK;
}

// bf16 partial outputs, then fp32 partial LSEs
size_t workspace_bytes(int64_t B, int64_t H_q, int64_t N_q, int64_t D, int64_t n_splits) {
  if (n_splits <= 1) return 0;
  return size_t(n_splits) * size_t(B * H_q * N_q) * size_t(2 * D + 4);
}

// Number of key splits the library picks (splits_for on the problem's shape).
int64_t choose_splits(const Problem& a) {
  const int64_t n_pairs = a.N_q * (a.H_q / a.H_kv);
  const Shape sh = problem_shape(a);
  return splits_for(sh, ((n_pairs + sh.pairs_per_wg - 1) / sh.pairs_per_wg) * a.B * a.H_kv, a.N_kv);
}

}  // namespace

// ---- counters of the work stealing between XCDs (work_item): one slot of
// 16 ints per (device, stream), in this file-scope device array (one copy per
// GPU).  Launches on one stream run one after another, and each leaves its
// slot at zero, so a slot serves every launch of its stream (forward and
// backward kernels alike).  As with the static scratch, host code only uses
// the address that hipGetSymbolAddress returns for the current device.
static constexpr int kStealSlots = 256;
static constexpr int kStealSlotInts = 16;
static __device__ __attribute__((aligned(256))) int steal_counters[kStealSlots * kStealSlotInts];

namespace {

// A launch steals work when its grid covers at least this many rounds of the
// device (shorter launches measured no gain); it keeps the first 70 % of each
// XCD's list static and launches up to 10 % more workgroups per list for the
// fast XCDs to claim with.
constexpr int64_t kStealMinRounds = 8;
constexpr int64_t kStealStaticPct = 70;
constexpr int64_t kStealSparePct = 10;

struct StealSlots {
  int* base = nullptr;
  int used = 0;
  hipStream_t stream[kStealSlots];
  bool zeroed[kStealSlots];
};
std::mutex g_steal_mu;
StealSlots g_steal[kMaxDevices];

}  // namespace

namespace ea02 {
namespace abi {

int* steal_slot(hipStream_t stream) {
  if (stream == hipStreamPerThread) return nullptr;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess) {
    (void)hipGetLastError();  // the query's error is not the launch's
    return nullptr;
  }
  if (cap != hipStreamCaptureStatusNone) return nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_steal_mu);
  StealSlots& d = g_steal[dev];
  if (!d.base) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(steal_counters)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    d.base = static_cast<int*>(ptr);
  }
  int i = 0;
  while (i < d.used && d.stream[i] != stream) ++i;
  if (i == d.used) {
    if (d.used == kStealSlots) return nullptr;
    d.stream[i] = stream;
    d.zeroed[i] = false;
    ++d.used;
  }
  int* slot = d.base + i * kStealSlotInts;
  if (!d.zeroed[i]) {
    if (hipMemsetAsync(slot, 0, kStealSlotInts * sizeof(int), stream) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    d.zeroed[i] = true;
  }
  return slot;
}

StealPlan plan_steal(hipStream_t stream, int64_t items, int64_t wg_per_cu) {
  StealPlan plan{nullptr, static_cast<int>(items), items};
  if (items < kStealMinRounds * wg_per_cu * device_cus() || items >= (int64_t(1) << 30)) return plan;
  int* slot = steal_slot(stream);
  if (!slot) return plan;
  plan.counters = slot;
  plan.n_static = static_cast<int>(8 * (items / 8 * kStealStaticPct / 100));
  plan.launch_grid = items + 8 * ((items / 8 * kStealSparePct + 99) / 100);
  return plan;
}

}  // namespace abi
}  // namespace ea02

namespace {

using ea02::abi::plan_steal;
using ea02::abi::StealPlan;

// Launch after every check passed: one pass when n_splits <= 1, else the split
// pass into the workspace followed by the merge.
int run(const Problem& a, int64_t n_splits, void* ws, void* stream) {
  const int G = static_cast<int>(a.H_q / a.H_kv);
  const int64_t n_pairs = a.N_q * G;
  const Shape sh = problem_shape(a);
  const int64_t n_pair_blocks = (n_pairs + sh.pairs_per_wg - 1) / sh.pairs_per_wg;
  const bool split = n_splits > 1;
  const int64_t grid = n_pair_blocks * a.B * a.H_kv * (split ? n_splits : 1);
  const int64_t rows = a.B * a.H_q * a.N_q;

  FwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.out);
  p.lse = a.lse;
  p.o_part = split ? static_cast<uint16_t*>(ws) : nullptr;
  p.lse_part = split ? reinterpret_cast<float*>(static_cast<uint16_t*>(ws) + size_t(n_splits) * size_t(rows) * size_t(a.D))
                     : nullptr;
  p.B = static_cast<int>(a.B);
  p.H_q = static_cast<int>(a.H_q);
  p.H_kv = static_cast<int>(a.H_kv);
  p.N_q = static_cast<int>(a.N_q);
  p.N_kv = static_cast<int>(a.N_kv);
  p.G = G;
  p.n_pairs = static_cast<int>(n_pairs);
  p.causal_off = a.is_causal ? static_cast<int>(a.N_kv - a.N_q) : 0;
  p.n_pair_blocks = static_cast<int>(n_pair_blocks);
  p.n_heads_wg = static_cast<int>(a.B * a.H_kv);
  p.n_splits = split ? static_cast<int>(n_splits) : 1;
  // A zero scale becomes the smallest normal float: finite scores times it
  // round to 0 in the exponent (uniform weights, as for a zero scale), while
  // masked scores (-inf) stay -inf instead of turning into NaN.
  p.scale_log2 = std::fmax(std::fabs(a.sm_scale) * ea02::kLog2e, FLT_MIN);
  p.q_sign = (a.sm_scale < 0.f) ? 0x80008000u : 0u;
  p.causal = a.is_causal;

  hipStream_t s = static_cast<hipStream_t>(stream);
  // the eight-wave single pass balances the XCDs (work_item)
  const StealPlan plan = (!split && sh.kind == Kind::kWide) ? plan_steal(s, grid, sh.wg_per_cu)
                                                           : StealPlan{nullptr, static_cast<int>(grid), grid};
  p.steal = plan.counters;
  p.n_items = static_cast<int>(grid);
  p.n_static = plan.n_static;
  const int g32 = static_cast<int>(plan.launch_grid);
  hipError_t err;
  if (!split)
    err = (a.D == 128) ? launch_fwd<128, false>(sh.kind, p, g32, s) : launch_fwd<64, false>(sh.kind, p, g32, s);
  else
    err = (a.D == 128) ? launch_fwd<128, true>(sh.kind, p, g32, s) : launch_fwd<64, true>(sh.kind, p, g32, s);
  if (err != hipSuccess) return ATTN_ERR_LAUNCH;
  if (split) {
    MergeParams m;
    m.o_part = p.o_part;
    m.lse_part = p.lse_part;
    m.o = p.o;
    m.lse = p.lse;
    m.rows = rows;
    m.n_splits = p.n_splits;
    err = (a.D == 128) ? launch_merge<128>(m, s) : launch_merge<64>(m, s);
    if (err != hipSuccess) return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                        int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t D,
                        float sm_scale, int is_causal, void* stream) {
  const Problem a{q, k, v, out, lse, B, H_q, H_kv, N, N, D, sm_scale, is_causal};
  bool empty = false;
  int st = check_sizes(a, 1, &empty);
  if (st != ATTN_OK || empty) return st;
  if ((st = check_buffers(a)) != ATTN_OK) return st;
  if ((st = check_alias(a, nullptr, 0)) != ATTN_OK) return st;
  return run(a, 1, nullptr, stream);
}

extern "C" int64_t attn_splitkv_num_splits(int64_t B, int64_t H_q, int64_t H_kv, int64_t N_q, int64_t N_kv,
                                           int64_t D, int is_causal) {
  const Problem a{nullptr, nullptr, nullptr, nullptr, nullptr, B, H_q, H_kv, N_q, N_kv, D, 1.f, is_causal};
  bool empty = false;
  if (check_sizes(a, 0, &empty) != ATTN_OK) return -1;
  if (empty) return 1;
  return choose_splits(a);
}

extern "C" size_t attn_splitkv_workspace_size(int64_t B, int64_t H_q, int64_t N_q, int64_t D, int64_t n_splits) {
  if (B < 0 || H_q < 0 || N_q < 0 || D < 0 || n_splits < 0 || n_splits > kMaxSplits) return 0;
  return workspace_bytes(B, H_q, N_q, D, n_splits);
}

extern "C" int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* out, float* lse,
                                int64_t B, int64_t H_q, int64_t H_kv, int64_t N_q, int64_t N_kv, int64_t D,
                                float sm_scale, int is_causal, int64_t n_splits, void* workspace,
                                size_t workspace_size, void* stream) {
  const Problem a{q, k, v, out, lse, B, H_q, H_kv, N_q, N_kv, D, sm_scale, is_causal};
  bool empty = false;
  int st = check_sizes(a, n_splits, &empty);
  if (st != ATTN_OK || empty) return st;
  if ((st = check_buffers(a)) != ATTN_OK) return st;
  const int64_t ns = n_splits == 0 ? choose_splits(a) : n_splits;
  const size_t need = workspace_bytes(B, H_q, N_q, D, ns);
  if (need > 0 && (!workspace || workspace_size < need || (reinterpret_cast<uintptr_t>(workspace) & 15u)))
    return ATTN_ERR_WORKSPACE;
  if ((st = check_alias(a, workspace, need)) != ATTN_OK) return st;
  return run(a, ns, workspace, stream);
}

// ---- the split forward without a caller workspace (for callers that cannot
// allocate device memory: code under HIP graph capture, tight serving loops).
// Its partial results live in this file-scope device array, one copy per GPU
// the library runs on, held until the process ends.  Host code never passes
// the array's name to a kernel (in host code it is a host-side stand-in):
// the first call on a device looks up that device's address with
// hipGetSymbolAddress and keeps it.
static constexpr size_t kStaticScratchBytes = size_t(16) << 20;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kStaticScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of this device's scratch (looked up once per device, with the
// device current), or nullptr when the lookup fails.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" size_t attn_static_scratch_bytes(void) { return kStaticScratchBytes; }

extern "C" int attn_fwd_splitkv_static(const void* q, const void* k, const void* v, void* out, float* lse,
                                       int64_t B, int64_t H_q, int64_t H_kv, int64_t N_q, int64_t N_kv,
                                       int64_t D, float sm_scale, int is_causal, int64_t n_splits,
                                       void* stream) {
  const Problem a{q, k, v, out, lse, B, H_q, H_kv, N_q, N_kv, D, sm_scale, is_causal};
  bool empty = false;
  int st = check_sizes(a, n_splits, &empty);
  if (st != ATTN_OK || empty) return st;
  if ((st = check_buffers(a)) != ATTN_OK) return st;
  int64_t ns = n_splits;
  if (ns == 0) {
    // the library's choice, lowered until its partials fit the static scratch
    ns = choose_splits(a);
    while (ns > 1 && workspace_bytes(B, H_q, N_q, D, ns) > kStaticScratchBytes) --ns;
  } else if (workspace_bytes(B, H_q, N_q, D, ns) > kStaticScratchBytes) {
    return ATTN_ERR_STATIC_SCRATCH;
  }
  if ((st = check_alias(a, nullptr, 0)) != ATTN_OK) return st;
  void* ws = nullptr;
  if (ns > 1 && !(ws = device_scratch())) return ATTN_ERR_LAUNCH;
  return run(a, ns, ws, stream);
}

extern "C" const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NEGATIVE_SIZE: return "a size argument is negative";
    case ATTN_ERR_HEAD_RATIO: return "H_kv must be >= 1 and divide H_q";
    case ATTN_ERR_HEAD_DIM:
      return "unsupported head dimension (D 64 or 128; MLA: d_c 512, d_R 64, d_nope 1..256, d_v a multiple of 32 "
             "up to 1024)";
    case ATTN_ERR_CAUSAL_FLAG: return "is_causal must be 0 or 1";
    case ATTN_ERR_SCALE: return "sm_scale must be finite";
    case ATTN_ERR_SIZE_OVERFLOW:
      return "sizes exceed the supported range (N <= 2^24, N_kv*D*2 <= 2^31, B*H_q*N_q < 2^31, N_q*H_q/H_kv <= 2^30)";
    case ATTN_ERR_NULL_POINTER: return "a buffer pointer is NULL";
    case ATTN_ERR_ALIGNMENT: return "q, k, v, out must be 16-byte aligned and lse 4-byte aligned";
    case ATTN_ERR_ALIAS: return "out or lse overlaps an input or each other";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_CAUSAL_SHAPE: return "is_causal needs N_q <= N_kv";
    case ATTN_ERR_NO_KEYS: return "N_kv is 0 while there are query rows";
    case ATTN_ERR_SPLITS: return "n_splits must be in [0, 256] (attn_bwd: [0, 64])";
    case ATTN_ERR_WORKSPACE: return "workspace is NULL, too small or not 16-byte aligned";
    case ATTN_ERR_STATIC_SCRATCH:
      return "the requested key splits need more partial-result memory than the library's static scratch "
             "(attn_static_scratch_bytes) holds";
    default: return "unknown status";
  }
}

extern "C" int attn_abi_version(void) { return 8; }
