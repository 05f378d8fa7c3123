// C ABI of the MLA decode path (declared in include/attn.h): the latent
// attention core with its key split and merge, the query absorption and the
// value up-projection.  The library allocates nothing and never synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "../../include/attn.h"
#include "attn_mla_kernel.hpp"
#include "abi_util.hpp"

namespace {

using ea02::abi::device_cus;
using ea02::abi::overlaps;

using ea02::MlaParams;
using ea02::MlaProjParams;
constexpr int kMlaP = 4;
constexpr int kMlaPairs = 64;  // (token, head) pairs per workgroup
constexpr int kMlaMaxSplits = 256;

bool mis16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

size_t mla_ws_bytes(int64_t B, int64_t H, int64_t S, int64_t n_splits) {
  if (n_splits <= 1) return 0;
  return size_t(n_splits) * size_t(B * H * S) * size_t(2 * ea02::kMlaDc + 4);  // bf16 partial O, fp32 LSE
}

// size checks shared by the core's entry points
int mla_check_sizes(int64_t B, int64_t H, int64_t S, int64_t T, int64_t d_c, int64_t d_r, int is_causal,
                    int64_t n_splits) {
  if (B < 0 || H < 0 || S < 0 || T < 0 || d_c < 0 || d_r < 0 || n_splits < 0) return ATTN_ERR_NEGATIVE_SIZE;
  if (d_c != ea02::kMlaDc || d_r != ea02::kMlaDr) return ATTN_ERR_HEAD_DIM;
  if (is_causal != 0 && is_causal != 1) return ATTN_ERR_CAUSAL_FLAG;
  if (n_splits > kMlaMaxSplits) return ATTN_ERR_SPLITS;
  if (is_causal && S > T) return ATTN_ERR_CAUSAL_SHAPE;
  if (B > (1 << 24) || H > (1 << 16) || S > (1 << 24) || T * ea02::kMlaRowBytes > (int64_t(1) << 31) ||
      S * H > (int64_t(1) << 30) || B * H * S > INT32_MAX)
    return ATTN_ERR_SIZE_OVERFLOW;
  const int64_t pbs = (S * H + kMlaPairs - 1) / kMlaPairs;
  if (pbs * B * std::max<int64_t>(n_splits, 1) > ea02::abi::max_launch_blocks(256)) return ATTN_ERR_SIZE_OVERFLOW;
  return ATTN_OK;
}

// (token, head) pairs per workgroup of the latent core that serves this shape
// (token, head) pairs per workgroup of the latent core that serves this
// shape: the sixteen-pair kernel (128 per workgroup, two waves per SIMD) once
// its workgroups, before any split, number at least an eighth of the CUs;
// below that it would need twice the splits of the four-wave kernel (64 per
// workgroup), whose partial outputs and re-read queries then cost more than
// its latency saves (measured at B = 1 and 8 with H = 128, S = 1).
int64_t mla_core_pairs(int64_t B, int64_t H, int64_t S) {
  const int64_t wide_wgs = ((S * H + ea02::kMla16Pairs - 1) / ea02::kMla16Pairs) * B;
  return 8 * wide_wgs >= device_cus() ? ea02::kMla16Pairs : kMlaPairs;
}

int64_t mla_choose_splits(int64_t B, int64_t H, int64_t S, int64_t T) {
  const int64_t pairs = mla_core_pairs(B, H, S);
  const int64_t wgs = ((S * H + pairs - 1) / pairs) * B;
  const int64_t cus = device_cus();
  if (wgs <= 0 || wgs >= cus) return 1;
  const int64_t tiles = (T + 31) / 32;
  int64_t n = (cus + wgs - 1) / wgs;
  n = std::min<int64_t>(n, tiles / 4);
  n = std::min<int64_t>(n, kMlaMaxSplits);
  return n < 1 ? 1 : n;
}

}  // namespace

extern "C" int64_t attn_mla_num_splits(int64_t B, int64_t H, int64_t S, int64_t T, int is_causal) {
  if (mla_check_sizes(B, H, S, T, ea02::kMlaDc, ea02::kMlaDr, is_causal, 0) != ATTN_OK) return -1;
  if (B == 0 || H == 0 || S == 0) return 1;
  return mla_choose_splits(B, H, S, T);
}

extern "C" size_t attn_mla_workspace_size(int64_t B, int64_t H, int64_t S, int64_t n_splits) {
  if (B < 0 || H < 0 || S < 0 || n_splits < 0 || n_splits > kMlaMaxSplits) return 0;
  return mla_ws_bytes(B, H, S, n_splits);
}

extern "C" int attn_mla_decode(const void* q_lat, const void* kv, void* out_lat, float* lse, int64_t B, int64_t H,
                               int64_t S, int64_t T, int64_t d_c, int64_t d_r, float sm_scale, int is_causal,
                               int64_t n_splits, void* workspace, size_t workspace_size, void* stream) {
  int st = mla_check_sizes(B, H, S, T, d_c, d_r, is_causal, n_splits);
  if (st != ATTN_OK) return st;
  if (!std::isfinite(sm_scale)) return ATTN_ERR_SCALE;
  if (B == 0 || H == 0 || S == 0) return ATTN_OK;
  if (T == 0) return ATTN_ERR_NO_KEYS;
  if (!q_lat || !kv || !out_lat || !lse) return ATTN_ERR_NULL_POINTER;
  if (mis16(q_lat) || mis16(kv) || mis16(out_lat) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return ATTN_ERR_ALIGNMENT;
  const int64_t ns = n_splits == 0 ? mla_choose_splits(B, H, S, T) : n_splits;
  const size_t need = mla_ws_bytes(B, H, S, ns);
  if (need > 0 && (!workspace || workspace_size < need || mis16(workspace))) return ATTN_ERR_WORKSPACE;
  const size_t nq = size_t(B * H * S) * ea02::kMlaDqk * 2, nkv = size_t(B * T) * ea02::kMlaDqk * 2;
  const size_t no = size_t(B * H * S) * ea02::kMlaDc * 2, nl = size_t(B * H * S) * 4;
  if (overlaps(out_lat, no, q_lat, nq) || overlaps(out_lat, no, kv, nkv) || overlaps(lse, nl, q_lat, nq) ||
      overlaps(lse, nl, kv, nkv) || overlaps(out_lat, no, lse, nl) || overlaps(workspace, need, q_lat, nq) ||
      overlaps(workspace, need, kv, nkv) || overlaps(workspace, need, out_lat, no) ||
      overlaps(workspace, need, lse, nl))
    return ATTN_ERR_ALIAS;

  const bool split = ns > 1;
  const int64_t rows = B * H * S;
  MlaParams p;
  p.q = static_cast<const uint16_t*>(q_lat);
  p.kv = static_cast<const uint16_t*>(kv);
  p.o = static_cast<uint16_t*>(out_lat);
  p.lse = lse;
  p.o_part = split ? static_cast<uint16_t*>(workspace) : nullptr;
  p.lse_part = split ? reinterpret_cast<float*>(static_cast<uint16_t*>(workspace) + size_t(ns) * size_t(rows) * ea02::kMlaDc)
                     : nullptr;
  p.B = static_cast<int>(B);
  p.H = static_cast<int>(H);
  p.S = static_cast<int>(S);
  p.T = static_cast<int>(T);
  p.n_pairs = static_cast<int>(S * H);
  p.causal_off = is_causal ? static_cast<int>(T - S) : 0;
  const int64_t pairs = mla_core_pairs(B, H, S);
  const bool wide = pairs == ea02::kMla16Pairs;
  p.n_pair_blocks = static_cast<int>((S * H + pairs - 1) / pairs);
  p.n_splits = split ? static_cast<int>(ns) : 1;
  p.scale_log2 = std::fmax(std::fabs(sm_scale) * ea02::kLog2e, FLT_MIN);
  p.q_sign = (sm_scale < 0.f) ? 0x80008000u : 0u;
  p.causal = is_causal;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(int64_t(p.n_pair_blocks) * B * p.n_splits));
  if (wide && split)
    hipLaunchKernelGGL((ea02::attn_mla16_kernel<kMlaP, true>), grid, dim3(512), 0, s, p);
  else if (wide)
    hipLaunchKernelGGL((ea02::attn_mla16_kernel<kMlaP, false>), grid, dim3(512), 0, s, p);
  else if (split)
    hipLaunchKernelGGL((ea02::attn_mla_kernel<kMlaP, true>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((ea02::attn_mla_kernel<kMlaP, false>), grid, dim3(256), 0, s, p);
  if (hipGetLastError() != hipSuccess) return ATTN_ERR_LAUNCH;
  if (split) {
    ea02::MergeParams m;
    m.o_part = p.o_part;
    m.lse_part = p.lse_part;
    m.o = p.o;
    m.lse = p.lse;
    m.rows = rows;
    m.n_splits = p.n_splits;
    // 128 threads per row (4 of the 512 values each) times 2 or 8 split
    // lanes, each thread with up to 4 or 16 splits loaded in one round.
    // (Slicing a row over several blocks, to spread a decode step's few rows
    // over more CUs, measured no faster: the merge is bound by the bytes of
    // partials it reads, and many-row steps got slower.)
    constexpr int kb = ea02::kMergeBatch;
    const hipError_t e = m.n_splits <= kb * 2   ? ea02::launch_merge_rows<ea02::kMlaDc, 256, kb>(m, s)
                         : m.n_splits <= kb * 8 ? ea02::launch_merge_rows<ea02::kMlaDc, 1024, kb>(m, s)
                                                : ea02::launch_merge_rows<ea02::kMlaDc, 1024, 4 * kb>(m, s);
    if (e != hipSuccess) return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

extern "C" int mla_absorb_q(const void* q_nope, const void* q_pe, const void* w_uk, void* q_lat, int64_t B,
                            int64_t H, int64_t S, int64_t d_nope, int64_t d_c, int64_t d_r, void* stream) {
  if (B < 0 || H < 0 || S < 0 || d_nope < 0 || d_c < 0 || d_r < 0) return ATTN_ERR_NEGATIVE_SIZE;
  if (d_c != ea02::kMlaDc || d_r != ea02::kMlaDr || d_nope < 1 || d_nope > ea02::kAbsorbMaxK) return ATTN_ERR_HEAD_DIM;
  if (B > (1 << 24) || H > (1 << 16) || S > (1 << 24) || B * S > INT32_MAX / 2 || B * H * S > INT32_MAX)
    return ATTN_ERR_SIZE_OVERFLOW;
  if (H * (ea02::kMlaDc / ea02::kAbsorbSlice) > INT32_MAX) return ATTN_ERR_SIZE_OVERFLOW;
  if (B == 0 || H == 0 || S == 0) return ATTN_OK;
  if (!q_nope || !q_pe || !w_uk || !q_lat) return ATTN_ERR_NULL_POINTER;
  if ((reinterpret_cast<uintptr_t>(q_nope) & 1u) || mis16(q_pe) || mis16(w_uk) || mis16(q_lat))
    return ATTN_ERR_ALIGNMENT;
  const size_t nn = size_t(B * H * S * d_nope) * 2, npe = size_t(B * H * S) * ea02::kMlaDr * 2;
  const size_t nw = size_t(H * d_nope) * ea02::kMlaDc * 2, nout = size_t(B * H * S) * ea02::kMlaDqk * 2;
  if (overlaps(q_lat, nout, q_nope, nn) || overlaps(q_lat, nout, q_pe, npe) || overlaps(q_lat, nout, w_uk, nw))
    return ATTN_ERR_ALIAS;
  MlaProjParams p;
  p.x = static_cast<const uint16_t*>(q_nope);
  p.x2 = static_cast<const uint16_t*>(q_pe);
  p.w = static_cast<const uint16_t*>(w_uk);
  p.y = static_cast<uint16_t*>(q_lat);
  p.B = static_cast<int>(B);
  p.H = static_cast<int>(H);
  p.S = static_cast<int>(S);
  p.d_n = static_cast<int>(d_nope);
  p.rows_per_head = static_cast<int>(B * S);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // one block per (head, 128-column slice), every row of the head in it
  const int kp = static_cast<int>((d_nope + 15) & ~int64_t(15));
  const dim3 grid(static_cast<unsigned>(H * (ea02::kMlaDc / ea02::kAbsorbSlice)));
  if (d_nope % 8 == 0 && (reinterpret_cast<uintptr_t>(q_nope) & 15) == 0)
    hipLaunchKernelGGL(ea02::mla_absorb_kernel<true>, grid, dim3(256), ea02::absorb_lds_bytes(kp), s, p);
  else
    hipLaunchKernelGGL(ea02::mla_absorb_kernel<false>, grid, dim3(256), ea02::absorb_lds_bytes(kp), s, p);
  if (hipGetLastError() != hipSuccess) return ATTN_ERR_LAUNCH;
  return ATTN_OK;
}

extern "C" int mla_up_project(const void* out_lat, const void* w_uv, void* out, int64_t B, int64_t H, int64_t S,
                              int64_t d_c, int64_t d_v, void* stream) {
  if (B < 0 || H < 0 || S < 0 || d_c < 0 || d_v < 0) return ATTN_ERR_NEGATIVE_SIZE;
  if (d_c != ea02::kMlaDc || d_v < 32 || d_v > 1024 || d_v % 32 != 0) return ATTN_ERR_HEAD_DIM;
  if (B > (1 << 24) || H > (1 << 16) || S > (1 << 24) || B * S > INT32_MAX / 2 || B * H * S > INT32_MAX)
    return ATTN_ERR_SIZE_OVERFLOW;
  // a dispatch counts its work-items in 32 bits
  const int64_t blocks = (B * S + 31) / 32 * H * (d_v / 32);
  if (blocks > ea02::abi::max_launch_blocks(64)) return ATTN_ERR_SIZE_OVERFLOW;
  if (B == 0 || H == 0 || S == 0) return ATTN_OK;
  if (!out_lat || !w_uv || !out) return ATTN_ERR_NULL_POINTER;
  if (mis16(out_lat) || mis16(w_uv) || (reinterpret_cast<uintptr_t>(out) & 1u)) return ATTN_ERR_ALIGNMENT;
  const size_t nx = size_t(B * H * S) * ea02::kMlaDc * 2, nw = size_t(H * d_v) * ea02::kMlaDc * 2;
  const size_t ny = size_t(B * H * S * d_v) * 2;
  if (overlaps(out, ny, out_lat, nx) || overlaps(out, ny, w_uv, nw)) return ATTN_ERR_ALIAS;
  MlaProjParams p;
  p.x = static_cast<const uint16_t*>(out_lat);
  p.x2 = nullptr;
  p.w = static_cast<const uint16_t*>(w_uv);
  p.y = static_cast<uint16_t*>(out);
  p.B = static_cast<int>(B);
  p.H = static_cast<int>(H);
  p.S = static_cast<int>(S);
  p.d_n = static_cast<int>(d_v);
  p.rows_per_head = static_cast<int>(B * S);
  hipLaunchKernelGGL(ea02::mla_up_kernel, dim3(static_cast<unsigned>(blocks)), dim3(64), 0,
                     static_cast<hipStream_t>(stream), p);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
