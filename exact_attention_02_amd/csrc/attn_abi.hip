// C ABI of the fused attention forward (declared in include/attn.h):
// argument validation, tile-configuration choice and kernel launch.
// The library allocates nothing, keeps no state and never synchronises.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>

#include "../../include/attn.h"
#include "attn_fwd_kernel.hpp"

namespace {

using ea02::FwdParams;

// Kernel shape: KQB query blocks of 32 rows per wave, KNW waves per
// workgroup, KP LDS stages.
constexpr int kQB = 1;
constexpr int kNW = kQB == 1 ? 8 : 4;
constexpr int kBN = kQB == 1 ? 64 : 32;
constexpr int kP = 4;

int gcd_int(int a, int b) {
  while (b) {
    int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

template <int D, int HW>
hipError_t launch(const FwdParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((ea02::attn_fwd_kernel<D, HW, kNW, kP, kQB, kBN>), dim3(grid), dim3(kNW * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdParams& p, int hw, int grid, hipStream_t stream) {
  switch (hw) {
    case 8: if constexpr (kNW >= 8) return launch<D, 8>(p, grid, stream); else return hipErrorInvalidValue;
    case 4: return launch<D, 4>(p, grid, stream);
    case 2: return launch<D, 2>(p, grid, stream);
    default: return launch<D, 1>(p, grid, stream);
  }
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                        int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t D,
                        float sm_scale, int is_causal, void* stream) {
  if (B < 0 || H_q < 0 || H_kv < 0 || N < 0 || D < 0) return ATTN_ERR_NEGATIVE_SIZE;
  if (H_kv < 1 || H_q % H_kv != 0) return ATTN_ERR_HEAD_RATIO;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if (is_causal != 0 && is_causal != 1) return ATTN_ERR_CAUSAL_FLAG;
  if (!std::isfinite(sm_scale)) return ATTN_ERR_SCALE;
  if (N > (int64_t(1) << 24) || B > (int64_t(1) << 24) || H_q > (int64_t(1) << 16))
    return ATTN_ERR_SIZE_OVERFLOW;
  const int G = static_cast<int>(H_q / H_kv);
  const int hw = gcd_int(G, kNW);
  const int BM = 32 * kQB * kNW / hw;
  const int64_t n_row_blocks = (N + BM - 1) / BM;
  const int64_t n_head_groups = G / hw;
  const int64_t n_heads_wg = B * H_kv * n_head_groups;
  const int64_t grid = n_heads_wg * n_row_blocks;
  if (grid > INT32_MAX) return ATTN_ERR_SIZE_OVERFLOW;
  if (B == 0 || H_q == 0 || N == 0) return ATTN_OK;
  if (!q || !k || !v || !out || !lse) return ATTN_ERR_NULL_POINTER;
  auto mis16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  if (mis16(q) || mis16(k) || mis16(v) || mis16(out) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return ATTN_ERR_ALIGNMENT;
  const size_t nq = size_t(B * H_q * N * D) * 2, nkv = size_t(B * H_kv * N * D) * 2;
  const size_t nl = size_t(B * H_q * N) * 4;
  if (overlaps(out, nq, q, nq) || overlaps(out, nq, k, nkv) || overlaps(out, nq, v, nkv) ||
      overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nkv) || overlaps(lse, nl, v, nkv) ||
      overlaps(out, nq, lse, nl))
    return ATTN_ERR_ALIAS;

  FwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.B = static_cast<int>(B);
  p.H_q = static_cast<int>(H_q);
  p.H_kv = static_cast<int>(H_kv);
  p.N = static_cast<int>(N);
  p.G = G;
  p.n_row_blocks = static_cast<int>(n_row_blocks);
  p.n_head_groups = static_cast<int>(n_head_groups);
  p.n_heads_wg = static_cast<int>(n_heads_wg);
  // A zero scale becomes the smallest normal float: finite scores times it
  // round to 0 in the exponent (uniform weights, as for a zero scale), while
  // masked scores (-inf) stay -inf instead of turning into NaN.
  p.scale_log2 = std::fmax(std::fabs(sm_scale) * ea02::kLog2e, FLT_MIN);
  p.q_sign = (sm_scale < 0.f) ? 0x80008000u : 0u;
  p.causal = is_causal;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err = (D == 128) ? launch_d<128>(p, hw, static_cast<int>(grid), s)
                                    : launch_d<64>(p, hw, static_cast<int>(grid), s);
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NEGATIVE_SIZE: return "a size argument is negative";
    case ATTN_ERR_HEAD_RATIO: return "H_kv must be >= 1 and divide H_q";
    case ATTN_ERR_HEAD_DIM: return "head dimension D must be 64 or 128";
    case ATTN_ERR_CAUSAL_FLAG: return "is_causal must be 0 or 1";
    case ATTN_ERR_SCALE: return "sm_scale must be finite";
    case ATTN_ERR_SIZE_OVERFLOW: return "sizes exceed the supported range (N <= 2^24, grid < 2^31)";
    case ATTN_ERR_NULL_POINTER: return "a buffer pointer is NULL";
    case ATTN_ERR_ALIGNMENT: return "q, k, v, out must be 16-byte aligned and lse 4-byte aligned";
    case ATTN_ERR_ALIAS: return "out or lse overlaps an input or each other";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" int attn_abi_version(void) { return 1; }
