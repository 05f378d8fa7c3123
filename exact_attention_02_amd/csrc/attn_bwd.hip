// C ABI of the attention backward (declared in include/attn.h): argument
// validation and the three kernel launches.  The library allocates nothing,
// keeps no state and never synchronises.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "../../include/attn.h"
#include "attn_bwd_kernel.hpp"

namespace {

using ea02::BwdParams;

// dK/dV: four waves of 32 keys (128 keys per workgroup), 64-row tiles of Q and
// dO, four LDS stages (136 KiB at D=128).  dQ: eight waves of 32 (row, head)
// pairs (256 per workgroup, two waves per SIMD), 64-key tiles of K and V, four
// stages (128 KiB at D=128).
constexpr int kKvNW = 4, kKvP = 4, kKvBP = 64;
constexpr int kQNW = 8, kQP = 4, kQBN = 64;

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Prep, dK/dV, dQ.  With no query rows only the dK/dV kernel runs: every key
// block then has no row tile and writes zeros.
template <int D>
hipError_t launch_all(const BwdParams& p, hipStream_t s) {
  hipError_t e;
  if (p.rows > 0) {
    const int64_t prep_blocks = (p.rows + (256 / (D / 8)) - 1) / (256 / (D / 8));
    hipLaunchKernelGGL((ea02::attn_bwd_prep_kernel<D>), dim3(static_cast<unsigned>(prep_blocks)), dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((ea02::attn_bwd_dkdv_kernel<D, kKvNW, kKvP, kKvBP>),
                     dim3(static_cast<unsigned>(p.n_heads_wg * p.n_key_blocks)), dim3(kKvNW * 64), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.rows > 0) {
    hipLaunchKernelGGL((ea02::attn_bwd_dq_kernel<D, kQNW, kQP, kQBN>),
                       dim3(static_cast<unsigned>(p.n_heads_wg * p.n_pair_blocks)), dim3(kQNW * 64), 0, s, p);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

extern "C" size_t attn_bwd_workspace_size(int64_t B, int64_t H_q, int64_t N_q) {
  if (B < 0 || H_q < 0 || N_q < 0) return 0;
  return size_t(B) * size_t(H_q) * size_t(N_q) * 8;
}

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H_q, int64_t H_kv,
                        int64_t N_q, int64_t N_kv, int64_t D, float sm_scale, int is_causal, void* workspace,
                        size_t workspace_size, void* stream) {
  if (B < 0 || H_q < 0 || H_kv < 0 || N_q < 0 || N_kv < 0 || D < 0) return ATTN_ERR_NEGATIVE_SIZE;
  if (H_kv < 1 || H_q % H_kv != 0) return ATTN_ERR_HEAD_RATIO;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if (is_causal != 0 && is_causal != 1) return ATTN_ERR_CAUSAL_FLAG;
  if (!std::isfinite(sm_scale)) return ATTN_ERR_SCALE;
  if (is_causal && N_q > N_kv) return ATTN_ERR_CAUSAL_SHAPE;
  const int64_t lim24 = int64_t(1) << 24;
  const int64_t G = H_kv > 0 ? H_q / H_kv : 0;
  // one kv group's Q / dO rows and one kv head's K / V rows take 32-bit byte offsets
  if (N_q > lim24 || N_kv > lim24 || B > lim24 || H_q > (int64_t(1) << 16) ||
      N_kv * D * 2 > (int64_t(1) << 31) || N_q * G * D * 2 > (int64_t(1) << 31) ||
      B * H_q * N_q > INT32_MAX)
    return ATTN_ERR_SIZE_OVERFLOW;
  const int64_t key_blocks = (N_kv + 32 * kKvNW - 1) / (32 * kKvNW);
  const int64_t pair_blocks = (N_q * G + 32 * kQNW - 1) / (32 * kQNW);
  if (B * H_kv * key_blocks > INT32_MAX || B * H_kv * pair_blocks > INT32_MAX) return ATTN_ERR_SIZE_OVERFLOW;
  if (B == 0 || H_q == 0 || (N_q == 0 && N_kv == 0)) return ATTN_OK;
  if (N_kv == 0) return ATTN_ERR_NO_KEYS;
  // with no query rows q, out, dout, lse and dq are empty and may be NULL
  if (!k || !v || !dk || !dv || (N_q > 0 && (!q || !out || !dout || !lse || !dq))) return ATTN_ERR_NULL_POINTER;
  auto mis16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; };
  if (mis16(q) || mis16(k) || mis16(v) || mis16(out) || mis16(dout) || mis16(dq) || mis16(dk) || mis16(dv) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return ATTN_ERR_ALIGNMENT;
  const size_t need = attn_bwd_workspace_size(B, H_q, N_q);
  if (need > 0 && (!workspace || workspace_size < need || (reinterpret_cast<uintptr_t>(workspace) & 15u)))
    return ATTN_ERR_WORKSPACE;
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
  p.n_key_blocks = static_cast<int>(key_blocks);
  p.n_pair_blocks = static_cast<int>(pair_blocks);
  // as in the forward: a zero scale becomes FLT_MIN in the exponent (uniform
  // weights, no 0 * inf); the gradient factors use the scale as given
  p.scale_log2 = std::fmax(std::fabs(sm_scale) * ea02::kLog2e, FLT_MIN);
  p.grad_scale = sm_scale;
  p.k_sign = (sm_scale < 0.f) ? 0x80008000u : 0u;
  p.q_sign = p.k_sign;
  p.rows = B * H_q * N_q;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err = (D == 128) ? launch_all<128>(p, s) : launch_all<64>(p, s);
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
