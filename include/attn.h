/*
 * attn.h -- C ABI of the MI355X (gfx950) fused attention forward library.
 *
 * The operation is the forward pass of exact scaled-dot-product attention in
 * the FlashAttention-2 style: one query tile stays on chip while key/value
 * tiles stream past, running row statistics (max m, sum l) rescale an fp32
 * output accumulator, causal tiles past the diagonal are skipped, query heads
 * are grouped onto kv heads, and a per-row log-sum-exp is written.
 * Sources: page "Attention Kernel 实现与正确性验证", sections 1.1-1.2 (the
 * three FA-2 tricks, the GQA-aware forward kernel); page "Triton Cuda
 * Attention", sections "在线 Softmax 核心算法" (exp2 form) and "变体改法"
 * (Causal, GQA, MQA); page "Flash Attention 与 Kernel 优化", sections
 * "对外接口", "causal mask" and "输出与保存状态" (log-sum-exp output).
 *
 * Link with libea02_attn.so.  All functions are thread-safe; the library
 * keeps no state between calls and never allocates device memory.
 */
#ifndef EA02_ATTN_H
#define EA02_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  0 is success; every other value names the first failed check. */
enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NEGATIVE_SIZE = 1,  /* B, H_q, H_kv, N or D below zero              */
  ATTN_ERR_HEAD_RATIO = 2,     /* H_kv < 1 or H_q not a multiple of H_kv       */
  ATTN_ERR_HEAD_DIM = 3,       /* D is neither 64 nor 128                      */
  ATTN_ERR_CAUSAL_FLAG = 4,    /* is_causal is neither 0 nor 1                 */
  ATTN_ERR_SCALE = 5,          /* sm_scale is NaN or infinite                  */
  ATTN_ERR_SIZE_OVERFLOW = 6,  /* N > 2^24 or the launch grid exceeds 2^31-1   */
  ATTN_ERR_NULL_POINTER = 7,   /* a buffer pointer is NULL for non-empty work  */
  ATTN_ERR_ALIGNMENT = 8,      /* q,k,v,out not 16-byte or lse not 4-byte aligned */
  ATTN_ERR_ALIAS = 9,          /* out or lse overlaps an input or each other   */
  ATTN_ERR_LAUNCH = 10         /* the HIP runtime rejected the kernel launch   */
};

/*
 * attn_fwd -- enqueue the attention forward on `stream`.
 *
 * For every batch b, query head h in [0, H_q) and query row i in [0, N):
 *   g         = floor(h * H_kv / H_q)           (grouped-query head map; MQA is H_kv = 1)
 *   s_ij      = sm_scale * dot(q[b,h,i,:], k[b,g,j,:])
 *   visible   = all j < N, or j <= i when is_causal (square, top-left aligned)
 *   out[b,h,i,:] = sum_j softmax_j(s_ij) * v[b,g,j,:]      over visible j
 *   lse[b,h,i]   = log(sum_j exp(s_ij))                   over visible j (natural log)
 *
 * Arguments
 *   q     device pointer, bf16, [B, H_q,  N, D] contiguous (row-major, D fastest)
 *   k, v  device pointers, bf16, [B, H_kv, N, D] contiguous
 *   out   device pointer, bf16, [B, H_q,  N, D] contiguous; written (round to nearest even)
 *   lse   device pointer, fp32, [B, H_q,  N]    contiguous; written
 *   B, H_q, H_kv, N, D   sizes; D must be 64 or 128; H_q % H_kv == 0
 *   sm_scale  score scale applied as given (callers normally pass 1/sqrt(D));
 *             any finite value, including 0 and negatives
 *   is_causal 0 or 1
 *   stream    a hipStream_t, or NULL for the default stream
 *
 * Ownership: the caller allocates and frees all five buffers; they must be
 * device memory of the current device.  out and lse must not overlap each
 * other or any input.
 *
 * Synchronisation: the call only enqueues work; results are visible to later
 * work on the same stream.  It never synchronises.
 *
 * Errors: the arguments are checked in the order of enum attn_status; on a
 * failed check nothing is enqueued and nothing is written.  Empty work
 * (B, H_q or N equal to 0) returns ATTN_OK without touching any pointer.
 * No exception crosses the ABI and the library never aborts.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t D,
             float sm_scale, int is_causal, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* attn_status_string(int status);

/* Library ABI version, currently 1. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EA02_ATTN_H */
