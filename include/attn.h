/*
 * attn.h -- C ABI of the MI355X (gfx950) fused attention library (forward,
 * split-KV forward and decode, backward, MLA decode).
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
 * Link with libea02_attn.so.  All functions are thread-safe and the library
 * never allocates device memory.  Results never depend on earlier calls.  The
 * only state a call leaves is host bookkeeping: long single-pass forwards
 * (eight-wave launches of at least eight rounds of the device) balance their
 * work between the XCDs through a few claim counters per (device, stream) in
 * a static device array, which every launch returns to zero.  Up to 256
 * streams per device get such a slot; calls on further streams, on
 * hipStreamPerThread or under graph capture use the static work order, with
 * bit-identical results.  The first such call on a stream also enqueues a
 * 64-byte clear of its slot.  A slot belongs to a stream handle: a stream
 * created with the handle of a destroyed one must not start a forward while
 * the destroyed stream's forward still runs.
 * Kernel shapes (not part of the contract): kv heads with more than 64
 * (query row, query head) pairs run on eight-wave workgroups with 64-key
 * tiles, or on four-wave ones when that grid is small (uneven causal rows
 * covering less than two rounds of the device, or less than one round even
 * after key splits); smaller kv heads (decode) on one-wave workgroups with
 * 32-key tiles.
 */
#ifndef EA02_ATTN_H
#define EA02_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  0 is success; every other value names the first failed check
 * (the order of the checks is given with each function). */
enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NEGATIVE_SIZE = 1,  /* B, H_q, H_kv, N or D below zero              */
  ATTN_ERR_HEAD_RATIO = 2,     /* H_kv < 1 or H_q not a multiple of H_kv       */
  ATTN_ERR_HEAD_DIM = 3,       /* D not 64 or 128 (MLA: its fixed dimensions) */
  ATTN_ERR_CAUSAL_FLAG = 4,    /* is_causal is neither 0 nor 1                 */
  ATTN_ERR_SCALE = 5,          /* sm_scale is NaN or infinite                  */
  ATTN_ERR_SIZE_OVERFLOW = 6,  /* N > 2^24, N*D*2 > 2^31 (one kv head's K rows
                                  take 32-bit byte offsets), B*H_q*N >= 2^31,
                                  or a launch would pass one dispatch's 2^32
                                  work-items (with room for the spare
                                  workgroups of work stealing)                */
  ATTN_ERR_NULL_POINTER = 7,   /* a buffer pointer is NULL for non-empty work  */
  ATTN_ERR_ALIGNMENT = 8,      /* q,k,v,out not 16-byte or lse not 4-byte aligned */
  ATTN_ERR_ALIAS = 9,          /* out or lse overlaps an input or each other   */
  ATTN_ERR_LAUNCH = 10,        /* the HIP runtime rejected the kernel launch   */
  ATTN_ERR_CAUSAL_SHAPE = 11,  /* is_causal with more query rows than keys     */
  ATTN_ERR_NO_KEYS = 12,       /* N_kv = 0 while there are query rows          */
  ATTN_ERR_SPLITS = 13,        /* n_splits above the entry point's maximum   */
  ATTN_ERR_WORKSPACE = 14,     /* split workspace NULL, too small or misaligned */
  ATTN_ERR_STATIC_SCRATCH = 15 /* attn_fwd_splitkv_static: the requested splits'
                                  partials exceed the static scratch          */
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
 * Numeric range: the softmax runs in fp32 on scores in log2 units
 * (s_ij * log2 e).  The result is specified while every such scaled score
 * is below 2^31 in magnitude and the fp32 products q.k are finite; the
 * rounding error of the largest score, times the scale, is then the exponent
 * of its weight and stays representable.  Beyond that range the output is
 * unspecified (it may be NaN).  The range depends on the data, so it is not
 * checked; with sm_scale = 1/sqrt(D) it holds for any inputs whose dot
 * products stay below about 2^30.
 *
 * Ownership: the caller allocates and frees all five buffers; they must be
 * device memory of the current device.  out and lse must not overlap each
 * other or any input.
 *
 * Synchronisation: the call only enqueues work; results are visible to later
 * work on the same stream.  It never synchronises.
 *
 * Errors: the arguments are checked in the order of enum attn_status up to
 * ATTN_ERR_LAUNCH; on a failed check nothing is enqueued and nothing is written.  Empty work
 * (B, H_q or N equal to 0) returns ATTN_OK without touching any pointer.
 * No exception crosses the ABI and the library never aborts.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t D,
             float sm_scale, int is_causal, void* stream);

/*
 * attn_fwd_splitkv -- the same forward for N_q query rows against N_kv keys,
 * optionally with the key axis split into n_splits ranges that are computed
 * in parallel and merged (decode: N_q = 1).
 *
 * Method: page "Attention Kernel 实现与正确性验证", section 2.4 (FlashMLA
 * decode v2, split-T): a partial kernel per (batch, head block, key split)
 * followed by a safe-softmax merge.  For key splits K_1..K_S of the visible
 * keys, with O_s and LSE_s the attention output and log-sum-exp over K_s
 * alone,
 *   LSE = log sum_s exp(LSE_s),   out = sum_s exp(LSE_s - LSE) * O_s,
 * which is exactly attention over all visible keys.  Each O_s is stored in
 * bf16 (normalised by its own sum, so |O_s| is bounded by the largest |v|)
 * and each LSE_s in fp32; the merge sums in fp32.
 *
 * Semantics as attn_fwd, with i in [0, N_q), j in [0, N_kv), and under
 * is_causal the mask aligned to the bottom-right corner: query row i sees keys
 * j <= i + (N_kv - N_q), so the last query row sees every key (for N_q = N_kv
 * this is attn_fwd's square mask; for N_q = 1 a causal and a non-causal call
 * agree).  This alignment is a reading: the pages only treat N_q = N_kv.
 *
 * Arguments (as attn_fwd, except)
 *   q, out   [B, H_q, N_q, D];  k, v  [B, H_kv, N_kv, D];  lse  [B, H_q, N_q]
 *   n_splits 0 = the library's choice (attn_splitkv_num_splits), 1 = one pass
 *            with no workspace and no merge, 2..256 = that many key ranges
 *            (a range may be empty when it exceeds a workgroup's key tiles)
 *   workspace, workspace_size  device scratch of at least
 *            attn_splitkv_workspace_size(B, H_q, N_q, D, n_splits') bytes,
 *            16-byte aligned, where n_splits' is the split count actually used;
 *            unused (may be NULL) when that count is 1.  Its contents are
 *            undefined on entry and after the call; calls that overlap on the
 *            same workspace race.
 *
 * Ownership: the caller allocates out, lse and the workspace; the library
 * allocates nothing.  Synchronisation as attn_fwd: two kernels are enqueued
 * on `stream` when n_splits' > 1, one otherwise.
 *
 * Errors, checked in this order; nothing is enqueued on failure:
 *   NEGATIVE_SIZE (any size or n_splits < 0), HEAD_RATIO, HEAD_DIM,
 *   CAUSAL_FLAG, SCALE, SPLITS (n_splits > 256), CAUSAL_SHAPE (is_causal and
 *   N_q > N_kv), SIZE_OVERFLOW (N_q or N_kv > 2^24, N_kv * D * 2 > 2^31,
 *   B * H_q * N_q >= 2^31, N_q * H_q / H_kv > 2^30, a launch past 2^32 work-items), then empty work (B, H_q or N_q = 0) returns ATTN_OK, then
 *   NO_KEYS (N_kv = 0), NULL_POINTER, ALIGNMENT, WORKSPACE, ALIAS (out, lse
 *   or the used workspace overlapping an input or each other), LAUNCH.
 */
int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* out, float* lse,
                     int64_t B, int64_t H_q, int64_t H_kv, int64_t N_q, int64_t N_kv, int64_t D,
                     float sm_scale, int is_causal, int64_t n_splits, void* workspace,
                     size_t workspace_size, void* stream);

/*
 * attn_fwd_splitkv_static -- attn_fwd_splitkv for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The partial results of the key splits live in a
 * static device array of the library (attn_static_scratch_bytes(), 16 MiB),
 * one per GPU, held until the process ends; there is no workspace argument
 * and the call allocates nothing (no hipMalloc, no allocating library call).
 * The first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress) once.
 *
 * Semantics, arguments and check order as attn_fwd_splitkv without
 * workspace/workspace_size; n_splits 0 takes the library's split count,
 * lowered until its partials fit the scratch; an explicit n_splits whose
 * partials (attn_splitkv_workspace_size) exceed the scratch returns
 * ATTN_ERR_STATIC_SCRATCH before anything is enqueued.  Every call on one
 * GPU shares that GPU's scratch: calls that overlap in time on one GPU (other
 * streams, other host threads) race and give undefined results; calls on
 * one stream are ordered and safe.  The scratch needs no clearing: each call
 * writes every partial it reads.
 */
int attn_fwd_splitkv_static(const void* q, const void* k, const void* v, void* out, float* lse,
                            int64_t B, int64_t H_q, int64_t H_kv, int64_t N_q, int64_t N_kv, int64_t D,
                            float sm_scale, int is_causal, int64_t n_splits, void* stream);

/* Size in bytes of the static scratch attn_fwd_splitkv_static uses (per GPU). */
size_t attn_static_scratch_bytes(void);


/*
 * attn_splitkv_num_splits -- the split count attn_fwd_splitkv uses for
 * n_splits = 0 on the current device: 1 when the unsplit launch already fills
 * every workgroup slot, otherwise enough splits for about two workgroups per
 * CU (one per CU for the eight-wave shape, which fits one workgroup per CU),
 * with at least eight key tiles per split and at most 256.  The shape is
 * chosen first, from the unsplit grid.  Returns -1 when the
 * sizes fail attn_fwd_splitkv's size checks (NEGATIVE_SIZE .. SIZE_OVERFLOW).
 * Queries the current device's CU count; enqueues nothing.
 */
int64_t attn_splitkv_num_splits(int64_t B, int64_t H_q, int64_t H_kv, int64_t N_q, int64_t N_kv,
                                int64_t D, int is_causal);

/*
 * attn_splitkv_workspace_size -- bytes of workspace for n_splits key ranges:
 * 0 when n_splits <= 1, else n_splits * B * H_q * N_q * (2 * D + 4) (bf16
 * partial outputs, then fp32 partial log-sum-exps).  0 for invalid sizes.
 */
size_t attn_splitkv_workspace_size(int64_t B, int64_t H_q, int64_t N_q, int64_t D, int64_t n_splits);

/*
 * attn_bwd -- enqueue the attention backward: dq, dk, dv of the scalar
 * sum(dout * out) for the forward of attn_fwd / attn_fwd_splitkv (same head
 * map, scale, mask and bottom-right alignment for N_q < N_kv).
 *
 * Method: page "Attention Kernel 实现与正确性验证", section 1.1 (third trick:
 * the backward recomputes the attention from Q, K and the saved log-sum-exp
 * instead of storing S); page "Flash Attention 与 Kernel 优化", "Autograd 包装与
 * 反向传播" (rebuild s, mask, p, then dv, dp, ds, dq, dk).  With L = lse:
 *   P  = exp(sm_scale q k^T - L)      (masked entries 0)
 *   dv = P^T dout,  dP = dout v^T,  Dl = rowsum(dout * out),  dS = P * (dP - Dl)
 *   dq = sm_scale dS k,  dk = sm_scale dS^T q
 * dk and dv sum over the H_q / H_kv query heads of each kv head.  P and dS
 * are rounded to bf16 for the products (fp32 accumulation), as the forward
 * rounds P.
 *
 * Arguments
 *   q, out, dout  bf16 [B, H_q, N_q, D];  k, v  bf16 [B, H_kv, N_kv, D]
 *   lse           fp32 [B, H_q, N_q], natural log (the forward's output)
 *   dq            bf16 [B, H_q, N_q, D], written
 *   dk, dv        bf16 [B, H_kv, N_kv, D], written (zeros when N_q = 0)
 *   sm_scale, is_causal as for the forward that produced out and lse
 *   n_splits      0 = the library's choice (attn_bwd_num_splits), 1 = none,
 *                 2..64 = the query heads and rows a kv head's key block sees
 *                 are cut into that many contiguous ranges, one workgroup
 *                 each, whose fp32 partial dk and dv are summed in range order
 *                 by one more kernel (a range may be empty)
 *   workspace     device scratch of at least attn_bwd_workspace_size(B, H_q,
 *                 H_kv, N_q, N_kv, D, is_causal, n_splits') bytes, 16-byte
 *                 aligned, where n_splits' is the split count used (unused
 *                 when N_q = 0): per row L log2 e and Dl, then the partial
 *                 sums of the dK/dV splits, then those of the dQ kernel's
 *                 key-range splits, which the library chooses itself (by the
 *                 rule of attn_bwd_num_splits applied to the dQ kernel's pair
 *                 blocks: more than one only when they are few or unbalanced);
 *                 contents undefined on entry and after; calls that overlap
 *                 on one workspace race
 * All buffers are contiguous device memory of the current device.  Three
 * kernels are enqueued on `stream`, and one more for each of the two split
 * kinds in use; the call never synchronises.  The result is deterministic
 * (no atomics) for given split counts; different split counts round
 * differently.
 *
 * Errors, checked in this order; nothing is enqueued on failure:
 *   NEGATIVE_SIZE (any size or n_splits < 0), HEAD_RATIO, HEAD_DIM,
 *   CAUSAL_FLAG, SCALE, SPLITS (n_splits > 64), CAUSAL_SHAPE, SIZE_OVERFLOW
 *   (N_q or N_kv > 2^24, N_kv*D*2 > 2^31, N_q*(H_q/H_kv)*D*2 > 2^31,
 *   B*H_q*N_q >= 2^31, a launch past 2^32 work-items), then empty work (B or H_q = 0, or
 *   N_q = N_kv = 0) returns ATTN_OK, then NO_KEYS (N_kv = 0 < N_q),
 *   NULL_POINTER (q, out, dout, lse, dq may be NULL only when N_q = 0),
 *   ALIGNMENT (16 bytes, lse 4), WORKSPACE, ALIAS (dq, dk, dv or the workspace
 *   overlapping an input or each other), LAUNCH.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H_q, int64_t H_kv,
             int64_t N_q, int64_t N_kv, int64_t D, float sm_scale, int is_causal, int64_t n_splits,
             void* workspace, size_t workspace_size, void* stream);

/*
 * attn_bwd_num_splits -- the split count attn_bwd uses for n_splits = 0 on
 * the current device: enough ranges that the heaviest key block's share is
 * no longer than an even share of all row tiles per CU (at least 4 tiles per
 * range), at most 64 and at most 1 GiB of partial sums, kept only when a cost
 * model (about 2 us per tile saved against the partial sums' traffic at about
 * 5 TB/s and one more launch) says the split pays; 1 when the key blocks are
 * already many and balanced.  Returns -1 when the sizes fail attn_bwd's size
 * checks (NEGATIVE_SIZE .. SIZE_OVERFLOW), 1 for empty work.  Queries the
 * current device's CU count; enqueues nothing.
 */
int64_t attn_bwd_num_splits(int64_t B, int64_t H_q, int64_t H_kv, int64_t N_q, int64_t N_kv, int64_t D,
                            int is_causal);

/*
 * attn_bwd_workspace_size -- bytes of workspace attn_bwd needs with n_splits
 * dK/dV ranges on the current device: B * H_q * N_q * 8 (per-row statistics),
 * then, each region starting at a multiple of 256 bytes, n_splits * 2 * B *
 * H_kv * N_kv * D * 4 when n_splits > 1 (fp32 partial dk, then dv, per range)
 * and q_splits * B * H_q * N_q * D * 4 when the library's dQ split count
 * q_splits is above 1 (fp32 partial dq per range).  0 when the sizes fail
 * attn_bwd's size checks (NEGATIVE_SIZE .. SIZE_OVERFLOW, n_splits included)
 * and when N_q or N_kv is 0.  Queries the current device's CU count.
 */
size_t attn_bwd_workspace_size(int64_t B, int64_t H_q, int64_t H_kv, int64_t N_q, int64_t N_kv, int64_t D,
                               int is_causal, int64_t n_splits);

/*
 * Multi-head latent attention (MLA) decode, absorbed form.  Page "Attention
 * Kernel 实现与正确性验证", section 2: with the key up-projection W_uk folded
 * into the query (2.1), every head scores against the same latent cache row
 * kv = [c_kv (512), k_pe (64)] and takes c_kv as its values; the value
 * up-projection W_uv is applied to the latent output (2.2).  Shapes are the
 * DeepSeek-V3 ones of 2.3 (d_c = 512, d_R = 64); the cache axis may be split
 * with a safe-softmax merge as in 2.4.  Three steps, three entry points:
 *
 *   mla_absorb_q:    q_lat[b,h,s] = [q_nope[b,h,s] W_uk[h], q_pe[b,h,s]]
 *   attn_mla_decode: out_lat[b,h,s] = softmax_j(sm_scale q_lat[b,h,s] . kv[b,j]) c_kv[b,j]
 *                    lse[b,h,s] = log sum_j exp(sm_scale q_lat[b,h,s] . kv[b,j])
 *   mla_up_project:  out[b,h,s] = out_lat[b,h,s] W_uv[h]^T
 *
 * For S > 1 query tokens, is_causal masks bottom-right: token s sees cache
 * positions j <= s + T - S.  The page scales scores by 1/sqrt(d_nope + d_R).
 * All tensors are contiguous bf16 device memory (lse fp32), row-major with
 * the last dimension fastest; products accumulate in fp32 and round to bf16
 * (nearest even) when stored.
 */

/*
 * attn_mla_decode -- the latent attention core.
 *   q_lat   [B, H, S, d_c + d_r]   kv   [B, T, d_c + d_r]
 *   out_lat [B, H, S, d_c] (written)   lse  [B, H, S] fp32 (written)
 *   d_c must be 512 and d_r 64.  n_splits, workspace: as attn_fwd_splitkv
 *   (0 = attn_mla_num_splits, 1 = one pass without workspace, at most 256;
 *   workspace of attn_mla_workspace_size bytes, 16-byte aligned).
 * Errors, in this order: NEGATIVE_SIZE, HEAD_DIM (d_c, d_r), CAUSAL_FLAG,
 * SPLITS, CAUSAL_SHAPE (S > T), SIZE_OVERFLOW (T * 1152 > 2^31, B*H*S >=
 * 2^31, ...), SCALE, then empty work (B, H or S = 0) returns ATTN_OK, then
 * NO_KEYS (T = 0), NULL_POINTER, ALIGNMENT (16 bytes, lse 4), WORKSPACE,
 * ALIAS, LAUNCH.  Two kernels are enqueued when the split count is above 1.
 */
int attn_mla_decode(const void* q_lat, const void* kv, void* out_lat, float* lse, int64_t B,
                    int64_t H, int64_t S, int64_t T, int64_t d_c, int64_t d_r, float sm_scale,
                    int is_causal, int64_t n_splits, void* workspace, size_t workspace_size,
                    void* stream);

/* Split count attn_mla_decode picks for n_splits = 0 on the current device
 * (1 when the unsplit grid has a workgroup per CU; else about one per CU,
 * at least four 32-key tiles per split); -1 for sizes it would reject. */
int64_t attn_mla_num_splits(int64_t B, int64_t H, int64_t S, int64_t T, int is_causal);

/* Workspace bytes of attn_mla_decode: 0 when n_splits <= 1, else
 * n_splits * B * H * S * (2 * 512 + 4) (bf16 partial outputs, then fp32
 * partial log-sum-exps).  0 for invalid sizes. */
size_t attn_mla_workspace_size(int64_t B, int64_t H, int64_t S, int64_t n_splits);

/*
 * mla_absorb_q -- q_lat = [q_nope W_uk[h], q_pe] per head.
 *   q_nope [B, H, S, d_nope] (1 <= d_nope <= 256), q_pe [B, H, S, d_r],
 *   w_uk [H, d_nope, d_c], q_lat [B, H, S, d_c + d_r] (written); d_c = 512,
 *   d_r = 64.  Errors: NEGATIVE_SIZE, HEAD_DIM, SIZE_OVERFLOW, empty work ->
 *   ATTN_OK, NULL_POINTER, ALIGNMENT (q_nope 2 bytes, others 16), ALIAS, LAUNCH.
 */
int mla_absorb_q(const void* q_nope, const void* q_pe, const void* w_uk, void* q_lat, int64_t B,
                 int64_t H, int64_t S, int64_t d_nope, int64_t d_c, int64_t d_r, void* stream);

/*
 * mla_up_project -- out = out_lat W_uv[h]^T per head.
 *   out_lat [B, H, S, d_c], w_uv [H, d_v, d_c], out [B, H, S, d_v] (written);
 *   d_c = 512, d_v a multiple of 32 in [32, 1024].  Errors: NEGATIVE_SIZE,
 *   HEAD_DIM, SIZE_OVERFLOW, empty work -> ATTN_OK, NULL_POINTER, ALIGNMENT
 *   (out_lat and w_uv 16 bytes, out 2), ALIAS, LAUNCH.
 */
int mla_up_project(const void* out_lat, const void* w_uv, void* out, int64_t B, int64_t H,
                   int64_t S, int64_t d_c, int64_t d_v, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* attn_status_string(int status);

/* Library ABI version, currently 8 (1: attn_fwd; 2: + split-KV; 3: + backward;
 * 4: + MLA decode; 5: backward row-range splits, attn_bwd_num_splits; 6:
 * backward dQ key-range splits, is_causal in attn_bwd_workspace_size; 7: +
 * attn_fwd_splitkv_static; 8: bf16 split partial outputs, smaller
 * attn_splitkv_workspace_size and attn_mla_workspace_size). */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EA02_ATTN_H */
