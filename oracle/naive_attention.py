"""CPU float64 oracle for the fused attention forward: naive, materialised attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only the test suite, the smoke check in the repository's entry module and the
CPU-baseline leg of the benchmark may import or call it.  It shares no code,
table or helper with the HIP library.

What it computes is the plain definition that the fused kernel must reproduce
up to rounding.  Flash attention is block-wise but equivalent to the softmax
over the whole key sequence (page "Attention Kernel 实现与正确性验证", section
1.1, the online-softmax trick; page "Flash Attention 与 Kernel 优化", section
"为什么需要 Flash Attention": what matters is that the softmax normalisation
stays correct).  So the oracle materialises the score rows, applies the causal
mask, takes the ordinary softmax and multiplies by V, in float64.

For one batch element b and query head h, with kv head g:

    g         = floor(h * H_kv / H_q)                         (GQA head map)
    S[i, j]   = sm_scale * sum_d Q[b,h,i,d] * K[b,g,j,d]
    S[i, j]   = -inf      where causal and j > i              (top-left causal)
    m_i       = max_j S[i, j]
    l_i       = sum_j exp(S[i, j] - m_i)
    O[b,h,i]  = sum_j exp(S[i, j] - m_i) * V[b,g,j] / l_i
    LSE[b,h,i]= m_i + ln(l_i)

Sources:
  * head map, scale, causal mask, the softmax statistics m, l and the final
    division by l: page "Attention Kernel 实现与正确性验证", section 1.2
    (Forward kernel, GQA-aware); page "Triton Cuda Attention", sections
    "在线 Softmax 核心算法" and "变体改法" (Causal, GQA: integer division, not
    modulo, groups query heads onto kv heads; H_q is an integer multiple of H_kv).
  * LSE = m + log(l): page "Flash Attention 与 Kernel 优化", section
    "输出与保存状态" (the l buffer keeps each row's log-sum-exp).
  * order: scale first, then mask (section 1.2 of the first page).

Readings where the pages are silent or disagree (each also listed in the
design notes):
  * LSE is in natural-log units of the scaled scores; the eps the third page
    adds inside log() is taken as 0 (every row sees at least one key, l >= 1).
  * causal alignment is square and top-left: row i sees keys 0..i.  With
    fewer query rows than keys (a KV-cache prefill or a decode step) the
    mask is bottom-right aligned: query row i sits at key position
    i + N_kv - N_q, the reading that reduces to the square case.
  * Q, K, V are the bf16 values the GPU receives, upcast exactly to float64
    by the caller; the oracle itself only ever sees float64 arrays.

Implementation shape: rows of one (b, h) are taken in blocks of at most
ROW_BLOCK, each block materialising its full score rows.  Under the causal
mask the keys after a block's last row carry weight exp(-inf) = 0 exactly, so
they are left out of that block's product; no other blocking, fusion or
reordering is done.
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 512


def kv_head(h: int, H_q: int, H_kv: int) -> int:
    """KV head serving query head h (grouped-query map by integer division)."""
    return (h * H_kv) // H_q


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("expected [B,H,N,D] arrays")
    B, H_q, N_q, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("K and V must be [B,H_kv,N_kv,D] matching Q")
    H_kv, N_kv = k.shape[1], k.shape[2]
    if H_kv < 1 or H_q % H_kv != 0:
        raise ValueError("H_q must be an integer multiple of H_kv")
    return B, H_q, H_kv, N_q, N_kv, D


def attention_rows(q, k, v, b: int, h: int, rows, *, is_causal: bool, sm_scale: float):
    """O and LSE of the given query rows of (b, h), in float64.

    q: [B,H_q,N_q,D], k, v: [B,H_kv,N_kv,D] float64 arrays; rows: 1-D integer
    array of query rows.  Returns (O [len(rows), D], LSE [len(rows)]).
    Causal masking is bottom-right aligned when N_q < N_kv (query row i sits
    at key position i + N_kv - N_q); for N_q == N_kv this is the square,
    top-left mask of the pages.
    """
    B, H_q, H_kv, N_q, N_kv, D = _check(q, k, v)
    if is_causal and N_q > N_kv:
        raise ValueError("causal attention needs N_q <= N_kv")
    off = N_kv - N_q if is_causal else 0
    rows = np.asarray(rows, dtype=np.int64)
    g = kv_head(h, H_q, H_kv)
    out = np.empty((rows.size, D), dtype=np.float64)
    lse = np.empty((rows.size,), dtype=np.float64)
    for s in range(0, rows.size, ROW_BLOCK):
        r = rows[s:s + ROW_BLOCK]
        # keys a causal row can see end at its own position; later keys weigh 0
        nk = int(r.max()) + off + 1 if is_causal else N_kv
        Kg = k[b, g, :nk, :]
        Vg = v[b, g, :nk, :]
        S = sm_scale * (q[b, h, r, :] @ Kg.T)              # [R, nk]
        if is_causal:
            j = np.arange(nk)[None, :]
            S = np.where(j > r[:, None] + off, -np.inf, S)
        m = S.max(axis=1)                                 # row max
        E = np.exp(S - m[:, None])                        # exp(-inf) = 0
        l = E.sum(axis=1)                                 # row sum
        out[s:s + ROW_BLOCK] = (E @ Vg) / l[:, None]
        lse[s:s + ROW_BLOCK] = m + np.log(l)
    return out, lse


def attention_forward(q, k, v, *, is_causal: bool, sm_scale: float):
    """Full O [B,H_q,N_q,D] and LSE [B,H_q,N_q] in float64 (definition above)."""
    B, H_q, H_kv, N_q, N_kv, D = _check(q, k, v)
    O = np.empty((B, H_q, N_q, D), dtype=np.float64)
    L = np.empty((B, H_q, N_q), dtype=np.float64)
    rows = np.arange(N_q, dtype=np.int64)
    for b in range(B):
        for h in range(H_q):
            O[b, h], L[b, h] = attention_rows(q, k, v, b, h, rows,
                                              is_causal=is_causal, sm_scale=sm_scale)
    return O, L


def merge_partials(o_parts, lse_parts):
    """Combine attention results over disjoint key subsets.

    The split-T pattern of page "Attention Kernel 实现与正确性验证", section
    2.4 (v2: a partial kernel per key split, then a safe-softmax merge): with
    o_parts [S, ..., D] the normalised outputs and lse_parts [S, ...] the
    log-sum-exps of the S splits,
        LSE = log sum_s exp(lse_s)          (taken relative to max_s lse_s)
        O   = sum_s exp(lse_s - LSE) * o_s
    A split that saw no key has lse = -inf and weight 0.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    w = np.exp(lse_parts - m[None])
    tot = w.sum(axis=0)
    lse = m + np.log(tot)
    out = (w[..., None] * o_parts).sum(axis=0) / tot[..., None]
    return out, lse
