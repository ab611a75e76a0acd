"""Exact attention in fp64: the definition, and the pages' tiled forms.

Test infrastructure only (see the package doc).

The definition (``head_attention_fp64``) follows the standard
scaled-dot-product attention the pages start from:
  * "PyTorch Transformer Flash Attention机制：内存访问优化与CUDA Kernel融合的底层实现"
    (zyxy.net), section 1: weights = softmax(Q K^T / sqrt(D)), output =
    weights V, tensors laid out (B, H, L, D);
  * "FlashAttention算法原理与性能优化实战" (intelliparadigm), section 1.1: S, P, O;
  * the Triton FA2 walkthrough: the softmax used is the safe one.
Per query row i of head (b, hq), in fp64 on the exactly upcast inputs:
  S_ij = s * sum_c Q[i,c] K[j,c]   (s = the float32 scale the kernel receives)
  visible keys: all j, or j <= i when causal
  m_i = max_j S_ij;  l_i = sum_j e^{S_ij - m_i};  P_ij = e^{S_ij - m_i} / l_i
  O[i,:] = sum_j P_ij V[j,:];  LSE_i = m_i + ln l_i
Grouped-query attention (intelliparadigm page, section 1.3, "MQA/GQA"): query
head hq reads K/V head floor(hq / G), G = Hq / Hkv (consecutive grouping; the
page gives no mapping, this is the reading taken).

The tiled forms exist only to pin the definition against the pages'
algorithms (they must agree with it to rounding):
  * ``tiled_kv_outer_normalised``: K/V blocks outer, Q blocks inner, the
    output kept normalised after every block (intelliparadigm page, sections
    1.2.1 and 1.2.2). The printed update multiplies the block's exponentials
    by its correction factor after already shifting them by the new maximum,
    which corrects twice; the reading taken shifts by the block's own maximum
    and then applies the correction once.
  * ``tiled_q_outer_deferred``: Q blocks outer, K/V blocks inner, unnormalised
    accumulator rescaled by e^{m_old - m_new} and divided by l once at the end
    (the Triton FA2 walkthrough: loop swap and fewer non-matmul operations).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


ROW_BLOCK = 1024  # query rows per block in the definition (bounds memory only)


def kv_head_of(hq: int, Hq: int, Hkv: int) -> int:
    """K/V head read by query head ``hq``: consecutive groups of G = Hq/Hkv."""
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return hq // (Hq // Hkv)


def _scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    return scale * (q @ k.T)


def _mask_causal(S: np.ndarray, q_pos: np.ndarray, k_pos: np.ndarray) -> np.ndarray:
    """Set S_ij = -inf where key j is after query i (causal: j visible iff j <= i)."""
    hidden = k_pos[None, :] > q_pos[:, None]
    return np.where(hidden, -np.inf, S)


def head_attention_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                        causal: bool, q_pos: Optional[np.ndarray] = None
                        ) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of one (batch, head): q [n,d] (rows at positions ``q_pos``), k, v [N,d].

    Returns (O [n,d], LSE [n]) in float64. ``q_pos`` defaults to 0..n-1; it
    lets a caller evaluate sampled rows of a long sequence one by one.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    if q_pos is None:
        q_pos = np.arange(n)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    O = np.empty((n, v.shape[1]), dtype=np.float64)
    LSE = np.empty((n,), dtype=np.float64)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        pos = q_pos[r0:r1]
        kend = k.shape[0] if not causal else min(k.shape[0], int(pos.max()) + 1)
        S = _scores(q[r0:r1], k[:kend], scale)
        if causal:
            S = _mask_causal(S, pos, np.arange(kend))
        m = np.max(S, axis=1)                      # pass 1: row maximum
        e = np.exp(S - m[:, None])
        l = np.sum(e, axis=1)                      # pass 2: shifted denominator
        P = e / l[:, None]                         # pass 3: probabilities
        O[r0:r1] = P @ v[:kend]
        LSE[r0:r1] = m + np.log(l)
    return O, LSE


def attention_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   causal: bool) -> Tuple[np.ndarray, np.ndarray]:
    """Attention over [B,Hq,N,d] queries and [B,Hkv,N,d] keys/values (float64).

    Returns (O [B,Hq,N,d], LSE [B,Hq,N]).
    """
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    O = np.empty(q.shape, dtype=np.float64)
    LSE = np.empty((B, Hq, N), dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            hk = kv_head_of(hq, Hq, Hkv)
            O[b, hq], LSE[b, hq] = head_attention_fp64(q[b, hq], k[b, hk], v[b, hk], scale, causal)
    return O, LSE


def tiled_kv_outer_normalised(q, k, v, scale: float, causal: bool, block_q: int, block_kv: int):
    """K/V-outer tiling with a normalised output after every block (one head).

    State per query row: running max m (init -inf), denominator l (init 0),
    output O (init 0). For key block j and query block i:
      m_blk = rowmax S_ij,  Pt = e^{S_ij - m_blk},  l_blk = rowsum Pt
      m_new = max(m, m_blk),  l_new = e^{m - m_new} l + e^{m_blk - m_new} l_blk
      O = (l e^{m - m_new} O + e^{m_blk - m_new} Pt V_j) / l_new
    Returns (O, LSE = m + ln l).
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    n, N = q.shape[0], k.shape[0]
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    O = np.zeros((n, v.shape[1]))
    with np.errstate(invalid="ignore"):
        for j0 in range(0, N, block_kv):
            j1 = min(N, j0 + block_kv)
            for i0 in range(0, n, block_q):
                i1 = min(n, i0 + block_q)
                S = _scores(q[i0:i1], k[j0:j1], scale)
                if causal:
                    S = _mask_causal(S, np.arange(i0, i1), np.arange(j0, j1))
                m_blk = np.max(S, axis=1)
                seen = np.isfinite(m_blk)  # rows with at least one visible key in this block
                if not seen.any():
                    continue
                rows = np.arange(i0, i1)[seen]
                S, m_blk = S[seen], m_blk[seen]
                Pt = np.exp(S - m_blk[:, None])
                l_blk = np.sum(Pt, axis=1)
                m_old, l_old = m[rows], l[rows]
                m_new = np.maximum(m_old, m_blk)
                c_old = np.exp(m_old - m_new)  # e^{-inf} = 0 for rows not seen before
                c_blk = np.exp(m_blk - m_new)
                l_new = c_old * l_old + c_blk * l_blk
                O[rows] = ((l_old * c_old)[:, None] * O[rows] + c_blk[:, None] * (Pt @ v[j0:j1])) / l_new[:, None]
                m[rows], l[rows] = m_new, l_new
    return O, m + np.log(l)


def tiled_q_outer_deferred(q, k, v, scale: float, causal: bool, block_q: int, block_kv: int):
    """Q-outer tiling with the normalisation deferred to the end (one head).

    For each query block: m = -inf, l = 0, acc = 0; for each key block that
    holds a visible key: m_new = max(m, rowmax S), Pt = e^{S - m_new},
    alpha = e^{m - m_new}, l = alpha l + rowsum Pt, acc = alpha acc + Pt V;
    finally O = acc / l and LSE = m + ln l.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    n, N = q.shape[0], k.shape[0]
    O = np.empty((n, v.shape[1]))
    LSE = np.empty(n)
    for i0 in range(0, n, block_q):
        i1 = min(n, i0 + block_q)
        m = np.full(i1 - i0, -np.inf)
        l = np.zeros(i1 - i0)
        acc = np.zeros((i1 - i0, v.shape[1]))
        jend = N if not causal else min(N, i1)  # blocks past the last visible key are skipped
        for j0 in range(0, jend, block_kv):
            j1 = min(N, j0 + block_kv)
            S = _scores(q[i0:i1], k[j0:j1], scale)
            if causal:
                S = _mask_causal(S, np.arange(i0, i1), np.arange(j0, j1))
            # Key 0 is visible to every row, so m_new is finite from the first block on even
            # when a row sees no key of a later block.
            m_new = np.maximum(m, np.max(S, axis=1))
            Pt = np.exp(S - m_new[:, None])
            alpha = np.exp(m - m_new)
            l = alpha * l + np.sum(Pt, axis=1)
            acc = alpha[:, None] * acc + Pt @ v[j0:j1]
            m = m_new
        O[i0:i1] = acc / l[:, None]
        LSE[i0:i1] = m + np.log(l)
    return O, LSE


def band_visible(q_pos: np.ndarray, k_pos: np.ndarray, left: Optional[int], right: Optional[int],
                 off: int) -> np.ndarray:
    """visible[i, j]: whether key ``k_pos[j]`` is visible to the query at ``q_pos[i]``.

    The Ascend operator on the intelliparadigm page (section 2.2) bounds a sliding window
    with pre_tokens (left edge) and next_tokens (right edge), both unlimited by default; its
    tiling (section 2.3) takes separate query and key lengths. The reading taken: the query
    at row i sits at key position i + off with off = Nk - Nq (its diagonal aligned to the end
    of the key sequence), and sees key j iff i + off - left <= j <= i + off + right, an
    unlimited edge (None) imposing nothing. Causal attention with Nq = Nk is left = None,
    right = 0.
    """
    rel = np.asarray(k_pos, np.int64)[None, :] - (np.asarray(q_pos, np.int64)[:, None] + off)
    vis = np.ones(rel.shape, dtype=bool)
    if left is not None:
        vis &= rel >= -left
    if right is not None:
        vis &= rel <= right
    return vis


def head_attention_band_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                             left: Optional[int], right: Optional[int], off: int = 0,
                             q_pos: Optional[np.ndarray] = None,
                             hidden: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of one (batch, head) under the band of ``band_visible``.

    Same definition as ``head_attention_fp64`` over each row's visible keys. A row that sees
    no key has an empty softmax; the reading taken is O = 0 and LSE = -inf (the log of an
    empty sum). ``hidden`` [n, N] (rows as given in q), when present, hides key j from row i
    wherever it is nonzero, on top of the band: the boolean attn_mask input of the Ascend
    operator (intelliparadigm page, section 2.2), the Mask step of FlashAttention-1's
    Algorithm 2 that the cnblogs page points to.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, N = q.shape[0], k.shape[0]
    if q_pos is None:
        q_pos = np.arange(n)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    O = np.zeros((n, v.shape[1]), dtype=np.float64)
    LSE = np.full((n,), -np.inf, dtype=np.float64)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        vis = band_visible(q_pos[r0:r1], np.arange(N), left, right, off)
        if hidden is not None:
            vis &= ~np.asarray(hidden[r0:r1], dtype=bool)
        S = np.where(vis, _scores(q[r0:r1], k, scale), -np.inf)
        seen = vis.any(axis=1)
        if not seen.any():
            continue
        S = S[seen]
        m = np.max(S, axis=1)
        e = np.exp(S - m[:, None])
        l = np.sum(e, axis=1)
        rows = np.arange(r0, r1)[seen]
        O[rows] = (e / l[:, None]) @ v
        LSE[rows] = m + np.log(l)
    return O, LSE


def mask_of_head(mask: Optional[np.ndarray], b: int, hq: int) -> Optional[np.ndarray]:
    """The [Nq, Nk] slice of a [Bm, Hm, Nq, Nk] mask for (b, hq); a size-1 batch or head axis
    is shared by every batch element or head."""
    if mask is None:
        return None
    return mask[b if mask.shape[0] > 1 else 0, hq if mask.shape[1] > 1 else 0]


def attention_band_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                        left: Optional[int], right: Optional[int],
                        mask: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Banded attention over [B,Hq,Nq,d] queries and [B,Hkv,Nk,d] keys/values (float64),
    with the diagonal offset off = Nk - Nq, and optionally a [Bm,Hm,Nq,Nk] mask (Bm in {1, B},
    Hm in {1, Hq}) whose nonzero entries hide keys. Returns (O [B,Hq,Nq,d], LSE [B,Hq,Nq])."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    O = np.empty(q.shape, dtype=np.float64)
    LSE = np.empty((B, Hq, Nq), dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            hk = kv_head_of(hq, Hq, Hkv)
            O[b, hq], LSE[b, hq] = head_attention_band_fp64(q[b, hq], k[b, hk], v[b, hk], scale, left, right,
                                                            off=Nk - Nq, hidden=mask_of_head(mask, b, hq))
    return O, LSE
