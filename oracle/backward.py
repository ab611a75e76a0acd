"""Gradients of exact attention in fp64 -- TEST INFRASTRUCTURE (see the package doc).

What the pages say about the backward pass. The forward keeps only Q, K, V and the softmax
statistics, and the backward recomputes the attention matrix from them instead of storing
it. The pages give the trade as about 30% more compute for about 90% less memory:
  * "FlashAttention算法原理与性能优化实战" (intelliparadigm), section 1.2.3, recomputation;
  * "Flash Attention是怎么做到又快又省显存的？" (cnblogs), 总结: recomputation as a
    tiling-based form of gradient checkpointing;
  * the Triton FA2 walkthrough: the forward's logsumexp L exists for the backward pass, whose
    benchmark it shows at B=4, H=48, d=64, causal.
The pages print no gradient formulas. The gradients of O = softmax(s*Q K^T [+ causal
mask]) V with respect to Q, K and V are plain calculus. Here they are written out for one
(batch, head) in fp64 on the exactly upcast inputs, with dO the gradient arriving at O:
  S   = s * Q K^T, hidden entries -inf (causal: key j visible to query i iff j <= i)
  P   = exp(S - LSE)            recomputed from the forward's saved LSE (the pages' point)
  dV  = P^T dO
  dP  = dO V^T
  D_i = sum_j P_ij dP_ij        (equal to sum_c dO_ic O_ic, the form the GPU path uses)
  dS  = P o (dP - D)            (o: elementwise; the softmax Jacobian applied row by row)
  dQ  = s * dS K ;  dK = s * dS^T Q
Grouped-query attention (intelliparadigm page, section 1.3): query head hq reads K/V head
floor(hq / G). A K/V head's gradients are therefore the sums over the G query heads that
read it.

The formula is pinned by tests that do not retype it. Central finite differences of the
forward definition (and of its pure-Python brute force) check it, and so do torch's float64
autograd through scaled_dot_product_attention and the invariants sum_j dK_j = 0 and
sum_j dV_j = sum_i dO_i.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .attention import band_visible, head_attention_band_fp64, head_attention_fp64, kv_head_of, mask_of_head

ROW_BLOCK = 1024  # query rows per block (bounds memory only)


def head_attention_bwd_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                            scale: float, causal: bool, lse: Optional[np.ndarray] = None
                            ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of one (batch, head): q, do [n,d] at rows 0..n-1; k, v [N,d].

    Returns (dQ [n,d], dK [N,d], dV [N,d]) in float64. ``lse`` is the forward's natural-log
    LSE of each row; it is recomputed from the definition when not given.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n, N = q.shape[0], k.shape[0]
    if lse is None:
        _, lse = head_attention_fp64(q, k, v, scale, causal)
    lse = np.asarray(lse, dtype=np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        kend = N if not causal else min(N, r1)
        S = scale * (q[r0:r1] @ k[:kend].T)
        if causal:
            hidden = np.arange(kend)[None, :] > np.arange(r0, r1)[:, None]
            S = np.where(hidden, -np.inf, S)
        P = np.exp(S - lse[r0:r1, None])            # recomputed probabilities
        dv[:kend] += P.T @ do[r0:r1]
        dP = do[r0:r1] @ v[:kend].T
        D = np.sum(P * dP, axis=1)
        dS = P * (dP - D[:, None])
        dq[r0:r1] = scale * (dS @ k[:kend])
        dk[:kend] += scale * (dS.T @ q[r0:r1])
    return dq, dk, dv


def attention_bwd_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                       causal: bool) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients over [B,Hq,N,d] queries and [B,Hkv,N,d] keys/values (float64).

    Returns (dQ [B,Hq,N,d], dK [B,Hkv,N,d], dV [B,Hkv,N,d]).
    """
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            hk = kv_head_of(hq, Hq, Hkv)
            g_q, g_k, g_v = head_attention_bwd_fp64(q[b, hq], k[b, hk], v[b, hk], do[b, hq], scale, causal)
            dq[b, hq] = g_q
            dk[b, hk] += g_k
            dv[b, hk] += g_v
    return dq, dk, dv


def head_attention_bwd_bound_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                                  o_used: np.ndarray, scale: float, causal: bool, u: float,
                                  e32: float = 2.0 ** -24, band: Optional[Tuple] = None,
                                  hidden: Optional[np.ndarray] = None
                                  ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """First-order elementwise error bounds (Bq [n,d], Bk [N,d], Bv [N,d]) for one head's
    gradients computed the way a tiled kernel does: S, dP and D accumulated in fp32 (unit
    roundoff ``e32``), D formed from ``o_used`` (the O it is given, e.g. stored in fp32 or in
    16 bits), P = exp(S - LSE) in fp32, P and dS rounded to a 16-bit type of unit roundoff ``u``
    before the products that consume them, and those products accumulated in fp32. The test
    suite sizes its parity bar from these; they are not part of the result.

    With d the head dimension, n the rows and N the keys, per element:
      rho_ij = d e32 s (|Q||K|^T)_ij + 4 e32              relative error of P (S, fma, exp)
      eta_ij = d e32 ((|dO||V|^T)_ij + sum_c |dO_ic O_ic|) + |sum_c dO_ic (O_used - O)_ic|
                                                           absolute error of dP - D
      Bv = sum_i (u + rho_ij + n e32) P_ij |dO_ic|
      Bq = s sum_j [(u + rho_ij + N e32) |dS_ij| + P_ij eta_ij] |K_jc|
      Bk = s sum_i [(u + rho_ij + n e32) |dS_ij| + P_ij eta_ij] |Q_ic|
    (a product sum_k a_k b_k whose factor a_k carries a relative error e moves by at most
    e sum_k |a_k b_k|; an fp32 sum of m terms by at most m e32 times the sum of magnitudes).
    ``band`` = (left, right, off) replaces ``causal`` by the band of ``attention.band_visible``,
    and ``hidden`` [n, N] (with a band) hides further keys where nonzero.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    o_used = np.asarray(o_used, dtype=np.float64)
    n, N = q.shape[0], k.shape[0]
    d = q.shape[1]
    if band is None:
        O, lse = head_attention_fp64(q, k, v, scale, causal)
    else:
        O, lse = head_attention_band_fp64(q, k, v, scale, *band, hidden=hidden)
    d_dev = np.abs(np.sum(do * (o_used - O), axis=1))
    d_mag = np.sum(np.abs(do * O), axis=1)
    bq = np.zeros(q.shape)
    bk = np.zeros(k.shape)
    bv = np.zeros(v.shape)
    g_d = d * e32
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        kend = N if (band is not None or not causal) else min(N, r1)
        S = scale * (q[r0:r1] @ k[:kend].T)
        if band is not None:
            vis = band_visible(np.arange(r0, r1), np.arange(kend), band[0], band[1], band[2])
            if hidden is not None:
                vis &= ~np.asarray(hidden[r0:r1, :kend], dtype=bool)
            seen = np.isfinite(lse[r0:r1])
            P = np.where(vis & seen[:, None],
                         np.exp(np.where(vis, S, 0.0) - np.where(seen, lse[r0:r1], 0.0)[:, None]), 0.0)
        else:
            if causal:
                hidden = np.arange(kend)[None, :] > np.arange(r0, r1)[:, None]
                S = np.where(hidden, -np.inf, S)
            P = np.exp(S - lse[r0:r1, None])
        dP = do[r0:r1] @ v[:kend].T
        D = np.sum(P * dP, axis=1)
        dS = np.abs(P * (dP - D[:, None]))
        rho = g_d * scale * (np.abs(q[r0:r1]) @ np.abs(k[:kend]).T) + 4 * e32
        eta = g_d * (np.abs(do[r0:r1]) @ np.abs(v[:kend]).T + d_mag[r0:r1, None]) + d_dev[r0:r1, None]
        bv[:kend] += ((u + rho + n * e32) * P).T @ np.abs(do[r0:r1])
        bq[r0:r1] = scale * (((u + rho + N * e32) * dS + P * eta) @ np.abs(k[:kend]))
        bk[:kend] += scale * (((u + rho + n * e32) * dS + P * eta).T @ np.abs(q[r0:r1]))
    return bq, bk, bv



def head_attention_bwd_band_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                                 left: Optional[int], right: Optional[int], off: int = 0,
                                 hidden: Optional[np.ndarray] = None
                                 ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of one head under the band of ``attention.band_visible`` and the optional
    ``hidden`` [n, N] mask (the same chain rule as ``head_attention_bwd_fp64``; hidden entries
    and rows that see no key have P = 0)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n, N = q.shape[0], k.shape[0]
    _, lse = head_attention_band_fp64(q, k, v, scale, left, right, off, hidden=hidden)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        vis = band_visible(np.arange(r0, r1), np.arange(N), left, right, off)
        if hidden is not None:
            vis &= ~np.asarray(hidden[r0:r1], dtype=bool)
        seen = np.isfinite(lse[r0:r1])
        S = scale * (q[r0:r1] @ k.T)
        P = np.where(vis & seen[:, None], np.exp(np.where(vis, S, 0.0) - np.where(seen, lse[r0:r1], 0.0)[:, None]), 0.0)
        dv += P.T @ do[r0:r1]
        dP = do[r0:r1] @ v.T
        D = np.sum(P * dP, axis=1)
        dS = P * (dP - D[:, None])
        dq[r0:r1] = scale * (dS @ k)
        dk += scale * (dS.T @ q[r0:r1])
    return dq, dk, dv


def attention_bwd_band_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                            left: Optional[int], right: Optional[int], mask: Optional[np.ndarray] = None
                            ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Banded gradients over [B,Hq,Nq,d] queries and [B,Hkv,Nk,d] keys/values, off = Nk - Nq,
    with the optional [Bm,Hm,Nq,Nk] mask of ``attention.attention_band_fp64``."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            hk = kv_head_of(hq, Hq, Hkv)
            g_q, g_k, g_v = head_attention_bwd_band_fp64(q[b, hq], k[b, hk], v[b, hk], do[b, hq], scale, left, right,
                                                         off=Nk - Nq, hidden=mask_of_head(mask, b, hq))
            dq[b, hq] = g_q
            dk[b, hk] += g_k
            dv[b, hk] += g_v
    return dq, dk, dv
