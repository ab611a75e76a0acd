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
from .additive import head_attention_additive_fp64
from .dropout import head_attention_dropout_fp64, keep_threshold

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


def head_attention_bwd_magnitude_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                                      scale: float, causal: bool, band: Optional[Tuple] = None,
                                      hidden: Optional[np.ndarray] = None, drop: Optional[Tuple] = None,
                                      add: Optional[np.ndarray] = None
                                      ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Magnitude sums (Mq [n,d], Mk [N,d], Mv [N,d]) of one head's gradients: each gradient
    element written out as a sum of products of the inputs (Q, K, V, dO), the probabilities P
    and the output O, with every term replaced by its magnitude. With A_ij = sum_c |dO_ic||V_jc|
    (the terms of dP_ij) and E_i = sum_c |dO_ic O_ic| (the terms of D_i):
      dV_jc = sum_i P_ij dO_ic                        Mv_jc = sum_i P_ij |dO_ic|
      dQ_ic = s sum_j P_ij (dP_ij - D_i) K_jc         Mq_ic = s sum_j P_ij (A_ij + E_i) |K_jc|
      dK_jc = s sum_i P_ij (dP_ij - D_i) Q_ic         Mk_jc = s sum_i P_ij (A_ij + E_i) |Q_ic|
    (P >= 0, so |P| = P.) These sums measure how far roundings of relative size u inside any
    evaluation of the chain rule can move each element: to first order by at most u per rounding
    a term passes through, times M. They depend on the problem only, not on how an
    implementation orders or tiles the sums. The test suite sizes its GPU bar from them; they are
    not part of the result. ``band`` = (left, right, off) replaces ``causal`` by the band of
    ``attention.band_visible``, and ``hidden`` [n, N] (with a band) hides further keys where
    nonzero; hidden keys and rows that see no key have P = 0.
    ``drop`` = (Z, keep_prob), with a band, is the dropout of dropout.py with the keep mask Z
    [n, N] held fixed: the terms that pass through dV or dP carry Z_ij / keep (dV_jc =
    sum_i (Z_ij / keep) P_ij dO_ic, dP_ij = (Z_ij / keep) sum_c dO_ic V_jc), so Mv and A take that
    factor, and E uses the dropped output O. ``add`` [n, N], with a band, is the additive mask
    of additive.py: P and O come from the masked scores (the terms are otherwise the same).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, N = q.shape[0], k.shape[0]
    if add is not None:
        if band is None or hidden is not None or drop is not None:
            raise ValueError("additive-mask magnitudes take a band and nothing else")
        O, lse = head_attention_additive_fp64(q, k, v, scale, band[0], band[1], band[2], add)
    elif drop is not None:
        if band is None or hidden is not None:
            raise ValueError("dropout magnitudes take a band and no hidden keys")
        O, lse = head_attention_dropout_fp64(q, k, v, scale, band[0], band[1], band[2], drop[0], drop[1])
        zk = np.asarray(drop[0], dtype=np.float64) * (256.0 / keep_threshold(drop[1]))
    elif band is None:
        O, lse = head_attention_fp64(q, k, v, scale, causal)
    else:
        O, lse = head_attention_band_fp64(q, k, v, scale, *band, hidden=hidden)
    E = np.sum(np.abs(do * O), axis=1)
    mq = np.zeros(q.shape)
    mk = np.zeros(k.shape)
    mv = np.zeros(v.shape)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        kend = N if (band is not None or not causal) else min(N, r1)
        S = scale * (q[r0:r1] @ k[:kend].T)
        if band is not None:
            vis = band_visible(np.arange(r0, r1), np.arange(kend), band[0], band[1], band[2])
            if hidden is not None:
                vis &= ~np.asarray(hidden[r0:r1, :kend], dtype=bool)
            if add is not None:
                Ma = np.asarray(add[r0:r1, :kend], dtype=np.float64)
                vis &= np.isfinite(Ma)
                S = S + np.where(vis, Ma, 0.0)
            seen = np.isfinite(lse[r0:r1])
            keep = vis & seen[:, None]
            # (exponents formed only where kept: a hidden pair's would be discarded anyway)
            P = np.where(keep, np.exp(np.where(keep, S - np.where(seen, lse[r0:r1], 0.0)[:, None], -np.inf)), 0.0)
        else:
            if causal:
                S = np.where(np.arange(kend)[None, :] > np.arange(r0, r1)[:, None], -np.inf, S)
            P = np.exp(S - lse[r0:r1, None])
        A = np.abs(do[r0:r1]) @ np.abs(v[:kend]).T
        PZ = P if drop is None else P * zk[r0:r1, :kend]
        W = PZ * A + P * E[r0:r1, None]
        mv[:kend] += PZ.T @ np.abs(do[r0:r1])
        mq[r0:r1] = scale * (W @ np.abs(k[:kend]))
        mk[:kend] += scale * (W.T @ np.abs(q[r0:r1]))
    return mq, mk, mv


# Unit roundoff of fp32, the precision of every sum and of the softmax statistics.
E32 = 2.0 ** -24


def bwd_parity_bar(m: np.ndarray, u: float, d: int, n_terms: int) -> np.ndarray:
    """Elementwise bar |g - g_ref| <= (2u + (d + n_terms) e32) * M for a gradient computed with
    16-bit operands in its products and fp32 everywhere else, M from
    ``head_attention_bwd_magnitude_fp64``.

    The precision is the method's, not one implementation's: the pages' kernels multiply
    fp16/bf16 operands and accumulate in fp32, with fp32 softmax statistics (intelliparadigm
    page, section 2.2: fp16/bf16 inputs with fp32 max and sum outputs; zyxy lecture, section 5:
    the FA2 kernels run in fp16/bf16). A term of a gradient passes through at most two roundings
    to the input type (unit roundoff u: 2^-11 for fp16, 2^-8 for bf16): its probability or
    score-gradient factor as a product operand, and O when the caller stored it in 16 bits
    (D then comes from that O). Its fp32 parts are a dot product over the head dimension d
    (S, dP, D) and a sum over the n_terms terms of the element (keys per row for dQ, rows of
    every query head of the group for dK and dV), each adding at most e32 per step. Every
    term's relative error is therefore at most 2u + (d + n_terms) e32 to first order; the
    second-order remainder (products of two of these) is below 2^-14 of the bar at the sizes
    tested.
    """
    return (2.0 * u + (d + n_terms) * E32) * np.asarray(m, dtype=np.float64)


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
