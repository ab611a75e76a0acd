"""Attention with an additive (float) mask, in fp64 -- TEST INFRASTRUCTURE (see the package doc).

What the pages say. The Ascend operator's optional attn_mask input may be fp16, fp32 or bool
(intelliparadigm page, section 2.2); the pages do not say what the float forms mean. The
reading taken: a float mask is added to the scaled scores before the softmax (PyTorch's
convention for a float attention mask, the framework of the zyxy lecture), so
    S_ij = s Q_i . K_j + M_ij,    O_i = sum_j softmax_j(S_i) V_j,    LSE_i = logsumexp_j S_ij,
over the keys the band leaves visible. An entry of -inf hides its key (its weight is exactly
0), so the boolean form is the special case M in {0, -inf}. A row whose visible keys all carry
-inf sees no key: O = 0 and LSE = -inf, as for an empty band. Entries are finite or -inf (NaN
and +inf have no softmax). The mask is an input, not a parameter: no gradient flows to it.
The gradients through Q, K and V follow the same chain rule as without it, with P formed from
the masked scores.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .attention import band_visible

ROW_BLOCK = 512


def _masked_scores(q: np.ndarray, k: np.ndarray, M: np.ndarray, scale: float, left: Optional[int],
                   right: Optional[int], off: int, r0: int, r1: int) -> Tuple[np.ndarray, np.ndarray]:
    """Rows [r0, r1): (S with -inf where a key is hidden, visible-and-finite flags)."""
    N = k.shape[0]
    vis = band_visible(np.arange(r0, r1), np.arange(N), left, right, off)
    Mr = np.asarray(M[r0:r1], dtype=np.float64)
    vis = vis & np.isfinite(Mr)
    S = np.where(vis, scale * (q[r0:r1] @ k.T) + np.where(vis, Mr, 0.0), -np.inf)
    return S, vis


def head_attention_additive_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                                 left: Optional[int], right: Optional[int], off: int,
                                 M: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """O [n, d] and LSE [n] of one head with the additive mask M [n, N] (module doc), under the
    band of ``attention.band_visible``: the three passes of the definition (row max, shifted
    exponentials and their sum, normalised product with V)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    O = np.zeros((n, v.shape[1]))
    L = np.full(n, -np.inf)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        S, vis = _masked_scores(q, k, M, scale, left, right, off, r0, r1)
        seen = vis.any(axis=1)
        if not seen.any():
            continue
        Ss = S[seen]
        m = Ss.max(axis=1)
        e = np.exp(Ss - m[:, None])
        l = e.sum(axis=1)
        rows = np.arange(r0, r1)[seen]
        O[rows] = (e / l[:, None]) @ v
        L[rows] = m + np.log(l)
    return O, L


def head_attention_bwd_additive_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                                     left: Optional[int], right: Optional[int], off: int, M: np.ndarray
                                     ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(dQ, dK, dV) of one head with the additive mask M held fixed: P = exp(S - LSE) from the
    masked scores, dV = P^T dO, dP = dO V^T, D_i = sum_j P_ij dP_ij, dS = P o (dP - D),
    dQ = s dS K, dK = s dS^T Q."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n = q.shape[0]
    _, L = head_attention_additive_fp64(q, k, v, scale, left, right, off, M)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        S, vis = _masked_scores(q, k, M, scale, left, right, off, r0, r1)
        seen = np.isfinite(L[r0:r1])
        P = np.where(vis & seen[:, None], np.exp(S - np.where(seen, L[r0:r1], 0.0)[:, None]), 0.0)
        dv += P.T @ do[r0:r1]
        dP = do[r0:r1] @ v.T
        D = np.sum(P * dP, axis=1)
        dS = P * (dP - D[:, None])
        dq[r0:r1] = scale * (dS @ k)
        dk += scale * (dS.T @ q[r0:r1])
    return dq, dk, dv
