"""Attention with dropout on the probabilities, in fp64 -- TEST INFRASTRUCTURE (see the package doc).

What the pages say. The Ascend operator takes a keep_prob attribute, 1.0 by default
(intelliparadigm page, section 2.2, and its Python call in section 4.1), and the cnblogs page
points to FlashAttention-1's Algorithm 2, which adds dropout (and the mask) to the loop of
Algorithm 1. The reading taken: dropout acts on the softmax probabilities after they are formed
and before they multiply V; each (query, key) pair is kept independently with probability keep,
and kept probabilities are scaled by 1 / keep, so that
    O_i = sum_j (Z_ij / keep) P_ij V_j,     LSE_i as without dropout,
with Z_ij in {0, 1}. The LSE stays the statistic of the undropped softmax: it is what the backward
recomputes P from. The gradients follow by the chain rule with Z fixed:
    dV = (Z o P / keep)^T dO,  dP = (dO V^T) o Z / keep,  D_i = sum_j P_ij dP_ij = dO_i . O_i,
    dS = P o (dP - D),  dQ = s dS K,  dK = s dS^T Q.

The random numbers (the pages name no generator; this is the reading taken). Z must be drawn
identically by the oracle and the GPU, so it comes from a counter-based generator, Philox4x32-10
(Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011): ten
rounds over a 128-bit counter and a 64-bit key, each round two 32x32->64-bit products with the
multipliers 0xD2511F53 and 0xCD9E8D57, the key bumped by the Weyl constants 0x9E3779B9 and
0xBB67AE85 between rounds. For head plane h = b * Hq + hq, query row i and key j:
    words = Philox4x32-10(counter = (j >> 2, i >> 2, h, offset), key = (seed low 32, high 32))
    byte  = (words[i & 3] >> (8 (j & 3))) & 0xFF,     Z_ij = 1 iff byte < T,
with T = round(256 keep) clamped to [1, 256]: one call covers a 4 x 4 block of (query, key)
pairs, byte 4 (i & 3) + (j & 3) of its output. keep is therefore taken in steps of 1/256: the
scale applied is 256 / T, the exact inverse of the keep probability used.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .attention import band_visible, head_attention_band_fp64

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 on arrays of counters (c0..c3, uint32-valued) and a key (k0, k1): the four
    output words as uint64 arrays holding 32-bit values."""
    c = [np.asarray(x, dtype=np.uint64) & MASK32 for x in (c0, c1, c2, c3)]
    k = [np.uint64(k0 & MASK32), np.uint64(k1 & MASK32)]
    for r in range(10):
        if r > 0:
            k = [np.uint64((int(k[0]) + W0) & MASK32), np.uint64((int(k[1]) + W1) & MASK32)]
        p0 = np.uint64(M0) * c[0]
        p1 = np.uint64(M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c = [hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0]
    return c


def keep_threshold(keep_prob: float) -> int:
    """T = round(256 keep_prob) clamped to [1, 256]: a pair is kept iff its random byte is < T."""
    return int(min(256, max(1, round(256.0 * float(keep_prob)))))


def keep_mask(seed: int, offset: int, plane: int, rows: np.ndarray, keys: np.ndarray, keep_prob: float) -> np.ndarray:
    """Z [len(rows), len(keys)] (bool) for head plane ``plane`` = b * Hq + hq (module doc)."""
    rows = np.asarray(rows, dtype=np.int64)[:, None]
    keys = np.asarray(keys, dtype=np.int64)[None, :]
    rr, kk = np.broadcast_arrays(rows, keys)
    words = philox4x32_10(kk >> 2, rr >> 2, np.full(rr.shape, plane), np.full(rr.shape, offset & MASK32),
                          seed & MASK32, (seed >> 32) & MASK32)
    sel = rr & 3
    w = np.where(sel == 0, words[0], np.where(sel == 1, words[1], np.where(sel == 2, words[2], words[3])))
    byte = (w >> (np.uint64(8) * (kk & 3).astype(np.uint64))) & np.uint64(0xFF)
    return byte < np.uint64(keep_threshold(keep_prob))


def head_attention_dropout_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                                left: Optional[int], right: Optional[int], off: int, Z: np.ndarray,
                                keep_prob: float) -> Tuple[np.ndarray, np.ndarray]:
    """O and LSE of one head with the keep mask Z [n, N] applied to the probabilities (module
    doc), under the band of ``attention.band_visible``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, N = q.shape[0], k.shape[0]
    _, L = head_attention_band_fp64(q, k, v, scale, left, right, off)
    vis = band_visible(np.arange(n), np.arange(N), left, right, off)
    seen = np.isfinite(L)
    S = scale * (q @ k.T)
    P = np.where(vis & seen[:, None], np.exp(np.where(vis, S, 0.0) - np.where(seen, L, 0.0)[:, None]), 0.0)
    inv_keep = 256.0 / keep_threshold(keep_prob)
    O = (P * Z * inv_keep) @ v
    return O, L


def head_attention_bwd_dropout_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                                    left: Optional[int], right: Optional[int], off: int, Z: np.ndarray,
                                    keep_prob: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(dQ, dK, dV) of one head with the keep mask Z fixed (module doc)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n, N = q.shape[0], k.shape[0]
    _, L = head_attention_band_fp64(q, k, v, scale, left, right, off)
    vis = band_visible(np.arange(n), np.arange(N), left, right, off)
    seen = np.isfinite(L)
    S = scale * (q @ k.T)
    P = np.where(vis & seen[:, None], np.exp(np.where(vis, S, 0.0) - np.where(seen, L, 0.0)[:, None]), 0.0)
    inv_keep = 256.0 / keep_threshold(keep_prob)
    Pd = P * Z * inv_keep
    dv = Pd.T @ do
    dP = (do @ v.T) * Z * inv_keep
    D = np.sum(P * dP, axis=1)
    dS = P * (dP - D[:, None])
    return scale * (dS @ k), scale * (dS.T @ q), dv
