"""Parity bars for the GPU path's other input types -- TEST INFRASTRUCTURE (see the package doc).

The result is always the fp64 definition of attention (attention.py). What a bar adds is how
far an evaluation in a stated precision may move each output, to first order, written from
that precision and the problem alone. The tests compare the GPU against the definition within
these bars.

fp32 inputs (the Ascend operator on the intelliparadigm page, section 2.2, accepts query, key
and value in fp32): every product and sum in fp32, unit roundoff e32 = 2^-24. For row i of a
head, with w_ij = exp(S_ij - LSE_i) over its n_i visible keys:
  * an exponent is a dot product of d terms, scaled, shifted by the running maximum and
    converted to base 2 (one fma), then exponentiated: its absolute error is at most
    (d + 8) e32 a_ij with a_ij = s sum_c |Q_ic K_jc| + 1 (the magnitude of its terms, plus the
    shift), which moves weight j by that much relative;
  * O_ic = sum_j w_ij V_jc with the weights' common factor divided out: a relative error
    delta_j of weight j moves O_ic by sum_j w_ij delta_j (V_jc - O_ic);
  * the sums over keys of P V and of P (the denominator) each run over n_i terms: at most
    n_i e32 sum_j w_ij |V_jc| and n_i e32 |O_ic| <= n_i e32 sum_j w_ij |V_jc|.
Together, per element:
  bar_O[i,c] = (d + 8) e32 sum_j w_ij a_ij |V_jc - O_ic| + 2 (n_i + 2) e32 sum_j w_ij |V_jc|
  bar_LSE[i] = (d + 8) e32 sum_j w_ij a_ij + (n_i + 4) e32 + 2 e32 |LSE_i|
(LSE = m + ln l: the exponent errors averaged by the weights, the denominator's sum, and the
final conversion and rounding.) These are worst-case sums, so they are conservative by about
the square root of the lengths; they still separate fp32 arithmetic from any 16-bit rounding
of the inputs or the probabilities, which moves outputs by 2^-11 to 2^-8 relative.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .attention import band_visible, head_attention_band_fp64

E32 = 2.0 ** -24
ROW_BLOCK = 512


def head_attention_f32_bar_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                                left: Optional[int], right: Optional[int], off: int = 0
                                ) -> Tuple[np.ndarray, np.ndarray]:
    """(bar_O [n, d], bar_LSE [n]) for one head evaluated in fp32 (module doc), under the band
    of ``attention.band_visible`` (causal: left None, right 0). Rows that see no key get 0."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, N = q.shape[0], k.shape[0]
    d = q.shape[1]
    O, L = head_attention_band_fp64(q, k, v, scale, left, right, off)
    bar_o = np.zeros((n, v.shape[1]))
    bar_l = np.zeros(n)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        vis = band_visible(np.arange(r0, r1), np.arange(N), left, right, off)
        seen = np.isfinite(L[r0:r1])
        S = scale * (q[r0:r1] @ k.T)
        W = np.where(vis & seen[:, None], np.exp(np.where(vis, S, 0.0) - np.where(seen, L[r0:r1], 0.0)[:, None]), 0.0)
        A = scale * (np.abs(q[r0:r1]) @ np.abs(k).T) + 1.0
        WA = W * A
        nvis = vis.sum(axis=1).astype(np.float64)
        # sum_j w_ij a_ij |V_jc - O_ic| = sum_j WA_ij |V_jc - O_ic|, per column c
        dev = np.empty((r1 - r0, v.shape[1]))
        for i in range(r1 - r0):
            dev[i] = WA[i] @ np.abs(v - O[r0 + i])
        bar_o[r0:r1] = (d + 8) * E32 * dev + 2.0 * (nvis + 2.0)[:, None] * E32 * (W @ np.abs(v))
        bar_l[r0:r1] = np.where(seen, (d + 8) * E32 * WA.sum(axis=1) + (nvis + 4.0) * E32
                                + 2.0 * E32 * np.abs(np.where(seen, L[r0:r1], 0.0)), 0.0)
    return bar_o, bar_l
