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

fp8 inputs (OCP e4m3 bytes with per-tensor descales; the zyxy lecture, section 5, lists fp8
among the FA2-generation input types). The oracle takes the represented values (byte value
times descale) exactly. Products of e4m3 values are exact; but the fp8 matrix instruction
sums 64 of them (the head dimension padded with zeros to a multiple of 64) far less exactly
than fp32 would: on MI355X its error over 65536 random e4m3 sums reached 2^-11.1 of the
largest product (a sum of 448 * 448 and 63 products of 2^-7 came out 200704.4375 against the
exact 200704.4921875), as if each product kept about 17 bits relative to the largest. So
each exponent's error is bounded per 64-long range by FP8_DOT_REL = 2^-10 times the range's
largest |Q_ic K_jc| (times the scale), plus the fp32 terms of the shift and the exponential
(fp8_exponent_error); the rest of the fp32 bar applies with Q, K, V the represented values.
In addition the probabilities
are rounded to e4m3 for the P V product and O is divided by the sum of the rounded values.
Measured against the row's largest weight, a probability p rounds within 2^-4 p (3 mantissa
bits) or, in e4m3's subnormal range, within 2^-10: the rounding reference is a running
maximum no larger than the row's, which only makes the subnormal step finer relative to the
row. With the rounded values in both numerator and denominator, O moves by exactly
sum_j dp_j (V_jc - O_ic) / sum_j (p_j + dp_j), so per element
  bar8_O[i,c] = sum_j (2^-4 w_ij + min(w_ij, 2^-10 w_max,i)) |V_jc - O_ic|
                / (1 - 2^-4 - sum_j min(w_ij, 2^-10 w_max,i)) + bar_O[i,c]
with w_max,i the row's largest weight, and bar8_LSE = bar_LSE (the LSE uses the unrounded
fp32 sum). A row whose denominator is not positive has no bound at this precision (inf).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .attention import band_visible, head_attention_band_fp64

E32 = 2.0 ** -24
ROW_BLOCK = 512


def f32_exponent_error(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """[n, N] bound on the fp32 error of each exponent (natural-log units): (d + 8) e32 a_ij with
    a_ij = s sum_c |Q_ic K_jc| + 1 (module doc)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = q.shape[1]
    return (d + 8) * E32 * (scale * (np.abs(q) @ np.abs(k).T) + 1.0)


def head_attention_f32_bar_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                                left: Optional[int], right: Optional[int], off: int = 0,
                                exponent_error=f32_exponent_error) -> Tuple[np.ndarray, np.ndarray]:
    """(bar_O [n, d], bar_LSE [n]) for one head evaluated in fp32 (module doc), under the band
    of ``attention.band_visible`` (causal: left None, right 0). Rows that see no key get 0.
    ``exponent_error(q_rows, k, scale)`` gives the bound on each exponent's error (the fp8 bar
    passes its own)."""
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
        WA = W * exponent_error(q[r0:r1], k, scale)
        nvis = vis.sum(axis=1).astype(np.float64)
        # sum_j w_ij E_ij |V_jc - O_ic| = sum_j WA_ij |V_jc - O_ic|, per column c
        dev = np.empty((r1 - r0, v.shape[1]))
        for i in range(r1 - r0):
            dev[i] = WA[i] @ np.abs(v - O[r0 + i])
        bar_o[r0:r1] = dev + 2.0 * (nvis + 2.0)[:, None] * E32 * (W @ np.abs(v))
        bar_l[r0:r1] = np.where(seen, WA.sum(axis=1) + (nvis + 4.0) * E32
                                + 2.0 * E32 * np.abs(np.where(seen, L[r0:r1], 0.0)), 0.0)
    return bar_o, bar_l


# The fp8 matrix instruction's error on a 64-long sum, relative to its largest product: measured at
# most 2^-11.1 on MI355X; the bar takes 2^-10.
FP8_DOT_REL = 2.0 ** -10


def fp8_exponent_error(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """[n, N] bound on each exponent's error with fp8 inputs (natural-log units): for every 64-long
    range of the head dimension that one fp8 instruction sums, FP8_DOT_REL times its largest
    product's magnitude (times the scale), plus 8 e32 a_ij for the shift, the conversion to base
    2 and the exponential (module doc)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n, d = q.shape
    err = 8 * E32 * (scale * (np.abs(q) @ np.abs(k).T) + 1.0)
    for c0 in range(0, d, 64):
        aq, ak = np.abs(q[:, c0:c0 + 64]), np.abs(k[:, c0:c0 + 64])
        mx = np.zeros((n, k.shape[0]))
        for c in range(aq.shape[1]):
            np.maximum(mx, aq[:, c:c + 1] * ak[:, c][None, :], out=mx)
        err += scale * FP8_DOT_REL * mx
    return err


def head_attention_fp8_bar_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                                left: Optional[int], right: Optional[int], off: int = 0
                                ) -> Tuple[np.ndarray, np.ndarray]:
    """(bar_O [n, d], bar_LSE [n]) for one head with e4m3 inputs (q, k, v: the represented values)
    and e4m3 probabilities in the P V product (module doc), under the band of
    ``attention.band_visible``. Rows that see no key get 0."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, N = q.shape[0], k.shape[0]
    d = q.shape[1]
    bar_o, bar_l = head_attention_f32_bar_fp64(q, k, v, scale, left, right, off,
                                               exponent_error=fp8_exponent_error)
    O, L = head_attention_band_fp64(q, k, v, scale, left, right, off)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        vis = band_visible(np.arange(r0, r1), np.arange(N), left, right, off)
        seen = np.isfinite(L[r0:r1])
        S = scale * (q[r0:r1] @ k.T)
        W = np.where(vis & seen[:, None], np.exp(np.where(vis, S, 0.0) - np.where(seen, L[r0:r1], 0.0)[:, None]), 0.0)
        wmax = W.max(axis=1, initial=0.0)
        sub = np.minimum(W, 2.0 ** -10 * wmax[:, None])
        den = 1.0 - 2.0 ** -4 - sub.sum(axis=1)
        U = 2.0 ** -4 * W + sub
        for i in range(r1 - r0):
            if not seen[i]:
                continue
            num = U[i] @ np.abs(v - O[r0 + i])
            bar_o[r0 + i] += num / den[i] if den[i] > 0 else np.inf
    return bar_o, bar_l
