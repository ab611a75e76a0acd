"""Softmax in fp64: the safe three-pass form and the online-normaliser form.

Test infrastructure only (see the package doc).

Sources (page titles as given by the pages):
  * "Flash Attention是怎么做到又快又省显存的？" (cnblogs, reposted from
    zhihu), section "时间复杂度": naive softmax, the overflow argument for
    fp16, safe softmax in three passes (max, shifted denominator, outputs),
    and the online normaliser recurrence d'_i = d'_{i-1} e^{m_{i-1}-m_i} +
    e^{x_i-m_i} that fuses the first two passes.
  * The Triton FA2 walkthrough (xrbh.cn quote/28716): PyTorch's softmax is
    the safe form.

Reading taken: the page's Python listing divides exponentials that were
never rescaled to the final maximum; its own formulas (outputs
e^{x_i - m_N} / d'_N) are followed instead.
"""
from __future__ import annotations

import numpy as np


def safe_softmax(x: np.ndarray, axis: int = -1) -> np.ndarray:
    """Three-pass safe softmax along ``axis`` (cnblogs page, "时间复杂度").

    pass 1: m = max_i x_i;  pass 2: d = sum_i e^{x_i - m};  pass 3: a_i = e^{x_i - m} / d.
    Entries equal to -inf (masked) get probability 0; a row must have at
    least one finite entry.
    """
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=axis, keepdims=True)  # pass 1
    e = np.exp(x - m)
    d = np.sum(e, axis=axis, keepdims=True)  # pass 2
    return e / d  # pass 3


def logsumexp(x: np.ndarray, axis: int = -1) -> np.ndarray:
    """Natural-log log-sum-exp, m + ln(sum e^{x-m}), the statistic a backward pass reuses."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=axis, keepdims=True)
    d = np.sum(np.exp(x - m), axis=axis, keepdims=True)
    return np.squeeze(m + np.log(d), axis=axis)


def online_softmax(x) -> np.ndarray:
    """Online-normaliser softmax of a 1-D sequence (cnblogs page, "时间复杂度").

    One pass keeps the running maximum m_i and the denominator d'_i taken
    relative to it, d'_i = d'_{i-1} * e^{m_{i-1} - m_i} + e^{x_i - m_i},
    starting from m_0 = -inf, d'_0 = 0; a second pass emits
    a_i = e^{x_i - m_N} / d'_N.
    """
    xs = [float(v) for v in np.asarray(x, dtype=np.float64).ravel()]
    m = -np.inf
    d = 0.0
    for xi in xs:
        m_new = max(m, xi)
        d = d * np.exp(m - m_new) + np.exp(xi - m_new)
        m = m_new
    return np.array([np.exp(xi - m) / d for xi in xs], dtype=np.float64)
