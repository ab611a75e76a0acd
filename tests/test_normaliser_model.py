"""Why O is normalised by the sum of the rounded probabilities, for fp16 and bf16 inputs (CPU).

The kernel multiplies V by P rounded to the input type (the 16-bit operand of the P V product)
and exponentiates against a reference that may sit up to 8 (log2 units) below a row's running
maximum: a key that dominates its row then has an exponential 2^x with x in (0, 8) and an
arbitrary mantissa, whose 16-bit rounding is up to u = 2^-11 (fp16) relative. This test models
one such row in numpy with the kernel's arithmetic (fp32 scores and exponentials, fp16 P):
  * normalised by the unrounded fp32 sum, O's error reaches about u |V| = 2.4e-3 for |V| = 5,
    above the 2e-3 fp16 bar;
  * normalised by the sum of the rounded values that multiply V, the weights sum to one and the
    dominant key's rounding cancels: the error stays below 1e-4.
The GPU test test_gpu_parity.py::test_dominant_key_stale_reference runs the same alignment on
the kernel.
"""
import numpy as np

C = np.float32(0.125 * 1.4426950408889634)  # scale 1/8 times log2(e)


def row_errors(a: float, v_dom: float, v_ref: float):
    """One row with a reference key (score a, first tile: sets the reference) and a dominant key
    (score 2a, later tile), every other key negligible. Returns (error with the unrounded sum,
    error with the rounded sum) of O against the exact softmax average, or None when the
    dominant exponential would fail the lane-sum check (>= 2^8) and trigger a rescale."""
    s_ref = np.float32(a)
    s_dom = np.float32(2.0 * a)
    m = np.float32(s_ref * C)                          # the reference: the first tile's row max
    x = np.float32(np.float64(s_dom) * np.float64(C) - np.float64(m))  # one fma, rounded once
    p = np.float32(np.exp2(np.float64(x)))
    if p >= 256.0:
        return None
    p16 = np.float64(np.float16(p))
    p = np.float64(p)
    exact_w = np.exp2(np.float64(s_dom - s_ref) * np.float64(C))
    exact = (exact_w * v_dom + v_ref) / (exact_w + 1.0)
    unrounded = (p16 * v_dom + v_ref) / (p + 1.0)
    rounded = (p16 * v_dom + v_ref) / (p16 + 1.0)
    return abs(unrounded - exact), abs(rounded - exact)


def test_dominant_key_normaliser():
    worst_unrounded = worst_rounded = 0.0
    for a in np.linspace(38.0, 44.5, 4001):
        r = row_errors(float(a), 5.0, -5.0)
        if r is None:
            continue
        worst_unrounded = max(worst_unrounded, r[0])
        worst_rounded = max(worst_rounded, r[1])
    print(f"dominant key, |V| = 5: unrounded-sum normaliser {worst_unrounded:.3e}, rounded-sum {worst_rounded:.3e}")
    assert worst_unrounded > 2e-3  # the unrounded sum breaks the fp16 bar on this alignment
    assert worst_rounded < 1e-4
