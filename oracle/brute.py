"""Pure-Python brute-force attention for tiny shapes — TEST INFRASTRUCTURE.

The same definition as ``attention.head_attention_fp64`` (zyxy.net lecture
page, section 1; intelliparadigm page, section 1.1; safe softmax from the
cnblogs page, "时间复杂度"), written with nested loops, ``math.exp`` and
``math.fsum`` (exactly rounded sums), no numpy arithmetic. It exists to pin
the numpy oracle on shapes with B, H <= 2, N <= ~16, d <= ~8.
"""
from __future__ import annotations

import math


def attention_brute(q, k, v, scale: float, causal: bool):
    """q: nested lists [B][Hq][N][d]; k, v: [B][Hkv][N][d]. Returns (O, LSE) as nested lists."""
    B, Hq, N = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    d = len(q[0][0][0])
    O = [[[[0.0] * d for _ in range(N)] for _ in range(Hq)] for _ in range(B)]
    LSE = [[[0.0] * N for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            for i in range(N):
                keys = range(i + 1) if causal else range(N)
                s = {j: scale * math.fsum(float(q[b][h][i][c]) * float(k[b][hk][j][c]) for c in range(d))
                     for j in keys}
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in keys}
                l = math.fsum(e.values())
                for c in range(d):
                    O[b][h][i][c] = math.fsum(e[j] * float(v[b][hk][j][c]) for j in keys) / l
                LSE[b][h][i] = m + math.log(l)
    return O, LSE
