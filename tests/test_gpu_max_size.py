"""GPU parity at the largest head plane the C ABI accepts: N * d = 2^30 - 2^16 elements (a
2 GiB bf16 plane per tensor), where the kernel's 32-bit byte offsets within a plane and its
prefetches past the plane's end come closest to 2^31.

A causal sliding window of 256 keys keeps the work small (every row sees at most 257 keys),
so the whole sequence runs in one launch of 65532 work-groups; rows at both ends and in the
middle are compared with the fp64 oracle on the key slice each row can see. Bars as in
test_gpu_parity.py: O within 1e-2 (bf16 inputs), LSE within 1e-4 relative with a floor of 1.
"""
import numpy as np
import pytest
import torch

import exact_attention_114_amd as fa
from exact_attention_114_amd import inputs as I
from oracle.attention import head_attention_band_fp64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MAX_PLANE = (1 << 30) - (1 << 16)


def test_largest_plane_d128_window():
    d, dt, left = 128, I.BF16, 256
    N = MAX_PLANE // d
    assert N * d == MAX_PLANE
    print(f"[gpu] fa_fwd largest plane N={N} d={d} {dt} window=({left}, 0)", flush=True)
    qkv = I.draw_qkv(1, 1, 1, N, d, dt, 1800)
    q, k, v = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV) for x in (qkv.q, qkv.k, qkv.v))
    scale = d ** -0.5
    O, L = fa.fwd(q, k, v, scale=scale, window=(left, 0))
    torch.cuda.synchronize()
    del q, k, v
    rng = np.random.Generator(np.random.PCG64(1801))
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 257, N // 2, N - 129, N - 128, N - 33, N - 2, N - 1],
                                     rng.integers(0, N, 24)]))
    Og = O[0, 0, torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    Lg = L[0, 0, torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    for idx, r in enumerate(rows):
        s = max(0, int(r) - left)  # the row's keys: s .. r
        qr = I.bits_to_f64(qkv.q[0, 0, r:r + 1], dt)
        ks = I.bits_to_f64(qkv.k[0, 0, s:r + 1], dt)
        vs = I.bits_to_f64(qkv.v[0, 0, s:r + 1], dt)
        O_ref, L_ref = head_attention_band_fp64(qr, ks, vs, I.scale_f32(scale), left, 0,
                                                q_pos=np.array([r - s]))
        err_o = np.abs(Og[idx] - O_ref[0]).max()
        assert err_o <= 1e-2, f"row {r}: max|dO| {err_o:.3e}"
        err_l = abs(Lg[idx] - L_ref[0]) / max(1.0, abs(L_ref[0]))
        assert err_l <= 1e-4, f"row {r}: LSE rel err {err_l:.3e}"


def test_largest_plane_d128_window_backward():
    """fa_bwd_ex at the same size. The gradients of the last 1024 query rows, and of the keys
    among the last 1024, depend only on those rows (each sees 257 keys, each key is seen by at
    most 257 rows): their O and LSE are set to the oracle's before the call, and dQ, dK, dV there
    are checked against the oracle's gradients of that slice within the backward bar
    (bwd_check.py)."""
    import bwd_check
    from oracle.backward import head_attention_bwd_band_fp64, head_attention_bwd_magnitude_fp64

    d, dt, left, blk = 128, I.BF16, 256, 1024
    N = MAX_PLANE // d
    print(f"[gpu] fa_bwd largest plane N={N} d={d} {dt} window=({left}, 0)", flush=True)
    qkv = I.draw_qkv(1, 1, 1, N, d, dt, 1810)
    dob = I.draw_dout(1, 1, N, d, dt, 1811)
    to = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    q, k, v, do = to(qkv.q), to(qkv.k), to(qkv.v), to(dob)
    scale = d ** -0.5
    sc = I.scale_f32(scale)
    O, L = fa.fwd(q, k, v, scale=scale, window=(left, 0))
    # the oracle's O and LSE for the last blk rows (keys from N - blk - left)
    r0, k0 = N - blk, N - blk - left
    qs = I.bits_to_f64(qkv.q[0, 0, r0:], dt)
    ks = I.bits_to_f64(qkv.k[0, 0, k0:], dt)
    vs = I.bits_to_f64(qkv.v[0, 0, k0:], dt)
    dos = I.bits_to_f64(dob[0, 0, r0:], dt)
    O_ref, L_ref = head_attention_band_fp64(qs, ks, vs, sc, left, 0, off=r0 - k0)
    O[0, 0, r0:] = torch.from_numpy(O_ref.astype(np.float32)).to(DEV)
    L[0, 0, r0:] = torch.from_numpy(L_ref.astype(np.float32)).to(DEV)
    dq, dk, dv = fa.bwd(q, k, v, O, L, do, scale=scale, window=(left, 0))
    torch.cuda.synchronize()
    got = (dq[0, 0, r0:].cpu().numpy().astype(np.float64), dk[0, 0, r0:].cpu().numpy().astype(np.float64),
           dv[0, 0, r0:].cpu().numpy().astype(np.float64))
    gq, gk, gv = head_attention_bwd_band_fp64(qs, ks, vs, dos, sc, left, 0, off=r0 - k0)
    mq, mk, mv = head_attention_bwd_magnitude_fp64(qs, ks, vs, dos, sc, False, band=(left, 0, r0 - k0))
    # keys k0 .. r0 - 1 are also seen by rows before r0: only keys from r0 on are complete here
    for name, g, r, m, n in (("dQ", got[0], gq, mq, left + 1), ("dK", got[1], gk[left:], mk[left:], left + 1),
                             ("dV", got[2], gv[left:], mv[left:], left + 1)):
        ratio = bwd_check.check_one("largest plane", name, g, r, m, dt, d, n)
        print(f"[bar] largest plane {name}: worst error/bar {ratio:.4f}", flush=True)
