"""GPU parity of the additive (float) attention mask, fa_fwd_float_mask and fa_bwd_float_mask,
against the fp64 oracle (oracle/additive.py), on the mask values as stored (fp16 values are
exactly representable in fp64).

Bars. Forward: the probabilities are rounded to the input type before P V, which moves weight j
by at most u relative; with the normaliser summing the same rounded values, O_ic moves by at
most u (sum_j P_ij |V_jc| + |O_ic|). The bar is the forward's (2e-3 fp16, 1e-2 bf16, about 4 u
and 2.5 u) times max(1, that magnitude). The mask also enters each exponent, evaluated in
fp32: its argument sums terms of size a_ij = |s S_ij| + |M_ij| + |LSE_i| with at most four
roundings, a relative weight error eps_ij = 4 e32 a_ij (e32 = 2^-24), which moves O_ic by
sum_j P_ij eps_ij |V_jc - O_ic|; the bar adds that. (For |M| of order 1 it is negligible; for
entries of -1e4 it is about 2^-24 * 4e4 and exceeds the 16-bit rounding: any fp32 evaluation
of s S + M has it.) LSE: 1e-4 relative, floor 1, plus eps averaged by the weights.
Backward: bwd_check.py's bar with the magnitude sums of the masked chain rule (oracle.backward,
``add``), plus 2 max_ij eps_ij times the same magnitudes (every term carries P, the D terms
twice).
"""

E32 = 2.0 ** -24
import math

import numpy as np
import pytest
import torch

import bwd_check
import exact_attention_114_amd as fa
from exact_attention_114_amd import inputs as I
from oracle.additive import head_attention_additive_fp64, head_attention_bwd_additive_fp64
from oracle.attention import band_visible

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_O = {I.F16: 2e-3, I.BF16: 1e-2}
TOL_LSE = 1e-4


def to_dev(bits, dt):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dt == I.F16 else torch.bfloat16).to(DEV)


def make_mask(kind, Bm, Hm, Nq, Nk, mdt, seed, pad=0):
    """A [Bm, Hm, Nq, Nk] mask (float64 values as stored in mdt) and its device tensor, with its
    rows padded by ``pad`` elements (a row stride of Nk + pad)."""
    g = np.random.Generator(np.random.PCG64(seed))
    if kind == "random":
        M = g.standard_normal((Bm, Hm, Nq, Nk)) * 3.0
        M[g.random(M.shape) < 0.15] = -np.inf
        M[..., Nq // 3, :] = -np.inf  # a row with every key hidden
    elif kind == "alibi":
        i = np.arange(Nq)[:, None] + (Nk - Nq)
        j = np.arange(Nk)[None, :]
        slopes = 2.0 ** (-8.0 * (np.arange(Hm) + 1) / Hm)
        M = -slopes[None, :, None, None] * np.abs(i - j)[None, None] * np.ones((Bm, 1, 1, 1))
    elif kind == "far":
        M = np.where(g.random((Bm, Hm, Nq, Nk)) < 0.5, -1.0e4, g.standard_normal((Bm, Hm, Nq, Nk)))
        M[..., : Nq // 4, :] = -1.0e4  # rows whose every key carries the same large offset
    else:
        raise ValueError(kind)
    tdt = torch.float16 if mdt == "f16" else torch.float32
    Mt = torch.from_numpy(M.astype(np.float32)).to(tdt)
    M = Mt.to(torch.float64).numpy()  # the values as stored
    full = torch.zeros((Bm, Hm, Nq, Nk + pad), dtype=tdt)
    full[..., :Nk] = Mt
    return M, full.to(DEV)[..., :Nk]


def plane(M, b, h):
    return M[b if M.shape[0] > 1 else 0, h if M.shape[1] > 1 else 0]


FWD_CASES = [  # (B, Hq, Hkv, Nq, Nk, d, dt, left, right, kind, mdt, Bm, Hm, pad)
    (2, 4, 2, 300, 300, 64, I.F16, None, 0, "random", "f16", 2, 4, 0),
    (1, 4, 1, 200, 333, 128, I.BF16, None, None, "random", "f32", 1, 4, 3),
    (2, 2, 2, 257, 257, 96, I.F16, None, None, "alibi", "f32", 1, 2, 3),
    (1, 3, 1, 129, 520, 48, I.BF16, 100, 20, "alibi", "f16", 1, 3, 8),
    (2, 2, 1, 190, 190, 32, I.F16, None, 0, "far", "f32", 2, 1, 2),
    (1, 2, 2, 400, 400, 80, I.BF16, None, None, "far", "f16", 1, 1, 0),
    (1, 2, 1, 333, 333, 112, I.F16, 64, 0, "random", "f16", 1, 1, 3),
]


def run_forward(B, Hq, Hkv, Nq, Nk, d, dt, left, right, kind, mdt, Bm, Hm, pad, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    qb, kb, vb = (I.to_bits(g.standard_normal(sh, dtype=np.float32), dt)
                  for sh in ((B, Hq, Nq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d)))
    M, Mt = make_mask(kind, Bm, Hm, Nq, Nk, mdt, seed + 1, pad)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = (to_dev(x, dt) for x in (qb, kb, vb))
    O, L = fa.fwd(qd, kd, vd, scale=scale, window=(left, right), mask=Mt)
    return qb, kb, vb, M, Mt, qd, kd, vd, O, L, scale


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dt,left,right,kind,mdt,Bm,Hm,pad", FWD_CASES)
def test_fwd_float_mask_parity(B, Hq, Hkv, Nq, Nk, d, dt, left, right, kind, mdt, Bm, Hm, pad):
    label = (f"fa_fwd_float_mask B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dt} band=({left},{right}) "
             f"{kind} {mdt} mask[{Bm},{Hm}] pad={pad}")
    print(f"[gpu] {label}", flush=True)
    qb, kb, vb, M, _, _, _, _, O, L, scale = run_forward(B, Hq, Hkv, Nq, Nk, d, dt, left, right, kind, mdt, Bm,
                                                         Hm, pad, seed=4000 + Nq + d)
    torch.cuda.synchronize()
    O = O.cpu().numpy().astype(np.float64)
    L = L.cpu().numpy().astype(np.float64)
    q, k, v = (I.bits_to_f64(x, dt) for x in (qb, kb, vb))
    s = I.scale_f32(scale)
    G = Hq // Hkv
    worst = 0.0
    for b in range(B):
        for h in range(Hq):
            Mp = plane(M, b, h)
            kk, vv = k[b, h // G], v[b, h // G]
            O_ref, L_ref = head_attention_additive_fp64(q[b, h], kk, vv, s, left, right, Nk - Nq, Mp)
            empty = np.isneginf(L_ref)
            assert (np.isneginf(L[b, h]) == empty).all(), f"{label}: rows without keys differ"
            assert (O[b, h][empty] == 0).all()
            seen = ~empty
            vis = band_visible(np.arange(Nq), np.arange(Nk), left, right, Nk - Nq) & np.isfinite(Mp)
            sS = s * (q[b, h] @ kk.T)
            Lz = np.where(seen, L_ref, 0.0)
            keep = vis & seen[:, None]
            P = np.where(keep, np.exp(np.where(keep, sS + np.where(vis, Mp, 0.0) - Lz[:, None], -np.inf)), 0.0)
            eps = 4 * E32 * (np.abs(sS) + np.where(vis, np.abs(Mp), 0.0) + np.abs(Lz)[:, None])
            if seen.any():
                err_l = np.abs(L[b, h][seen] - L_ref[seen])
                bar_l = TOL_LSE * np.maximum(1.0, np.abs(L_ref[seen])) + (P * eps).sum(axis=1)[seen]
                assert (err_l <= bar_l).all(), f"{label}: LSE error / bar {(err_l / bar_l).max():.3f}"
            dev = np.stack([(P * eps)[i] @ np.abs(vv - O_ref[i]) for i in range(Nq)])
            bar = TOL_O[dt] * np.maximum(1.0, P @ np.abs(vv) + np.abs(O_ref)) + dev
            ratio = (np.abs(O[b, h] - O_ref) / bar).max()
            worst = max(worst, ratio)
            assert ratio <= 1.0, f"{label}: plane ({b}, {h}) error / bar = {ratio:.3f}"
    print(f"[gpu]   worst error / bar {worst:.3f}", flush=True)


def test_zero_mask_equals_no_mask_and_neg_inf_equals_byte_mask():
    """A zero float mask gives the unmasked result; a {0, -inf} mask gives the byte mask's: equal
    up to rounding order (the additive-mask kernel takes 32-key steps where the others take 64),
    within the forward's fp16 bar on O and 1e-5 on the LSE; the rows with no visible key agree
    exactly."""
    B, Hq, Hkv, N, d, dt = 1, 2, 1, 300, 64, I.F16
    g = np.random.Generator(np.random.PCG64(4100))
    qd, kd, vd = (to_dev(I.to_bits(g.standard_normal((B, h, N, d), dtype=np.float32), dt), dt)
                  for h in (Hq, Hkv, Hkv))
    print("[gpu] fa_fwd_float_mask zero and {0,-inf} masks", flush=True)
    zero = torch.zeros((1, 1, N, N), dtype=torch.float16, device=DEV)
    O0, L0 = fa.fwd(qd, kd, vd, causal=True)
    Oz, Lz = fa.fwd(qd, kd, vd, causal=True, mask=zero)
    hid = torch.from_numpy(g.random((1, Hq, N, N)) < 0.3)
    hid_pad = torch.zeros((1, Hq, N, N + 4), dtype=torch.uint8)
    hid_pad[..., :N] = hid.to(torch.uint8)
    Ob, Lb = fa.fwd(qd, kd, vd, causal=True, mask=hid_pad.to(DEV)[..., :N], splits=1)
    ninf = torch.where(hid, torch.tensor(float("-inf")), torch.tensor(0.0)).to(torch.float32).to(DEV)
    Of, Lf = fa.fwd(qd, kd, vd, causal=True, mask=ninf)
    torch.cuda.synchronize()
    assert (Oz - O0).abs().max().item() <= TOL_O[dt] and (Lz - L0).abs().max().item() <= 1e-5
    assert (Of - Ob).abs().max().item() <= TOL_O[dt] and torch.equal(torch.isinf(Lf), torch.isinf(Lb))
    fin = torch.isfinite(Lb)
    assert (Lf[fin] - Lb[fin]).abs().max().item() <= 1e-5
    assert (Of[~fin.unsqueeze(-1).expand_as(Of)] == 0).all()


BWD_CASES = [  # (B, Hq, Hkv, Nq, Nk, d, dt, left, right, kind, mdt, Bm, Hm, pad)
    (1, 2, 1, 257, 257, 64, I.F16, None, 0, "random", "f16", 1, 2, 3),
    (2, 4, 2, 200, 200, 128, I.BF16, None, None, "alibi", "f32", 1, 4, 4),
    (1, 2, 2, 129, 300, 96, I.F16, None, 0, "far", "f32", 1, 1, 0),
    (1, 4, 1, 300, 190, 48, I.BF16, 50, 10, "random", "f32", 1, 4, 2),
    (1, 2, 1, 65, 65, 32, I.F16, None, None, "random", "f16", 1, 1, 3),
    (1, 2, 1, 300, 300, 112, I.BF16, 64, 0, "alibi", "f16", 1, 2, 0),
    (1, 2, 2, 200, 200, 80, I.F16, None, None, "far", "f16", 1, 2, 0),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dt,left,right,kind,mdt,Bm,Hm,pad", BWD_CASES)
def test_float_mask_forward_then_backward(B, Hq, Hkv, Nq, Nk, d, dt, left, right, kind, mdt, Bm, Hm, pad):
    """End to end: the GPU forward's O and LSE feed fa_bwd_float_mask, against the oracle's gradients."""
    label = (f"fa_bwd_float_mask B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dt} band=({left},{right}) "
             f"{kind} {mdt}")
    print(f"[gpu] {label}", flush=True)
    seed = 4200 + Nq + d
    qb, kb, vb, M, Mt, qd, kd, vd, O, L, scale = run_forward(B, Hq, Hkv, Nq, Nk, d, dt, left, right, kind, mdt, Bm,
                                                             Hm, pad, seed)
    g = np.random.Generator(np.random.PCG64(seed + 7))
    dob = I.to_bits(g.standard_normal((B, Hq, Nq, d), dtype=np.float32), dt)
    dq, dk, dv = fa.bwd(qd, kd, vd, O, L, to_dev(dob, dt), scale=scale, window=(left, right), mask=Mt)
    torch.cuda.synchronize()
    q, k, v, do = (I.bits_to_f64(x, dt) for x in (qb, kb, vb, dob))
    s = I.scale_f32(scale)
    G = Hq // Hkv
    ref = [np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)]
    for b in range(B):
        for h in range(Hq):
            a, c, e = head_attention_bwd_additive_fp64(q[b, h], k[b, h // G], v[b, h // G], do[b, h], s, left, right,
                                                       Nk - Nq, plane(M, b, h))
            ref[0][b, h] = a
            ref[1][b, h // G] += c
            ref[2][b, h // G] += e
    got = [t.cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]
    mags = bwd_check.magnitudes(q, k, v, do, s, band=(left, right), add=M)
    # the largest exponent error over the visible pairs (module doc)
    amax = 0.0
    for b in range(B):
        for h in range(Hq):
            _, Lr = head_attention_additive_fp64(q[b, h], k[b, h // G], v[b, h // G], s, left, right, Nk - Nq,
                                                 plane(M, b, h))
            Mp = plane(M, b, h)
            vis = band_visible(np.arange(Nq), np.arange(Nk), left, right, Nk - Nq) & np.isfinite(Mp)
            a = np.abs(s * (q[b, h] @ k[b, h // G].T)) + np.where(vis, np.abs(Mp), 0.0) \
                + np.where(np.isfinite(Lr), np.abs(Lr), 0.0)[:, None]
            amax = max(amax, float(np.where(vis, a, 0.0).max()))
    bwd_check.check(label, got, ref, mags, dt, d, Nk, G * Nq, extra_rel=2 * 4 * E32 * amax)


def test_alibi_at_a_benchmark_shape_sampled_rows():
    """fa_fwd_float_mask on the full-size causal N = 8192 workload (B=4, H=48, d=64, fp16) with an
    fp16 distance bias -2^-3 |i - j| shared by the heads (the bench.py --variant alibi form):
    sampled rows of four heads against the oracle."""
    w = I.WORKLOADS["causal_b4_h48_n8192_d64_f16"]
    print(f"[gpu] fa_fwd_float_mask {w.name} alibi", flush=True)
    qkv = I.workload_qkv(w)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (qkv.q, qkv.k, qkv.v))
    i = torch.arange(w.N, device=DEV, dtype=torch.float32)[:, None]
    j = torch.arange(w.N, device=DEV, dtype=torch.float32)[None, :]
    Mt = (-0.125 * (i - j).abs()).to(torch.float16)[None, None].contiguous()
    O, L = fa.fwd(qd, kd, vd, scale=w.scale, causal=True, mask=Mt)
    torch.cuda.synchronize()
    O = O.cpu().numpy()
    L = L.cpu().numpy()
    s = I.scale_f32(w.scale)
    rng = np.random.default_rng(w.seed + 5)
    rows = np.array(sorted({0, 1, 127, 128, 4095, w.N - 1} | {int(x) for x in rng.integers(0, w.N, 12)}))
    M = Mt[0, 0][torch.from_numpy(rows).to(DEV)].to(torch.float64).cpu().numpy()
    worst = 0.0
    for b, h in [(0, 0), (1, 5), (2, 24), (3, 47)]:
        k = I.bits_to_f64(qkv.k[b, h], w.dtype)
        v = I.bits_to_f64(qkv.v[b, h], w.dtype)
        for n, r in enumerate(rows):
            q = I.bits_to_f64(qkv.q[b, h, r:r + 1], w.dtype)
            O_ref, L_ref = head_attention_additive_fp64(q, k, v, s, None, 0, int(r), M[n:n + 1])
            vis = np.arange(w.N) <= r
            sS = s * (q @ k.T)[0]
            P = np.where(vis, np.exp(np.where(vis, sS + M[n] - L_ref[0], -np.inf)), 0.0)
            eps = 4 * E32 * (np.abs(sS) + np.abs(M[n]) + abs(L_ref[0]))
            assert abs(L[b, h, r] - L_ref[0]) <= TOL_LSE * max(1.0, abs(L_ref[0])) + (P * eps).sum()
            bar = TOL_O[w.dtype] * np.maximum(1.0, P @ np.abs(v) + np.abs(O_ref[0])) + (P * eps) @ np.abs(v - O_ref[0])
            ratio = (np.abs(O[b, h, r] - O_ref[0]) / bar).max()
            worst = max(worst, ratio)
            assert ratio <= 1.0, f"row ({b}, {h}, {r}): error / bar {ratio:.3f}"
    print(f"[gpu]   worst error / bar {worst:.3f}", flush=True)
