"""GPU parity of the mask input (fa_fwd_mask): a byte mask whose nonzero entries hide keys, on
top of the band, shared across batch elements or heads when its axis has size 1.

Bars as for the forward: O within 2e-3 (fp16) or 1e-2 (bf16) of the fp64 oracle, LSE within
1e-4 relative with a floor of 1, rows the mask hides completely exactly O = 0 and LSE = -inf.
Masks: random (independent bytes), block-structured (whole tiles hidden or kept, which takes
the kernel's skip path and can leave a row's first tiles empty), and key padding.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_114_amd as fa
from exact_attention_114_amd import binding as bnd
from exact_attention_114_amd import inputs as I
from oracle.attention import attention_band_fp64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_O = {I.F16: 2e-3, I.BF16: 1e-2}
TOL_LSE = 1e-4


def to_dev(bits, dt):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dt == I.F16 else torch.bfloat16).to(DEV)


def draw(B, Hq, Hkv, Nq, Nk, d, dt, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return tuple(I.to_bits(g.standard_normal(s, dtype=np.float32), dt)
                 for s in ((B, Hq, Nq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d)))


def make_mask(kind, shape, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    Bm, Hm, Nq, Nk = shape
    if kind == "random":
        m = (g.random(shape) < 0.3).astype(np.uint8)
    elif kind == "blocks":
        # 32 x 32 blocks hidden or kept as wholes, plus a few single bytes
        blk = (g.random((Bm, Hm, (Nq + 31) // 32, (Nk + 31) // 32)) < 0.5).astype(np.uint8)
        m = np.repeat(np.repeat(blk, 32, axis=2), 32, axis=3)[:, :, :Nq, :Nk].copy()
        m[..., g.integers(0, Nq, 8), g.integers(0, Nk, 8)] ^= 1
    else:  # key padding: element b keeps its first len_b keys
        lens = g.integers(1, Nk + 1, Bm)
        m = np.broadcast_to((np.arange(Nk)[None, None, None, :] >= lens[:, None, None, None]),
                            shape).astype(np.uint8).copy()
    return m


def mask_to_dev(mask):
    """The mask on the GPU with its rows padded to a multiple of 4 bytes, passed as a view."""
    Nk = mask.shape[-1]
    padded = np.ones(mask.shape[:-1] + ((Nk + 3) // 4 * 4,), np.uint8)
    padded[..., :Nk] = mask
    return torch.from_numpy(padded).to(DEV)[..., :Nk]


def run(B, Hq, Hkv, Nq, Nk, d, dt, band, mask, seed, splits=None, out16=False, values=None):
    qb, kb, vb = draw(B, Hq, Hkv, Nq, Nk, d, dt, seed) if values is None else values
    scale = 1.0 / math.sqrt(d)
    print(f"[gpu] fa_fwd_mask B={B} Hq={Hq} Nq={Nq} Nk={Nk} d={d} {dt} band={band} mask={mask.shape} "
          f"splits={splits}", flush=True)
    out_dtype = (torch.float16 if dt == I.F16 else torch.bfloat16) if out16 else torch.float32
    tm = mask_to_dev(mask)
    O, L = fa.fwd(to_dev(qb, dt), to_dev(kb, dt), to_dev(vb, dt), scale=scale, window=band, mask=tm,
                  splits=splits, out_dtype=out_dtype)
    torch.cuda.synchronize()
    q, k, v = (I.bits_to_f64(x, dt) for x in (qb, kb, vb))
    O_ref, L_ref = attention_band_fp64(q, k, v, I.scale_f32(scale), *band, mask=mask)
    O = O.float().cpu().numpy().astype(np.float64)
    L = L.cpu().numpy().astype(np.float64)
    empty = np.isneginf(L_ref)
    assert (np.isneginf(L) == empty).all() and (O[empty] == 0).all()
    bar = TOL_O[dt]
    if out16:
        bits = I.to_bits(np.abs(O_ref).astype(np.float32), dt)
        bar = bar + 0.5 * (I.bits_to_f64(bits + np.uint16(1), dt) - I.bits_to_f64(bits, dt))
    assert (np.abs(O - O_ref) <= bar).all(), f"max|dO| {np.abs(O - O_ref).max():.3e}"
    seen = ~empty
    if seen.any():
        err = (np.abs(L[seen] - L_ref[seen]) / np.maximum(1.0, np.abs(L_ref[seen]))).max()
        assert err <= TOL_LSE, f"LSE rel err {err:.3e}"
    return O, L


@pytest.mark.parametrize("kind", ["random", "blocks", "padding"])
@pytest.mark.parametrize("mshape", ["shared", "batch", "full"])
@pytest.mark.parametrize("d,dt", [(64, I.F16), (128, I.BF16)])
def test_mask_kinds_and_broadcast(kind, mshape, d, dt):
    B, Hq, Hkv, Nq, Nk = 2, 4, 2, 200, 264
    Bm, Hm = {"shared": (1, 1), "batch": (B, 1), "full": (B, Hq)}[mshape]
    mask = make_mask(kind, (Bm, Hm, Nq, Nk), 1500 + d)
    run(B, Hq, Hkv, Nq, Nk, d, dt, (None, None), mask, 1510 + d)


@pytest.mark.parametrize("band", [(None, 0), (40, 0), (30, 20)])
@pytest.mark.parametrize("d,dt", [(64, I.BF16), (128, I.F16), (96, I.BF16), (32, I.F16)])
def test_mask_with_band(band, d, dt):
    mask = make_mask("random", (1, 1, 150, 150), 1520 + d)
    run(1, 4, 4, 150, 150, d, dt, band, mask, 1530 + d)


@pytest.mark.parametrize("d", [64, 128])
def test_mask_large_grid_and_rows_hidden(d):
    """Above 512 work-groups (32-key steps at d = 128); some rows hidden completely."""
    B, Hq, Hkv, N = 2, 16, 4, 2100
    mask = make_mask("blocks", (B, 1, N, N), 1540 + d)
    mask[:, :, 5] = 1
    mask[:, :, 1000:1003] = 1
    O, L = run(B, Hq, Hkv, N, N, d, I.BF16, (None, 0), mask, 1550 + d)
    assert np.isneginf(L[:, :, 5]).all()


def test_causal_mask_equals_causal_flag_bitwise():
    qb, kb, vb = draw(2, 4, 2, 333, 333, 128, I.BF16, 1560)
    q, k, v = (to_dev(x, I.BF16) for x in (qb, kb, vb))
    i = np.arange(333)
    causal = (i[None, :] > i[:, None]).astype(np.uint8)[None, None]
    a = fa.fwd(q, k, v, causal=True)
    # 333 keys is not a multiple of 4: pad the mask's rows and pass a view
    padded = np.ones((1, 1, 333, 336), np.uint8)
    padded[..., :333] = causal
    b = fa.fwd(q, k, v, mask=torch.from_numpy(padded).to(DEV)[..., :333])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_zero_mask_equals_no_mask_bitwise():
    qb, kb, vb = draw(1, 8, 2, 300, 512, 64, I.F16, 1570)
    q, k, v = (to_dev(x, I.F16) for x in (qb, kb, vb))
    a = fa.fwd(q, k, v, window=(100, 0))
    b = fa.fwd(q, k, v, window=(100, 0), mask=torch.zeros(1, 1, 300, 512, dtype=torch.bool, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("splits", [0, 3])
def test_mask_with_split_keys(splits):
    mask = make_mask("random", (1, 1, 100, 3000), 1580)
    run(1, 4, 2, 100, 3000, 128, I.BF16, (None, 0), mask, 1581, splits=splits)
    run(1, 2, 2, 70, 2000, 64, I.F16, (None, None), make_mask("padding", (1, 2, 70, 2000), 1582)[:1], 1583,
        splits=splits, out16=True)


def test_mask_rescale_path():
    """Scores that rise along the keys force the reference to move; the mask hides some of the
    tiles where it would move (the rare path reloads the tile's mask)."""
    B, Hq, Hkv, N, d, dt = 1, 4, 2, 333, 64, I.F16
    g = np.random.Generator(np.random.PCG64(1590))
    q = g.standard_normal((B, Hq, N, d), dtype=np.float32) + np.float32(1.0)
    k = g.standard_normal((B, Hkv, N, d), dtype=np.float32)
    k += (np.float32(3.0) * np.arange(N, dtype=np.float32) / np.float32(N))[:, None]
    k[:, :, N - 5, :] = np.float32(16.0)
    v = g.standard_normal((B, Hkv, N, d), dtype=np.float32)
    values = tuple(I.to_bits(x, dt) for x in (q, k, v))
    mask = make_mask("random", (1, 1, N, N), 1591)
    mask[..., N - 5] = 0  # the spike stays visible: it moves the reference on the last tiles
    run(B, Hq, Hkv, N, N, d, dt, (None, None), mask, 0, values=values)


# ---------------------------------------------------------------- the mask's key hull
# The pre-pass records, per Q-tile and 1024 keys, the first and last key some row may see, and
# the attention kernel skips the tiles outside. Document masks (packed sequences: a query sees
# only its own document) hide most tiles from every row of a Q-tile; key padding hides a tail.


@pytest.mark.parametrize("band", [(None, 0), (None, None), (700, 0)])
@pytest.mark.parametrize("d,dt", [(64, I.F16), (128, I.BF16)])
def test_document_mask_skips_tiles(band, d, dt):
    """Documents of 37..1200 tokens in sequences of 2500 (three hull chunks, a ragged end)."""
    B, Hq, Hkv, N = 2, 4, 2, 2500
    lens = I.document_lengths(B, N, 1600 + d, 37, 1200)
    mask = I.document_mask(lens, N)
    run(B, Hq, Hkv, N, N, d, dt, band, mask, 1610 + d)


def test_document_mask_per_head_and_split():
    """A plane per (batch, head): each head packs its own documents; with and without split keys,
    and Nq < Nk (the queries are the last rows of the sequence)."""
    B, Hq, Hkv, Nq, Nk = 2, 3, 3, 300, 2600
    planes = [I.document_mask(I.document_lengths(1, Nk, 1620 + i, 50, 900), Nk)[0, 0, Nk - Nq:]
              for i in range(B * Hq)]
    mask = np.stack(planes).reshape(B, Hq, Nq, Nk)
    for splits in (None, 0, 3):
        run(B, Hq, Hkv, Nq, Nk, 64, I.F16, (None, 0), mask, 1630, splits=splits)


def test_mask_hides_whole_q_tiles():
    """Q-tiles whose rows see nothing (mask rows all ones) write O = 0, LSE = -inf; a padding
    mask hides every key past each sequence's length."""
    B, Hq, Hkv, N = 2, 2, 1, 700
    mask = make_mask("padding", (B, 1, N, N), 1640)
    mask[0, 0, 128:256] = 1  # the second Q-tile of batch 0 sees no key
    O, L = run(B, Hq, Hkv, N, N, 128, I.BF16, (None, None), mask, 1641)
    assert np.isneginf(L[0, :, 128:256]).all() and (O[0, :, 128:256] == 0).all()


def test_document_mask_gqa_workload_sampled_rows():
    """The GQA workload at full size with the document mask the benchmark uses (bench.py
    --mask document), on rows the oracle computes one by one."""
    from oracle.attention import head_attention_band_fp64

    w = I.WORKLOADS["gqa_causal_b4_hq32_hkv8_n8192_d128_bf16"]
    lens = I.document_lengths(w.B, w.N, w.seed + 2000, w.N // 8, w.N // 2)
    mask = I.document_mask(lens, w.N)
    qkv = I.workload_qkv(w)
    print(f"[gpu] fa_fwd_mask {w.name} document mask {[len(r) for r in lens]}", flush=True)
    O, L = fa.fwd(*(to_dev(x, w.dtype) for x in (qkv.q, qkv.k, qkv.v)), scale=w.scale, window=w.band,
                  mask=torch.from_numpy(mask).to(DEV))
    torch.cuda.synchronize()
    O = O.cpu().numpy().astype(np.float64)
    L = L.cpu().numpy().astype(np.float64)
    rng = np.random.Generator(np.random.PCG64(1650))
    starts = np.cumsum([0] + lens[0][:-1])
    rows = np.unique(np.concatenate([starts, starts + 1, starts - 1, [w.N - 1], rng.integers(0, w.N, 24)]))
    rows = rows[(rows >= 0) & (rows < w.N)]
    for b, h in [(0, 0), (0, 5), (3, 31)]:
        if b != 0:
            starts = np.cumsum([0] + lens[b][:-1])
            rows = np.unique(np.concatenate([starts, starts + 1, rng.integers(0, w.N, 24)]))
            rows = rows[(rows >= 0) & (rows < w.N)]
        q = I.bits_to_f64(qkv.q[b, h][rows], w.dtype)
        k = I.bits_to_f64(qkv.k[b, h // (w.Hq // w.Hkv)], w.dtype)
        v = I.bits_to_f64(qkv.v[b, h // (w.Hq // w.Hkv)], w.dtype)
        O_ref, L_ref = head_attention_band_fp64(q, k, v, I.scale_f32(w.scale), None, 0, q_pos=rows,
                                                hidden=mask[b, 0][rows])
        err_o = np.abs(O[b, h][rows] - O_ref).max()
        assert err_o <= TOL_O[w.dtype], f"head ({b},{h}) max|dO| {err_o:.3e}"
        err_l = (np.abs(L[b, h][rows] - L_ref) / np.maximum(1.0, np.abs(L_ref))).max()
        assert err_l <= TOL_LSE, f"head ({b},{h}) LSE rel err {err_l:.3e}"


def test_mask_errors_raise():
    qb, kb, vb = draw(1, 2, 2, 64, 30, 64, I.F16, 1595)
    q, k, v = (to_dev(x, I.F16) for x in (qb, kb, vb))
    with pytest.raises(bnd.FaError):  # 30 keys: row stride 30 is not a multiple of 4
        fa.fwd(q, k, v, mask=torch.zeros(1, 1, 64, 30, dtype=torch.bool, device=DEV))
    with pytest.raises(bnd.FaError):
        fa.fwd(q, k, v, mask=torch.zeros(1, 3, 64, 32, dtype=torch.bool, device=DEV)[..., :30])


# ---------------------------------------------------------------- gradients

def run_bwd(B, Hq, Hkv, Nq, Nk, d, dt, band, mask, seed):
    """fa_bwd_mask against the fp64 gradients, within the bar of the unmasked backward tests
    (bwd_check.py)."""
    import bwd_check
    from oracle.backward import attention_bwd_band_fp64

    g = np.random.Generator(np.random.PCG64(seed))
    qb, kb, vb, dob = (I.to_bits(g.standard_normal(s, dtype=np.float32), dt)
                       for s in ((B, Hq, Nq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d), (B, Hq, Nq, d)))
    scale = 1.0 / math.sqrt(d)
    sc = I.scale_f32(scale)
    q, k, v, do = (I.bits_to_f64(x, dt) for x in (qb, kb, vb, dob))
    O, L = attention_band_fp64(q, k, v, sc, *band, mask=mask)
    o32 = O.astype(np.float32)
    print(f"[gpu] fa_bwd_mask B={B} Hq={Hq} Nq={Nq} Nk={Nk} d={d} {dt} band={band} mask={mask.shape}", flush=True)
    grads = fa.bwd(to_dev(qb, dt), to_dev(kb, dt), to_dev(vb, dt), torch.from_numpy(o32).to(DEV),
                   torch.from_numpy(L.astype(np.float32)).to(DEV), to_dev(dob, dt), scale=scale, window=band,
                   mask=mask_to_dev(mask))
    torch.cuda.synchronize()
    got = [t.cpu().numpy().astype(np.float64) for t in grads]
    ref = attention_bwd_band_fp64(q, k, v, do, sc, *band, mask=mask)
    mags = bwd_check.magnitudes(q, k, v, do, sc, band=band, mask=mask)
    bwd_check.check(f"mask B={B} Hq={Hq} Nq={Nq} Nk={Nk} d={d} {dt} band={band}", got, ref, mags, dt, d, Nk,
                    (Hq // Hkv) * Nq)


@pytest.mark.parametrize("kind", ["random", "blocks", "padding"])
@pytest.mark.parametrize("d,dt", [(64, I.F16), (128, I.BF16), (96, I.BF16), (32, I.F16)])
def test_bwd_mask_kinds(kind, d, dt):
    mask = make_mask(kind, (2, 1, 150, 260), 1600 + d)
    run_bwd(2, 4, 2, 150, 260, d, dt, (None, None), mask, 1610 + d)


@pytest.mark.parametrize("band", [(None, 0), (40, 10)])
@pytest.mark.parametrize("d,dt", [(64, I.BF16), (128, I.F16)])
def test_bwd_mask_with_band_and_hidden_rows(band, d, dt):
    mask = make_mask("random", (1, 4, 200, 200), 1620 + d)
    mask[:, 1, 7] = 1
    run_bwd(1, 4, 2, 200, 200, d, dt, band, mask, 1630 + d)


# ---------------------------------------------------------------- backward over the mask's summaries
# fa_bwd_mask runs the same pre-pass: the dQ kernel reads the packed bits and stays inside each
# Q-tile's key hull, and the dK/dV kernel visits only the Q-tiles flagged for its key tile.


@pytest.mark.parametrize("band", [(None, 0), (None, None)])
@pytest.mark.parametrize("d,dt", [(64, I.F16), (128, I.BF16)])
def test_bwd_document_mask(band, d, dt):
    """Documents of 37..600 tokens in sequences of 1300 (two hull chunks, a ragged end)."""
    B, Hq, Hkv, N = 2, 4, 2, 1300
    mask = I.document_mask(I.document_lengths(B, N, 1700 + d, 37, 600), N)
    run_bwd(B, Hq, Hkv, N, N, d, dt, band, mask, 1710 + d)


def test_bwd_document_mask_per_head_planes():
    """A plane per (batch, head), GQA 2:1 (the dK/dV flags are merged over the sibling heads),
    Nq < Nk."""
    B, Hq, Hkv, Nq, Nk = 1, 4, 2, 300, 1100
    planes = [I.document_mask(I.document_lengths(1, Nk, 1720 + i, 40, 500), Nk)[0, 0, Nk - Nq:]
              for i in range(B * Hq)]
    run_bwd(B, Hq, Hkv, Nq, Nk, 64, I.BF16, (None, 0), np.stack(planes).reshape(B, Hq, Nq, Nk), 1730)


def test_bwd_mask_hidden_q_tiles_and_keys():
    """A Q-tile whose rows see nothing (zero dQ) and a key range no query sees (zero dK, dV)."""
    B, Hq, Hkv, N = 1, 2, 1, 700
    mask = np.zeros((1, 1, N, N), np.uint8)
    mask[..., 128:256, :] = 1   # rows of the second Q-tile see nothing
    mask[..., 384:640] = 1      # keys 384..639 are hidden from every query
    run_bwd(B, Hq, Hkv, N, N, 128, I.F16, (None, None), mask, 1740)


@pytest.mark.parametrize("nq,nk", [(1, 1), (3, 7), (1, 33), (5, 1024), (130, 1025), (64, 2048)])
def test_mask_small_and_chunk_edges(nq, nk):
    """Tiny and ragged key counts and Nk on the 1024-key chunk edge (forward, causal and not)."""
    for band in ((None, None), (None, 0)):
        run(1, 2, 1, nq, nk, 64, I.F16, band, make_mask("random", (1, 2, nq, nk), 1750 + nk), 1760 + nk)


def test_mask_all_hidden_forward_and_backward():
    """Every key hidden: O = 0 and LSE = -inf for every row, and all three gradients zero."""
    B, Hq, Hkv, N, d = 1, 2, 1, 300, 128
    mask = np.ones((1, 1, N, N), np.uint8)
    O, L = run(B, Hq, Hkv, N, N, d, I.BF16, (None, None), mask, 1770)
    assert np.isneginf(L).all() and (O == 0).all()
    run_bwd(B, Hq, Hkv, N, N, d, I.BF16, (None, None), mask, 1771)
