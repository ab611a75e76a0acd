"""Host checks of the seeded input module: storage rounding and the workloads' FLOP counts.

  * bf16 and fp16 rounding agree bit for bit with torch's own conversions (round to
    nearest, ties to even), on random values and on ties, extremes and subnormals;
  * each workload's algorithmic FLOP count equals 4 d times the number of visible
    (query, key) pairs counted by brute force over the band on a scaled-down copy.
"""
import dataclasses

import numpy as np
import pytest
import torch

from exact_attention_114_amd import inputs as I


def edge_values():
    g = np.random.Generator(np.random.PCG64(3))
    x = g.standard_normal(20000, dtype=np.float32) * np.float32(5)
    # ties at bf16 precision (low 16 bits exactly 0x8000) on even and odd mantissas
    ties = (np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7F8000], dtype=np.uint32)).view(np.float32)
    extremes = np.array([3.4028235e38, -3.4028235e38, 1e-45, -1e-45, 0.0, -0.0, 1.1754944e-38,
                         65504.0, 65520.0, 6e-8, 1.00390625], dtype=np.float32)
    return np.concatenate([x, ties, extremes])


def test_bf16_rounding_matches_torch():
    x = edge_values()
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(I.f32_to_bf16_bits(x), want)


def test_bf16_rounding_rejects_non_finite():
    with pytest.raises(ValueError):
        I.f32_to_bf16_bits(np.array([1.0, np.nan], dtype=np.float32))


def test_f16_rounding_matches_torch():
    x = edge_values()
    x = x[np.abs(x) < 65520.0]  # beyond this fp16 overflows to inf
    want = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(I.f32_to_f16_bits(x), want)


def visible_pairs(nq, nk, causal, left):
    off = nk - nq
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    vis = np.ones((nq, nk), dtype=bool)
    if causal:
        vis &= j <= i + off
    if left is not None:
        vis &= j >= i + off - left
    return int(vis.sum())


@pytest.mark.parametrize("name", list(I.WORKLOADS))
def test_workload_flops_count_visible_pairs(name):
    w = I.WORKLOADS[name]
    # scale lengths down by a power of two so brute force stays small; counts scale exactly
    # for the banded and separate-length forms, and by n^2 (less the diagonal's half) otherwise
    f = max(1, max(w.N, w.nk) // 512)
    small = dataclasses.replace(w, N=w.N // f, n_keys=None if w.n_keys is None else w.nk // f,
                                window_left=None if w.window_left is None else w.window_left // f)
    pairs = visible_pairs(small.N, small.nk, small.causal, small.window_left)
    exact = 4.0 * small.B * small.Hq * small.d * pairs
    if small.causal and small.window_left is None and small.nk == small.N:
        # causal square: the count is N^2/2 by convention, the exact pairs add N/2
        assert small.flops == pytest.approx(exact - 2.0 * small.B * small.Hq * small.d * small.N, rel=1e-12)
    else:
        assert small.flops == pytest.approx(exact, rel=1e-12)


def test_chunk_workload_shapes():
    w = I.WORKLOADS["chunk_causal_b1_hq32_hkv8_nq512_nk32768_d128_bf16"]
    assert w.q_shape() == (1, 32, 512, 128) and w.kv_shape() == (1, 8, 32768, 128)
    qkv = I.draw_qkv(1, 2, 1, 8, 4, I.BF16, 5, Nk=24)
    assert qkv.q.shape == (1, 2, 8, 4) and qkv.k.shape == (1, 1, 24, 4) and qkv.v.shape == (1, 1, 24, 4)


def test_document_lengths_and_mask():
    """Packed documents: lengths drawn in [min, max] (the last one cut), summing to N per
    sequence, reproducible from the seed; the mask is block diagonal over them (0 inside a
    document, 1 across documents) and shared by the heads."""
    lens = I.document_lengths(3, 1000, 17, 100, 400)
    assert lens == I.document_lengths(3, 1000, 17, 100, 400)
    assert lens != I.document_lengths(3, 1000, 18, 100, 400)
    for row in lens:
        assert sum(row) == 1000
        assert all(100 <= n <= 400 for n in row[:-1]) and 1 <= row[-1] <= 400
    m = I.document_mask(lens, 1000)
    assert m.shape == (3, 1, 1000, 1000) and m.dtype == np.uint8
    for b, row in enumerate(lens):
        doc = np.repeat(np.arange(len(row)), row)  # document of each position
        expect = (doc[:, None] != doc[None, :]).astype(np.uint8)
        assert np.array_equal(m[b, 0], expect)
