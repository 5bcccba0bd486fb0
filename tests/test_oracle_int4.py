"""Pins of the oracle's INT4 weight-only GEMV (oracle_int4_gemv) to values
fixed by hand and by a dense fp64 matrix product.

Format read from the pages' INT4 decode passages (which fix no layout):
two's-complement 4-bit codes, eight per uint32 along k (code j in bits
4j..4j+3 is element 8*word + j), one bf16 scale per `group` consecutive k
of each output row, bf16 activations.
"""
import numpy as np
import pytest

import oracle
import synth

# two's complement of the 16 four-bit patterns, written out
SIGNED = [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]


def _bf(vals):
    return synth.bf16_from_f32(np.asarray(vals, np.float32))


def test_hand_example_sum_of_squares():
    """word 0x89ABCDEF holds codes -1..-8 at positions 0..7; with x = 1..8
    and scale 0.5 the output is -0.5 * (1 + 4 + ... + 64) = -102."""
    x = _bf([[1, 2, 3, 4, 5, 6, 7, 8]])
    w = np.array([[0x89ABCDEF]], np.uint32)
    s = _bf([[0.5]])
    y, ya = oracle.int4_gemv(x, w, s, group=8)
    assert y[0, 0] == -102.0 and ya[0, 0] == 102.0


@pytest.mark.parametrize("j", range(8))
def test_code_position_and_sign(j):
    """Every 4-bit pattern u at every position j of a word: a one-hot x at
    element j reads back SIGNED[u] times the scale."""
    x = np.zeros((1, 8), np.float32)
    x[0, j] = 1.0
    for u in range(16):
        w = np.array([[u << (4 * j)]], np.uint32)
        y, _ = oracle.int4_gemv(_bf(x), w, _bf([[0.25]]), group=8)
        assert y[0, 0] == SIGNED[u] * 0.25, (j, u)


def test_group_scale_mapping():
    """k = 384 in groups of 128 with scales 1, 2, 4: one-hot x at the edges
    of each group picks the code times that group's scale."""
    k = 384
    w = np.full((1, k // 8), 0x33333333, np.uint32)   # every code 3
    s = _bf([[1.0, 2.0, 4.0]])
    for kk, sc in [(0, 1), (127, 1), (128, 2), (255, 2), (256, 4), (383, 4)]:
        x = np.zeros((1, k), np.float32)
        x[0, kk] = 1.0
        y, _ = oracle.int4_gemv(_bf(x), w, s, group=128)
        assert y[0, 0] == 3 * sc, kk


def _dense(w, s, group):
    """Independent dense decode: nibbles by shift-and-mask over a new axis,
    sign by subtracting 16 where the top bit is set."""
    n, kw = w.shape
    nib = (w[:, :, None] >> (4 * np.arange(8, dtype=np.uint32))[None, None, :]) & 0xF
    q = nib.astype(np.int64).reshape(n, kw * 8)
    q = q - 16 * (q >= 8)
    sc = np.repeat(synth.bf16_to_f32(s).astype(np.float64), group, axis=1)
    return q * sc


@pytest.mark.parametrize("m,n,k,group", [(1, 5, 256, 128), (3, 17, 384, 128), (8, 9, 512, 64)])
def test_matches_dense_product(m, n, k, group):
    rng = np.random.default_rng(m * 1000 + n)
    x = _bf(rng.standard_normal((m, k)))
    w = rng.integers(0, 1 << 32, (n, k // 8), dtype=np.uint64).astype(np.uint32)
    s = _bf(rng.uniform(-0.1, 0.1, (n, k // group)))
    y, ya = oracle.int4_gemv(x, w, s, group=group)
    W = _dense(w, s, group)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    ref = xf @ W.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(ya, np.abs(xf) @ np.abs(W).T, rtol=1e-12, atol=1e-12)
    # a subset of columns gives the same values and leaves the rest unset
    yc, _ = oracle.int4_gemv(x, w, s, group=group, cols=[n - 1, 0])
    assert np.array_equal(yc[:, [0, n - 1]], y[:, [0, n - 1]])
    if n > 2:
        assert np.isnan(yc[:, 1]).all()


def test_invalid_shapes():
    x = _bf(np.zeros((1, 192)))
    w = np.zeros((1, 24), np.uint32)
    with pytest.raises((ValueError, AssertionError)):
        oracle.int4_gemv(x, w, _bf(np.ones((1, 1))), group=128)
