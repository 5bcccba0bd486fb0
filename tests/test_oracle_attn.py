"""CPU pins of the oracle's paged decode attention.

What is pinned: decode attention over a paged cache equals textbook
softmax(q K̂ᵀ·sm_scale)·V̂ on unpaged copies (brute force, with torch's
independent e4m3 codec), plus the special cases that reduce to closed forms
(identical keys -> mean of values, one token -> its value, a dominant key ->
its value), invariances (physical page permutation), the abort and no-tracker
semantics (remio.ai, section "Sicherheit gemeinsamer KV-Caches wird zum
Produktionsthema": a mismatch aborts the request; a no-op tracker when the
check is disabled), and the log-sum-exp combine of split chunks.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from helpers import (dense_attention, dense_reference, dequant_dense,
                     oracle_attn, oracle_caches, slots_of, small_problem)

F32_TOL = dict(rtol=3e-7, atol=1e-30)


@pytest.mark.parametrize("kv_dtype", [synth.KV_FP8, synth.KV_BF16])
@pytest.mark.parametrize("dk,S,hq,hkv", [(16, 16, 2, 1), (32, 32, 4, 2),
                                         (128, 16, 8, 2), (128, 64, 3, 3)])
def test_p7_paged_equals_dense_bruteforce(kv_dtype, dk, S, hq, hkv):
    pr = small_problem(11 + dk + S + hq, [1, 17, 40], hq, hkv, dk, dk, S, kv_dtype)
    kc, vc, ts = oracle_caches(pr)
    got = oracle_attn(pr, kc, vc, ts)
    want = dense_reference(pr)
    np.testing.assert_allclose(got, want.astype(np.float32), **F32_TOL)


def test_p7_latent_per_token_equals_dense():
    pr = small_problem(5, [3, 64, 130], 16, 1, 48, 32, 64, synth.KV_FP8, latent=True)
    kc, vc, ts = oracle_caches(pr)
    assert vc is None
    got = oracle_attn(pr, kc, vc, ts)
    want = dense_reference(pr, ts)
    np.testing.assert_allclose(got, want.astype(np.float32), **F32_TOL)


def test_p8_identical_keys_give_mean_of_values():
    pr = small_problem(8, [37, 5], 4, 2, 32, 32, 16, synth.KV_FP8)
    for s in range(2):
        pr["ks"][s][:] = pr["ks"][s][0:1]          # every key the same
    kc, vc, ts = oracle_caches(pr)
    got = oracle_attn(pr, kc, vc, ts)
    for s in range(2):
        _, vh = dequant_dense(pr["ks"][s], pr["vs"][s], pr["k_scale"],
                              pr["v_scale"], synth.KV_FP8)
        for h in range(4):
            want = vh[:, h // 2, :].mean(axis=0)
            np.testing.assert_allclose(got[s, h], want.astype(np.float32), **F32_TOL)


@pytest.mark.parametrize("kv_dtype", [synth.KV_FP8, synth.KV_BF16])
def test_p9_single_token_returns_its_value(kv_dtype):
    pr = small_problem(9, [1, 1], 4, 2, 32, 32, 16, kv_dtype)
    kc, vc, ts = oracle_caches(pr)
    got = oracle_attn(pr, kc, vc, ts)
    for s in range(2):
        _, vh = dequant_dense(pr["ks"][s], pr["vs"][s], pr["k_scale"],
                              pr["v_scale"], kv_dtype)
        for h in range(4):
            assert np.array_equal(got[s, h], vh[0, h // 2].astype(np.float32))


@pytest.mark.parametrize("kv_dtype", [synth.KV_FP8, synth.KV_BF16])
def test_p10_physical_permutation_is_bit_identical(kv_dtype):
    pr = small_problem(10, [33, 70, 16], 8, 2, 128, 128, 16, kv_dtype, num_pages=20)
    kc, vc, ts = oracle_caches(pr)
    base = oracle_attn(pr, kc, vc, ts)
    rng = np.random.default_rng(99)
    pr2 = dict(pr)
    perm = rng.permutation(pr["P"])       # new physical home of every page
    bt2 = pr["bt"].copy()
    bt2[bt2 >= 0] = perm[bt2[bt2 >= 0]]
    pr2["bt"] = bt2
    kc2, vc2, ts2 = oracle_caches(pr2)
    moved = oracle_attn(pr2, kc2, vc2, ts2)
    assert np.array_equal(base, moved)
    assert not np.array_equal(kc, kc2)


def test_p11_dominant_key_returns_its_value():
    pr = small_problem(12, [29], 2, 1, 16, 16, 16, synth.KV_BF16)
    k = synth.bf16_to_f32(pr["ks"][0]).copy()
    k[:] = -1.0
    k[13] = 1.0                              # key 13 matches q, others oppose
    pr["ks"][0] = synth.bf16_from_f32(k)
    pr["q"][:] = synth.bf16_from_f32(np.full((1, 2, 16), 4.0, np.float32))
    kc, vc, ts = oracle_caches(pr)
    # score gap = sm_scale * 4 * 16 * 2 = 128 * sm_scale; with sm_scale 1: 128
    got = oracle_attn(pr, kc, vc, ts, sm_scale=1.0)
    v13 = synth.bf16_to_f32(pr["vs"][0][13, 0])
    for h in range(2):
        assert np.array_equal(got[0, h], v13)


def test_p12_mha_is_independent_heads():
    pr = small_problem(13, [20, 45], 3, 3, 32, 32, 16, synth.KV_FP8)
    kc, vc, ts = oracle_caches(pr)
    got = oracle_attn(pr, kc, vc, ts)
    for h in range(3):
        one = dict(pr)
        one.update(hq=1, hkv=1, q=pr["q"][:, h:h + 1].copy(),
                   ks=[k[:, h:h + 1].copy() for k in pr["ks"]],
                   vs=[v[:, h:h + 1].copy() for v in pr["vs"]],
                   k_scale=pr["k_scale"][h:h + 1].copy(),
                   v_scale=pr["v_scale"][h:h + 1].copy())
        kc1, vc1, ts1 = oracle_caches(one)
        o1 = oracle_attn(one, kc1, vc1, ts1)
        assert np.array_equal(got[:, h], o1[:, 0])


def test_p13_latent_values_are_first_dims_of_keys():
    """V-in-K: the oracle's latent output equals attention with an explicit V
    equal to the first Dv dims of each dequantised key."""
    pr = small_problem(14, [70, 9], 16, 1, 64, 48, 64, synth.KV_FP8, latent=True)
    kc, vc, ts = oracle_caches(pr)
    got = oracle_attn(pr, kc, vc, ts)
    for s in range(2):
        l = int(pr["lens"][s])
        tok = ts[slots_of(pr["bt"][s], 64, l)]
        kh, _ = dequant_dense(pr["ks"][s], None, None, None, synth.KV_FP8, tok)
        vh = kh[:, :, :48].copy()
        want = dense_attention(pr["q"][s], kh, vh, pr["sm_scale"], 16)
        np.testing.assert_allclose(got[s], want.astype(np.float32), **F32_TOL)


@pytest.mark.parametrize("kv_dtype", [synth.KV_FP8, synth.KV_BF16])
def test_p14_abort_zeroes_only_that_sequence(kv_dtype):
    pr = small_problem(15, [17, 64, 100, 255], 8, 2, 128, 128, 16, kv_dtype, num_pages=64)
    kc, vc, ts = oracle_caches(pr)
    free = oracle_attn(pr, kc, vc, ts)
    ver = np.array([0, 3, 0, -1], np.int32)
    got = oracle_attn(pr, kc, vc, ts, verdict=ver)
    assert np.all(got[1] == 0) and np.all(got[3] == 0)
    assert np.array_equal(got[0], free[0]) and np.array_equal(got[2], free[2])
    allzero = oracle_attn(pr, kc, vc, ts, verdict=np.zeros(4, np.int32))
    assert np.array_equal(allzero, free)


def test_edge_rows_len0_malformed_bad_page():
    pr = small_problem(16, [0, 20, 40, 33], 4, 2, 32, 32, 16, synth.KV_FP8)
    kc, vc, ts = oracle_caches(pr)
    bt = pr["bt"].copy()
    bt[3, 1] = pr["P"]                      # out of range page id
    lens = pr["lens"].copy()
    lens[2] = bt.shape[1] * 16 + 1          # longer than the block table
    got = oracle_attn(pr, kc, vc, ts, bt=bt, lens=lens)
    assert np.all(got[0] == 0)
    assert np.all(np.isnan(got[2])) and np.all(np.isnan(got[3]))
    assert np.all(np.isfinite(got[1]))
    # the same faults under a tracker verdict are aborts: zeros
    ver = oracle.validate_page_tags(np.zeros(pr["P"], np.uint32), bt,
                                    np.zeros(bt.shape, np.uint32), lens, 16)
    assert list(ver) == [0, 0, -1, 2]
    got = oracle_attn(pr, kc, vc, ts, bt=bt, lens=lens, verdict=ver)
    assert np.all(got[2] == 0) and np.all(got[3] == 0)


def test_rows_subset_matches_full():
    pr = small_problem(17, [50, 80], 8, 2, 128, 128, 16, synth.KV_FP8)
    kc, vc, ts = oracle_caches(pr)
    full = oracle_attn(pr, kc, vc, ts)
    rows = [(1, 5), (0, 0), (1, 7)]
    part = oracle_attn(pr, kc, vc, ts, rows=rows, num_threads=2)
    for s, h in rows:
        assert np.array_equal(part[s, h], full[s, h])
    assert np.isnan(part[0, 1]).all()


@pytest.mark.parametrize("chunk", [16, 48, 64])
def test_p15_split_combine_equals_unsplit(chunk):
    """Chunk partials (acc, m, l) in fp64 merged by M = max m_c,
    L = sum l_c e^(m_c - M), out = sum e^(m_c - M) acc_c / L equal the
    unsplit oracle."""
    pr = small_problem(18, [200, 31, 64], 4, 2, 128, 128, 16, synth.KV_FP8)
    kc, vc, ts = oracle_caches(pr)
    ref = oracle_attn(pr, kc, vc, ts)
    q = synth.bf16_to_f32(pr["q"]).astype(np.float64)
    for s in range(3):
        l = int(pr["lens"][s])
        kh, vh = dequant_dense(pr["ks"][s], pr["vs"][s], pr["k_scale"],
                               pr["v_scale"], synth.KV_FP8)
        for h in range(4):
            g = h // 2
            parts = []
            for c0 in range(0, l, chunk):
                z = pr["sm_scale"] * (kh[c0:c0 + chunk, g] @ q[s, h])
                m = z.max()
                w = np.exp(z - m)
                parts.append((w @ vh[c0:c0 + chunk, g], m, w.sum()))
            M = max(p[1] for p in parts)
            L = sum(p[2] * math.exp(p[1] - M) for p in parts)
            out = sum(p[0] * math.exp(p[1] - M) for p in parts) / L
            np.testing.assert_allclose(ref[s, h], out.astype(np.float32), rtol=4e-7, atol=1e-30)


def test_workload1_oracle_runs_and_aborts_injected():
    b = synth.make_batch(1)
    ver = oracle.validate_page_tags(b.page_tags, b.block_table, b.expected_tags,
                                    b.seq_lens, 16)
    assert (ver != 0).sum() == 1
