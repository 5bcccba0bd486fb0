"""CPU pins of the oracle's KV write (quantise + scatter) and page-tag
validation.

KV write: the pages say the cache is stored as e4m3 instead of BF16
(manulx.blog, section "Bộ nhớ đệm KV FP8 tăng gấp đôi dung lượng ngữ cảnh").
Pins: scatter by construction (sentinel caches), the format is a bijection,
rounding error bound against the fp32 quotient, the per-token scale maps the
token's largest magnitude to ±448, BF16 writes are bit copies.

Validation: every page carries a tag that changes on reallocation and a
request is aborted when its expected tags no longer match (remio.ai, section
"Sicherheit gemeinsamer KV-Caches wird zum Produktionsthema"). Pins:
verdicts equal the mismatches injected by construction.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth
from helpers import slots_of


def _rand_bf16(rng, shape, scale=1.0):
    return synth.bf16_from_f32((rng.standard_normal(shape) * scale).astype(np.float32))


def test_p5_scatter_touches_exactly_the_addressed_slots():
    rng = np.random.default_rng(1)
    P, S, hkv, dk, dv, T = 9, 16, 2, 32, 16, 20
    slots = rng.choice(P * S, size=T, replace=False).astype(np.int64)
    slots[3] = -1                      # skipped
    slots[7] = P * S + 5               # out of range: skipped
    k = _rand_bf16(rng, (T, hkv, dk))
    v = _rand_bf16(rng, (T, hkv, dv))
    kc = np.full(P * hkv * S * dk, 0xAB, np.uint8)
    vc = np.full(P * hkv * S * dv, 0xAB, np.uint8)
    ks = np.full(hkv, 0.01, np.float32)
    vs = np.full(hkv, 0.02, np.float32)
    oracle.kv_write_fp8(k, v, slots, S, P, synth.SCALE_PER_HEAD, ks, vs, None, kc, vc)
    # mark which (slot) each written byte belongs to by writing a second
    # time into empty caches with the BF16 variant and id payloads
    kid = np.zeros((T, hkv, dk), np.uint16)
    vid = np.zeros((T, hkv, dv), np.uint16)
    for t in range(T):
        kid[t] = t + 1
        vid[t] = t + 1
    kc16 = np.zeros(P * hkv * S * dk, np.uint16)
    vc16 = np.zeros(P * hkv * S * dv, np.uint16)
    oracle.kv_write_bf16(kid, vid, slots, S, P, kc16, vc16)
    valid = [t for t in range(T) if 0 <= slots[t] < P * S]
    # each valid token owns exactly hkv*dk K elements and hkv*dv V elements
    for t in valid:
        assert (kc16 == t + 1).sum() == hkv * dk
        assert (vc16 == t + 1).sum() == hkv * dv
    assert (kc16 == 4).sum() == 0 and (kc16 == 8).sum() == 0   # slots -1, OOR
    # the FP8 write changed bytes only where the id write landed
    assert np.all((kc != 0xAB) <= (kc16 != 0))
    assert np.all((vc != 0xAB) <= (vc16 != 0))
    # a page region holds the tokens of that page only
    per_page = hkv * S * dk
    for t in valid:
        page = slots[t] // S
        idx = np.nonzero(kc16 == t + 1)[0]
        assert idx.min() >= page * per_page and idx.max() < (page + 1) * per_page


def test_format_is_a_bijection_and_matches_header_example():
    """Writing every slot once fills every element exactly once; one element
    is checked against the address formula printed in include/pda.h."""
    P, S, hkv, dk, dv = 3, 16, 2, 32, 16
    T = P * S
    slots = np.arange(T, dtype=np.int64)
    kid = np.zeros((T, hkv, dk), np.uint16)
    vid = np.zeros((T, hkv, dv), np.uint16)
    for t in range(T):
        for h in range(hkv):
            kid[t, h] = (t * hkv + h) * dk + np.arange(dk) + 1
            vid[t, h] = (t * hkv + h) * dv + np.arange(dv) + 1
    kc = np.zeros(P * hkv * S * dk, np.uint16)
    vc = np.zeros(P * hkv * S * dv, np.uint16)
    oracle.kv_write_bf16(kid, vid, slots, S, P, kc, vc)
    assert np.array_equal(np.sort(kc), np.arange(1, kc.size + 1))
    assert np.array_equal(np.sort(vc), np.arange(1, vc.size + 1))
    # header example: page 2, head 1, offset 5, dim 19
    p, h, o, d = 2, 1, 5, 19
    t = p * S + o
    k_at = (((p * hkv + h) * (dk // 16) + d // 16) * S + o) * 16 + d % 16
    assert kc[k_at] == kid[t, h, d]
    d = 11
    v_at = ((((p * hkv + h) * (S // 2) + o // 2) * (dv // 8) + d // 8) * 8 + d % 8) * 2 + o % 2
    assert vc[v_at] == vid[t, h, d]


def test_quantisation_error_bound_and_saturation():
    """Every stored code decodes to within half a code spacing of the fp32
    quotient x/scale (or to ±448 when |x/scale| >= 448)."""
    rng = np.random.default_rng(2)
    P, S, hkv, dk, dv, T = 4, 16, 2, 64, 64, 40
    k = _rand_bf16(rng, (T, hkv, dk), 3.0)
    v = _rand_bf16(rng, (T, hkv, dv), 3.0)
    slots = np.arange(T, dtype=np.int64)
    ks = np.array([0.004, 0.03], np.float32)   # head 0 saturates often
    vs = np.array([0.02, 0.5], np.float32)
    kc = np.zeros(P * hkv * S * dk, np.uint8)
    vc = np.zeros(P * hkv * S * dv, np.uint8)
    oracle.kv_write_fp8(k, v, slots, S, P, synth.SCALE_PER_HEAD, ks, vs, None, kc, vc)
    # locate codes through the id trick, then compare values
    kid = np.arange(1, T * hkv * dk + 1, dtype=np.uint16).reshape(T, hkv, dk)
    vid = np.arange(1, T * hkv * dv + 1, dtype=np.uint16).reshape(T, hkv, dv)
    kc16 = np.zeros(kc.size, np.uint16)
    vc16 = np.zeros(vc.size, np.uint16)
    oracle.kv_write_bf16(kid, vid, slots, S, P, kc16, vc16)
    dec = oracle.e4m3_decode_all()
    nsat = 0
    for cache, ids, data, sc, D in ((kc, kc16, k, ks, dk), (vc, vc16, v, vs, dv)):
        where = np.argsort(ids)[ids.size - T * hkv * D:]
        codes = cache[where].reshape(T, hkv, D)
        x = synth.bf16_to_f32(data) / sc[None, :, None]
        got = dec[codes]
        a = np.abs(x.astype(np.float64))
        sat = a >= 448
        nsat += sat.sum()
        assert np.all(got[sat] == np.sign(x[sat]) * 448)
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
        half = np.where(a < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))
        assert np.all(np.abs(got[~sat] - x[~sat]) <= half[~sat])
    assert nsat > 0


def test_per_token_scale_maps_amax_to_448():
    rng = np.random.default_rng(3)
    P, S, dk, T = 4, 64, 576, 50
    k = _rand_bf16(rng, (T, 1, dk), 2.0)
    k[5] = 0                                 # all-zero token -> scale 1
    slots = rng.choice(P * S, T, replace=False).astype(np.int64)
    kc = np.zeros(P * S * dk, np.uint8)
    ts = np.full(P * S, -1.0, np.float32)
    oracle.kv_write_fp8(k, None, slots, S, P, synth.SCALE_PER_TOKEN, None, None, ts, kc, None)
    written = np.zeros(P * S, bool)
    written[slots] = True
    assert np.all(ts[~written] == -1.0)
    assert ts[slots[5]] == 1.0
    kid = np.arange(1, T * dk + 1, dtype=np.uint32)
    for t in range(T):
        if t == 5:
            continue
        x = synth.bf16_to_f32(k[t, 0])
        amax = np.abs(x).max()
        sc = ts[slots[t]]
        assert sc > 0 and abs(sc * np.float32(448) - amax) <= amax * 2.0 ** -22
    _ = kid
    # the largest-magnitude element of each token encodes to ±448
    kc16 = np.zeros(P * S * dk, np.uint16)
    ids = np.tile(np.arange(1, dk + 1, dtype=np.uint16), (T, 1)).reshape(T, 1, dk)
    for t in range(T):
        if t == 5:
            continue
        kc16[:] = 0
        oracle.kv_write_bf16(ids[t:t + 1], None, slots[t:t + 1], S, P, kc16, None)
        x = synth.bf16_to_f32(k[t, 0])
        dmax = int(np.argmax(np.abs(x)))
        pos = int(np.nonzero(kc16 == dmax + 1)[0][0])
        assert kc[pos] & 0x7F == 0x7E


def test_bf16_write_is_bit_copy():
    rng = np.random.default_rng(4)
    P, S, hkv, dk, dv, T = 3, 16, 1, 16, 16, 48
    k = rng.integers(0, 65536, (T, hkv, dk), dtype=np.uint16)
    v = rng.integers(0, 65536, (T, hkv, dv), dtype=np.uint16)
    slots = rng.permutation(P * S).astype(np.int64)
    kc = np.zeros(P * hkv * S * dk, np.uint16)
    vc = np.zeros(P * hkv * S * dv, np.uint16)
    oracle.kv_write_bf16(k, v, slots, S, P, kc, vc)
    assert np.array_equal(np.sort(kc), np.sort(k.ravel()))
    assert np.array_equal(np.sort(vc), np.sort(v.ravel()))


def test_kv_write_rejects_bad_arguments():
    k = np.zeros((1, 1, 15, ), np.uint16).reshape(1, 1, 15)
    with pytest.raises(ValueError):
        oracle.kv_write_bf16(k, k, np.zeros(1, np.int64), 16, 1,
                             np.zeros(16 * 15, np.uint16), np.zeros(16 * 15, np.uint16))


# --- validation ---------------------------------------------------------------

def test_p6_verdicts_equal_injected_positions_workload1():
    b = synth.make_batch(1)
    ver = oracle.validate_page_tags(b.page_tags, b.block_table, b.expected_tags,
                                    b.seq_lens, b.cfg.page_size)
    want = np.zeros(b.B, np.int32)
    for s, j in b.injected:
        want[s] = j + 1 if want[s] == 0 else min(want[s], j + 1)
    assert len(b.injected) == 1
    assert np.array_equal(ver, want)


def test_p6_verdicts_equal_injected_positions_workload5():
    b = synth.make_batch(5)
    ver = oracle.validate_page_tags(b.page_tags, b.block_table, b.expected_tags,
                                    b.seq_lens, b.cfg.page_size)
    want = np.zeros(b.B, np.int32)
    for s, j in b.injected:
        want[s] = j + 1 if want[s] == 0 else min(want[s], j + 1)
    assert len(b.injected) == len(b.used_pages()) // 10000 >= 1
    assert np.array_equal(ver, want)


def test_p6_no_injection_all_clear_and_edge_cases():
    b = synth.make_batch(1, inject=0)
    S = b.cfg.page_size
    ver = oracle.validate_page_tags(b.page_tags, b.block_table, b.expected_tags,
                                    b.seq_lens, S)
    assert np.all(ver == 0)
    bt = b.block_table.copy()
    lens = b.seq_lens.copy()
    # entries past ceil(len/S) are never read: garbage there is fine
    bt[0, 5:] = 10 ** 6
    # out-of-range page id in block 1 of seq 1
    bt[1, 1] = b.num_pages
    # negative page id in block 0 of seq 2
    bt[2, 0] = -3
    ver = oracle.validate_page_tags(b.page_tags, bt, b.expected_tags, lens, S)
    assert list(ver) == [0, 2, 1, 0]
    # malformed lengths
    lens2 = lens.copy()
    lens2[0] = -1
    lens2[3] = b.max_blocks * S + 1
    ver = oracle.validate_page_tags(b.page_tags, b.block_table, b.expected_tags, lens2, S)
    assert ver[0] == -1 and ver[3] == -1
    # len 0 reads nothing and passes; exact capacity passes
    lens3 = lens.copy()
    lens3[0] = 0
    ver = oracle.validate_page_tags(b.page_tags, b.block_table, b.expected_tags, lens3, S)
    assert ver[0] == 0


def test_p6_tag_compare_is_full_32_bit():
    tags = np.array([0xFFFFFFFF, 0x00000000, 0x80000000], np.uint32)
    bt = np.array([[0, 1, 2]], np.int32)
    exp = np.array([[0xFFFFFFFF, 0x00000000, 0x00000000]], np.uint32)
    ver = oracle.validate_page_tags(tags, bt, exp, np.array([48], np.int32), 16)
    assert ver[0] == 3
    exp[0, 2] = 0x80000000
    assert oracle.validate_page_tags(tags, bt, exp, np.array([48], np.int32), 16)[0] == 0
    exp[0, 0] = 0x7FFFFFFF
    assert oracle.validate_page_tags(tags, bt, exp, np.array([48], np.int32), 16)[0] == 1
