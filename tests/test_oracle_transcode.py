"""CPU pins of the oracle's BF16 -> FP8 page transcode.

The pages keep the prefill pool's cache in BF16 and the decode pool's in FP8
(aifeed.sk, section "Kompresia sa oplatí inde pri vstupe a inde pri
výstupe"; manulx.blog, section "Bộ nhớ đệm KV FP8 tăng gấp đôi dung lượng
ngữ cảnh"); a request's pages are re-encoded when it moves between them,
each token as the decode pool's kv write would quantise it. Pins:
  * a hand-built page: codes worked out by hand at hand-computed byte
    positions of the documented cache format;
  * every re-encoded code decodes to the e4m3 value nearest the fp32
    quotient, by torch's float8_e4m3fn codec (independent of the oracle's);
  * composition: a BF16 cache written by kv_write_bf16 and transcoded equals
    kv_write_fp8 of the same rows, bit for bit, per-token scales included;
  * untouched bytes: slots at or past valid, pages no pair names and pairs
    with out-of-range ids or counts keep their sentinel.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import torch_e4m3_roundtrip

SENT = 0xAB


def _bits(xs):
    return synth.bf16_from_f32(np.asarray(xs, np.float32))


def test_hand_built_page():
    # Hkv 1, Dk 16, Dv 8, S 2: one K column group and one V dim group per page
    S, hkv, dk, dv, Ps, Pd = 2, 1, 16, 8, 2, 3
    k_src = np.zeros(Ps * hkv * S * dk, np.uint16)
    v_src = np.zeros(Ps * hkv * S * dv, np.uint16)
    kx = [1.0, -2.5, np.nan, 1000.0, -0.0, 2.0 ** -12, 2.0 ** -9] + [0.0] * 9
    # source page 1, slot 0: K element (page*S + slot)*16 + d; V element
    # ((page*(S/2) + slot/2)*8 + d)*2 + slot%2
    k_src[(1 * S + 0) * 16: (1 * S + 0) * 16 + 16] = _bits(kx)
    v_src[(1 * 8 + 0) * 2] = _bits([3.0])[0]
    kd = np.full(Pd * hkv * S * dk, SENT, np.uint8)
    vd = np.full(Pd * hkv * S * dv, SENT, np.uint8)
    oracle.kv_transcode_bf16_to_fp8(k_src, v_src, [1], [2], [1], hkv, dk, dv, S, Ps, Pd,
                                    synth.SCALE_PER_HEAD, np.float32([0.5]),
                                    np.float32([1.0]), None, kd, vd)
    # x / 0.5: 2 -> 0x40; -5 -> 0xCA; NaN -> 0x7F; 2000 saturates -> 0x7E;
    # -0 -> 0x80; 2^-11 rounds to +0 -> 0x00; 2^-8 = 2 * 2^-9 -> 0x02
    want = [0x40, 0xCA, 0x7F, 0x7E, 0x80, 0x00, 0x02] + [0x00] * 9
    base = (2 * S + 0) * 16      # destination page 2, slot 0
    assert kd[base: base + 16].tolist() == want
    assert vd[(2 * 8 + 0) * 2] == 0x44   # 3.0 -> 1.5 * 2^1
    # slot 1 of page 2 (past valid) and pages 0, 1 untouched
    written = np.zeros(kd.size, bool)
    written[base: base + 16] = True
    assert np.all(kd[~written] == SENT)
    vw = np.zeros(vd.size, bool)
    vw[[(2 * 8 + d) * 2 for d in range(8)]] = True
    assert np.all(vd[~vw] == SENT)


def _pool(rng, P, hkv, dk, dv, S, latent):
    """A BF16 pool written with kv_write_bf16 from seeded rows (every slot)."""
    T = P * S
    k = synth.bf16_from_f32((rng.standard_normal((T, hkv, dk)) * 3).astype(np.float32))
    v = None if latent else synth.bf16_from_f32(
        (rng.standard_normal((T, hkv, dv)) * 3).astype(np.float32))
    # specials in a few rows
    k[1, 0, :4] = _bits([np.nan, np.inf, -np.inf, -0.0])
    k[2, 0, :] = 0   # an all-zero row: per-token scale 1.0
    kc = np.zeros(P * hkv * S * dk, np.uint16)
    vc = None if latent else np.zeros(P * hkv * S * dv, np.uint16)
    slots = np.arange(T, dtype=np.int64)
    oracle.kv_write_bf16(k, v, slots, S, P, kc, vc)
    return k, v, kc, vc


@pytest.mark.parametrize("latent", [False, True])
def test_composition_with_kv_write(latent):
    rng = np.random.default_rng(7 + latent)
    if latent:
        hkv, dk, dv, S, mode = 1, 576, 0, 64, synth.SCALE_PER_TOKEN
    else:
        hkv, dk, dv, S, mode = 2, 128, 128, 16, synth.SCALE_PER_HEAD
    Ps, Pd = 6, 9
    k, v, kc, vc = _pool(rng, Ps, hkv, dk, dv, S, latent)
    src = np.int32([4, 0, 5, 2, 3])
    dst = np.int32([7, 1, 2, 8, 0])
    valid = np.int32([S, 1, S - 3, 0, S // 2 + 1])
    ks = None if latent else np.float32(rng.uniform(0.01, 0.05, hkv))
    vs = None if latent else np.float32(rng.uniform(0.01, 0.05, hkv))
    kd = np.full(Pd * hkv * S * dk, SENT, np.uint8)
    vd = None if latent else np.full(Pd * hkv * S * dv, SENT, np.uint8)
    ts = np.full(Pd * S, -7.0, np.float32) if latent else None
    oracle.kv_transcode_bf16_to_fp8(kc, vc, src, dst, valid, hkv, dk, dv, S, Ps, Pd, mode,
                                    ks, vs, ts, kd, vd)
    # the same rows written straight to the FP8 pool
    kd2 = np.full_like(kd, SENT)
    vd2 = None if latent else np.full_like(vd, SENT)
    ts2 = np.full(Pd * S, -7.0, np.float32) if latent else None
    rows = np.concatenate([sp * S + np.arange(n) for sp, n in zip(src, valid)]).astype(int)
    slots = np.concatenate([dp * S + np.arange(n) for dp, n in zip(dst, valid)]).astype(np.int64)
    oracle.kv_write_fp8(k[rows], None if latent else v[rows], slots, S, Pd, mode, ks, vs,
                        ts2, kd2, vd2)
    assert np.array_equal(kd, kd2)
    if not latent:
        assert np.array_equal(vd, vd2)
    else:
        assert np.array_equal(ts.view(np.uint32), ts2.view(np.uint32))
        # untouched scale slots keep their sentinel
        assert (ts == -7.0).sum() == Pd * S - int(valid.sum())


def test_codes_are_nearest_e4m3_of_the_quotient():
    rng = np.random.default_rng(11)
    hkv, dk, dv, S, Ps, Pd = 2, 32, 16, 8, 3, 3
    k, v, kc, vc = _pool(rng, Ps, hkv, dk, dv, S, False)
    ks = np.float32([0.02, 0.03])
    vs = np.float32([0.025, 0.04])
    kd = np.full(Pd * hkv * S * dk, SENT, np.uint8)
    vd = np.full(Pd * hkv * S * dv, SENT, np.uint8)
    oracle.kv_transcode_bf16_to_fp8(kc, vc, [0, 1, 2], [2, 0, 1], [S, S, S], hkv, dk, dv, S,
                                    Ps, Pd, synth.SCALE_PER_HEAD, ks, vs, None, kd, vd)
    table = oracle.e4m3_decode_all()
    # with every slot copied, destination page d holds source page p's
    # elements at the same in-page positions
    for p, d in ((0, 2), (1, 0), (2, 1)):
        for cache_s, cache_d, sc, D in ((kc, kd, ks, dk), (vc, vd, vs, dv)):
            n = hkv * S * D
            x = synth.bf16_to_f32(cache_s[p * n:(p + 1) * n]).reshape(hkv, -1)
            y = x / sc[:, None]
            got = table[cache_d[d * n:(d + 1) * n]].reshape(hkv, -1)
            fin = np.isfinite(y) & (np.abs(y) < 448)
            assert np.array_equal(got[fin], torch_e4m3_roundtrip(y[fin]))
            assert np.all(np.isnan(got[np.isnan(y)]))
            big = np.isfinite(y) & (np.abs(y) >= 448) | np.isinf(y)
            assert np.all(np.abs(got[big]) == 448)


def test_invalid_pairs_write_nothing():
    rng = np.random.default_rng(3)
    hkv, dk, dv, S, Ps, Pd = 1, 16, 8, 4, 2, 2
    _, _, kc, vc = _pool(rng, Ps, hkv, dk, dv, S, False)
    kd = np.full(Pd * hkv * S * dk, SENT, np.uint8)
    vd = np.full(Pd * hkv * S * dv, SENT, np.uint8)
    oracle.kv_transcode_bf16_to_fp8(kc, vc, [-1, 2, 0, 0, 1], [0, 0, -1, 2, 1],
                                    [S, S, S, S, S + 1], hkv, dk, dv, S, Ps, Pd,
                                    synth.SCALE_PER_HEAD, np.float32([0.1]),
                                    np.float32([0.1]), None, kd, vd)
    assert np.all(kd == SENT) and np.all(vd == SENT)


def test_per_token_scale_ignores_every_nan():
    """The per-token scale is amax/448 over the token's non-NaN values; a
    signaling NaN (bf16 0x7F81: exponent all ones, quiet bit clear) is ignored
    like a quiet one, wherever it sits in the row."""
    dk, S, P = 32, 2, 1
    base = np.float32(np.linspace(-3.0, 5.0, dk))
    for pos in (0, 5, 17, 31):
        for nan_bits in (0x7FC0, 0xFFC0, 0x7F81, 0xFF81):
            k = synth.bf16_from_f32(base)
            k[pos] = nan_bits
            x = synth.bf16_to_f32(k)
            amax = np.float32(np.max(np.abs(x[~np.isnan(x)])))
            want = np.float32(amax / np.float32(448.0))
            kc = np.zeros(P * S * dk, np.uint8)
            ts = np.zeros(P * S, np.float32)
            oracle.kv_write_fp8(k.reshape(1, 1, dk), None, np.int64([1]), S, P,
                                synth.SCALE_PER_TOKEN, None, None, ts, kc, None)
            assert ts[1] == want, (pos, hex(nan_bits), ts[1], want)
