"""GPU parity of kv_write_check, the kv write and the page-tag check in one
launch: cache bytes, per-token scales and verdicts bit-exact against the
oracle's kv write and tag check on the same inputs, for FP8 per-head, FP8
per-token (latent) and BF16 caches, and either half alone."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import log

pytestmark = pytest.mark.gpu


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).cuda()


def _tag_case(rng, B, S, P, mb):
    """Random sequences over a pool with faults planted in some of them."""
    lens = rng.integers(0, mb * S + 1, B).astype(np.int32)
    tags = rng.integers(0, 2 ** 32, P, dtype=np.uint64).astype(np.uint32)
    bt = rng.integers(0, P, (B, mb)).astype(np.int32)
    exp = tags[bt]
    for s in rng.choice(B, max(1, B // 4), replace=False):
        j = int(rng.integers(0, mb))
        if rng.integers(0, 2) == 0:
            exp[s, j] ^= np.uint32(1 << int(rng.integers(0, 32)))
        else:
            bt[s, j] = P + int(rng.integers(0, 5))
    lens[0] = 0
    if B > 2:
        lens[1] = -3
    return tags, bt, exp, lens


def _check_args(tags, bt, exp, lens):
    return _dev(tags), _dev(bt), _dev(exp), _dev(lens)


@pytest.mark.parametrize("T,B", [(37, 19), (0, 19), (37, 0)])
def test_fp8_per_head(gpu, T, B):
    log(f"kv_write_check fp8 per-head T={T} B={B}")
    rng = np.random.default_rng(11 + T + B)
    hkv, d, S, P, mb = 2, 128, 16, 96, 7
    k = synth.bf16_from_f32(rng.standard_normal((max(T, 1), hkv, d)).astype(np.float32))[:T]
    v = synth.bf16_from_f32(rng.standard_normal((max(T, 1), hkv, d)).astype(np.float32))[:T]
    slots = rng.choice(P * S, T, replace=False).astype(np.int64)
    if T > 3:
        slots[3] = -1
    ks = np.array([0.011, 0.02], np.float32)
    vs = np.array([0.007, 0.03], np.float32)
    kc = np.full(P * hkv * S * d, 0x5A, np.uint8)
    vc = kc.copy()
    if T:
        oracle.kv_write_fp8(k, v, slots, S, P, synth.SCALE_PER_HEAD, ks, vs, None, kc, vc)
    tags, bt, exp, lens = _tag_case(rng, max(B, 1), S, P, mb)
    tags, bt, exp, lens = tags, bt[:B], exp[:B], lens[:B]
    want = oracle.validate_page_tags(tags, bt, exp, lens, S) if B else np.zeros(0, np.int32)
    gk = _dev(np.full(kc.size, 0x5A, np.uint8))
    gv = _dev(np.full(vc.size, 0x5A, np.uint8))
    ver = torch.full((B,), 12345, dtype=torch.int32, device="cuda")
    gt, gb, ge, gl = _check_args(tags, bt.reshape(B, mb), exp.reshape(B, mb), lens)
    gpu.kv_write_check(_dev(k.reshape(T, hkv, d)), _dev(v.reshape(T, hkv, d)), _dev(slots), gk, gv,
                       gt, gb, ge, gl, ver, page_size=S, num_pages=P, kv_dtype=gpu.KV_FP8_E4M3,
                       scale_mode=gpu.SCALE_PER_HEAD, k_scale=_dev(ks), v_scale=_dev(vs))
    torch.cuda.synchronize()
    assert np.array_equal(gk.cpu().numpy().view(np.uint8), kc)
    assert np.array_equal(gv.cpu().numpy().view(np.uint8), vc)
    assert np.array_equal(ver.cpu().numpy(), want)


def test_fp8_per_token_latent(gpu):
    log("kv_write_check fp8 per-token latent")
    rng = np.random.default_rng(21)
    T, dk, S, P, B, mb = 70, 576, 64, 12, 9, 4
    x = (rng.standard_normal((T, 1, dk)) * np.exp(rng.uniform(-6, 6, (T, 1, 1)))).astype(np.float32)
    k = synth.bf16_from_f32(x)
    slots = rng.choice(P * S, T, replace=False).astype(np.int64)
    kc = np.full(P * S * dk, 0xA5, np.uint8)
    ts = np.full(P * S, -2.0, np.float32)
    oracle.kv_write_fp8(k, None, slots, S, P, synth.SCALE_PER_TOKEN, None, None, ts, kc, None)
    tags, bt, exp, lens = _tag_case(rng, B, S, P, mb)
    want = oracle.validate_page_tags(tags, bt, exp, lens, S)
    gk = _dev(np.full(kc.size, 0xA5, np.uint8))
    gts = _dev(np.full(P * S, -2.0, np.float32))
    ver = torch.full((B,), 12345, dtype=torch.int32, device="cuda")
    gpu.kv_write_check(_dev(k), None, _dev(slots), gk, None, *_check_args(tags, bt, exp, lens),
                       ver, page_size=S, num_pages=P, kv_dtype=gpu.KV_FP8_E4M3,
                       scale_mode=gpu.SCALE_PER_TOKEN, token_scale=gts)
    torch.cuda.synchronize()
    assert np.array_equal(gts.cpu().numpy().view(np.uint32), ts.view(np.uint32))
    assert np.array_equal(gk.cpu().numpy().view(np.uint8), kc)
    assert np.array_equal(ver.cpu().numpy(), want)


def test_bf16(gpu):
    log("kv_write_check bf16")
    rng = np.random.default_rng(31)
    T, hkv, d, S, P, B, mb = 45, 2, 128, 16, 64, 13, 6
    k = synth.bf16_from_f32(rng.standard_normal((T, hkv, d)).astype(np.float32))
    v = synth.bf16_from_f32(rng.standard_normal((T, hkv, d)).astype(np.float32))
    slots = rng.choice(P * S, T, replace=False).astype(np.int64)
    kc = np.full(P * hkv * S * d, 0x1234, np.uint16)
    vc = kc.copy()
    oracle.kv_write_bf16(k, v, slots, S, P, kc, vc)
    tags, bt, exp, lens = _tag_case(rng, B, S, P, mb)
    want = oracle.validate_page_tags(tags, bt, exp, lens, S)
    gk = _dev(np.full(kc.size, 0x1234, np.uint16))
    gv = _dev(np.full(vc.size, 0x1234, np.uint16))
    ver = torch.full((B,), 12345, dtype=torch.int32, device="cuda")
    gpu.kv_write_check(_dev(k), _dev(v), _dev(slots), gk, gv, *_check_args(tags, bt, exp, lens),
                       ver, page_size=S, num_pages=P, kv_dtype=gpu.KV_BF16,
                       scale_mode=gpu.SCALE_NONE)
    torch.cuda.synchronize()
    assert np.array_equal(gk.cpu().numpy().view(np.uint16), kc)
    assert np.array_equal(gv.cpu().numpy().view(np.uint16), vc)
    assert np.array_equal(ver.cpu().numpy(), want)


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_workload_step_matches_two_launches(gpu, kv):
    """The device step's fused launch leaves the same caches and verdicts as
    kv_write + validate_page_tags on the tiny batch (one injected mismatch).
    The caches are refilled before each variant, so only the step's tokens
    hold data afterwards."""
    log(f"kv_write_check tiny batch {kv} against the two-launch step")
    from synth import device as workload
    b = synth.make_batch(1)
    dt = gpu.KV_FP8_E4M3 if kv == "fp8" else gpu.KV_BF16
    db = workload.build(b, dt)
    outs = []
    for fused in (True, False):
        db.k_cache.fill_(0x33)
        db.v_cache.fill_(0x33)
        db.verdict.fill_(777)
        if fused:
            db.write_check()
        else:
            db.write_step()
            db.validate()
        torch.cuda.synchronize()
        outs.append((db.k_cache.cpu().numpy().copy(), db.v_cache.cpu().numpy().copy(),
                     db.verdict.cpu().numpy().copy()))
    for a, c in zip(outs[0], outs[1]):
        assert np.array_equal(a, c)
    assert (outs[0][0] != 0x33).any()
    want = oracle.validate_page_tags(b.page_tags, b.block_table, b.expected_tags, b.seq_lens,
                                     b.cfg.page_size)
    assert np.array_equal(outs[0][2], want)
    assert (want != 0).sum() >= 1
