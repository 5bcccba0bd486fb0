"""GPU parity of kv_write_fp8 / kv_write_bf16 against the oracle: cache
bytes, per-token scales and the scatter must be bit-exact.

The all-patterns sweep feeds every bf16 bit pattern (including ±0, ±inf,
NaNs, subnormals) through the gfx950 e4m3 conversion at three scales, which
audits its rounding, saturation, sign-of-zero and NaN handling against the
oracle's definition.
"""
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


def _host(t, dtype):
    return t.cpu().numpy().view(dtype)


@pytest.mark.parametrize("scale", [1.0, 0.0123, 3.0])
def test_all_bf16_patterns_bit_exact(gpu, scale):
    log(f"kv_write_fp8 all-bf16 sweep scale={scale}")
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    T, hkv, d, S = 512, 1, 128, 16
    P = T // S
    k = pats.reshape(T, hkv, d)
    v = pats[::-1].copy().reshape(T, hkv, d)
    slots = np.arange(T, dtype=np.int64)
    ks = np.array([scale], np.float32)
    vs = np.array([scale * 0.5], np.float32)
    kc = np.full(P * hkv * S * d, 0x5A, np.uint8)
    vc = kc.copy()
    oracle.kv_write_fp8(k, v, slots, S, P, synth.SCALE_PER_HEAD, ks, vs, None, kc, vc)
    gk = _dev(np.full(kc.size, 0x5A, np.uint8))
    gv = _dev(np.full(vc.size, 0x5A, np.uint8))
    gpu.kv_write_fp8(_dev(k), _dev(v), _dev(slots), gk, gv, page_size=S, num_pages=P,
                     k_scale=_dev(ks), v_scale=_dev(vs))
    torch.cuda.synchronize()
    gkh, gvh = _host(gk, np.uint8), _host(gv, np.uint8)
    bad = np.nonzero(gkh != kc)[0]
    assert bad.size == 0, f"{bad.size} K codes differ, first at {bad[:8]}: gpu {gkh[bad[:8]]} oracle {kc[bad[:8]]}"
    assert np.array_equal(gvh, vc)


def test_per_token_latent_bit_exact(gpu):
    log("kv_write_fp8 per-token latent")
    rng = np.random.default_rng(5)
    T, dk, S = 300, 576, 64
    P = 8
    x = (rng.standard_normal((T, 1, dk)) * np.exp(rng.uniform(-12, 8, (T, 1, 1)))).astype(np.float32)
    k = synth.bf16_from_f32(x)
    k[7] = 0                                    # amax 0 -> scale 1
    k[9, 0, :5] = 0x7FC0                        # NaN values are ignored by amax
    k[11, 0, 3] = 0x7F81                        # signaling NaNs too, mid-row
    k[12, 0, 400] = 0xFF81
    slots = rng.choice(P * S, T, replace=False).astype(np.int64)
    slots[3] = -1
    kc = np.full(P * S * dk, 0xA5, np.uint8)
    ts = np.full(P * S, -2.0, np.float32)
    oracle.kv_write_fp8(k, None, slots, S, P, synth.SCALE_PER_TOKEN, None, None, ts, kc, None)
    gk = _dev(np.full(kc.size, 0xA5, np.uint8))
    gts = _dev(np.full(P * S, -2.0, np.float32))
    gpu.kv_write_fp8(_dev(k), None, _dev(slots), gk, None, page_size=S, num_pages=P,
                     scale_mode=gpu.SCALE_PER_TOKEN, token_scale=gts)
    torch.cuda.synchronize()
    assert np.array_equal(gts.cpu().numpy().view(np.uint32), ts.view(np.uint32))
    assert np.array_equal(_host(gk, np.uint8), kc)


def test_bf16_copy_and_skipped_slots(gpu):
    log("kv_write_bf16 + skipped slots")
    rng = np.random.default_rng(6)
    T, hkv, dk, dv, S, P = 70, 2, 128, 128, 16, 9
    k = rng.integers(0, 65536, (T, hkv, dk)).astype(np.uint16)
    v = rng.integers(0, 65536, (T, hkv, dv)).astype(np.uint16)
    slots = rng.choice(P * S, T, replace=False).astype(np.int64)
    slots[0] = -1
    slots[5] = P * S
    slots[6] = -(1 << 40)
    kc = np.full(P * hkv * S * dk, 0x1234, np.uint16)
    vc = np.full(P * hkv * S * dv, 0x1234, np.uint16)
    oracle.kv_write_bf16(k, v, slots, S, P, kc, vc)
    gk, gv = _dev(kc.copy()), _dev(vc.copy())
    gk.fill_(0x1234)
    gv.fill_(0x1234)
    gpu.kv_write_bf16(_dev(k), _dev(v), _dev(slots), gk, gv, page_size=S, num_pages=P)
    torch.cuda.synchronize()
    assert np.array_equal(_host(gk, np.uint16), kc)
    assert np.array_equal(_host(gv, np.uint16), vc)
    # FP8 variant with the same skipped slots
    kc8 = np.full(P * hkv * S * dk, 0x3C, np.uint8)
    vc8 = kc8.copy()
    ks = np.array([0.02, 0.5], np.float32)
    vs = np.array([0.1, 0.03], np.float32)
    kb = synth.bf16_from_f32(rng.standard_normal((T, hkv, dk)).astype(np.float32))
    vb = synth.bf16_from_f32(rng.standard_normal((T, hkv, dv)).astype(np.float32))
    oracle.kv_write_fp8(kb, vb, slots, S, P, synth.SCALE_PER_HEAD, ks, vs, None, kc8, vc8)
    gk8 = _dev(np.full(kc8.size, 0x3C, np.uint8))
    gv8 = _dev(np.full(vc8.size, 0x3C, np.uint8))
    gpu.kv_write_fp8(_dev(kb), _dev(vb), _dev(slots), gk8, gv8, page_size=S, num_pages=P,
                     k_scale=_dev(ks), v_scale=_dev(vs))
    torch.cuda.synchronize()
    assert np.array_equal(_host(gk8, np.uint8), kc8)
    assert np.array_equal(_host(gv8, np.uint8), vc8)


@pytest.mark.parametrize("kv_dtype", [synth.KV_FP8, synth.KV_BF16])
def test_workload1_caches_bit_exact(gpu, kv_dtype):
    log(f"workload 1 cache build, dtype {kv_dtype}")
    from synth import device as workload
    from gpu_helpers import oracle_subset
    b = synth.make_batch(1)
    data = [b.kv(s) for s in range(b.B)]
    db = workload.build(b, kv_dtype, data=data)
    sub = oracle_subset(b, data, list(range(b.B)), kv_dtype, db.host_scales)
    S, hkv, d = 16, 2, 128
    pe = hkv * S * d
    elt = np.uint8 if kv_dtype == synth.KV_FP8 else np.uint16
    gk = workload_pages(db.k_cache, sub["pages"], pe, elt)
    gv = workload_pages(db.v_cache, sub["pages"], pe, elt)
    assert np.array_equal(gk.ravel(), sub["kc"])
    assert np.array_equal(gv.ravel(), sub["vc"])
    # pages no sequence uses keep their poison
    used = set(sub["pages"])
    free = [p for p in range(b.num_pages) if p not in used]
    fk = workload_pages(db.k_cache, free, pe, elt)
    assert np.all(fk == synth.poison_value(kv_dtype))


def workload_pages(t, pages, pe, elt):
    from gpu_helpers import gpu_pages
    return gpu_pages(t, pages, pe).view(elt)
