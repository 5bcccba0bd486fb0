"""GPU parity of kv_transcode_bf16_to_fp8 (BF16 prefill-pool pages re-encoded
as FP8 decode-pool pages) against the oracle: every destination byte and
every per-token scale bit-exact, untouched bytes included.

Sources mix seeded N(0, 3) values with raw random bf16 bit patterns (NaNs,
infinities, subnormals), so the encoder's saturation, NaN and sign-of-zero
handling is exercised on the paged layout too. Pairs have ragged valid
counts (0, 1, odd, full) and a few carry out-of-range ids or counts, which
must write nothing.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import log

pytestmark = pytest.mark.gpu

SENT = 0xAB


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def _src(rng, n):
    x = synth.bf16_from_f32((rng.standard_normal(n) * 3).astype(np.float32))
    wild = rng.random(n) < 0.05
    x[wild] = rng.integers(0, 1 << 16, int(wild.sum()), dtype=np.uint16)
    return x


def _pairs(rng, Ps, Pd, S, n):
    src = rng.integers(0, Ps, n).astype(np.int32)
    dst = rng.permutation(Pd)[:n].astype(np.int32)
    valid = rng.integers(0, S + 1, n).astype(np.int32)
    valid[:4] = [S, 0, 1, S - 1]
    # out-of-range pairs: write nothing
    bad_src = np.int32([Ps, 0, 0])
    bad_dst = np.int32([dst[0], -1, dst[1]])
    bad_valid = np.int32([S, S, S + 1])
    return (np.concatenate([src, bad_src]), np.concatenate([dst, bad_dst]),
            np.concatenate([valid, bad_valid]))


CASES = [
    # (hkv, dk, dv, S, latent)
    (8, 128, 128, 16, False),
    (2, 128, 128, 64, False),
    (1, 576, 0, 64, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"hkv{c[0]}_dk{c[1]}_S{c[3]}")
def test_transcode_parity(gpu, case):
    hkv, dk, dv, S, latent = case
    log(f"transcode parity {case}")
    rng = np.random.default_rng(100 + hkv + S)
    Ps, Pd, n = 40, 48, 32
    kc = _src(rng, Ps * hkv * S * dk)
    vc = None if latent else _src(rng, Ps * hkv * S * dv)
    src, dst, valid = _pairs(rng, Ps, Pd, S, n)
    mode = synth.SCALE_PER_TOKEN if latent else synth.SCALE_PER_HEAD
    kscale = None if latent else rng.uniform(0.005, 0.05, hkv).astype(np.float32)
    vscale = None if latent else rng.uniform(0.005, 0.05, hkv).astype(np.float32)
    # oracle
    kd = np.full(Pd * hkv * S * dk, SENT, np.uint8)
    vd = None if latent else np.full(Pd * hkv * S * dv, SENT, np.uint8)
    ts = np.full(Pd * S, -7.0, np.float32) if latent else None
    oracle.kv_transcode_bf16_to_fp8(kc, vc, src, dst, valid, hkv, dk, dv, S, Ps, Pd, mode,
                                    kscale, vscale, ts, kd, vd)
    # GPU
    gkd = torch.full((kd.size,), SENT, dtype=torch.uint8, device="cuda")
    gvd = None if latent else torch.full((vd.size,), SENT, dtype=torch.uint8, device="cuda")
    gts = torch.full((Pd * S,), -7.0, dtype=torch.float32, device="cuda") if latent else None
    gpu.kv_transcode_bf16_to_fp8(
        _dev(kc), None if latent else _dev(vc), _dev(src), _dev(dst), _dev(valid), gkd, gvd,
        num_kv_heads=hkv, head_dim_k=dk, head_dim_v=dv, page_size=S, src_num_pages=Ps,
        dst_num_pages=Pd, scale_mode=mode,
        k_scale=None if latent else _dev(kscale), v_scale=None if latent else _dev(vscale),
        token_scale=gts)
    torch.cuda.synchronize()
    got = gkd.cpu().numpy()
    if not np.array_equal(got, kd):
        bad = np.nonzero(got != kd)[0]
        page_elems = hkv * S * dk
        pages = np.unique(bad // page_elems)
        log(f"K mismatches: {bad.size}, first {bad[:8].tolist()}, dst pages {pages[:8].tolist()}")
        log(f"  gpu {got[bad[:8]].tolist()} oracle {kd[bad[:8]].tolist()}")
        if latent:
            g = gts.cpu().numpy()
            for pg in pages[:3]:
                sl = slice(pg * S, pg * S + S)
                log(f"  page {pg} scales gpu {g[sl][:6].tolist()} oracle {ts[sl][:6].tolist()}")
    assert np.array_equal(got, kd), "K bytes differ"
    if not latent:
        assert np.array_equal(gvd.cpu().numpy(), vd), "V bytes differ"
    else:
        assert np.array_equal(gts.cpu().numpy().view(np.uint32), ts.view(np.uint32))


def test_transcode_full_pool_sampled(gpu):
    """The 64 x 8192 shape: 32768 BF16 pages (8 kv heads, D 128, S 16; 2 GiB)
    re-encoded through a seeded permutation in one call; 48 sampled pairs are
    re-encoded by the oracle from host copies of their source pages."""
    hkv, dk, dv, S = 8, 128, 128, 16
    P = 32768
    log("transcode full pool: generating 2 GiB of bf16 pages")
    gen = torch.Generator(device="cuda").manual_seed(2024)
    ksrc = (torch.randn(P * hkv * S * dk, generator=gen, device="cuda") * 3).to(torch.bfloat16)
    vsrc = (torch.randn(P * hkv * S * dv, generator=gen, device="cuda") * 3).to(torch.bfloat16)
    rng = np.random.default_rng(5)
    dst = rng.permutation(P).astype(np.int32)
    src = np.arange(P, dtype=np.int32)
    valid = np.full(P, S, np.int32)
    valid[rng.choice(P, 512, replace=False)] = rng.integers(0, S, 512)
    kscale = rng.uniform(0.005, 0.05, hkv).astype(np.float32)
    vscale = rng.uniform(0.005, 0.05, hkv).astype(np.float32)
    kd = torch.full((P * hkv * S * dk,), SENT, dtype=torch.uint8, device="cuda")
    vd = torch.full((P * hkv * S * dv,), SENT, dtype=torch.uint8, device="cuda")
    gpu.kv_transcode_bf16_to_fp8(
        ksrc.view(torch.int16), vsrc.view(torch.int16), _dev(src), _dev(dst), _dev(valid), kd,
        vd, num_kv_heads=hkv, head_dim_k=dk, head_dim_v=dv, page_size=S, src_num_pages=P,
        dst_num_pages=P, scale_mode=synth.SCALE_PER_HEAD, k_scale=_dev(kscale),
        v_scale=_dev(vscale))
    torch.cuda.synchronize()
    sample = rng.choice(P, 48, replace=False)
    sample[:2] = [0, P - 1]
    nk, nv = hkv * S * dk, hkv * S * dv
    pk = ksrc.view(torch.int16).view(P, nk)[torch.from_numpy(sample).cuda()].cpu().numpy()
    pv = vsrc.view(torch.int16).view(P, nv)[torch.from_numpy(sample).cuda()].cpu().numpy()
    n = len(sample)
    okd = np.full(n * nk, SENT, np.uint8)
    ovd = np.full(n * nv, SENT, np.uint8)
    oracle.kv_transcode_bf16_to_fp8(pk.view(np.uint16).ravel(), pv.view(np.uint16).ravel(),
                                    np.arange(n), np.arange(n), valid[sample], hkv, dk, dv, S,
                                    n, n, synth.SCALE_PER_HEAD, kscale, vscale, None, okd, ovd)
    gk = kd.view(P, nk)[torch.from_numpy(dst[sample].astype(np.int64)).cuda()].cpu().numpy()
    gv = vd.view(P, nv)[torch.from_numpy(dst[sample].astype(np.int64)).cuda()].cpu().numpy()
    assert np.array_equal(gk.ravel(), okd), "K pages differ"
    assert np.array_equal(gv.ravel(), ovd), "V pages differ"


def _pattern_pages(P, hkv, S, D, shift):
    """P pages whose (page, head) blocks hold every bf16 bit pattern in turn,
    each head's run rotated by `shift` patterns so heads see different values."""
    n = S * D
    e = np.arange(P * n, dtype=np.int64) % (P * n)
    out = np.empty(P * hkv * n, np.uint16)
    v = out.reshape(P, hkv, n)
    for h in range(hkv):
        v[:, h, :] = ((e + h * shift) & 0xFFFF).reshape(P, n)
    return out


SCALE_SETS = {
    # every scale inside [2^-64, 2^64]: reciprocal path
    "fast": [1.0, 0.0123, 3.0, 2.0 ** -64, 2.0 ** 64, float(np.float32(1.9999999)),
             7.3 / 448, 1e-5],
    # one scale outside the interval sends the whole page through the division
    "mixed": [1.0, 2.0 ** -70, 0.02, 0.5, 3.0, 0.0123, 1e-5, 0.25],
    "far": [2.0 ** 70, 2.0 ** -100, 1e-38, 3e37, 2.0 ** 65, 2.0 ** -65, 1e-30, 1e30],
}


@pytest.mark.parametrize("name", sorted(SCALE_SETS))
def test_transcode_all_bf16_patterns(gpu, name):
    """Per-head scales: every bf16 pattern of K and V under each of 8 head
    scales, bit-exact against the oracle."""
    hkv, dk, dv, S = 8, 128, 128, 16
    P = 65536 // (S * dk)
    log(f"transcode all bf16 patterns, scales {name}")
    kc = _pattern_pages(P, hkv, S, dk, 977)
    vc = _pattern_pages(P, hkv, S, dv, 3001)
    kscale = np.float32(SCALE_SETS[name])
    vscale = np.float32(SCALE_SETS[name][::-1])
    src = np.arange(P, dtype=np.int32)
    dst = src[::-1].copy()
    valid = np.full(P, S, np.int32)
    valid[3] = 5
    kd = np.full(P * hkv * S * dk, SENT, np.uint8)
    vd = np.full(P * hkv * S * dv, SENT, np.uint8)
    oracle.kv_transcode_bf16_to_fp8(kc, vc, src, dst, valid, hkv, dk, dv, S, P, P,
                                    synth.SCALE_PER_HEAD, kscale, vscale, None, kd, vd)
    gkd = torch.full((kd.size,), SENT, dtype=torch.uint8, device="cuda")
    gvd = torch.full((vd.size,), SENT, dtype=torch.uint8, device="cuda")
    gpu.kv_transcode_bf16_to_fp8(
        _dev(kc), _dev(vc), _dev(src), _dev(dst), _dev(valid), gkd, gvd, num_kv_heads=hkv,
        head_dim_k=dk, head_dim_v=dv, page_size=S, src_num_pages=P, dst_num_pages=P,
        scale_mode=synth.SCALE_PER_HEAD, k_scale=_dev(kscale), v_scale=_dev(vscale))
    torch.cuda.synchronize()
    for what, g, o in (("K", gkd, kd), ("V", gvd, vd)):
        got = g.cpu().numpy()
        bad = np.nonzero(got != o)[0]
        if bad.size:
            log(f"{what} mismatches {bad.size}: idx {bad[:6].tolist()} gpu "
                f"{got[bad[:6]].tolist()} oracle {o[bad[:6]].tolist()}")
        assert bad.size == 0, f"{what} bytes differ"


def test_transcode_per_token_scale_ranges(gpu):
    """Latent pages with per-token scales inside and outside [2^-64, 2^64]:
    rows of bf16 patterns up to 2^20 in magnitude plus NaNs (reciprocal path),
    rows of subnormals only (subnormal scale), rows holding an infinity
    (infinite scale), rows near the bf16 maximum, and all-zero rows (scale 1)."""
    dk, S = 576, 64
    rng = np.random.default_rng(31)
    allp = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = synth.bf16_to_f32(allp)
    with np.errstate(invalid="ignore"):
        mid = allp[np.isnan(f) | (np.abs(f) <= 2.0 ** 20)]
        sub = allp[(np.abs(f) < 2.0 ** -126) & ~np.isnan(f)]
        big = allp[np.isfinite(f) & (np.abs(f) >= 2.0 ** 100)]
    rows = []
    for i in range(0, mid.size, dk):
        r = mid[i:i + dk]
        rows.append(np.concatenate([r, rng.choice(mid, dk - r.size)]) if r.size < dk else r)
    for _ in range(16):
        rows.append(rng.choice(sub, dk))
        r = rng.choice(mid, dk)
        r[rng.integers(0, dk)] = 0x7F80 if rng.random() < 0.5 else 0xFF80
        rows.append(r)
        rows.append(rng.choice(big, dk))
        rows.append(np.zeros(dk, np.uint16))
    rows = np.stack(rows)
    order = rng.permutation(rows.shape[0])
    rows = rows[order]
    P = rows.shape[0] // S + 1
    slots = np.zeros((P * S, dk), np.uint16)
    slots[:rows.shape[0]] = rows
    # latent K format: [page][column group][slot][16]
    kc = slots.reshape(P, S, dk // 16, 16).transpose(0, 2, 1, 3).copy().ravel()
    src = np.arange(P, dtype=np.int32)
    dst = np.roll(src, 3)
    valid = np.full(P, S, np.int32)
    kd = np.full(P * S * dk, SENT, np.uint8)
    ts = np.full(P * S, -7.0, np.float32)
    oracle.kv_transcode_bf16_to_fp8(kc, None, src, dst, valid, 1, dk, 0, S, P, P,
                                    synth.SCALE_PER_TOKEN, None, None, ts, kd, None)
    log(f"per-token scale ranges: {rows.shape[0]} rows over {P} pages")
    gkd = torch.full((kd.size,), SENT, dtype=torch.uint8, device="cuda")
    gts = torch.full((P * S,), -7.0, dtype=torch.float32, device="cuda")
    gpu.kv_transcode_bf16_to_fp8(
        _dev(kc), None, _dev(src), _dev(dst), _dev(valid), gkd, None, num_kv_heads=1,
        head_dim_k=dk, head_dim_v=0, page_size=S, src_num_pages=P, dst_num_pages=P,
        scale_mode=synth.SCALE_PER_TOKEN, k_scale=None, v_scale=None, token_scale=gts)
    torch.cuda.synchronize()
    assert np.array_equal(gts.cpu().numpy().view(np.uint32), ts.view(np.uint32))
    got = gkd.cpu().numpy()
    bad = np.nonzero(got != kd)[0]
    if bad.size:
        log(f"K mismatches {bad.size}: idx {bad[:6].tolist()} gpu {got[bad[:6]].tolist()} "
            f"oracle {kd[bad[:6]].tolist()}")
    assert bad.size == 0, "K bytes differ"
