"""Shared test helpers: small seeded problems and an independent dense
attention reference (numpy fp64 + torch's float8_e4m3fn codec). Nothing here
is used by the product path."""
from __future__ import annotations

import math

import numpy as np
import torch

import synth


def torch_e4m3_roundtrip(x_over_scale: np.ndarray) -> np.ndarray:
    """fp64 value of the e4m3 code nearest to x (|x| < 464), via torch."""
    t = torch.from_numpy(np.ascontiguousarray(x_over_scale, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def dequant_dense(kb, vb, k_scale, v_scale, kv_dtype, tok_scale=None):
    """Dense fp64 K̂, V̂ of one sequence from its bf16 inputs, the way the
    format stores them. kb [L, Hkv, Dk] uint16; vb [L, Hkv, Dv] or None."""
    k = synth.bf16_to_f32(kb)
    v = None if vb is None else synth.bf16_to_f32(vb)
    if kv_dtype == synth.KV_BF16:
        return k.astype(np.float64), None if v is None else v.astype(np.float64)
    if tok_scale is not None:   # per token, latent
        sc = tok_scale.astype(np.float32)[:, None, None]
        kh = torch_e4m3_roundtrip(k / sc) * sc.astype(np.float64)
        return kh, None
    ks = k_scale.astype(np.float32)[None, :, None]
    vs = v_scale.astype(np.float32)[None, :, None]
    kh = torch_e4m3_roundtrip(k / ks) * ks.astype(np.float64)
    vh = torch_e4m3_roundtrip(v / vs) * vs.astype(np.float64)
    return kh, vh


def dense_attention(q_bits, kh, vh, sm_scale, group, v_in_k=False, dv=None):
    """Textbook softmax(q K̂ᵀ sm_scale) V̂ per query head, fp64.
    q_bits [Hq, Dk] uint16; kh [L, Hkv, Dk]; vh [L, Hkv, Dv]."""
    q = synth.bf16_to_f32(q_bits).astype(np.float64)
    hq = q.shape[0]
    if v_in_k:
        vh = kh[:, :, :dv]
    out = np.zeros((hq, vh.shape[2]))
    for h in range(hq):
        g = h // group
        z = sm_scale * (kh[:, g, :] @ q[h])
        w = np.exp(z - z.max())
        out[h] = (w[:, None] * vh[:, g, :]).sum(0) / w.sum()
    return out


def small_problem(seed, lens, hq, hkv, dk, dv, S, kv_dtype, num_pages=None,
                  latent=False):
    """Random bf16 data, a page assignment and per-head scales for a small
    problem. Returns a dict of host arrays."""
    rng = np.random.default_rng(seed)
    B = len(lens)
    npages = [-(-l // S) for l in lens]
    used = sum(npages)
    P = num_pages or used + 3
    perm = rng.permutation(P)
    max_blocks = max(max(npages), 1)
    bt = np.full((B, max_blocks), -1, np.int32)
    pos = 0
    for s in range(B):
        bt[s, :npages[s]] = perm[pos:pos + npages[s]]
        pos += npages[s]
    ks = [synth.bf16_from_f32(rng.standard_normal((l, hkv, dk), dtype=np.float32)) for l in lens]
    vs = None if latent else [synth.bf16_from_f32(rng.standard_normal((l, hkv, dv), dtype=np.float32)) for l in lens]
    q = synth.bf16_from_f32(rng.standard_normal((B, hq, dk), dtype=np.float32))
    k_scale = v_scale = None
    if kv_dtype == synth.KV_FP8 and not latent:
        kam = np.max([np.abs(synth.bf16_to_f32(k)).max(axis=(0, 2)) for k in ks if len(k)], axis=0)
        vam = np.max([np.abs(synth.bf16_to_f32(v)).max(axis=(0, 2)) for v in vs if len(v)], axis=0)
        k_scale = (kam / np.float32(448)).astype(np.float32)
        v_scale = (vam / np.float32(448)).astype(np.float32)
    return dict(lens=np.asarray(lens, np.int32), P=P, bt=bt, ks=ks, vs=vs, q=q,
                k_scale=k_scale, v_scale=v_scale, S=S, hq=hq, hkv=hkv, dk=dk,
                dv=dv, kv_dtype=kv_dtype, latent=latent,
                sm_scale=1.0 / math.sqrt(dk))


def slots_of(bt_row, S, n):
    t = np.arange(n, dtype=np.int64)
    return bt_row[t // S].astype(np.int64) * S + t % S


def oracle_caches(pr, fill=None):
    """Write every token of a small problem into fresh caches with the
    oracle's kv_write. Returns (k_cache, v_cache, token_scale)."""
    import oracle
    P, S, hkv, dk, dv = pr["P"], pr["S"], pr["hkv"], pr["dk"], pr["dv"]
    fp8 = pr["kv_dtype"] == synth.KV_FP8
    dt = np.uint8 if fp8 else np.uint16
    if fill is None:
        fill = synth.poison_value(pr["kv_dtype"])
    kc = np.full(P * hkv * S * dk, fill, dt)
    vc = None if pr["latent"] else np.full(P * hkv * S * dv, fill, dt)
    ts = np.full(P * S, np.nan, np.float32) if pr["latent"] else None
    for s, l in enumerate(pr["lens"]):
        if l == 0:
            continue
        slots = slots_of(pr["bt"][s], S, int(l))
        v = None if pr["latent"] else pr["vs"][s]
        if fp8:
            mode = synth.SCALE_PER_TOKEN if pr["latent"] else synth.SCALE_PER_HEAD
            oracle.kv_write_fp8(pr["ks"][s], v, slots, S, P, mode,
                                None if pr["latent"] else pr["k_scale"],
                                None if pr["latent"] else pr["v_scale"],
                                ts, kc, vc)
        else:
            oracle.kv_write_bf16(pr["ks"][s], v, slots, S, P, kc, vc)
    return kc, vc, ts


def oracle_attn(pr, kc, vc, ts=None, verdict=None, bt=None, lens=None, **kw):
    import oracle
    if pr["latent"]:
        mode = synth.SCALE_PER_TOKEN
    elif pr["kv_dtype"] == synth.KV_FP8:
        mode = synth.SCALE_PER_HEAD
    else:
        mode = synth.SCALE_NONE
    return oracle.paged_decode_attn(
        pr["q"], kc, vc, ts if pr["latent"] else pr["k_scale"],
        None if pr["latent"] else pr["v_scale"],
        pr["bt"] if bt is None else bt, pr["lens"] if lens is None else lens,
        num_kv_heads=pr["hkv"], head_dim_v=pr["dv"], page_size=pr["S"],
        num_pages=pr["P"], kv_dtype=pr["kv_dtype"], scale_mode=mode,
        v_in_k=pr["latent"], sm_scale=kw.pop("sm_scale", pr["sm_scale"]),
        verdict=verdict, **kw)


def dense_reference(pr, ts=None, sm_scale=None):
    B = len(pr["lens"])
    out = np.zeros((B, pr["hq"], pr["dv"]))
    for s in range(B):
        l = int(pr["lens"][s])
        if l == 0:
            continue
        tok = None
        if pr["latent"]:
            tok = ts[slots_of(pr["bt"][s], pr["S"], l)]
        kh, vh = dequant_dense(pr["ks"][s], None if pr["latent"] else pr["vs"][s],
                               pr["k_scale"], pr["v_scale"], pr["kv_dtype"], tok)
        out[s] = dense_attention(pr["q"][s], kh, vh,
                                 pr["sm_scale"] if sm_scale is None else sm_scale,
                                 pr["hq"] // pr["hkv"], v_in_k=pr["latent"],
                                 dv=pr["dv"])
    return out
