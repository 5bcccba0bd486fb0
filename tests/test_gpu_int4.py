"""GPU parity of int4_gemv_bf16 (weight-only INT4 decode GEMV) against the
oracle's fp64 sum.

Inputs: bf16 activations N(0, 1) with exact zeros and negative zeros mixed
in, uniformly random packed words (every 4-bit code), bf16 scales of both
signs. Shapes span ragged row counts (not multiples of the 8 or 32 rows
of a workgroup), token counts from 1 (vector-ALU kernel) to 100 (matrix-core
kernel: partial 16-token tiles, two grid rows of 64 tokens) and k from one
scale group to 32768.

Tolerance, from the kernel's arithmetic: every term enters an fp32 chain
whose partial sums are bounded by 280 * sum|x| * |scale| per 16-element
chunk (codes are offset by 136 and the offset is subtracted at the head of
the chain), with under 8192 roundings on any path, so
|y - exact| <= 8192 * 2^-24 * sum_k |x_k| * |scale_k|; on top, the
root-mean-square error over all outputs must stay under 1e-5 of the
outputs' own root mean square (a statistical guard: measured at most
3e-7 for the vector-ALU kernel and 1.6e-6 for the matrix-core kernel,
whose group sums cancel the 136 offset between two fp32 accumulators,
while a single wrong code moves an output by about |x| * |scale|, ~1e-3
of it).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import log

pytestmark = pytest.mark.gpu

GUARD = 64


def _inputs(m, n, k, seed):
    rng = np.random.default_rng(seed)
    xf = rng.standard_normal((m, k)).astype(np.float32)
    xf[rng.random((m, k)) < 0.02] = 0.0
    xf[rng.random((m, k)) < 0.02] = -0.0
    x = synth.bf16_from_f32(xf)
    w = rng.integers(0, 1 << 32, (n, k // 8), dtype=np.uint64).astype(np.uint32)
    s = synth.bf16_from_f32(rng.uniform(-0.05, 0.05, (n, k // 128)).astype(np.float32))
    return x, w, s


def _bound(x, s, cols):
    xa = np.abs(synth.bf16_to_f32(x).astype(np.float64))
    sa = np.abs(synth.bf16_to_f32(s).astype(np.float64))[cols]
    sx = np.repeat(sa, 128, axis=1)                       # [cols][k]
    return 8192 * 2.0 ** -24 * (xa @ sx.T) + 1e-30


def _run(gpu, x, w, s):
    m, n = x.shape[0], w.shape[0]
    buf = torch.full((m * n + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    buf[m * n:] = 12345.0
    y = buf[:m * n].view(m, n)
    gpu.int4_gemv_bf16(torch.from_numpy(x.view(np.int16)).cuda(),
                       torch.from_numpy(w.view(np.int32)).cuda(),
                       torch.from_numpy(s.view(np.int16)).cuda(), y)
    torch.cuda.synchronize()
    out = buf.cpu().numpy()
    assert (out[m * n:] == 12345.0).all(), "write past the output"
    return out[:m * n].reshape(m, n).astype(np.float64)


def _compare(got, ref, bound, what):
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: unwritten or non-finite outputs"
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    log(f"{what}: max err {err.max():.3e}, worst err/bound {(err / bound).max():.3e} at {worst}")
    assert (err <= bound).all(), f"{what}: error above the bound at {worst}"
    rel = np.sqrt((err ** 2).mean()) / max(np.sqrt((ref ** 2).mean()), 1e-30)
    log(f"{what}: rms rel {rel:.3e}")
    assert rel <= 1e-5, f"{what}: rms relative error {rel:.3e}"


# (tokens, rows, k)
CASES = [(1, 16, 128), (1, 100, 384), (1, 21, 32768), (3, 37, 1024), (4, 64, 2048), (5, 33, 640),
         (8, 50, 8192), (13, 20, 256), (17, 7, 128), (2, 1, 1152), (40, 24, 256),
         (64, 33, 512), (100, 9, 128), (16, 32, 4096), (32, 70, 256), (33, 200, 1024)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"m{c[0]}_n{c[1]}_k{c[2]}")
def test_int4_gemv_parity(gpu, case):
    m, n, k = case
    log(f"int4 gemv parity m={m} n={n} k={k}")
    x, w, s = _inputs(m, n, k, seed=m * 7919 + n * 31 + k)
    ref, _ = oracle.int4_gemv(x, w, s)
    got = _run(gpu, x, w, s)
    _compare(got, ref, _bound(x, s, np.arange(n)), f"m{m} n{n} k{k}")


@pytest.mark.parametrize("m", [1, 8, 64])
def test_int4_gemv_full_size_sampled(gpu, m):
    """The measured shape, 8192 x 8192 weights: every output computed on the
    GPU, 96 sampled columns (first and last included) by the oracle."""
    n = k = 8192
    log(f"int4 gemv full size m={m}")
    x, w, s = _inputs(m, n, k, seed=4242 + m)
    got = _run(gpu, x, w, s)
    rng = np.random.default_rng(m)
    cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 94, replace=False)]))
    ref, _ = oracle.int4_gemv(x, w, s, cols=cols)
    _compare(got[:, cols], ref[:, cols], _bound(x, s, cols), f"full m{m}")
