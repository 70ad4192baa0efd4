"""Parity of the fp8 matrix-instruction GEMM (fs_gemm_f8, the kernel behind an
fp8 model's prefill Q/K/V and gate/up products) with the oracle's product.

The operands are quantized on the CPU by the oracle's rule (oracle/fp8.py:
e4m3 codes, one power-of-two scale per row), so the GPU multiplies exactly
the codes the oracle does.  The oracle's result is the float64 sum of
(code * scale) products, exact here.  Each product of two e4m3 values is
exact in fp32 and the scales are powers of two, so the GPU's only error is
its summation.  Round-to-nearest fp32 additions in any order would stay within
K * 2^-24 * sum_k |a_k w_k| of the exact sum (the recursive-summation bound
gamma_K); the matrix unit's adder for the 64 products of one instruction is
not documented as round-to-nearest, and it breaks that bound (measured 1.05 x
it on a single K = 64 instruction and up to 2.6 x it over these shapes), so
the bound tested allows a unit roundoff of 2^-22 per addition:
K * 2^-22 * sum_k |a_k w_k|.  A swapped scale, a dropped
or misplaced 16-value K chunk moves an output by at least 16 / K of that sum,
far outside it.
Shapes span one stage (K = 64), K not a multiple of the ring or unroll depth,
ragged M and N edges, the model's products, and the full 4 x 4096-token
Q/K/V product on sampled outputs.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import fp8 as F

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    from tests.gpu_common import need_gpu
    need_gpu()


def _quant(x):
    vals, scales = F.quantize_rows(x)
    return vals, scales, F.e4m3_code(vals)


def _operands(seed, M, N, K):
    a = synth.activation_rows(seed, M, K)
    w = synth.activation_rows(seed + 1, N, K) * np.float32(0.02)
    return _quant(a), _quant(w)


def _run(A, W, M, N, K):
    from dense_gqa_transformer_amd.model import gemm_f8
    av, asc, ac = A
    wv, wsc, wc = W
    dev = lambda t: torch.from_numpy(np.ascontiguousarray(t)).cuda()
    out = gemm_f8(dev(ac), dev(asc), dev(wc), dev(wsc))
    torch.cuda.synchronize()
    return out


def _bound_check(g, exact, mag, K, what):
    assert np.all(np.isfinite(g)), what
    bound = K * 2.0 ** -22 * mag + 1e-30
    worst = float(np.max(np.abs(g - exact) / bound))
    assert worst <= 1.0, f"{what}: error {worst:.3g} x the summation bound"
    return worst


def _check(got, A, W, what):
    """Every output of got [M, N] against the exact product."""
    av, asc, _ = A
    wv, wsc, _ = W
    a = av * asc[:, None].astype(np.float64)
    w = wv * wsc[:, None].astype(np.float64)
    return _bound_check(got, a @ w.T, np.abs(a) @ np.abs(w).T, av.shape[1], what)


def _check_pairs(g, A, W, rows, cols, what):
    """Sampled outputs g[i] = C[rows[i], cols[i]] against the exact product."""
    av, asc, _ = A
    wv, wsc, _ = W
    a = av[rows] * asc[rows, None].astype(np.float64)
    w = wv[cols] * wsc[cols, None].astype(np.float64)
    return _bound_check(g, np.einsum("ik,ik->i", a, w), np.einsum("ik,ik->i", np.abs(a), np.abs(w)),
                        av.shape[1], what)


@pytest.mark.parametrize("M,N,K", [(1, 8, 64), (3, 40, 192), (37, 200, 704), (256, 256, 640),
                                   (300, 520, 1024), (1100, 4096, 1024), (512, 1024, 3072),
                                   (700, 6144, 1024), (129, 1032, 2048)])
def test_gemm_f8_matches_oracle(M, N, K):
    A, W = _operands(7000 + M + N + K, M, N, K)
    got = _run(A, W, M, N, K).cpu().numpy().astype(np.float64)
    worst = _check(got, A, W, f"fs_gemm_f8 {M}x{N}x{K}")
    print(f"fs_gemm_f8 {M}x{N}x{K}: worst {worst:.3g} of the bound", flush=True)


def test_gemm_f8_special_rows():
    # zero rows (scale 0), saturated rows, rows of subnormal codes, one huge and one tiny scale
    M, N, K = 64, 96, 256
    rng = np.random.default_rng(5)
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[3] = 0.0
    a[5] = 448.0 * np.sign(a[5])
    a[6] = rng.standard_normal(K).astype(np.float32) * np.float32(2.0 ** -100)
    a[7] = rng.standard_normal(K).astype(np.float32) * np.float32(2.0 ** 60)
    a[8, :] = 0.0
    a[8, 10] = 1.0                                          # everything else zero
    a[9] = np.linspace(-1, 1, K, dtype=np.float32) * np.float32(2.0 ** -9)
    w = rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
    w[0] = 0.0
    A, W = _quant(a), _quant(w)
    got = _run(A, W, M, N, K).cpu().numpy().astype(np.float64)
    _check(got, A, W, "fs_gemm_f8 special rows")
    assert np.all(got[3] == 0.0) and np.all(got[:, 0] == 0.0)


def test_gemm_f8_full_size_qkv_sampled():
    # the Q/K/V product of a 4 x 4096-token prefill of the 0.6B shape, checked
    # on sampled outputs (every tile edge of the last tile row / column included)
    M, N, K = 4 * 4096, 4096, 1024
    A, W = _operands(9100, M, N, K)
    got = _run(A, W, M, N, K)
    rng = np.random.default_rng(9101)
    rows = np.concatenate([rng.integers(0, M, 3000), np.full(64, M - 1), np.arange(64)])
    cols = np.concatenate([rng.integers(0, N, 3000), np.arange(N - 64, N), np.arange(64)])
    g = got[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy().astype(np.float64)
    worst = _check_pairs(g, A, W, rows, cols, "fs_gemm_f8 16384x4096x1024 sampled")
    print(f"fs_gemm_f8 16384x4096x1024 sampled: worst {worst:.3g} of the bound", flush=True)
