"""Pins of the training-side GEMM oracle (oracle/training.py), CPU only.

Closed forms: the block orientation of the transposed quantizer read off its
scale bytes, and dgrad / wgrad on operands that NVFP4 represents exactly along
the contraction axis (then the 4-bit products equal numpy's fp64 matmul of
the original matrices, which are small dyadic numbers, exactly)."""

import numpy as np

from oracle import formats as F
from oracle import nvfp4 as Q
from oracle import training as T

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def test_transposed_blocks_run_along_rows():
    """s_g = 1 (amax 2688); block (column k, rows 16b..16b+15) holds 6 v_kb, so
    its scale byte is the E4M3 byte of v_kb and that element's code is 7."""
    m, k = 48, 32
    rng = np.random.default_rng(0)
    x = np.zeros((m, k))
    e4m3_vals = F.E4M3_GRID[1:0x7F]
    v = rng.choice(e4m3_vals[e4m3_vals >= 2.0 ** -6], size=(k, m // 16))
    v[0, 0] = 448.0
    for kk in range(k):
        for b in range(m // 16):
            x[16 * b + (kk * 7 + b) % 16, kk] = 6.0 * v[kk, b]
    t = T.quantize_transposed(x)
    assert t.s_g == 1.0 and t.shape == (k, m)
    assert np.array_equal(F.E4M3_GRID[t.scales], v)
    codes = Q.unpack_codes(t.packed)
    for kk in range(k):
        for b in range(m // 16):
            assert codes[kk, 16 * b + (kk * 7 + b) % 16] == 7


def _exact_along_rows(m, k, seed):
    """[m x k] with values 1.75 q (q on the E2M1 grid, random sign) and +-10.5 once
    in every (column, 16-row block): NVFP4 with blocks along the rows stores it
    exactly (s_g = 2^-8, every block scale 448)."""
    rng = np.random.default_rng(seed)
    x = 1.75 * rng.choice(GRID, size=(m, k)) * rng.choice([-1.0, 1.0], size=(m, k))
    for b in range(m // 16):
        r = 16 * b + rng.integers(0, 16, size=k)
        x[r, np.arange(k)] = 10.5 * rng.choice([-1.0, 1.0], size=k)
    return x


def test_exact_operands_round_trip_only_along_their_blocks():
    x = _exact_along_rows(64, 48, seed=1)
    t = T.quantize_transposed(x)
    assert t.s_g == 2.0 ** -8 and np.all(t.scales == 0x7E)
    assert np.array_equal(Q.dequantize(t, "f32"), x.T)
    # blocked along the other axis the same matrix is not exact: orientation matters
    assert not np.array_equal(Q.dequantize(Q.quantize(x), "f32"), x)


def test_wgrad_equals_exact_matmul():
    m, n, k = 64, 32, 48                   # tokens, out features, in features
    x = _exact_along_rows(m, k, seed=2)
    dy = _exact_along_rows(m, n, seed=3)
    y, a = T.wgrad(T.quantize_transposed(dy), T.quantize_transposed(x))
    assert y.shape == (n, k)
    assert np.array_equal(y, dy.T @ x)
    assert np.array_equal(a, np.abs(dy.T) @ np.abs(x))


def test_dgrad_equals_exact_matmul():
    m, n, k = 48, 64, 32
    w = _exact_along_rows(n, k, seed=4)            # W [N x K], blocks along N when transposed
    dy = _exact_along_rows(n, m, seed=5).T.copy()  # dY [M x N], exact with blocks along N
    y, _ = T.dgrad(Q.quantize(dy), T.quantize_transposed(w))
    assert y.shape == (m, k)
    assert np.array_equal(y, dy @ w)
