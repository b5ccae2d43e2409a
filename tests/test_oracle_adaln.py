"""Pins of the fused LayerNorm + adaLN modulate + NVFP4 oracle (oracle/adaln.py), CPU only.

Each pin checks the oracle against something it does not compute itself:
numpy's IEEE fp32 arithmetic (one correctly rounded operation per ufunc call),
torch's float64 layer_norm, Fraction arithmetic, and closed forms.
"""

from fractions import Fraction

import numpy as np
import torch

import synth
from oracle import adaln as A
from oracle import formats as F
from oracle import nvfp4 as Q


def _inputs(rows, cols, rpg, seed):
    xb = synth.channel_outliers_bf16(rows, cols, seed=seed, ch_seed=seed + 1)
    x = F.bf16_bits_to_f64(xb)
    ng = -(-rows // rpg)
    shift, scale = synth.adaln_modulation(ng, cols, seed=seed + 2)
    return x, shift.astype(np.float64), scale.astype(np.float64)


def test_modulate_equals_eager_numpy_float32():
    """Each step is one IEEE fp32 operation: numpy float32 ufuncs give the same bits."""
    x, shift, scale = _inputs(37, 96, 5, seed=60)
    mu, rstd = A.row_stats(x, 1e-6)
    # a few special rows: x == mu (exact zeros), scale -1 (gain 0), scale < -1
    x[3] = x[3, 0]
    scale[1, :7] = -1.0
    scale[2, :9] = -3.5
    mu, rstd = A.row_stats(x, 1e-6)
    got = A.modulate(x, mu, rstd, shift, scale, 5)
    g = np.arange(37) // 5
    x32, mu32, r32 = x.astype(np.float32), mu.astype(np.float32), rstd.astype(np.float32)
    n = (x32 - mu32[:, None]) * r32[:, None]
    a = np.float32(1.0) + scale.astype(np.float32)[g]
    ref = n * a + shift.astype(np.float32)[g]
    assert ref.dtype == np.float32
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    assert np.array_equal(got, ref.astype(np.float64))


def test_row_stats_match_torch_layer_norm():
    """Biased variance, eps inside the square root: torch's layer_norm (no affine) in fp64."""
    x, _, _ = _inputs(64, 256, 64, seed=61)
    for eps in (1e-6, 0.5):
        mu, rstd = A.row_stats(x, eps)
        ln = torch.nn.functional.layer_norm(torch.from_numpy(x), (256,), eps=eps).numpy()
        ours = (x - mu[:, None]) * rstd[:, None]
        # mu and rstd are rounded to fp32 (2^-24 relative each)
        tol = 2.0 ** -22 * (np.abs(ln) + np.abs(mu[:, None] * rstd[:, None]))
        assert np.all(np.abs(ours - ln) <= tol)


def test_row_stats_exact_mean_and_fraction_variance():
    x, _, _ = _inputs(6, 48, 6, seed=62)
    eps = 1e-6
    mu, rstd = A.row_stats(x, eps)
    for r in range(6):
        s = sum(Fraction(v) for v in x[r])
        m = s / 48
        assert mu[r] == F.round_fraction_to_binary(m, F.F32)
        var = sum((Fraction(v) - m) ** 2 for v in x[r]) / 48
        want = 1.0 / np.sqrt(float(var + Fraction(float(np.float32(eps)))))
        assert abs(rstd[r] - want) <= 2.0 ** -23 * want


def test_modulate_fraction_brute_force():
    x, shift, scale = _inputs(4, 32, 2, seed=63)
    mu, rstd = A.row_stats(x, 1e-6)
    got = A.modulate(x, mu, rstd, shift, scale, 2)
    rn = lambda q: Fraction(F.round_fraction_to_binary(q, F.F32))   # noqa: E731
    for r in range(4):
        g = r // 2
        for c in range(32):
            n = rn(rn(Fraction(x[r, c]) - Fraction(mu[r])) * Fraction(rstd[r]))
            a = rn(1 + Fraction(scale[g, c]))
            want = rn(rn(n * a) + Fraction(shift[g, c]))
            assert Fraction(got[r, c]) == want


def test_alternating_rows_closed_form():
    """Rows +-8 alternating: mu 0, var 64, rstd 1/8 (eps below half an ulp),
    n = +-1, x' = 1.75 or -1.25 with scale 0.5, shift 0.25; NVFP4: the block
    holding the tensor amax gets scale 448 (0x7E), 1.75 -> code 7 (6 after
    scaling), -1.25 -> 4 after scaling -> code 0xE."""
    x = np.tile(np.array([8.0, -8.0]), (4, 8))
    shift = np.full((1, 16), 0.25)
    scale = np.full((1, 16), 0.5)
    t, mu, rstd = A.adaln_quantize(x, shift, scale, 4, 2.0 ** -30)
    assert np.all(mu == 0.0) and np.all(rstd == 0.125)
    assert t.s_g == float(np.float32(np.float32(1.75) / np.float32(2688)))
    assert np.all(t.scales == 0x7E)
    assert np.all(t.packed == 0xE7)


def test_constant_rows_take_their_group_shift():
    """x constant along a row: x - mu = +0, so x' = RN32(0 * a) + shift = shift of the row's group."""
    rows, cols, rpg = 7, 32, 3
    x = np.repeat(np.arange(1, rows + 1, dtype=np.float64)[:, None] * 0.375, cols, axis=1)
    shift = np.arange(3 * cols, dtype=np.float64).reshape(3, cols) * 0.5 - 7.0
    scale = np.full((3, cols), 0.25)
    mu, rstd = A.row_stats(x, 1e-6)
    assert np.array_equal(mu, x[:, 0])
    xp = A.modulate(x, mu, rstd, shift, scale, rpg)
    assert np.array_equal(xp, shift[np.arange(rows) // rpg])


def test_group_index_and_single_group():
    assert list(A.group_index(7, 3)) == [0, 0, 0, 1, 1, 1, 2]
    x, shift, scale = _inputs(10, 32, 10, seed=64)
    t1, _, _ = A.adaln_quantize(x, shift, scale, 10, 1e-6)
    t2, _, _ = A.adaln_quantize(x, np.repeat(shift, 10, axis=0), np.repeat(scale, 10, axis=0), 1, 1e-6)
    assert np.array_equal(t1.packed, t2.packed) and np.array_equal(t1.scales, t2.scales)


def test_zero_modulation_is_plain_layer_norm_then_quantize():
    """shift = scale = 0: x' is the fp32 LayerNorm output, and the NVFP4 tensor is its quantization."""
    x, shift, scale = _inputs(16, 64, 16, seed=65)
    t, mu, rstd = A.adaln_quantize(x, np.zeros_like(shift), np.zeros_like(scale), 16, 1e-6)
    n = (x.astype(np.float32) - mu.astype(np.float32)[:, None]) * rstd.astype(np.float32)[:, None]
    ref = Q.quantize(n.astype(np.float64))
    assert np.array_equal(t.packed, ref.packed) and np.array_equal(t.scales, ref.scales)
    assert t.s_g == ref.s_g
