"""Pins of the oracle's W4A4 GEMM and its acceptance checks (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import nvfp4 as Q


def _random_nvfp4(rng, rows, cols, s_g=None):
    packed = rng.integers(0, 256, (rows, cols // 2)).astype(np.uint8)
    scales = rng.integers(0, 127, (rows, cols // 16)).astype(np.uint8)
    if s_g is None:
        s_g = float(np.float32(rng.uniform(1e-3, 1e-1)))
    return Q.NVFP4(packed, scales, s_g)


def _fraction_values(t):
    """Exact rational value of every element, decoded with an independent table."""
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
            Fraction(4), Fraction(6)]
    rows, cols = t.shape
    out = []
    for r in range(rows):
        row = []
        for c in range(cols):
            byte = int(t.packed[r, c // 2])
            code = byte & 0xF if c % 2 == 0 else byte >> 4
            v = mags[code & 7] * (-1 if code & 8 else 1)
            sb = int(t.scales[r, c // 16])
            e, m = sb >> 3, sb & 7
            s = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
            row.append(v * s * Fraction(t.s_g))
        out.append(row)
    return out


def test_exact_int_matmul_matches_integer_matmul():
    rng = np.random.default_rng(0)
    a = rng.integers(-(2**22) + 1, 2**22, (17, 300))
    b = rng.integers(-(2**22) + 1, 2**22, (300, 9))
    a[0, :] = 2**22 - 1
    b[:, 0] = -(2**22) + 1
    ref = a.astype(object) @ b.astype(object)
    assert np.array_equal(Q.exact_int_matmul(a, b).astype(object), ref)


@pytest.mark.parametrize("seed", [1, 2])
def test_gemm_matches_fraction_brute_force(seed):
    rng = np.random.default_rng(seed)
    x = _random_nvfp4(rng, 5, 64)
    w = _random_nvfp4(rng, 3, 64)
    y, a = Q.gemm(x, w)
    fx, fw = _fraction_values(x), _fraction_values(w)
    for i in range(5):
        for j in range(3):
            ey = sum(p * q for p, q in zip(fx[i], fw[j]))
            ea = sum(abs(p * q) for p, q in zip(fx[i], fw[j]))
            assert abs(Fraction(y[i, j]) - ey) <= abs(ey) * Fraction(1, 2**51)
            assert abs(Fraction(a[i, j]) - ea) <= ea * Fraction(1, 2**51)
    yp, ap = Q.gemm_pairs(x, w, [0, 4, 2], [1, 2, 0])
    assert np.array_equal(yp, y[[0, 4, 2], [1, 2, 0]]) or np.allclose(yp, y[[0, 4, 2], [1, 2, 0]], rtol=2**-50)


def test_gemm_integer_special_case():
    # s_g = 1 and every scale byte 0x38 (= 1.0): Y = sum_k q_x q_w, an integer matmul of 2q / 4
    rng = np.random.default_rng(5)
    m, n, k = 7, 6, 96
    cx = rng.integers(0, 16, (m, k)).astype(np.uint8)
    cw = rng.integers(0, 16, (n, k)).astype(np.uint8)
    x = Q.NVFP4(Q.pack_codes(cx), np.full((m, k // 16), 0x38, np.uint8), 1.0)
    w = Q.NVFP4(Q.pack_codes(cw), np.full((n, k // 16), 0x38, np.uint8), 1.0)
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12] * 2) * np.repeat([1, -1], 8)   # 2 * E2M1 by code
    ref = (twice[cx] @ twice[cw].T) / 4.0
    y, _ = Q.gemm(x, w)
    assert np.array_equal(y, ref)


def test_gemm_single_block_closed_form():
    # K = 16: Y = s_gx s_gw s_bx s_bw sum_k q_x q_w
    rng = np.random.default_rng(9)
    cx = rng.integers(0, 16, (1, 16)).astype(np.uint8)
    cw = rng.integers(0, 16, (1, 16)).astype(np.uint8)
    sx, sw = 0x45, 0x2A
    gx, gw = float(np.float32(0.37)), float(np.float32(1.9e-3))
    x = Q.NVFP4(Q.pack_codes(cx), np.array([[sx]], np.uint8), gx)
    w = Q.NVFP4(Q.pack_codes(cw), np.array([[sw]], np.uint8), gw)
    qx = np.array([F.e2m1_decode(c) for c in cx[0]])
    qw = np.array([F.e2m1_decode(c) for c in cw[0]])
    exact = Fraction(gx) * Fraction(gw) * Fraction(F.e4m3_decode(sx)) * Fraction(F.e4m3_decode(sw)) \
        * sum(Fraction(a) * Fraction(b) for a, b in zip(qx, qw))
    y, _ = Q.gemm(x, w)
    assert y[0, 0] == float(exact)


def test_check_gemm_bf16_accepts_neighbours_and_rejects_two_ulps():
    y_ref = np.array([1.0 + 2.0 ** -9, 3.0, -2.0])
    a_ref = np.array([1e-9, 1e-9, 1e-9])
    rb = F.round_f64_to_binary(y_ref, F.BF16)
    bits = F.f64_to_bf16_bits(rb)

    def away(n):   # the bf16 number n steps further from zero
        return F.bf16_bits_to_f64((bits + n).astype(np.uint16))

    ok, n_clause, n_fail = Q.check_gemm_bf16(away(1), y_ref, a_ref)
    assert ok and n_clause == 0
    ok, _, n_fail = Q.check_gemm_bf16(away(2), y_ref, a_ref)
    assert not ok and n_fail == 3


def test_check_gemm_bf16_cancellation_clause():
    # |Y_ref| tiny compared with A_ref: a value off by many ulps passes via the clause
    y_ref = np.array([1e-6] + [1.0] * 2000)
    a_ref = np.array([10.0] + [1.0] * 2000)
    y = F.round_f64_to_binary(y_ref, F.BF16)
    y[0] = 5e-3
    ok, n_clause, n_fail = Q.check_gemm_bf16(y, y_ref, a_ref)
    assert ok and n_clause == 1 and n_fail == 0


def test_check_gemm_f32():
    y_ref = np.array([1.0, -2.0])
    a_ref = np.array([100.0, 1.0])
    ok, _ = Q.check_gemm_f32(np.array([1.09, -2.0009]), y_ref, a_ref)
    assert ok
    ok, _ = Q.check_gemm_f32(np.array([1.0, -2.0011]), y_ref, a_ref)
    assert not ok
