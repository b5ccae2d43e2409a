"""Pins of the oracle's number formats and exact rounding helpers (CPU only).

Each test checks the oracle against something other than itself: a library
conversion (torch float8_e4m3fn, numpy float32 casts, torch bfloat16), values
from the pages, a table typed from the OCP Microscaling E2M1 definition, or
exact rational arithmetic.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


def _golden(path):
    out = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split()
            out[k] = float(v)
    return out


# ---------------------------------------------------------------- E2M1


def test_e2m1_table_matches_ocp_values():
    # OCP MX v1.0 E2M1 magnitudes for codes 0..7, typed in by hand
    expected = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [F.e2m1_decode(c) for c in range(8)] == expected
    for c in range(8):
        v = F.e2m1_decode(c + 8)
        assert v == -expected[c] and math.copysign(1.0, v) == -1.0  # 0x8 is -0.0


def test_e2m1_is_finer_near_zero(golden_dir):
    # techwalker section 一: non-uniform spacing, finer for small values
    facts = _golden(os.path.join(golden_dir, "format_facts.txt"))
    assert 2 ** int(facts["value_bits"]) == 16
    gaps = np.diff(F.E2M1_MAGNITUDES[1:])
    assert np.all(np.diff(gaps) >= 0) and gaps[-1] > gaps[0]


def test_e2m1_midpoints():
    assert list(F.E2M1_MIDPOINTS) == [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


# ---------------------------------------------------------------- E4M3


def test_e4m3_all_bytes_match_torch_float8_e4m3fn():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = F.E4M3_TABLE
    assert np.array_equal(np.isnan(lib), np.isnan(ours))
    ok = ~np.isnan(lib)
    assert np.array_equal(lib[ok], ours[ok])
    assert np.array_equal(np.signbit(lib[ok]), np.signbit(ours[ok]))


def test_e4m3_grid_and_constants():
    assert F.E4M3_GRID.size == 127 and F.E4M3_MAX == 448.0
    assert np.all(np.diff(F.E4M3_GRID) > 0)
    assert F.E4M3_GRID[1] == 2.0 ** -9           # smallest subnormal
    assert 6 * F.E4M3_MAX == 2688


# ---------------------------------------------------------------- rounding helpers


def _rng():
    return np.random.default_rng(1234)


def test_round_f64_to_f32_matches_numpy_cast():
    rng = _rng()
    v = rng.standard_normal(200000) * np.exp2(rng.integers(-150, 100, 200000))
    # exact midpoints of fp32 and their neighbours
    base = rng.standard_normal(2000).astype(np.float32).astype(np.float64)
    mids = base + np.ldexp(1.0, np.frexp(base)[1] - 25)
    v = np.concatenate([v, mids, np.nextafter(mids, 0), np.nextafter(mids, 10), [0.0, -0.0]])
    ours = F.round_f64_to_binary(v, F.F32)
    lib = v.astype(np.float32).astype(np.float64)
    assert np.array_equal(ours, lib)


def test_round_f64_to_bf16_matches_torch_on_f32_inputs():
    rng = _rng()
    v32 = (rng.standard_normal(200000) * np.exp2(rng.integers(-140, 100, 200000))).astype(np.float32)
    # bf16 midpoints exactly
    b = torch.from_numpy(rng.standard_normal(5000).astype(np.float32)).to(torch.bfloat16).float().numpy()
    mids = (b.astype(np.float64) + np.ldexp(1.0, np.frexp(b.astype(np.float64))[1] - 9)).astype(np.float32)
    v32 = np.concatenate([v32, mids])
    lib = torch.from_numpy(v32).to(torch.bfloat16).double().numpy()
    ours = F.round_f64_to_binary(v32.astype(np.float64), F.BF16)
    assert np.array_equal(ours, lib)


def _frac_round(fr, fmt):
    return F.round_fraction_to_binary(fr, fmt)


def test_round_fraction_matches_numpy_for_exact_doubles():
    rng = _rng()
    v = rng.standard_normal(3000) * np.exp2(rng.integers(-149, 60, 3000))
    for x in v:
        assert _frac_round(Fraction(float(x)), F.F32) == float(np.float32(x))


def test_round_fraction_thirds_by_hand():
    # 1/3 = 0.0101..b; fp32 keeps 24 bits: 0x3EAAAAAB
    assert np.float32(_frac_round(Fraction(1, 3), F.F32)).view(np.uint32) == 0x3EAAAAAB
    # bf16(1/3) = 0x3EAB
    v = np.float32(_frac_round(Fraction(1, 3), F.BF16)).view(np.uint32)
    assert v == 0x3EAB0000
    # ties to even: 1 + 2^-24 -> 1.0 ; 1 + 3*2^-24 -> 1 + 2^-22
    assert _frac_round(Fraction(1) + Fraction(1, 2**24), F.F32) == 1.0
    assert _frac_round(Fraction(1) + Fraction(3, 2**24), F.F32) == 1.0 + 2.0 ** -22


def test_round_sum_matches_fractions():
    rng = _rng()
    n = 4000
    a = (rng.standard_normal(n) * np.exp2(rng.integers(-40, 10, n))).astype(np.float32).astype(np.float64)
    c = (rng.standard_normal(n) * np.exp2(rng.integers(-40, 10, n))).astype(np.float32).astype(np.float64)
    # force sums that sit exactly on bf16 midpoints plus a tiny extra term
    mid = np.float32(1.0 + 2.0 ** -8)
    a[:200] = float(mid)
    c[:200] = np.ldexp(rng.choice([-1.0, 1.0], 200), rng.integers(-80, -30, 200))
    a[200:210] = float(mid)
    c[200:210] = 0.0
    for fmt in (F.BF16, F.F32):
        ours = F.round_sum_to_binary(a, c, fmt)
        ref = [_frac_round(Fraction(float(x)) + Fraction(float(y)), fmt) for x, y in zip(a, c)]
        assert np.array_equal(ours, np.array(ref))


# ---------------------------------------------------------------- golden storage ratio


def test_storage_ratio_printed_on_pages(golden_dir):
    g = _golden(os.path.join(golden_dir, "storage_ratio.txt"))
    facts = _golden(os.path.join(golden_dir, "format_facts.txt"))
    per_value = facts["value_bits"] / 8 + facts["block_scale_bits"] / 8 / facts["block_size"]
    assert per_value == 0.5625
    assert 2 * per_value == g["bytes_per_two_values"]
    ratio = g["bf16_bytes_per_two_values"] / (2 * per_value)
    assert abs(ratio - g["ratio"]) <= g["ratio_abs_tolerance"]
