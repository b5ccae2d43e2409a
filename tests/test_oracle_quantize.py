"""Pins of the oracle's NVFP4 quantize / dequantize (CPU only).

The brute-force reference here is written independently of the oracle: it
works on exact rationals and picks the nearest grid value by minimising the
distance (ties to the even code), instead of counting midpoints.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import nvfp4 as Q

# ---------------------------------------------------------------- brute force

E2M1_MAGS = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
E4M3_VALS = []
for byte in range(0x7F):
    e, m = byte >> 3, byte & 7
    E4M3_VALS.append(Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))


def _nearest_even(value, grid):
    """Index of the grid value nearest to ``value`` (ties to the even index)."""
    best = None
    for i, g in enumerate(grid):
        d = abs(value - g)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def _to_f32(fr):
    # RN32 of a rational by bisection over float32 neighbours (independent of oracle code)
    x = np.float32(float(fr))            # within one ulp
    cands = [np.nextafter(x, np.float32(-np.inf)), x, np.nextafter(x, np.float32(np.inf))]
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - fr)
        even = (np.float32(c).view(np.uint32) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, float(c))
    return best[1]


def brute_quantize(x):
    """(codes [rows, cols], scale bytes [rows, cols/16], s_g) from exact rationals."""
    rows, cols = x.shape
    fx = [[Fraction(float(v)) for v in row] for row in x]
    amax = max((abs(v) for row in fx for v in row), default=Fraction(0))
    s_g = Fraction(1) if amax == 0 else Fraction(_to_f32(amax / 2688))
    codes = np.zeros((rows, cols), dtype=np.uint8)
    sbytes = np.zeros((rows, cols // 16), dtype=np.uint8)
    for r in range(rows):
        for kb in range(cols // 16):
            blk = fx[r][16 * kb:16 * kb + 16]
            b = max(abs(v) for v in blk)
            sb = _nearest_even(b / (6 * s_g), E4M3_VALS)
            sbytes[r, kb] = sb
            s_b = E4M3_VALS[sb]
            for j, v in enumerate(blk):
                mag = 0 if s_b == 0 else _nearest_even(abs(v) / (s_b * s_g), E2M1_MAGS)
                neg = math.copysign(1.0, float(x[r, 16 * kb + j])) < 0
                codes[r, 16 * kb + j] = mag | (8 if neg else 0)
    return codes, sbytes, float(s_g)


def _check_against_brute(x, amax=None):
    q = Q.quantize(x)
    codes, sbytes, s_g = brute_quantize(x)
    assert q.s_g == s_g
    assert np.array_equal(q.scales, sbytes)
    assert np.array_equal(Q.unpack_codes(q.packed), codes)


# ---------------------------------------------------------------- tests vs brute force


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quantize_random_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    x[rng.random(x.shape) < 0.05] *= 30
    x[0, :16] *= 1e-4                       # a block far below the tensor amax
    _check_against_brute(x.astype(np.float64))


def test_quantize_ties_and_tiny_blocks_match_brute_force():
    # s_g = 1 (amax 2688); blocks whose values sit exactly on E2M1 midpoints
    x = np.zeros((2, 48))
    x[0, 0] = 2688.0
    x[0, 16:32] = [6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, -5, 0, -0.0, 0.1, 4.5, 5.5]
    x[1, :16] = 6 * 2.0 ** -10 * np.array([1] + [0.3] * 15)   # t = 2^-10: scale byte 0
    x[1, 16:32] = 6 * 1.5 * 2.0 ** -9 * np.array([1] + [0.25] * 15)  # t = 1.5*2^-9
    x[1, 32:48] = -1e-30
    _check_against_brute(x)


def test_e2m1_ties_by_hand():
    # s_g = 1, block amax 6 -> t = 1 -> s_b = 1.0 (byte 0x38); codes of exact ties
    x = np.zeros((1, 32))
    x[0, 0] = 2688.0
    x[0, 16:24] = [6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    q = Q.quantize(x)
    assert q.s_g == 1.0 and q.scales[0, 1] == 0x38
    got = Q.unpack_codes(q.packed)[0, 16:24]
    # RNE ties: 0.25->0, 0.75->1.0(2), 1.25->1.0(2), 1.75->2.0(4), 2.5->2.0(4), 3.5->4.0(6), 5->4.0(6)
    assert list(got) == [7, 0, 2, 2, 4, 4, 6, 6]


def test_e4m3_scale_rounding_matches_torch():
    # s_g = 1: s_b = E4M3_RNE(b / 6).  For b = 6 v with v fp32, b / 6 = v exactly,
    # so torch's float32 -> float8_e4m3fn RNE conversion is an independent reference.
    rng = np.random.default_rng(7)
    grid = F.E4M3_GRID
    mids = (grid[:-1] + grid[1:]) / 2
    v = np.concatenate([grid, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        rng.uniform(0, 448, 100000), np.exp2(rng.uniform(-14, 8.8, 100000))])
    v = v.astype(np.float32).astype(np.float64)
    v = v[v <= 448]
    ours = Q.block_scale_bytes(6.0 * v, 1.0)
    lib = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, lib)
    # saturation above 448 (torch would give NaN past 464)
    assert np.all(Q.block_scale_bytes(6.0 * np.array([449.0, 470.0, 1e6]), 1.0) == 0x7E)


def test_block_holding_amax_gets_scale_0x7e_and_code_7():
    rng = np.random.default_rng(3)
    for _ in range(20):
        x = rng.standard_normal((8, 128)) * np.exp2(rng.integers(-20, 20))
        x = x.astype(np.float32).astype(np.float64)
        q = Q.quantize(x)
        r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        assert q.scales[r, c // 16] == 0x7E
        assert Q.unpack_codes(q.packed)[r, c] & 7 == 7


def test_small_scale_case_amax_code_4():
    # t = 1.5 * 2^-9 rounds to s_b = 2^-8 (tie, to even byte 0x02); r = 4.5 -> magnitude 4
    x = np.zeros((1, 32))
    x[0, 0] = 2688.0
    x[0, 16] = 6 * 1.5 * 2.0 ** -9
    q = Q.quantize(x)
    assert q.scales[0, 1] == 0x02
    assert Q.unpack_codes(q.packed)[0, 16] == 6          # magnitude 4.0 is code 6


def test_zero_tensor_and_signed_zeros():
    x = np.zeros((2, 32))
    x[1, 3] = -0.0
    q = Q.quantize(x)
    assert q.s_g == 1.0 and np.all(q.scales == 0)
    codes = Q.unpack_codes(q.packed)
    assert codes[1, 3] == 8 and np.sum(codes) == 8


def test_round_trip_of_representable_values():
    # values q * s_b * s_g with each block holding a magnitude 6 element round-trip exactly
    rng = np.random.default_rng(11)
    s_g = float(np.float32(0.0123))
    rows, cols = 16, 64
    sb = F.E4M3_GRID[rng.integers(1, 127, (rows, cols // 16))]
    qm = F.E2M1_MAGNITUDES[rng.integers(0, 8, (rows, cols))]
    qm.reshape(rows, cols // 16, 16)[:, :, 0] = 6.0
    sign = rng.choice([-1.0, 1.0], (rows, cols))
    x = sign * qm * np.repeat(sb, 16, axis=1) * s_g
    amax = 2688.0 * s_g                      # force s_g exactly (the tensor amax may be smaller)
    assert Q.global_scale(amax) == s_g
    q = Q.quantize(x, amax=amax)
    assert np.array_equal(Q.dequantize(q, "f32"), F.round_f64_to_binary(x, F.F32))
    assert np.array_equal(Q.decoded_qsb(q) * s_g, x)


def test_global_scale_by_hand():
    assert Q.global_scale(2688.0) == 1.0
    assert Q.global_scale(0.0) == 1.0
    # 1 / 2688 rounded to fp32 by hand: 2688 = 21 * 2^7; 1/21 = 0.000011000011..b
    assert Q.global_scale(1.0) == float(np.float32(1.0) / np.float32(2688.0))


def test_global_scale_subnormal_and_underflow():
    # 2688 * 2^-149 = 21 * 2^-142 is an fp32 subnormal and gives s_g = 2^-149 exactly
    assert Q.global_scale(21.0 * 2.0 ** -142) == 2.0 ** -149
    # 2^-140 / 2688 = 2^-147 / 21 is below half of 2^-149: RN32 gives 0, read as 2^-149
    assert Q.global_scale(2.0 ** -140) == 2.0 ** -149
    # a subnormal quotient that rounds normally: 2^-120 / 2688 = 2^-127 / 21, and
    # 2^-127 / 21 = 2^-149 * (2^22 / 21) rounds to 199729 * 2^-149 (2^22 / 21 = 199728.76)
    assert Q.global_scale(2.0 ** -120) == 199729 * 2.0 ** -149
    # every block scale and code stays defined: the largest block of a tensor with that
    # s_g takes byte 0x7E (448), exactly as for a normal s_g
    x = np.zeros((1, 16))
    x[0, 0] = 2.0 ** -140
    q = Q.quantize(x)
    assert q.s_g == 2.0 ** -149 and int(q.scales[0, 0]) <= 0x7E


# ---------------------------------------------------------------- packing & layouts


def test_pack_hand_built_row():
    codes = np.array([[0x1, 0x2, 0xF, 0x8, 0x7, 0x0]], dtype=np.uint8)
    assert list(Q.pack_codes(codes)[0]) == [0x21, 0x8F, 0x07]
    assert np.array_equal(Q.unpack_codes(Q.pack_codes(codes)), codes)


def test_tiled_layout_offsets_by_hand():
    cols = 256                              # 16 blocks per row, 4 tiles of 64 columns
    assert Q.tiled_offset(0, 0, cols) == 0
    assert Q.tiled_offset(0, 3, cols) == 3
    assert Q.tiled_offset(1, 0, cols) == 4
    assert Q.tiled_offset(127, 3, cols) == 511
    assert Q.tiled_offset(0, 4, cols) == 512
    assert Q.tiled_offset(128, 0, cols) == 4 * 512
    assert Q.tiled_offset(130, 5, cols) == (4 + 1) * 512 + 2 * 4 + 1


def test_tiled_layout_is_a_bijection():
    rows, cols = 256, 192
    sb = np.random.default_rng(0).integers(0, 127, (rows, cols // 16)).astype(np.uint8)
    flat = Q.layout_scales(sb, Q.SCALES_TILED)
    r, kb = np.meshgrid(np.arange(rows), np.arange(cols // 16), indexing="ij")
    offs = Q.tiled_offset(r, kb, cols)
    assert np.unique(offs).size == offs.size and offs.max() == rows * cols // 16 - 1
    assert np.array_equal(Q.unlayout_scales(flat, rows, cols, Q.SCALES_TILED), sb)


# ---------------------------------------------------------------- dequantize


def test_dequantize_exhaustive_codes_and_scales():
    # every code x every finite non-negative scale byte, for s_g = 1 and two odd s_g
    codes = np.arange(16, dtype=np.uint8)
    for s_g in (1.0, float(np.float32(0.0123456)), float(np.float32(3.3e-30))):
        packed_rows, scale_rows = [], []
        for sb in range(0x7F):
            c = np.tile(codes, 2)[None, :32]
            packed_rows.append(Q.pack_codes(c)[0])
            scale_rows.append([sb, sb])
        t = Q.NVFP4(np.array(packed_rows), np.array(scale_rows), s_g)
        f32 = Q.dequantize(t, "f32")
        b16 = Q.dequantize(t, "bf16")
        for sb in range(0x7F):
            for j in range(16):
                exact = Fraction(F.e2m1_decode(j)) * Fraction(F.E4M3_GRID[sb]) * Fraction(s_g)
                assert f32[sb, j] == F.round_fraction_to_binary(exact, F.F32)
                assert b16[sb, j] == F.round_fraction_to_binary(exact, F.BF16)
                if j == 8:
                    assert math.copysign(1.0, f32[sb, j]) == -1.0


def test_dequantize_bf16_is_single_rounding_not_via_f32():
    # v = 1.5 * s_g sits just below the bf16 midpoint M = 2 + 2^-6 + 2^-7 (between the
    # odd 2 + 2^-6 and the even 2 + 2^-5).  RN32(v) = M (an fp32 tie resolved to the
    # even M), and RN_bf16(M) goes to the even 2 + 2^-5, but v < M so the single
    # rounding gives 2 + 2^-6.
    v = Fraction(2) + Fraction(1, 64) + Fraction(1, 128) - Fraction(1, 2**23)
    s_g = v / Fraction(3, 2)
    assert float(np.float32(float(s_g))) == float(s_g)
    t = Q.NVFP4(Q.pack_codes(np.array([[3] + [0] * 15], dtype=np.uint8)), np.array([[0x38]]), float(s_g))
    got = Q.dequantize(t, "bf16")[0, 0]
    assert got == F.round_fraction_to_binary(v, F.BF16) == 2.0 + 2.0 ** -6
    two_step = torch.tensor([float(np.float32(float(v)))]).to(torch.bfloat16).item()
    assert two_step == 2.0 + 2.0 ** -5       # the double rounding differs
