"""GPU parity of nvfp4_quantize / nvfp4_dequantize against the oracle (bit-exact)."""

import numpy as np
import pytest
import torch

import synth
from helpers import (assert_same_nvfp4, bf16_tensor, dev, f32_tensor, from_oracle, to_oracle)
from oracle import formats as F
from oracle import nvfp4 as Q

pytestmark = pytest.mark.gpu

import w4a4_gemm_amd as nv  # noqa: E402  (fails loudly when the library is missing)


def _quantize_and_compare(x64, x_dev, layout, amax=None):
    amax_t = None if amax is None else torch.tensor([amax], dtype=torch.float32, device=dev())
    got = to_oracle(nv.nvfp4_quantize(x_dev, layout=layout, amax=amax_t))
    want = Q.quantize(x64, amax=amax)
    assert_same_nvfp4(got, want)
    return got


@pytest.mark.parametrize("layout", [nv.SCALES_ROWMAJOR, nv.SCALES_TILED])
def test_tiny_fp32_round_trip(layout):
    d = synth.tiny()
    x = d["x"]
    q = _quantize_and_compare(x.astype(np.float64), f32_tensor(x), layout)
    t = from_oracle(q, layout)
    for dt, fmt in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        y = nv.nvfp4_dequantize(t, dt).float().cpu().numpy().astype(np.float64)
        want = Q.dequantize(q, fmt)
        assert np.array_equal(y, want), f"{fmt}: {np.sum(y != want)} values differ"


def test_attn_proj_activation_bf16_tiled():
    d = synth.attn_proj(m=512, k=3072, n=64)
    x64 = F.bf16_bits_to_f64(d["x"])
    _quantize_and_compare(x64, bf16_tensor(d["x"]), nv.SCALES_TILED)


def test_ragged_rows_and_cols_rowmajor():
    # 300 rows (not a multiple of 64), 592 columns (37 blocks: a 16-column tail group)
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((300, 592)) * np.exp2(rng.integers(-8, 8, (300, 1)))).astype(np.float32)
    bits = synth.to_bf16_bits(x)
    _quantize_and_compare(F.bf16_bits_to_f64(bits), bf16_tensor(bits), nv.SCALES_ROWMAJOR)
    _quantize_and_compare(x.astype(np.float64), f32_tensor(x), nv.SCALES_ROWMAJOR)


def test_seeded_shape_sweep():
    """24 seeded tensors: rows in [1, 600], cols a multiple of 16 up to 1600 (tiled layout
    where rows % 128 == 0 and cols % 64 == 0), row magnitudes spread over 2^-20 .. 2^20,
    fp32 or bf16 input, a third with the amax given; every byte bit-exact."""
    rng = np.random.default_rng(78)
    for i in range(24):
        r, c = int(rng.integers(1, 601)), 16 * int(rng.integers(1, 101))
        if i % 3 == 0:
            r, c = 128 * int(rng.integers(1, 5)), 64 * int(rng.integers(1, 26))
        x = (rng.standard_normal((r, c)) * np.exp2(rng.integers(-20, 21, (r, 1)))).astype(np.float32)
        layout = nv.SCALES_TILED if (r % 128 == 0 and c % 64 == 0) else nv.SCALES_ROWMAJOR
        amax = float(np.float32(np.max(np.abs(x)) * 1.5)) if i % 3 == 1 else None
        print(f"[sweep {i}] {r} x {c} layout {layout} amax {amax}", flush=True)
        if rng.integers(2):
            bits = synth.to_bf16_bits(x)
            _quantize_and_compare(F.bf16_bits_to_f64(bits), bf16_tensor(bits), layout, amax=amax)
        else:
            _quantize_and_compare(x.astype(np.float64), f32_tensor(x), layout, amax=amax)


def test_strided_input():
    rng = np.random.default_rng(6)
    big = rng.standard_normal((130, 256)).astype(np.float32)
    xd = f32_tensor(big)[:, :192]                 # row stride 256 > cols
    _quantize_and_compare(big[:, :192].astype(np.float64), xd, nv.SCALES_ROWMAJOR)


def test_exact_ties_and_special_blocks():
    x = np.zeros((64, 64), dtype=np.float32)
    x[0, 0] = 2688.0                              # s_g = 1
    ties = np.array([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, -5, 0, -0.0, 0.1, 4.5, 5.5])
    x[1, :16] = ties
    x[2, :16] = 6 * 2.0 ** -10 * np.array([1] + [0.3] * 15)       # scale byte 0
    x[3, :16] = 6 * 1.5 * 2.0 ** -9 * np.array([1] + [0.25] * 15)  # E4M3 tie, r = 4.5
    x[4, :16] = -1e-30
    x[5, 16:32] = -0.0
    # every E4M3 midpoint as a block amax (s_g = 1: b = 6 * midpoint)
    mids = (F.E4M3_GRID[:-1] + F.E4M3_GRID[1:]) / 2
    x[6:, 32:48] = 0.125
    flat = np.zeros(58 * 16)
    flat[: mids.size] = 6 * mids
    x[6:, 48:64] = flat.reshape(58, 16)
    # E2M1 ties under many scales: value = midpoint * s_b with s_b * 6 the block amax
    rng = np.random.default_rng(0)
    for r in range(6, 64):
        sb = F.E4M3_GRID[rng.integers(8, 120)]
        x[r, :16] = sb * rng.choice(F.E2M1_MIDPOINTS, 16)
        x[r, 0] = 6 * sb
    x = x.astype(np.float32)
    _quantize_and_compare(x.astype(np.float64), f32_tensor(x), nv.SCALES_ROWMAJOR)


def test_all_zero_and_signed_zero():
    x = np.zeros((64, 32), dtype=np.float32)
    x[7, 3] = -0.0
    got = _quantize_and_compare(x.astype(np.float64), f32_tensor(x), nv.SCALES_ROWMAJOR)
    assert got.s_g == 1.0


@pytest.mark.parametrize("scale", [2.0 ** -106, 2.0 ** -111, 2.0 ** -125, 2.0 ** -135,
                                   2.0 ** -145, 2.0 ** 100])
def test_extreme_tensor_scales(scale):
    # s_g < 2^-100 takes the pre-scaled encoder, down to subnormal s_g (2^-125 and
    # below, where 1 / (6 s_g) is beyond the fp32 range) and to an amax whose
    # quotient underflows (2^-145: s_g read as 2^-149); a huge scale stays in range too
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((64, 128)) * scale).astype(np.float32)
    got = _quantize_and_compare(x.astype(np.float64), f32_tensor(x), nv.SCALES_ROWMAJOR)
    if scale == 2.0 ** -145:
        assert got.s_g == 2.0 ** -149


@pytest.mark.parametrize("scale", [2.0 ** -125, 2.0 ** -135])
def test_subnormal_bf16_tensor(scale):
    rng = np.random.default_rng(19)
    bits = synth.to_bf16_bits((rng.standard_normal((128, 256)) * scale).astype(np.float32))
    x = synth.bf16_bits_to_f32(bits)
    _quantize_and_compare(x.astype(np.float64), bf16_tensor(bits), nv.SCALES_TILED)


def test_given_amax_path():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((128, 256)).astype(np.float32)
    amax = float(np.max(np.abs(x)) * np.float32(1.5))   # a producer's (larger) amax
    _quantize_and_compare(x.astype(np.float64), f32_tensor(x), nv.SCALES_TILED, amax=amax)


def test_empty_tensor():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=dev())
    t = nv.nvfp4_quantize(x, layout=nv.SCALES_ROWMAJOR)
    torch.cuda.synchronize()
    assert float(t.global_scale.cpu()[0]) == 1.0


def test_bf16_dequant_single_rounding_cases():
    # exhaustive codes x scale bytes with s_g chosen so fp32 products land on bf16 midpoints
    from fractions import Fraction
    v = Fraction(2) + Fraction(1, 64) + Fraction(1, 128) - Fraction(1, 2**23)
    s_gs = [float(v / Fraction(3, 2)), 1.0, float(np.float32(0.0123456)), float(np.float32(7.1e-3))]
    codes = np.tile(np.arange(16, dtype=np.uint8), 2)[None, :32]
    for s_g in s_gs:
        packed = np.repeat(Q.pack_codes(codes), 127, axis=0)
        scales = np.repeat(np.arange(127, dtype=np.uint8)[:, None], 2, axis=1)
        q = Q.NVFP4(packed, scales, s_g)
        t = from_oracle(q, nv.SCALES_ROWMAJOR)
        for dt, fmt in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
            y = nv.nvfp4_dequantize(t, dt).float().cpu().numpy().astype(np.float64)
            want = Q.dequantize(q, fmt)
            same = (y == want) & (np.signbit(y) == np.signbit(want))
            assert same.all(), f"s_g={s_g} {fmt}: {np.sum(~same)} differ"


def test_dequantize_large_random_bytes_both_layouts():
    rng = np.random.default_rng(12)
    rows, cols = 1024, 1024
    packed = rng.integers(0, 256, (rows, cols // 2)).astype(np.uint8)
    scales = rng.integers(0, 127, (rows, cols // 16)).astype(np.uint8)
    q = Q.NVFP4(packed, scales, float(np.float32(0.0377)))
    for layout in (nv.SCALES_ROWMAJOR, nv.SCALES_TILED):
        t = from_oracle(q, layout)
        for dt, fmt in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
            y = nv.nvfp4_dequantize(t, dt).float().cpu().numpy().astype(np.float64)
            assert np.array_equal(y, Q.dequantize(q, fmt))


def test_dequantize_seeded_shape_sweep():
    """16 seeded NVFP4 tensors of random bytes: rows in [1, 600], cols a multiple of 16 up
    to 1600 (tiled where rows % 128 == 0 and cols % 64 == 0), every finite scale byte,
    s_g over 2^-30 .. 2^30 with random significands; fp32 and bf16 output bit-exact."""
    rng = np.random.default_rng(82)
    for i in range(16):
        r, c = int(rng.integers(1, 601)), 16 * int(rng.integers(1, 101))
        if i % 4 == 0:
            r, c = 128 * int(rng.integers(1, 5)), 64 * int(rng.integers(1, 26))
        packed = rng.integers(0, 256, (r, c // 2)).astype(np.uint8)
        scales = rng.integers(0, 127, (r, c // 16)).astype(np.uint8)
        s_g = float(np.float32(rng.uniform(1.0, 2.0) * 2.0 ** int(rng.integers(-30, 31))))
        q = Q.NVFP4(packed, scales, s_g)
        layout = nv.SCALES_TILED if (r % 128 == 0 and c % 64 == 0) else nv.SCALES_ROWMAJOR
        print(f"[sweep {i}] {r} x {c} layout {layout} s_g {s_g!r}", flush=True)
        t = from_oracle(q, layout)
        for dt, fmt in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
            y = nv.nvfp4_dequantize(t, dt).float().cpu().numpy().astype(np.float64)
            assert np.array_equal(y, Q.dequantize(q, fmt)), (i, fmt)


def test_deterministic_bytes():
    d = synth.attn_proj(m=256, k=1024, n=64)
    xd = bf16_tensor(d["x"])
    a = nv.nvfp4_quantize(xd)
    b = nv.nvfp4_quantize(xd)
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)


@pytest.mark.slow
def test_full_size_attn_proj_activation():
    d = synth.attn_proj()
    x64 = F.bf16_bits_to_f64(d["x"])
    _quantize_and_compare(x64, bf16_tensor(d["x"]), nv.SCALES_TILED)


@pytest.mark.slow
def test_quantize_dequantize_beyond_4gib():
    """98304 x 22528 bf16 (2.2 G values, 4.4 GB; value 2^30 lies in row 47662 and value
    2^31 in row 95325): s_g from the amax pass over all of it, and the codes, scale
    bytes (tiled) and bf16 dequantization (a 4.4 GB output) of four 128-row bands --
    the first, those holding input byte offsets 2^31 and 2^32, the last -- bit-exact."""
    m, n = 98304, 22528
    bits = synth.to_bf16_bits(synth.normal_f32((m, n), 1.0, 41))
    bits[m - 1, n - 1] = 0x4220                       # 40.0, the largest magnitude, last
    amax = float(F.bf16_bits_to_f64(np.array([np.max(bits & 0x7FFF)], dtype=np.uint16))[0])
    assert amax == 40.0
    q = nv.nvfp4_quantize(bf16_tensor(bits), layout=nv.SCALES_TILED)
    y = nv.nvfp4_dequantize(q, torch.bfloat16)
    torch.cuda.synchronize()
    s_g = float(q.global_scale.cpu()[0])
    flat = q.scales.cpu().numpy()
    for r0 in (0, 47616, 95232, m - 128):
        band = Q.quantize(F.bf16_bits_to_f64(bits[r0:r0 + 128]), amax=amax)
        assert s_g == band.s_g
        r, kb = np.meshgrid(np.arange(r0, r0 + 128), np.arange(n // 16), indexing="ij")
        assert np.array_equal(flat[Q.tiled_offset(r, kb, n)], band.scales), f"scales, band {r0}"
        assert np.array_equal(q.codes[r0:r0 + 128].cpu().numpy(), band.packed), f"codes, band {r0}"
        yb = y[r0:r0 + 128].float().cpu().numpy().astype(np.float64)
        assert np.array_equal(yb, Q.dequantize(band, "bf16")), f"dequantized, band {r0}"
