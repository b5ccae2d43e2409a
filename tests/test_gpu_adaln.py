"""GPU parity of nvfp4_adaln_quantize (LayerNorm + adaLN modulate + NVFP4) against
oracle/adaln.py.

Row statistics are real-valued (fp64 inside the kernel, rounded once to fp32):
they are compared with the oracle's within one fp32 rounding plus the fp64
summation error, |d mu| <= 2^-24 |mu| + 2^-50 sum|x| / cols and
|d rstd| <= 2^-23 rstd.  Given the kernel's fp32 statistics, x' and its NVFP4
encoding are unique, so codes, scale bytes and s_g must equal the oracle's
bit for bit (the oracle is fed the kernel's statistics: both sides take every
rounding decision in the same precision).
"""

import numpy as np
import pytest
import torch

import synth
from helpers import assert_same_nvfp4, bf16_tensor, dev, f32_tensor, to_oracle
from oracle import adaln as A
from oracle import formats as F
from oracle import nvfp4 as Q

pytestmark = pytest.mark.gpu

import w4a4_gemm_amd as nv  # noqa: E402


def _check_stats(x64, stats, eps):
    mu, rstd = stats[:, 0].astype(np.float64), stats[:, 1].astype(np.float64)
    mu_ref, rstd_ref = A.row_stats(x64, eps)
    tol_mu = 2.0 ** -24 * np.abs(mu_ref) + 2.0 ** -50 * np.mean(np.abs(x64), axis=1)
    assert np.all(np.abs(mu - mu_ref) <= tol_mu), "row means differ"
    assert np.all(np.abs(rstd - rstd_ref) <= 2.0 ** -23 * rstd_ref), "row rstd differ"
    return mu, rstd, float(np.mean((mu == mu_ref) & (rstd == rstd_ref)))


def _run(x_np, x_dev, shift, scale, rpg, eps, layout, ld=None):
    rows, cols = x_np.shape
    xin = x_dev
    if ld is not None:           # strided input: a view into a wider buffer
        buf = torch.zeros((rows, ld), dtype=x_dev.dtype, device=dev())
        buf[:, :cols] = x_dev
        xin = buf[:, :cols]
    t, stats = nv.nvfp4_adaln_quantize(xin, f32_tensor(shift), f32_tensor(scale), rpg, eps,
                                       layout=layout)
    torch.cuda.synchronize()
    x64 = F.bf16_bits_to_f64(x_np) if x_np.dtype == np.uint16 else x_np.astype(np.float64)
    mu, rstd, same = _check_stats(x64, stats.cpu().numpy(), eps)
    want, _, _ = A.adaln_quantize(x64, shift.astype(np.float64), scale.astype(np.float64), rpg,
                                  eps, stats=(mu, rstd))
    assert_same_nvfp4(to_oracle(t), want)
    return same


@pytest.mark.parametrize("layout", [nv.SCALES_ROWMAJOR, nv.SCALES_TILED])
def test_bf16_several_tiles_two_groups(layout):
    rows = 384 if layout == nv.SCALES_TILED else 300      # ragged rows for row-major scales
    d = synth.adaln_input(m=rows, k=320, seed=72)         # 320 columns: 2.5 column tiles
    rpg = 100
    shift, scale = synth.adaln_modulation(-(-rows // rpg), 320, seed=73)
    same = _run(d["x"], bf16_tensor(d["x"]), shift, scale, rpg, 1e-6, layout)
    assert same > 0.99


def test_seeded_shape_sweep():
    """16 seeded inputs: rows in [1, 500], cols a multiple of 16 up to 2400 (tiled layout
    where rows % 128 == 0 and cols % 64 == 0), rows per modulation group from 1 to all,
    row offsets and magnitudes varied, bf16 or fp32; bytes bit-exact on the kernel's
    statistics."""
    rng = np.random.default_rng(80)
    for i in range(16):
        rows, cols = int(rng.integers(1, 501)), 16 * int(rng.integers(1, 151))
        if i % 4 == 0:
            rows, cols = 128 * int(rng.integers(1, 4)), 64 * int(rng.integers(1, 38))
        rpg = int(rng.integers(1, rows + 1))
        x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-8, 9, (rows, 1)))
             + rng.standard_normal((rows, 1)) * 4).astype(np.float32)
        shift, scale = synth.adaln_modulation(-(-rows // rpg), cols, seed=600 + i)
        layout = nv.SCALES_TILED if (rows % 128 == 0 and cols % 64 == 0) else nv.SCALES_ROWMAJOR
        print(f"[sweep {i}] {rows} x {cols} rows/group {rpg} layout {layout}", flush=True)
        if rng.integers(2):
            bits = synth.to_bf16_bits(x)
            _run(bits, bf16_tensor(bits), shift, scale, rpg, 1e-6, layout)
        else:
            _run(x, f32_tensor(x), shift, scale, rpg, 1e-6, layout)


def test_fp32_small_groups_tiled():
    # rows_per_group 5 < 29: a lane's eight rows can meet more than two groups
    x = synth.normal_f32((256, 192), 2.0, seed=74) + np.float32(0.5)
    shift, scale = synth.adaln_modulation(-(-256 // 5), 192, seed=75)
    _run(x, f32_tensor(x), shift, scale, 5, 1e-5, nv.SCALES_TILED)


def test_strided_rows_and_one_group():
    d = synth.adaln_input(m=200, k=256, seed=76)
    shift, scale = synth.adaln_modulation(1, 256, seed=77)
    _run(d["x"], bf16_tensor(d["x"]), shift, scale, 200, 1e-6, nv.SCALES_ROWMAJOR, ld=264)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_long_rows_are_swept_from_memory(dtype):
    # rows longer than the register-resident case (64 lanes x 8 chunks of 16 bytes)
    cols = 4160 if dtype == "bf16" else 2064
    d = synth.adaln_input(m=40, k=cols, seed=78, dtype=dtype)
    shift, scale = synth.adaln_modulation(1, cols, seed=79)
    x = d["x"]
    xd = bf16_tensor(x) if dtype == "bf16" else f32_tensor(x)
    _run(x, xd, shift, scale, 880, 1e-6, nv.SCALES_ROWMAJOR)


def test_constant_rows_and_large_eps():
    rows, cols = 130, 64
    x = np.repeat(np.linspace(-3, 3, rows, dtype=np.float32)[:, None], cols, axis=1)
    x[::3] = synth.normal_f32((len(x[::3]), cols), 1.0, seed=80)
    shift, scale = synth.adaln_modulation(-(-rows // 40), cols, seed=81)
    _run(x, f32_tensor(x), shift, scale, 40, 0.75, nv.SCALES_ROWMAJOR)


def test_empty_and_single_row():
    shift, scale = synth.adaln_modulation(1, 64, seed=82)
    t, _ = nv.nvfp4_adaln_quantize(torch.empty((0, 64), dtype=torch.bfloat16, device=dev()),
                                   f32_tensor(shift), f32_tensor(scale), 1,
                                   layout=nv.SCALES_ROWMAJOR)
    torch.cuda.synchronize()
    assert float(t.global_scale.cpu()[0]) == 1.0
    x = synth.normal_f32((1, 64), 1.0, seed=83)
    _run(x, f32_tensor(x), shift, scale, 1, 1e-6, nv.SCALES_ROWMAJOR)


@pytest.mark.parametrize("m", [4096, 8192])
def test_block_input_full_size_sampled_rows(m):
    """DiT block inputs, m x 3072 bf16 (attention projection 4096 rows; FFN 8192
    rows, the measured launch), 880-row modulation groups, tiled scales: every
    row's statistics, s_g, and the encoding of sampled rows (the oracle's x' over
    the whole tensor gives the amax)."""
    d = synth.adaln_input(m=m, k=3072, seed=72)
    x, shift, scale, rpg = d["x"], d["shift"], d["scale"], d["rows_per_group"]
    t, stats = nv.nvfp4_adaln_quantize(bf16_tensor(x), f32_tensor(shift), f32_tensor(scale), rpg,
                                       1e-6, layout=nv.SCALES_TILED)
    got = to_oracle(t)
    print(f"[adaln full size] {m} rows quantized", flush=True)
    x64 = F.bf16_bits_to_f64(x)
    mu, rstd, same = _check_stats(x64, stats.cpu().numpy(), 1e-6)
    assert same > 0.999
    sh, sc = shift.astype(np.float64), scale.astype(np.float64)
    xp = A.modulate(x64, mu, rstd, sh, sc, rpg)
    amax = float(np.max(np.abs(xp)))
    # rows whose fp32 statistics differ from the oracle's (within the tolerance)
    mu_ref, rstd_ref = A.row_stats(x64, 1e-6)
    diff = np.nonzero((mu != mu_ref) | (rstd != rstd_ref))[0]
    print(f"[adaln full size] {m} rows: {len(diff)} with statistics other than the oracle's",
          flush=True)
    rows = np.sort(np.random.default_rng(84).choice(m, 96, replace=False))
    rows = np.unique(np.concatenate([rows, [0, 879, 880, m - 1], diff]))  # group edges too
    want = Q.quantize(xp[rows], amax=amax)
    assert got.s_g == want.s_g
    assert np.array_equal(got.scales[rows], want.scales)
    assert np.array_equal(got.packed[rows], want.packed)
    if len(diff):
        # those rows against the oracle on its own statistics: x' moves by at most a
        # few fp32 ulps, so a code may move only to a neighbouring E2M1 value where
        # the two x' straddle a rounding boundary (same scale byte), and the scale
        # byte only where the block maximum straddles an E4M3 boundary
        xo = A.modulate(x64, mu_ref, rstd_ref, sh, sc, rpg)
        own = Q.quantize(xo[diff], amax=float(np.max(np.abs(xo))))
        if own.s_g != got.s_g:          # the tensor's largest |x'| sits in such a row
            return
        same_scale = np.repeat(got.scales[diff] == own.scales, 16, axis=1)
        dg = Q.dequantize(Q.NVFP4(got.packed[diff], got.scales[diff], got.s_g), "f32")
        do = Q.dequantize(own, "f32")
        # one E2M1 step (at most 2) times s_b s_g, where the scale bytes agree
        step = 2.0 * np.repeat(F.E4M3_GRID[got.scales[diff]], 16, axis=1) * got.s_g
        assert np.all(np.abs(dg - do)[same_scale] <= step[same_scale])
        assert np.mean(got.packed[diff] == own.packed) > 0.99
