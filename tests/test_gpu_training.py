"""GPU parity of the transposed quantize (bit-exact against oracle/training.py) and of
the training-side GEMMs it feeds: dgrad dX = dY W and wgrad dW = dY^T X on
nvfp4_gemm_w4a4, against the oracle's exact products with the forward GEMM's
acceptance rule (fp32 out: |Y - Y_ref| <= 1e-3 A_ref; bf16 out: within one bf16 ulp
of RN_bf16(Y_ref), or the cancellation clause on at most 0.1% of the elements)."""

import numpy as np
import pytest
import torch

import synth
from helpers import assert_same_nvfp4, bf16_tensor, dev, f32_tensor, to_oracle
from oracle import formats as F
from oracle import nvfp4 as Q
from oracle import training as T

pytestmark = pytest.mark.gpu

import w4a4_gemm_amd as nv  # noqa: E402


def _qt(x64, x_dev, layout, amax=None):
    amax_t = None if amax is None else torch.tensor([amax], dtype=torch.float32, device=dev())
    got = to_oracle(nv.nvfp4_quantize_transposed(x_dev, layout=layout, amax=amax_t))
    want = T.quantize_transposed(x64, amax=amax)
    assert_same_nvfp4(got, want)
    return got


@pytest.mark.parametrize("layout", [nv.SCALES_ROWMAJOR, nv.SCALES_TILED])
def test_bf16_several_tiles(layout):
    d = synth.attn_proj(m=384, k=256, n=16)
    _qt(F.bf16_bits_to_f64(d["x"]), bf16_tensor(d["x"]), layout)


def test_ragged_tiles_fp32_and_bf16():
    # 304 rows (output columns, not a multiple of 128), 336 columns (output rows, ragged)
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((304, 336)) * np.exp2(rng.integers(-6, 6, (1, 336)))).astype(np.float32)
    _qt(x.astype(np.float64), f32_tensor(x), nv.SCALES_ROWMAJOR)
    bits = synth.to_bf16_bits(x)
    _qt(F.bf16_bits_to_f64(bits), bf16_tensor(bits), nv.SCALES_ROWMAJOR)


def test_seeded_shape_sweep():
    """16 seeded inputs: rows and cols multiples of 16 up to 800 and 704 (tiled layout
    where cols % 128 == 0 and rows % 64 == 0), column magnitudes over 2^-10 .. 2^10,
    bf16 or fp32, a quarter with the amax given; bytes bit-exact."""
    rng = np.random.default_rng(81)
    for i in range(16):
        rows, cols = 16 * int(rng.integers(1, 51)), 16 * int(rng.integers(1, 45))
        if i % 4 == 0:
            rows, cols = 64 * int(rng.integers(1, 13)), 128 * int(rng.integers(1, 6))
        x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-10, 11, (1, cols)))).astype(np.float32)
        layout = nv.SCALES_TILED if (cols % 128 == 0 and rows % 64 == 0) else nv.SCALES_ROWMAJOR
        amax = float(np.float32(np.max(np.abs(x)) * 1.25)) if i % 4 == 1 else None
        print(f"[sweep {i}] {rows} x {cols} layout {layout} amax {amax}", flush=True)
        if rng.integers(2):
            bits = synth.to_bf16_bits(x)
            _qt(F.bf16_bits_to_f64(bits), bf16_tensor(bits), layout, amax=amax)
        else:
            _qt(x.astype(np.float64), f32_tensor(x), layout, amax=amax)


def test_strided_input_and_given_amax():
    x = synth.entry_outliers_f32(256, 128, seed=22, idx_seed=23)
    buf = torch.zeros((256, 160), dtype=torch.float32, device=dev())
    buf[:, :128] = f32_tensor(x)
    x64 = x.astype(np.float64)
    got = to_oracle(nv.nvfp4_quantize_transposed(buf[:, :128], layout=nv.SCALES_TILED))
    assert_same_nvfp4(got, T.quantize_transposed(x64))
    _qt(x64, f32_tensor(x), nv.SCALES_TILED, amax=float(np.max(np.abs(x64))) * 2.0)


def test_empty():
    t = nv.nvfp4_quantize_transposed(torch.empty((0, 64), dtype=torch.bfloat16, device=dev()),
                                     layout=nv.SCALES_ROWMAJOR)
    torch.cuda.synchronize()
    assert t.rows == 64 and t.cols == 0 and float(t.global_scale.cpu()[0]) == 1.0


def _check(y_dev, yref, aref, bf16):
    y = y_dev.float().cpu().numpy().astype(np.float64)
    res = Q.check_gemm_bf16(y, yref, aref) if bf16 else Q.check_gemm_f32(y, yref, aref)
    assert res[0], res


@pytest.mark.parametrize("bf16_out", [False, True])
def test_wgrad_and_dgrad_small(bf16_out):
    m, n, k = 512, 384, 256          # tokens, out features, in features
    x = synth.channel_outliers_bf16(m, k, seed=24, ch_seed=25)
    w = synth.weights_bf16(n, k, seed=26)
    dy = synth.weights_bf16(m, n, seed=27, std=1e-3)            # upstream gradient
    x64, w64, dy64 = (F.bf16_bits_to_f64(a) for a in (x, w, dy))
    xd, wd, dyd = bf16_tensor(x), bf16_tensor(w), bf16_tensor(dy)
    dtype = torch.bfloat16 if bf16_out else torch.float32
    # wgrad: dW [n x k] = dY^T X, contraction over the tokens
    a, b = nv.nvfp4_quantize_transposed(dyd), nv.nvfp4_quantize_transposed(xd)
    dw = nv.nvfp4_gemm_w4a4(a, b, dtype=dtype)
    ya, yb = T.quantize_transposed(dy64), T.quantize_transposed(x64)
    assert_same_nvfp4(to_oracle(a), ya)
    assert_same_nvfp4(to_oracle(b), yb)
    _check(dw, *T.wgrad(ya, yb), bf16_out)
    # dgrad: dX [m x k] = dY W, contraction over the out features
    a, b = nv.nvfp4_quantize(dyd), nv.nvfp4_quantize_transposed(wd)
    dx = nv.nvfp4_gemm_w4a4(a, b, dtype=dtype)
    ya, yb = Q.quantize(dy64), T.quantize_transposed(w64)
    assert_same_nvfp4(to_oracle(b), yb)
    _check(dx, *T.dgrad(ya, yb), bf16_out)


@pytest.mark.parametrize("bf16_out", [False, True])
def test_wgrad_over_ragged_token_count(bf16_out):
    """880 tokens (one latent frame): wgrad contracts over K = 880, a multiple of 16
    but not of 64, so the transposed operands take row-major scales and the GEMM
    ends with a partial K step."""
    m, n, k = 880, 192, 320
    x = synth.channel_outliers_bf16(m, k, seed=31, ch_seed=32)
    dy = synth.weights_bf16(m, n, seed=33, std=1e-3)
    x64, dy64 = F.bf16_bits_to_f64(x), F.bf16_bits_to_f64(dy)
    a = nv.nvfp4_quantize_transposed(bf16_tensor(dy), layout=nv.SCALES_ROWMAJOR)
    b = nv.nvfp4_quantize_transposed(bf16_tensor(x))    # default layout: row-major here
    assert b.layout == nv.SCALES_ROWMAJOR
    dw = nv.nvfp4_gemm_w4a4(a, b, dtype=torch.bfloat16 if bf16_out else torch.float32)
    ya, yb = T.quantize_transposed(dy64), T.quantize_transposed(x64)
    assert_same_nvfp4(to_oracle(a), ya)
    assert_same_nvfp4(to_oracle(b), yb)
    _check(dw, *T.wgrad(ya, yb), bf16_out)


def test_attn_proj_wgrad_full_size_sampled():
    """wgrad of the attention projection: dW [3072 x 3072] = dY^T X over 4096 tokens;
    both transposed operands bit-exact in full, the product on sampled rows."""
    d = synth.attn_proj(m=4096, k=3072, n=16)
    x = d["x"]
    dy = synth.weights_bf16(4096, 3072, seed=28, std=1e-3)
    a = nv.nvfp4_quantize_transposed(bf16_tensor(dy))
    b = nv.nvfp4_quantize_transposed(bf16_tensor(x))
    dw = nv.nvfp4_gemm_w4a4(a, b, dtype=torch.float32)
    ya = T.quantize_transposed(F.bf16_bits_to_f64(dy))
    yb = T.quantize_transposed(F.bf16_bits_to_f64(x))
    assert_same_nvfp4(to_oracle(a), ya)
    assert_same_nvfp4(to_oracle(b), yb)
    rows = np.sort(np.random.default_rng(29).choice(3072, 24, replace=False))
    yref, aref = Q.gemm(ya, yb, rows=rows)
    _check(dw[torch.from_numpy(rows).to(dev())], yref, aref, False)


@pytest.mark.slow
def test_ffn_wgrad_full_size_sampled():
    """The measured launch: wgrad of FFN GEMM1, dW1 [14336 x 3072] = dY1^T X over 8192
    tokens, with the operands the benchmark uses (X the FFN input, dY1 ~ N(0, 1e-3)
    from the device generator seeded 90).  Transposed operands: s_g and sampled
    output rows bit-exact (the oracle takes the tensor amax of the whole input);
    dW1 on sampled rows within the GEMM tolerance."""
    f = synth.ffn_pair()
    x = f["x"]
    gen = torch.Generator(device=dev()).manual_seed(90)
    dy_t = (torch.randn((8192, 14336), generator=gen, device=dev()) * 1e-3).to(torch.bfloat16)
    a = nv.nvfp4_quantize_transposed(dy_t)
    b = nv.nvfp4_quantize_transposed(bf16_tensor(x))
    dw = nv.nvfp4_gemm_w4a4(a, b, dtype=torch.float32)
    torch.cuda.synchronize()
    print("[wgrad full size] device done", flush=True)
    dy64 = dy_t.float().cpu().numpy().astype(np.float64)
    got_a = to_oracle(a)
    rows = np.unique(np.concatenate([[0, 14335], np.random.default_rng(30).choice(14336, 22,
                                                                                  replace=False)]))
    amax = float(np.max(np.abs(dy64)))
    want_a = T.quantize_transposed(dy64[:, rows], amax=amax)
    assert got_a.s_g == want_a.s_g
    assert np.array_equal(got_a.packed[rows], want_a.packed)
    assert np.array_equal(got_a.scales[rows], want_a.scales)
    yb = T.quantize_transposed(F.bf16_bits_to_f64(x))
    assert_same_nvfp4(to_oracle(b), yb)
    print("[wgrad full size] operands checked", flush=True)
    ya = Q.NVFP4(want_a.packed, want_a.scales, want_a.s_g)
    yref, aref = Q.gemm(ya, yb)
    _check(dw[torch.from_numpy(rows).to(dev())], yref, aref, False)
