"""GPU parity of nvfp4_gemm_w4a4 against the exact oracle product.

Tolerance (stated for the W4A4 GEMM): fp32 output  |Y - Y_ref| <= 1e-3 * A_ref
with A_ref = sum_k |x^ w^|; bf16 output within one bf16 ulp of RN_bf16(Y_ref),
or |Y - Y_ref| <= ulp_bf16(Y)/2 + 1e-3 A_ref for at most 0.1% of the elements
(the cancellation clause).  The operands fed to the GPU are the oracle's own
NVFP4 bytes, so the GEMM is checked on identical inputs.
"""

import numpy as np
import pytest
import torch

import synth
from helpers import assert_same_nvfp4, bf16_tensor, dev, f32_tensor, from_oracle, to_oracle
from oracle import formats as F
from oracle import nvfp4 as Q

pytestmark = pytest.mark.gpu

import w4a4_gemm_amd as nv  # noqa: E402


def _operands_from_f32(x, w):
    return Q.quantize(x.astype(np.float64)), Q.quantize(w.astype(np.float64))


def _run(xq, wq, dtype, layout_x=nv.SCALES_TILED, layout_w=nv.SCALES_TILED, amax=False):
    xt, wt = from_oracle(xq, layout_x), from_oracle(wq, layout_w)
    am = torch.zeros(1, dtype=torch.float32, device=dev()) if amax else None
    y = nv.nvfp4_gemm_w4a4(xt, wt, dtype, y_amax=am)
    torch.cuda.synchronize()
    out = y.float().cpu().numpy().astype(np.float64)
    return (out, float(am.cpu()[0])) if amax else out


def test_tiny_fp32_out():
    d = synth.tiny()
    xq, wq = _operands_from_f32(d["x"], d["w"])
    y = _run(xq, wq, torch.float32)
    y_ref, a_ref = Q.gemm(xq, wq)
    ok, worst = Q.check_gemm_f32(y, y_ref, a_ref)
    assert ok, f"worst error / bound = {worst}"
    # much tighter than the bound in practice (fp32 accumulation of exact products)
    assert np.max(np.abs(y - y_ref) / np.maximum(a_ref, 1e-30)) < 2e-6


def test_tiny_bf16_out_and_amax():
    d = synth.tiny()
    xq, wq = _operands_from_f32(d["x"], d["w"])
    y, amax = _run(xq, wq, torch.bfloat16, amax=True)
    y_ref, a_ref = Q.gemm(xq, wq)
    ok, n_clause, n_fail = Q.check_gemm_bf16(y, y_ref, a_ref)
    assert ok, (n_clause, n_fail)
    assert amax == np.max(np.abs(y))


@pytest.mark.parametrize("lx,lw", [(nv.SCALES_ROWMAJOR, nv.SCALES_ROWMAJOR),
                                   (nv.SCALES_TILED, nv.SCALES_ROWMAJOR)])
def test_scale_layouts(lx, lw):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((256, 512)).astype(np.float32)
    w = (rng.standard_normal((384, 512)) * 0.02).astype(np.float32)
    xq, wq = _operands_from_f32(x, w)
    y = _run(xq, wq, torch.float32, lx, lw)
    y_ref, a_ref = Q.gemm(xq, wq)
    assert Q.check_gemm_f32(y, y_ref, a_ref)[0]


@pytest.mark.parametrize("m,n,k", [(300, 200, 192), (1, 1, 64), (257, 193, 128), (64, 520, 64)])
def test_ragged_shapes(m, n, k):
    rng = np.random.default_rng(m * 7 + n)
    x = rng.standard_normal((m, k)).astype(np.float32)
    w = rng.standard_normal((n, k)).astype(np.float32)
    xq, wq = _operands_from_f32(x, w)
    y = _run(xq, wq, torch.float32, nv.SCALES_ROWMAJOR, nv.SCALES_ROWMAJOR)
    y_ref, a_ref = Q.gemm(xq, wq)
    assert Q.check_gemm_f32(y, y_ref, a_ref)[0]
    yb = _run(xq, wq, torch.bfloat16, nv.SCALES_ROWMAJOR, nv.SCALES_ROWMAJOR)
    assert Q.check_gemm_bf16(yb, y_ref, a_ref)[0]


def test_seeded_shape_sweep():
    """32 seeded shapes: M, N in [1, 700], K a multiple of 16 up to 1200 (a quarter of the
    cases with 128-row multiples and K % 64 == 0, so that the tiled scale layout is drawn
    too), row scales spread over 2^-12 .. 2^12, bf16 or fp32 output."""
    rng = np.random.default_rng(77)
    for i in range(32):
        m, n, k = int(rng.integers(1, 701)), int(rng.integers(1, 701)), 16 * int(rng.integers(1, 76))
        if i % 4 == 0:
            m, n, k = 128 * int(rng.integers(1, 6)), 128 * int(rng.integers(1, 6)), 64 * int(rng.integers(1, 19))
        x = rng.standard_normal((m, k)) * np.exp2(rng.integers(-12, 13, (m, 1)))
        w = rng.standard_normal((n, k)) * 0.02
        xq, wq = _operands_from_f32(x.astype(np.float32), w.astype(np.float32))
        lx = nv.SCALES_TILED if (m % 128 == 0 and k % 64 == 0 and rng.integers(2)) else nv.SCALES_ROWMAJOR
        lw = nv.SCALES_TILED if (n % 128 == 0 and k % 64 == 0 and rng.integers(2)) else nv.SCALES_ROWMAJOR
        dt = torch.bfloat16 if rng.integers(2) else torch.float32
        print(f"[sweep {i}] M={m} N={n} K={k} layouts {lx}{lw} {dt}", flush=True)
        y = _run(xq, wq, dt, lx, lw)
        y_ref, a_ref = Q.gemm(xq, wq)
        if dt == torch.float32:
            assert Q.check_gemm_f32(y, y_ref, a_ref)[0], i
        else:
            assert Q.check_gemm_bf16(y, y_ref, a_ref)[0], i


@pytest.mark.parametrize("m,n,k", [(96, 80, 16), (130, 70, 48), (257, 193, 80), (64, 300, 208),
                                   (40, 24, 1040)])
def test_ragged_k(m, n, k):
    """K a multiple of 16 but not of 64: the last K step is partial (row-major
    scales, rows on 8-byte code and 1-byte scale boundaries)."""
    rng = np.random.default_rng(m + 5 * k)
    x = rng.standard_normal((m, k)).astype(np.float32)
    w = rng.standard_normal((n, k)).astype(np.float32)
    xq, wq = _operands_from_f32(x, w)
    y_ref, a_ref = Q.gemm(xq, wq)
    y = _run(xq, wq, torch.float32, nv.SCALES_ROWMAJOR, nv.SCALES_ROWMAJOR)
    assert Q.check_gemm_f32(y, y_ref, a_ref)[0]
    yb, am = _run(xq, wq, torch.bfloat16, nv.SCALES_ROWMAJOR, nv.SCALES_ROWMAJOR, amax=True)
    assert Q.check_gemm_bf16(yb, y_ref, a_ref)[0]
    assert am == float(np.max(np.abs(yb)))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_row_stride_mixed_whole_and_edge_tiles(dtype):
    """Y written into a wider buffer (ld_y > N): wave tiles wholly inside Y and
    tiles on its bottom and right edges in one launch, with max|Y| folded over
    both; the padding columns stay untouched."""
    rng = np.random.default_rng(12)
    m, n, k, ld = 384, 448, 256, 480
    x = rng.standard_normal((m, k)).astype(np.float32)
    w = rng.standard_normal((n, k)).astype(np.float32)
    xq, wq = _operands_from_f32(x, w)
    y_ref, a_ref = Q.gemm(xq, wq)
    big = torch.full((m, ld), float("nan"), dtype=dtype, device=dev())
    am = torch.zeros(1, dtype=torch.float32, device=dev())
    nv.nvfp4_gemm_w4a4(from_oracle(xq, nv.SCALES_TILED), from_oracle(wq, nv.SCALES_ROWMAJOR),
                       dtype, out=big[:, :n], y_amax=am)
    torch.cuda.synchronize()
    full = big.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(full[:, n:]))
    y = full[:, :n]
    if dtype == torch.float32:
        assert Q.check_gemm_f32(y, y_ref, a_ref)[0]
    else:
        assert Q.check_gemm_bf16(y, y_ref, a_ref)[0]
    assert float(am.cpu()[0]) == float(np.max(np.abs(y)))


def test_output_beyond_4gib():
    """Y of 70000 x 32768 bf16 (4.6 GB, 65536 bytes per row): whole wave tiles and
    the ragged last tile row at byte offsets past 2^31 and 2^32, max|Y| folded over
    all of them; sampled outputs, with the last row and column, against exact dot
    products."""
    rng = np.random.default_rng(21)
    m, n, k = 70000, 32768, 64
    xq = Q.quantize(rng.standard_normal((m, k)))
    wq = Q.quantize(rng.standard_normal((n, k)) * 0.02)
    am = torch.zeros(1, dtype=torch.float32, device=dev())
    y = nv.nvfp4_gemm_w4a4(from_oracle(xq, nv.SCALES_ROWMAJOR), from_oracle(wq, nv.SCALES_TILED),
                           torch.bfloat16, y_amax=am)
    rows = rng.integers(0, m, 3000)
    cols = rng.integers(0, n, 3000)
    rows[:8] = [m - 1, m - 1, 32767, 32768, 65535, 65536, 69887, 69888]
    cols[:8] = [n - 1, 0, n - 1, 0, 255, 256, n - 1, 0]
    got = y[torch.from_numpy(rows).to(dev()), torch.from_numpy(cols).to(dev())]
    ymax = float(y.abs().amax().float().cpu())
    got = got.float().cpu().numpy().astype(np.float64)
    del y
    y_ref, a_ref = Q.gemm_pairs(xq, wq, rows, cols)
    ok, n_clause, n_fail = Q.check_gemm_bf16(got, y_ref, a_ref)
    assert ok, (n_clause, n_fail)
    assert float(am.cpu()[0]) == ymax


def test_empty_k_gives_zeros():
    """K == 0: the sum over k is empty, so Y = 0 (and max|Y| = 0)."""
    xq = Q.quantize(np.zeros((70, 0)))
    wq = Q.quantize(np.zeros((50, 0)))
    y, am = _run(xq, wq, torch.bfloat16, nv.SCALES_ROWMAJOR, nv.SCALES_ROWMAJOR, amax=True)
    assert y.shape == (70, 50) and not np.any(y) and am == 0.0


def test_random_codes_and_all_scale_bytes():
    # arbitrary code bytes and every scale byte (incl. subnormal scales), odd s_g
    rng = np.random.default_rng(4)
    m, n, k = 256, 256, 2048
    xq = Q.NVFP4(rng.integers(0, 256, (m, k // 2)).astype(np.uint8),
                 rng.integers(0, 127, (m, k // 16)).astype(np.uint8), float(np.float32(3.1e-3)))
    wq = Q.NVFP4(rng.integers(0, 256, (n, k // 2)).astype(np.uint8),
                 rng.integers(0, 127, (n, k // 16)).astype(np.uint8), float(np.float32(0.77)))
    y = _run(xq, wq, torch.float32)
    y_ref, a_ref = Q.gemm(xq, wq)
    assert Q.check_gemm_f32(y, y_ref, a_ref)[0]


def test_integer_case_is_exact():
    # s_g = 1, all scales 1.0: every output is a small integer combination, exact in fp32
    rng = np.random.default_rng(8)
    m, n, k = 256, 384, 512
    xq = Q.NVFP4(rng.integers(0, 256, (m, k // 2)).astype(np.uint8),
                 np.full((m, k // 16), 0x38, np.uint8), 1.0)
    wq = Q.NVFP4(rng.integers(0, 256, (n, k // 2)).astype(np.uint8),
                 np.full((n, k // 16), 0x38, np.uint8), 1.0)
    y = _run(xq, wq, torch.float32)
    y_ref, _ = Q.gemm(xq, wq)
    assert np.array_equal(y, y_ref)


def test_attn_proj_reduced():
    d = synth.attn_proj(m=512, k=3072, n=768)
    xq = Q.quantize(F.bf16_bits_to_f64(d["x"]))
    wq = Q.quantize(F.bf16_bits_to_f64(d["w"]))
    y = _run(xq, wq, torch.bfloat16)
    y_ref, a_ref = Q.gemm(xq, wq)
    ok, n_clause, n_fail = Q.check_gemm_bf16(y, y_ref, a_ref)
    assert ok, (n_clause, n_fail)


def test_attn_proj_end_to_end_on_device():
    # quantize on the GPU, then GEMM on the GPU; the quantized bytes match the
    # oracle's (checked elsewhere), so the product is checked against the oracle
    d = synth.attn_proj(m=512, k=3072, n=512)
    xt = nv.nvfp4_quantize(bf16_tensor(d["x"]))
    wt = nv.nvfp4_quantize(bf16_tensor(d["w"]))
    y = nv.nvfp4_gemm_w4a4(xt, wt, torch.bfloat16).float().cpu().numpy().astype(np.float64)
    xq = Q.quantize(F.bf16_bits_to_f64(d["x"]))
    wq = Q.quantize(F.bf16_bits_to_f64(d["w"]))
    y_ref, a_ref = Q.gemm(xq, wq)
    assert Q.check_gemm_bf16(y, y_ref, a_ref)[0]


@pytest.mark.slow
def test_attn_proj_full_size_sampled():
    """4096 x 3072 x 3072, bf16 out, in the launch configuration the bench times:
    4096 sampled outputs checked against exact dot products."""
    d = synth.attn_proj()
    xq = Q.quantize(F.bf16_bits_to_f64(d["x"]))
    wq = Q.quantize(F.bf16_bits_to_f64(d["w"]))
    y = _run(xq, wq, torch.bfloat16)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, 4096, 4096)
    cols = rng.integers(0, 3072, 4096)
    # corners of every tile edge too
    rows[:8] = [0, 0, 4095, 4095, 255, 256, 2047, 2048]
    cols[:8] = [0, 3071, 0, 3071, 191, 192, 255, 256]
    y_ref, a_ref = Q.gemm_pairs(xq, wq, rows, cols)
    ok, n_clause, n_fail = Q.check_gemm_bf16(y[rows, cols], y_ref, a_ref)
    assert ok, (n_clause, n_fail)


@pytest.mark.slow
@pytest.mark.parametrize("stage", ["gemm1", "gemm2"])
def test_ffn_full_size_sampled(stage):
    """The FFN pair's launches as the benchmark runs them (GEMM1 8192 x 14336 x 3072
    on 256-wide tiles, 1792 workgroups; GEMM2 8192 x 3072 x 14336 on 192-wide tiles,
    512 workgroups), tiled scales, bf16 out with the fused max|Y|: 4096 sampled
    outputs plus tile corners against exact dot products, and max|Y| against the
    whole output."""
    d = synth.ffn_pair()
    if stage == "gemm1":
        aq = Q.quantize(F.bf16_bits_to_f64(d["x"]))
        bq = Q.quantize(F.bf16_bits_to_f64(d["w1"]))
    else:
        # stands in for the requantized Y1: N(0, 1) activations of its shape
        y1 = synth.to_bf16_bits(synth.normal_f32((8192, 14336), 1.0, 24))
        aq = Q.quantize(F.bf16_bits_to_f64(y1))
        bq = Q.quantize(F.bf16_bits_to_f64(d["w2"]))
    y, amax = _run(aq, bq, torch.bfloat16, amax=True)
    print(f"[ffn {stage} full size] device done", flush=True)
    m, n = y.shape
    rng = np.random.default_rng(5)
    rows = rng.integers(0, m, 4096)
    cols = rng.integers(0, n, 4096)
    rows[:8] = [0, 0, m - 1, m - 1, 255, 256, 127, 128]
    cols[:8] = [0, n - 1, 0, n - 1, 255, 256, 191, 192]
    y_ref, a_ref = Q.gemm_pairs(aq, bq, rows, cols)
    ok, n_clause, n_fail = Q.check_gemm_bf16(y[rows, cols], y_ref, a_ref)
    assert ok, (n_clause, n_fail)
    assert amax == float(np.max(np.abs(y)))


@pytest.mark.slow
def test_ffn_stage_parity():
    """FFN pair, reduced M: GEMM1 -> requant with the fused amax -> GEMM2, each stage
    on oracle-made inputs; the chain on the device checked by properties."""
    d = synth.ffn_pair(m=256)
    xq = Q.quantize(F.bf16_bits_to_f64(d["x"]))
    w1q = Q.quantize(F.bf16_bits_to_f64(d["w1"]))
    w2q = Q.quantize(F.bf16_bits_to_f64(d["w2"]))
    # stage 1: GEMM1 with fused amax
    y1, amax = _run(xq, w1q, torch.bfloat16, amax=True)
    y1_ref, a1_ref = Q.gemm(xq, w1q)
    assert Q.check_gemm_bf16(y1, y1_ref, a1_ref)[0]
    assert amax == np.max(np.abs(y1))
    # stage 2: requantize the oracle's bf16 Y1 on the device with the given amax
    y1_bits = F.f64_to_bf16_bits(F.round_f64_to_binary(y1_ref, F.BF16))
    y1o = F.bf16_bits_to_f64(y1_bits)
    am = float(np.max(np.abs(y1o)))
    got = to_oracle(nv.nvfp4_quantize(bf16_tensor(y1_bits),
                                      amax=torch.tensor([am], dtype=torch.float32, device=dev())))
    want = Q.quantize(y1o, amax=am)
    assert got.s_g == want.s_g and np.array_equal(got.scales, want.scales)
    assert np.array_equal(got.packed, want.packed)
    # stage 3: GEMM2 on the oracle's NVFP4 Y1
    y2 = _run(want, w2q, torch.bfloat16)
    y2_ref, a2_ref = Q.gemm(want, w2q)
    assert Q.check_gemm_bf16(y2, y2_ref, a2_ref)[0]


@pytest.mark.slow
def test_ffn_chain_full_size_on_device():
    """The FFN pair exactly as the benchmark runs it, every stage on the device's
    own output: the 8192 x 3072 input quantize (bit-exact against the oracle over
    the whole tensor), GEMM1 with the fused max|Y1|, the requantize of the stored
    bf16 Y1 with that amax (bit-exact on four 128-row bands against the oracle's
    quantize of the same stored rows, which with a given amax is row-local), and
    GEMM2 on the device's NVFP4 Y1 (sampled outputs against exact dot products of
    those bytes)."""
    d = synth.ffn_pair()
    x = bf16_tensor(d["x"])
    xq = nv.NVFP4Tensor(8192, 3072, nv.SCALES_TILED, device=dev())
    ws = torch.empty(nv.nvfp4_workspace_bytes(nv.OP_QUANTIZE, 8192, 3072, 0), dtype=torch.uint8,
                     device=dev())
    nv.nvfp4_quantize(x, out=xq, workspace=ws)
    w1q = nv.nvfp4_quantize(bf16_tensor(d["w1"]))
    w2q = nv.nvfp4_quantize(bf16_tensor(d["w2"]))
    amax = torch.zeros(1, dtype=torch.float32, device=dev())
    y1 = nv.nvfp4_gemm_w4a4(xq, w1q, torch.bfloat16, y_amax=amax)
    y1q = nv.nvfp4_quantize(y1, layout=nv.SCALES_TILED, amax=amax)
    y2 = nv.nvfp4_gemm_w4a4(y1q, w2q, torch.bfloat16)
    torch.cuda.synchronize()
    print("[ffn chain full size] device done", flush=True)

    # stage 0: the input quantize, whole tensor
    assert_same_nvfp4(to_oracle(xq), Q.quantize(F.bf16_bits_to_f64(d["x"])))
    # the fused amax is max|Y1| as stored
    y1_bits = y1.view(torch.int16).cpu().numpy().view(np.uint16)
    am = float(amax.cpu()[0])
    assert am == float(np.max(np.abs(F.bf16_bits_to_f64(y1_bits))))
    # stage 2: requantize, bit-exact on 128-row bands (first, middle, last, random)
    got = to_oracle(y1q)
    assert got.s_g == Q.global_scale(am)
    rng = np.random.default_rng(7)
    for r0 in sorted({0, 4096, 8064, int(rng.integers(1, 63)) * 128}):
        band = Q.quantize(F.bf16_bits_to_f64(y1_bits[r0:r0 + 128]), amax=am)
        assert np.array_equal(got.scales[r0:r0 + 128], band.scales), f"scale bytes, band {r0}"
        assert np.array_equal(got.packed[r0:r0 + 128], band.packed), f"codes, band {r0}"
    # stage 3: GEMM2 on the device's NVFP4 Y1
    w2o = to_oracle(w2q)
    y = y2.float().cpu().numpy().astype(np.float64)
    rows = rng.integers(0, 8192, 2048)
    cols = rng.integers(0, 3072, 2048)
    rows[:4] = [0, 0, 8191, 8191]
    cols[:4] = [0, 3071, 0, 3071]
    y_ref, a_ref = Q.gemm_pairs(got, w2o, rows, cols)
    ok, n_clause, n_fail = Q.check_gemm_bf16(y[rows, cols], y_ref, a_ref)
    assert ok, (n_clause, n_fail)
