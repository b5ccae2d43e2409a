"""GPU test of nvfp4_quantize_noalloc (the allocation-free quantize): called
through the C ABI, its output must equal nvfp4_quantize's byte for byte, on two
calls in a row that share the library's scratch array, the second with a
smaller input."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from helpers import assert_same_nvfp4, bf16_tensor, dev, f32_tensor, to_oracle
from oracle import formats as F
from oracle import nvfp4 as Q

pytestmark = pytest.mark.gpu

import w4a4_gemm_amd as nv  # noqa: E402  (fails loudly when the library is missing)


def _noalloc_c(x, out, amax=None):
    """One call of the C entry point on the current stream (no workspace)."""
    cs = out.c()
    st = nv._lib.nvfp4_quantize_noalloc(
        ctypes.c_void_p(x.data_ptr()), nv.BF16 if x.dtype == torch.bfloat16 else nv.F32,
        x.shape[0], x.shape[1], x.stride(0),
        ctypes.c_void_p(amax.data_ptr() if amax is not None else 0), ctypes.byref(cs),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == nv.OK, nv.nvfp4_status_string(st)
    return out


def _same(a, b):
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes)
    assert torch.equal(a.scales, b.scales)
    assert torch.equal(a.global_scale, b.global_scale)


def test_two_calls_match_the_workspace_entry_point():
    big = synth.attn_proj(m=1024, k=3072, n=64)["x"]             # bf16 bits
    small = synth.ffn_pair(m=256, d=1024, f=128)["x"]
    xb, xs = bf16_tensor(big), bf16_tensor(small)
    # both no-alloc calls first, back to back on the stream: the second (smaller)
    # overwrites the scratch that the first used
    ob = _noalloc_c(xb, nv.NVFP4Tensor(1024, 3072, nv.SCALES_TILED, device=dev()))
    os_ = _noalloc_c(xs, nv.NVFP4Tensor(256, 1024, nv.SCALES_TILED, device=dev()))
    _same(ob, nv.nvfp4_quantize(xb, layout=nv.SCALES_TILED))
    _same(os_, nv.nvfp4_quantize(xs, layout=nv.SCALES_TILED))
    # and the bytes are the oracle's
    assert_same_nvfp4(to_oracle(os_), Q.quantize(F.bf16_bits_to_f64(small)))


def test_fp32_rowmajor_ragged_and_given_amax():
    rng = np.random.default_rng(11)
    x1 = (rng.standard_normal((300, 592)) * 3).astype(np.float32)
    x2 = (rng.standard_normal((45, 96)) * 0.01).astype(np.float32)
    d1, d2 = f32_tensor(x1), f32_tensor(x2)
    o1 = _noalloc_c(d1, nv.NVFP4Tensor(300, 592, nv.SCALES_ROWMAJOR, device=dev()))
    o2 = _noalloc_c(d2, nv.NVFP4Tensor(45, 96, nv.SCALES_ROWMAJOR, device=dev()))
    _same(o1, nv.nvfp4_quantize(d1, layout=nv.SCALES_ROWMAJOR))
    _same(o2, nv.nvfp4_quantize(d2, layout=nv.SCALES_ROWMAJOR))
    # a producer-supplied amax: no scratch is used
    amax = torch.tensor([float(np.abs(x2).max())], dtype=torch.float32, device=dev())
    o3 = _noalloc_c(d2, nv.NVFP4Tensor(45, 96, nv.SCALES_ROWMAJOR, device=dev()), amax)
    _same(o3, nv.nvfp4_quantize(d2, layout=nv.SCALES_ROWMAJOR, amax=amax))


def test_binding_and_empty_input():
    x = bf16_tensor(synth.attn_proj(m=128, k=256, n=64)["x"])
    _same(nv.nvfp4_quantize_noalloc(x), nv.nvfp4_quantize(x))
    e = torch.empty((0, 64), dtype=torch.float32, device=dev())
    out = nv.nvfp4_quantize_noalloc(e, layout=nv.SCALES_ROWMAJOR)
    torch.cuda.synchronize()
    assert float(out.global_scale.cpu()[0]) == 1.0
