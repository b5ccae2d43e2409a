"""The binding rejects caller-supplied buffers of the wrong shape, dtype, device
or size before any pointer reaches the C ABI (which cannot see buffer sizes).
CPU only: every case here raises before a library call."""

import pytest
import torch

import w4a4_gemm_amd as nv


def _t(rows, cols, layout=nv.SCALES_ROWMAJOR):
    return nv.NVFP4Tensor(rows, cols, layout, device="cpu")


def test_dequantize_out_shape_and_dtype():
    t = _t(128, 64)
    with pytest.raises(ValueError, match="shape"):
        nv.nvfp4_dequantize(t, out=torch.empty((128, 32)))
    with pytest.raises(ValueError, match="shape"):
        nv.nvfp4_dequantize(t, out=torch.empty((64, 128)))
    with pytest.raises(ValueError, match="float16|torch.float32"):
        nv.nvfp4_dequantize(t, out=torch.empty((128, 64), dtype=torch.float16))
    with pytest.raises(ValueError, match="unit stride"):
        nv.nvfp4_dequantize(t, out=torch.empty((64, 128)).t())


def test_nvfp4_tensor_buffers_are_checked():
    t = _t(128, 64)
    t.codes = torch.empty((128, 16), dtype=torch.uint8)          # half the codes
    with pytest.raises(ValueError, match="codes"):
        nv.nvfp4_dequantize(t)
    t = _t(128, 64)
    t.scales = torch.empty(128 * 4 - 1, dtype=torch.uint8)
    with pytest.raises(ValueError, match="scales"):
        nv.nvfp4_dequantize(t)
    t = _t(128, 64)
    t.global_scale = torch.empty(1, dtype=torch.float64)
    with pytest.raises(ValueError, match="global_scale"):
        nv.nvfp4_dequantize(t)


def test_gemm_out_and_amax():
    x, w = _t(128, 64), _t(32, 64)
    with pytest.raises(ValueError, match="shape"):
        nv.nvfp4_gemm_w4a4(x, w, out=torch.empty((128, 16), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="shape"):
        nv.nvfp4_gemm_w4a4(x, w, out=torch.empty((32, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="y_amax"):
        nv.nvfp4_gemm_w4a4(x, w, out=torch.empty((128, 32), dtype=torch.bfloat16),
                           y_amax=torch.empty(1, dtype=torch.float64))


def test_quantize_out_and_workspace():
    x = torch.empty((128, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="codes"):
        bad = _t(128, 64)
        bad.codes = torch.empty(10, dtype=torch.uint8)
        nv.nvfp4_quantize(x, out=bad)
    with pytest.raises(ValueError, match="workspace"):
        nv.nvfp4_quantize(x, out=_t(128, 64), workspace=torch.empty(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="amax"):
        nv.nvfp4_quantize(x, out=_t(128, 64), amax=torch.empty(1, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="codes"):
        bad = _t(128, 64)
        bad.codes = torch.empty(10, dtype=torch.uint8)
        nv.nvfp4_quantize_noalloc(x, out=bad)


def test_kv_outputs_and_page_list():
    c = nv.KVCache(1, 2, 32, 16, 4, 2, torch.arange(4), 4, device="cpu")
    pages = torch.tensor([0, 1], dtype=torch.int32)
    with pytest.raises(ValueError, match="k_out"):
        nv.nvfp4_kv_dequant_blocks(c, 0, pages, k_out=torch.empty((31, 2, 32), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="v_out"):
        nv.nvfp4_kv_dequant_blocks(c, 0, pages, v_out=torch.empty((32, 2, 32), dtype=torch.float32))
    with pytest.raises(ValueError, match="logical_pages"):
        nv.nvfp4_kv_dequant_blocks(c, 0, pages.long())
    q = torch.empty((5, 2, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out"):
        nv.nvfp4_kv_attention(c, 0, pages, 16, q, 1.0, out=torch.empty((4, 2, 32), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="logical_pages"):
        nv.nvfp4_kv_attention(c, 0, pages.long(), 16, q, 1.0)
    with pytest.raises(ValueError, match="pages"):
        nv.nvfp4_kv_window_pages(4096, 256, 0, 0, 0, 1024, pages=torch.empty(2, dtype=torch.int32),
                                 max_pages=8)
