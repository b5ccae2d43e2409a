"""The C-ABI library loads, exports every symbol the header declares, and rejects
bad arguments before launching anything (CPU only: no compute calls)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "nvfp4.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_hot_path_calls():
    names = _declared_functions()
    for n in ("nvfp4_quantize", "nvfp4_dequantize", "nvfp4_gemm_w4a4", "nvfp4_kv_quantize",
              "nvfp4_kv_dequant_blocks"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import w4a4_gemm_amd as nv
    lib = ctypes.CDLL(nv.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(nv.EXPORTS) <= set(_declared_functions())


def test_library_was_built_from_these_sources():
    import importlib.util
    import w4a4_gemm_amd as nv
    spec = importlib.util.spec_from_file_location(
        "srchash", os.path.join(ROOT, "w4a4_gemm_amd", "srchash.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert nv._lib.nvfp4_source_hash().decode() == mod.source_hash()


def test_version_and_status_strings():
    import w4a4_gemm_amd as nv
    assert nv.nvfp4_abi_version() == 1
    assert nv.nvfp4_status_string(0) == "ok"
    assert "shape" in nv.nvfp4_status_string(-2)
    assert nv.nvfp4_status_string(123) == "unknown status"


def test_workspace_and_page_sizes():
    import w4a4_gemm_amd as nv
    assert nv.nvfp4_kv_page_bytes(24, 128, 256) == 884736
    assert nv.nvfp4_kv_page_bytes(24, 120, 256) == 0
    assert nv.nvfp4_workspace_bytes(nv.OP_QUANTIZE, 4096, 3072, 1) == 0
    assert nv.nvfp4_workspace_bytes(nv.OP_QUANTIZE, 4096, 3072, 0) > 0
    assert nv.nvfp4_workspace_bytes(nv.OP_KV_QUANTIZE, 7040, 24, 128) > 0
    assert nv.nvfp4_workspace_bytes(99, 1, 1, 1) == 0


def test_argument_errors_return_before_launch():
    import w4a4_gemm_amd as nv
    lib = nv._lib
    T = nv._Tensor
    good = T(16, 16, 64, 128, 64, nv.SCALES_ROWMAJOR)
    # bad dtype / null input
    assert lib.nvfp4_quantize(16, 7, 128, 64, 64, None, ctypes.byref(good), None, 0, None) == nv.EINVAL
    assert lib.nvfp4_quantize(None, nv.BF16, 128, 64, 64, None, ctypes.byref(good), 256, 4096,
                              None) == nv.EINVAL
    # cols % 16
    bad = T(16, 16, 64, 128, 40, nv.SCALES_ROWMAJOR)
    assert lib.nvfp4_quantize(16, nv.BF16, 128, 40, 40, None, ctypes.byref(bad), None, 0,
                              None) == nv.ESHAPE
    # tiled layout needs rows % 128
    tiled = T(16, 16, 64, 100, 64, nv.SCALES_TILED)
    assert lib.nvfp4_quantize(16, nv.BF16, 100, 64, 64, None, ctypes.byref(tiled), None, 0,
                              None) == nv.ESHAPE
    # missing workspace
    assert lib.nvfp4_quantize(16, nv.BF16, 128, 64, 64, None, ctypes.byref(good), None, 0,
                              None) == nv.EWORKSPACE
    # a row stride beyond any tensor (it would overflow once scaled by the element size)
    assert lib.nvfp4_quantize(16, nv.BF16, 128, 64, 1 << 62, None, ctypes.byref(good), 256, 4096,
                              None) == nv.ESHAPE
    # ld_x < cols
    assert lib.nvfp4_quantize(16, nv.BF16, 128, 64, 32, None, ctypes.byref(good), 256, 4096,
                              None) == nv.ESHAPE
    # GEMM K mismatch, ld_y < N, K % 16 (any multiple of 16 is accepted: ragged K)
    w = T(16, 16, 64, 64, 128, nv.SCALES_ROWMAJOR)
    assert lib.nvfp4_gemm_w4a4(ctypes.byref(good), ctypes.byref(w), 16, nv.BF16, 64, None,
                               None) == nv.ESHAPE
    k48 = T(16, 16, 64, 64, 48, nv.SCALES_ROWMAJOR)
    assert lib.nvfp4_gemm_w4a4(ctypes.byref(k48), ctypes.byref(k48), 16, nv.BF16, 32, None,
                               None) == nv.ESHAPE
    k40 = T(16, 16, 64, 64, 40, nv.SCALES_ROWMAJOR)
    assert lib.nvfp4_gemm_w4a4(ctypes.byref(k40), ctypes.byref(k40), 16, nv.BF16, 64, None,
                               None) == nv.ESHAPE
    assert lib.nvfp4_gemm_w4a4(ctypes.byref(good), ctypes.byref(good), 16, 5, 128, None,
                               None) == nv.EINVAL
    # empty GEMM is a no-op
    e = T(16, 16, 64, 0, 64, nv.SCALES_ROWMAJOR)
    assert lib.nvfp4_gemm_w4a4(ctypes.byref(e), ctypes.byref(good), None, nv.BF16, 128, None,
                               None) == nv.OK
    # dequantize: bad out dtype
    assert lib.nvfp4_dequantize(ctypes.byref(good), 16, 9, 64, None) == nv.EINVAL
    # more rows than one grid dimension can cover (2^28 is the limit)
    huge = T(16, 16, 64, (1 << 28) + 32, 16, nv.SCALES_ROWMAJOR)
    assert lib.nvfp4_dequantize(ctypes.byref(huge), 16, nv.F32, 16, None) == nv.ESHAPE


def test_kv_argument_errors():
    import w4a4_gemm_amd as nv
    lib = nv._lib
    C = nv._KVCache
    good = C(256, 28, 1, 24, 128, 256, 28, 2, 16, 16, 16, 16, 16)
    # null k
    assert lib.nvfp4_kv_quantize(ctypes.byref(good), 0, 0, None, 16, 7040, 0, 256, 1 << 20,
                                 None) == nv.EINVAL
    # layer out of range, chunk out of range, too many tokens for max_pages
    assert lib.nvfp4_kv_quantize(ctypes.byref(good), 1, 0, 16, 16, 7040, 0, 256, 1 << 20,
                                 None) == nv.ESHAPE
    assert lib.nvfp4_kv_quantize(ctypes.byref(good), 0, 2, 16, 16, 7040, 0, 256, 1 << 20,
                                 None) == nv.ESHAPE
    assert lib.nvfp4_kv_quantize(ctypes.byref(good), 0, 0, 16, 16, 7200, 0, 256, 1 << 20,
                                 None) == nv.ESHAPE
    # a start token so large that start + T would overflow int64
    assert lib.nvfp4_kv_quantize(ctypes.byref(good), 0, 0, 16, 16, 7040, (1 << 63) - 100, 256,
                                 1 << 20, None) == nv.ESHAPE
    # a chunk after the first shorter than a page
    assert lib.nvfp4_kv_quantize(ctypes.byref(good), 0, 1, 16, 16, 100, 256, 256, 1 << 20,
                                 None) == nv.ESHAPE
    # the first chunk of a layer starting inside a page (its earlier slots would
    # belong to no chunk)
    assert lib.nvfp4_kv_quantize(ctypes.byref(good), 0, 0, 16, 16, 300, 100, 256, 1 << 20,
                                 None) == nv.ESHAPE
    # workspace too small
    assert lib.nvfp4_kv_quantize(ctypes.byref(good), 0, 0, 16, 16, 7040, 0, 256, 16,
                                 None) == nv.EWORKSPACE
    # head_dim not a multiple of 16
    bad = C(256, 28, 1, 24, 120, 256, 28, 2, 16, 16, 16, 16, 16)
    assert lib.nvfp4_kv_dequant_blocks(ctypes.byref(bad), 0, 16, 4, 16, 16, None) == nv.ESHAPE
    # zero pages is a no-op; negative is an error
    assert lib.nvfp4_kv_dequant_blocks(ctypes.byref(good), 0, None, 0, None, None, None) == nv.OK
    assert lib.nvfp4_kv_dequant_blocks(ctypes.byref(good), 0, 16, -1, 16, 16, None) == nv.EINVAL


def test_kv_attention_argument_errors():
    import w4a4_gemm_amd as nv
    lib = nv._lib                                  # argtypes set: int64 n_q, float scale
    C = nv._KVCache
    good = C(256, 28, 1, 24, 128, 256, 28, 2, 16, 16, 16, 16, 16)
    # nothing to do: no query rows
    assert lib.nvfp4_kv_attention(ctypes.byref(good), 0, 16, 4, 256, 16, 0, 0.1, 16, None, 0, None) == nv.OK
    # head_dim other than 64 or 128, page_tokens not a multiple of 64
    d80 = C(256, 28, 1, 24, 80, 256, 28, 2, 16, 16, 16, 16, 16)
    assert lib.nvfp4_kv_attention(ctypes.byref(d80), 0, 16, 4, 256, 16, 8, 0.1, 16, None, 0, None) == nv.ESHAPE
    p100 = C(256, 28, 1, 24, 128, 100, 28, 2, 16, 16, 16, 16, 16)
    assert lib.nvfp4_kv_attention(ctypes.byref(p100), 0, 16, 4, 100, 16, 8, 0.1, 16, None, 0, None) == nv.ESHAPE
    # last page token count out of range, negative sizes, null query / output
    assert lib.nvfp4_kv_attention(ctypes.byref(good), 0, 16, 4, 257, 16, 8, 0.1, 16, None, 0, None) == nv.EINVAL
    assert lib.nvfp4_kv_attention(ctypes.byref(good), 0, 16, -1, 0, 16, 8, 0.1, 16, None, 0, None) == nv.EINVAL
    assert lib.nvfp4_kv_attention(ctypes.byref(good), 0, 16, 4, 256, 16, -8, 0.1, 16, None, 0, None) == nv.EINVAL
    assert lib.nvfp4_kv_attention(ctypes.byref(good), 0, 16, 4, 256, None, 8, 0.1, 16, None, 0, None) == nv.EINVAL
    assert lib.nvfp4_kv_attention(ctypes.byref(good), 0, 16, 4, 256, 16, 8, 0.1, None, None, 0, None) == nv.EINVAL
    # misaligned query rows, layer out of range
    assert lib.nvfp4_kv_attention(ctypes.byref(good), 0, 16, 4, 256, 18, 8, 0.1, 16, None, 0, None) == nv.ESHAPE
    assert lib.nvfp4_kv_attention(ctypes.byref(good), 1, 16, 4, 256, 16, 8, 0.1, 16, None, 0, None) == nv.ESHAPE
    # a small grid splits the window over workgroups: the workspace is then required
    need = nv.nvfp4_workspace_bytes(nv.OP_KV_ATTENTION, 100, 24, 68 * 256)
    assert need > 0
    assert nv.nvfp4_workspace_bytes(nv.OP_KV_ATTENTION, 7040, 24, 68 * 256) == 0
    assert lib.nvfp4_kv_attention(ctypes.byref(good), 0, 16, 68, 256, 16, 100, 0.1, 16, None, 0,
                                  None) == nv.EWORKSPACE


def test_window_pages_host_side():
    import w4a4_gemm_amd as nv
    lib = nv._lib
    n, last = ctypes.c_int32(-1), ctypes.c_int32(-1)
    # empty cache: no list, nothing launched
    assert lib.nvfp4_kv_window_pages(0, 256, 1024, 0, 0, 16384, None, 0, ctypes.byref(n),
                                     ctypes.byref(last), None) == nv.OK
    assert (n.value, last.value) == (0, 0)
    # the list would not fit: rejected before any launch
    assert lib.nvfp4_kv_window_pages(65536, 256, 1024, 0, 0, 16384, 16, 67, ctypes.byref(n),
                                     ctypes.byref(last), None) == nv.ESHAPE
    # shot ranges whose end would overflow int64 are clipped to the cache first:
    # a shot starting past the end contributes nothing ...
    assert lib.nvfp4_kv_window_pages(100, 64, 0, (1 << 63) - 10, 100, 0, None, 0,
                                     ctypes.byref(n), ctypes.byref(last), None) == nv.OK
    assert (n.value, last.value) == (0, 0)
    # ... and an endless shot from token 50 covers pages 0 and 1 (too many for one entry)
    assert lib.nvfp4_kv_window_pages(100, 64, 0, 50, (1 << 63) - 1, 0, 16, 1, ctypes.byref(n),
                                     ctypes.byref(last), None) == nv.ESHAPE
    # bad sizes and missing outputs
    assert lib.nvfp4_kv_window_pages(100, 0, 0, 0, 0, 0, 16, 8, ctypes.byref(n),
                                     ctypes.byref(last), None) == nv.EINVAL
    assert lib.nvfp4_kv_window_pages(100, 64, -1, 0, 0, 0, 16, 8, ctypes.byref(n),
                                     ctypes.byref(last), None) == nv.EINVAL
    assert lib.nvfp4_kv_window_pages(100, 64, 0, 0, 0, 10, 16, 8, None, ctypes.byref(last),
                                     None) == nv.EINVAL
    # a non-empty list needs the device array
    assert lib.nvfp4_kv_window_pages(100, 64, 0, 0, 0, 10, None, 8, ctypes.byref(n),
                                     ctypes.byref(last), None) == nv.EINVAL


def test_adaln_quantize_argument_errors():
    import w4a4_gemm_amd as nv
    lib = nv._lib
    T = nv._Tensor
    good = T(16, 16, 64, 128, 64, nv.SCALES_ROWMAJOR)
    ws = nv.nvfp4_workspace_bytes(nv.OP_ADALN_QUANTIZE, 128, 64, 0)
    assert ws > 0

    def call(x=256, dtype=nv.BF16, rows=128, cols=64, ld=64, sh=512, sc=512, rpg=880, eps=1e-6,
             stats=512, out=good, w=256, wb=ws):
        return lib.nvfp4_adaln_quantize(x, dtype, rows, cols, ld, sh, sc, rpg, eps, stats,
                                        ctypes.byref(out), w, wb, None)

    assert call(dtype=9) == nv.EINVAL
    assert call(rpg=0) == nv.EINVAL
    assert call(eps=0.0) == nv.EINVAL
    assert call(eps=-1.0) == nv.EINVAL
    assert call(eps=float("inf")) == nv.EINVAL
    assert call(eps=float("nan")) == nv.EINVAL
    assert call(x=None) == nv.EINVAL
    assert call(sh=None) == nv.EINVAL
    assert call(sc=None) == nv.EINVAL
    assert call(stats=None) == nv.EINVAL
    assert call(rows=-1) == nv.EINVAL
    assert call(cols=48, ld=48) == nv.ESHAPE                  # out->cols differs
    assert call(ld=60) == nv.ESHAPE                           # ld * 2 % 16
    assert call(sh=520) == nv.ESHAPE                          # shift not 16-byte aligned
    assert call(stats=516) == nv.ESHAPE                       # stats not 8-byte aligned
    assert call(w=None) == nv.EWORKSPACE
    assert call(wb=ws - 4) == nv.EWORKSPACE
    assert call(w=272) == nv.EWORKSPACE                       # not 256-byte aligned
    tiled_bad = T(16, 16, 64, 100, 64, nv.SCALES_TILED)
    assert call(rows=100, out=tiled_bad) == nv.ESHAPE


def test_quantize_transposed_argument_errors():
    import w4a4_gemm_amd as nv
    lib = nv._lib
    T = nv._Tensor
    out = T(16, 16, 64, 64, 128, nv.SCALES_ROWMAJOR)        # X^T of a 128 x 64 input
    ws = nv.nvfp4_workspace_bytes(nv.OP_QUANTIZE, 128, 64, 0)

    def call(x=256, dtype=nv.BF16, rows=128, cols=64, ld=64, amax=None, o=out, w=256, wb=ws):
        return lib.nvfp4_quantize_transposed(x, dtype, rows, cols, ld, amax, ctypes.byref(o), w,
                                             wb, None)

    assert call(dtype=5) == nv.EINVAL
    assert call(x=None) == nv.EINVAL
    assert call(rows=-16) == nv.EINVAL
    assert call(rows=64) == nv.ESHAPE                         # out is not [cols x rows]
    assert call(o=T(16, 16, 64, 128, 64, nv.SCALES_ROWMAJOR)) == nv.ESHAPE
    assert call(cols=56, ld=56, o=T(16, 16, 64, 56, 128, nv.SCALES_ROWMAJOR)) == nv.ESHAPE
    assert call(ld=60) == nv.ESHAPE
    assert call(amax=258) == nv.ESHAPE
    assert call(w=None) == nv.EWORKSPACE
    assert call(o=T(16, 16, 64, 64, 128, nv.SCALES_TILED)) == nv.ESHAPE   # tiled needs 128 | out rows
    wide = 65535 * 128 + 16                                   # beyond the grid's column tiles
    assert call(cols=wide, ld=wide, o=T(16, 16, 64, wide, 128, nv.SCALES_ROWMAJOR)) == nv.ESHAPE


def test_default_scale_layout():
    import w4a4_gemm_amd as nv
    # tiled where the shape allows it, row-major otherwise (the GEMM takes either)
    assert nv.default_layout(4096, 3072) == nv.SCALES_TILED
    assert nv.default_layout(880, 3072) == nv.SCALES_ROWMAJOR      # rows % 128
    assert nv.default_layout(256, 48) == nv.SCALES_ROWMAJOR        # cols % 64
    assert nv.default_layout(0, 64) == nv.SCALES_TILED
