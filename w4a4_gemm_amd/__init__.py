"""Python binding of the NVFP4 hot path on AMD Instinct MI355X (gfx950).

A thin ctypes layer over ``libnvfp4.so`` (C ABI in ``include/nvfp4.h``).
Functions carry the C names; they only marshal torch tensors (device memory,
the current HIP stream) into pointers and sizes.  Every step of the path runs
in the library's HIP kernels; there is no Python or CPU fallback, and a
missing or broken library raises at import time.

    import w4a4_gemm_amd as nv
    xq = nv.nvfp4_quantize(x)                       # NVFP4Tensor
    y  = nv.nvfp4_gemm_w4a4(xq, wq, torch.bfloat16)
"""

import ctypes
import importlib.util
import os

import torch

__all__ = [
    "NVFP4Tensor", "KVCache", "LIB_PATH",
    "nvfp4_abi_version", "nvfp4_status_string", "nvfp4_workspace_bytes", "nvfp4_kv_page_bytes",
    "nvfp4_quantize", "nvfp4_dequantize", "nvfp4_gemm_w4a4", "nvfp4_adaln_quantize",
    "nvfp4_quantize_transposed", "nvfp4_quantize_noalloc",
    "nvfp4_kv_quantize", "nvfp4_kv_dequant_blocks", "nvfp4_kv_attention", "nvfp4_kv_window_pages",
    "SCALES_ROWMAJOR", "SCALES_TILED", "OP_QUANTIZE", "OP_KV_QUANTIZE", "OP_KV_ATTENTION",
    "OP_ADALN_QUANTIZE", "default_layout",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4.so")

# enums (include/nvfp4.h)
OK, EINVAL, ESHAPE, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
SCALES_ROWMAJOR, SCALES_TILED = 0, 1
OP_QUANTIZE, OP_KV_QUANTIZE, OP_KV_ATTENTION, OP_ADALN_QUANTIZE = 0, 1, 2, 3
ABI_VERSION = 1

EXPORTS = (
    "nvfp4_abi_version", "nvfp4_status_string", "nvfp4_source_hash", "nvfp4_workspace_bytes",
    "nvfp4_kv_page_bytes",
    "nvfp4_quantize", "nvfp4_dequantize", "nvfp4_gemm_w4a4", "nvfp4_adaln_quantize",
    "nvfp4_quantize_transposed", "nvfp4_quantize_noalloc",
    "nvfp4_kv_quantize", "nvfp4_kv_dequant_blocks", "nvfp4_kv_attention", "nvfp4_kv_window_pages",
)


class _Tensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("global_scale", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("scale_layout", ctypes.c_int32)]


class _KVCache(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_void_p), ("n_phys_pages", ctypes.c_int64),
                ("n_layers", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_tokens", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("max_chunks", ctypes.c_int32),
                ("page_table", ctypes.c_void_p), ("page_chunk", ctypes.c_void_p),
                ("k_mean", ctypes.c_void_p), ("k_gscale", ctypes.c_void_p),
                ("v_gscale", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python w4a4_gemm_amd/build.py` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "nvfp4_abi_version": (ctypes.c_int, []),
        "nvfp4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "nvfp4_source_hash": (ctypes.c_char_p, []),
        "nvfp4_workspace_bytes": (sz, [i32, i64, i64, i64]),
        "nvfp4_kv_page_bytes": (i64, [i32, i32, i32]),
        "nvfp4_quantize": (ctypes.c_int, [vp, i32, i64, i64, i64, vp, ctypes.POINTER(_Tensor),
                                          vp, sz, vp]),
        "nvfp4_quantize_noalloc": (ctypes.c_int, [vp, i32, i64, i64, i64, vp,
                                                  ctypes.POINTER(_Tensor), vp]),
        "nvfp4_dequantize": (ctypes.c_int, [ctypes.POINTER(_Tensor), vp, i32, i64, vp]),
        "nvfp4_quantize_transposed": (ctypes.c_int, [vp, i32, i64, i64, i64, vp,
                                                     ctypes.POINTER(_Tensor), vp, sz, vp]),
        "nvfp4_adaln_quantize": (ctypes.c_int, [vp, i32, i64, i64, i64, vp, vp, i64, ctypes.c_float,
                                                vp, ctypes.POINTER(_Tensor), vp, sz, vp]),
        "nvfp4_gemm_w4a4": (ctypes.c_int, [ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), vp,
                                           i32, i64, vp, vp]),
        "nvfp4_kv_quantize": (ctypes.c_int, [ctypes.POINTER(_KVCache), i32, i32, vp, vp, i64, i64,
                                             vp, sz, vp]),
        "nvfp4_kv_dequant_blocks": (ctypes.c_int, [ctypes.POINTER(_KVCache), i32, vp, i32, vp, vp,
                                                   vp]),
        "nvfp4_kv_attention": (ctypes.c_int, [ctypes.POINTER(_KVCache), i32, vp, i32, i32, vp, i64,
                                              ctypes.c_float, vp, vp, sz, vp]),
        "nvfp4_kv_window_pages": (ctypes.c_int, [i64, i32, i64, i64, i64, i64, vp, i32,
                                                 ctypes.POINTER(i32), ctypes.POINTER(i32), vp]),
    }
    for name, (res, args) in sig.items():
        if not hasattr(lib, name):
            raise ImportError(f"{LIB_PATH} lacks {name}: rebuild it with "
                              "`python w4a4_gemm_amd/build.py`")
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    if lib.nvfp4_abi_version() != ABI_VERSION:
        raise ImportError("libnvfp4.so ABI version mismatch: rebuild the library")
    # the library must have been built from the sources next to it
    spec = importlib.util.spec_from_file_location(
        "nvfp4_srchash", os.path.join(os.path.dirname(LIB_PATH), "srchash.py"))
    srchash = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(srchash)
    want, got = srchash.source_hash(), lib.nvfp4_source_hash().decode()
    if got != want:
        raise ImportError(f"{LIB_PATH} was built from other sources (hash {got[:12]}, sources "
                          f"{want[:12]}): rebuild it with `python w4a4_gemm_amd/build.py`")
    return lib


_lib = _load()


def _check(status, what):
    if status != OK:
        msg = _lib.nvfp4_status_string(status).decode()
        raise RuntimeError(f"{what} failed: status {status} ({msg})")


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else ctypes.c_void_p(0)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_buffer(t, name, dtype, device, numel=None, shape=None):
    """A caller-supplied buffer: its dtype, device, size and layout are checked
    here because the C ABI sees only a pointer."""
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _need(t.device == torch.device(device), f"{name} must be on {device}, got {t.device}")
    if shape is not None:
        _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got "
              f"{tuple(t.shape)}")
        _need(t.dim() == 0 or t.stride(-1) == 1 or t.numel() == 0,
              f"{name} must have unit stride in its last dimension")
    else:
        _need(t.is_contiguous(), f"{name} must be contiguous")
        _need(t.numel() >= numel, f"{name} holds {t.numel()} elements, needs {numel}")


def _check_nvfp4(t, name, device=None):
    """An NVFP4Tensor's three buffers hold rows x cols codes, scale bytes and s_g."""
    _need(isinstance(t, NVFP4Tensor), f"{name} must be an NVFP4Tensor")
    device = t.global_scale.device if device is None else device
    n = t.rows * t.cols
    _check_buffer(t.codes, f"{name}.codes", torch.uint8, device, numel=n // 2)
    _check_buffer(t.scales, f"{name}.scales", torch.uint8, device, numel=n // 16)
    _check_buffer(t.global_scale, f"{name}.global_scale", torch.float32, device, numel=1)


def _dtype_code(dt):
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {dt}")


# ------------------------------------------------------------------ plain calls


def nvfp4_abi_version():
    return _lib.nvfp4_abi_version()


def nvfp4_status_string(status):
    return _lib.nvfp4_status_string(status).decode()


def nvfp4_workspace_bytes(op, a, b, c):
    return int(_lib.nvfp4_workspace_bytes(op, a, b, c))


def nvfp4_kv_page_bytes(n_heads, head_dim, page_tokens):
    return int(_lib.nvfp4_kv_page_bytes(n_heads, head_dim, page_tokens))


class NVFP4Tensor:
    """Device buffers of an NVFP4 tensor [rows x cols]: codes, scale bytes, s_g."""

    def __init__(self, rows, cols, layout=SCALES_TILED, device="cuda", codes=None, scales=None,
                 global_scale=None):
        self.rows, self.cols, self.layout = int(rows), int(cols), int(layout)
        self.codes = codes if codes is not None else torch.empty(
            (rows, cols // 2), dtype=torch.uint8, device=device)
        self.scales = scales if scales is not None else torch.empty(
            (rows * cols // 16,), dtype=torch.uint8, device=device)
        self.global_scale = global_scale if global_scale is not None else torch.empty(
            (1,), dtype=torch.float32, device=device)

    def c(self):
        return _Tensor(self.codes.data_ptr() if self.codes.numel() else 0,
                       self.scales.data_ptr() if self.scales.numel() else 0,
                       self.global_scale.data_ptr(), self.rows, self.cols, self.layout)

    @property
    def shape(self):
        return self.rows, self.cols


def default_layout(rows, cols):
    """The tiled scale layout where the shape allows it (rows % 128 == 0 and
    cols % 64 == 0), else row-major; the GEMM takes either."""
    return SCALES_TILED if rows % 128 == 0 and cols % 64 == 0 else SCALES_ROWMAJOR


def nvfp4_quantize(x, layout=None, amax=None, out=None, workspace=None, stream=None):
    """Quantize a 2-D bf16/fp32 CUDA tensor (row stride x.stride(0)) to NVFP4
    (``layout`` None: default_layout of the shape)."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    if layout is None:
        layout = default_layout(rows, cols)
    if out is None:
        out = NVFP4Tensor(rows, cols, layout, device=x.device)
    _check_nvfp4(out, "out", x.device)
    if amax is not None:
        _check_buffer(amax, "amax", torch.float32, x.device, numel=1)
    need = nvfp4_workspace_bytes(OP_QUANTIZE, rows, cols, 1 if amax is not None else 0)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace is not None:
        _check_buffer(workspace, "workspace", torch.uint8, x.device, numel=need)
    cs = out.c()
    st = _lib.nvfp4_quantize(_ptr(x), _dtype_code(x.dtype), rows, cols, x.stride(0),
                             _ptr(amax), ctypes.byref(cs), _ptr(workspace),
                             workspace.numel() if workspace is not None else 0, _stream(stream))
    _check(st, "nvfp4_quantize")
    return out


def nvfp4_quantize_noalloc(x, layout=None, amax=None, out=None, stream=None):
    """nvfp4_quantize without a workspace: the library's per-device scratch array
    holds the amax partials (calls that overlap on one GPU race).  ``out`` must be
    given by callers that cannot allocate."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    if layout is None:
        layout = default_layout(rows, cols)
    if out is None:
        out = NVFP4Tensor(rows, cols, layout, device=x.device)
    _check_nvfp4(out, "out", x.device)
    if amax is not None:
        _check_buffer(amax, "amax", torch.float32, x.device, numel=1)
    cs = out.c()
    st = _lib.nvfp4_quantize_noalloc(_ptr(x), _dtype_code(x.dtype), rows, cols, x.stride(0),
                                     _ptr(amax), ctypes.byref(cs), _stream(stream))
    _check(st, "nvfp4_quantize_noalloc")
    return out


def nvfp4_quantize_transposed(x, layout=None, amax=None, out=None, workspace=None,
                              stream=None):
    """NVFP4 of x^T (blocks of 16 along x's rows) for a 2-D bf16/fp32 CUDA tensor
    (``layout`` None: default_layout of the [cols x rows] output)."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    if layout is None:
        layout = default_layout(cols, rows)
    if out is None:
        out = NVFP4Tensor(cols, rows, layout, device=x.device)
    _check_nvfp4(out, "out", x.device)
    if amax is not None:
        _check_buffer(amax, "amax", torch.float32, x.device, numel=1)
    need = nvfp4_workspace_bytes(OP_QUANTIZE, rows, cols, 1 if amax is not None else 0)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace is not None:
        _check_buffer(workspace, "workspace", torch.uint8, x.device, numel=need)
    cs = out.c()
    st = _lib.nvfp4_quantize_transposed(_ptr(x), _dtype_code(x.dtype), rows, cols, x.stride(0),
                                        _ptr(amax), ctypes.byref(cs), _ptr(workspace),
                                        workspace.numel() if workspace is not None else 0,
                                        _stream(stream))
    _check(st, "nvfp4_quantize_transposed")
    return out


def nvfp4_adaln_quantize(x, shift, scale, rows_per_group, eps=1e-6, layout=None,
                         out=None, row_stats=None, workspace=None, stream=None):
    """LayerNorm + adaLN modulate + NVFP4 of a 2-D bf16/fp32 CUDA tensor -> (NVFP4Tensor, row_stats).

    ``shift``/``scale``: fp32 [ceil(rows / rows_per_group), cols]; ``row_stats``
    receives fp32 [rows, 2] = (mean, rstd) per row."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    for v in (shift, scale):
        if v.dtype != torch.float32 or not v.is_contiguous():
            raise ValueError("shift and scale must be contiguous fp32")
    rows, cols = x.shape
    if layout is None:
        layout = default_layout(rows, cols)
    groups = -(-rows // rows_per_group) if rows_per_group > 0 else 0
    if rows and cols and (shift.shape != (groups, cols) or scale.shape != (groups, cols)):
        raise ValueError(f"shift/scale must be [{groups}, {cols}]")
    if out is None:
        out = NVFP4Tensor(rows, cols, layout, device=x.device)
    _check_nvfp4(out, "out", x.device)
    for v, name in ((shift, "shift"), (scale, "scale")):
        _need(v.device == x.device, f"{name} must be on {x.device}")
    if row_stats is None:
        row_stats = torch.empty((rows, 2), dtype=torch.float32, device=x.device)
    _check_buffer(row_stats, "row_stats", torch.float32, x.device, numel=2 * rows)
    need = nvfp4_workspace_bytes(OP_ADALN_QUANTIZE, rows, cols, 0)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check_buffer(workspace, "workspace", torch.uint8, x.device, numel=need)
    cs = out.c()
    st = _lib.nvfp4_adaln_quantize(_ptr(x), _dtype_code(x.dtype), rows, cols, x.stride(0),
                                   _ptr(shift), _ptr(scale), rows_per_group, eps, _ptr(row_stats),
                                   ctypes.byref(cs), _ptr(workspace), workspace.numel(),
                                   _stream(stream))
    _check(st, "nvfp4_adaln_quantize")
    return out, row_stats


def nvfp4_dequantize(t, dtype=torch.float32, out=None, stream=None):
    """x^ = q s_b s_g of an NVFP4Tensor as fp32 or bf16 [rows x cols]; ``out``
    may be a row-strided 2-D view."""
    _check_nvfp4(t, "t")
    if out is None:
        out = torch.empty((t.rows, t.cols), dtype=dtype, device=t.codes.device)
    _check_buffer(out, "out", out.dtype if out.dtype in (torch.float32, torch.bfloat16) else dtype,
                  t.codes.device, shape=(t.rows, t.cols))
    cs = t.c()
    st = _lib.nvfp4_dequantize(ctypes.byref(cs), _ptr(out), _dtype_code(out.dtype),
                               out.stride(0) if t.rows > 1 else t.cols, _stream(stream))
    _check(st, "nvfp4_dequantize")
    return out


def nvfp4_gemm_w4a4(x, w, dtype=torch.bfloat16, out=None, y_amax=None, stream=None):
    """Y = X W^T for NVFP4 X [M x K], W [N x K]; ``out`` may be a row-strided 2-D view."""
    _check_nvfp4(x, "x")
    _check_nvfp4(w, "w", x.codes.device)
    if out is None:
        out = torch.empty((x.rows, w.rows), dtype=dtype, device=x.codes.device)
    _check_buffer(out, "out", out.dtype if out.dtype in (torch.float32, torch.bfloat16) else dtype,
                  x.codes.device, shape=(x.rows, w.rows))
    if y_amax is not None:
        _check_buffer(y_amax, "y_amax", torch.float32, x.codes.device, numel=1)
    xs, ws = x.c(), w.c()
    st = _lib.nvfp4_gemm_w4a4(ctypes.byref(xs), ctypes.byref(ws), _ptr(out), _dtype_code(out.dtype),
                              out.stride(0) if x.rows > 1 else w.rows, _ptr(y_amax),
                              _stream(stream))
    _check(st, "nvfp4_gemm_w4a4")
    return out


# ------------------------------------------------------------------ KV cache


class KVCache:
    """Device buffers of a paged NVFP4 KV cache (layout in include/nvfp4.h)."""

    def __init__(self, n_layers, n_heads, head_dim, page_tokens, max_pages, max_chunks,
                 page_table, n_phys_pages, device="cuda"):
        self.n_layers, self.n_heads, self.head_dim = n_layers, n_heads, head_dim
        self.page_tokens, self.max_pages, self.max_chunks = page_tokens, max_pages, max_chunks
        self.n_phys_pages = n_phys_pages
        self.page_bytes = nvfp4_kv_page_bytes(n_heads, head_dim, page_tokens)
        self.pool = torch.zeros((n_phys_pages, self.page_bytes), dtype=torch.uint8, device=device)
        self.page_table = torch.as_tensor(page_table, dtype=torch.int32).reshape(
            n_layers, max_pages).to(device).contiguous()
        self.page_chunk = torch.zeros((n_layers, max_pages, 2), dtype=torch.int32, device=device)
        self.k_mean = torch.zeros((n_layers, max_chunks, n_heads, head_dim), dtype=torch.float32,
                                  device=device)
        self.k_gscale = torch.zeros((n_layers, max_chunks), dtype=torch.float32, device=device)
        self.v_gscale = torch.zeros((n_layers, max_chunks), dtype=torch.float32, device=device)
        self._c = _KVCache(self.pool.data_ptr(), n_phys_pages, n_layers, n_heads, head_dim,
                           page_tokens, max_pages, max_chunks, self.page_table.data_ptr(),
                           self.page_chunk.data_ptr(), self.k_mean.data_ptr(),
                           self.k_gscale.data_ptr(), self.v_gscale.data_ptr())
        self._ws = None

    def c(self):
        return self._c

    def workspace(self, T):
        need = nvfp4_workspace_bytes(OP_KV_QUANTIZE, T, self.n_heads, self.head_dim)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.pool.device)
        return self._ws


def nvfp4_kv_quantize(cache, layer, chunk_id, k, v, start_token, workspace=None, stream=None):
    """Write one chunk (K, V bf16 [T, n_heads, head_dim]) into the cache in place."""
    T = k.shape[0]
    if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("K and V must be bf16")
    if not (k.is_contiguous() and v.is_contiguous()) or k.shape != v.shape:
        raise ValueError("K and V must be contiguous [T, n_heads, head_dim] of the same shape")
    if tuple(k.shape[1:]) != (cache.n_heads, cache.head_dim):
        raise ValueError("K shape does not match the cache")
    _need(k.device == cache.pool.device and v.device == cache.pool.device,
          "K and V must be on the cache's device")
    ws = workspace if workspace is not None else cache.workspace(T)
    _check_buffer(ws, "workspace", torch.uint8, cache.pool.device,
                  numel=nvfp4_workspace_bytes(OP_KV_QUANTIZE, T, cache.n_heads, cache.head_dim))
    st = _lib.nvfp4_kv_quantize(ctypes.byref(cache.c()), layer, chunk_id, _ptr(k), _ptr(v), T,
                                start_token, _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "nvfp4_kv_quantize")


def nvfp4_kv_dequant_blocks(cache, layer, logical_pages, k_out=None, v_out=None, stream=None):
    """Dequantize the listed logical pages -> (K^, V^) bf16 [n*page_tokens, H, D]."""
    _check_buffer(logical_pages, "logical_pages", torch.int32, cache.pool.device, numel=0)
    n = logical_pages.numel()
    shape = (n * cache.page_tokens, cache.n_heads, cache.head_dim)
    if k_out is None:
        k_out = torch.empty(shape, dtype=torch.bfloat16, device=cache.pool.device)
    if v_out is None:
        v_out = torch.empty(shape, dtype=torch.bfloat16, device=cache.pool.device)
    need = shape[0] * shape[1] * shape[2]
    _check_buffer(k_out, "k_out", torch.bfloat16, cache.pool.device, numel=need)
    _check_buffer(v_out, "v_out", torch.bfloat16, cache.pool.device, numel=need)
    st = _lib.nvfp4_kv_dequant_blocks(ctypes.byref(cache.c()), layer, _ptr(logical_pages), n,
                                      _ptr(k_out), _ptr(v_out), _stream(stream))
    _check(st, "nvfp4_kv_dequant_blocks")
    return k_out, v_out


def nvfp4_kv_attention(cache, layer, logical_pages, last_page_tokens, q, softmax_scale,
                       out=None, workspace=None, stream=None):
    """Attention of q bf16 [n_q, H, D] over the listed window, read from the NVFP4 pages."""
    if q.dtype != torch.bfloat16 or not q.is_contiguous():
        raise TypeError("q must be contiguous bf16 [n_q, n_heads, head_dim]")
    if tuple(q.shape[1:]) != (cache.n_heads, cache.head_dim):
        raise ValueError("q must be [n_q, n_heads, head_dim]")
    _need(q.device == cache.pool.device, "q must be on the cache's device")
    if out is None:
        out = torch.empty_like(q)
    _check_buffer(out, "out", torch.bfloat16, q.device, numel=q.numel())
    _need(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    _check_buffer(logical_pages, "logical_pages", torch.int32, q.device, numel=0)
    n = logical_pages.numel()
    need = nvfp4_workspace_bytes(OP_KV_ATTENTION, q.shape[0], cache.n_heads, n * cache.page_tokens)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _check_buffer(workspace, "workspace", torch.uint8, q.device, numel=need)
    st = _lib.nvfp4_kv_attention(ctypes.byref(cache.c()), layer, _ptr(logical_pages), n,
                                 last_page_tokens, _ptr(q), q.shape[0], float(softmax_scale),
                                 _ptr(out), _ptr(workspace),
                                 workspace.numel() if workspace is not None else 0,
                                 _stream(stream))
    _check(st, "nvfp4_kv_attention")
    return out


def nvfp4_kv_window_pages(total_tokens, page_tokens, global_sink_tokens, shot_start,
                          shot_sink_tokens, window_tokens, pages=None, max_pages=None,
                          device="cuda", stream=None):
    """Logical page list of a multi-shot sink window -> (device int32 pages, last_page_tokens).

    ``pages`` (device int32) receives the list; by default one is allocated with room for
    every page of the cache.  The returned tensor is the filled prefix."""
    if pages is None:
        n_max = max(1, -(-total_tokens // page_tokens))
        pages = torch.empty(n_max, dtype=torch.int32, device=device)
    if max_pages is None:
        max_pages = pages.numel()
    _check_buffer(pages, "pages", torch.int32, pages.device, numel=max_pages)
    n, last = ctypes.c_int32(0), ctypes.c_int32(0)
    st = _lib.nvfp4_kv_window_pages(total_tokens, page_tokens, global_sink_tokens, shot_start,
                                    shot_sink_tokens, window_tokens, _ptr(pages), max_pages,
                                    ctypes.byref(n), ctypes.byref(last), _stream(stream))
    _check(st, "nvfp4_kv_window_pages")
    return pages[:n.value], last.value
