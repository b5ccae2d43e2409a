"""NVFP4 quantize / dequantize / W4A4 GEMM -- exact CPU oracle (test infrastructure only).

Definition followed (techwalker.com LongLive-2.0 report summary, section 一;
zuobiaodaohang LongLive blog, section "NVFP4：数据体积砍到 1/4"): a tensor is
stored as 4-bit E2M1 values, every 16 consecutive values share one FP8 scale,
and the whole tensor shares one FP32 scale.  Where the pages leave a step open
the reading is stated at the step.

For a row-major tensor X[rows, cols] with blocks of 16 along ``cols``:

1. amax = max |x| over the tensor.  s_g = RN32(amax / 2688), 2688 = 6 * 448
   (largest E2M1 magnitude times largest E4M3 value).  Reading: amax == 0
   gives s_g = 1.  s_g is the *decode* scale: x ~ q * s_b * s_g.
2. Block scale: b = max |x| over the block; s_b = E4M3 value nearest to the
   exact quotient b / (6 s_g), ties to even, saturating at 448.
3. Code: if s_b == 0 the magnitude is 0; else the E2M1 magnitude nearest to
   the exact quotient |x| / (s_b s_g), ties to even, saturating at 6.  The sign
   bit is the sign bit of x (so -0.0 and negatives that round to 0 give 0x8).
4. Packing: byte j of a row holds code 2j in bits 3:0 and code 2j+1 in bits 7:4.
5. Scale bytes: row-major [rows][cols/16], or the 128x4 tiled layout
   offset(r, kb) = ((r//128)*(cols//64) + kb//4)*512 + (r%128)*4 + kb%4.
6. Dequantize: fp32 = RN32(q s_b s_g); bf16 = RN_bf16(q s_b s_g), each a
   single rounding of the exact product.
7. GEMM  Y = X W^T  with X[M,K], W[N,K] NVFP4: the exact value
   Y = s_gx s_gw sum_k (q_x s_bx)(q_w s_bw), and A = sum_k |x^ w^|.

Exactness notes: rounding is done by counting the grid midpoints that lie
below the value (plus the even-side tie rule), and every comparison is
``b  vs  (6 s_g) * midpoint``  or  ``|x|  vs  (s_b s_g) * midpoint``.  Those
products have at most 24+2+5 = 31 significant bits, so they are exact in fp64,
and b, |x| are fp32 or bf16 numbers: every comparison is exact.
"""

from fractions import Fraction

import numpy as np

from . import formats as F

SCALES_ROWMAJOR = 0
SCALES_TILED = 1
BLOCK = 16
GLOBAL_DIVISOR = 2688            # 6 * 448


# --------------------------------------------------------------------------
# step 1: global scale
# --------------------------------------------------------------------------


def global_scale(amax: float) -> float:
    """s_g = RN32(amax / 2688); 1.0 when amax == 0 (reading); 2^-149, the
    smallest positive fp32, when a nonzero amax / 2688 rounds to zero (reading:
    the pages define no block scale for s_g = 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 1.0
    s = F.round_fraction_to_binary(Fraction(amax) / GLOBAL_DIVISOR, F.F32)
    return s if s != 0.0 else 2.0 ** -149


# --------------------------------------------------------------------------
# step 2: block scale bytes
# --------------------------------------------------------------------------


def block_scale_bytes(block_amax: np.ndarray, s_g: float) -> np.ndarray:
    """E4M3 byte nearest to b / (6 s_g), ties to even byte, saturating.

    Index = number of grid midpoints strictly below the quotient, plus one if
    the quotient equals a midpoint whose upper neighbour has an even byte.
    """
    b = np.asarray(block_amax, dtype=np.float64)
    thr = (6.0 * s_g) * F.E4M3_MIDPOINTS          # exact, see module note
    idx = np.searchsorted(thr, b, side="left")     # count of thr < b
    at = np.minimum(idx, thr.size - 1)
    tie = (idx < thr.size) & (thr[at] == b)
    up = tie & ((idx + 1) % 2 == 0)
    return (idx + up).astype(np.uint8)


# --------------------------------------------------------------------------
# step 3: element codes
# --------------------------------------------------------------------------


def element_codes(x: np.ndarray, s_b: np.ndarray, s_g: float) -> np.ndarray:
    """E2M1 codes of x given the (broadcast) block scale values s_b."""
    x = np.asarray(x, dtype=np.float64)
    s_b = np.broadcast_to(np.asarray(s_b, dtype=np.float64), x.shape)
    ax = np.abs(x)
    scale = s_b * s_g                               # <= 4 + 24 bits: exact
    mag = np.zeros(x.shape, dtype=np.int64)
    for k, mid in enumerate(F.E2M1_MIDPOINTS):
        t = scale * mid                             # <= 31 bits: exact
        mag += ax > t
        if (k + 1) % 2 == 0:                        # tie goes to the even code
            mag += ax == t
    mag = np.where(s_b == 0.0, 0, mag)
    sign = np.signbit(x).astype(np.int64) << 3
    return (mag | sign).astype(np.uint8)


# --------------------------------------------------------------------------
# steps 4-5: packing and scale layouts
# --------------------------------------------------------------------------


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """[rows, cols] 4-bit codes -> [rows, cols/2] bytes, even index in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] & 0xF) | ((codes[:, 1::2] & 0xF) << 4)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def tiled_offset(r, kb, cols: int):
    """Byte offset of the scale of (row r, block kb) in the tiled layout."""
    r = np.asarray(r, dtype=np.int64)
    kb = np.asarray(kb, dtype=np.int64)
    return ((r // 128) * (cols // 64) + kb // 4) * 512 + (r % 128) * 4 + kb % 4


def layout_scales(sb_rowmajor: np.ndarray, layout: int) -> np.ndarray:
    """[rows, cols/16] scale bytes -> flat bytes in the requested layout."""
    rows, nkb = sb_rowmajor.shape
    if layout == SCALES_ROWMAJOR:
        return np.ascontiguousarray(sb_rowmajor).reshape(-1).copy()
    assert layout == SCALES_TILED and rows % 128 == 0 and (nkb * 16) % 64 == 0
    out = np.zeros(rows * nkb, dtype=np.uint8)
    r, kb = np.meshgrid(np.arange(rows), np.arange(nkb), indexing="ij")
    out[tiled_offset(r, kb, nkb * 16)] = sb_rowmajor
    return out


def unlayout_scales(flat: np.ndarray, rows: int, cols: int, layout: int) -> np.ndarray:
    nkb = cols // 16
    flat = np.asarray(flat, dtype=np.uint8).reshape(-1)
    if layout == SCALES_ROWMAJOR:
        return flat.reshape(rows, nkb).copy()
    r, kb = np.meshgrid(np.arange(rows), np.arange(nkb), indexing="ij")
    return flat[tiled_offset(r, kb, cols)]


# --------------------------------------------------------------------------
# public: quantize / dequantize
# --------------------------------------------------------------------------


class NVFP4:
    """An oracle NVFP4 tensor: packed codes, scale bytes (row-major), s_g."""

    def __init__(self, packed, scales_rm, s_g):
        self.packed = np.asarray(packed, dtype=np.uint8)     # [rows, cols/2]
        self.scales = np.asarray(scales_rm, dtype=np.uint8)  # [rows, cols/16]
        self.s_g = float(s_g)

    @property
    def shape(self):
        return self.packed.shape[0], self.packed.shape[1] * 2

    def scales_in(self, layout):
        return layout_scales(self.scales, layout)


def quantize(x: np.ndarray, amax: float | None = None) -> NVFP4:
    """Quantize a 2-D array of exact values (fp32 or bf16 numbers as fp64).

    ``amax`` overrides step 1's tensor amax (a producer that already knows
    max|x|); by default it is computed.
    """
    x = np.asarray(x, dtype=np.float64)
    assert x.ndim == 2 and x.shape[1] % BLOCK == 0
    assert np.all(np.isfinite(x)), "non-finite input is outside the contract"
    rows, cols = x.shape
    if amax is None:
        amax = float(np.max(np.abs(x))) if x.size else 0.0
    s_g = global_scale(amax)
    xb = x.reshape(rows, cols // BLOCK, BLOCK)
    b = np.max(np.abs(xb), axis=2) if x.size else np.zeros((rows, 0))
    sb_bytes = block_scale_bytes(b, s_g)
    s_b = F.E4M3_GRID[sb_bytes]
    codes = element_codes(xb, s_b[:, :, None], s_g).reshape(rows, cols)
    return NVFP4(pack_codes(codes), sb_bytes, s_g)


def decoded_qsb(t: NVFP4) -> np.ndarray:
    """q * s_b for every element (exact fp64: at most 2 + 4 significant bits)."""
    rows, cols = t.shape
    q = F.E2M1_MAGNITUDES[unpack_codes(t.packed) & 7]
    q = np.where(unpack_codes(t.packed) & 8, -q, q)
    s_b = np.repeat(F.E4M3_GRID[t.scales], BLOCK, axis=1)
    return q * s_b


def dequantize(t: NVFP4, out: str = "f32") -> np.ndarray:
    """Dequantized values as exact fp64 numbers of the output format.

    out = "f32": RN32(q s_b s_g);  out = "bf16": RN_bf16(q s_b s_g).
    q s_b s_g has at most 6 + 24 significant bits, so it is exact in fp64 and
    one rounding to the output format is the exact single rounding.
    """
    exact = decoded_qsb(t) * t.s_g
    fmt = F.F32 if out == "f32" else F.BF16
    return F.round_f64_to_binary(exact, fmt)


# --------------------------------------------------------------------------
# GEMM
# --------------------------------------------------------------------------

_UNIT_EXP = -10       # every q*s_b is an integer multiple of 2^-10


def _qsb_units(t: NVFP4) -> np.ndarray:
    """q * s_b as int64 multiples of 2^-10 (|value| <= 2688 * 1024 < 2^22)."""
    v = np.ldexp(decoded_qsb(t), -_UNIT_EXP)
    iv = v.astype(np.int64)
    assert np.array_equal(iv.astype(np.float64), v)
    return iv


def exact_int_matmul(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Exact a @ b for int64 matrices with |entries| < 2^22 and inner dim <= 2^18.

    Each operand is split into 11-bit halves, so every fp64 BLAS product is
    at most 2^22 and every partial sum at most 2^40: all four fp64 matmuls are
    exact, and they recombine exactly in int64 (|terms| <= 2^62).
    """
    a = np.asarray(a, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    assert np.all(np.abs(a) < 2**22) and np.all(np.abs(b) < 2**22)
    assert a.shape[1] <= 2**18
    ah, al = np.divmod(a, 2**11)          # a = ah*2^11 + al, 0 <= al < 2^11
    bh, bl = np.divmod(b, 2**11)
    f = lambda u, v: (u.astype(np.float64) @ v.astype(np.float64)).astype(np.int64)
    return (f(ah, bh) << 22) + ((f(ah, bl) + f(al, bh)) << 11) + f(al, bl)


def gemm(x: NVFP4, w: NVFP4, rows=None, cols=None):
    """Y = X W^T and A = sum_k |x^ w^| as fp64 (within 2 fp64 ulps of the exact
    values: the exact integer sum is converted once and scaled once).

    ``rows``/``cols`` optionally select output rows / columns (index arrays)
    so that samples of a large product are computed exactly and cheaply.
    """
    xi = _qsb_units(x)
    wi = _qsb_units(w)
    if rows is not None:
        xi = xi[np.asarray(rows)]
    if cols is not None:
        wi = wi[np.asarray(cols)]
    acc = exact_int_matmul(xi, wi.T)               # units of 2^-20
    aab = exact_int_matmul(np.abs(xi), np.abs(wi).T)
    s = x.s_g * w.s_g                              # exact in fp64 (48 bits)
    y = np.ldexp(acc.astype(np.float64), 2 * _UNIT_EXP) * s
    a = np.ldexp(aab.astype(np.float64), 2 * _UNIT_EXP) * s
    return y, a


def gemm_pairs(x: NVFP4, w: NVFP4, rows, cols):
    """Exact Y[r_i, c_i] and A[r_i, c_i] for index pairs (one dot product each)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    xi = _qsb_units(x)[rows]
    wi = _qsb_units(w)[cols]
    acc = np.array([int(np.dot(a, b)) for a, b in zip(xi, wi)], dtype=object)
    aab = np.array([int(np.dot(np.abs(a), np.abs(b))) for a, b in zip(xi, wi)], dtype=object)
    s = x.s_g * w.s_g
    y = np.array([float(Fraction(int(v)) * Fraction(s) / 2**20) for v in acc])
    a = np.array([float(Fraction(int(v)) * Fraction(s) / 2**20) for v in aab])
    return y, a


# --------------------------------------------------------------------------
# GEMM acceptance (tolerance stated by the target, with the cancellation clause)
# --------------------------------------------------------------------------


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Unit in the last place of bf16 at |v| (subnormal-aware)."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    return np.ldexp(1.0, np.maximum(e - 1, -126) - 7)


def _bf16_order(v: np.ndarray) -> np.ndarray:
    """Monotone integer index of bf16 values (adjacent bf16 numbers differ by 1)."""
    bits = (np.asarray(v, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
    return np.where(bits & 0x8000, -(bits & 0x7FFF), bits)


def check_gemm_f32(y, y_ref, a_ref, rel=1e-3):
    """fp32 output: |Y - Y_ref| <= rel * A_ref elementwise.  Returns (ok, worst)."""
    err = np.abs(np.asarray(y, np.float64) - y_ref)
    bound = rel * a_ref
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0
    return bool(np.all(err <= bound)), worst


def check_gemm_bf16(y, y_ref, a_ref, rel=1e-3, clause_frac=1e-3):
    """bf16 output: within 1 bf16 ulp of RN_bf16(Y_ref); an element also passes
    if |Y - Y_ref| <= ulp_bf16(Y)/2 + rel*A_ref (cancellation clause), and at
    most ``clause_frac`` of the elements may need the clause.
    Returns (ok, n_clause, n_fail)."""
    y = np.asarray(y, np.float64)
    ref_b = F.round_f64_to_binary(y_ref, F.BF16)
    within_ulp = np.abs(_bf16_order(y) - _bf16_order(ref_b)) <= 1
    clause = ~within_ulp & (np.abs(y - y_ref) <= bf16_ulp(y) / 2 + rel * a_ref)
    fail = ~within_ulp & ~clause
    n_clause = int(np.sum(clause))
    n_fail = int(np.sum(fail))
    ok = n_fail == 0 and n_clause <= clause_frac * max(y.size, 1)
    return ok, n_clause, n_fail
