"""Producer-fused activation quantize: LayerNorm + adaLN modulate + NVFP4 --
exact CPU oracle (test infrastructure only).

What the pages fix: the NVFP4 inference path fuses the adaLN step into one
kernel (zuobiaodaohang LongLive blog, section "NVFP4：数据体积砍到 1/4",
"further optimisation" item), and scaling and quantization are merged into
one kernel (ai-manual.ru LongLive-2.0 article, section "Как это работает под
капотом").  The activations that feed the W4A4 linears of a DiT block are the
adaLN-modulated, layer-normalised residual stream, so the fused producer reads
the residual x once per pass and emits NVFP4 directly.

Readings (the pages name the step but do not define it):

* adaLN is LayerNorm without its own affine parameters followed by the
  modulation  x' = n * (1 + scale) + shift, the DiT form.  ``shift`` and
  ``scale`` are fp32 vectors over the channels, one pair per group of
  ``rows_per_group`` consecutive rows (a latent frame of a chunk-wise
  generated video carries its own conditioning); rows_per_group = rows gives
  one pair for the whole tensor.
* Row statistics: mu = mean of the row, var = mean of (x - mu)^2 (biased),
  rstd = 1 / sqrt(var + eps); both stored as fp32.  They are real-valued
  quantities that the kernel may evaluate in any order, so they are compared
  within a tolerance (``row_stats`` evaluates them in fp64: an exact mean via
  math.fsum, a two-pass variance).
* Elementwise arithmetic is fp32 with one rounding per operation, in the
  order the formula is written (the eager fp32 evaluation, no fused
  multiply-add):  n = RN32(RN32(x - mu) * rstd),  a = RN32(1 + scale),
  x' = RN32(RN32(n * a) + shift).
* x' (fp32 values) is then quantized exactly as ``oracle.nvfp4.quantize``
  defines; the tensor amax is max |x'|.

Given the fp32 statistics, x' and the NVFP4 result are unique, so the kernel's
codes, scales and s_g are compared bit for bit against ``adaln_quantize`` fed
the kernel's own statistics (the decision is taken in the same precision on
both sides), and the statistics against ``row_stats`` within a tolerance.

Exactness: every step uses ``formats.round_sum_to_binary`` (RNE of an exact
sum, TwoSum) or ``formats.round_f64_to_binary`` of a product of two fp32
numbers, which is exact in fp64 (24 + 24 significant bits).
"""

import math

import numpy as np

from . import formats as F
from . import nvfp4 as Q


def row_stats(x: np.ndarray, eps: float):
    """(mu, rstd) per row as fp64 arrays of fp32 values.

    mu = RN32(S / cols) with S the exact row sum (math.fsum is correctly
    rounded, and the fp64 quotient then rounds once more to fp32);
    var = fp64 two-pass mean of (x - S/cols)^2; rstd = RN32(1 / sqrt(var + eps)).
    """
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    mu64 = np.array([math.fsum(r) for r in x]) / cols if cols else np.zeros(rows)
    var = np.mean((x - mu64[:, None]) ** 2, axis=1) if cols else np.zeros(rows)
    rstd = 1.0 / np.sqrt(var + float(np.float32(eps)))
    return F.round_f64_to_binary(mu64, F.F32), F.round_f64_to_binary(rstd, F.F32)


def group_index(rows: int, rows_per_group: int) -> np.ndarray:
    """Modulation group of every row: row // rows_per_group."""
    return np.arange(rows) // rows_per_group


def modulate(x, mu, rstd, shift, scale, rows_per_group):
    """x' = RN32(RN32(n * RN32(1 + scale)) + shift), n = RN32(RN32(x - mu) * rstd)."""
    x = F.f32(x)
    rows, cols = x.shape
    mu = F.f32(mu)[:, None]
    rstd = F.f32(rstd)[:, None]
    g = group_index(rows, rows_per_group)
    shift = F.f32(shift)[g]
    scale = F.f32(scale)[g]
    d = F.round_sum_to_binary(x, -mu, F.F32)
    n = F.round_f64_to_binary(d * rstd, F.F32)
    a = F.round_sum_to_binary(np.ones_like(scale), scale, F.F32)
    p = F.round_f64_to_binary(n * a, F.F32)
    return F.round_sum_to_binary(p, shift, F.F32)


def adaln_quantize(x, shift, scale, rows_per_group, eps, stats=None):
    """(NVFP4 tensor, mu, rstd).  ``stats`` = (mu, rstd) replaces ``row_stats``."""
    x = np.asarray(x, dtype=np.float64)
    mu, rstd = row_stats(x, eps) if stats is None else stats
    xp = modulate(x, mu, rstd, shift, scale, rows_per_group)
    return Q.quantize(xp), mu, rstd
