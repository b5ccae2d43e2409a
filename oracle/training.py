"""Training-side NVFP4 GEMMs (dgrad, wgrad) -- exact CPU oracle (test infrastructure only).

What the pages fix: LongLive-2.0 trains in NVFP4 (techwalker.com LongLive-2.0
report summary, section 一: training 2.15x faster than BF16; section 四:
NVFP4-aware training; section 五: teacher, student and critic all NVFP4
during distillation).  A linear's backward pass then multiplies in 4 bits
too: for Y = X W^T (X [M x K], W [N x K]),

    dgrad  dX [M x K] = dY W        contraction over N
    wgrad  dW [N x K] = dY^T X      contraction over M (the tokens)

Readings (the pages give no backward recipe):

* Every GEMM operand is quantized with the forward quantizer (same two-level
  scaling and round-to-nearest-even), blocks of 16 along that GEMM's
  contraction axis.  So dY is quantized as is for dgrad (blocks along N) and
  transposed for wgrad (blocks along M); W is quantized transposed for dgrad
  (blocks along N); X transposed for wgrad (blocks along M).  A transposed
  operand's tensor amax is that of the untransposed tensor.
* Stochastic rounding, random Hadamard transforms and 2-D weight blocks are
  not on the pages and are not part of this reading.
* The products then reuse the forward GEMM definition ``nvfp4.gemm``:
  Y = A B^T with both operands K-major NVFP4.
"""

import numpy as np

from . import nvfp4 as Q


def quantize_transposed(x: np.ndarray, amax: float | None = None) -> Q.NVFP4:
    """NVFP4 of X^T: output row k holds column k of X, blocks of 16 along X's rows."""
    x = np.asarray(x, dtype=np.float64)
    assert x.ndim == 2 and x.shape[0] % Q.BLOCK == 0
    return Q.quantize(np.ascontiguousarray(x.T), amax=amax)


def dgrad(dy_q: Q.NVFP4, w_t_q: Q.NVFP4):
    """dX = dY W from NVFP4 dY [M x N] and NVFP4 W^T [K x N]: exact (value, abs-sum)."""
    return Q.gemm(dy_q, w_t_q)


def wgrad(dy_t_q: Q.NVFP4, x_t_q: Q.NVFP4):
    """dW = dY^T X from NVFP4 dY^T [N x M] and NVFP4 X^T [K x M]: exact (value, abs-sum)."""
    return Q.gemm(dy_t_q, x_t_q)
