"""CPU oracle for the NVFP4 hot path -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, exact reference that the HIP kernels are
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product library
(``w4a4_gemm_amd``) never imports, calls or links anything here, and this
package never imports the product library.  The two share no code; the only
common module is ``synth`` (seeded input generators, no method arithmetic).

What it computes, and where the pages define it:

* NVFP4 two-level block quantization -- 4-bit E2M1 values, one FP8 (E4M3)
  scale per 16 consecutive values, one FP32 scale per tensor
  (techwalker.com LongLive-2.0 report summary, section 一 "给AI视频生成做一次
  瘦身手术"; zuobiaodaohang LongLive blog, section "NVFP4：数据体积砍到 1/4").
* Dequantization and the W4A4 matrix product, "all matrix multiplications in
  4-bit" (techwalker summary, section 四, first key).
* The NVFP4 KV cache: K mean-subtracted, then NVFP4-quantized; many cache
  blocks of a window dequantized at once (techwalker summary, section 四,
  second key), attention over such a window, and the multi-shot sink window
  as a page list (techwalker summary, section 六).
* The producer-fused activation quantize: LayerNorm + adaLN modulate + NVFP4
  in one step (zuobiaodaohang LongLive blog, section "NVFP4：数据体积砍到
  1/4"; ai-manual.ru LongLive-2.0 article, section "Как это работает под
  капотом").
* The training-side GEMMs (dgrad, wgrad) with operands quantized along the
  contraction axis, including the transposed quantizer (techwalker summary,
  sections 一 and 五: NVFP4 training and distillation).

Every rounding is a single round-to-nearest-even of the exact real value,
evaluated with exact comparisons (fp64 products that are provably exact,
integer arithmetic, or ``fractions.Fraction``).  Each module states the
argument for exactness next to the code that relies on it.

Pins: every public function is pinned in ``tests/test_oracle_*.py`` against
something other than itself (library conversions, exhaustive tables,
closed forms, ``Fraction`` brute force, values printed on the pages).
"""

from . import formats, nvfp4, kvcache, window, adaln, training  # noqa: F401
