"""CPU oracle for the QuantWM 2-bit KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 restatement
of what the method computes, written from the QuantWM pages (arXiv
2609.26425 v2 and its digests).  Only the test-suite, the smoke check of the
package entry point and the CPU-baseline leg of the benchmark may import it.
It shares no code with the HIP library and imports nothing from it; the two
meet only on inputs produced by the `datagen` module.

Modules
  formats    - number formats (bf16 / fp16 rounding), exact quotient rounding,
               the packed storage layout
  stats      - Query second moment, channel weights, principal basis (Jacobi)
  lloyd      - seeded Forgy initialisation and Lloyd iterations
  quantize   - QSAC centroid choice, INT2 residual codec, PSAC coefficients,
               value quantization
  attention  - dequantization and softmax attention over the compressed cache,
               top-1 token selection, the BF16 decoder
  prq        - QVG's progressive (multi-stage) residual quantization
  accounting - bits per token-head and compression ratios

Parity pins: every function is pinned by tests under tests/test_oracle_*.py
against closed forms, library routines, brute force or values printed on the
pages.  No function of this package is "parity unpinned".
"""
from . import formats, stats, lloyd, quantize, attention, accounting  # noqa: F401
