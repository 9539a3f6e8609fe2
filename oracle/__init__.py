"""CPU oracle for the quantized linear layer (test infrastructure only).

This package is the plain, slow, obviously-correct definition that the HIP
library is checked against.  It is *test infrastructure*: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (``decode_nvfp4_rtn_amd``) never imports it and
shares no code with it; the two meet only in the seeded input generator
(``decode_nvfp4_rtn_amd/synth.py``), which draws random numbers and holds none
of the method's arithmetic.

Arithmetic convention.  Every binary32 operation of the method is evaluated
once in float64 and then rounded to float32 (``rn32``).  For a single
+, -, *, / on binary32 operands this equals the correctly rounded binary32
result, because float64 carries 53 >= 2*24+2 bits (S. A. Figueroa, "When is
double rounding innocuous?", SIGNUM Newsletter 30(3), 1995).  The final
matrix products are taken in float64 on exactly dequantized operands.

Modules
-------
formats  E2M1 / E4M3 codecs, binary32 and bfloat16 rounding.
nvfp4    NVFP4 round-to-nearest quantizer (activations and weights).
int4     Symmetric INT4 quantizer with 128-element groups and bf16 scales.
sparse24 2:4 magnitude pruning along k on top of int4.
lut2     2-bit per-row codebook (K-means, Lloyd iterations).
gemm     Matrix products on dequantized operands and the pass rule.

Pins (what ties each function to something other than itself) live in
``tests/test_oracle_*.py``.  ``lut2.lloyd`` is pinned to scikit-learn's
KMeans (Lloyd's algorithm from the same initial centroids, ten iterations)
on rows whose clusters all stay populated; its start, tie rule, empty-cluster
rule, final rounding and re-assignment are pinned by closed forms, brute
force and special cases.
"""

from . import formats, nvfp4, int4, sparse24, lut2, gemm  # noqa: F401
