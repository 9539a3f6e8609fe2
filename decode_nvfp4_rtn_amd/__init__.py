"""MI355X-native (gfx950) quantized linear layer: NVFP4 W4A4 prefill and
weight-only (INT4 group-128, 2-bit codebook) decode.

The compute lives in the C-ABI shared library ``libqlin.so`` (hand-written HIP
kernels, declared in ``include/qlin.h``).  ``decode_nvfp4_rtn_amd.qlin`` is
the thin Python binding over it; importing it loads the library and raises if
it has not been built.  ``synth`` draws the seeded synthetic inputs and
``configs`` lists the measured layer shapes.
"""

__version__ = "0.1.0"
