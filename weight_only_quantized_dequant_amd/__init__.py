"""Weight-only-quantized linear layers (W8 / W4-g32 / W6-e3m2 weights, fp16 activations) for AMD MI355X.

The library is ``libwq.so`` (include/wq.h); ``weight_only_quantized_dequant_amd.wq`` is
its Python binding, and ``weight_only_quantized_dequant_amd.build`` compiles it in place
for gfx950. Importing this package loads nothing; the binding loads the library on first
use.
"""

__version__ = "1.0"
