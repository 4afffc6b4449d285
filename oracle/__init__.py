"""CPU oracle for the weight-only-quantized linear layer.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct CPU
statement of what the device path computes. It exists so that tests can check the
library against something written independently of it. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it. The product path (the C-ABI library and its Python binding) never imports,
links or calls anything here, and this package imports nothing from the product.

What it computes: ``y[M,N] = x[M,K] . dequant(Wq)[N,K]^T`` with fp16 (or bfloat16)
activations and these weight formats: int8 per output row, int4 asymmetric in groups of
32 along K, FP6 e3m2 per output row (in two layouts: one for gfx950's bf6 convert and
one split 2+4 into power-of-two-wide parts), and, as further bit widths, FP4 e2m1 and FP5
e2m2 per output row and int3 asymmetric in groups of 32. These pages describe the method:

* gpt-fast write-up (m.greenbasetech.com): decode is bound by memory bandwidth, and
  int8, then groupwise int4, weight quantization cut the bytes per parameter.
* gpt-fast guide "终极PyTorch原生Transformer文本生成：gpt-fast极速体验指南"
  (www.jsqmd.com), section "量化技术深度解析": int4 with group size 32; section
  "混合精度训练与推理": bfloat16 as an alternative to fp16.
* FP6-LLM news "单卡跑Llama 70B快过双卡，微软硬生生把FP6搞到了A100里"
  (m.zhengruan.com), section "重新设计内核方案": FP6 weights dequantized to FP16
  inside one fused kernel, with the weights bit-level pre-packed offline into aligned
  32/64-bit blocks.

The pages fix no bit format, scale rule, rounding mode or layout. Every such choice
made here is a reading, and each is listed in the design notes of this repository.

Modules:
  formats   fp16 and bfloat16 rounding, the e3m2, e2m1 and e2m2 code tables and encodings
  quantize  int8 / int4-g32 / int3-g32 / fp6 / fp4 / fp5 quantizers (fp64 arithmetic)
  layout    the packed byte layout: a scalar bit-writer/reader and a vectorised packer
  linear    dequantisation to fp16 or bfloat16 and the fp64 reference linear, plus its error bound
  decode    the decode step around the linears (RMSNorm, rotary embedding, attention over a key/value
            cache, silu(gate)*up, residual stream, output layer, next token), imported as oracle.decode

Parity status: every function here is pinned by ``tests/test_oracle_*.py``. No
function is "parity unpinned".
"""

from .formats import (
    fp16_bits,
    fp16_from_bits,
    bf16_bits,
    bf16_from_bits,
    e3m2_value,
    e3m2_table,
    e3m2_encode,
    e2m1_value,
    e2m1_table,
    e2m1_encode,
    e2m2_value,
    e2m2_table,
    e2m2_encode,
)
from .quantize import (quantize_int8, quantize_int4_g32, quantize_int3_g32, quantize_fp6, quantize_fp4, quantize_fp5,
                       OracleRangeError)
from .layout import (
    FMT_F16,
    FMT_W8,
    FMT_W4G32,
    FMT_W6E3M2,
    FMT_W4E2M1,
    FMT_BF16,
    FMT_W5E2M2,
    FMT_W3G32,
    FMT_W6E3M2_P24,
    packed_bytes,
    scales_count,
    zeros_count,
    pack_scalar,
    unpack_scalar,
    pack_vectorized,
    unpack_vectorized,
)
from .linear import (
    ACT_F16,
    ACT_BF16,
    dequant_values,
    dequant_fp16,
    dequant_bf16,
    linear_ref,
    error_bound,
    quantize_and_pack,
)

__all__ = [
    "fp16_bits", "fp16_from_bits", "bf16_bits", "bf16_from_bits", "e3m2_value", "e3m2_table", "e3m2_encode",
    "e2m1_value", "e2m1_table", "e2m1_encode", "e2m2_value", "e2m2_table", "e2m2_encode",
    "quantize_int8", "quantize_int4_g32", "quantize_int3_g32", "quantize_fp6", "quantize_fp4", "quantize_fp5", "OracleRangeError",
    "FMT_F16", "FMT_W8", "FMT_W4G32", "FMT_W6E3M2", "FMT_W4E2M1", "FMT_BF16", "FMT_W5E2M2",
    "FMT_W3G32", "FMT_W6E3M2_P24",
    "packed_bytes", "scales_count", "zeros_count",
    "pack_scalar", "unpack_scalar", "pack_vectorized", "unpack_vectorized",
    "ACT_F16", "ACT_BF16", "dequant_values", "dequant_fp16", "dequant_bf16", "linear_ref", "error_bound",
    "quantize_and_pack",
]
