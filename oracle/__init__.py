"""CPU oracle (float64) for GPTQ's per-layer quantization path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never imports, links or
calls it, and this package imports nothing from the product path: the two
share no code.  Shared seeded inputs come from
``post_weight_quantization_syrk_amd.synth``, which holds no step of the method.

Sources, cited by page title and section:
  [P1] "GPTQ：基于近似二阶信息的大模型权重量化" (freeguideonline.com tutorial)
  [P2] "GPTQ-2D: 三次时间复杂度的双侧自适应舍入" (ai-feeds.com paper summary)
  [P4] "GPTQ: практическое квантование языковых моделей без потери смысла"
       (serverflow.ru blog)
  [P5] "GPTQ/AWQ量化中Group Size的精确含义与计算" (group-size explainer)
"""
from .gptq_oracle import (NotSPD, hessian, hessian_entry, prepare, reversed_route_U,
                          group_params, quantize_values, gptq, column_loop, rtn,
                          layer_loss, fp16_rne, maxq_for)
from .storage import (bits_per_weight, model_gigabytes, round_half_up, pack_rows,
                      unpack_rows, words_per_row, fp16_bits)
from .gptq2d_oracle import two_sided_quartic, two_sided_antidiagonal
from .act_order import activation_order, gptq_ordered
from .dequant_gemm import dequantize, dequant_matmul

__all__ = [
    "NotSPD", "hessian", "hessian_entry", "prepare", "reversed_route_U", "group_params",
    "quantize_values", "gptq", "column_loop", "rtn", "layer_loss", "fp16_rne",
    "maxq_for", "bits_per_weight", "model_gigabytes", "round_half_up", "pack_rows",
    "unpack_rows", "words_per_row", "fp16_bits", "two_sided_quartic",
    "two_sided_antidiagonal", "activation_order", "gptq_ordered", "dequantize",
    "dequant_matmul",
]
