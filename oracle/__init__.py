"""Plain fp64 CPU oracle for the tiled attention forward pass.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the graft entry's
smoke check and the benchmark's CPU-baseline leg may import anything here. The
HIP library never calls into this package and this package never calls into
the HIP library; the two share no code, headers, tables or constants. The only
thing both sides consume is the seeded input generator in ``attn_inputs``,
which holds no attention arithmetic.

Modules
  attention  exact two-pass attention (the definition) and the online-softmax
             recurrence, both fp64
  fp8        the OCP E4M3FN number format and the per-block / per-tensor
             quantiser, from the format definition
  rotation   incoherent processing: the random-sign Hadamard rotation of Q
             and K (its definition in fp64, and the fp32 butterfly whose
             values decide the rotated quantiser's codes)
  decode     attention of a few queries against a longer key/value sequence
             (the last positions, bottom-right causal alignment), fp64
  merge      the merge of partial results over disjoint key sets (their
             log-sum-exp weighted combination), fp64
  paged      decode attention against a paged key/value cache: the block
             table's page gather, then the decode oracle
  metrics    the error measures used to compare a result with the oracle

Sources (web pages on FlashAttention-3, cited by title and section):
  [WGC]  "Warp Group Cluster 优化：Flash Attention V3 在 H100 上的 FP8 融合计算实践"
  [JJ]   "大模型加速-核心网络算子-Flash Attention V3"
  [YT]   "FlashAttention V3：优化框架吞吐量的关键技术实践"

Every function in this package is pinned by CPU tests against something
other than itself: the attention, decode, paged and merge oracles by library
routines, closed forms, invariants and brute force (``tests/test_oracle*.py``),
the E4M3 model and the quantiser by torch's float8 type, the format facts the
pages print and the quantiser's defining error bound at every block magnitude
(``tests/test_fp8_model.py``), and the error measures by closed-form cases
(``tests/test_oracle_metrics.py``).
"""
from .attention import (allowed_range, attention_two_pass, attention_online,
                        probabilities, attention_rows)
from .fp8 import (E4M3_MAX, e4m3_decode_table, e4m3_decode, e4m3_encode,
                  quantize, dequantize, QUANT_BLOCK_ROWS)
from .decode import attention_decode
from .paged import attention_decode_paged, gather_pages
from .merge import lse_merge
from .rotation import hadamard_matrix, rotate, rotate_fp32, fwht_fp32
from .metrics import max_abs, l1_rel, rmse_rel

__all__ = [
    "allowed_range", "attention_two_pass", "attention_online", "probabilities",
    "attention_rows", "E4M3_MAX", "e4m3_decode_table", "e4m3_decode",
    "e4m3_encode", "quantize", "dequantize", "QUANT_BLOCK_ROWS", "max_abs",
    "l1_rel", "rmse_rel", "lse_merge", "attention_decode", "attention_decode_paged",
    "gather_pages", "hadamard_matrix", "rotate", "rotate_fp32", "fwht_fp32",
]
