"""CPU oracle for int8 / int4 / 2-bit KV-cache decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the benchmark's CPU-baseline leg use it.  It shares no
code, constants or helpers with the HIP library and imports nothing from it.

The oracle is plain numpy.  Quantization decisions (codes, scales) are taken in
float32, the precision the source pages' engine uses, with IEEE-rounded
division and C ``roundf`` (ties away from zero).  Attention outputs are
computed in float64 from the dequantized operands: the exact value, up to
float64 rounding, of the quantity the single-pass kernel approximates in
float32.

Sources (cited by these short names throughout):

  [P1] "Day 9-3: q8 KV precision comparison -- how much does quantization move
       the attention output" (jianying88.com, news/32654).  Sec. 1 experiment
       design, Sec. 2 the quantization rule, Sec. 3 the measured errors,
       Sec. 4 exercises (amplitude x3).
  [P2] "0.8MB runs Qwen, part 9-1: the engine's KV is quantized too -- q8 KV
       halves cache and decode bandwidth" (developer.aliyun.com, article
       1767759).  Sec. 2 allocation and per-(token, head) write path, byte
       accounting.
  [P3] "Day 9-2: flash_attn_single_q_q8_neon -- one query, one pass over all
       KV" (dtytms.com, news/32657).  Sec. 1 why one pass suffices, Sec. 2
       segments 1 (Q quantization), 2 (scoring + online softmax), 3 (final
       normalization), Sec. 3 the two-pass contrast, Sec. 4 exercises.
  [P4] "UltraQuant: 4-bit KV cache quantization on AMD GPUs" (seekfood.cn,
       news/2668800).  Sec. 3.2 group-wise asymmetric INT4, Sec. 3.3
       temporal-adaptive precision, Sec. 5.2 failure checklist.

Parity status per function is listed in each module's header.
"""
from . import kvq8, kvq4, kvq4_0, kvq2  # noqa: F401
