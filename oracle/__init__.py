"""Oracle for paged-KV GQA split-KV decode attention: TEST INFRASTRUCTURE ONLY.

Plain, slow CPU implementations written from the pages' description of the method
(decode attention over a paged GQA KV cache, split-KV tiles planned per step by
greedy bin-packing, a log-sum-exp combine, FP8 KV with per-tile scales, block-sparse
decode under a precomputed block mask, the fused KV append and variable-length
prefill), in float64 except where the method fixes float32 steps (the append).
Only the tests, the smoke check and the bench's CPU-baseline leg may import this
package; the product path never does, and nothing here shares code with the HIP
library.

Modules: ``formats`` (exact bf16 / e4m3fn decoders), ``attention`` (the attention
definition, dense and block-sparse), ``combine`` (log-sum-exp merge), ``plan`` (LPT
planner spec), ``append`` (rotary embedding, paged write, FP8 quantise-on-write, in
the float32 steps it specifies), ``prefill`` (causal prefill over the paged cache).
Parity unpinned: the exact bf16 bits of the HIP outputs (compared by tolerance
only), and the quality of the automatic tile-size rule (its result is specified and
matched exactly, but the pages fix no particular tile size).
"""

from . import formats, attention, combine, plan  # noqa: F401
from .attention import decode_attention, partial_attention, gather_kv, sparse_keys  # noqa: F401
from .combine import lse_merge  # noqa: F401
