"""Oracle for paged-KV GQA split-KV decode attention: TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 CPU implementations written from the pages' description of
the method (decode attention over a paged GQA KV cache, split-KV tiles planned per
step by greedy bin-packing, a log-sum-exp combine, FP8 KV with per-tile scales, and
block-sparse decode under a precomputed block mask).
Only the tests, the smoke check and the bench's CPU-baseline leg may import this
package; the product path never does, and nothing here shares code with the HIP
library.

Modules: ``formats`` (exact bf16 / e4m3fn decoders), ``attention`` (the attention
definition), ``combine`` (log-sum-exp merge), ``plan`` (LPT planner spec).
Parity unpinned: the exact bf16 bits of the HIP outputs (compared by tolerance
only), and the quality of the automatic tile-size rule (its result is specified and
matched exactly, but the pages fix no particular tile size).
"""

from . import formats, attention, combine, plan  # noqa: F401
from .attention import decode_attention, partial_attention, gather_kv, sparse_keys  # noqa: F401
from .combine import lse_merge  # noqa: F401
