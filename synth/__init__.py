"""Seeded synthetic workloads shared by the tests, the bench and the oracle checks."""

from .configs import (ALL, TINY, LLAMA8B, MIXED, LONG, FP8_SPEC, softmax_scale,  # noqa: F401
                      ALL_PREFILL, PREFILL_VARLEN, PREFILL_LONG, PREFILL_CHUNK_FP8)
from .gen import (DecodeInputs, make_inputs, apply_poison, algorithmic_bytes,  # noqa: F401
                  f32_to_bf16_bits, f32_to_e4m3fn, draw_seq_lens, BF16_NAN, FP8_NAN,
                  make_block_mask, attended_pages, sparse_algorithmic_bytes, rope_tables,
                  new_token_rows, append_algorithmic_bytes, PrefillInputs,
                  make_prefill_inputs, prefill_flops)
