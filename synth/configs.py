"""The five synthetic decode workloads (shapes only; values come from ``synth.gen``).

Each workload is a plain dict. ``seq_lens`` is either a fixed tuple or a recipe
(``("loguniform", lo, hi)`` / ``("uniform_int", lo, hi)``) that ``synth.gen`` draws
first from the seeded generator. Names describe the workload, never a list index.
"""

import math

TINY = dict(
    name="tiny",
    desc="tiny GQA paged decode: B=4, seq_lens {17,64,100,255}, 4 q / 1 kv head, "
         "D=64, page 16, bf16 KV, 1 query token",
    batch=4, seq_lens=(17, 64, 100, 255), q_len=1,
    num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=16, kv_format="bf16",
)

LLAMA8B = dict(
    name="llama8b",
    desc="Llama-3-8B-shaped decode: B=64, seq_len 4096, 32 q / 8 kv heads, D=128, "
         "page 16, bf16 KV, 1 query token",
    batch=64, seq_lens=("const", 4096), q_len=1,
    num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, kv_format="bf16",
)

MIXED = dict(
    name="mixed",
    desc="mixed-length decode: B=128, seq_lens log-uniform in [128, 32768] (seed 0), "
         "32 q / 8 kv heads, D=128, page 16, bf16 KV, 1 query token",
    batch=128, seq_lens=("loguniform", 128, 32768), q_len=1,
    num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, kv_format="bf16",
)

LONG = dict(
    name="long",
    desc="long-context small-batch decode: B=2, seq_len 65536, 64 q / 8 kv heads, "
         "D=128, page 64, bf16 KV, 1 query token",
    batch=2, seq_lens=("const", 65536), q_len=1,
    num_q_heads=64, num_kv_heads=8, head_dim=128, page_size=64, kv_format="bf16",
)

FP8_SPEC = dict(
    name="fp8_spec",
    desc="FP8-KV speculative decode: B=32, seq_lens uniform in [1024, 16384] (seed 0), "
         "32 q / 8 kv heads, D=128, page 64, e4m3fn KV with an fp32 scale per "
         "64-token page per kv head, 4 query tokens causal within the draft",
    batch=32, seq_lens=("uniform_int", 1024, 16384), q_len=4,
    num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64, kv_format="fp8",
)

ALL = {c["name"]: c for c in (TINY, LLAMA8B, MIXED, LONG, FP8_SPEC)}

# Variable-length prefill over the same paged cache. ``q_lens`` is a recipe like
# ``seq_lens`` above; ``prefix`` (the tokens already in the cache before the chunk,
# 0 for a whole prompt) is a fixed tuple or a recipe; kv length = prefix + q length.
PREFILL_VARLEN = dict(
    name="prefill_varlen",
    desc="variable-length prefill: B=8 prompts, lengths log-uniform in [128, 16384] "
         "(seed 0), 32 q / 8 kv heads, D=128, page 16, bf16 KV, causal",
    batch=8, q_lens=("loguniform", 128, 16384), prefix=("const", 0),
    num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, kv_format="bf16",
)

PREFILL_LONG = dict(
    name="prefill_long",
    desc="long prefill: one 65536-token prompt, 32 q / 8 kv heads, D=128, page 64, "
         "bf16 KV, causal",
    batch=1, q_lens=("const", 65536), prefix=("const", 0),
    num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64, kv_format="bf16",
)

PREFILL_CHUNK_FP8 = dict(
    name="prefill_chunk_fp8",
    desc="chunked prefill over an FP8 cache: B=4 chunks of 2048 tokens after prefixes "
         "uniform in [0, 16384] (seed 0), 32 q / 8 kv heads, D=128, page 64, e4m3fn KV "
         "with per-page scales, causal",
    batch=4, q_lens=("const", 2048), prefix=("uniform_int", 0, 16384),
    num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64, kv_format="fp8",
)

ALL_PREFILL = {c["name"]: c for c in (PREFILL_VARLEN, PREFILL_LONG, PREFILL_CHUNK_FP8)}


def softmax_scale(head_dim):
    """1/sqrt(head_dim), the scale every workload uses (passed to both sides as fp32)."""
    return 1.0 / math.sqrt(head_dim)
