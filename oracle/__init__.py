"""CPU oracle for the int4 weight-streaming decode step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: it is read by the tests, by the smoke check
of the graft entry point and by the CPU-baseline leg of the benchmark, and by
nothing else.  It shares no code with the HIP library or its Python binding.

The oracle is plain numpy in float64: every step is the textbook definition,
applied to the same packed int4 codes and bf16 scales the GPU receives, so
quantisation loss is outside the comparison.  Sources are cited by page title
and section:
  * "Primer" -- the primer page "把基础打牢" (learn.longtimenohack.com, chasing
    primer), sections 1.1 (transformer block), 1.2 (prefill vs decode),
    1.3 (roofline), 1.4 (memory bill).
  * "Unsloth article" -- the zhichai.top article on how Unsloth runs Qwen 27B
    (archives/14776), sections 一 to 四 and its reference list.
  * "Roofline reply" -- the forum reply "从屋顶线模型看 Unsloth" (zhichai.net topic
    178634300), sections 一 to 八.

Parity status of each function is listed in the module docstring of
oracle.decode.
"""

from .decode import (  # noqa: F401
    bf16_round_bits,
    bf16_to_f64,
    decode_layer,
    decode_stack,
    prefill,
    dequant_int4,
    embed_tokens,
    gqa_decode_attention,
    greedy_decode,
    lm_head_argmax,
    lm_head_chunked_argmax,
    matvec,
    rmsnorm,
    rope,
    rope_angles,
    silu,
    swiglu,
    unpack_int4,
)
from .sample import gumbel_scores, philox4x32_10, sample_tokens, sample_tokens_topk, top_k_rows, uniforms  # noqa: F401
