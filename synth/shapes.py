"""Model shapes of the decode workloads.

The 27B shape (64 query heads served by 8 KV heads, a vocabulary of about 152k
rows, a very wide SwiGLU) is the one the Unsloth/Qwen-27B article describes in
its sections 二.2 and 三; the other shapes are the common 7B- and 70B-class dense
GQA decoders the primer's section 1.1 uses for its size intuition.  Layer
widths the pages leave blank are fixed here as stated in the workload list.
"""

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    group: int
    rms_eps: float
    rope_base: float
    kv_len: int          # cached tokens before the step (the new token sits at this position)
    vocab: int = 0       # LM-head rows (0: no LM head in this workload)
    lm_chunk: int = 8192

    @property
    def q_width(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def gqa_group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw) -> "ModelShape":
        return replace(self, **kw)


SHAPES = {
    # one decoder layer, D=256, 4 query / 2 KV heads, hd 64, d_ff 688, 127 cached tokens
    "tiny": ModelShape("tiny", 1, 256, 4, 2, 64, 688, 64, 1e-6, 1e4, 127),
    # 7B-class stack
    "7b": ModelShape("7b", 28, 3584, 28, 4, 128, 18944, 128, 1e-6, 1e6, 4096),
    # 27B-class stack (the pages' model)
    "27b": ModelShape("27b", 64, 5120, 64, 8, 128, 17408, 128, 1e-6, 1e6, 8192),
    # 27B stack plus a 152064-row int4 LM head, chunks of 8192 rows
    "27b_lm": ModelShape("27b_lm", 64, 5120, 64, 8, 128, 17408, 128, 1e-6, 1e6, 8192, vocab=152064),
    # 70B-class stack, 32768 cached tokens per sequence
    "70b": ModelShape("70b", 80, 8192, 64, 8, 128, 28672, 128, 1e-6, 5e5, 32768),
}
