"""Closed-form algorithmic bytes and FLOPs of one decode step.

The roofline view comes from the Roofline reply (sections 一 and 二: intensity =
operations / bytes moved, batch-1 decode sits far below the ridge) and from the
Primer (section 1.2: decode time is bounded by reading every weight once;
section 1.3: roofline; section 1.4: the memory bill, whose KV term is
2 * H_kv * d_h * bytes * L * B * S).

Algorithmic bytes of one step are what the step must move at least once:
int4 codes and bf16 scales (or bf16 weights) of the seven matrices of every
layer, the two bf16 norm gains, the bf16 KV read over pos+1 keys and the bf16
K/V write of the new token, per sequence, plus the LM head's codes and scales
when present.  Activation vectors (kilobytes against megabytes) are excluded.
"""

import math

HBM_PEAK_BYTES_PER_S = 8.0e12          # MI355X published HBM3E bandwidth


def matrix_bytes(n: int, k: int, group: int, weight_dtype: str = "int4") -> int:
    if weight_dtype == "int4":
        return n * k // 2 + n * math.ceil(k / group) * 2
    if weight_dtype == "bf16":
        return n * k * 2
    raise ValueError(weight_dtype)


def layer_matrices(shape):
    D, qw, kvw, F = shape.d_model, shape.q_width, shape.kv_width, shape.d_ff
    return {"wq": (qw, D), "wk": (kvw, D), "wv": (kvw, D), "wo": (D, qw),
            "wg": (F, D), "wu": (F, D), "wd": (D, F)}


def layer_weight_bytes(shape, weight_dtype: str = "int4") -> int:
    return sum(matrix_bytes(n, k, shape.group, weight_dtype) for n, k in layer_matrices(shape).values()) \
        + 2 * shape.d_model * 2


def kv_read_bytes(shape, batch: int, keys: int) -> int:
    return batch * 2 * shape.n_kv_heads * keys * shape.head_dim * 2


def kv_write_bytes(shape, batch: int) -> int:
    return batch * 2 * shape.n_kv_heads * shape.head_dim * 2


def lm_head_bytes(vocab: int, d_model: int, group: int) -> int:
    return matrix_bytes(vocab, d_model, group, "int4")


def step_bytes(shape, batch: int, keys: int, weight_dtype: str = "int4", n_layers=None, lm_head: bool = False) -> int:
    """Algorithmic HBM bytes of one decode step; `keys` = pos + 1 keys attended."""
    L = shape.n_layers if n_layers is None else n_layers
    per_layer = layer_weight_bytes(shape, weight_dtype) + kv_read_bytes(shape, batch, keys) + kv_write_bytes(shape, batch)
    total = L * per_layer
    if lm_head:
        total += lm_head_bytes(shape.vocab, shape.d_model, shape.group)
    return total


def phase_bytes(shape, phase: str, batch: int, keys: float, weight_dtype: str = "int4") -> float:
    """Algorithmic HBM bytes of one launch of one kernel of the step:
    qkv (Wq, Wk, Wv, the attention norm gain, the new K/V), attention (the
    cache over `keys` keys), wo, gate_up (Wg, Wu, the FFN norm gain), down,
    lm_head (the whole head: one launch sweeps every chunk) and stream
    (the streaming kernel: the whole stack of one call)."""
    m = layer_matrices(shape)
    mb = {n: matrix_bytes(r, c, shape.group, weight_dtype) for n, (r, c) in m.items()}
    if phase == "qkv":
        return mb["wq"] + mb["wk"] + mb["wv"] + shape.d_model * 2 + kv_write_bytes(shape, batch)
    if phase == "attention":
        return kv_read_bytes(shape, batch, keys)
    if phase == "wo":
        return mb["wo"]
    if phase == "gate_up":
        return mb["wg"] + mb["wu"] + shape.d_model * 2
    if phase == "down":
        return mb["wd"]
    if phase == "lm_head":
        return lm_head_bytes(shape.vocab, shape.d_model, shape.group)
    if phase == "stream":
        return step_bytes(shape, batch, keys, weight_dtype)
    raise ValueError(phase)


def step_flops(shape, batch: int, keys: int, n_layers=None, lm_head: bool = False) -> int:
    """2 x multiply-adds of one step over the batch (matrix products and attention)."""
    L = shape.n_layers if n_layers is None else n_layers
    macs_w = sum(n * k for n, k in layer_matrices(shape).values())
    macs_attn = 2 * shape.n_q_heads * keys * shape.head_dim
    total = L * batch * 2 * (macs_w + macs_attn)
    if lm_head:
        total += batch * 2 * shape.vocab * shape.d_model
    return total


def prefill_flops(shape, n_tokens: int, pos0: int = 0, n_layers=None) -> dict:
    """2 x multiply-adds of a prefill of n_tokens prompt tokens at positions
    pos0 .. pos0 + n_tokens - 1 (token t attends pos0 + t + 1 keys), per
    projection of one layer and in total."""
    L = shape.n_layers if n_layers is None else n_layers
    m = layer_matrices(shape)
    per = {"qkv": 2 * n_tokens * (m["wq"][0] + m["wk"][0] + m["wv"][0]) * shape.d_model,
           "wo": 2 * n_tokens * m["wo"][0] * m["wo"][1],
           "gate_up": 2 * n_tokens * (m["wg"][0] + m["wu"][0]) * m["wg"][1],
           "down": 2 * n_tokens * m["wd"][0] * m["wd"][1]}
    keys = n_tokens * pos0 + n_tokens * (n_tokens + 1) // 2
    per["attention"] = 4 * shape.n_q_heads * shape.head_dim * keys      # q.k and p.v per key
    return {"per_layer": per, "total": L * sum(per.values())}


def decode_latency_bound_s(weight_bytes: float, bandwidth: float) -> float:
    """Lower bound of one decode step: every weight read once (Primer 1.2)."""
    return weight_bytes / bandwidth


def estimate_mem(params_B, L, D, H_q, H_kv, d_h, S, B, bytes_per=2) -> dict:
    """The Primer's section 1.4 memory bill, in bytes: weights, KV cache,
    Adam state (two fp32 moments plus an fp16 master copy) and training
    activations (B*S*L*D*2*bytes)."""
    return {
        "weights": params_B * 1e9 * bytes_per,
        "kv": 2 * H_kv * d_h * bytes_per * L * B * S,
        "adam": params_B * 1e9 * (4 + 4 + 2),
        "act": B * S * L * D * 2 * bytes_per,
    }
