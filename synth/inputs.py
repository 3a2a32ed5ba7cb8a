"""Seeded host-side generators for every input of the decode step.

Recipe (the workload list of the decode benchmark):
  * weights are drawn N(0, 0.02) in float32 and quantised to int4 with a
    zero-point of 8: per group of `group` consecutive inputs along K, the scale is
    the bf16 round-to-nearest-even of max|w| / 7 (computed in float32), and the
    code is clip(rint(w / scale) + 8, 0, 15) with rint rounding half to even;
    an all-zero group gets scale 0 and code 8.  Two codes share a byte, the
    even-K code in the low nibble.  The last group of a row may be short.
  * norm gains are bf16(1 + 0.1 N(0, 1)).
  * the KV cache holds bf16 N(0, 1) values for slots below each sequence's
    position; every other slot holds a bf16 quiet NaN so that any read of a
    slot the step must not touch poisons the result.
  * the new token's hidden state is bf16 N(0, 1), carried as float32.
  * the bf16-weight variant draws the same N(0, 0.02) weights and rounds them
    to bf16 instead of quantising.

Every tensor comes from numpy's PCG64 seeded with SeedSequence([seed, layer,
tensor id, extra]), so any subset can be regenerated independently.
"""

import numpy as np

TENSOR_IDS = {
    "attn_norm": 0, "wq": 1, "wk": 2, "wv": 3, "wo": 4, "ffn_norm": 5,
    "wg": 6, "wu": 7, "wd": 8, "k_cache": 9, "v_cache": 10, "x": 11,
    "w_lm": 12, "lm_hidden": 13, "embed": 14,
}

BF16_QNAN = np.uint16(0x7FC0)


def rng_for(seed: int, layer: int, tensor: str, extra: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, TENSOR_IDS[tensor], extra])))


def bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_int4(w: np.ndarray, group: int):
    """Offline int4 quantiser of the input recipe.  w: float32 [N][K], K even.

    Returns (codes uint8 [N][K/2], scales uint16 bf16 bits [N][ceil(K/group)]).
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    assert k % 2 == 0
    ng = (k + group - 1) // group
    pad = ng * group - k
    wp = np.pad(w, ((0, 0), (0, pad))) if pad else w
    wg = wp.reshape(n, ng, group)
    amax = np.abs(wg).max(axis=2)                                   # float32
    s_bits = bf16_bits(amax / np.float32(7.0))
    s = bf16_value(s_bits)                                          # float32
    safe = np.where(s == 0, np.float32(1.0), s)
    q = np.rint(wg / safe[:, :, None]).astype(np.int32) + 8
    q = np.where((s == 0)[:, :, None], 8, q)
    q = np.clip(q, 0, 15).reshape(n, ng * group)[:, :k].astype(np.uint8)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(codes), np.ascontiguousarray(s_bits)


def _normal_weights(seed, layer, name, n, k):
    return rng_for(seed, layer, name).standard_normal((n, k), dtype=np.float32) * np.float32(0.02)


def _gain(seed, layer, name, d):
    return bf16_bits(np.float32(1.0) + np.float32(0.1) * rng_for(seed, layer, name).standard_normal(d, dtype=np.float32))


def make_layer(shape, seed: int, layer: int, weight_dtype: str = "int4") -> dict:
    """All parameters of one decoder layer.  Matrices are stored [out][in].

    int4 matrices are dicts {codes, scales, n, k, group}; bf16 matrices are
    dicts {bf16 [n][k] uint16, n, k}.
    """
    D, qw, kvw, F = shape.d_model, shape.q_width, shape.kv_width, shape.d_ff
    dims = {"wq": (qw, D), "wk": (kvw, D), "wv": (kvw, D), "wo": (D, qw),
            "wg": (F, D), "wu": (F, D), "wd": (D, F)}
    out = {"attn_norm": _gain(seed, layer, "attn_norm", D), "ffn_norm": _gain(seed, layer, "ffn_norm", D)}
    for name, (n, k) in dims.items():
        w = _normal_weights(seed, layer, name, n, k)
        if weight_dtype == "int4":
            codes, scales = quantize_int4(w, shape.group)
            out[name] = {"codes": codes, "scales": scales, "n": n, "k": k, "group": shape.group}
        elif weight_dtype == "bf16":
            out[name] = {"bf16": bf16_bits(w), "n": n, "k": k}
        else:
            raise ValueError(weight_dtype)
    return out


def make_kv(shape, seed: int, layer: int, batch: int, pos, capacity: int):
    """Logical KV cache [B][Hkv][capacity][hd] bf16 bits for K and V.

    Slots t < pos[b] hold bf16 N(0,1); all others hold a quiet NaN.
    """
    pos = np.broadcast_to(np.asarray(pos, dtype=np.int64), (batch,))
    H, hd = shape.n_kv_heads, shape.head_dim
    kc = np.full((batch, H, capacity, hd), BF16_QNAN, dtype=np.uint16)
    vc = np.full((batch, H, capacity, hd), BF16_QNAN, dtype=np.uint16)
    for b in range(batch):
        p = int(pos[b])
        if p > 0:
            kc[b, :, :p, :] = bf16_bits(rng_for(seed, layer, "k_cache", b).standard_normal((H, p, hd), dtype=np.float32))
            vc[b, :, :p, :] = bf16_bits(rng_for(seed, layer, "v_cache", b).standard_normal((H, p, hd), dtype=np.float32))
    return kc, vc


def make_x(shape, seed: int, batch: int, step: int = 0) -> np.ndarray:
    """New-token hidden states [B][D]: bf16 N(0,1) values as float32."""
    return bf16_value(bf16_bits(rng_for(seed, 0, "x", step).standard_normal((batch, shape.d_model), dtype=np.float32)))


def make_lm_head(vocab: int, d_model: int, group: int, seed: int) -> dict:
    """int4 LM-head matrix [vocab][d_model], quantised N(0, 0.02), built in row blocks."""
    codes = np.empty((vocab, d_model // 2), dtype=np.uint8)
    ng = (d_model + group - 1) // group
    scales = np.empty((vocab, ng), dtype=np.uint16)
    blk = 8192
    for i, r0 in enumerate(range(0, vocab, blk)):
        r1 = min(vocab, r0 + blk)
        w = rng_for(seed, i, "w_lm").standard_normal((r1 - r0, d_model), dtype=np.float32) * np.float32(0.02)
        codes[r0:r1], scales[r0:r1] = quantize_int4(w, group)
    return {"codes": codes, "scales": scales, "n": vocab, "k": d_model, "group": group}


def make_hidden(d_model: int, seed: int, batch: int) -> np.ndarray:
    """Final hidden state fed to the LM head: bf16 N(0,1) values as float32 [B][D]."""
    return bf16_value(bf16_bits(rng_for(seed, 0, "lm_hidden").standard_normal((batch, d_model), dtype=np.float32)))


def make_embedding(vocab: int, d_model: int, seed: int) -> np.ndarray:
    """bf16 embedding table [vocab][d_model] (bit patterns), N(0,1) values."""
    return bf16_bits(rng_for(seed, 0, "embed").standard_normal((vocab, d_model), dtype=np.float32))

