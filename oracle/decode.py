"""float64 reference of one decode step of a dense GQA decoder stack with int4 weights.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Each function is the plain definition of one step, written from the pages:
  * Primer 1.1: a decoder block is RMSNorm -> q, k, v projections -> heads ->
    rotary position encoding of q and k -> causal softmax attention scaled by
    1/sqrt(head_dim) -> merge heads -> output projection added to the residual
    -> RMSNorm -> feed-forward network added to the residual.
  * Primer 1.2: at decode one token enters, every layer reads all cached K/V
    of its layer and appends the new token's K/V; the last hidden state times
    the embedding matrix gives the vocabulary logits, from which a token is
    sampled (greedy here).  Prefill runs the prompt's tokens through the same
    computation; each prompt token gets what decoding it after the tokens
    before it would give (prefill()).
  * Unsloth article 二.1: the feed-forward network is SwiGLU, SiLU of the gate
    projection times the up projection, then the down projection.
  * Unsloth article 二.2: grouped-query attention -- each KV head serves a
    group of query heads, addressed by index, no copy.
  * Unsloth article 二.3: weights live in HBM as int4 codes plus scale factors
    and are expanded to floating point only at the point of use.
  * Unsloth article 三: the large vocabulary's logits are produced chunk by
    chunk instead of being materialised at once.

Readings where the pages are silent (each listed with its reason in the design
notes): RMSNorm is x * rsqrt(mean(x^2) + eps) * gain; weights are stored
[out][in] and groups run along the input axis; a code c stands for (c - 8) *
scale; RoPE rotates the half-split pairs (i, i + hd/2) by pos * base^(-2i/hd)
with the angle in float64; the query head h reads KV head h // (Hq/Hkv); the
new token's K and V are rounded to bf16 (round to nearest even) when appended
and read back from the cache; no final RMSNorm before the LM head; ties of the
greedy argmax go to the lowest token id.

Parity pins (tests/test_oracle_pins.py) cover every function here; none is
"parity unpinned".
"""

import numpy as np


# ----------------------------------------------------------------------------- bf16

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_round_bits(x) -> np.ndarray:
    """float64 -> bf16 bit patterns, round to nearest even, for finite values in
    the bf16 normal range (the KV values of this workload).  Computed from the
    definition: keep 8 significant bits of the binary significand."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0)                  # round half to even at 8 significant bits
    v = np.ldexp(r, e - 8)                  # exactly representable in bf16
    return (v.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------- int4 weights

def unpack_int4(codes: np.ndarray, k: int) -> np.ndarray:
    """Two 4-bit codes per byte; the even input index sits in the low nibble
    (Unsloth article 二.3: int4 storage).  Returns int64 codes [N][k] in 0..15."""
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[0]
    out = np.empty((n, codes.shape[1] * 2), dtype=np.int64)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out[:, :k]


def dequant_int4(codes: np.ndarray, scales: np.ndarray, k: int, group: int) -> np.ndarray:
    """W[n, i] = (c[n, i] - 8) * scale[n, i // group]  (Unsloth article 二.3:
    codes are expanded by their scale factor at the point of use)."""
    c = unpack_int4(codes, k).astype(np.float64)
    s = bf16_to_f64(scales)
    return (c - 8.0) * s[:, np.arange(k) // group]


# Recently expanded small matrices, kept so that a long sequence of decode
# steps over the same weights does not expand them again at every step (the
# values are the same either way).  Each entry holds the code and scale arrays
# it was made from, so an entry is only reused for those very arrays.
_DENSE_MEMO = []
_DENSE_MEMO_MAX, _DENSE_MEMO_ELEMS = 16, 1 << 22


def _dense(mat: dict, r0: int = 0, r1=None) -> np.ndarray:
    r1 = mat["n"] if r1 is None else r1
    if "codes" in mat:
        small = (r1 - r0) * mat["k"] <= _DENSE_MEMO_ELEMS
        if small:
            for codes, scales, a, b, w in _DENSE_MEMO:
                if codes is mat["codes"] and scales is mat["scales"] and a == r0 and b == r1:
                    return w
        w = dequant_int4(mat["codes"][r0:r1], mat["scales"][r0:r1], mat["k"], mat["group"])
        if small:
            _DENSE_MEMO.append((mat["codes"], mat["scales"], r0, r1, w))
            del _DENSE_MEMO[:-_DENSE_MEMO_MAX]
        return w
    return bf16_to_f64(mat["bf16"][r0:r1])


def matvec(mat: dict, h: np.ndarray, block_rows: int = 8192) -> np.ndarray:
    """y[b, n] = sum_i W[n, i] * h[b, i]  (Primer 1.1: the projections h @ W,
    with W stored [out][in]).  Rows are dequantised a block at a time only to
    bound host memory; each output is the plain dot product."""
    h = np.asarray(h, dtype=np.float64)
    out = np.empty((h.shape[0], mat["n"]), dtype=np.float64)
    for r0 in range(0, mat["n"], block_rows):
        r1 = min(mat["n"], r0 + block_rows)
        out[:, r0:r1] = h @ _dense(mat, r0, r1).T
    return out


# ----------------------------------------------------------------------------- elementwise pieces

def rmsnorm(x: np.ndarray, gain_bits: np.ndarray, eps: float) -> np.ndarray:
    """x * 1/sqrt(mean(x^2) + eps) * gain over the last axis (Primer 1.1 names
    RMSNorm; the formula is the standard root-mean-square normalisation)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * bf16_to_f64(gain_bits)


def rope_angles(pos: int, head_dim: int, base: float) -> np.ndarray:
    """phi_i = pos * base^(-2i/head_dim), i < head_dim/2, in float64 (RoFormer,
    cited by the Unsloth article's reference list; Roofline reply 五: rotation
    of dimension pairs)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return float(pos) * np.power(float(base), -2.0 * i / head_dim)


def rope(t: np.ndarray, pos: int, base: float) -> np.ndarray:
    """Rotate each pair (t[i], t[i + hd/2]) by phi_i:
    t'[i] = t[i] cos - t[i+hd/2] sin,  t'[i+hd/2] = t[i] sin + t[i+hd/2] cos."""
    t = np.asarray(t, dtype=np.float64)
    hd = t.shape[-1]
    phi = rope_angles(pos, hd, base)
    c, s = np.cos(phi), np.sin(phi)
    a, b = t[..., : hd // 2], t[..., hd // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) (the Swish of the Unsloth article's SwiGLU)."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """SiLU(x W_gate) elementwise-times (x W_up)  (Unsloth article 二.1)."""
    return silu(gate) * np.asarray(up, dtype=np.float64)


# ----------------------------------------------------------------------------- attention

def gqa_decode_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, pos) -> np.ndarray:
    """Decode attention of one new token per sequence.

    q: [B][Hq][hd] float64 (already rotated); k_cache, v_cache: bf16 bits
    [B][Hkv][cap][hd] holding the new token's K/V at slot pos[b].  The query at
    position p sees keys 0..p (the causal mask of Primer 1.1 admits exactly
    these); scores are q.k / sqrt(hd); query head h reads KV head h // G
    (Unsloth article 二.2).  Returns o [B][Hq][hd]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, hd = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    o = np.empty_like(q)
    for b in range(B):
        p = int(pos[b])
        for h in range(Hq):
            j = h // G
            kk = bf16_to_f64(k_cache[b, j, : p + 1])
            vv = bf16_to_f64(v_cache[b, j, : p + 1])
            s = kk @ q[b, h] / np.sqrt(hd)
            a = np.exp(s - s.max())
            a /= a.sum()
            o[b, h] = a @ vv
    return o


# ----------------------------------------------------------------------------- layer / stack

def decode_layer(shape, layer: dict, x: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, pos) -> dict:
    """One decoder layer at decode (Primer 1.1 block, Primer 1.2 decode step).

    x: [B][D]; caches: bf16 bits [B][Hkv][cap][hd] (not modified; updated copies
    are returned).  Returns the layer output z and every intermediate."""
    x = np.asarray(x, dtype=np.float64)
    B = x.shape[0]
    Hq, Hkv, hd = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    pos = np.broadcast_to(np.asarray(pos, dtype=np.int64), (B,))

    h = rmsnorm(x, layer["attn_norm"], shape.rms_eps)
    q = matvec(layer["wq"], h).reshape(B, Hq, hd)
    k = matvec(layer["wk"], h).reshape(B, Hkv, hd)
    v = matvec(layer["wv"], h).reshape(B, Hkv, hd)
    q_rot = np.stack([rope(q[b], int(pos[b]), shape.rope_base) for b in range(B)])
    k_rot = np.stack([rope(k[b], int(pos[b]), shape.rope_base) for b in range(B)])

    k_new = bf16_round_bits(k_rot)
    v_new = bf16_round_bits(v)
    kc = k_cache.copy()
    vc = v_cache.copy()
    for b in range(B):
        kc[b, :, pos[b], :] = k_new[b]
        vc[b, :, pos[b], :] = v_new[b]

    o = gqa_decode_attention(q_rot, kc, vc, pos).reshape(B, Hq * hd)
    y = x + matvec(layer["wo"], o)
    h2 = rmsnorm(y, layer["ffn_norm"], shape.rms_eps)
    gate = matvec(layer["wg"], h2)
    up = matvec(layer["wu"], h2)
    act = swiglu(gate, up)
    z = y + matvec(layer["wd"], act)
    return {"z": z, "h": h, "q_rot": q_rot, "k_rot": k_rot, "v": v, "k_new": k_new, "v_new": v_new,
            "k_cache": kc, "v_cache": vc, "o": o, "y": y, "h2": h2, "gate": gate, "up": up, "act": act}


def decode_stack(shape, layers: list, x: np.ndarray, caches: list, pos) -> dict:
    """Layers applied in order, each feeding its output to the next (Primer 1.2)."""
    z = np.asarray(x, dtype=np.float64)
    new_caches = []
    for layer, (kc, vc) in zip(layers, caches):
        r = decode_layer(shape, layer, z, kc, vc, pos)
        z = r["z"]
        new_caches.append((r["k_cache"], r["v_cache"]))
    return {"z": z, "caches": new_caches}


def prefill(shape, layers: list, x: np.ndarray, caches: list, pos0: int) -> dict:
    """Prefill of a prompt by its definition (Primer 1.2, prefill vs decode):
    every prompt token gets what decoding it at position pos0 + t, after the
    tokens before it, gives.  x [T][D]; caches hold the sequence's earlier
    tokens below pos0 (batch dimension 1).  Returns each token's output
    z [T][D] and the caches with the T prompt tokens' K/V appended."""
    x = np.asarray(x, dtype=np.float64)
    zs = []
    for t in range(x.shape[0]):
        r = decode_stack(shape, layers, x[t:t + 1], caches, [pos0 + t])
        caches = r["caches"]
        zs.append(r["z"][0])
    return {"z": np.stack(zs), "caches": caches}


# ----------------------------------------------------------------------------- LM head

def lm_head_argmax(w_lm: dict, h: np.ndarray):
    """Full logits W_lm h, greedy token = lowest id attaining the maximum
    (Primer 1.2: logits over the vocabulary, then sampling; greedy here).
    Returns (tokens int64 [B], max logit [B], logits [B][V])."""
    logits = matvec(w_lm, h)
    tok = np.argmax(logits, axis=1)          # first maximum = lowest id
    return tok, logits[np.arange(logits.shape[0]), tok], logits


def lm_head_chunked_argmax(w_lm: dict, h: np.ndarray, chunk_rows: int):
    """Same result computed chunk by chunk with a running greedy argmax, never
    holding more than one chunk of logits (Unsloth article 三: chunked logits).
    A later chunk replaces the running best only on a strictly larger logit."""
    h = np.asarray(h, dtype=np.float64)
    B = h.shape[0]
    best = np.full(B, -np.inf)
    tok = np.zeros(B, dtype=np.int64)
    for r0 in range(0, w_lm["n"], chunk_rows):
        r1 = min(w_lm["n"], r0 + chunk_rows)
        lg = h @ _dense(w_lm, r0, r1).T
        i = np.argmax(lg, axis=1)
        m = lg[np.arange(B), i]
        upd = m > best
        best = np.where(upd, m, best)
        tok = np.where(upd, r0 + i, tok)
    return tok, best


# ----------------------------------------------------------------------------- the decode loop

def embed_tokens(table_bits: np.ndarray, tokens) -> np.ndarray:
    """Hidden state of each sequence's last token: row tokens[b] of the bf16
    embedding table [V][D] (Primer 1.2: each decode step starts from the
    embedding of the token generated last).  Ids outside the table raise."""
    tokens = np.asarray(tokens, dtype=np.int64)
    if np.any(tokens < 0) or np.any(tokens >= table_bits.shape[0]):
        raise IndexError("token id outside the embedding table")
    return bf16_to_f64(table_bits[tokens])


def greedy_decode(shape, layers: list, table_bits: np.ndarray, w_lm: dict, tokens, caches: list, pos, steps: int,
                  temperature=None, seed: int = 0, top_k: int = 0) -> dict:
    """`steps` rounds of Primer 1.2's decode loop: embed the last token, run
    the stack (appending each layer's K/V at pos), take the LM head's token,
    advance every position by one.  The token is the greedy one, or with a
    temperature the Gumbel-max draw of oracle.sample with each sequence's
    position as its counter word ("max_logit" then holds the winning perturbed
    score and "logits" the perturbed scores); with top_k > 0 as well, the draw
    is restricted to the top_k largest logits (oracle.sample_tokens_topk; the
    scores of the other rows are -inf, and "raw" holds the step's logits).
    Returns per-step tokens, maximum scores and scores, the final hidden state
    and the caches."""
    from .sample import sample_tokens, sample_tokens_topk
    tok = np.asarray(tokens, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    out = {"tokens": [], "max_logit": [], "logits": []}
    for _ in range(steps):
        r = decode_stack(shape, layers, embed_tokens(table_bits, tok), caches, pos)
        caches = r["caches"]
        tok, mx, logits = lm_head_argmax(w_lm, r["z"])
        out.setdefault("raw", []).append(logits)
        if temperature is not None and top_k > 0:
            tok, mx, logits = sample_tokens_topk(logits, temperature, top_k, seed, pos)
        elif temperature is not None:
            tok, mx, logits = sample_tokens(logits, temperature, seed, pos)
        out["tokens"].append(tok.copy())
        out["max_logit"].append(mx)
        out["logits"].append(logits)
        out["z"] = r["z"]
        pos = pos + 1
    out["caches"] = caches
    return out

