"""float64 reference of temperature sampling from the LM head's logits.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Primer 1.2 ends each decode step by sampling a token from the vocabulary
logits and does not say how.  The greedy argmax is one reading. This module is
the other plain one: a draw from softmax(logits / T).  It is computed by the
Gumbel-max method (E. J. Gumbel, 1954, as used for sampling by Maddison,
Tarlow and Minka, "A* sampling", 2014): add independent standard Gumbel noise
g_v = -log(-log(u_v)) to every logit / T and take the argmax.  The argmax is
then distributed exactly as softmax(logits / T).  So the chunked running
argmax of the LM head serves sampling unchanged: no logit needs to be kept.

The uniforms u_v come from the counter-based generator Philox4x32-10 (Salmon,
Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11),
so that any row of any chunk can draw its own number with no state:
  * counter (v, b, c_b, 0): row v, sequence b, and c_b, a per-sequence counter
    word the caller supplies (the decode loop passes the token's position);
  * key (seed mod 2^32, seed >> 32);
  * the first output word x gives u = (floor(x / 512) + 1/2) / 2^23, which
    lies strictly inside (0, 1) and is exact in float32 as well (24 bits).

Top-k sampling (the "optional temperature/top-k" of the decode loop's
sample step): the draw from softmax(logits / T) restricted to the k largest
logits (equal logits ranked by lower id), renormalised over them.  With the
same Gumbel noise it is the argmax of the perturbed scores over those k rows
only, so k = V is plain temperature sampling and k = 1 the greedy token.

Parity pins (tests/test_oracle_pins.py): the published Philox4x32-10
known-answer vectors; the empirical frequencies of many draws against
softmax(logits / T), and against the renormalised softmax over the top k; a
vanishing temperature, and k = 1, giving the greedy token; k = V giving the
plain draw; equal logits at the cut kept by lower id.
"""

import numpy as np

_M0, _M1 = 0xD2511F53, 0xCD9E8D57          # Philox4x32 round multipliers
_W0, _W1 = 0x9E3779B9, 0xBB67AE85          # key schedule (Weyl) increments
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds (SC'11 paper, section 4.2), vectorised over
    numpy arrays of 32-bit words.  Each round multiplies words 0 and 2 by the
    round multipliers, mixes the high halves with words 1 and 3 and the round
    key, and permutes; the key is bumped by the Weyl increments between rounds.
    Returns the four output words as uint64 arrays holding 32-bit values."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK for x in (c0, c1, c2, c3)]
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(_W0)) & _MASK
            k1 = (k1 + np.uint64(_W1)) & _MASK
        p0 = np.uint64(_M0) * c[0]                # exact: 32 x 32 -> 64 bits
        p1 = np.uint64(_M1) * c[2]
        c = [((p1 >> np.uint64(32)) ^ c[1] ^ k0) & _MASK, p1 & _MASK,
             ((p0 >> np.uint64(32)) ^ c[3] ^ k1) & _MASK, p0 & _MASK]
    return c


def uniforms(n_rows: int, b: int, counter: int, seed: int) -> np.ndarray:
    """u_v for v = 0..n_rows-1 of sequence b (float64, strictly inside (0, 1))."""
    v = np.arange(n_rows, dtype=np.uint64)
    x = philox4x32_10(v, b, counter & 0xFFFFFFFF, 0, seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)[0]
    return ((x >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def gumbel_scores(logits: np.ndarray, temperature: float, seed: int, counters) -> np.ndarray:
    """logit_v / T + g_v for every sequence b (logits [B][V], float64)."""
    logits = np.asarray(logits, dtype=np.float64)
    out = np.empty_like(logits)
    for b in range(logits.shape[0]):
        u = uniforms(logits.shape[1], b, int(counters[b]), seed)
        out[b] = logits[b] / temperature - np.log(-np.log(u))
    return out


def sample_tokens(logits: np.ndarray, temperature: float, seed: int, counters):
    """Token = lowest id attaining the largest perturbed score.  Returns
    (tokens int64 [B], that score [B], the scores [B][V])."""
    if not (temperature > 0.0 and np.isfinite(temperature)):
        raise ValueError("temperature must be positive and finite")
    s = gumbel_scores(logits, temperature, seed, counters)
    tok = np.argmax(s, axis=1)
    return tok, s[np.arange(s.shape[0]), tok], s


def top_k_rows(logits_row: np.ndarray, top_k: int) -> np.ndarray:
    """Ids of the top_k largest logits of one row, larger logit first, equal
    logits by lower id."""
    v = np.asarray(logits_row, dtype=np.float64)
    order = np.lexsort((np.arange(v.size), -v))
    return order[:top_k]


def sample_tokens_topk(logits: np.ndarray, temperature: float, top_k: int, seed: int, counters):
    """Top-k sampling: token = lowest id attaining the largest perturbed score
    logit_v / T + g_v among the top_k rows of each sequence (same noise as
    sample_tokens).  Returns (tokens [B], that score [B], the scores [B][V]
    with rows outside the top k set to -inf)."""
    logits = np.asarray(logits, dtype=np.float64)
    if not 1 <= top_k <= logits.shape[1]:
        raise ValueError("top_k must lie in 1..V")
    _, _, s = sample_tokens(logits, temperature, seed, counters)
    masked = np.full_like(s, -np.inf)
    for b in range(s.shape[0]):
        keep = top_k_rows(logits[b], top_k)
        masked[b, keep] = s[b, keep]
    tok = np.argmax(masked, axis=1)
    return tok, masked[np.arange(s.shape[0]), tok], masked
