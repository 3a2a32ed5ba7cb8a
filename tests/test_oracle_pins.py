"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a worked
fixture under tests/golden/, a closed form, an invariant, brute force on tiny
inputs, or a library routine (scipy) computing the same quantity by a different
route.  They are chosen so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them.
"""

import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ int4 format

def test_unpack_matches_golden_bytes():
    g = _golden("int4_format.json")
    codes = np.array(g["bytes"], dtype=np.uint8)[None, :]
    got = oracle.unpack_int4(codes, 2 * len(g["bytes"]))[0]
    assert got.tolist() == g["codes"]


def test_dequant_matches_golden_values():
    g = _golden("int4_format.json")
    codes = np.array(g["bytes"], dtype=np.uint8)[None, :]
    k = 2 * len(g["bytes"])
    scales = np.array([[int(g["scale_bits_hex"], 16)]], dtype=np.uint16)
    w = oracle.dequant_int4(codes, scales, k, group=k)
    assert w[0].tolist() == g["dequant"]


def test_unpack_is_a_bijection_over_all_bytes():
    allb = np.arange(256, dtype=np.uint8)[None, :]
    c = oracle.unpack_int4(allb, 512)[0]
    lo, hi = c[0::2], c[1::2]
    assert np.all((lo >= 0) & (lo <= 15) & (hi >= 0) & (hi <= 15))
    assert np.array_equal(lo + 16 * hi, np.arange(256))


def test_dequant_group_index_with_ragged_last_group():
    # K=6, group=4: inputs 0..3 use scale 0, inputs 4..5 use scale 1
    codes = np.array([[0x99, 0x99, 0x99]], dtype=np.uint8)  # all codes 9 -> (9-8) = 1
    scales = synth.bf16_bits(np.array([[0.5, 2.0]], dtype=np.float32))
    w = oracle.dequant_int4(codes, scales, 6, 4)
    assert w[0].tolist() == [0.5, 0.5, 0.5, 0.5, 2.0, 2.0]


def test_quantiser_round_trip_error_bound():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((7, 688)) * 0.02).astype(np.float32)
    w[3, 64:128] = 0.0                         # an all-zero group
    codes, scales = synth.quantize_int4(w, 64)
    deq = oracle.dequant_int4(codes, scales, 688, 64)
    s = oracle.bf16_to_f64(scales)[:, np.arange(688) // 64]
    assert np.all(np.abs(deq - w) <= s / 2 + 1e-12)
    assert np.all(deq[3, 64:128] == 0.0)
    c = oracle.unpack_int4(codes, 688)
    assert np.all(np.abs(c - 8) <= 7)


def test_matvec_against_per_element_brute_force():
    rng = np.random.default_rng(2)
    n, k, g = 5, 24, 8
    codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = synth.bf16_bits(rng.uniform(0.001, 0.02, size=(n, k // g)).astype(np.float32))
    h = rng.standard_normal((2, k))
    mat = {"codes": codes, "scales": scales, "n": n, "k": k, "group": g}
    got = oracle.matvec(mat, h)
    for b in range(2):
        for r in range(n):
            acc = 0.0
            for i in range(k):
                byte = int(codes[r, i // 2])
                c = (byte >> 4) if i % 2 else (byte & 15)
                sc = float(synth.bf16_value(scales[r, i // g]))
                acc += (c - 8) * sc * h[b, i]
            assert abs(got[b, r] - acc) <= 1e-12 * max(1.0, abs(acc))


# ------------------------------------------------------------------ bf16 rounding

@pytest.mark.parametrize("val,bits", [
    (1.0, 0x3F80), (-2.5, 0xC020), (1.0 + 2.0 ** -8, 0x3F80),          # tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),                                       # tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),                              # just above the tie
    (0.0078125, 0x3C00), (3.0e-3, 0x3B45),
])
def test_bf16_round_bits_known_values(val, bits):
    assert int(oracle.bf16_round_bits(np.array([val]))[0]) == bits
    assert oracle.bf16_to_f64(np.array([bits], dtype=np.uint16))[0] == pytest.approx(val, rel=2 ** -8)


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_hand_example():
    g = synth.bf16_bits(np.array([1.0, 1.0], dtype=np.float32))
    out = oracle.rmsnorm(np.array([3.0, 4.0]), g, 0.0)
    r = np.sqrt(12.5)
    assert np.allclose(out, [3.0 / r, 4.0 / r], rtol=1e-15)


def test_rmsnorm_output_rms_equals_gain_closed_form():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(5120) * 0.37
    c = 1.5
    g = synth.bf16_bits(np.full(5120, c, dtype=np.float32))
    eps = 1e-6
    out = oracle.rmsnorm(x, g, eps)
    ms = np.mean(x * x)
    assert np.sqrt(np.mean(out * out)) == pytest.approx(c * np.sqrt(ms / (ms + eps)), rel=1e-13)


def test_rmsnorm_scale_invariance_and_gain_is_elementwise():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(64)
    gains = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    g = synth.bf16_bits(gains)
    a = oracle.rmsnorm(x, g, 0.0)
    b = oracle.rmsnorm(7.25 * x, g, 0.0)
    assert np.allclose(a, b, rtol=1e-13)
    one = synth.bf16_bits(np.ones(64, dtype=np.float32))
    assert np.allclose(a, oracle.rmsnorm(x, one, 0.0) * synth.bf16_value(g), rtol=1e-13)


# ------------------------------------------------------------------ RoPE

def test_rope_position_zero_is_identity():
    t = np.random.default_rng(5).standard_normal((3, 128))
    assert np.array_equal(oracle.rope(t, 0, 1e6), t)


def test_rope_hd2_is_plain_rotation_by_pos_radians():
    # hd = 2: one pair, theta_0 = base^0 = 1, angle = pos
    for p in (1, 5, 127):
        out = oracle.rope(np.array([1.0, 0.0]), p, 1e4)
        assert np.allclose(out, [np.cos(p), np.sin(p)], atol=1e-15)


def test_rope_half_split_pairing_and_frequencies():
    # hd = 4, base 100: theta = [1, 100^-0.5 = 0.1]; pairs are (0,2) and (1,3)
    p = 3
    out = oracle.rope(np.array([1.0, 0.0, 0.0, 0.0]), p, 100.0)
    assert np.allclose(out, [np.cos(3.0), 0.0, np.sin(3.0), 0.0], atol=1e-15)
    out = oracle.rope(np.array([0.0, 1.0, 0.0, 0.0]), p, 100.0)
    assert np.allclose(out, [0.0, np.cos(0.3), 0.0, np.sin(0.3)], atol=1e-15)
    assert oracle.rope_angles(1, 64, 1e4)[1] == pytest.approx(1e4 ** (-2.0 / 64), rel=1e-15)


def test_rope_preserves_pair_norms():
    t = np.random.default_rng(6).standard_normal(128)
    out = oracle.rope(t, 8192, 1e6)
    assert np.allclose(t[:64] ** 2 + t[64:] ** 2, out[:64] ** 2 + out[64:] ** 2, rtol=1e-12)


def test_rope_dot_product_depends_only_on_relative_position():
    rng = np.random.default_rng(7)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for m, n, d in [(10, 3, 100), (4096, 4000, 777), (0, 5, 8192)]:
        a = oracle.rope(q, m, 1e6) @ oracle.rope(k, n, 1e6)
        b = oracle.rope(q, m + d, 1e6) @ oracle.rope(k, n + d, 1e6)
        assert a == pytest.approx(b, rel=1e-9, abs=1e-9)


# ------------------------------------------------------------------ attention

def _bits(a):
    return oracle.bf16_round_bits(a)


def test_attention_single_key_returns_its_value():
    rng = np.random.default_rng(8)
    kc = _bits(rng.standard_normal((1, 1, 4, 8)))
    vc = _bits(rng.standard_normal((1, 1, 4, 8)))
    q = rng.standard_normal((1, 3, 8))
    o = oracle.gqa_decode_attention(q, kc, vc, [0])
    assert np.allclose(o[0], np.tile(oracle.bf16_to_f64(vc[0, 0, 0]), (3, 1)), rtol=1e-15)


def test_attention_equal_keys_give_mean_value():
    rng = np.random.default_rng(9)
    kc = np.tile(_bits(rng.standard_normal(16)), (1, 2, 10, 1))
    vc = _bits(rng.standard_normal((1, 2, 10, 16)))
    q = rng.standard_normal((1, 4, 16))
    o = oracle.gqa_decode_attention(q, kc, vc, [6])
    for h in range(4):
        assert np.allclose(o[0, h], oracle.bf16_to_f64(vc[0, h // 2, :7]).mean(axis=0), rtol=1e-13)


def test_attention_two_key_closed_form():
    # hd = 2, q = (a, 0), k0 = 0, k1 = (c, 0): weight of key 1 = sigmoid(a c / sqrt 2)
    a, c = 1.75, 0.5
    kc = _bits(np.array([[[[0.0, 0.0], [c, 0.0]]]]))
    v0, v1 = np.array([1.0, -2.0]), np.array([0.25, 3.0])
    vc = _bits(np.array([[[v0, v1]]]))
    o = oracle.gqa_decode_attention(np.array([[[a, 0.0]]]), kc, vc, [1])
    w1 = expit(a * c / np.sqrt(2.0))
    assert np.allclose(o[0, 0], (1 - w1) * v0 + w1 * v1, rtol=1e-14)


def test_gqa_equals_mha_on_replicated_kv_and_ignores_poisoned_slots():
    rng = np.random.default_rng(10)
    B, Hq, Hkv, cap, hd = 2, 8, 2, 12, 16
    pos = [5, 9]
    kc = _bits(rng.standard_normal((B, Hkv, cap, hd)))
    vc = _bits(rng.standard_normal((B, Hkv, cap, hd)))
    for b in range(B):                         # poison slots beyond each position
        kc[b, :, pos[b] + 1:] = 0x7FC0
        vc[b, :, pos[b] + 1:] = 0x7FC0
    q = rng.standard_normal((B, Hq, hd))
    got = oracle.gqa_decode_attention(q, kc, vc, pos)
    # multi-head attention over KV heads repeated G times (an explicit copy), scipy softmax
    G = Hq // Hkv
    K = np.repeat(oracle.bf16_to_f64(kc), G, axis=1)
    V = np.repeat(oracle.bf16_to_f64(vc), G, axis=1)
    for b in range(B):
        for h in range(Hq):
            n = pos[b] + 1
            w = softmax(K[b, h, :n] @ q[b, h] / np.sqrt(hd))
            assert np.allclose(got[b, h], w @ V[b, h, :n], rtol=1e-12, atol=1e-14)
    assert np.all(np.isfinite(got))


# ------------------------------------------------------------------ SwiGLU

def test_silu_and_swiglu_closed_forms():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert oracle.silu(np.array([1.0]))[0] == pytest.approx(0.7310585786300049, rel=1e-15)
    assert oracle.silu(np.array([40.0]))[0] == pytest.approx(40.0, rel=1e-15)
    assert abs(oracle.silu(np.array([-40.0]))[0]) < 1e-15
    g = np.linspace(-6, 6, 25)
    u = np.linspace(2, -3, 25)
    assert np.allclose(oracle.swiglu(g, u), g * expit(g) * u, rtol=1e-14)


# ------------------------------------------------------------------ whole layer: decode step == last row of the sequence form

def _sequence_layer(shape, layer, X):
    """Independent sequence form of one decoder layer over S positions with an
    explicit causal mask and KV heads broadcast by copying (the form the
    Unsloth article 二.2 calls the naive one).  K and V pass through bf16 as in a
    cache.  Returns outputs [S][D] and the bf16 caches [Hkv][S][hd]."""
    S, D = X.shape
    Hq, Hkv, hd = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    G = Hq // Hkv

    def W(name):
        m = layer[name]
        return oracle.dequant_int4(m["codes"], m["scales"], m["k"], m["group"])

    def norm(A, gname):
        gain = synth.bf16_value(layer[gname]).astype(np.float64)
        return np.stack([a * gain / np.sqrt(np.dot(a, a) / a.size + shape.rms_eps) for a in A])

    H = norm(X, "attn_norm")
    Q, Kp, Vp = H @ W("wq").T, H @ W("wk").T, H @ W("wv").T
    half = hd // 2
    inv = shape.rope_base ** (-np.arange(half) * 2.0 / hd)

    def rot(v, p):
        out = v.copy()
        for i in range(half):
            ang = p * inv[i]
            x0, x1 = v[i], v[i + half]
            out[i] = x0 * np.cos(ang) - x1 * np.sin(ang)
            out[i + half] = x0 * np.sin(ang) + x1 * np.cos(ang)
        return out

    Qh = np.stack([[rot(Q[p, h * hd:(h + 1) * hd], p) for h in range(Hq)] for p in range(S)])
    Kh = np.stack([[rot(Kp[p, j * hd:(j + 1) * hd], p) for j in range(Hkv)] for p in range(S)])
    Vh = np.stack([[Vp[p, j * hd:(j + 1) * hd] for j in range(Hkv)] for p in range(S)])
    Kb = oracle.bf16_to_f64(oracle.bf16_round_bits(Kh))
    Vb = oracle.bf16_to_f64(oracle.bf16_round_bits(Vh))
    Kr = np.repeat(Kb, G, axis=1)           # [S][Hq][hd] broadcast copy
    Vr = np.repeat(Vb, G, axis=1)
    mask = np.triu(np.full((S, S), -np.inf), 1)
    attn = np.zeros((S, Hq * hd))
    for h in range(Hq):
        sc = Qh[:, h, :] @ Kr[:, h, :].T / np.sqrt(hd) + mask
        attn[:, h * hd:(h + 1) * hd] = softmax(sc, axis=1) @ Vr[:, h, :]
    Y = X + attn @ W("wo").T
    H2 = norm(Y, "ffn_norm")
    gate, up = H2 @ W("wg").T, H2 @ W("wu").T
    Z = Y + (gate * expit(gate) * up) @ W("wd").T
    kc = oracle.bf16_round_bits(Kh).transpose(1, 0, 2)
    vc = oracle.bf16_round_bits(Vh).transpose(1, 0, 2)
    return Z, kc, vc


def test_decode_layer_equals_last_row_of_sequence_form():
    shape = synth.SHAPES["tiny"].with_(d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16, d_ff=96, group=16)
    layer = synth.make_layer(shape, seed=11, layer=0)
    S = 9
    X = np.random.default_rng(12).standard_normal((S, shape.d_model))
    Z, kc, vc = _sequence_layer(shape, layer, X)
    cap = 12
    kcache = np.full((1, shape.n_kv_heads, cap, shape.head_dim), 0x7FC0, dtype=np.uint16)
    vcache = kcache.copy()
    kcache[0, :, : S - 1] = kc[:, : S - 1]
    vcache[0, :, : S - 1] = vc[:, : S - 1]
    r = oracle.decode_layer(shape, layer, X[S - 1][None, :], kcache, vcache, [S - 1])
    assert np.allclose(r["z"][0], Z[S - 1], rtol=1e-12, atol=1e-12)
    # the step appended exactly slot S-1 and left every other slot untouched
    assert np.array_equal(r["k_cache"][0, :, S - 1], kc[:, S - 1])
    assert np.array_equal(r["v_cache"][0, :, S - 1], vc[:, S - 1])
    assert np.array_equal(r["k_cache"][0, :, : S - 1], kcache[0, :, : S - 1])
    assert np.array_equal(r["k_cache"][0, :, S:], kcache[0, :, S:])


def test_decode_stack_is_layer_composition():
    shape = synth.SHAPES["tiny"].with_(d_model=32, n_q_heads=2, n_kv_heads=1, head_dim=16, d_ff=48, group=16, n_layers=2)
    layers = [synth.make_layer(shape, 13, l) for l in range(2)]
    caches = [synth.make_kv(shape, 13, l, 1, 4, 8) for l in range(2)]
    x = synth.make_x(shape, 13, 1)
    r = oracle.decode_stack(shape, layers, x, caches, [4])
    z = x
    for l in range(2):
        z = oracle.decode_layer(shape, layers[l], z, caches[l][0], caches[l][1], [4])["z"]
    assert np.array_equal(r["z"], z)


def test_prefill_equals_sequence_form_on_every_row():
    """The oracle's prefill (token after token) against the causal-mask
    sequence form over the whole prompt: every row, and every appended slot."""
    shape = synth.SHAPES["tiny"].with_(d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16, d_ff=96, group=16)
    layer = synth.make_layer(shape, seed=21, layer=0)
    S, cap = 11, 16
    X = np.random.default_rng(22).standard_normal((S, shape.d_model))
    Z, kc, vc = _sequence_layer(shape, layer, X)
    poison = np.full((1, shape.n_kv_heads, cap, shape.head_dim), 0x7FC0, dtype=np.uint16)
    r = oracle.prefill(shape, [layer], X, [(poison, poison.copy())], 0)
    assert np.allclose(r["z"], Z, rtol=1e-12, atol=1e-12)
    k_out, v_out = r["caches"][0]
    assert np.array_equal(k_out[0, :, :S], kc) and np.array_equal(v_out[0, :, :S], vc)
    assert np.array_equal(k_out[0, :, S:], poison[0, :, S:])


def test_prefill_after_a_history_equals_the_tail_of_one_long_prefill():
    """A prompt split in two (the second part after the first's cache) gives
    the same rows as one prefill over the whole prompt."""
    shape = synth.SHAPES["tiny"].with_(d_model=32, n_q_heads=2, n_kv_heads=1, head_dim=16, d_ff=48, group=16, n_layers=2)
    layers = [synth.make_layer(shape, 23, l) for l in range(2)]
    cap = 16
    empty = [(np.zeros((1, 1, cap, 16), dtype=np.uint16), np.zeros((1, 1, cap, 16), dtype=np.uint16)) for _ in range(2)]
    X = np.random.default_rng(24).standard_normal((9, shape.d_model))
    whole = oracle.prefill(shape, layers, X, empty, 0)
    head = oracle.prefill(shape, layers, X[:4], empty, 0)
    tail = oracle.prefill(shape, layers, X[4:], head["caches"], 4)
    assert np.array_equal(tail["z"], whole["z"][4:])
    for l in range(2):
        for i in range(2):
            assert np.array_equal(tail["caches"][l][i], whole["caches"][l][i])


# ------------------------------------------------------------------ LM head

def _tiny_lm(V, D, g, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((V, D)) * 0.02).astype(np.float32)
    codes, scales = synth.quantize_int4(w, g)
    return {"codes": codes, "scales": scales, "n": V, "k": D, "group": g}


@pytest.mark.parametrize("chunk", [1, 3, 7, 16, 37, 64, 100])
def test_chunked_argmax_equals_full_argmax(chunk):
    lm = _tiny_lm(37, 32, 16, 14)
    h = np.random.default_rng(15).standard_normal((3, 32))
    tok, mx, logits = oracle.lm_head_argmax(lm, h)
    t2, m2 = oracle.lm_head_chunked_argmax(lm, h, chunk)
    assert np.array_equal(tok, t2)
    assert np.allclose(mx, m2, rtol=1e-13)   # BLAS may sum in another order per chunk shape
    # brute force
    W = oracle.dequant_int4(lm["codes"], lm["scales"], 32, 16)
    for b in range(3):
        vals = [sum(W[v, i] * h[b, i] for i in range(32)) for v in range(37)]
        best = max(range(37), key=lambda v: (vals[v], -v))
        assert tok[b] == best


def test_argmax_ties_go_to_lowest_id_across_chunks():
    lm = _tiny_lm(20, 16, 16, 16)
    lm["codes"][17] = lm["codes"][4]          # rows 4 and 17 identical
    lm["scales"][17] = lm["scales"][4]
    lm["codes"][4] = np.uint8(0xFF)           # make row 4 large: all codes 15
    lm["codes"][17] = np.uint8(0xFF)
    lm["scales"][4] = lm["scales"][17] = synth.bf16_bits(np.array([0.05], dtype=np.float32))[0]
    h = np.ones((1, 16))
    for chunk in (1, 5, 8, 20):
        t, _ = oracle.lm_head_chunked_argmax(lm, h, chunk)
        assert t[0] == 4
    assert oracle.lm_head_argmax(lm, h)[0][0] == 4


# ------------------------------------------------------------------ the decode loop (Primer 1.2)

def test_embed_tokens_reads_table_rows():
    V, D = 9, 12
    # row v, column d holds (v - 3) / 4 + d / 64: dyadic values, exact in bf16
    vals = np.array([[(v - 3) / 4 + d / 64 for d in range(D)] for v in range(V)], dtype=np.float32)
    table = synth.bf16_bits(vals)
    x = oracle.embed_tokens(table, [5, 0, 8, 5])
    assert x.dtype == np.float64 and x.shape == (4, D)
    for i, v in enumerate([5, 0, 8, 5]):
        assert np.array_equal(x[i], [(v - 3) / 4 + d / 64 for d in range(D)])
    with pytest.raises(IndexError):
        oracle.embed_tokens(table, [9])
    with pytest.raises(IndexError):
        oracle.embed_tokens(table, [-1])


def _identity_layer(shape, g):
    """Every code 8 (weight 0 whatever the scale): attention and FFN add
    nothing, so a layer returns its input unchanged."""
    D, qw, kvw, F = shape.d_model, shape.q_width, shape.kv_width, shape.d_ff
    dims = {"wq": (qw, D), "wk": (kvw, D), "wv": (kvw, D), "wo": (D, qw), "wg": (F, D), "wu": (F, D), "wd": (D, F)}
    one = synth.bf16_bits(np.ones(D, dtype=np.float32))
    layer = {"attn_norm": one, "ffn_norm": one}
    for n, (r, c) in dims.items():
        layer[n] = {"codes": np.full((r, c // 2), 0x88, dtype=np.uint8),
                    "scales": synth.bf16_bits(np.full((r, (c + g - 1) // g), 0.01, dtype=np.float32)),
                    "n": r, "k": c, "group": g}
    return layer


def test_greedy_decode_follows_a_cyclic_successor_model():
    """Closed form: with identity layers, one-hot embeddings e_v and an LM
    head whose row u is 7 * 0.125 * e_{u-1}, the logits of x = e_v peak at
    u = v + 1 (mod V), so greedy decoding from t yields t+1, t+2, ...; the
    appended K/V slots are zeros (k = v = 0) and the positions advance."""
    shape = synth.SHAPES["tiny"].with_(d_model=32, n_q_heads=2, n_kv_heads=1, head_dim=16, d_ff=32, group=16, n_layers=2)
    V, D, g = 20, 32, 16
    table = synth.bf16_bits(np.eye(V, D, dtype=np.float32))
    codes = np.full((V, D), 8, dtype=np.uint8)
    for u in range(V):
        codes[u, (u - 1) % V] = 15                        # (15 - 8) * 0.125 = 0.875
    lm = {"codes": (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8),
          "scales": synth.bf16_bits(np.full((V, D // g), 0.125, dtype=np.float32)), "n": V, "k": D, "group": g}
    layers = [_identity_layer(shape, g) for _ in range(2)]
    caches = [synth.make_kv(shape, 21, l, 2, [5, 9], 16) for l in range(2)]
    r = oracle.greedy_decode(shape, layers, table, lm, [3, 19], caches, [5, 9], 4)
    assert [list(t) for t in r["tokens"]] == [[4, 0], [5, 1], [6, 2], [7, 3]]
    assert np.allclose(r["max_logit"], 0.875)
    assert np.array_equal(r["z"], oracle.embed_tokens(table, [6, 2]))   # last step's input passes through
    for l in range(2):
        kc, vc = r["caches"][l]
        for b, p0 in enumerate([5, 9]):
            for s in range(4):                          # slots p0 .. p0+3 hold zeros (RoPE may give -0.0)
                assert np.all(synth.bf16_value(kc[b, :, p0 + s]) == 0) and np.all(synth.bf16_value(vc[b, :, p0 + s]) == 0)


# ----------------------------------------------------------------------------- temperature sampling

def test_philox_matches_the_published_known_answers():
    """oracle.sample's generator reproduces the Philox4x32-10 known-answer
    vectors published with the generator (tests/golden/philox4x32_10_kat.json)."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for v in kat["vectors"]:
        c = [int(x, 16) for x in v["ctr"]]
        k = [int(x, 16) for x in v["key"]]
        out = oracle.philox4x32_10(*c, *k)
        assert [int(o) for o in out] == [int(x, 16) for x in v["out"]]


def test_uniforms_lie_inside_the_unit_interval_and_are_uniform():
    u = oracle.uniforms(200_000, 3, 17, 0x1234_5678_9ABC_DEF0)
    assert u.min() > 0.0 and u.max() < 1.0
    n = u.size
    assert abs(u.mean() - 0.5) < 5 * np.sqrt(1 / 12 / n)
    counts = np.histogram(u, bins=20, range=(0.0, 1.0))[0]
    chi2 = np.sum((counts - n / 20) ** 2 / (n / 20))
    assert chi2 < 60.0                       # df 19: p < 1e-5 above this
    # the counter words and the key all change the stream
    assert not np.array_equal(u[:64], oracle.uniforms(64, 4, 17, 0x1234_5678_9ABC_DEF0))
    assert not np.array_equal(u[:64], oracle.uniforms(64, 3, 18, 0x1234_5678_9ABC_DEF0))
    assert not np.array_equal(u[:64], oracle.uniforms(64, 3, 17, 0x1234_5678_9ABC_DEF1))
    assert not np.array_equal(u[:64], oracle.uniforms(64, 3, 17, 0x1234_5679_9ABC_DEF0))


def test_gumbel_max_draws_follow_the_tempered_softmax():
    """Many independent draws (one per sequence index) land on each token with
    the probability softmax(logits / T): a wrong sign, a dropped temperature or
    a wrong noise law changes these frequencies."""
    logits = np.array([1.0, 0.5, 0.0, -1.0, 2.0, 0.2, -0.3])
    T, n = 0.7, 40_000
    p = softmax(logits / T)
    tok, score, s = oracle.sample_tokens(np.tile(logits, (n, 1)), T, 99, np.zeros(n, dtype=np.int64))
    assert np.array_equal(score, s[np.arange(n), tok])
    freq = np.bincount(tok, minlength=logits.size) / n
    sigma = np.sqrt(p * (1 - p) / n)
    assert np.all(np.abs(freq - p) < 5 * sigma), (freq, p)
    chi2 = np.sum((freq - p) ** 2 / p) * n
    assert chi2 < 35.0                       # df 6: p < 1e-5 above this
    # at T = 2 the same logits give a flatter law
    tok2 = oracle.sample_tokens(np.tile(logits, (n, 1)), 2.0, 5, np.zeros(n, dtype=np.int64))[0]
    p2 = softmax(logits / 2.0)
    freq2 = np.bincount(tok2, minlength=logits.size) / n
    assert np.all(np.abs(freq2 - p2) < 5 * np.sqrt(p2 * (1 - p2) / n))


def test_vanishing_temperature_gives_the_greedy_token():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((4, 1000))
    tok = oracle.sample_tokens(logits, 1e-9, 7, [0, 1, 2, 3])[0]
    assert np.array_equal(tok, np.argmax(logits, axis=1))
    with pytest.raises(ValueError):
        oracle.sample_tokens(logits, 0.0, 7, [0, 1, 2, 3])


# ----------------------------------------------------------------------------- top-k sampling

def test_topk_draws_follow_the_renormalised_softmax_over_the_top_k():
    """Frequencies of many top-k draws: softmax(logits / T) over the k largest
    logits, renormalised, and never a row outside them."""
    logits = np.array([1.0, 0.5, 0.0, -1.0, 2.0, 0.2, -0.3])
    T, n, k = 0.9, 40_000, 3
    keep = np.array([4, 0, 1])                            # 2.0, 1.0, 0.5
    p = np.zeros(logits.size)
    p[keep] = softmax(logits[keep] / T)
    tok = oracle.sample_tokens_topk(np.tile(logits, (n, 1)), T, k, 31, np.zeros(n, dtype=np.int64))[0]
    freq = np.bincount(tok, minlength=logits.size) / n
    assert np.all(freq[p == 0] == 0)
    sigma = np.sqrt(p[keep] * (1 - p[keep]) / n)
    assert np.all(np.abs(freq[keep] - p[keep]) < 5 * sigma), (freq, p)


def test_topk_one_is_greedy_and_topk_v_is_the_plain_draw():
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((5, 800))
    ctr = [3, 1, 4, 1, 5]
    t1 = oracle.sample_tokens_topk(logits, 1.7, 1, 11, ctr)[0]
    assert np.array_equal(t1, np.argmax(logits, axis=1))
    tv, sv, _ = oracle.sample_tokens_topk(logits, 1.7, 800, 11, ctr)
    t0, s0, _ = oracle.sample_tokens(logits, 1.7, 11, ctr)
    assert np.array_equal(tv, t0) and np.array_equal(sv, s0)
    with pytest.raises(ValueError):
        oracle.sample_tokens_topk(logits, 1.0, 0, 11, ctr)


def test_topk_cut_keeps_equal_logits_by_lower_id():
    v = np.array([0.5, 2.0, 1.0, 1.0, 1.0, -3.0])
    assert list(oracle.top_k_rows(v, 3)) == [1, 2, 3]
    assert list(oracle.top_k_rows(v, 1)) == [1]
    # a draw at k = 3 never lands on row 4 although its logit equals row 3's
    n = 5000
    tok = oracle.sample_tokens_topk(np.tile(v, (n, 1)), 1.0, 3, 2, np.zeros(n, dtype=np.int64))[0]
    assert set(np.unique(tok)) <= {1, 2, 3}
