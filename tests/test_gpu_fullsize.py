"""Parity at the full sizes of the timed workloads, through the C ABI.

Inputs come from the seeded device generator (the bench's own), are copied
to the host, and the CPU oracle recomputes the same step:
  * one 27B-shaped layer at 8192 cached tokens: int4 at batch 1 (matrix-vector
    path) and batch 16 (matrix-core path), bf16 weights at batch 1;
  * one 70B-shaped layer (D 8192, d_ff 28672, 32768 cached tokens, RoPE base
    5e5) at batch 1 and at batch 32 (matrix-core path, 32 positions);
  * two chained 27B-shaped int4 layers over two decode steps (the second step
    reads the K/V the first one appended);
  * the 152064 x 5120 int4 LM head (batch 1 and 16);
  * one 27B-shaped layer prefilled with a 512-token prompt (i4d_prefill, the
    launch configuration of bench.py --prefill 512): sampled tokens recomputed
    one by one, each against the cache the GPU built for the tokens before it.
Batches are independent sequences, so at batch 32 the oracle recomputes a
sample of the sequences (first, middle, last) while the GPU runs all of them.
Same bars as the other parity tests: float outputs relative L2 <= 1e-3 and
max |err| <= 5e-3 * RMS; the appended K/V slot within one bf16 rounding step
and every other slot bit-identical; token ids exact unless the oracle's top-2
gap is a near-tie.  Each case prints the oracle's seconds.
"""

import time

import numpy as np
import pytest
import torch

import oracle
import synth
from int4_weight_streaming_decode_amd import binding as B
from synth import gpu as G
from tests.gpu_util import assert_close, config_of, k_from_tiles, v_from_tiles, workspace

pytestmark = pytest.mark.gpu

MATS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def _print_case(*a):
    print("CASE", *a, flush=True)


def _host_mat(m):
    if "codes" in m:
        return {"codes": m["codes"].cpu().numpy(), "scales": m["scales"].cpu().numpy().view(np.uint16),
                "n": m["n"], "k": m["k"], "group": m["group"]}
    return {"bf16": m["bf16"].cpu().numpy().view(np.uint16), "n": m["n"], "k": m["k"]}


def _bits(t):
    return t.cpu().numpy().view(np.uint16)


class _FullLayer:
    """One layer's device tensors (seeded device generator), its ABI structs and
    the host copies the oracle reads."""

    def __init__(self, shape, seed, layer, wdtype, batch, cap):
        self.p = G.make_layer_gpu(shape, seed, layer, wdtype)
        mats = {}
        for n in MATS:
            m = self.p[n]
            if wdtype == "int4":
                mats[n] = B.make_mat(m["codes"], m["scales"], m["n"], m["k"], m["group"], B.WEIGHT_INT4)
            else:
                mats[n] = B.make_mat(m["bf16"], None, m["n"], m["k"], 0, B.WEIGHT_BF16)
        self.layer = B.make_layer(self.p["attn_norm"], self.p["ffn_norm"], mats)
        self.k, self.v = G.make_kv_gpu(shape, seed, layer, batch, cap)
        self.kv = B.make_kv(self.k, self.v, cap)
        self.kshape = (batch, shape.n_kv_heads, cap, shape.head_dim)
        self.host = {"attn_norm": _bits(self.p["attn_norm"]), "ffn_norm": _bits(self.p["ffn_norm"])}
        self.host.update({n: _host_mat(self.p[n]) for n in MATS})

    def caches(self, sel=None):
        kc = k_from_tiles(_bits(self.k), self.kshape)
        vc = v_from_tiles(_bits(self.v), self.kshape)
        if sel is not None:
            kc, vc = kc[sel], vc[sel]
        return kc, vc


def _check_slots(kg, vg, kref, vref, k0, v0, pos, what, untouched=None):
    """Appended slot within one bf16 rounding step (or the float bar); an
    untouched slot (default: the one before the appended slot) bit-identical to
    the cache before the call."""
    for b, pb in enumerate(pos):
        for name, g_, r_ in (("K", kg, kref), ("V", vg, vref)):
            gv = synth.bf16_value(g_[b, :, pb]).astype(np.float64)
            rv = synth.bf16_value(r_[b, :, pb]).astype(np.float64)
            ulp = np.ldexp(1.0, np.frexp(np.abs(rv))[1] - 8)
            rms = np.sqrt(np.mean(rv * rv))
            assert np.all(np.abs(gv - rv) <= np.maximum(5e-3 * rms, ulp)), f"{what}: {name} slot {pb} of b={b}"
        u = pb - 1 if untouched is None else untouched
        assert np.array_equal(kg[b, :, u], k0[b, :, u]) and np.array_equal(vg[b, :, u], v0[b, :, u]), f"{what}: slot {u}"


def _full_layer_case(shape, wdtype, batch, pos, sample=None):
    pos0 = max(pos)
    cap = ((pos0 + 1 + 15) // 16) * 16
    sel = list(range(batch)) if sample is None else sample
    _print_case(f"{shape.name} {wdtype} layer full size", "batch", batch, "pos", pos[:3], "oracle rows", sel)
    L = _FullLayer(shape, 5, 0, wdtype, batch, cap)
    x = G.make_x_gpu(shape, 6, batch)
    kc, vc = L.caches(sel)                        # the oracle's copies, before slot pos[b] is appended
    cfg = config_of(shape)
    ws = workspace(cfg, batch, pos0)
    out = torch.full((batch, shape.d_model), float("nan"), dtype=torch.float32, device="cuda")
    B.decode_layer(cfg, L.layer, batch, x, out, L.kv, torch.tensor(pos, dtype=torch.int32, device="cuda"), pos0, ws)
    torch.cuda.synchronize()
    assert B.read_device_status(ws) == 0
    psel = [pos[b] for b in sel]
    t0 = time.perf_counter()
    ref = oracle.decode_layer(shape, L.host, x.cpu().numpy()[sel].astype(np.float64), kc, vc, psel)
    print(f"oracle: {time.perf_counter() - t0:.1f} s for {len(sel)} sequence(s)", flush=True)
    got = out.cpu().numpy()[sel]
    for i, b in enumerate(sel):
        assert_close(got[i], ref["z"][i], what=f"{shape.name} {wdtype} layer b={b}")
    kg, vg = L.caches(sel)
    _check_slots(kg, vg, ref["k_cache"], ref["v_cache"], kc, vc, psel, f"{shape.name} {wdtype}")


@pytest.mark.parametrize("batch", [1, 16])
def test_27b_layer_at_full_size(batch):
    shape = synth.SHAPES["27b"]
    _full_layer_case(shape, "int4", batch, [shape.kv_len - 37 * b for b in range(batch)])


def test_27b_bf16_layer_at_full_size():
    shape = synth.SHAPES["27b"]
    _full_layer_case(shape, "bf16", 1, [shape.kv_len])


def test_70b_layer_at_full_size_batch1():
    shape = synth.SHAPES["70b"]
    _full_layer_case(shape, "int4", 1, [shape.kv_len])


def test_70b_layer_at_full_size_batch32():
    shape = synth.SHAPES["70b"]
    # 32 sequences at staggered positions up to 32768 cached tokens (matrix-core path)
    _full_layer_case(shape, "int4", 32, [shape.kv_len - 211 * b for b in range(32)], sample=[0, 13, 31])


def test_27b_two_layers_two_steps():
    """Two chained full-size layers, two decode steps: step 2 attends over the
    K/V that step 1 appended in both layers."""
    shape = synth.SHAPES["27b"]
    pos0 = shape.kv_len
    cap = ((pos0 + 2 + 15) // 16) * 16
    _print_case("27b two layers two steps", pos0)
    Ls = [_FullLayer(shape, 9, l, "int4", 1, cap) for l in range(2)]
    caches = [L.caches() for L in Ls]
    xs = [G.make_x_gpu(shape, 20 + s, 1) for s in range(2)]
    cfg = config_of(shape)
    ws = workspace(cfg, 1, pos0 + 1, n_layers=2)
    larr = [L.layer for L in Ls]
    karr = [L.kv for L in Ls]
    outs = []
    for s in range(2):
        out = torch.full((1, shape.d_model), float("nan"), dtype=torch.float32, device="cuda")
        B.decode_stack(cfg, larr, 1, xs[s], out, karr, torch.tensor([pos0 + s], dtype=torch.int32, device="cuda"),
                       pos0 + s, ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert B.read_device_status(ws) == 0
    t0 = time.perf_counter()
    ref_caches = caches
    for s in range(2):
        r = oracle.decode_stack(shape, [L.host for L in Ls], xs[s].cpu().numpy().astype(np.float64), ref_caches,
                                [pos0 + s])
        assert_close(outs[s].cpu().numpy()[0], r["z"][0], what=f"27b 2-layer stack step {s}")
        ref_caches = r["caches"]
    print(f"oracle: {time.perf_counter() - t0:.1f} s", flush=True)
    for l, L in enumerate(Ls):
        kg, vg = L.caches()
        kref, vref = ref_caches[l]
        k0, v0 = caches[l]
        for s in range(2):
            _check_slots(kg, vg, kref, vref, k0, v0, [pos0 + s], f"27b stack layer {l} step {s}", untouched=pos0 - 1)


@pytest.mark.parametrize("batch", [1, 16])
def test_lm_head_at_full_size(batch):
    shape = synth.SHAPES["27b_lm"]
    _print_case("lm head full size", shape.vocab, shape.d_model, batch)
    W = G.make_lm_head_gpu(shape.vocab, shape.d_model, shape.group, 2)
    mat = B.make_mat(W["codes"], W["scales"], W["n"], W["k"], W["group"], B.WEIGHT_INT4)
    h = G.make_x_gpu(shape, 8, batch)
    cfg = config_of(shape)
    ws = workspace(cfg, batch, 0, vocab=shape.vocab)
    tok = torch.full((batch,), -1, dtype=torch.int32, device="cuda")
    mx = torch.empty((batch,), dtype=torch.float32, device="cuda")
    B.lm_head_chunked(mat, batch, h, shape.lm_chunk, tok, mx, ws)
    torch.cuda.synchronize()
    tok_ref, mx_ref, logits = oracle.lm_head_argmax(_host_mat(W), h.cpu().numpy().astype(np.float64))
    t = tok.cpu().numpy()
    for b in range(batch):
        srt = np.sort(logits[b])
        rms = np.sqrt(np.mean(logits[b] ** 2))
        print(f"b={b}: token {t[b]} (oracle {tok_ref[b]}), top-2 gap {srt[-1] - srt[-2]:.3e}, RMS {rms:.3e}", flush=True)
        if srt[-1] - srt[-2] > 1e-3 * rms:
            assert t[b] == tok_ref[b]
        else:
            assert logits[b][t[b]] >= srt[-1] - 1e-3 * rms
    assert_close(mx.cpu().numpy(), mx_ref, what="full LM head max logit")


@pytest.mark.parametrize("name,sample", [("27b", (0, 1, 63, 64, 255, 300, 511)), ("70b", (0, 63, 300, 511))])
def test_prefill_layer_512_tokens_sampled(monkeypatch, name, sample):
    """i4d_prefill of a 512-token prompt (positions 0..511) through one
    27B- or 70B-shaped int4 layer (70B: D 8192, 64/8 heads, d_ff 28672).  For
    sampled tokens t the oracle decodes token t against the GPU's cache slots
    0..t-1 (the slots from t on poisoned): the output row to the float bar and
    the K/V it appends at slot t within one bf16 rounding step of the GPU's
    slot t.  Slots past the prompt untouched."""
    shape = synth.SHAPES[name].with_(n_layers=1)
    n = 512
    cap = n + 16
    _print_case(f"prefill {name} layer full size", n, "tokens")
    L = _FullLayer(shape, 9, 0, "int4", 1, cap)
    k0, v0 = L.caches()
    x = G.make_x_gpu(shape, 10, n)
    cfg = config_of(shape)
    ws = torch.zeros(B.prefill_workspace_size(cfg, n), dtype=torch.uint8, device="cuda")
    B.workspace_init(ws)
    out = torch.full_like(x, float("nan"))
    B.prefill(cfg, [L.layer], n, x, out, [L.kv], 0, ws)
    torch.cuda.synchronize()
    assert B.read_device_status(ws) == 0
    kc, vc = L.caches()
    got = out.cpu().numpy()
    xh = x.cpu().numpy().astype(np.float64)
    assert np.array_equal(kc[:, :, n:], k0[:, :, n:]) and np.array_equal(vc[:, :, n:], v0[:, :, n:])
    # expand the layer's matrices once for all sampled tokens (same values)
    monkeypatch.setattr(oracle.decode, "_DENSE_MEMO_ELEMS", 1 << 28)
    monkeypatch.setattr(oracle.decode, "_DENSE_MEMO", [])
    t0 = time.time()
    for t in sample:
        kt, vt = kc.copy(), vc.copy()
        kt[:, :, t:] = 0x7FC0
        vt[:, :, t:] = 0x7FC0
        r = oracle.decode_layer(shape, L.host, xh[t:t + 1], kt, vt, [t])
        assert_close(got[t], r["z"][0], what=f"prefill token {t}")
        _check_slots(kc, vc, r["k_cache"], r["v_cache"], kc, vc, [t], f"prefill token {t}")
    print(f"oracle {time.time() - t0:.1f} s", flush=True)
