"""Parity at the full sizes of the timed workloads, through the C ABI.

Inputs come from the seeded device generator (the bench's own), are copied
to the host, and the CPU oracle recomputes the same step: one 27B-shaped
layer at 8192 cached tokens (batch 1 on the matrix-vector path, batch 16 on
the matrix-core path) and the 152064 x 5120 int4 LM head (batch 1 and 16).
Same bars as the other parity tests: float outputs relative L2 <= 1e-3 and
max |err| <= 5e-3 * RMS; the appended K/V slot within one bf16 rounding step;
token ids exact unless the oracle's top-2 gap is a near-tie.
"""

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
    return {"codes": m["codes"].cpu().numpy(), "scales": m["scales"].cpu().numpy().view(np.uint16),
            "n": m["n"], "k": m["k"], "group": m["group"]}


def _bits(t):
    return t.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("batch", [1, 16])
def test_27b_layer_at_full_size(batch):
    shape = synth.SHAPES["27b"]
    pos0 = shape.kv_len                                   # 8192 cached tokens
    pos = [pos0 - 37 * b for b in range(batch)]           # batch 16: sequences at different positions
    cap = ((pos0 + 1 + 15) // 16) * 16
    _print_case("27b layer full size", batch, pos[:3])
    p = G.make_layer_gpu(shape, 5, 0)
    k, v = G.make_kv_gpu(shape, 5, 0, batch, cap)
    x = G.make_x_gpu(shape, 6, batch)
    mats = {n: B.make_mat(p[n]["codes"], p[n]["scales"], p[n]["n"], p[n]["k"], p[n]["group"], B.WEIGHT_INT4) for n in MATS}
    layer = B.make_layer(p["attn_norm"], p["ffn_norm"], mats)
    kv = B.make_kv(k, v, cap)
    # the oracle's copies, taken before the call appends slot pos[b]
    kshape = (batch, shape.n_kv_heads, cap, shape.head_dim)
    kc = k_from_tiles(_bits(k), kshape)
    vc = v_from_tiles(_bits(v), kshape)
    host_layer = {"attn_norm": _bits(p["attn_norm"]), "ffn_norm": _bits(p["ffn_norm"])}
    host_layer.update({n: _host_mat(p[n]) for n in MATS})
    cfg = config_of(shape)
    ws = workspace(cfg, batch, pos0)
    out = torch.full((batch, shape.d_model), float("nan"), dtype=torch.float32, device="cuda")
    B.decode_layer(cfg, layer, batch, x, out, kv, torch.tensor(pos, dtype=torch.int32, device="cuda"), pos0, ws)
    torch.cuda.synchronize()
    assert B.read_device_status(ws) == 0
    ref = oracle.decode_layer(shape, host_layer, x.cpu().numpy().astype(np.float64), kc, vc, pos)
    got = out.cpu().numpy()
    for b in range(batch):
        assert_close(got[b], ref["z"][b], what=f"27b layer b={b}")
    kg = k_from_tiles(_bits(k), kshape)
    vg = v_from_tiles(_bits(v), kshape)
    for b, pb in enumerate(pos):
        for name, g_, r_ in (("K", kg, ref["k_cache"]), ("V", vg, ref["v_cache"])):
            gv = synth.bf16_value(g_[b, :, pb]).astype(np.float64)
            rv = synth.bf16_value(r_[b, :, pb]).astype(np.float64)
            ulp = np.ldexp(1.0, np.frexp(np.abs(rv))[1] - 8)
            rms = np.sqrt(np.mean(rv * rv))
            assert np.all(np.abs(gv - rv) <= np.maximum(5e-3 * rms, ulp)), f"{name} slot {pb} of b={b}"
        # one untouched slot per sequence, bit-identical
        assert np.array_equal(kg[b, :, pb - 1], kc[b, :, pb - 1]) and np.array_equal(vg[b, :, pb - 1], vc[b, :, pb - 1])


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
