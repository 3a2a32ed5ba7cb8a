"""Whole-prompt prefill (i4d_prefill): the prompt runs as int4 GEMMs with the
tokens as the wide dimension and a causal attention tiled over the prompt,
against the oracle decoding the same tokens one after another (Primer 1.2:
prefill gives every prompt token what decoding would).  Every token's output
to the usual float bar, every appended K/V slot within one bf16 rounding step,
every other slot bit-identical.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from int4_weight_streaming_decode_amd import binding as B
from tests.gpu_util import DevKV, DevLayer, assert_close, assert_close_bf16, config_of, dev

pytestmark = pytest.mark.gpu

# head_dim 128, groups of 128
SHAPE_A = synth.SHAPES["tiny"].with_(name="prefill_a", d_model=512, n_q_heads=4, n_kv_heads=2, head_dim=128, d_ff=1024,
                                     group=128, rope_base=1e6)
# head_dim 64, four query heads per KV head, groups of 256, a long down projection (its K axis is split)
SHAPE_B = synth.SHAPES["tiny"].with_(name="prefill_b", d_model=512, n_q_heads=8, n_kv_heads=2, head_dim=64, d_ff=4096,
                                     group=256, rope_base=1e4)


def run_prefill(shape, n_tokens, pos0, n_layers=2, seed=41):
    cap = ((pos0 + n_tokens + 15) // 16 + 1) * 16
    print("CASE prefill", shape.name, n_tokens, pos0, flush=True)
    layers = [synth.make_layer(shape, seed, l) for l in range(n_layers)]
    caches = [synth.make_kv(shape, seed, l, 1, [pos0], cap) for l in range(n_layers)]   # slots >= pos0 poisoned
    x = np.stack([synth.make_x(shape, seed, 1, step=t)[0] for t in range(n_tokens)])
    Ls = [DevLayer(l) for l in layers]
    kvs = [DevKV(*c) for c in caches]
    cfg = config_of(shape)
    nws = B.prefill_workspace_size(cfg, n_tokens)
    assert nws > 0
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
    B.workspace_init(ws)
    out = torch.full((n_tokens, shape.d_model), float("nan"), dtype=torch.float32, device="cuda")
    B.prefill(cfg, [l.layer for l in Ls], n_tokens, dev(x), out, [k.kv for k in kvs], pos0, ws)
    torch.cuda.synchronize()
    assert B.read_device_status(ws) == 0
    ref = oracle.prefill(shape, layers, x.astype(np.float64), caches, pos0)
    return out.cpu().numpy(), kvs, caches, ref, cap


def check(shape, n_tokens, pos0):
    got, kvs, caches, ref, cap = run_prefill(shape, n_tokens, pos0)
    for t in range(n_tokens):
        assert_close(got[t], ref["z"][t], what=f"token {t}")
    for l, kv in enumerate(kvs):
        kg, vg = kv.host()
        for name, g_, r_, c0 in (("K", kg, ref["caches"][l][0], caches[l][0]), ("V", vg, ref["caches"][l][1], caches[l][1])):
            sl = slice(pos0, pos0 + n_tokens)
            assert_close_bf16(synth.bf16_value(g_[0, :, sl]), synth.bf16_value(r_[0, :, sl]), what=f"layer {l} {name} slots")
            mask = np.ones(cap, dtype=bool)
            mask[sl] = False
            assert np.array_equal(g_[0][:, mask], c0[0][:, mask]), f"layer {l} {name}: other slots changed"


@pytest.mark.parametrize("n_tokens,pos0", [(128, 0), (512, 0), (77, 40), (1, 63), (200, 300), (2048, 5)])
def test_prefill_equals_sequential_decode(n_tokens, pos0):
    check(SHAPE_A, n_tokens, pos0)


@pytest.mark.parametrize("n_tokens,pos0", [(128, 0), (333, 17)])
def test_prefill_hd64_group256_split_k(n_tokens, pos0):
    check(SHAPE_B, n_tokens, pos0)


def test_prefill_in_two_calls_equals_one_call():
    """The second half of a prompt after the first half's cache gives the same
    outputs and cache as one call over the whole prompt (same kernels, same
    per-token arithmetic), bit for bit."""
    shape, n, cut = SHAPE_A, 160, 96
    cap = 176
    layers = [synth.make_layer(shape, 43, l) for l in range(2)]
    Ls = [DevLayer(l) for l in layers]
    x = np.stack([synth.make_x(shape, 43, 1, step=t)[0] for t in range(n)])
    cfg = config_of(shape)

    def fresh_caches():
        return [DevKV(*synth.make_kv(shape, 43, l, 1, [0], cap)) for l in range(2)]

    def call(kvs, xs, pos0):
        ws = torch.zeros(B.prefill_workspace_size(cfg, xs.shape[0]), dtype=torch.uint8, device="cuda")
        B.workspace_init(ws)
        out = torch.empty((xs.shape[0], shape.d_model), dtype=torch.float32, device="cuda")
        B.prefill(cfg, [l.layer for l in Ls], xs.shape[0], dev(xs), out, [k.kv for k in kvs], pos0, ws)
        torch.cuda.synchronize()
        assert B.read_device_status(ws) == 0
        return out.cpu().numpy()

    one = fresh_caches()
    z1 = call(one, x, 0)
    two = fresh_caches()
    call(two, x[:cut], 0)
    z2 = call(two, x[cut:], cut)
    # rows after the cut see the same cache contents; the GEMM sums each
    # token's row in the same order whatever tile it falls in
    assert np.array_equal(z2, z1[cut:])
    for a, b in zip(one, two):
        for u, v in zip(a.host(), b.host()):
            assert np.array_equal(u, v)


def test_prefill_replays_from_a_graph():
    """i4d_prefill captured in a graph (it enqueues kernels only: no memset, no
    allocation) and replayed three times, with eager work, a synchronisation
    and the output poisoned between replays: every replay gives the eager
    call's outputs and cache, bit for bit."""
    shape, n, pos0, cap = SHAPE_A, 200, 30, 240
    print("CASE prefill graph", n, pos0, flush=True)
    layers = [synth.make_layer(shape, 47, l) for l in range(2)]
    caches = [synth.make_kv(shape, 47, l, 1, [pos0], cap) for l in range(2)]
    x = dev(np.stack([synth.make_x(shape, 47, 1, step=t)[0] for t in range(n)]))
    Ls = [DevLayer(l) for l in layers]
    cfg = config_of(shape)

    def state():
        kvs = [DevKV(*c) for c in caches]
        ws = torch.zeros(B.prefill_workspace_size(cfg, n), dtype=torch.uint8, device="cuda")
        B.workspace_init(ws)
        return kvs, ws, torch.empty((n, shape.d_model), dtype=torch.float32, device="cuda")

    kvs, ws, out = state()
    B.prefill(cfg, [l.layer for l in Ls], n, x, out, [k.kv for k in kvs], pos0, ws)
    torch.cuda.synchronize()
    ref_out, ref_kv = out.cpu().numpy(), [k.host() for k in kvs]

    kvs2, ws2, out2 = state()
    larr, karr = [l.layer for l in Ls], [k.kv for k in kvs2]
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=gs):
        B.prefill(cfg, larr, n, x, out2, karr, pos0, ws2)
    torch.cuda.current_stream().wait_stream(gs)
    torch.cuda.synchronize()
    for rep in range(3):
        out2.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _ = (torch.ones(1024, device="cuda") * 2).sum().item()      # eager work between replays
        assert np.array_equal(out2.cpu().numpy().view(np.uint32), ref_out.view(np.uint32)), f"replay {rep}"
        for a, b in zip([k.host() for k in kvs2], ref_kv):
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), f"replay {rep}: cache"
    assert B.read_device_status(ws2) == 0
