"""A chunk of prompt tokens of one sequence through the stack at once
(i4d_prefill_chunk), against the oracle decoding the same tokens one after
another (Primer 1.2: prefill gives every prompt token what decoding would).
Float outputs to the usual bar per token; the appended slots within one bf16
rounding step; every other slot bit-identical.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from int4_weight_streaming_decode_amd import binding as B
from tests.gpu_util import DevKV, DevLayer, assert_close, config_of, dev, rel_l2, workspace

pytestmark = pytest.mark.gpu

SHAPE = synth.SHAPES["tiny"].with_(name="prefill", d_model=512, n_q_heads=4, n_kv_heads=2, head_dim=128, d_ff=1024,
                                   group=128, rope_base=1e6)


@pytest.mark.parametrize("n_tokens,pos0", [(5, 40), (24, 40), (32, 0), (1, 63)])
def test_prefill_chunk_equals_sequential_decode(n_tokens, pos0):
    n_layers, cap = 2, 112
    print("CASE prefill", n_tokens, pos0, flush=True)
    layers = [synth.make_layer(SHAPE, 33, l) for l in range(n_layers)]
    caches = [synth.make_kv(SHAPE, 33, l, 1, [pos0], cap) for l in range(n_layers)]   # slots >= pos0 poisoned
    x = np.stack([synth.make_x(SHAPE, 33, 1, step=t)[0] for t in range(n_tokens)])
    pos = np.arange(pos0, pos0 + n_tokens, dtype=np.int32)
    Ls = [DevLayer(l) for l in layers]
    kvs = [DevKV(*c) for c in caches]
    cfg = config_of(SHAPE)
    ws = workspace(cfg, n_tokens, cap - 1, n_layers=n_layers)
    out = torch.full((n_tokens, SHAPE.d_model), float("nan"), dtype=torch.float32, device="cuda")
    B.prefill_chunk(cfg, [l.layer for l in Ls], n_tokens, dev(x), out, [k.kv for k in kvs], dev(pos), int(pos[-1]), ws)
    torch.cuda.synchronize()
    assert B.read_device_status(ws) == 0
    ref_caches = caches
    got = out.cpu().numpy()
    for t in range(n_tokens):
        r = oracle.decode_stack(SHAPE, layers, x[t:t + 1].astype(np.float64), ref_caches, [pos0 + t])
        ref_caches = r["caches"]
        assert_close(got[t], r["z"][0], what=f"token {t}")
    for l in range(n_layers):
        kg, vg = kvs[l].host()
        for name, g_, r_, c0 in (("K", kg, ref_caches[l][0], caches[l][0]), ("V", vg, ref_caches[l][1], caches[l][1])):
            gv = synth.bf16_value(g_[0, :, pos0:pos0 + n_tokens]).astype(np.float64)
            rv = synth.bf16_value(r_[0, :, pos0:pos0 + n_tokens]).astype(np.float64)
            ulp = np.ldexp(1.0, np.frexp(np.abs(rv))[1] - 8)
            rms = np.sqrt(np.mean(rv * rv))
            assert rel_l2(gv, rv) <= 1e-3, f"layer {l} {name}"
            assert np.all(np.abs(gv - rv) <= np.maximum(5e-3 * rms, ulp)), f"layer {l} {name}"
            mask = np.ones(cap, dtype=bool)
            mask[pos0:pos0 + n_tokens] = False
            assert np.array_equal(g_[0][:, mask], c0[0][:, mask]), f"layer {l} {name}: other slots changed"
