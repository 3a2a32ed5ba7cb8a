"""Activations far outside fp16 range, through every batch path of one layer.

The matrix-vector and matrix-core paths stage activations as fp16.  Each
staged chunk (matrix-vector) or sequence row (matrix-core) is multiplied by
a power of two that keeps its largest value below 2^15, and the inverse
multiplies the results, so the layer still meets the float bar against the
oracle and no value turns into inf.  The inputs here reach about 2^24 in the
residual stream, and the SwiGLU output that feeds W_down passes 1e5 (the up
projection's scales are multiplied by 2^18).

Bar: relative L2 <= 1e-3 and max |err| <= 5e-3 * RMS per sequence; status 0.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from int4_weight_streaming_decode_amd import binding as B
from tests.gpu_util import DevKV, DevLayer, assert_close, config_of, dev, workspace

pytestmark = pytest.mark.gpu

SMALL = synth.SHAPES["tiny"].with_(name="s512", d_model=512, n_q_heads=4, n_kv_heads=2, head_dim=128,
                                   d_ff=1024, group=128, rope_base=1e6)


def _large_layer(shape, seed):
    layer = synth.make_layer(shape, seed, 0)
    wu = dict(layer["wu"])
    s = synth.bf16_value(wu["scales"]).astype(np.float64) * 262144.0
    wu["scales"] = synth.bf16_bits(s.astype(np.float32))
    layer["wu"] = wu
    return layer


@pytest.mark.parametrize("batch,mode,path", [
    (1, B.EXEC_PHASES, "matrix-vector, one sequence"),
    (4, B.EXEC_AUTO, "matrix-vector, four sequences"),
    (16, B.EXEC_AUTO, "matrix cores, sixteen sequences"),
])
def test_layer_with_activations_beyond_fp16_range(batch, mode, path):
    shape = SMALL
    print("CASE large activations", path, flush=True)
    pos = [300 - 7 * b for b in range(batch)]
    cap = ((max(pos) + 1 + 15) // 16) * 16 + 16
    layer = _large_layer(shape, 17 + batch)
    kc, vc = synth.make_kv(shape, 17 + batch, 0, batch, pos, cap)
    x = (synth.make_x(shape, 17 + batch, batch).astype(np.float64) * 2.0 ** 24).astype(np.float32)
    ref = oracle.decode_layer(shape, layer, x.astype(np.float64), kc, vc, pos)
    assert np.max(np.abs(ref["act"])) > 65504.0 and np.max(np.abs(x)) > 65504.0
    L, kvd = DevLayer(layer), DevKV(kc, vc)
    cfg = config_of(shape, mode)
    ws = workspace(cfg, batch, max(pos))
    out = torch.full((batch, shape.d_model), float("nan"), dtype=torch.float32, device="cuda")
    B.decode_layer(cfg, L.layer, batch, dev(x), out, kvd.kv, dev(np.array(pos, dtype=np.int32)), max(pos), ws)
    torch.cuda.synchronize()
    assert B.read_device_status(ws) == 0
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    for b in range(batch):
        assert_close(got[b], ref["z"][b], what=f"{path}: sequence {b}")
