"""The streaming decode kernel (exec_mode 2, and what auto picks at batch 1)
against the CPU oracle, through the C ABI.

Shapes are small enough for the oracle to finish in seconds but cover what
the kernel's schedule depends on: several 512-input units per row, q/k/v rows
split over the compute units in proportion, G = 2 and G = 7 query heads per KV
head, attention splits of one and of several load rounds, three layers whose
exchange regions chain, and positions that advance over several calls.

Bars: float outputs relative L2 <= 1e-3 and max |err| <= 5e-3 * RMS; each
appended K/V element within max(5e-3 * RMS, one bf16 rounding step), at least
98 % of them identical after rounding, every other slot bit-identical.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from int4_weight_streaming_decode_amd import binding as B
from tests.gpu_util import DevKV, DevLayer, assert_close, assert_close_bf16, bf16_ulp_diff, config_of, dev, workspace

pytestmark = pytest.mark.gpu

SMALL = synth.SHAPES["tiny"].with_(name="s512", d_model=512, n_q_heads=4, n_kv_heads=2, head_dim=128,
                                   d_ff=1024, group=128, rope_base=1e6)
G7 = synth.SHAPES["tiny"].with_(name="g7", d_model=1024, n_q_heads=28, n_kv_heads=4, head_dim=128,
                                d_ff=1536, group=128, rope_base=1e6)
SHAPES = {"s512": SMALL, "g7": G7}


def _print_case(*a):
    print("CASE", *a, flush=True)


def _run_stack(shape, layers, caches, x, pos, exec_mode=B.EXEC_STREAM, ws=None, cap=None):
    Ls = [DevLayer(l) for l in layers]
    kvs = [DevKV(*c) for c in caches]
    cfg = config_of(shape, exec_mode)
    ws = ws if ws is not None else workspace(cfg, 1, kvs[0].cap - 1, n_layers=len(layers))
    out = torch.full((1, shape.d_model), float("nan"), dtype=torch.float32, device="cuda")
    B.decode_stack(cfg, [l.layer for l in Ls], 1, dev(x), out, [k.kv for k in kvs], dev(np.array(pos, dtype=np.int32)),
                   pos[0], ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), [k.host() for k in kvs], B.read_device_status(ws)


def _check_caches(got, before, ref, pos, what):
    for l, ((kg, vg), (k0, v0), (kr, vr)) in enumerate(zip(got, before, ref)):
        for name, g_, r_, o_ in (("K", kg, kr, k0), ("V", vg, vr, v0)):
            assert_close_bf16(synth.bf16_value(g_[0, :, pos]), synth.bf16_value(r_[0, :, pos]),
                              what=f"{what} layer {l} {name} slot {pos}")
            assert np.mean(bf16_ulp_diff(g_[0, :, pos], r_[0, :, pos]) <= 1) >= 0.98
            mask = np.ones(g_.shape[2], dtype=bool)
            mask[pos] = False
            assert np.array_equal(g_[0][:, mask], o_[0][:, mask]), f"{what} layer {l} {name}: other slots changed"


@pytest.mark.parametrize("name,n_layers,pos", [
    ("s512", 1, 127),         # one attention subtile per split
    ("s512", 3, 5000),        # three chained layers, several subtiles per split
    ("s512", 1, 40000),       # splits of more than one load round
    ("s512", 1, 1024),        # p = splits * 16: the new key extends the last split by one subtile
    ("s512", 1, 16384),       # ... which is then a second round holding the new key alone
    ("g7", 2, 2049),          # 7 query heads per KV head, q/k/v split over 28 + 4 + 4 heads
])
def test_stream_stack_matches_oracle(name, n_layers, pos):
    shape = SHAPES[name]
    _print_case("stream stack", name, n_layers, pos)
    cap = ((pos + 1 + 15) // 16) * 16 + 16
    layers = [synth.make_layer(shape, 40 + pos, l) for l in range(n_layers)]
    caches = [synth.make_kv(shape, 40 + pos, l, 1, [pos], cap) for l in range(n_layers)]
    x = synth.make_x(shape, 40 + pos, 1)
    ref = oracle.decode_stack(shape, layers, x.astype(np.float64), caches, [pos])
    out, got, status = _run_stack(shape, layers, caches, x, [pos])
    assert status == 0, status
    assert_close(out, ref["z"], what=f"stream {name} x{n_layers} @ {pos}")
    _check_caches(got, caches, ref["caches"], pos, "stream")


def test_stream_is_bit_reproducible_and_agrees_with_phase_launches():
    """Fixed reduction orders: two runs give the same bits.  The phase
    launches stage activations as fp16 and the streaming kernel as 16-bit
    integers per 32-input run, so the two modes agree to the float bar."""
    shape = SMALL
    pos = 3000
    _print_case("stream reproducible")
    cap = ((pos + 1 + 15) // 16) * 16
    layers = [synth.make_layer(shape, 77, l) for l in range(3)]
    caches = [synth.make_kv(shape, 77, l, 1, [pos], cap) for l in range(3)]
    x = synth.make_x(shape, 77, 1)
    a = _run_stack(shape, layers, caches, x, [pos])
    b = _run_stack(shape, layers, caches, x, [pos])
    c = _run_stack(shape, layers, caches, x, [pos], exec_mode=B.EXEC_PHASES)
    assert a[2] == 0 and b[2] == 0 and c[2] == 0
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32)), "two runs differ"
    for l in range(3):
        assert np.array_equal(a[1][l][0], b[1][l][0]) and np.array_equal(a[1][l][1], b[1][l][1])
    assert_close(a[0], c[0], what="stream vs phase launches")


def test_stream_large_activations():
    """Activations far beyond fp16 range (residual stream near 2^24, SwiGLU
    outputs near 1e5 through an up projection whose scales are multiplied by
    2^16): every run's power of two adapts, so the result still meets the bar
    and no status bit is set."""
    shape = SMALL
    pos = 300
    _print_case("stream large activations")
    cap = ((pos + 1 + 15) // 16) * 16
    layer = synth.make_layer(shape, 91, 0)
    wu = dict(layer["wu"])
    s = synth.bf16_value(wu["scales"]).astype(np.float64) * 65536.0
    wu["scales"] = synth.bf16_bits(s.astype(np.float32))
    layer["wu"] = wu
    caches = [synth.make_kv(shape, 91, 0, 1, [pos], cap)]
    x = (synth.make_x(shape, 91, 1).astype(np.float64) * 2.0 ** 24).astype(np.float32)
    ref = oracle.decode_layer(shape, layer, x.astype(np.float64), caches[0][0], caches[0][1], [pos])
    assert np.max(np.abs(ref["act"])) > 65504.0 and np.max(np.abs(x)) > 65504.0
    out, got, status = _run_stack(shape, [layer], caches, x, [pos])
    assert status == 0, status
    assert_close(out, ref["z"], what="stream with large activations")


def test_stream_bad_position_sets_status_and_skips_append():
    shape = SMALL
    _print_case("stream bad position")
    cap = 64
    layers = [synth.make_layer(shape, 5, 0)]
    caches = [synth.make_kv(shape, 5, 0, 1, [20], cap)]
    x = synth.make_x(shape, 5, 1)
    Ls = [DevLayer(l) for l in layers]
    kvs = [DevKV(*c) for c in caches]
    cfg = config_of(shape, B.EXEC_STREAM)
    ws = workspace(cfg, 1, 20)
    out = torch.empty((1, shape.d_model), dtype=torch.float32, device="cuda")
    # pos[0] = 40 > max_pos = 20: flagged, nothing appended, the kernel still ends
    B.decode_stack(cfg, [l.layer for l in Ls], 1, dev(x), out, [k.kv for k in kvs], dev(np.array([40], dtype=np.int32)),
                   20, ws)
    torch.cuda.synchronize()
    st = B.read_device_status(ws)
    assert st & B.I4D_DEV_BAD_POS and not st & B.I4D_DEV_BARRIER_TIMEOUT, st
    k_gpu, v_gpu = kvs[0].host()
    assert np.array_equal(k_gpu, caches[0][0]) and np.array_equal(v_gpu, caches[0][1])


def test_stream_graph_replays_equal_the_eager_call():
    """A captured step (an ordinary launch inside the capture) replayed three
    times, with eager work in between: every replay equals the eager call bit
    for bit (the launch epoch advances on the device, so each replay uses
    fresh exchange tags)."""
    shape = SMALL
    pos = 700
    _print_case("stream graph replay")
    cap = ((pos + 1 + 15) // 16) * 16
    layers = [synth.make_layer(shape, 13, l) for l in range(2)]
    caches = [synth.make_kv(shape, 13, l, 1, [pos], cap) for l in range(2)]
    x = synth.make_x(shape, 13, 1)
    Ls = [DevLayer(l) for l in layers]
    kvs = [DevKV(*c) for c in caches]
    cfg = config_of(shape, B.EXEC_STREAM)
    ws = workspace(cfg, 1, cap - 1, n_layers=2)
    xd = dev(x)
    pd = dev(np.array([pos], dtype=np.int32))
    out = torch.full((1, shape.d_model), float("nan"), dtype=torch.float32, device="cuda")
    larr, karr = [l.layer for l in Ls], [k.kv for k in kvs]
    B.decode_stack(cfg, larr, 1, xd, out, karr, pd, pos, ws)
    torch.cuda.synchronize()
    eager = out.cpu().numpy().copy()
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gs):
        B.decode_stack(cfg, larr, 1, xd, out, karr, pd, pos, ws)
    torch.cuda.current_stream().wait_stream(gs)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), eager.view(np.uint32)), f"replay {rep}"
        B.decode_stack(cfg, larr, 1, xd, out, karr, pd, pos, ws)      # eager work between replays
        torch.cuda.synchronize()
    assert B.read_device_status(ws) == 0


def test_auto_mode_takes_the_streaming_kernel_at_batch_1():
    shape = SMALL
    pos = 200
    cap = ((pos + 1 + 15) // 16) * 16
    layers = [synth.make_layer(shape, 3, 0)]
    caches = [synth.make_kv(shape, 3, 0, 1, [pos], cap)]
    x = synth.make_x(shape, 3, 1)
    B.launch_timing_start("stream", 16)
    _run_stack(shape, layers, caches, x, [pos], exec_mode=B.EXEC_AUTO)
    _, n = B.launch_timing_stop()
    assert n == 1
