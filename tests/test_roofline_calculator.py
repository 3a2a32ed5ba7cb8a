"""The closed-form byte/FLOP calculator against the numbers the pages print."""

import json
import os

import pytest

import synth
from int4_weight_streaming_decode_amd import roofline

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_closed_forms.json")


@pytest.fixture(scope="module")
def pages():
    with open(GOLDEN) as f:
        return json.load(f)


def test_roofline_reply_27b_intensity(pages):
    g = pages["roofline_reply_section_2"]
    flops = 2 * g["params"]
    byts = g["params"] * g["bytes_per_param"]
    assert flops == g["flops_per_token"] and byts == g["bytes_per_token"]
    assert flops / byts == g["intensity"]
    assert 100.0 / g["ridge"] == pytest.approx(g["utilisation_pct"], abs=0.01)


def test_primer_7b_decode_bound(pages):
    g = pages["primer_section_1_2"]
    t = roofline.decode_latency_bound_s(g["weight_bytes"], g["bandwidth"])
    assert t * 1e3 == pytest.approx(g["ms_per_token"], abs=0.05)
    assert 1.0 / t == pytest.approx(g["tokens_per_s"], rel=0.03)   # the page rounds 214 to "about 210"


def test_primer_memory_bill(pages):
    g = pages["primer_section_1_4"]
    m = roofline.estimate_mem(**g["args"])
    p = g["printed_GB"]
    assert m["weights"] / 1e9 == pytest.approx(p["weights"])
    assert m["adam"] / 1e9 == pytest.approx(p["adam"])
    assert m["act"] / 1e9 == pytest.approx(p["act"], abs=0.5)
    # the page prints 0.6 GB for KV; its own formula gives 2.68 GB (recorded contradiction)
    assert m["kv"] / 1e9 == pytest.approx(g["formula_kv_GB"], abs=0.01)
    assert m["kv"] / 1e9 != pytest.approx(p["kv"], abs=0.1)


def test_primer_70b_flop_sum(pages):
    g = pages["primer_section_1_1"]
    s = g["L"] * (4 * g["D"] ** 2 + 2 * g["D"] * g["d_ff"])
    assert s == pytest.approx(g["formula_value"], rel=1e-3)


def test_int4_bytes_per_weight_and_27b_step():
    # g = 128 with bf16 scales: 0.5 + 2/128 = 0.515625 bytes per weight
    assert roofline.matrix_bytes(128, 1024, 128) / (128 * 1024) == 0.515625
    s = synth.SHAPES["27b"]
    b = roofline.step_bytes(s, 1, s.kv_len + 1)
    # 64 layers x (186.5 MB weights + 33.6 MB KV read + 4 KB write)
    assert b / 1e9 == pytest.approx(14.087, abs=0.002)
    assert roofline.step_bytes(s, 1, s.kv_len + 1, "bf16") / 1e9 == pytest.approx(48.454, abs=0.002)
    lm = synth.SHAPES["27b_lm"]
    assert roofline.step_bytes(lm, 1, lm.kv_len + 1, lm_head=True) / 1e9 == pytest.approx(14.489, abs=0.002)


def test_phase_bytes_add_up_to_the_step():
    s = synth.SHAPES["27b_lm"]
    keys = s.kv_len + 1
    parts = sum(roofline.phase_bytes(s, p, 1, keys) for p in ("qkv", "attention", "wo", "gate_up", "down"))
    assert parts * s.n_layers == roofline.step_bytes(s, 1, keys)
    assert roofline.phase_bytes(s, "stream", 1, keys) == roofline.step_bytes(s, 1, keys)
    assert roofline.phase_bytes(s, "lm_head", 1, keys) == roofline.lm_head_bytes(s.vocab, s.d_model, s.group)
    # gate/up of the 27B shape: two 17408 x 5120 int4 matrices with groups of 128, plus the norm gain
    assert roofline.phase_bytes(s, "gate_up", 1, keys) == 2 * (17408 * 2560 + 17408 * 40 * 2) + 5120 * 2


def test_step_flops_is_two_flops_per_parameter_plus_attention():
    """Roofline reply 二: a decode token costs two FLOPs (one multiply-add) per
    weight.  The parameters are counted from a layer the input generator
    actually builds; the attention term is one multiply-add per (query head,
    key, dim) for the scores and again for the weighted sum of values."""
    s = synth.SHAPES["tiny"].with_(n_layers=3)
    layer = synth.make_layer(s, 0, 0)
    params = sum(layer[n]["codes"].size * 2 for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"))
    assert roofline.step_flops(s, 1, 0) == 2 * params * s.n_layers
    keys = 128
    attn = 2 * (s.n_q_heads * keys * s.head_dim) * 2 * s.n_layers
    assert roofline.step_flops(s, 1, keys) == 2 * params * s.n_layers + attn
    assert roofline.step_flops(s, 4, keys) == 4 * roofline.step_flops(s, 1, keys)


@pytest.mark.parametrize("batch,intensity", [(1, 4.8), (4, 11.4), (16, 17.2), (32, 18.8)])
def test_70b_batch_sweep_intensity(batch, intensity):
    """The 70B-shaped stack's roofline position per batch (FLOP per algorithmic
    byte of the whole step, KV 32768): the KV read grows with the batch, the
    weight read does not."""
    s = synth.SHAPES["70b"]
    keys = s.kv_len + 1
    assert roofline.step_flops(s, batch, keys) / roofline.step_bytes(s, batch, keys) == pytest.approx(intensity, abs=0.05)


def test_prefill_flops_is_the_sum_of_per_token_decode_flops():
    """A prompt of n tokens from position p0 costs what n decode steps at
    positions p0 .. p0 + n - 1 (keys p0 + t + 1) cost together."""
    s = synth.SHAPES["27b"]
    for n, p0 in ((1, 0), (512, 0), (77, 300)):
        total = roofline.prefill_flops(s, n, p0)["total"]
        assert total == sum(roofline.step_flops(s, 1, p0 + t + 1) for t in range(n))
    per = roofline.prefill_flops(s, 512, 0)["per_layer"]
    assert per["gate_up"] == 2 * 512 * 2 * s.d_ff * s.d_model
