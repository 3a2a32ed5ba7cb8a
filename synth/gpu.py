"""Seeded GPU-side generation of the large benchmark inputs (torch on the device).

Same recipe as synth.inputs (N(0, 0.02) weights quantised to int4 with
zero-point 8 and bf16 group scales of max|w|/7; bf16 N(0,1) KV; bf16 gains),
drawn with torch's device generator so that 14-70 GB of weights take seconds
instead of host minutes.  Values drawn here differ from the numpy generator's
(different random streams); the quantiser is the same rule and a GPU test
checks that both quantisers agree on identical weights.
"""

import torch


def quantize_int4_torch(w: torch.Tensor, group: int):
    """float32 [n][k] (k even) -> (codes uint8 [n][k/2], scales int16 bf16 bits [n][ceil(k/group)])."""
    n, k = w.shape
    ng = (k + group - 1) // group
    pad = ng * group - k
    wp = torch.nn.functional.pad(w, (0, pad)) if pad else w
    wg = wp.view(n, ng, group)
    amax = wg.abs().amax(dim=2)
    s = (amax / 7.0).to(torch.bfloat16)
    sf = s.float()
    safe = torch.where(sf == 0, torch.ones_like(sf), sf)
    q = torch.round(wg / safe.unsqueeze(2)) + 8          # round half to even
    q = torch.where((sf == 0).unsqueeze(2), torch.full_like(q, 8), q)
    q = q.clamp_(0, 15).to(torch.uint8).view(n, ng * group)[:, :k]
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).contiguous()
    return codes, s.view(torch.int16).contiguous()


def _gen(seed: int, layer: int, tensor: int) -> torch.Generator:
    g = torch.Generator(device="cuda")
    g.manual_seed(((seed * 1_000_003 + layer) * 101 + tensor) & 0x7FFFFFFFFFFFFFFF)
    return g


def _normal(shape, seed, layer, tensor, std=1.0):
    return torch.randn(shape, generator=_gen(seed, layer, tensor), device="cuda", dtype=torch.float32) * std


def make_layer_gpu(shape, seed: int, layer: int, weight_dtype: str = "int4") -> dict:
    """Device tensors of one layer: gains as int16 (bf16 bits); matrices as
    {codes, scales, n, k, group} (int4) or {bf16, n, k}."""
    D, qw, kvw, F = shape.d_model, shape.q_width, shape.kv_width, shape.d_ff
    dims = {"wq": (1, qw, D), "wk": (2, kvw, D), "wv": (3, kvw, D), "wo": (4, D, qw),
            "wg": (6, F, D), "wu": (7, F, D), "wd": (8, D, F)}
    out = {}
    for name, tid in (("attn_norm", 0), ("ffn_norm", 5)):
        out[name] = (1.0 + 0.1 * _normal((D,), seed, layer, tid)).to(torch.bfloat16).view(torch.int16)
    for name, (tid, n, k) in dims.items():
        w = _normal((n, k), seed, layer, tid, 0.02)
        if weight_dtype == "int4":
            codes, scales = quantize_int4_torch(w, shape.group)
            out[name] = {"codes": codes, "scales": scales, "n": n, "k": k, "group": shape.group}
        else:
            out[name] = {"bf16": w.to(torch.bfloat16).view(torch.int16), "n": n, "k": k}
        del w
    return out


def make_kv_gpu(shape, seed: int, layer: int, batch: int, capacity: int):
    """K [B][Hkv][cap/16][hd/32][16][32] and V [B][Hkv][cap/16][hd][16] (the
    library's 16-position cache tiles), bf16 N(0,1) bits as int16.  The values
    are i.i.d., so they are drawn directly in the tiled order."""
    H, hd = shape.n_kv_heads, shape.head_dim
    assert capacity % 16 == 0 and hd % 32 == 0
    k = _normal((batch, H, capacity // 16, hd // 32, 16, 32), seed, layer, 9).to(torch.bfloat16).view(torch.int16)
    v = _normal((batch, H, capacity // 16, hd, 16), seed, layer, 10).to(torch.bfloat16).view(torch.int16)
    return k, v


def make_x_gpu(shape, seed: int, batch: int) -> torch.Tensor:
    return _normal((batch, shape.d_model), seed, 0, 11).to(torch.bfloat16).float()


def make_lm_head_gpu(vocab: int, d_model: int, group: int, seed: int) -> dict:
    codes = torch.empty((vocab, d_model // 2), dtype=torch.uint8, device="cuda")
    ng = (d_model + group - 1) // group
    scales = torch.empty((vocab, ng), dtype=torch.int16, device="cuda")
    for i, r0 in enumerate(range(0, vocab, 8192)):
        r1 = min(vocab, r0 + 8192)
        w = _normal((r1 - r0, d_model), seed, i, 12, 0.02)
        codes[r0:r1], scales[r0:r1] = quantize_int4_torch(w, group)
    return {"codes": codes, "scales": scales, "n": vocab, "k": d_model, "group": group}
