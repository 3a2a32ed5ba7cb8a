"""Test glue: move synth arrays to the GPU in the library's layouts and compare results.

Layout conversion only (the K/V caches are handed to the library in its
16-position tiles); no decode arithmetic lives here.
"""

import numpy as np
import torch

from int4_weight_streaming_decode_amd import binding as B

MAT_NAMES = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


class DevMat:
    def __init__(self, m: dict):
        if "codes" in m:
            self.data = dev(m["codes"])
            self.scales = dev(m["scales"])
            self.mat = B.make_mat(self.data, self.scales, m["n"], m["k"], m["group"], B.WEIGHT_INT4)
        else:
            self.data = dev(m["bf16"])
            self.scales = None
            self.mat = B.make_mat(self.data, None, m["n"], m["k"], 0, B.WEIGHT_BF16)


class DevLayer:
    def __init__(self, layer: dict):
        self.attn_norm = dev(layer["attn_norm"])
        self.ffn_norm = dev(layer["ffn_norm"])
        self.mats = {n: DevMat(layer[n]) for n in MAT_NAMES}
        self.layer = B.make_layer(self.attn_norm, self.ffn_norm, {n: self.mats[n].mat for n in MAT_NAMES})


def k_to_tiles(kc: np.ndarray) -> np.ndarray:
    """[B][H][cap][hd] -> [B][H][cap/16][hd/32][16][32]."""
    b, h, cap, hd = kc.shape
    return np.ascontiguousarray(kc.reshape(b, h, cap // 16, 16, hd // 32, 32).transpose(0, 1, 2, 4, 3, 5))


def v_to_tiles(vc: np.ndarray) -> np.ndarray:
    """[B][H][cap][hd] -> [B][H][cap/16][hd][16]."""
    b, h, cap, hd = vc.shape
    return np.ascontiguousarray(vc.reshape(b, h, cap // 16, 16, hd).transpose(0, 1, 2, 4, 3))


def k_from_tiles(kt: np.ndarray, shape) -> np.ndarray:
    b, h, cap, hd = shape
    return np.ascontiguousarray(kt.reshape(b, h, cap // 16, hd // 32, 16, 32).transpose(0, 1, 2, 4, 3, 5).reshape(shape))


def v_from_tiles(vt: np.ndarray, shape) -> np.ndarray:
    b, h, cap, hd = shape
    return np.ascontiguousarray(vt.reshape(b, h, cap // 16, hd, 16).transpose(0, 1, 2, 4, 3).reshape(shape))


class DevKV:
    """K and V given as [B][Hkv][cap][hd]; held on the device in the library's tiles."""

    def __init__(self, kc: np.ndarray, vc: np.ndarray):
        self.shape = kc.shape
        self.cap = kc.shape[2]
        self.k = dev(k_to_tiles(kc))
        self.v = dev(v_to_tiles(vc))
        self.kv = B.make_kv(self.k, self.v, self.cap)

    def host(self):
        return k_from_tiles(host_u16(self.k), self.shape), v_from_tiles(host_u16(self.v), self.shape)


def config_of(shape, exec_mode=B.EXEC_AUTO):
    return B.make_config(shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.d_ff,
                         shape.rms_eps, shape.rope_base, exec_mode)


def workspace(cfg, batch, max_pos, vocab=0, n_layers=1):
    n = B.workspace_size(cfg, n_layers, batch, max_pos, vocab)
    assert n > 0
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    B.workspace_init(ws)
    return ws


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def assert_close(got, ref, rel=1e-3, abs_frac=5e-3, what=""):
    """The float bar: relative L2 <= rel and max |err| <= abs_frac * RMS(ref)."""
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = rel_l2(got, ref)
    rms = np.sqrt(np.mean(ref * ref))
    mx = float(np.max(np.abs(got - ref))) if got.size else 0.0
    print(f"PARITY {what}: rel-L2 {r:.3e} max-abs/RMS {mx / max(rms, 1e-300):.3e}", flush=True)
    assert r <= rel, f"{what}: rel-L2 {r:.3e} > {rel}"
    assert mx <= abs_frac * rms, f"{what}: max-abs {mx:.3e} > {abs_frac} * RMS {rms:.3e}"
    return r, mx / max(rms, 1e-300)


def assert_close_bf16(got, ref, rel=1e-3, abs_frac=5e-3, what=""):
    """The float bar for values stored in bf16: relative L2 <= rel, and each
    element within max(abs_frac * RMS(ref), one bf16 ulp of the reference) --
    a correctly computed value may land one rounding step away."""
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = rel_l2(got, ref)
    rms = np.sqrt(np.mean(ref * ref))
    ulp = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 8)      # bf16 spacing at |ref|
    err = np.abs(got - ref)
    print(f"PARITY {what}: rel-L2 {r:.3e} max-abs/RMS {err.max() / max(rms, 1e-300):.3e}", flush=True)
    assert r <= rel, f"{what}: rel-L2 {r:.3e} > {rel}"
    bad = err > np.maximum(abs_frac * rms, ulp)
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond max(5e-3*RMS, 1 ulp); worst {err.max():.3e}"
    return r


def bf16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps between two arrays of finite bf16 bit patterns."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(a_bits) - ordered(b_bits))
