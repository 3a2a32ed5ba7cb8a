"""Host-side checks of the C ABI: the library loads, exports every declared
entry point, and rejects bad arguments before enqueuing any GPU work.

No call here reaches a HIP API (validation happens first), so these run on a
machine without a GPU.
"""

import ctypes
import os
import re

import pytest

from int4_weight_streaming_decode_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "i4decode.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(i4d_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libi4decode.so not built: run __graft_entry__.build()")
    return B.lib()


def test_every_declared_symbol_is_exported(lib):
    syms = declared_symbols()
    assert len(syms) >= 10
    for s in syms:
        assert hasattr(lib, s), s


def test_no_kernel_of_the_library_needs_scratch(lib):
    """Every kernel in the built library's gfx950 code object declares a
    private segment of 0 bytes (no register spills or arrays in per-lane
    scratch memory); the launchers also refuse such a kernel at run time."""
    import sys
    sys.path.insert(0, ROOT)
    import __graft_entry__ as g
    assert g.kernels_with_scratch(B.LIB_PATH) == []


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert B.status_string(code)
    assert B.status_string(-99) == "unknown status"


def _cfg(**kw):
    base = dict(d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, d_ff=688, rms_eps=1e-6, rope_base=1e4)
    base.update(kw)
    return B.make_config(**base)


def test_workspace_size_is_pure_and_validates(lib):
    assert B.workspace_size(_cfg(), 1, 1, 127) > 0
    assert B.workspace_size(_cfg(), 64, 8, 32767) > B.workspace_size(_cfg(), 64, 1, 32767)
    assert B.workspace_size(_cfg(), 64, 1, 127) > B.workspace_size(_cfg(), 1, 1, 127)
    assert B.workspace_size(_cfg(), 1, 1, 127) >= B.WS_MIN_BYTES
    assert B.workspace_size(_cfg(head_dim=96), 1, 1, 127) == 0          # unsupported head_dim
    assert B.workspace_size(_cfg(n_q_heads=6, n_kv_heads=4), 1, 1, 127) == 0  # Hq % Hkv != 0
    assert B.workspace_size(_cfg(), 1, 33, 127) == 0                    # batch > 32
    assert B.workspace_size(_cfg(), 1, 16, 127) > B.workspace_size(_cfg(), 1, 4, 127)   # matrix-core scratch
    assert B.workspace_size(_cfg(), 1, 16, 127, 1000) >= B.workspace_size(_cfg(), 1, 16, 127)
    assert B.workspace_size(_cfg(), 1, 0, 127) == 0
    assert B.workspace_size(_cfg(), 0, 1, 127) == 0                     # no layers


class _FakeDev:
    """An address stand-in: validation never dereferences pointers."""

    def __init__(self, addr, nbytes=1 << 30):
        self.addr, self.n = addr, nbytes

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.n

    def element_size(self):
        return 1


def _mat(n, k, group=64, addr=0x10000, dtype=B.WEIGHT_INT4):
    return B.I4dMat(addr, addr + 0x8000000, n, k, group, dtype)


def _layer(cfg, group=64, **override):
    D, qw, kvw, F = cfg.d_model, cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim, cfg.d_ff
    mats = {"wq": _mat(qw, D, group), "wk": _mat(kvw, D, group), "wv": _mat(kvw, D, group),
            "wo": _mat(D, qw, group), "wg": _mat(F, D, group), "wu": _mat(F, D, group), "wd": _mat(D, F, group)}
    mats.update(override)
    return B.I4dLayer(0x20000, mats["wq"], mats["wk"], mats["wv"], mats["wo"], 0x30000, mats["wg"], mats["wu"], mats["wd"])


def _call_layer(cfg, layer, batch=1, x_in=0x100000, x_out=0x200000, cap=256, max_pos=127, ws=0x400000, ws_bytes=1 << 30):
    kv = B.I4dKv(0x500000, 0x600000, cap)
    return B.lib().i4d_decode_layer(ctypes.byref(cfg), ctypes.byref(layer), batch, ctypes.c_void_p(x_in),
                                    ctypes.c_void_p(x_out), ctypes.byref(kv), ctypes.c_void_p(0x700000), max_pos,
                                    ctypes.c_void_p(ws), ws_bytes, None)


def test_decode_layer_argument_validation(lib):
    cfg = _cfg()
    L = _layer(cfg)
    assert lib.i4d_decode_layer(None, ctypes.byref(L), 1, None, None, None, None, 0, None, 0, None) == B.I4D_EINVAL
    assert _call_layer(cfg, L, batch=0) == B.I4D_ERANGE
    assert _call_layer(cfg, L, batch=33) == B.I4D_ERANGE
    assert _call_layer(cfg, L, batch=16) == B.I4D_EUNSUPPORTED          # K = 688, group 64: not on the MFMA path
    assert _call_layer(cfg, L, x_out=0x100000) == B.I4D_EINVAL           # x_out aliases x_in
    assert _call_layer(cfg, L, x_in=0x100004) == B.I4D_EALIGN
    assert _call_layer(cfg, L, max_pos=256) == B.I4D_ERANGE                # max_pos >= capacity
    assert _call_layer(cfg, L, cap=250) == B.I4D_EINVAL                    # capacity % 16 != 0
    assert _call_layer(cfg, L, cap=248) == B.I4D_EINVAL
    assert _call_layer(cfg, L, ws_bytes=100) == B.I4D_EWORKSPACE
    assert _call_layer(cfg, L, ws=0x400010) == B.I4D_EALIGN
    assert _call_layer(cfg, _layer(cfg, wq=_mat(255, 256))) == B.I4D_EINVAL   # wrong row count
    assert _call_layer(cfg, _layer(cfg, wo=_mat(256, 256, addr=0x10008))) == B.I4D_EALIGN
    assert _call_layer(cfg, _layer(cfg, group=12)) == B.I4D_EINVAL             # group % 8 != 0
    assert _call_layer(_cfg(head_dim=80), L) == B.I4D_EINVAL
    mixed = _layer(cfg, wd=_mat(256, 688, dtype=B.WEIGHT_BF16))
    assert _call_layer(cfg, mixed) == B.I4D_EINVAL


def test_lm_head_and_gemv_validation(lib):
    w = _mat(1000, 256)
    h = ctypes.c_void_p(0x100000)
    out = ctypes.c_void_p(0x200000)
    ws = ctypes.c_void_p(0x400000)
    assert lib.i4d_lm_head_chunked(ctypes.byref(w), 1, h, 0, out, out, ws, 1 << 20, None) == B.I4D_ERANGE
    assert lib.i4d_lm_head_chunked(ctypes.byref(w), 0, h, 64, out, out, ws, 1 << 20, None) == B.I4D_ERANGE
    assert lib.i4d_lm_head_chunked(ctypes.byref(w), 1, h, 64, out, out, ws, 16, None) == B.I4D_EWORKSPACE
    wb = _mat(1000, 256, dtype=B.WEIGHT_BF16)
    assert lib.i4d_lm_head_chunked(ctypes.byref(wb), 1, h, 64, out, out, ws, 1 << 20, None) == B.I4D_EINVAL
    assert lib.i4d_gemv(ctypes.byref(_mat(10, 12)), 1, h, out, None, 0, None) == B.I4D_EINVAL   # k % 8 != 0
    assert lib.i4d_gemv(ctypes.byref(w), 33, h, out, None, 0, None) == B.I4D_ERANGE
    assert lib.i4d_gemv(ctypes.byref(w), 16, h, out, None, 0, None) == B.I4D_EUNSUPPORTED      # group 64
    w128 = _mat(1000, 256, group=128)
    assert lib.i4d_gemv(ctypes.byref(w128), 16, h, out, None, 0, None) == B.I4D_EWORKSPACE
    assert lib.i4d_lm_head_chunked(ctypes.byref(w128), 16, h, 64, out, out, ws, 1 << 20, None) == B.I4D_EWORKSPACE
    assert lib.i4d_dequant_int4(None, out, None) == B.I4D_EINVAL


def test_lm_head_noalloc_validation(lib):
    """The workspace-free LM head checks its arguments before any device call:
    it takes the matrix-vector path only (batch 1..8)."""
    w = _mat(1000, 256)
    h = ctypes.c_void_p(0x100000)
    out = ctypes.c_void_p(0x200000)
    f = lib.i4d_lm_head_chunked_noalloc
    assert f(ctypes.byref(w), 9, h, 64, out, out, None) == B.I4D_ERANGE      # batch above 8: no scratch for the MFMA path
    assert f(ctypes.byref(w), 0, h, 64, out, out, None) == B.I4D_ERANGE
    assert f(ctypes.byref(w), 1, h, 0, out, out, None) == B.I4D_ERANGE       # chunk_rows must be positive
    assert f(ctypes.byref(w), 1, None, 64, out, out, None) == B.I4D_EINVAL
    assert f(ctypes.byref(w), 1, ctypes.c_void_p(0x100004), 64, out, out, None) == B.I4D_EALIGN
    assert f(ctypes.byref(_mat(1000, 256, dtype=B.WEIGHT_BF16)), 1, h, 64, out, out, None) == B.I4D_EINVAL
    assert f(None, 1, h, 64, out, out, None) == B.I4D_EINVAL


def test_binding_raises_with_status():
    with pytest.raises(B.I4DError) as e:
        B._check(B.I4D_EALIGN, "x")
    assert e.value.code == B.I4D_EALIGN


def test_ws_min_bytes_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define I4D_WS_MIN_BYTES \((\d+) \+ (\d+) \* (\d+) \* (\d+)\)", text)
    assert m, "I4D_WS_MIN_BYTES not found"
    a, b, c, d = map(int, m.groups())
    assert B.WS_MIN_BYTES == a + b * c * d


def test_launch_timing_validation(lib):
    ms, n = ctypes.c_float(1.0), ctypes.c_int32(7)
    assert lib.i4d_launch_timing_start(0, 10) == B.I4D_EINVAL
    assert lib.i4d_launch_timing_start(8, 10) == B.I4D_EINVAL
    assert lib.i4d_launch_timing_start(B.TIME_KERNELS["gate_up"], 0) == B.I4D_EINVAL
    assert lib.i4d_launch_timing_start(B.TIME_KERNELS["gate_up"], 65537) == B.I4D_EINVAL
    assert lib.i4d_launch_timing_stop(None, ctypes.byref(n)) == B.I4D_EINVAL
    # nothing was timed: no event is read
    assert lib.i4d_launch_timing_stop(ctypes.byref(ms), ctypes.byref(n)) == B.I4D_OK
    assert n.value == 0 and ms.value == 0.0


def test_time_kernel_ids_match_header():
    text = open(HEADER).read()
    ids = {m.group(1).lower(): int(m.group(2)) for m in re.finditer(r"#define I4D_TIME_(\w+)\s+(\d+)", text)}
    assert ids == B.TIME_KERNELS


def test_embed_and_decode_step_validation(lib):
    """Every check happens before anything is enqueued (no GPU is touched:
    each call returns an error code)."""
    cfg = _cfg()
    L = _layer(cfg)
    kv = B.I4dKv(0x500000, 0x600000, 256)
    lm = _mat(1000, 256)
    P = ctypes.c_void_p
    tok, mx, pos, xb, ws, emb = P(0x700000), P(0x710000), P(0x720000), P(0x800000), P(0x400000), P(0x900000)

    def step(cfg=cfg, layer=L, emb=emb, lm=lm, batch=1, tokens=tok, pos=pos, xb=xb, ws_bytes=1 << 30, max_pos=127):
        return lib.i4d_decode_step(ctypes.byref(cfg), 1, ctypes.byref(layer), emb, ctypes.byref(lm), batch, tokens, mx,
                                   pos, max_pos, xb, ctypes.byref(kv), ws, ws_bytes, None)

    assert step(emb=None) == B.I4D_EINVAL
    assert step(tokens=None) == B.I4D_EINVAL
    assert step(pos=None) == B.I4D_EINVAL
    assert step(lm=_mat(1000, 128)) == B.I4D_EINVAL             # LM head width != d_model
    assert step(emb=P(0x900001)) == B.I4D_EALIGN
    assert step(batch=33) == B.I4D_ERANGE
    assert step(max_pos=256) == B.I4D_ERANGE                    # max_pos >= capacity
    assert step(xb=P(0x800004)) == B.I4D_EALIGN
    assert step(ws_bytes=100) == B.I4D_EWORKSPACE
    assert lib.i4d_embed(None, 10, 256, 1, tok, xb, ws, 1 << 20, None) == B.I4D_EINVAL
    assert lib.i4d_embed(emb, 0, 256, 1, tok, xb, ws, 1 << 20, None) == B.I4D_EINVAL
    assert lib.i4d_embed(emb, 10, 256, 0, tok, xb, ws, 1 << 20, None) == B.I4D_ERANGE
    assert lib.i4d_embed(emb, 10, 256, 1, tok, xb, ws, 100, None) == B.I4D_EWORKSPACE


def test_sampling_validation(lib):
    """Temperature and counter checks of the sampling entry points; every call
    here fails validation before anything is enqueued."""
    w = _mat(1000, 256)
    P = ctypes.c_void_p
    h, out, ws, ctr = P(0x100000), P(0x200000), P(0x400000), P(0x300000)

    def lm(temperature=1.0, counter=ctr, chunk=64, batch=1):
        return lib.i4d_lm_head_sample(ctypes.byref(w), batch, h, chunk, temperature, 12345, counter, out, out, ws,
                                      1 << 20, None)

    for t in (0.0, -1.0, float("nan"), float("inf"), 1e-39, 3e38):     # 1e-39: 1/T overflows; 3e38: 1/T subnormal
        assert lm(temperature=t) == B.I4D_EINVAL, t
    assert lm(counter=None) == B.I4D_EINVAL
    assert lm(counter=P(0x300002)) == B.I4D_EALIGN
    assert lm(chunk=0) == B.I4D_ERANGE                                # valid sampler, then the LM head's own checks
    assert lm(batch=33) == B.I4D_ERANGE
    cfg = _cfg()
    L = _layer(cfg)
    kv = B.I4dKv(0x500000, 0x600000, 256)
    tok, pos, xb, emb = P(0x700000), P(0x720000), P(0x800000), P(0x900000)

    def step(temperature=0.8, pos=pos, max_pos=127):
        return lib.i4d_decode_step_sample(ctypes.byref(cfg), 1, ctypes.byref(L), emb, ctypes.byref(w), 1, tok, out, pos,
                                          max_pos, xb, ctypes.byref(kv), temperature, 7, ws, 1 << 30, None)

    assert step(pos=None) == B.I4D_EINVAL
    assert step(temperature=0.0) == B.I4D_EINVAL
    assert step(max_pos=256) == B.I4D_ERANGE


def test_paged_kv_validation(lib):
    """Page-table fields are checked on the host before anything is enqueued."""
    cfg = _cfg()
    layer = _layer(cfg)

    def call(pages=0x300000, page_size=32, n_pages=8, cap=256):
        kv = B.I4dKv(0x500000, 0x600000, cap, pages, page_size, n_pages)
        return lib.i4d_decode_layer(ctypes.byref(cfg), ctypes.byref(layer), 1, ctypes.c_void_p(0x100000),
                                    ctypes.c_void_p(0x200000), ctypes.byref(kv), ctypes.c_void_p(0x700000), 127,
                                    ctypes.c_void_p(0x400000), 16, None)

    assert call(page_size=24) == B.I4D_EINVAL          # not a multiple of 16
    assert call(page_size=0) == B.I4D_EINVAL
    assert call(page_size=96) == B.I4D_EINVAL          # capacity 256 is not a multiple of 96
    assert call(n_pages=0) == B.I4D_EINVAL
    assert call(pages=0x300002) == B.I4D_EALIGN
    assert call() == B.I4D_EWORKSPACE                  # a valid table: the next check (a 16-byte workspace) fails


def test_prefill_chunk_validation(lib):
    """Chunk width 1..32; the persistent mode does not take prompt chunks.
    Every call fails validation before anything is enqueued."""
    P = ctypes.c_void_p

    def call(cfg, n_tokens=8):
        layer = _layer(cfg)
        kv = B.I4dKv(0x500000, 0x600000, 256)
        return lib.i4d_prefill_chunk(ctypes.byref(cfg), 1, ctypes.byref(layer), n_tokens, P(0x100000), P(0x200000),
                                     ctypes.byref(kv), P(0x700000), 127, P(0x400000), 1 << 30, None)

    assert call(_cfg(), n_tokens=0) == B.I4D_ERANGE
    assert call(_cfg(), n_tokens=33) == B.I4D_ERANGE
    assert call(_cfg(exec_mode=2)) == B.I4D_EUNSUPPORTED


def test_prefill_validation(lib):
    """Whole-prompt prefill: token count, first position, alignment, cache
    capacity, workspace size and the matrix-core weight conditions are all
    checked before anything is enqueued."""
    P = ctypes.c_void_p
    cfg_ok = _cfg(d_model=512, d_ff=1024, head_dim=128, n_q_heads=4, n_kv_heads=2)

    def call(cfg, n_tokens=64, pos0=0, cap=256, x_in=0x100000, ws_bytes=1 << 40, group=128):
        layer = _layer(cfg, group=group)
        kv = B.I4dKv(0x500000, 0x600000, cap)
        return lib.i4d_prefill(ctypes.byref(cfg), 1, ctypes.byref(layer), n_tokens, P(x_in), P(0x200000),
                               ctypes.byref(kv), pos0, P(0x400000), ws_bytes, None)

    assert call(cfg_ok, n_tokens=0) == B.I4D_ERANGE
    assert call(cfg_ok, n_tokens=65537) == B.I4D_ERANGE
    assert call(cfg_ok, pos0=-1) == B.I4D_ERANGE
    assert call(cfg_ok, x_in=0x100004) == B.I4D_EALIGN
    assert call(cfg_ok, ws_bytes=16) == B.I4D_EWORKSPACE
    assert call(cfg_ok, n_tokens=200, pos0=100, cap=288) == B.I4D_ERANGE      # last position 299 >= capacity
    assert call(_cfg()) == B.I4D_EUNSUPPORTED                                  # d_ff 688: not a multiple of 256
    assert call(cfg_ok, group=64) == B.I4D_EUNSUPPORTED                        # groups of 64
    assert call(_cfg(head_dim=96)) == B.I4D_EINVAL
    n1 = B.prefill_workspace_size(cfg_ok, 1)
    assert 0 < n1 < B.prefill_workspace_size(cfg_ok, 512) < B.prefill_workspace_size(cfg_ok, 4096)
    assert B.prefill_workspace_size(cfg_ok, 0) == 0
    assert B.prefill_workspace_size(cfg_ok, 65537) == 0


def test_topk_sampling_validation(lib):
    """Top-k sampling: k range, temperature, the merge bound and the workspace
    size are checked before anything is enqueued."""
    P = ctypes.c_void_p
    w = _mat(151936, 512, 128)

    def call(top_k=40, T=0.8, batch=1, ws_bytes=1 << 40, mat=w):
        return lib.i4d_lm_head_sample_topk(ctypes.byref(mat), batch, P(0x100000), top_k, ctypes.c_float(T),
                                           ctypes.c_uint64(7), P(0x300000), P(0x200000), P(0x210000), P(0x400000),
                                           ws_bytes, None)

    assert call(top_k=0) == B.I4D_ERANGE
    assert call(top_k=65) == B.I4D_ERANGE
    assert call(T=0.0) == B.I4D_EINVAL
    assert call(T=float("inf")) == B.I4D_EINVAL
    assert call(batch=33) == B.I4D_ERANGE
    assert call(ws_bytes=16) == B.I4D_EWORKSPACE
    assert call(mat=_mat(300000, 512, 128), top_k=64) == B.I4D_EUNSUPPORTED    # 293 slices x 64 > 16384
    n1 = B.topk_workspace_size(w, 1, 40)
    assert n1 >= 151936 * 4 and B.topk_workspace_size(w, 4, 40) > n1
    assert B.topk_workspace_size(w, 1, 0) == 0 and B.topk_workspace_size(w, 1, 65) == 0
