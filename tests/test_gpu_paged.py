"""Paged KV caches (the i4d_kv page table) through the C ABI.

Each sequence's positions live in pages of a shared pool, in a shuffled order
with unused pages poisoned by NaN.  The layer, the stack and a prompt chunk
must give bit-identical outputs to the same call on contiguous caches (the
arithmetic is the same, only the addresses differ).  They must also match the
oracle to the usual bar, the appended slot must land in its mapped page, and
every other byte of the pool must stay unchanged.  A page id outside the pool
is never dereferenced: attention reads page 0, the append is dropped, and the
status word gets I4D_DEV_BAD_PAGE.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from int4_weight_streaming_decode_amd import binding as B
from tests.gpu_util import (DevKV, DevLayer, assert_close, config_of, dev, host_u16, k_from_tiles, k_to_tiles,
                            v_from_tiles, v_to_tiles, workspace)

pytestmark = pytest.mark.gpu

SHAPE = synth.SHAPES["tiny"].with_(name="paged", d_model=512, n_q_heads=4, n_kv_heads=2, head_dim=128, d_ff=1024,
                                   group=128, rope_base=1e6)
SHAPE64 = synth.SHAPES["tiny"].with_(name="paged_hd64", d_model=768, n_q_heads=8, n_kv_heads=2, head_dim=64,
                                     d_ff=1536, group=128, rope_base=1e4)
NAN16 = np.uint16(0x7FC0)


def _print_case(*a):
    print("CASE", *a, flush=True)


class DevPagedKV:
    """Contiguous caches [B][Hkv][cap][hd] scattered into a pool of pages of P
    positions (page order shuffled, `extra` unused pages poisoned)."""

    def __init__(self, kc, vc, P, seed, extra=3):
        b, h, cap, hd = kc.shape
        self.P, self.pps, self.shape = P, cap // P, kc.shape
        self.n_pages = b * self.pps + extra
        rng = np.random.default_rng(seed)
        self.table = rng.permutation(self.n_pages)[: b * self.pps].reshape(b, self.pps).astype(np.int32)
        kp = np.full((self.n_pages, h, P, hd), NAN16, dtype=np.uint16)
        vp = np.full((self.n_pages, h, P, hd), NAN16, dtype=np.uint16)
        for s in range(b):
            for i in range(self.pps):
                kp[self.table[s, i]] = kc[s, :, i * P:(i + 1) * P]
                vp[self.table[s, i]] = vc[s, :, i * P:(i + 1) * P]
        self.k = dev(k_to_tiles(kp))
        self.v = dev(v_to_tiles(vp))
        self.pages = dev(self.table)
        self.kv = B.make_kv(self.k, self.v, cap, self.pages, P, self.n_pages)

    def pools(self):
        b, h, cap, hd = self.shape
        ps = (self.n_pages, h, self.P, hd)
        return k_from_tiles(host_u16(self.k), ps), v_from_tiles(host_u16(self.v), ps)

    def gather(self):
        """The pool read back as contiguous [B][Hkv][cap][hd] caches."""
        kp, vp = self.pools()
        kc = np.concatenate([kp[self.table[:, i]] for i in range(self.pps)], axis=2)
        vc = np.concatenate([vp[self.table[:, i]] for i in range(self.pps)], axis=2)
        return kc, vc


@pytest.mark.parametrize("shape,batch,P", [(SHAPE, 3, 32), (SHAPE, 16, 64), (SHAPE64, 5, 16), (SHAPE64, 20, 32)])
def test_paged_layer_equals_contiguous_and_oracle(shape, batch, P):
    rng = np.random.default_rng(batch * 7 + P)
    cap = 320
    pos = [int(p) for p in rng.integers(0, cap - 1, size=batch)]
    pos[0] = cap - 1
    _print_case("paged decode_layer", shape.name, batch, P, pos[:4])
    layer = synth.make_layer(shape, 50 + batch, 0)
    kc, vc = synth.make_kv(shape, 50 + batch, 0, batch, pos, cap)
    x = synth.make_x(shape, 50 + batch, batch)
    L = DevLayer(layer)
    cfg = config_of(shape)
    outs = []
    for paged in (False, True):
        kvd = DevPagedKV(kc, vc, P, seed=batch) if paged else DevKV(kc, vc)
        before = kvd.pools() if paged else None
        ws = workspace(cfg, batch, max(pos))
        out = torch.full((batch, shape.d_model), float("nan"), dtype=torch.float32, device="cuda")
        B.decode_layer(cfg, L.layer, batch, dev(x), out, kvd.kv, dev(np.array(pos, dtype=np.int32)), max(pos), ws)
        torch.cuda.synchronize()
        assert B.read_device_status(ws) == 0
        outs.append((out.cpu().numpy(), kvd.gather() if paged else kvd.host()))
        if paged:
            after = kvd.pools()
            changed = np.zeros(after[0].shape[:1] + after[0].shape[2:3], dtype=bool)     # [page][slot]
            for b, p in enumerate(pos):
                changed[kvd.table[b, p // P], p % P] = True
            for name, a0, a1 in (("K", before[0], after[0]), ("V", before[1], after[1])):
                diff_slots = np.any(a0 != a1, axis=(1, 3))                           # [page][slot], raw bits
                assert not np.any(diff_slots & ~changed), f"{name}: pool bytes outside the appended slots changed"
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32)), "paged output differs from contiguous"
    for c in range(2):
        assert np.array_equal(outs[0][1][c], outs[1][1][c]), "paged cache differs from contiguous"
    ref = oracle.decode_layer(shape, layer, x.astype(np.float64), kc, vc, pos)
    assert_close(outs[1][0], ref["z"], what="paged layer")


def test_paged_stack_and_prefill_equal_contiguous():
    shape, batch, P, cap, n_layers = SHAPE, 4, 48, 240, 2
    pos = [100, 7, 239, 64]
    _print_case("paged stack + prefill", batch, P)
    layers = [synth.make_layer(shape, 70, l) for l in range(n_layers)]
    caches = [synth.make_kv(shape, 70, l, batch, pos, cap) for l in range(n_layers)]
    x = synth.make_x(shape, 70, batch)
    Ls = [DevLayer(l) for l in layers]
    cfg = config_of(shape)
    res = []
    for paged in (False, True):
        kvs = [DevPagedKV(*c, P, seed=l) if paged else DevKV(*c) for l, c in enumerate(caches)]
        ws = workspace(cfg, 5, max(pos), n_layers=n_layers)             # 5: the prompt chunk's width
        out = torch.empty((batch, shape.d_model), dtype=torch.float32, device="cuda")
        B.decode_stack(cfg, [l.layer for l in Ls], batch, dev(x), out, [k.kv for k in kvs], dev(np.array(pos, dtype=np.int32)),
                       max(pos), ws)
        # a prompt chunk of 5 tokens for sequence 1 (positions 8..12) on the updated caches
        xp = synth.make_x(shape, 71, 5)
        outp = torch.empty((5, shape.d_model), dtype=torch.float32, device="cuda")
        if paged:
            one = [B.make_kv(k.k, k.v, cap, k.pages[1:2], P, k.n_pages) for k in kvs]     # sequence 1's table row
        else:
            one = [B.make_kv(k.k[1:2], k.v[1:2], cap) for k in kvs]
        B.prefill_chunk(cfg, [l.layer for l in Ls], 5, dev(xp), outp, one, dev(np.arange(8, 13, dtype=np.int32)), 12, ws)
        torch.cuda.synchronize()
        assert B.read_device_status(ws) == 0
        res.append((out.cpu().numpy(), outp.cpu().numpy(), [k.gather() if paged else k.host() for k in kvs]))
    for i in range(2):
        assert np.array_equal(res[0][i].view(np.uint32), res[1][i].view(np.uint32)), f"output {i} differs"
    for l in range(n_layers):
        for c in range(2):
            assert np.array_equal(res[0][2][l][c], res[1][2][l][c]), f"layer {l} cache {c} differs"
    ref = oracle.decode_stack(shape, layers, x.astype(np.float64), caches, pos)
    assert_close(res[1][0], ref["z"], what="paged stack")


def test_page_id_outside_the_pool_is_not_dereferenced():
    """One table entry points past the pool: the kernels read page 0 instead
    and drop that append; the status word reports it."""
    shape, batch, P, cap = SHAPE, 2, 32, 128
    pos = [100, 50]
    _print_case("paged bad page id", batch, P)
    layer = synth.make_layer(shape, 90, 0)
    kc, vc = synth.make_kv(shape, 90, 0, batch, pos, cap)
    kvd = DevPagedKV(kc, vc, P, seed=9)
    table = kvd.table.copy()
    table[0, 100 // P] = kvd.n_pages + 1000          # the page holding sequence 0's new slot
    kvd.pages.copy_(torch.from_numpy(table).cuda())
    before = kvd.pools()
    ws = workspace(config_of(shape), batch, max(pos))
    out = torch.empty((batch, shape.d_model), dtype=torch.float32, device="cuda")
    B.decode_layer(config_of(shape), DevLayer(layer).layer, batch, dev(synth.make_x(shape, 90, batch)), out, kvd.kv,
                   dev(np.array(pos, dtype=np.int32)), max(pos), ws)
    torch.cuda.synchronize()
    assert B.read_device_status(ws) & B.I4D_DEV_BAD_PAGE
    after = kvd.pools()
    # only sequence 1's appended slot changed anywhere in the pool
    for a0, a1 in ((before[0], after[0]), (before[1], after[1])):
        diff = np.argwhere(np.any(a0 != a1, axis=(1, 3)))
        assert [tuple(d) for d in diff] == [(kvd.table[1, 50 // P], 50 % P)]


@pytest.mark.parametrize("name,pos,P", [("27b", [20000], 256), ("tiny", [16000, 13000, 9000, 15000], 64)])
def test_paged_attention_over_several_rounds(name, pos, P):
    """Splits long enough that each wave loads its subtiles in more than one
    round, so the page ids of every later round come from the read issued a
    round ahead.  Bit-identical to the contiguous cache and within the bar of
    the oracle."""
    from tests.test_gpu_parity import _attn_case
    shape = synth.SHAPES[name]
    batch = len(pos)
    _print_case("paged attention, several rounds", name, pos, P)
    q, kc, vc = _attn_case(shape, batch, pos, seed=sum(pos))
    pad = -kc.shape[2] % P                            # capacity to a whole number of pages (poisoned slots)
    kc = np.pad(kc, ((0, 0), (0, 0), (0, pad), (0, 0)), constant_values=NAN16)
    vc = np.pad(vc, ((0, 0), (0, 0), (0, pad), (0, 0)), constant_values=NAN16)
    cfg = config_of(shape)
    ws = workspace(cfg, batch, max(pos))
    outs = []
    for kvd in (DevKV(kc, vc), DevPagedKV(kc, vc, P, seed=3)):
        o = torch.full((batch, shape.n_q_heads, shape.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        B.attention(cfg, batch, dev(q), kvd.kv, dev(np.array(pos, dtype=np.int32)), max(pos), o, ws)
        torch.cuda.synchronize()
        assert B.read_device_status(ws) == 0
        outs.append(o.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), "paged attention differs from contiguous"
    ref = oracle.gqa_decode_attention(q.astype(np.float64), kc, vc, pos)
    for b in range(batch):
        assert_close(outs[1][b], ref[b], what=f"paged attention b={b}")


@pytest.mark.parametrize("n_tokens", [24, 32])
def test_paged_prefill_on_the_matrix_cores_equals_contiguous(n_tokens):
    """A prompt chunk of 24 or 32 tokens (matrix-core path, every entry sharing
    one cache) written through a page table: bit-identical to the contiguous
    cache, and equal to the oracle decoding the tokens one after another."""
    shape, P, cap, start = SHAPE, 32, 128, 40
    _print_case("paged prefill", n_tokens, P)
    layers = [synth.make_layer(shape, 110, 0)]
    kc, vc = synth.make_kv(shape, 110, 0, 1, [start], cap)
    x = synth.make_x(shape, 111, n_tokens)
    pos = np.arange(start, start + n_tokens, dtype=np.int32)
    L = DevLayer(layers[0])
    cfg = config_of(shape)
    res = []
    for paged in (False, True):
        kvd = DevPagedKV(kc, vc, P, seed=n_tokens) if paged else DevKV(kc, vc)
        ws = workspace(cfg, n_tokens, cap - 1)
        out = torch.empty((n_tokens, shape.d_model), dtype=torch.float32, device="cuda")
        B.prefill_chunk(cfg, [L.layer], n_tokens, dev(x), out, [kvd.kv], dev(pos), int(pos[-1]), ws)
        torch.cuda.synchronize()
        assert B.read_device_status(ws) == 0
        res.append((out.cpu().numpy(), kvd.gather() if paged else kvd.host()))
    assert np.array_equal(res[0][0].view(np.uint32), res[1][0].view(np.uint32)), "paged prefill output differs"
    for c in range(2):
        assert np.array_equal(res[0][1][c], res[1][1][c]), "paged prefill cache differs"
    caches = [(kc, vc)]
    for t in range(n_tokens):
        r = oracle.decode_stack(shape, layers, x[t:t + 1].astype(np.float64), caches, [int(pos[t])])
        caches = r["caches"]
        assert_close(res[1][0][t], r["z"][0], what=f"paged prefill token {t}")


@pytest.mark.parametrize("n_tokens,pos0,P", [(200, 40, 32), (333, 0, 64)])
def test_paged_whole_prompt_prefill_equals_contiguous(n_tokens, pos0, P):
    """i4d_prefill (GEMMs over the prompt, causal prompt attention) on a paged
    cache: outputs and caches bit-identical to the contiguous call, outputs to
    the oracle's bar, and unused pages untouched."""
    shape = SHAPE
    cap = ((pos0 + n_tokens + P - 1) // P + 1) * P
    _print_case("paged whole-prompt prefill", n_tokens, pos0, P)
    layers = [synth.make_layer(shape, 97, l) for l in range(2)]
    caches = [synth.make_kv(shape, 97, l, 1, [pos0], cap) for l in range(2)]
    x = np.stack([synth.make_x(shape, 97, 1, step=t)[0] for t in range(n_tokens)])
    Ls = [DevLayer(l) for l in layers]
    cfg = config_of(shape)
    res = []
    for paged in (False, True):
        kvs = [DevPagedKV(kc, vc, P, seed=n_tokens + l) if paged else DevKV(kc, vc) for l, (kc, vc) in enumerate(caches)]
        before = [k.pools() for k in kvs] if paged else None
        ws = torch.zeros(B.prefill_workspace_size(cfg, n_tokens), dtype=torch.uint8, device="cuda")
        B.workspace_init(ws)
        out = torch.empty((n_tokens, shape.d_model), dtype=torch.float32, device="cuda")
        B.prefill(cfg, [l.layer for l in Ls], n_tokens, dev(x), out, [k.kv for k in kvs], pos0, ws)
        torch.cuda.synchronize()
        assert B.read_device_status(ws) == 0
        res.append((out.cpu().numpy(), [k.gather() if paged else k.host() for k in kvs]))
        if paged:
            for k, (kb, vb) in zip(kvs, before):
                used = set(k.table.ravel().tolist())
                ka, va = k.pools()
                for pg in range(k.n_pages):
                    if pg not in used:
                        assert np.array_equal(ka[pg], kb[pg]) and np.array_equal(va[pg], vb[pg]), f"unused page {pg}"
    assert np.array_equal(res[0][0].view(np.uint32), res[1][0].view(np.uint32)), "paged prefill output differs"
    for l in range(2):
        for c in range(2):
            assert np.array_equal(res[0][1][l][c], res[1][1][l][c]), f"layer {l} cache {c} differs"
    ref = oracle.prefill(shape, layers, x.astype(np.float64), caches, pos0)
    for t in range(0, n_tokens, 37):
        assert_close(res[1][0][t], ref["z"][t], what=f"paged prefill token {t}")


def test_prefill_with_a_page_id_outside_the_pool():
    """A prompt prefill whose table points one page past the pool: the GEMM
    epilogue drops the appends into that page, the prompt attention reads page
    0 in its place (so the outputs are not meaningful), the status word
    reports it, and no page changes except at the slots the prompt appends
    into valid pages."""
    shape, P, n, pos0 = SHAPE, 32, 80, 20
    cap = 128
    _print_case("paged prefill bad page id", n, pos0, P)
    layer = synth.make_layer(shape, 91, 0)
    kc, vc = synth.make_kv(shape, 91, 0, 1, [pos0], cap)
    kvd = DevPagedKV(kc, vc, P, seed=19)
    table = kvd.table.copy()
    bad = 64 // P                                    # logical page 2: slots 64..95, inside the prompt
    table[0, bad] = kvd.n_pages + 1000
    kvd.pages.copy_(torch.from_numpy(table).cuda())
    before = kvd.pools()
    x = np.stack([synth.make_x(shape, 91, 1, step=t)[0] for t in range(n)])
    cfg = config_of(shape)
    ws = torch.zeros(B.prefill_workspace_size(cfg, n), dtype=torch.uint8, device="cuda")
    B.workspace_init(ws)
    out = torch.empty((n, shape.d_model), dtype=torch.float32, device="cuda")
    B.prefill(cfg, [DevLayer(layer).layer], n, dev(x), out, [kvd.kv], pos0, ws)
    torch.cuda.synchronize()
    assert B.read_device_status(ws) & B.I4D_DEV_BAD_PAGE      # the outputs are not meaningful then
    after = kvd.pools()
    # changed (page, slot) pairs: exactly the prompt's slots that map to valid pages
    want = sorted((int(kvd.table[0, s // P]), s % P) for s in range(pos0, pos0 + n) if s // P != bad)
    for a0, a1 in ((before[0], after[0]), (before[1], after[1])):
        diff = sorted(tuple(int(v) for v in d) for d in np.argwhere(np.any(a0 != a1, axis=(1, 3))))
        assert diff == want
