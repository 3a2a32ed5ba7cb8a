"""i4d_lm_head_chunked_noalloc (the LM head whose argmax keys live in the
library's own device array) against i4d_lm_head_chunked (keys in the
caller's workspace), through the C ABI.

Both run the same kernels on the same inputs, so tokens and max logits must
agree bit for bit.  Two calls in a row, the second with a smaller vocabulary,
width and batch, check that the array's earlier contents never leak into a
later result; the second call is also checked against the CPU oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from int4_weight_streaming_decode_amd import binding as B
from synth import gpu as G
from tests.gpu_util import assert_close, config_of, workspace

pytestmark = pytest.mark.gpu


def _host_mat(m):
    return {"codes": m["codes"].cpu().numpy(), "scales": m["scales"].cpu().numpy().view(np.uint16),
            "n": m["n"], "k": m["k"], "group": m["group"]}


def _both(vocab, d_model, batch, seed):
    print("CASE noalloc lm head", vocab, d_model, batch, flush=True)
    W = G.make_lm_head_gpu(vocab, d_model, 128, seed)
    mat = B.make_mat(W["codes"], W["scales"], W["n"], W["k"], W["group"], B.WEIGHT_INT4)
    shape = synth.SHAPES["tiny"].with_(d_model=d_model)
    h = G.make_x_gpu(shape, seed + 1, batch)
    ws = workspace(config_of(shape), batch, 0, vocab=vocab)
    tok_ws = torch.full((batch,), -1, dtype=torch.int32, device="cuda")
    mx_ws = torch.full((batch,), float("nan"), dtype=torch.float32, device="cuda")
    tok_na = torch.full((batch,), -1, dtype=torch.int32, device="cuda")
    mx_na = torch.full((batch,), float("nan"), dtype=torch.float32, device="cuda")
    B.lm_head_chunked(mat, batch, h, 4096, tok_ws, mx_ws, ws)
    B.lm_head_chunked_noalloc(mat, batch, h, 4096, tok_na, mx_na)
    torch.cuda.synchronize()
    return W, h, (tok_ws.cpu().numpy(), mx_ws.cpu().numpy()), (tok_na.cpu().numpy(), mx_na.cpu().numpy())


def test_noalloc_lm_head_equals_the_workspace_entry_point():
    # first call: a larger problem fills more of the array
    _, _, (t1, m1), (t2, m2) = _both(40000, 2048, 8, 11)
    assert np.array_equal(t1, t2), (t1, t2)
    assert np.array_equal(m1.view(np.uint32), m2.view(np.uint32))
    assert np.all(t2 >= 0) and np.all(t2 < 40000)
    # second call, smaller: vocabulary, width and batch all shrink
    W, h, (t1, m1), (t2, m2) = _both(3001, 512, 3, 12)
    assert np.array_equal(t1, t2), (t1, t2)
    assert np.array_equal(m1.view(np.uint32), m2.view(np.uint32))
    tok_ref, mx_ref, logits = oracle.lm_head_argmax(_host_mat(W), h.cpu().numpy().astype(np.float64))
    for b in range(3):
        srt = np.sort(logits[b])
        rms = np.sqrt(np.mean(logits[b] ** 2))
        if srt[-1] - srt[-2] > 1e-3 * rms:
            assert t2[b] == tok_ref[b]
        else:
            assert logits[b][t2[b]] >= srt[-1] - 1e-3 * rms
    assert_close(m2, mx_ref, what="no-alloc LM head max logit")


def test_noalloc_lm_head_rejects_batches_above_8():
    W = G.make_lm_head_gpu(1000, 256, 128, 3)
    mat = B.make_mat(W["codes"], W["scales"], W["n"], W["k"], W["group"], B.WEIGHT_INT4)
    h = torch.zeros((9, 256), dtype=torch.float32, device="cuda")
    tok = torch.empty((9,), dtype=torch.int32, device="cuda")
    mx = torch.empty((9,), dtype=torch.float32, device="cuda")
    with pytest.raises(B.I4DError):
        B.lm_head_chunked_noalloc(mat, 9, h, 64, tok, mx)
