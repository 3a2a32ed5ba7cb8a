"""ctypes binding of libi4decode.so (include/i4decode.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of the library.  Tensors are torch device tensors; their data pointers
and torch's current HIP stream are handed to the C entry points, which return a
status code that is turned into an exception here.  The library is loaded on
first use; if it has not been built, loading raises.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libi4decode.so")

I4D_OK = 0
I4D_EINVAL = -1
I4D_EALIGN = -2
I4D_EWORKSPACE = -3
I4D_ERANGE = -4
I4D_EHIP = -5
I4D_EUNSUPPORTED = -6
WS_MIN_BYTES = 16384 + 4096 * 32 * 8    # I4D_WS_MIN_BYTES
I4D_DEV_BAD_POS = 1
I4D_DEV_BARRIER_TIMEOUT = 2
I4D_DEV_BAD_TOKEN = 4
I4D_DEV_BAD_PAGE = 8
I4D_DEV_NONFINITE = 16

WEIGHT_INT4 = 0
WEIGHT_BF16 = 1

EXEC_AUTO = 0
EXEC_PHASES = 1
EXEC_STREAM = 2


class I4dMat(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("n", ctypes.c_int32), ("k", ctypes.c_int32), ("group", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class I4dLayer(ctypes.Structure):
    _fields_ = [("attn_norm", ctypes.c_void_p), ("wq", I4dMat), ("wk", I4dMat), ("wv", I4dMat), ("wo", I4dMat),
                ("ffn_norm", ctypes.c_void_p), ("wg", I4dMat), ("wu", I4dMat), ("wd", I4dMat)]


class I4dConfig(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_base", ctypes.c_double), ("exec_mode", ctypes.c_int32)]


class I4dKv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("capacity", ctypes.c_int32),
                ("pages", ctypes.c_void_p), ("page_size", ctypes.c_int32), ("n_pages", ctypes.c_int32)]


class I4DError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: status {code} ({status_string(code)})")


_lib = None


def lib():
    """The loaded library; raises if libi4decode.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() (hipcc for gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.i4d_workspace_size.argtypes = [ctypes.POINTER(I4dConfig), I, I, I, I]
        L.i4d_workspace_size.restype = Z
        L.i4d_workspace_init.argtypes = [P, Z, P]
        L.i4d_decode_layer.argtypes = [ctypes.POINTER(I4dConfig), ctypes.POINTER(I4dLayer), I, P, P,
                                       ctypes.POINTER(I4dKv), P, I, P, Z, P]
        L.i4d_decode_stack.argtypes = [ctypes.POINTER(I4dConfig), I, ctypes.POINTER(I4dLayer), I, P, P,
                                       ctypes.POINTER(I4dKv), P, I, P, Z, P]
        L.i4d_lm_head_chunked.argtypes = [ctypes.POINTER(I4dMat), I, P, I, P, P, P, Z, P]
        L.i4d_lm_head_chunked_noalloc.argtypes = [ctypes.POINTER(I4dMat), I, P, I, P, P, P]
        L.i4d_lm_head_sample.argtypes = [ctypes.POINTER(I4dMat), I, P, I, ctypes.c_float, ctypes.c_uint64, P, P, P, P, Z, P]
        L.i4d_dequant_int4.argtypes = [ctypes.POINTER(I4dMat), P, P]
        L.i4d_embed.argtypes = [P, I, I, I, P, P, P, Z, P]
        L.i4d_prefill_chunk.argtypes = [ctypes.POINTER(I4dConfig), I, ctypes.POINTER(I4dLayer), I, P, P,
                                        ctypes.POINTER(I4dKv), P, I, P, Z, P]
        L.i4d_decode_step_sample_topk.argtypes = [ctypes.POINTER(I4dConfig), I, ctypes.POINTER(I4dLayer), P,
                                                  ctypes.POINTER(I4dMat), I, P, P, P, I, P, ctypes.POINTER(I4dKv), I,
                                                  ctypes.c_float, ctypes.c_uint64, P, Z, P]
        L.i4d_topk_workspace_size.argtypes = [ctypes.POINTER(I4dMat), I, I]
        L.i4d_topk_workspace_size.restype = Z
        L.i4d_lm_head_sample_topk.argtypes = [ctypes.POINTER(I4dMat), I, P, I, ctypes.c_float, ctypes.c_uint64, P, P, P, P,
                                              Z, P]
        L.i4d_prefill_workspace_size.argtypes = [ctypes.POINTER(I4dConfig), I]
        L.i4d_prefill_workspace_size.restype = Z
        L.i4d_prefill.argtypes = [ctypes.POINTER(I4dConfig), I, ctypes.POINTER(I4dLayer), I, P, P, ctypes.POINTER(I4dKv), I,
                                  P, Z, P]
        L.i4d_decode_step.argtypes = [ctypes.POINTER(I4dConfig), I, ctypes.POINTER(I4dLayer), P, ctypes.POINTER(I4dMat), I,
                                      P, P, P, I, P, ctypes.POINTER(I4dKv), P, Z, P]
        L.i4d_decode_step_sample.argtypes = [ctypes.POINTER(I4dConfig), I, ctypes.POINTER(I4dLayer), P,
                                             ctypes.POINTER(I4dMat), I, P, P, P, I, P, ctypes.POINTER(I4dKv),
                                             ctypes.c_float, ctypes.c_uint64, P, Z, P]
        L.i4d_gemv.argtypes = [ctypes.POINTER(I4dMat), I, P, P, P, Z, P]
        L.i4d_attention.argtypes = [ctypes.POINTER(I4dConfig), I, P, ctypes.POINTER(I4dKv), P, I, P, P, Z, P]
        L.i4d_read_device_status.argtypes = [P, ctypes.POINTER(ctypes.c_int32), P]
        L.i4d_launch_timing_start.argtypes = [I, I]
        L.i4d_launch_timing_stop.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32)]
        L.i4d_read_probe.argtypes = [P, Z, P, P]
        L.i4d_status_string.argtypes = [ctypes.c_int]
        L.i4d_status_string.restype = ctypes.c_char_p
        for name in ("i4d_workspace_init", "i4d_decode_layer", "i4d_decode_stack", "i4d_lm_head_chunked", "i4d_embed",
                     "i4d_decode_step", "i4d_prefill_chunk", "i4d_lm_head_sample", "i4d_decode_step_sample",
                     "i4d_dequant_int4", "i4d_gemv", "i4d_attention", "i4d_read_device_status",
                     "i4d_launch_timing_start", "i4d_launch_timing_stop", "i4d_read_probe",
                     "i4d_lm_head_chunked_noalloc", "i4d_prefill", "i4d_lm_head_sample_topk",
                     "i4d_decode_step_sample_topk"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().i4d_status_string(int(code)).decode()


def _check(rc: int, where: str):
    if rc != I4D_OK:
        raise I4DError(rc, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ------------------------------------------------------------------ struct builders

def make_config(d_model, n_q_heads, n_kv_heads, head_dim, d_ff, rms_eps, rope_base, exec_mode=EXEC_AUTO) -> I4dConfig:
    return I4dConfig(d_model, n_q_heads, n_kv_heads, head_dim, d_ff, rms_eps, rope_base, exec_mode)


def make_mat(data, scales, n, k, group, dtype=WEIGHT_INT4) -> I4dMat:
    """data/scales: torch tensors (scales None for bf16)."""
    return I4dMat(data.data_ptr(), scales.data_ptr() if scales is not None else None, n, k, group, dtype)


def make_layer(attn_norm, ffn_norm, mats: dict) -> I4dLayer:
    """mats: name -> I4dMat for wq, wk, wv, wo, wg, wu, wd."""
    return I4dLayer(attn_norm.data_ptr(), mats["wq"], mats["wk"], mats["wv"], mats["wo"],
                    ffn_norm.data_ptr(), mats["wg"], mats["wu"], mats["wd"])


def make_kv(k_cache, v_cache, capacity, pages=None, page_size=0, n_pages=0) -> I4dKv:
    """Contiguous cache, or (pages: device int32 [B][capacity / page_size]) a paged pool of n_pages pages."""
    return I4dKv(k_cache.data_ptr(), v_cache.data_ptr(), capacity, pages.data_ptr() if pages is not None else None,
                 page_size, n_pages)


# ------------------------------------------------------------------ entry points (same names as the C ABI)

def workspace_size(cfg: I4dConfig, n_layers: int, batch: int, max_pos: int, vocab: int = 0) -> int:
    return int(lib().i4d_workspace_size(ctypes.byref(cfg), n_layers, batch, max_pos, vocab))


def workspace_init(ws, stream=None):
    _check(lib().i4d_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "i4d_workspace_init")


def decode_layer(cfg, layer: I4dLayer, batch, x_in, x_out, kv: I4dKv, pos, max_pos, ws, stream=None):
    _check(lib().i4d_decode_layer(ctypes.byref(cfg), ctypes.byref(layer), batch, _ptr(x_in), _ptr(x_out),
                                  ctypes.byref(kv), _ptr(pos), max_pos, _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)), "i4d_decode_layer")


def decode_stack(cfg, layers, batch, x_in, x_out, kvs, pos, max_pos, ws, stream=None):
    """layers: sequence (or prebuilt ctypes array) of I4dLayer; kvs: likewise of I4dKv."""
    n = len(layers)
    larr = layers if isinstance(layers, ctypes.Array) else (I4dLayer * n)(*layers)
    karr = kvs if isinstance(kvs, ctypes.Array) else (I4dKv * n)(*kvs)
    _check(lib().i4d_decode_stack(ctypes.byref(cfg), n, larr, batch, _ptr(x_in), _ptr(x_out), karr, _ptr(pos),
                                  max_pos, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "i4d_decode_stack")


def lm_head_chunked(w_lm: I4dMat, batch, h, chunk_rows, token_out, max_logit_out, ws, stream=None):
    _check(lib().i4d_lm_head_chunked(ctypes.byref(w_lm), batch, _ptr(h), chunk_rows, _ptr(token_out),
                                     _ptr(max_logit_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "i4d_lm_head_chunked")


def lm_head_chunked_noalloc(w_lm: I4dMat, batch, h, chunk_rows, token_out, max_logit_out, stream=None):
    """Greedy LM head (batch <= 8) with the library's own device scratch: no workspace argument."""
    _check(lib().i4d_lm_head_chunked_noalloc(ctypes.byref(w_lm), batch, _ptr(h), chunk_rows, _ptr(token_out),
                                             _ptr(max_logit_out), _stream(stream)), "i4d_lm_head_chunked_noalloc")


def lm_head_sample(w_lm: I4dMat, batch, h, chunk_rows, temperature, seed, counter, token_out, score_out, ws, stream=None):
    """Gumbel-max draw from softmax(logits / temperature); counter: device int32 [B]."""
    _check(lib().i4d_lm_head_sample(ctypes.byref(w_lm), batch, _ptr(h), chunk_rows, float(temperature), int(seed),
                                    _ptr(counter), _ptr(token_out), _ptr(score_out), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)), "i4d_lm_head_sample")


def prefill_chunk(cfg, layers, n_tokens, x_in, x_out, kvs, pos, max_pos, ws, stream=None):
    """n_tokens prompt tokens of one sequence (x [n][D], positions pos [n] on the device) through the stack."""
    n = len(layers)
    larr = layers if isinstance(layers, ctypes.Array) else (I4dLayer * n)(*layers)
    karr = kvs if isinstance(kvs, ctypes.Array) else (I4dKv * n)(*kvs)
    _check(lib().i4d_prefill_chunk(ctypes.byref(cfg), n, larr, n_tokens, _ptr(x_in), _ptr(x_out), karr, _ptr(pos), max_pos,
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "i4d_prefill_chunk")


def topk_workspace_size(w_lm: I4dMat, batch: int, top_k: int) -> int:
    return int(lib().i4d_topk_workspace_size(ctypes.byref(w_lm), batch, top_k))


def lm_head_sample_topk(w_lm: I4dMat, batch, h, top_k, temperature, seed, counter, token_out, score_out, ws,
                        stream=None):
    _check(lib().i4d_lm_head_sample_topk(ctypes.byref(w_lm), batch, _ptr(h), int(top_k), float(temperature),
                                         int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(counter), _ptr(token_out),
                                         _ptr(score_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "i4d_lm_head_sample_topk")


def prefill_workspace_size(cfg: I4dConfig, n_tokens: int) -> int:
    return int(lib().i4d_prefill_workspace_size(ctypes.byref(cfg), n_tokens))


def prefill(cfg, layers, n_tokens, x_in, x_out, kvs, pos0, ws, stream=None):
    """A whole prompt of one sequence (x [n][D] at positions pos0 .. pos0 + n - 1) through the stack."""
    n = len(layers)
    larr = layers if isinstance(layers, ctypes.Array) else (I4dLayer * n)(*layers)
    karr = kvs if isinstance(kvs, ctypes.Array) else (I4dKv * n)(*kvs)
    _check(lib().i4d_prefill(ctypes.byref(cfg), n, larr, n_tokens, _ptr(x_in), _ptr(x_out), karr, int(pos0), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream)), "i4d_prefill")


def embed(table, vocab, d_model, batch, tokens, x_out, ws, stream=None):
    _check(lib().i4d_embed(_ptr(table), vocab, d_model, batch, _ptr(tokens), _ptr(x_out), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(stream)), "i4d_embed")


def decode_step(cfg, layers, embed_table, w_lm: I4dMat, batch, tokens, max_logit_out, pos, max_pos, x_buf, kvs, ws,
                stream=None):
    """One greedy decode step; tokens (device int32 [B]) are replaced by the next tokens and pos advances by one."""
    n = len(layers)
    larr = layers if isinstance(layers, ctypes.Array) else (I4dLayer * n)(*layers)
    karr = kvs if isinstance(kvs, ctypes.Array) else (I4dKv * n)(*kvs)
    _check(lib().i4d_decode_step(ctypes.byref(cfg), n, larr, _ptr(embed_table), ctypes.byref(w_lm), batch, _ptr(tokens),
                                 _ptr(max_logit_out), _ptr(pos), max_pos, _ptr(x_buf), karr, _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)), "i4d_decode_step")


def decode_step_sample(cfg, layers, embed_table, w_lm: I4dMat, batch, tokens, score_out, pos, max_pos, x_buf, kvs,
                       temperature, seed, ws, stream=None):
    """decode_step with the token drawn at `temperature` (counter word: each sequence's position)."""
    n = len(layers)
    larr = layers if isinstance(layers, ctypes.Array) else (I4dLayer * n)(*layers)
    karr = kvs if isinstance(kvs, ctypes.Array) else (I4dKv * n)(*kvs)
    _check(lib().i4d_decode_step_sample(ctypes.byref(cfg), n, larr, _ptr(embed_table), ctypes.byref(w_lm), batch,
                                        _ptr(tokens), _ptr(score_out), _ptr(pos), max_pos, _ptr(x_buf), karr,
                                        float(temperature), int(seed), _ptr(ws), ws.numel() * ws.element_size(),
                                        _stream(stream)), "i4d_decode_step_sample")


def decode_step_sample_topk(cfg, layers, embed_table, w_lm: I4dMat, batch, tokens, score_out, pos, max_pos, x_buf,
                            kvs, top_k, temperature, seed, ws, stream=None):
    """decode_step with the token drawn by top-k sampling (counter word: each sequence's position)."""
    n = len(layers)
    larr = layers if isinstance(layers, ctypes.Array) else (I4dLayer * n)(*layers)
    karr = kvs if isinstance(kvs, ctypes.Array) else (I4dKv * n)(*kvs)
    _check(lib().i4d_decode_step_sample_topk(ctypes.byref(cfg), n, larr, _ptr(embed_table), ctypes.byref(w_lm), batch,
                                             _ptr(tokens), _ptr(score_out), _ptr(pos), max_pos, _ptr(x_buf), karr,
                                             int(top_k), float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream(stream)),
           "i4d_decode_step_sample_topk")


def dequant_int4(w: I4dMat, out, stream=None):
    _check(lib().i4d_dequant_int4(ctypes.byref(w), _ptr(out), _stream(stream)), "i4d_dequant_int4")


def gemv(w: I4dMat, batch, x, y, ws=None, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().i4d_gemv(ctypes.byref(w), batch, _ptr(x), _ptr(y), _ptr(ws), nbytes, _stream(stream)), "i4d_gemv")


def attention(cfg, batch, q, kv: I4dKv, pos, max_pos, o, ws, stream=None):
    _check(lib().i4d_attention(ctypes.byref(cfg), batch, _ptr(q), ctypes.byref(kv), _ptr(pos), max_pos, _ptr(o),
                               _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "i4d_attention")


# kernels that i4d_launch_timing_start can time (values of I4D_TIME_*)
TIME_KERNELS = {"qkv": 1, "attention": 2, "wo": 3, "gate_up": 4, "down": 5, "lm_head": 6, "stream": 7}


def launch_timing_start(kernel: str, max_launches: int):
    _check(lib().i4d_launch_timing_start(TIME_KERNELS[kernel], int(max_launches)), "i4d_launch_timing_start")


def launch_timing_stop():
    """(summed launch time in ms, number of timed launches)."""
    ms, n = ctypes.c_float(0.0), ctypes.c_int32(0)
    _check(lib().i4d_launch_timing_stop(ctypes.byref(ms), ctypes.byref(n)), "i4d_launch_timing_stop")
    return float(ms.value), int(n.value)


def read_probe(buf, sink, stream=None):
    """Measurement aid: read all of `buf` (a device tensor) once into the XOR sink (device int32)."""
    _check(lib().i4d_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)), "i4d_read_probe")


def read_device_status(ws, stream=None) -> int:
    out = ctypes.c_int32(0)
    _check(lib().i4d_read_device_status(_ptr(ws), ctypes.byref(out), _stream(stream)), "i4d_read_device_status")
    return int(out.value)
