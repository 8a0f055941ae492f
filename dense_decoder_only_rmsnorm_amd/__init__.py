"""Python binding of the MI355X Llama-3 decoder forward pass.

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of ``libllama_mi355x.so`` (built from ``csrc/`` by ``build.py``),
called through its C ABI (``include/llama_mi355x.h``).  PyTorch supplies
device memory and streams.  The entry points keep the C names:
``llama_layer_forward``, ``llama_prefill``, ``llama_decode_step``,
``lm_head_argmax``, ``llama_sample_top_p``, ``llama_generate``,
``llama_layer_forward_docs``, ``llama_prefill_docs``, ``llama_decode_step_docs``,
``llama_decode_step_noalloc``, plus
``llama_ffn_hidden_dim``, ``llama_workspace_bytes`` and
``llama_generate_workspace_bytes``.

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libllama_mi355x.so")

LLAMA_OK, LLAMA_ERR_ARG, LLAMA_ERR_SHAPE, LLAMA_ERR_UNSUPPORTED, LLAMA_ERR_WORKSPACE, LLAMA_ERR_HIP = 0, -1, -2, -3, -4, -5
LLAMA_F32, LLAMA_BF16 = 0, 1
ERROR_NAMES = {-1: "LLAMA_ERR_ARG", -2: "LLAMA_ERR_SHAPE", -3: "LLAMA_ERR_UNSUPPORTED", -4: "LLAMA_ERR_WORKSPACE",
               -5: "LLAMA_ERR_HIP"}
EXPORTED = ("llama_ffn_hidden_dim", "llama_workspace_bytes", "llama_layer_forward", "llama_prefill",
            "llama_decode_step", "lm_head_argmax", "llama_sample_top_p", "llama_generate_workspace_bytes",
            "llama_generate", "llama_layer_forward_docs", "llama_prefill_docs", "llama_decode_step_docs",
            "llama_decode_step_noalloc", "llama_decode_noalloc_max_bytes", "llama_last_error",
            "llama_timing_enable", "llama_timing_report")
LLAMA_GEN_GRAPH = 2


class LlamaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {message}")
        self.code = code


class llama_args(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("vocab_size", ctypes.c_int32), ("multiple_of", ctypes.c_int32),
                ("ffn_dim_multiplier", ctypes.c_float), ("norm_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("max_batch_size", ctypes.c_int32), ("max_seq_len", ctypes.c_int32), ("dtype", ctypes.c_int32)]


LAYER_FIELDS = ("attention_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w1", "w2", "w3")


class llama_layer_w(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_FIELDS]


class llama_model_w(ctypes.Structure):
    _fields_ = [("tok_embeddings", ctypes.c_void_p), ("layers", ctypes.POINTER(llama_layer_w)),
                ("norm", ctypes.c_void_p), ("output", ctypes.c_void_p)]


class llama_kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m dense_decoder_only_rmsnorm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        A = ctypes.POINTER(llama_args)
        L.llama_ffn_hidden_dim.argtypes = [A]
        L.llama_ffn_hidden_dim.restype = i32
        L.llama_workspace_bytes.argtypes = [A, i32, i32]
        L.llama_workspace_bytes.restype = sz
        L.llama_layer_forward.argtypes = [A, ctypes.POINTER(llama_layer_w), vp, vp, i32, i32, i32,
                                          ctypes.POINTER(llama_kv), vp, sz, vp]
        L.llama_layer_forward.restype = ctypes.c_int
        L.llama_prefill.argtypes = [A, ctypes.POINTER(llama_model_w), vp, i32, i32, ctypes.POINTER(llama_kv), vp, vp,
                                    vp, vp, sz, vp]
        L.llama_prefill.restype = ctypes.c_int
        L.llama_decode_step.argtypes = [A, ctypes.POINTER(llama_model_w), vp, vp, i32, ctypes.POINTER(llama_kv), vp,
                                        vp, vp, sz, vp]
        L.llama_decode_step.restype = ctypes.c_int
        L.llama_decode_step_noalloc.argtypes = [A, ctypes.POINTER(llama_model_w), vp, vp, i32,
                                                ctypes.POINTER(llama_kv), vp, vp, vp]
        L.llama_decode_step_noalloc.restype = ctypes.c_int
        L.llama_decode_noalloc_max_bytes.argtypes = []
        L.llama_decode_noalloc_max_bytes.restype = sz
        L.lm_head_argmax.argtypes = [A, vp, vp, vp, i32, vp, vp, vp, sz, vp]
        L.lm_head_argmax.restype = ctypes.c_int
        L.llama_layer_forward_docs.argtypes = [A, ctypes.POINTER(llama_layer_w), vp, vp, i32, i32, i32,
                                               ctypes.POINTER(llama_kv), vp, vp, sz, vp]
        L.llama_layer_forward_docs.restype = ctypes.c_int
        L.llama_prefill_docs.argtypes = [A, ctypes.POINTER(llama_model_w), vp, vp, i32, i32, ctypes.POINTER(llama_kv),
                                         vp, vp, vp, vp, sz, vp]
        L.llama_prefill_docs.restype = ctypes.c_int
        L.llama_decode_step_docs.argtypes = [A, ctypes.POINTER(llama_model_w), vp, vp, vp, i32,
                                             ctypes.POINTER(llama_kv), vp, vp, vp, sz, vp]
        L.llama_decode_step_docs.restype = ctypes.c_int
        L.llama_sample_top_p.argtypes = [vp, i32, i32, ctypes.c_float, ctypes.c_float, vp, vp, vp]
        L.llama_sample_top_p.restype = ctypes.c_int
        L.llama_generate_workspace_bytes.argtypes = [A, i32, i32]
        L.llama_generate_workspace_bytes.restype = sz
        L.llama_generate.argtypes = [A, ctypes.POINTER(llama_model_w), vp, i32, ctypes.POINTER(i32), i32, i32, i32,
                                     ctypes.c_float, ctypes.c_float, vp, ctypes.POINTER(llama_kv), vp, vp, i32,
                                     ctypes.POINTER(i32), vp, sz, vp]
        L.llama_generate.restype = ctypes.c_int
        L.llama_timing_enable.argtypes = [ctypes.c_int]
        L.llama_timing_enable.restype = ctypes.c_int
        L.llama_timing_report.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
        L.llama_timing_report.restype = ctypes.c_int64
        L.llama_last_error.argtypes = []
        L.llama_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().llama_last_error().decode()


def _check(rc: int):
    if rc != LLAMA_OK:
        raise LlamaError(rc, last_error())


def _p(t) -> Optional[int]:
    """Device pointer of a tensor (or None)."""
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def make_args(dim: int, n_layers: int, n_heads: int, n_kv_heads: int, vocab_size: int, multiple_of: int,
              ffn_dim_multiplier: Optional[float], norm_eps: float, rope_theta: float, max_batch_size: int = 1,
              max_seq_len: int = 1, dtype: int = LLAMA_BF16) -> llama_args:
    return llama_args(dim, n_layers, n_heads, n_kv_heads, vocab_size, multiple_of,
                      -1.0 if ffn_dim_multiplier is None else float(ffn_dim_multiplier), norm_eps, rope_theta,
                      max_batch_size, max_seq_len, dtype)


def layer_struct(layer: dict) -> llama_layer_w:
    """llama_layer_w from a dict of device tensors keyed by checkpoint names."""
    return llama_layer_w(*[_p(layer[n]) for n in LAYER_FIELDS])


def model_struct(tok_embeddings, layers: Sequence[dict], norm, output):
    """(llama_model_w, keep-alive array) from device tensors."""
    arr = (llama_layer_w * max(1, len(layers)))(*[layer_struct(l) for l in layers])
    m = llama_model_w(_p(tok_embeddings), ctypes.cast(arr, ctypes.POINTER(llama_layer_w)), _p(norm), _p(output))
    return m, arr


def kv_array(caches: Sequence):
    """HOST array of llama_kv from (k, v) tensor pairs."""
    arr = (llama_kv * max(1, len(caches)))(*[llama_kv(_p(k), _p(v)) for k, v in caches])
    return arr


def llama_ffn_hidden_dim(args: llama_args) -> int:
    r = lib().llama_ffn_hidden_dim(ctypes.byref(args))
    _check(min(r, 0))
    return r


def llama_workspace_bytes(args: llama_args, batch: int, seq_len: int) -> int:
    n = lib().llama_workspace_bytes(ctypes.byref(args), batch, seq_len)
    if n == 0:
        raise LlamaError(LLAMA_ERR_ARG, last_error() or "invalid arguments")
    return n


def llama_layer_forward(args: llama_args, layer: dict, x, y, batch: int, seq_len: int, start_pos: int = 0,
                        kv=None, ws=None, stream=None):
    lw = layer_struct(layer)
    kvs = llama_kv(_p(kv[0]), _p(kv[1])) if kv is not None else None
    rc = lib().llama_layer_forward(ctypes.byref(args), ctypes.byref(lw), _p(x), _p(y), batch, seq_len, start_pos,
                                   ctypes.byref(kvs) if kvs is not None else None, _p(ws),
                                   ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)


def llama_layer_forward_docs(args: llama_args, layer: dict, x, y, batch: int, seq_len: int, start_pos: int = 0,
                             kv=None, doc_ids=None, ws=None, stream=None):
    """``doc_ids``: int32 device tensor [batch, start_pos + seq_len] (document-level mask) or None."""
    lw = layer_struct(layer)
    kvs = llama_kv(_p(kv[0]), _p(kv[1])) if kv is not None else None
    rc = lib().llama_layer_forward_docs(ctypes.byref(args), ctypes.byref(lw), _p(x), _p(y), batch, seq_len,
                                        start_pos, ctypes.byref(kvs) if kvs is not None else None, _p(doc_ids),
                                        _p(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)


def llama_prefill_docs(args: llama_args, model, ids, doc_ids, batch: int, seq_len: int, kv=None, hidden=None,
                       logits=None, next_id=None, ws=None, stream=None):
    m = model[0]
    rc = lib().llama_prefill_docs(ctypes.byref(args), ctypes.byref(m), _p(ids), _p(doc_ids), batch, seq_len,
                                  kv if kv is not None else None, _p(hidden), _p(logits), _p(next_id), _p(ws),
                                  ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)


def llama_prefill(args: llama_args, model, ids, batch: int, seq_len: int, kv=None, hidden=None, logits=None,
                  next_id=None, ws=None, stream=None):
    """``model`` is a (llama_model_w, keep-alive) pair from model_struct; kv a kv_array or None."""
    m = model[0]
    rc = lib().llama_prefill(ctypes.byref(args), ctypes.byref(m), _p(ids), batch, seq_len,
                             kv if kv is not None else None, _p(hidden), _p(logits), _p(next_id), _p(ws),
                             ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)


def llama_decode_step(args: llama_args, model, ids, pos, batch: int, kv, logits=None, next_id=None, ws=None,
                      stream=None):
    m = model[0]
    rc = lib().llama_decode_step(ctypes.byref(args), ctypes.byref(m), _p(ids), _p(pos), batch, kv, _p(logits),
                                 _p(next_id), _p(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)


def llama_decode_step_noalloc(args: llama_args, model, ids, pos, batch: int, kv, logits=None, next_id=None,
                              stream=None):
    """llama_decode_step with the library's static scratch in place of a workspace."""
    m = model[0]
    rc = lib().llama_decode_step_noalloc(ctypes.byref(args), ctypes.byref(m), _p(ids), _p(pos), batch, kv,
                                         _p(logits), _p(next_id), _stream(stream))
    _check(rc)


def llama_decode_noalloc_max_bytes() -> int:
    return int(lib().llama_decode_noalloc_max_bytes())


def llama_decode_step_docs(args: llama_args, model, ids, pos, doc_start, batch: int, kv, logits=None, next_id=None,
                           ws=None, stream=None):
    m = model[0]
    rc = lib().llama_decode_step_docs(ctypes.byref(args), ctypes.byref(m), _p(ids), _p(pos), _p(doc_start), batch,
                                      kv, _p(logits), _p(next_id), _p(ws), ws.numel() * ws.element_size(),
                                      _stream(stream))
    _check(rc)


def lm_head_argmax(args: llama_args, h, final_norm_w, w_out, M: int, logits=None, argmax=None, ws=None,
                   stream=None):
    rc = lib().lm_head_argmax(ctypes.byref(args), _p(h), _p(final_norm_w), _p(w_out), M, _p(logits), _p(argmax),
                              _p(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)


def llama_sample_top_p(logits, M: int, V: int, temperature: float, top_p: float, u, out_id, stream=None):
    rc = lib().llama_sample_top_p(_p(logits), M, V, temperature, top_p, _p(u), _p(out_id), _stream(stream))
    _check(rc)


def llama_generate_workspace_bytes(args: llama_args, batch: int, max_prompt_len: int) -> int:
    n = lib().llama_generate_workspace_bytes(ctypes.byref(args), batch, max_prompt_len)
    if n == 0:
        raise LlamaError(LLAMA_ERR_ARG, last_error() or "invalid arguments")
    return n


def llama_generate(args: llama_args, model, prompt, prompt_stride: int, prompt_len: Sequence[int], batch: int,
                   max_gen_len: int, eos_id: int, temperature: float, top_p: float, uniforms, kv, tokens, out_len,
                   flags: int = 0, ws=None, stream=None) -> int:
    """``prompt_len`` is a host sequence; returns the number of decode steps run."""
    m = model[0]
    lens = (ctypes.c_int32 * max(1, len(prompt_len)))(*[int(x) for x in prompt_len])
    steps = ctypes.c_int32(0)
    rc = lib().llama_generate(ctypes.byref(args), ctypes.byref(m), _p(prompt), prompt_stride, lens, batch,
                              max_gen_len, eos_id, temperature, top_p, _p(uniforms), kv, _p(tokens), _p(out_len),
                              flags, ctypes.byref(steps), _p(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)
    return steps.value


def llama_timing_enable(on: bool = True):
    _check(lib().llama_timing_enable(1 if on else 0))


def llama_timing_report() -> dict:
    """{kernel_name: (launches, total_ms)} since the last enable/report."""
    buf = ctypes.create_string_buffer(1 << 20)
    n = lib().llama_timing_report(buf, len(buf))
    _check(min(int(n), 0))
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split()
        out[name] = (int(cnt), float(ms))
    return out


__all__ = ["llama_timing_enable", "llama_timing_report", "lib", "last_error", "LlamaError", "llama_args", "llama_layer_w", "llama_model_w", "llama_kv",
           "make_args", "layer_struct", "model_struct", "kv_array", "llama_ffn_hidden_dim",
           "llama_workspace_bytes", "llama_layer_forward", "llama_prefill", "llama_decode_step", "lm_head_argmax",
           "llama_sample_top_p", "llama_generate_workspace_bytes", "llama_generate", "LLAMA_GEN_GRAPH",
           "llama_layer_forward_docs", "llama_prefill_docs", "llama_decode_step_docs",
           "LLAMA_F32", "LLAMA_BF16", "EXPORTED"]
