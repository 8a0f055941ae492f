"""The C-ABI library without a GPU: it loads, exports every declared symbol,
derives the FFN size like the oracle, sizes workspaces, and rejects bad
arguments before touching HIP."""
import ctypes
import os
import re

import pytest
import torch

import dense_decoder_only_rmsnorm_amd as M
import inputs as I
from oracle import llama as OL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = []
    inc = os.path.join(ROOT, "include")
    for f in os.listdir(inc):
        if not f.endswith(".h"):
            continue
        text = open(os.path.join(inc, f)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = M.lib()
    decl = _declared_symbols()
    assert set(M.EXPORTED) <= set(decl)
    for name in decl:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("key", ["c1", "c2", "c3_s17", "c4", "c5"])
def test_ffn_hidden_dim_agrees_with_oracle(key):
    cfg = I.CONFIGS[key]
    args = M.make_args(cfg.dim, cfg.n_layers, cfg.n_heads, cfg.n_kv_heads, cfg.vocab_size, cfg.multiple_of,
                       cfg.ffn_dim_multiplier, cfg.norm_eps, cfg.rope_theta)
    assert M.llama_ffn_hidden_dim(args) == OL.ffn_hidden_dim(cfg.dim, cfg.multiple_of, cfg.ffn_dim_multiplier)


def _args(**kw):
    base = dict(dim=512, n_layers=2, n_heads=8, n_kv_heads=4, vocab_size=68, multiple_of=256,
                ffn_dim_multiplier=None, norm_eps=1e-5, rope_theta=5e5, max_batch_size=4, max_seq_len=64,
                dtype=M.LLAMA_BF16)
    base.update(kw)
    return M.make_args(**base)


def test_workspace_bytes_grows_with_tokens():
    a = _args()
    n1 = M.llama_workspace_bytes(a, 1, 16)
    n2 = M.llama_workspace_bytes(a, 2, 64)
    assert 0 < n1 < n2
    with pytest.raises(M.LlamaError):
        M.llama_workspace_bytes(_args(dim=500), 1, 16)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation returns first


def _layer_fake():
    return M.llama_layer_w(*([0x1000] * 9))


def _call_layer(a, x=FAKE, y=FAKE, batch=1, seq=8, start=0, kv=None, ws=FAKE, ws_bytes=1 << 40):
    return M.lib().llama_layer_forward(ctypes.byref(a), ctypes.byref(_layer_fake()), x, y, batch, seq, start,
                                       kv, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dim=510, n_heads=6, n_kv_heads=3), M.LLAMA_ERR_SHAPE),    # hd 85: odd
    (dict(n_heads=8, n_kv_heads=3), M.LLAMA_ERR_SHAPE),              # heads % kv_heads
    (dict(dim=640, n_heads=8, n_kv_heads=4), M.LLAMA_ERR_UNSUPPORTED),  # hd 80
    (dict(n_heads=8, n_kv_heads=8, dim=256 * 8 * 4), M.LLAMA_ERR_UNSUPPORTED),  # hd 256
    (dict(dtype=7), M.LLAMA_ERR_ARG),
    (dict(dim=0), M.LLAMA_ERR_ARG),
])
def test_model_validation_errors(kw, code):
    assert _call_layer(_args(**kw)) == code
    assert M.last_error()


def test_argument_errors_return_before_hip():
    a = _args()
    assert _call_layer(a, x=None) == M.LLAMA_ERR_ARG
    assert _call_layer(a, ws=None) == M.LLAMA_ERR_ARG
    assert _call_layer(a, start=3) == M.LLAMA_ERR_ARG  # start_pos > 0 needs a cache
    assert _call_layer(a, batch=0) == M.LLAMA_ERR_ARG
    kv = M.llama_kv(0x1000, 0x1000)
    assert _call_layer(a, kv=ctypes.byref(kv), batch=5) == M.LLAMA_ERR_SHAPE  # > max_batch_size
    assert _call_layer(a, kv=ctypes.byref(kv), start=60, seq=8) == M.LLAMA_ERR_SHAPE  # > max_seq_len
    need = M.llama_workspace_bytes(a, 1, 8)
    assert _call_layer(a, ws_bytes=1024) == M.LLAMA_ERR_WORKSPACE
    assert "workspace" in M.last_error()
    assert need > 1024


def test_decode_and_head_argument_errors():
    a = _args()
    L = M.lib()
    layers = (M.llama_layer_w * 2)(_layer_fake(), _layer_fake())
    model = M.llama_model_w(0x1000, ctypes.cast(layers, ctypes.POINTER(M.llama_layer_w)), 0x1000, 0x1000)
    kvs = (M.llama_kv * 2)(M.llama_kv(0x1000, 0x1000), M.llama_kv(0x1000, 0x1000))
    rc = L.llama_decode_step(ctypes.byref(a), ctypes.byref(model), FAKE, None, 2, kvs, None, FAKE, FAKE, 1 << 40, None)
    assert rc == M.LLAMA_ERR_ARG  # pos is NULL
    rc = L.llama_decode_step(ctypes.byref(a), ctypes.byref(model), FAKE, FAKE, 9, kvs, None, FAKE, FAKE, 1 << 40, None)
    assert rc == M.LLAMA_ERR_SHAPE  # batch > max_batch_size
    rc = L.llama_decode_step(ctypes.byref(a), ctypes.byref(model), FAKE, FAKE, 2, kvs, None, FAKE, FAKE, 64, None)
    assert rc == M.LLAMA_ERR_WORKSPACE
    rc = L.lm_head_argmax(ctypes.byref(a), FAKE, None, FAKE, 0, None, FAKE, FAKE, 1 << 40, None)
    assert rc == M.LLAMA_ERR_ARG  # M < 1
    rc = L.llama_prefill(ctypes.byref(a), ctypes.byref(model), None, 1, 8, None, None, None, FAKE, FAKE, 1 << 40, None)
    assert rc == M.LLAMA_ERR_ARG  # ids NULL


def test_noalloc_decode_argument_errors_and_scratch_limit():
    # the allocation-free decode step validates like llama_decode_step and
    # refuses a step whose workspace exceeds its static scratch, all before
    # any HIP call
    L = M.lib()
    cap = M.llama_decode_noalloc_max_bytes()
    assert cap == 96 << 20
    layers = (M.llama_layer_w * 2)(_layer_fake(), _layer_fake())
    model = M.llama_model_w(0x1000, ctypes.cast(layers, ctypes.POINTER(M.llama_layer_w)), 0x1000, 0x1000)
    kvs = (M.llama_kv * 2)(M.llama_kv(0x1000, 0x1000), M.llama_kv(0x1000, 0x1000))
    a = _args()
    assert L.llama_decode_step_noalloc(ctypes.byref(a), ctypes.byref(model), FAKE, None, 2, kvs, None, FAKE,
                                       None) == M.LLAMA_ERR_ARG
    assert L.llama_decode_step_noalloc(ctypes.byref(a), ctypes.byref(model), FAKE, FAKE, 9, kvs, None, FAKE,
                                       None) == M.LLAMA_ERR_SHAPE
    big = _args(dim=4096, n_heads=32, n_kv_heads=8, vocab_size=128256, multiple_of=1024, ffn_dim_multiplier=1.3,
                max_batch_size=64, max_seq_len=131072)
    assert M.llama_workspace_bytes(big, 64, 1) > cap
    rc = L.llama_decode_step_noalloc(ctypes.byref(big), ctypes.byref(model), FAKE, FAKE, 64, kvs, None, FAKE, None)
    assert rc == M.LLAMA_ERR_WORKSPACE and b"scratch" in L.llama_last_error()
    # the 64-sequence 8B-shaped step over a 4224-position cache fits
    fits = _args(dim=4096, n_heads=32, n_kv_heads=8, vocab_size=128256, multiple_of=1024, ffn_dim_multiplier=1.3,
                 max_batch_size=64, max_seq_len=4224)
    assert M.llama_workspace_bytes(fits, 64, 1) <= cap


@pytest.mark.skipif(torch.cuda.is_available(), reason="forces the no-device path; only meaningful without a GPU")
def test_no_device_reports_hip_error():
    a = _args()
    need = M.llama_workspace_bytes(a, 1, 8)
    rc = _call_layer(a, ws_bytes=need, ws=ctypes.c_void_p(0x10000))
    assert rc == M.LLAMA_ERR_HIP
    assert M.last_error()


def test_sampler_argument_errors():
    L = M.lib()
    rc = L.llama_sample_top_p(None, 2, 100, 0.6, 0.9, FAKE, FAKE, None)
    assert rc == M.LLAMA_ERR_ARG
    assert L.llama_sample_top_p(FAKE, 0, 100, 0.6, 0.9, FAKE, FAKE, None) == M.LLAMA_ERR_ARG
    assert L.llama_sample_top_p(FAKE, 2, 100, 0.0, 0.9, FAKE, FAKE, None) == M.LLAMA_ERR_ARG  # T must be > 0
    assert L.llama_sample_top_p(FAKE, 2, 100, 0.6, -0.1, FAKE, FAKE, None) == M.LLAMA_ERR_ARG
    assert L.llama_sample_top_p(FAKE, 2, 131073, 0.6, 0.9, FAKE, FAKE, None) == M.LLAMA_ERR_UNSUPPORTED


def _gen(a, lens, batch=None, max_gen=4, eos=-1, temp=0.0, uni=FAKE, stride=None, ws_bytes=1 << 40, kv=True):
    layers = (M.llama_layer_w * 2)(_layer_fake(), _layer_fake())
    model = M.llama_model_w(0x1000, ctypes.cast(layers, ctypes.POINTER(M.llama_layer_w)), 0x1000, 0x1000)
    kvs = (M.llama_kv * 2)(M.llama_kv(0x1000, 0x1000), M.llama_kv(0x1000, 0x1000)) if kv else None
    n = len(lens)
    arr = (ctypes.c_int32 * max(n, 1))(*lens)
    steps = ctypes.c_int32(-7)
    rc = M.lib().llama_generate(ctypes.byref(a), ctypes.byref(model), FAKE, stride or max(lens), arr,
                                n if batch is None else batch, max_gen, eos, temp, 0.9, uni, kvs, FAKE, FAKE, 0,
                                ctypes.byref(steps), FAKE, ws_bytes, None)
    return rc, steps.value


def test_generate_argument_errors():
    a = _args()
    assert _gen(a, [3, 0])[0] == M.LLAMA_ERR_ARG           # empty prompt
    assert _gen(a, [3, 65])[0] == M.LLAMA_ERR_ARG          # prompt longer than max_seq_len
    assert _gen(a, [3, 5], stride=4)[0] == M.LLAMA_ERR_ARG  # stride below the longest prompt
    assert _gen(a, [3, 5], max_gen=-1)[0] == M.LLAMA_ERR_ARG
    assert _gen(a, [3, 5], temp=-1.0)[0] == M.LLAMA_ERR_ARG
    assert _gen(a, [3, 5], temp=0.6, uni=None)[0] == M.LLAMA_ERR_ARG  # sampling needs uniforms
    assert _gen(a, [3] * 5)[0] == M.LLAMA_ERR_SHAPE         # batch > max_batch_size
    assert _gen(_args(max_batch_size=128), [3] * 65)[0] == M.LLAMA_ERR_UNSUPPORTED  # batch > 64
    assert _gen(a, [3, 5], kv=False)[0] == M.LLAMA_ERR_ARG
    rc, steps = _gen(a, [3, 5], ws_bytes=1024)
    assert rc == M.LLAMA_ERR_WORKSPACE and steps == -7
    assert "workspace" in M.last_error()


def test_generate_workspace_bytes():
    a = _args()
    n1 = M.llama_generate_workspace_bytes(a, 1, 8)
    n2 = M.llama_generate_workspace_bytes(a, 4, 64)
    assert 0 < n1 < n2
    # at least a decode step's and a prefill call's workspace
    assert n2 >= M.llama_workspace_bytes(a, 4, 64)
    with pytest.raises(M.LlamaError):
        M.llama_generate_workspace_bytes(a, 65, 8)


def test_document_entry_points_argument_errors():
    a = _args()
    L = M.lib()
    layers = (M.llama_layer_w * 2)(_layer_fake(), _layer_fake())
    model = M.llama_model_w(0x1000, ctypes.cast(layers, ctypes.POINTER(M.llama_layer_w)), 0x1000, 0x1000)
    kvs = (M.llama_kv * 2)(M.llama_kv(0x1000, 0x1000), M.llama_kv(0x1000, 0x1000))
    rc = L.llama_decode_step_docs(ctypes.byref(a), ctypes.byref(model), FAKE, None, FAKE, 2, kvs, None, FAKE, FAKE,
                                  1 << 40, None)
    assert rc == M.LLAMA_ERR_ARG  # pos is NULL
    rc = L.llama_decode_step_docs(ctypes.byref(a), ctypes.byref(model), FAKE, FAKE, FAKE, 9, kvs, None, FAKE, FAKE,
                                  1 << 40, None)
    assert rc == M.LLAMA_ERR_SHAPE  # batch > max_batch_size
    rc = L.llama_prefill_docs(ctypes.byref(a), ctypes.byref(model), None, FAKE, 1, 8, None, None, None, FAKE, FAKE,
                              1 << 40, None)
    assert rc == M.LLAMA_ERR_ARG  # ids NULL
    rc = L.llama_layer_forward_docs(ctypes.byref(a), ctypes.byref(_layer_fake()), FAKE, FAKE, 1, 8, 3, None, FAKE,
                                    FAKE, 1 << 40, None)
    assert rc == M.LLAMA_ERR_ARG  # start_pos > 0 without a cache
