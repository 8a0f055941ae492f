"""Run-to-run determinism of the HIP path: the same call twice on the same
inputs must give bit-identical outputs (logits, ids, hidden states, KV
caches).  The kernels stage operands through double-buffered LDS with
hand-placed waits and barriers and reduce split-K partials in a fixed order;
a missing wait or a stage race would show as a difference between two runs
well before it shows against the oracle's tolerance.
"""
import numpy as np
import pytest
import torch

import dense_decoder_only_rmsnorm_amd as M
import inputs as I
from dense_decoder_only_rmsnorm_amd import runtime as R
from gpu_util import say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _equal(a, b, name):
    same = torch.equal(a, b)
    if not same:
        d = (a.float() - b.float()).abs()
        say(f"  {name}: {int((d > 0).sum())} elements differ, max {float(d.max()):.3e}")
    assert same, f"{name} differs between two identical runs"


def test_prefill_small_stack_twice():
    cfg = I.CONFIGS["c2"]
    B, S = cfg.batch, cfg.seq_len
    say(f"case determinism prefill c2 B={B} S={S}")
    dm = R.DeviceModel(cfg)
    args = dm.args
    cap = S
    args.max_seq_len, args.max_batch_size = cap, B
    ids = torch.from_numpy(I.prompt_ids(cfg)).cuda()
    ws = R.workspace(args, B, S)
    outs = []
    for _ in range(2):
        caches = R.kv_caches(cfg, cfg.n_layers, B, cap)
        hidden = torch.empty((B, S, cfg.dim), dtype=torch.float32, device="cuda")
        logits = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device="cuda")
        nid = torch.empty(B, dtype=torch.int32, device="cuda")
        M.llama_prefill(args, dm.struct, ids, B, S, kv=M.kv_array(caches), hidden=hidden, logits=logits,
                        next_id=nid, ws=ws)
        torch.cuda.synchronize()
        outs.append((hidden, logits, nid, caches))
    (h0, l0, n0, c0), (h1, l1, n1, c1) = outs
    _equal(h0, h1, "hidden")
    _equal(l0, l1, "logits")
    _equal(n0, n1, "next ids")
    for l in range(cfg.n_layers):
        _equal(c0[l][0], c1[l][0], f"k cache layer {l}")
        _equal(c0[l][1], c1[l][1], f"v cache layer {l}")


@pytest.mark.parametrize("docs", [False, True], ids=["causal", "documents"])
def test_layer_8b_s2048_twice(docs):
    cfg = I.CONFIGS["c3_s2048"]
    S = cfg.seq_len
    say(f"case determinism 8B layer S={S} documents={docs}")
    dm = R.DeviceModel(cfg, with_head=False)
    x = torch.from_numpy(I.hidden_x(cfg)).cuda()
    args = R.args_for(cfg, max_batch=1, max_seq=S)
    ws = R.workspace(args, 1, S)
    doc = torch.from_numpy(I.document_ids(cfg.seed, "determinism_docs", 1, S, 512)).cuda() if docs else None
    outs = []
    for _ in range(2):
        y = torch.empty_like(x)
        kv = R.kv_caches(cfg, 1, 1, S)[0]
        if docs:
            M.llama_layer_forward_docs(args, dm.layers[0], x, y, 1, S, 0, kv=kv, doc_ids=doc, ws=ws)
        else:
            M.llama_layer_forward(args, dm.layers[0], x, y, 1, S, 0, kv=kv, ws=ws)
        torch.cuda.synchronize()
        outs.append((y, kv))
    _equal(outs[0][0], outs[1][0], "layer output")
    _equal(outs[0][1][0], outs[1][1][0], "k cache")
    _equal(outs[0][1][1], outs[1][1][1], "v cache")


def test_decode_8b_shapes_two_layers_twice():
    cfg = I.CONFIGS["c5"].with_(n_layers=2)
    B, P, cap = cfg.batch, cfg.cache_len, cfg.cache_cap
    say(f"case determinism decode 8B shapes B={B} cache {P}, 2 layers")
    dm = R.DeviceModel(cfg)
    caches = []
    for l in range(cfg.n_layers):
        pair = []
        for which in ("k", "v"):
            t = torch.zeros((B, cap, cfg.n_kv_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
            t[:, :P] = R.bits_to_device(I.kv_cache_bits(cfg, l, which))
            pair.append(t)
        caches.append(tuple(pair))
    ids = torch.from_numpy(I.prompt_ids(cfg).reshape(-1).astype(np.int32)).cuda()
    pos = torch.full((B,), P, dtype=torch.int32, device="cuda")
    ws = R.workspace(dm.args, B, 1)
    outs = []
    for _ in range(2):
        logits = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device="cuda")
        nid = torch.empty(B, dtype=torch.int32, device="cuda")
        M.llama_decode_step(dm.args, dm.struct, ids, pos, B, M.kv_array(caches), logits=logits, next_id=nid, ws=ws)
        torch.cuda.synchronize()
        outs.append((logits, nid, [(k[:, P].clone(), v[:, P].clone()) for (k, v) in caches]))
    _equal(outs[0][0], outs[1][0], "decode logits")
    _equal(outs[0][1], outs[1][1], "decode ids")
    for l in range(cfg.n_layers):
        _equal(outs[0][2][l][0], outs[1][2][l][0], f"new k layer {l}")
        _equal(outs[0][2][l][1], outs[1][2][l][1], f"new v layer {l}")
