"""The allocation-free decode step (llama_decode_step_noalloc, scratch in a
static device array of the library) against llama_decode_step with a
caller workspace: bit-identical logits, ids and cache writes, on two calls
in a row, the second with a smaller batch and ragged positions (the scratch
keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import dense_decoder_only_rmsnorm_amd as M
import inputs as I
from dense_decoder_only_rmsnorm_amd import runtime as R
from gpu_util import say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _caches(cfg, B, P, cap):
    out = []
    for l in range(cfg.n_layers):
        pair = []
        for which in ("k", "v"):
            t = torch.zeros((B, cap, cfg.n_kv_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
            t[:, :P] = R.bits_to_device(I.kv_cache_bits(cfg, l, which))
            pair.append(t)
        out.append(tuple(pair))
    return out


def test_noalloc_decode_equals_workspace_decode_twice():
    cfg = I.CONFIGS["c5"].with_(n_layers=2)
    B, P, cap = cfg.batch, cfg.cache_len, cfg.cache_cap
    say(f"case no-alloc decode, 8B shapes, 2 layers, B={B} then B=5, cache {P}")
    dm = R.DeviceModel(cfg)
    need = M.llama_workspace_bytes(dm.args, B, 1)
    assert need <= M.llama_decode_noalloc_max_bytes()
    ref_caches = _caches(cfg, B, P, cap)
    na_caches = [(k.clone(), v.clone()) for (k, v) in ref_caches]
    ids = torch.from_numpy(I.prompt_ids(cfg).reshape(-1).astype(np.int32)).cuda()
    ws = R.workspace(dm.args, B, 1)
    calls = [(B, torch.full((B,), P, dtype=torch.int32, device="cuda")),
             (5, torch.tensor([P, 100, 2048, P - 1, 1], dtype=torch.int32, device="cuda"))]
    for n, pos in calls:
        say(f"  call with batch {n}")
        lr = torch.full((n, cfg.vocab_size), float("nan"), dtype=torch.float32, device="cuda")
        ln = torch.full((n, cfg.vocab_size), float("nan"), dtype=torch.float32, device="cuda")
        ir = torch.full((n,), -1, dtype=torch.int32, device="cuda")
        i_n = torch.full((n,), -2, dtype=torch.int32, device="cuda")
        M.llama_decode_step(dm.args, dm.struct, ids[:n], pos, n, M.kv_array(ref_caches), logits=lr, next_id=ir,
                            ws=ws)
        M.llama_decode_step_noalloc(dm.args, dm.struct, ids[:n], pos, n, M.kv_array(na_caches), logits=ln,
                                    next_id=i_n)
        torch.cuda.synchronize()
        assert torch.isfinite(ln).all()
        assert torch.equal(lr, ln), f"logits differ (max {float((lr - ln).abs().max()):.3e})"
        assert torch.equal(ir, i_n)
        for l in range(cfg.n_layers):
            assert torch.equal(ref_caches[l][0], na_caches[l][0]), f"k cache layer {l}"
            assert torch.equal(ref_caches[l][1], na_caches[l][1]), f"v cache layer {l}"


def test_noalloc_decode_rejects_a_step_beyond_its_scratch():
    cfg = I.CONFIGS["c5"].with_(n_layers=1)
    dm = R.DeviceModel(cfg)
    a = R.args_for(cfg, max_batch=64, max_seq=131072)
    assert M.llama_workspace_bytes(a, 64, 1) > M.llama_decode_noalloc_max_bytes()
    caches = [(torch.zeros(1, dtype=torch.bfloat16, device="cuda"),) * 2]
    ids = torch.zeros(64, dtype=torch.int32, device="cuda")
    pos = torch.zeros(64, dtype=torch.int32, device="cuda")
    nid = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(M.LlamaError) as e:
        M.llama_decode_step_noalloc(a, dm.struct, ids, pos, 64, M.kv_array(caches), next_id=nid)
    assert e.value.code == M.LLAMA_ERR_WORKSPACE
