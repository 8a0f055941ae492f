"""GPU parity of the document-level attention mask [P2 appendix item 1]:
packed documents attend only within themselves.  The HIP path (through
llama_layer_forward_docs / llama_prefill_docs / llama_decode_step_docs) is
compared with the oracle's
document_mask on seeded packed sequences (document lengths uniform in
[1, max_doc])."""
import numpy as np
import pytest
import torch

import dense_decoder_only_rmsnorm_amd as M
import inputs as I
from dense_decoder_only_rmsnorm_amd import runtime as R
from gpu_util import BF16_TOL, F32_TOL, assert_argmax, assert_close, host, say
from oracle import llama as OL
from oracle import runner as OR

from test_gpu_parity import small_cfg

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DOC_CASES = [
    # dtype, D, H, G, S, B, max_doc
    ("bf16", 256, 4, 2, 100, 2, 30),     # hd 64
    ("bf16", 384, 4, 1, 130, 1, 40),     # hd 96
    ("bf16", 1024, 8, 2, 600, 2, 200),   # hd 128: eight-wave kernel, documents across 64-key tiles
    ("bf16", 1024, 8, 2, 300, 1, 1),     # hd 128: every token its own document
    ("bf16", 512, 4, 4, 520, 1, 700),    # hd 128 MHA, one or two long documents
    ("f32", 256, 4, 2, 100, 2, 30),
    ("f32", 512, 4, 4, 70, 1, 9),
]


def _ids(t):
    return torch.from_numpy(np.ascontiguousarray(t, dtype=np.int32)).cuda()


@pytest.mark.parametrize("dtype,D,H,G,S,B,max_doc", DOC_CASES)
def test_layer_forward_documents(dtype, D, H, G, S, B, max_doc):
    cfg = small_cfg(dtype, D, H, G, S, B, seed=13)
    docs = I.document_ids(13, f"docs-{dtype}-{D}-{S}", B, S, max_doc)
    say(f"case layer docs {cfg.key} S={S} B={B} max_doc={max_doc} ({docs.max() + 1} documents in row 0)")
    dm = R.DeviceModel(cfg, with_head=False)
    x = I.hidden_x(cfg)
    xd = torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    kv = R.kv_caches(cfg, 1, B, S)[0]
    args = R.args_for(cfg, max_batch=B, max_seq=S)
    ws = R.workspace(args, B, S)
    M.llama_layer_forward_docs(args, dm.layers[0], xd, y, B, S, 0, kv=kv, doc_ids=_ids(docs), ws=ws)
    torch.cuda.synchronize()
    ref = OR.layer(cfg, x, taps=True, doc_ids=docs)
    tol = BF16_TOL if cfg.bf16 else F32_TOL
    assert_close(host(y), ref["y"], tol, "layer output (document mask)")
    # the plain causal result differs wherever a document starts after position 0
    if docs.max() > 0:
        assert not np.allclose(ref["y"], OR.layer(cfg, x)["y"], rtol=1e-3, atol=1e-3)


@pytest.mark.parametrize("dtype,D,H,G", [("bf16", 1024, 8, 2), ("bf16", 256, 4, 2), ("f32", 256, 4, 2)])
def test_single_document_equals_causal_bitwise(dtype, D, H, G):
    S, B = 333, 2
    cfg = small_cfg(dtype, D, H, G, S, B, seed=14)
    say(f"case one document = causal {cfg.key}")
    dm = R.DeviceModel(cfg, with_head=False)
    xd = torch.from_numpy(I.hidden_x(cfg)).cuda()
    y1, y2 = torch.empty_like(xd), torch.empty_like(xd)
    args = R.args_for(cfg, max_batch=B, max_seq=S)
    ws = R.workspace(args, B, S)
    M.llama_layer_forward(args, dm.layers[0], xd, y1, B, S, 0, kv=None, ws=ws)
    M.llama_layer_forward_docs(args, dm.layers[0], xd, y2, B, S, 0, kv=None,
                               doc_ids=_ids(np.full((B, S), 7)), ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunked_prefill_with_documents(dtype):
    # a document spans the chunk boundary; the second chunk's queries see the
    # cached part of their document only
    S1, S2 = 200, 150
    cfg = small_cfg(dtype, 1024 if dtype == "bf16" else 512, 8, 2, S1 + S2, 2, seed=15)
    docs = I.document_ids(15, f"docs-chunked-{dtype}", 2, S1 + S2, 90)
    say(f"case chunked prefill with documents {cfg.key}")
    dm = R.DeviceModel(cfg, with_head=False)
    x = I.hidden_x(cfg)
    cap = 384
    kv = R.kv_caches(cfg, 1, 2, cap)[0]
    args = R.args_for(cfg, max_batch=2, max_seq=cap)
    ws = R.workspace(args, 2, S1 + S2)
    x1 = torch.from_numpy(np.ascontiguousarray(x[:, :S1])).cuda()
    x2 = torch.from_numpy(np.ascontiguousarray(x[:, S1:])).cuda()
    y1, y2 = torch.empty_like(x1), torch.empty_like(x2)
    M.llama_layer_forward_docs(args, dm.layers[0], x1, y1, 2, S1, 0, kv=kv,
                               doc_ids=_ids(docs[:, :S1]), ws=ws)
    M.llama_layer_forward_docs(args, dm.layers[0], x2, y2, 2, S2, S1, kv=kv, doc_ids=_ids(docs), ws=ws)
    torch.cuda.synchronize()
    ref = OR.layer(cfg, x, doc_ids=docs)["y"]
    tol = BF16_TOL if cfg.bf16 else F32_TOL
    assert_close(np.concatenate([host(y1), host(y2)], axis=1), ref, tol, "chunked layer output (documents)")


def test_prefill_c2_packed_documents():
    cfg = I.CONFIGS["c2"]
    B, S = cfg.batch, cfg.seq_len
    docs = I.document_ids(cfg.seed, "c2_documents", B, S, 300)
    say(f"case prefill c2 packed documents ({[int(d.max()) + 1 for d in docs]} documents)")
    dm = R.DeviceModel(cfg)
    ids = I.prompt_ids(cfg)
    hidden = torch.empty((B, S, cfg.dim), dtype=torch.float32, device="cuda")
    logits = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device="cuda")
    nid = torch.empty(B, dtype=torch.int32, device="cuda")
    args = dm.args
    ws = R.workspace(args, B, S)
    M.llama_prefill_docs(args, dm.struct, _ids(ids), _ids(docs), B, S, hidden=hidden, logits=logits, next_id=nid,
                         ws=ws)
    torch.cuda.synchronize()
    ref = OR.prefill(cfg, ids, all_hidden=True, doc_ids=docs)
    assert_close(host(hidden), ref["hidden"], BF16_TOL, "c2 packed final hidden")
    assert_close(host(logits), ref["logits"], BF16_TOL, "c2 packed logits")
    assert_argmax(nid.cpu().numpy(), ref["logits"], "c2 packed argmax")


def test_8b_layer_s2048_documents_sampled_rows():
    cfg = I.CONFIGS["c3_s2048"]
    docs = I.document_ids(cfg.seed, "c3_documents", 1, 2048, 512)
    starts = [int(p) for p in np.nonzero(np.diff(docs[0]))[0] + 1]
    say(f"case one 8B layer S=2048, {len(starts) + 1} documents, rows sampled")
    dm = R.DeviceModel(cfg, with_head=False)
    x = I.hidden_x(cfg)
    xd = torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    args = R.args_for(cfg, max_batch=1, max_seq=2048)
    ws = R.workspace(args, 1, 2048)
    M.llama_layer_forward_docs(args, dm.layers[0], xd, y, 1, 2048, 0, kv=None, doc_ids=_ids(docs), ws=ws)
    torch.cuda.synchronize()
    rows = sorted(set([0, 1, 63, 64, 255, 1000, 2047] + starts[:3] + [p - 1 for p in starts[:3]] + starts[-2:]))
    ref = OR.layer(cfg, x, rows=rows, doc_ids=docs)["y"]
    assert_close(host(y)[:, rows], ref, BF16_TOL, "8B layer S=2048 documents, sampled rows")


@pytest.mark.parametrize("dtype,D,H,G", [("bf16", 1024, 8, 2), ("bf16", 256, 4, 2), ("f32", 256, 4, 2)])
def test_decode_after_packed_prefill(dtype, D, H, G):
    # prefill of packed documents into the cache, then one decode step:
    # sequences 0 and 2 continue their last document, sequence 1 starts a new one
    S, B, cap = 300, 3, 384
    cfg = small_cfg(dtype, D, H, G, S, B, L=2, V=3000, seed=16).with_(kind="prefill")
    docs = I.document_ids(16, f"docs-decode-{dtype}-{D}", B, S, 120)
    say(f"case decode after packed prefill {cfg.key}")
    dm = R.DeviceModel(cfg)
    args = dm.args
    args.max_batch_size, args.max_seq_len = B, cap
    ids = I.prompt_ids(cfg)
    caches = R.kv_caches(cfg, cfg.n_layers, B, cap)
    kvs = M.kv_array(caches)
    ws = R.workspace(args, B, S)
    nid = torch.empty(B, dtype=torch.int32, device="cuda")
    M.llama_prefill_docs(args, dm.struct, _ids(ids), _ids(docs), B, S, kv=kvs, next_id=nid, ws=ws)
    new_ids = np.array([5, 77, 2999], dtype=np.int32)
    last_start = [int(S - np.argmax(docs[b][::-1] != docs[b][-1])) if np.any(docs[b] != docs[b][-1]) else 0
                  for b in range(B)]
    doc_start = np.array([last_start[0], S, last_start[2]], dtype=np.int32)
    pos = torch.full((B,), S, dtype=torch.int32, device="cuda")
    logits = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device="cuda")
    M.llama_decode_step_docs(args, dm.struct, _ids(new_ids), pos, _ids(doc_start), B, kvs, logits=logits,
                             next_id=nid, ws=ws)
    torch.cuda.synchronize()
    ocaches = [[] for _ in range(B)]
    OR.prefill(cfg, ids, caches=ocaches, doc_ids=docs)
    ext = [np.append(docs[b], docs[b][-1] if doc_start[b] < S else docs[b][-1] + 1) for b in range(B)]
    m = OR.model_of(cfg)
    ref = OL.decode_step(new_ids, ocaches, lambda r: m.rows("tok_embeddings", r), m.layer, m.get("norm"),
                         m.get("output"), OR.args_of(cfg), doc_ids=ext)
    tol = BF16_TOL if cfg.bf16 else F32_TOL
    assert_close(host(logits), ref["logits"], tol, "decode logits (document mask)")
    assert_argmax(nid.cpu().numpy(), ref["logits"], "decode argmax (document mask)")
    # the plain causal step differs for the sequences whose document started after position 0
    plain = OL.decode_step(new_ids, ocaches, lambda r: m.rows("tok_embeddings", r), m.layer, m.get("norm"),
                           m.get("output"), OR.args_of(cfg))
    assert not np.allclose(plain["logits"][1], ref["logits"][1], rtol=1e-3, atol=1e-3)
