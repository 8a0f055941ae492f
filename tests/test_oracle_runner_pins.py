"""Pins of the helpers that bind the oracle to the seeded configurations
(``oracle/runner.py``) and of the script that stores the oracle's own
32-layer 8B prefill result (``tests/golden/make_prefill_8b_oracle.py``).

CPU only.  Each helper is checked against something other than itself:
  * ``runner._layer_rows`` (sampled rows of one layer, each run as a
    one-token step over its prefix) against ``layer_forward`` on the whole
    sequence and against the scalar brute-force layer;
  * ``runner.decode`` (per-sequence seeded caches) against the scalar
    brute-force layer fed the caches sliced from the whole seeded block, and
    against ``decode_step`` on those independently assembled caches;
  * the golden script's composition against ``oracle.llama.prefill``.
Pages: [P2] "Build your own Llama 3 architecture from scratch" notes, 3.3
(KV cache: a token at position p attends to the cached keys 0..p-1 and its
own), 4 (Transformer.forward); [P1] "llama3-from-scratch" sections 10-12.
"""
import importlib.util
import os

import numpy as np
import pytest

import inputs as I
from oracle import brute as BR
from oracle import llama as L
from oracle import runner as OR

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(kind="layer", D=32, H=4, G=2, S=21, B=2, n_layers=1, V=40, dtype="bf16", cache_len=0, seed=41):
    return I.Config(f"tiny-{kind}", dim=D, n_layers=n_layers, n_heads=H, n_kv_heads=G, vocab_size=V,
                    multiple_of=16, ffn_dim_multiplier=None, norm_eps=1e-5, rope_theta=500000.0, dtype=dtype,
                    batch=B, seq_len=S, seed=seed, norm_std=0.1, weight_std=0.2, cache_len=cache_len,
                    cache_cap=cache_len + 4, kind=kind)


def _lists(lw):
    return {k: np.asarray(v, dtype=np.float64).tolist() for k, v in lw.items()}


@pytest.mark.parametrize("rows", [[0], [0, 1, 20], [7, 3, 19, 20], [20]])
def test_layer_rows_equal_full_layer(rows):
    cfg = _tiny()
    x = I.hidden_x(cfg)
    full = OR.layer(cfg, x)["y"]
    got = OR.layer(cfg, x, rows=rows)["y"]
    assert got.shape == (cfg.batch, len(rows), cfg.dim)
    assert np.allclose(got, full[:, rows], rtol=1e-12, atol=1e-12)


def test_layer_rows_equal_brute_force():
    cfg = _tiny(S=9, B=1)
    x = I.hidden_x(cfg)
    lw = OR.model_of(cfg).layer(0)
    rows = [0, 4, 8]
    got = OR.layer(cfg, x, rows=rows)["y"][0]
    ref, _, _ = BR.layer_forward(np.asarray(x[0], np.float64).tolist(), _lists(lw), OR.args_of(cfg))
    assert np.allclose(got, np.asarray(ref)[rows], rtol=1e-11, atol=1e-11)


def test_layer_rows_with_documents_equal_full_layer():
    cfg = _tiny(S=24, B=2)
    x = I.hidden_x(cfg)
    docs = I.document_ids(cfg.seed, "runner_pin_docs", cfg.batch, cfg.seq_len, 7)
    full = OR.layer(cfg, x, doc_ids=docs)["y"]
    rows = [0, 5, 11, 23]
    got = OR.layer(cfg, x, rows=rows, doc_ids=docs)["y"]
    assert np.allclose(got, full[:, rows], rtol=1e-12, atol=1e-12)


def _brute_decode(cfg, b):
    """Scalar decode of sequence b over its seeded cache: embedding row, each
    layer as brute.layer_forward at position cache_len with the cached keys
    and values (sliced from the whole batch's seeded block) as its past, final
    norm and explicit dot products for the logits."""
    m = OR.model_of(cfg)
    a = OR.args_of(cfg)
    ids = I.prompt_ids(cfg).reshape(-1)
    h = [np.asarray(m.rows("tok_embeddings", ids[b:b + 1])[0], np.float64).tolist()]
    P = cfg.cache_len
    for l in range(cfg.n_layers):
        kb = I.kv_cache_block(cfg, l, "k")[b]  # [P, G, hd] of the whole block, sequence b
        vb = I.kv_cache_block(cfg, l, "v")[b]
        past_k = [[kb[t, g].astype(np.float64).tolist() for g in range(cfg.n_kv_heads)] for t in range(P)]
        past_v = [[vb[t, g].astype(np.float64).tolist() for g in range(cfg.n_kv_heads)] for t in range(P)]
        h, _, _ = BR.layer_forward(h, _lists(m.layer(l)), a, pos0=P, past_k=past_k, past_v=past_v)
    hf = BR.rms_norm(h[0], np.asarray(m.get("norm"), np.float64).tolist(), cfg.norm_eps)
    return BR.matvec(np.asarray(m.get("output"), np.float64).tolist(), hf)


def test_decode_equals_brute_force_over_seeded_caches():
    cfg = _tiny(kind="decode", S=1, B=3, n_layers=2, cache_len=6)
    seqs = [2, 0]
    res = OR.decode(cfg, seqs)
    for i, b in enumerate(seqs):
        ref = _brute_decode(cfg, b)
        assert np.allclose(res["logits"][i], ref, rtol=1e-10, atol=1e-10), f"sequence {b}"
        assert res["ids"][i] == int(np.argmax(ref))


def test_decode_equals_decode_step_on_block_caches():
    # caches assembled from the whole seeded block (not per-sequence draws)
    cfg = _tiny(kind="decode", S=1, B=4, n_layers=2, cache_len=9, D=64, H=4, G=1)
    m = OR.model_of(cfg)
    blocks = {(l, w): I.kv_cache_block(cfg, l, w) for l in range(cfg.n_layers) for w in ("k", "v")}
    seqs = [3, 1]
    caches = [[{"k": blocks[(l, "k")][b], "v": blocks[(l, "v")][b]} for l in range(cfg.n_layers)] for b in seqs]
    ids = I.prompt_ids(cfg).reshape(-1)[seqs]
    ref = L.decode_step(ids, caches, lambda r: m.rows("tok_embeddings", r), m.layer, m.get("norm"), m.get("output"),
                        OR.args_of(cfg))
    new_kv = []
    got = OR.decode(cfg, seqs, new_kv=new_kv)
    assert np.array_equal(got["logits"], ref["logits"])
    assert np.array_equal(got["ids"], ref["ids"])
    assert len(new_kv) == len(seqs) * cfg.n_layers


def _golden_script():
    spec = importlib.util.spec_from_file_location("make_prefill_8b_oracle",
                                                  os.path.join(GOLDEN, "make_prefill_8b_oracle.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_golden_script_composition_equals_oracle_prefill():
    G = _golden_script()
    cfg = _tiny(kind="prefill", S=30, B=1, n_layers=3, V=57)
    rows, depths = (0, 13, 29), (1, 3)
    got = G.run(cfg, rows=rows, depths=depths, log=lambda s: None)
    ref = OR.prefill(cfg, all_hidden=True)
    assert np.allclose(got["logits"], ref["logits"][0], rtol=1e-12, atol=1e-12)
    assert int(got["argmax"]) == int(ref["ids"][0])
    assert np.isclose(float(got["top2_gap"]), float(L.top2_gap(ref["logits"])[0]))
    assert np.allclose(got["hidden_rows"][-1], ref["hidden"][0][list(rows)], rtol=1e-6, atol=1e-6)
    one = OR.prefill(cfg, n_layers=1, all_hidden=True)
    assert np.allclose(got["hidden_rows"][0], one["hidden"][0][list(rows)], rtol=1e-6, atol=1e-6)


def test_golden_8b_prefill_file_matches_its_inputs():
    path = os.path.join(GOLDEN, "prefill_8b_s8192_oracle.npz")
    if not os.path.exists(path):
        pytest.skip("the stored 8B prefill result has not been generated")
    G = _golden_script()
    z = np.load(path, allow_pickle=False)
    cfg = I.CONFIGS["c4"]
    assert str(z["ids_sha256"]) == G.ids_hash(I.prompt_ids(cfg)[0])
    lg = z["logits"]
    assert lg.shape == (cfg.vocab_size,) and np.all(np.isfinite(lg))
    assert int(z["argmax"]) == int(np.argmax(lg))
    s = np.sort(lg)
    assert np.isclose(float(z["top2_gap"]), s[-1] - s[-2])
    assert z["hidden_rows"].shape == (len(z["depths"]), len(z["rows"]), cfg.dim)
    assert int(z["depths"][-1]) == cfg.n_layers
    # logits = hf . W_out^T at a few vocabulary rows (the stored hf and logits agree)
    m = OR.model_of(cfg)
    vrows = np.array([0, int(z["argmax"]), cfg.vocab_size - 1])
    w = m.rows("output", vrows).astype(np.float64)
    assert np.allclose(w @ z["hf"], lg[vrows], rtol=1e-12, atol=1e-12)


def _script(name):
    spec = importlib.util.spec_from_file_location(name, os.path.join(GOLDEN, name + ".py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_golden_decode_script_equals_oracle_decode():
    G = _script("make_decode_8b_oracle")
    cfg = _tiny(kind="decode", S=1, B=5, n_layers=3, cache_len=7, V=300)
    got = G.run(cfg, seq_groups=2, kv_layers=(0, 2), log=lambda s: None)
    new_kv = []
    ref = OR.decode(cfg, list(range(cfg.batch)), new_kv=new_kv)
    lg = ref["logits"]
    assert np.array_equal(got["argmax"], ref["ids"])
    assert np.allclose(got["top2_gap"], L.top2_gap(lg))
    # (the oracle's LM head is one matrix product per call: grouping the
    # sequences differently changes the BLAS summation order, not the values
    # beyond rounding)
    assert np.allclose(got["stride_val"], lg[:, got["stride_idx"]], rtol=1e-12, atol=1e-12)
    for b in range(cfg.batch):
        assert got["top_idx"][b, 0] == ref["ids"][b]
        assert np.allclose(got["top_val"][b], np.sort(lg[b])[::-1][:G.TOPK], rtol=1e-12, atol=1e-12)
    for (b, l, k, v) in new_kv:
        if l in (0, 2):
            i = (0, 2).index(l)
            assert np.allclose(got["new_k"][i, b], k.reshape(-1), rtol=1e-6, atol=1e-6)
            assert np.allclose(got["new_v"][i, b], v.reshape(-1), rtol=1e-6, atol=1e-6)


def test_golden_8b_decode_file_matches_its_inputs():
    path = os.path.join(GOLDEN, "decode_8b_b64_oracle.npz")
    if not os.path.exists(path):
        pytest.skip("the stored 8B decode result has not been generated")
    z = np.load(path, allow_pickle=False)
    cfg = I.CONFIGS["c5"]
    import hashlib
    ids = I.prompt_ids(cfg).reshape(-1).astype(np.int32)
    assert str(z["ids_sha256"]) == hashlib.sha256(ids.tobytes()).hexdigest()
    assert z["argmax"].shape == (cfg.batch,)
    assert np.array_equal(z["argmax"], z["top_idx"][:, 0])
    assert np.allclose(z["top2_gap"], z["top_val"][:, 0] - z["top_val"][:, 1])
    assert np.all(z["max_abs"] >= np.abs(z["top_val"][:, 0]))
