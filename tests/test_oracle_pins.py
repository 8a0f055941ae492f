"""Pins of the fp64 oracle against what the pages and mathematics fix.

CPU only.  Each test names the passage it pins.  Pages:
  [P1] "机器学习 | 从0开发大模型—译llama3-from-scratch"
  [P2] "Build your own Llama 3 architecture from scratch" notes
  [P3] "大语言模型实现llama3-from-scratch：输出层与预测"
  [P4] joto.ai post on the Llama architecture
"""
import math
import os

import numpy as np
import pytest

from oracle import brute as BR
from oracle import llama as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def tiny_layer(rng, D=16, H=4, G=2, F=24, norm_std=0.1):
    hd = D // H
    s = 0.3
    lw = {
        "wq": rng.normal(0, s, (H * hd, D)), "wk": rng.normal(0, s, (G * hd, D)),
        "wv": rng.normal(0, s, (G * hd, D)), "wo": rng.normal(0, s, (D, H * hd)),
        "w1": rng.normal(0, s, (F, D)), "w2": rng.normal(0, s, (D, F)), "w3": rng.normal(0, s, (F, D)),
        "attention_norm": 1.0 + rng.normal(0, norm_std, D), "ffn_norm": 1.0 + rng.normal(0, norm_std, D),
    }
    return lw


def tiny_args(D=16, H=4, G=2, L_=2, V=11, eps=1e-5, theta=500000.0):
    return dict(dim=D, n_layers=L_, n_heads=H, n_kv_heads=G, vocab_size=V, norm_eps=eps, rope_theta=theta)


def as_lists(lw):
    return {k: v.tolist() for k, v in lw.items()}


# ---------------------------------------------------------------------------
# RoPE frequency table: printed values [P1 6.7]
# ---------------------------------------------------------------------------
def test_rope_frequencies_match_printed_table():
    printed = np.array([float(r[0]) for r in _read_golden("rope_freqs_theta500000_hd128.txt")])
    assert printed.shape == (64,)
    got = L.rope_frequencies(128, 500000.0)
    # 5 significant figures: half a unit in the 4th decimal of the mantissa
    half_ulp = 0.5e-4 * 10.0 ** np.floor(np.log10(printed))
    assert np.all(np.abs(got - printed) <= half_ulp * 1.0001), np.max(np.abs(got - printed) / half_ulp)


def test_rope_frequencies_use_head_dim_not_model_dim():
    # [P2 3.4 passes dim=self.head_dim]: for hd=128 the last frequency is 500000^(-126/128).
    f = L.rope_frequencies(128, 500000.0)
    assert f[0] == 1.0
    assert math.isclose(f[-1], 500000.0 ** (-126 / 128), rel_tol=1e-14)
    assert len(L.rope_frequencies(96, 500000.0)) == 48


# ---------------------------------------------------------------------------
# Causal mask: printed 17x17 [P1 7.1]
# ---------------------------------------------------------------------------
def test_causal_mask_matches_printed_17x17():
    rows = _read_golden("causal_mask_17.txt")
    printed = np.array([[-np.inf if t == "-inf" else 0.0 for t in r] for r in rows])
    assert printed.shape == (17, 17)
    got = L.causal_mask(np.arange(17), np.arange(17))
    assert np.array_equal(got, printed)


def test_causal_mask_with_offset_positions():
    # chunked / decode queries at absolute positions see keys 0..p (reading A6)
    got = L.causal_mask(np.array([3, 4]), np.arange(6))
    assert np.array_equal(np.isinf(got), np.array([[0, 0, 0, 0, 1, 1], [0, 0, 0, 0, 0, 1]], dtype=bool))


# ---------------------------------------------------------------------------
# RMSNorm [P1 5; P2 3.1; P3]
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("c", [1e-3, 0.5, 3.0, -7.0])
def test_rmsnorm_constant_row_closed_form(c):
    eps = 1e-5
    y = L.rms_norm(np.full((2, 64), c), np.ones(64), eps)
    assert np.allclose(y, c / math.sqrt(c * c + eps), rtol=1e-14, atol=0)


def test_rmsnorm_output_rms_and_scale_invariance():
    rng = np.random.default_rng(0)
    x = rng.normal(0, 2.0, (5, 96))
    eps = 1e-5
    y = L.rms_norm(x, np.ones(96), eps)
    m = np.mean(x * x, axis=-1)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), np.sqrt(m / (m + eps)), rtol=1e-13)
    y0 = L.rms_norm(x, np.ones(96), 0.0)
    assert np.allclose(L.rms_norm(x * 37.0, np.ones(96), 0.0), y0, rtol=1e-13)


def test_rmsnorm_weight_and_brute_force():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 1, 40)
    w = rng.normal(1, 0.3, 40)
    assert np.allclose(L.rms_norm(x, w, 1e-5), BR.rms_norm(x.tolist(), w.tolist(), 1e-5), rtol=1e-13)
    # the weight multiplies per element after normalizing
    assert np.allclose(L.rms_norm(x, w, 1e-5), L.rms_norm(x, np.ones(40), 1e-5) * w, rtol=1e-14)


# ---------------------------------------------------------------------------
# RoPE [P1 6.6-6.9; P2 3.2; P4]
# ---------------------------------------------------------------------------
def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(2)
    x = rng.normal(size=(1, 3, 64))
    assert np.array_equal(L.apply_rope(x, [0], 500000.0), x)


def test_rope_first_pair_rotates_counterclockwise_by_p():
    # theta_0 = 1, so at position p the first pair turns by p radians: (1,0) -> (cos p, sin p)
    x = np.zeros((1, 1, 4))
    x[0, 0, 0] = 1.0
    y = L.apply_rope(x, [2], 500000.0)
    assert np.allclose(y[0, 0], [math.cos(2), math.sin(2), 0, 0], atol=1e-15)


def test_rope_pairs_are_adjacent_elements():
    # element 1 pairs with element 0 (not with element hd/2 + 1 as in a rotate-half layout)
    x = np.zeros((1, 1, 8))
    x[0, 0, 1] = 1.0
    y = L.apply_rope(x, [1], 500000.0)
    assert np.allclose(y[0, 0], [-math.sin(1), math.cos(1), 0, 0, 0, 0, 0, 0], atol=1e-15)


def test_rope_preserves_pair_norms_and_inverts():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(6, 2, 128))
    pos = np.array([0, 5, 17, 1000, 4096, 8191])
    y = L.apply_rope(x, pos, 500000.0)
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-12)
    back = L.apply_rope(y, -pos, 500000.0)
    assert np.allclose(back, x, atol=1e-11)


def test_rope_scores_depend_only_on_relative_position():
    # [P2 3.2; P4]: q_m . k_n depends only on m - n
    rng = np.random.default_rng(4)
    q = rng.normal(size=(1, 1, 128))
    k = rng.normal(size=(1, 1, 128))
    for m, n, d in [(7, 3, 100), (0, 0, 4096), (50, 90, 8000)]:
        a = np.dot(L.apply_rope(q, [m], 5e5).ravel(), L.apply_rope(k, [n], 5e5).ravel())
        b = np.dot(L.apply_rope(q, [m + d], 5e5).ravel(), L.apply_rope(k, [n + d], 5e5).ravel())
        assert math.isclose(a, b, rel_tol=1e-9, abs_tol=1e-9)


def test_rope_equals_block_diagonal_rotation_matrix():
    # [P4]: dim/2 independent 2-D rotations (brute oracle builds each 2x2 block with cos/sin)
    rng = np.random.default_rng(5)
    x = rng.normal(size=(3, 1, 16))
    pos = [1, 9, 333]
    y = L.apply_rope(x, pos, 10000.0)
    for s, p in enumerate(pos):
        assert np.allclose(y[s, 0], BR.rope_vec(x[s, 0].tolist(), p, 10000.0), atol=1e-12)


# ---------------------------------------------------------------------------
# Attention [P1 6.11-8; P2 3.4]
# ---------------------------------------------------------------------------
def _rand_qkv(rng, S=5, H=4, G=2, hd=4, L_=None):
    L_ = S if L_ is None else L_
    return rng.normal(size=(S, H, hd)), rng.normal(size=(L_, G, hd)), rng.normal(size=(L_, G, hd))


def test_attention_first_row_is_first_value():
    rng = np.random.default_rng(6)
    q, k, v = _rand_qkv(rng)
    o = L.attention(q, k, v, np.arange(5), np.arange(5)).reshape(5, 4, 4)
    for h in range(4):
        assert np.allclose(o[0, h], v[0, h // 2], atol=1e-15)


def test_attention_zero_query_gives_prefix_mean():
    rng = np.random.default_rng(7)
    q, k, v = _rand_qkv(rng, S=6)
    q[:] = 0.0
    o = L.attention(q, k, v, np.arange(6), np.arange(6)).reshape(6, 4, 4)
    for i in range(6):
        for h in range(4):
            assert np.allclose(o[i, h], v[: i + 1, h // 2].mean(axis=0), atol=1e-14)


def test_attention_probabilities_rows_sum_to_one_and_mask_is_exact_zero():
    rng = np.random.default_rng(8)
    q, k, v = _rand_qkv(rng, S=7)
    _, p = L.attention(q, k, v, np.arange(7), np.arange(7), return_probs=True)
    assert np.allclose(p.sum(-1), 1.0, rtol=1e-14)
    assert np.all(p[:, np.triu_indices(7, 1)[0], np.triu_indices(7, 1)[1]] == 0.0)


def test_attention_two_key_closed_form_pins_scale():
    # query at position 1 sees two keys; P(key 1) = 1 / (1 + exp((s0 - s1)/sqrt(hd)))
    hd = 16
    q = np.zeros((2, 1, hd)); q[1, 0, 0] = 2.0
    k = np.zeros((2, 1, hd)); k[0, 0, 0] = 1.0; k[1, 0, 0] = 3.0
    v = np.zeros((2, 1, hd)); v[1, 0, 5] = 1.0
    o = L.attention(q, k, v, np.arange(2), np.arange(2))
    p1 = 1.0 / (1.0 + math.exp((2.0 - 6.0) / math.sqrt(hd)))
    assert math.isclose(o[1, 5], p1, rel_tol=1e-14)


def _repeat_kv_expand(x, n_rep):
    # [L, G, hd] -> [L, G*n_rep, hd]: new axis after the KV axis, expanded, then flattened
    Lk, G, hd = x.shape
    return np.broadcast_to(x[:, :, None, :], (Lk, G, n_rep, hd)).reshape(Lk, G * n_rep, hd)


@pytest.mark.parametrize("H,G", [(8, 2), (4, 4), (4, 1), (6, 3)])
def test_gqa_equals_mha_with_repeated_kv(H, G):
    # [P2 3.4 repeat_kv; MHA when G == H, MQA when G == 1]
    rng = np.random.default_rng(9)
    q, k, v = _rand_qkv(rng, S=6, H=H, G=G, hd=8)
    gqa = L.attention(q, k, v, np.arange(6), np.arange(6))
    mha = L.attention(q, _repeat_kv_expand(k, H // G), _repeat_kv_expand(v, H // G), np.arange(6), np.arange(6))
    assert np.allclose(gqa, mha, atol=1e-14)


def test_gqa_head_group_is_contiguous():
    # head h must read KV head h // n_rep: give KV head 1 a distinct value and look which q heads see it
    S, H, G, hd = 1, 4, 2, 4
    q = np.zeros((S, H, hd)); k = np.zeros((S, G, hd)); v = np.zeros((S, G, hd))
    v[0, 1, :] = 1.0
    o = L.attention(q, k, v, [0], [0]).reshape(H, hd)
    assert np.array_equal(o[:, 0], [0.0, 0.0, 1.0, 1.0])


# ---------------------------------------------------------------------------
# FFN [P1 9.3; P2 3.5]
# ---------------------------------------------------------------------------
def test_ffn_hidden_dims():
    assert L.ffn_hidden_dim(4096, 1024, 1.3) == 14336  # value printed for the 8B model [P2 3.5]
    assert L.ffn_hidden_dim(512, 256, None) == 1536
    assert L.ffn_hidden_dim(768, 256, None) == 2048


def test_silu_special_values():
    assert L.silu(0.0) == 0.0
    assert math.isclose(float(L.silu(1.0)), 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    assert math.isclose(float(L.silu(40.0)), 40.0, rel_tol=1e-15)
    assert abs(float(L.silu(-40.0))) < 1e-15


def test_ffn_zero_gate_weight_gives_zero_and_brute_force():
    rng = np.random.default_rng(10)
    x = rng.normal(size=(3, 16))
    w1, w2, w3 = rng.normal(size=(24, 16)), rng.normal(size=(16, 24)), rng.normal(size=(24, 16))
    assert np.all(L.feed_forward(x, np.zeros_like(w1), w2, w3) == 0.0)
    for s in range(3):
        g = BR.matvec(w1.tolist(), x[s].tolist())
        u = BR.matvec(w3.tolist(), x[s].tolist())
        ref = BR.matvec(w2.tolist(), [BR.silu(g[i]) * u[i] for i in range(24)])
        assert np.allclose(L.feed_forward(x[s:s + 1], w1, w2, w3)[0], ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Decoder block [P2 3.6; P1 9-10]
# ---------------------------------------------------------------------------
def test_block_with_zero_output_projections_is_identity():
    rng = np.random.default_rng(11)
    lw = tiny_layer(rng)
    lw["wo"][:] = 0.0
    lw["w2"][:] = 0.0
    h = rng.normal(size=(5, 16))
    assert np.array_equal(L.layer_forward(h, lw, tiny_args(), np.arange(5)), h)


@pytest.mark.parametrize("H,G", [(4, 2), (4, 4), (4, 1)])
def test_layer_matches_brute_force(H, G):
    rng = np.random.default_rng(12)
    lw = tiny_layer(rng, H=H, G=G)
    a = tiny_args(H=H, G=G, theta=10000.0)
    h = rng.normal(size=(5, 16))
    got = L.layer_forward(h, lw, a, np.arange(5))
    ref, _, _ = BR.layer_forward(h.tolist(), as_lists(lw), a)
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-11)


def test_layer_with_cache_matches_brute_force_offset():
    # a chunk at positions 3..5 attending over a cache of positions 0..2 [P2 3.3]
    rng = np.random.default_rng(13)
    lw = tiny_layer(rng)
    a = tiny_args(theta=10000.0)
    h = rng.normal(size=(6, 16))
    full = L.layer_forward(h, lw, a, np.arange(6))
    cache = {"k": np.zeros((0, 2, 4)), "v": np.zeros((0, 2, 4))}
    L.layer_forward(h[:3], lw, a, np.arange(3), cache=cache)
    tail = L.layer_forward(h[3:], lw, a, np.arange(3, 6), cache=cache)
    assert np.allclose(tail, full[3:], rtol=1e-12, atol=1e-12)
    _, bk, bv = BR.layer_forward(h[:3].tolist(), as_lists(lw), a)
    bref, _, _ = BR.layer_forward(h[3:].tolist(), as_lists(lw), a, pos0=3, past_k=bk, past_v=bv)
    assert np.allclose(tail, bref, rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------------------
# Output head [P1 11-12; P3]
# ---------------------------------------------------------------------------
def test_lm_head_brute_force_and_argmax_ties():
    rng = np.random.default_rng(14)
    hf = rng.normal(size=(2, 16))
    w = rng.normal(size=(11, 16))
    lg = L.lm_head(hf, w)
    for b in range(2):
        assert np.allclose(lg[b], BR.matvec(w.tolist(), hf[b].tolist()), rtol=1e-13)
    t = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0]])
    assert L.argmax_first(t).tolist() == [1, 0]
    assert np.allclose(L.top2_gap(np.array([[0.0, 2.5, 1.0]])), [1.5])


# ---------------------------------------------------------------------------
# Whole stack
# ---------------------------------------------------------------------------
def _tiny_model(rng, a, F=24):
    D, V = a["dim"], a["vocab_size"]
    layers = [tiny_layer(rng, D=D, H=a["n_heads"], G=a["n_kv_heads"], F=F) for _ in range(a["n_layers"])]
    emb = rng.normal(0, 1.0, (V, D))
    norm_w = 1.0 + rng.normal(0, 0.1, D)
    w_out = rng.normal(0, 0.5, (V, D))
    return layers, emb, norm_w, w_out


def test_stack_matches_brute_force():
    rng = np.random.default_rng(15)
    a = tiny_args(theta=10000.0)
    layers, emb, norm_w, w_out = _tiny_model(rng, a)
    ids = np.array([[3, 1, 4, 1, 5], [9, 2, 6, 5, 3]])
    out = L.prefill(ids, lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a, all_hidden=True)
    for b in range(2):
        h, logits, best = BR.forward(ids[b].tolist(), emb.tolist(), [as_lists(lw) for lw in layers],
                                     norm_w.tolist(), w_out.tolist(), a)
        assert np.allclose(out["hidden"][b], h, rtol=1e-11, atol=1e-11)
        assert np.allclose(out["logits"][b], logits, rtol=1e-10, atol=1e-10)
        assert out["ids"][b] == best


def test_prefill_last_row_equals_decode_after_shorter_prefill():
    # KV-cache identity [P2 3.3]: decode at p = S-1 after prefill(S-1) reproduces prefill(S)'s last row
    rng = np.random.default_rng(16)
    a = tiny_args(theta=500000.0)
    layers, emb, norm_w, w_out = _tiny_model(rng, a)
    ids = np.array([[3, 1, 4, 1, 5, 9], [2, 7, 1, 8, 2, 8]])
    full = L.prefill(ids, lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a)
    caches = [[], []]
    L.prefill(ids[:, :-1], lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a, caches=caches)
    dec = L.decode_step(ids[:, -1], caches, lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a)
    assert np.allclose(dec["logits"], full["logits"], rtol=1e-11, atol=1e-11)
    assert np.array_equal(dec["ids"], full["ids"])


def test_prefill_is_causal():
    rng = np.random.default_rng(17)
    a = tiny_args(theta=500000.0)
    layers, emb, norm_w, w_out = _tiny_model(rng, a)
    ids = np.array([[3, 1, 4, 1, 5, 9]])
    ids2 = ids.copy()
    ids2[0, 4:] = [10, 0]
    h1 = L.prefill(ids, lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a, all_hidden=True)["hidden"]
    h2 = L.prefill(ids2, lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a, all_hidden=True)["hidden"]
    assert np.array_equal(h1[0, :4], h2[0, :4])
    assert not np.allclose(h1[0, 4:], h2[0, 4:])


# ---------------------------------------------------------------------------
# Document-level attention mask [P2 appendix item 1]
# ---------------------------------------------------------------------------
def test_document_mask_single_document_is_causal():
    pos = np.arange(7)
    assert np.array_equal(L.document_mask(pos, pos, [3] * 7), L.causal_mask(pos, pos))


def test_document_mask_runs_and_offsets():
    # ids [5, 5, 9, 9, 9, 5]: documents {0,1}, {2,3,4}, {5} (a repeated id after
    # another document starts a new document)
    m = L.document_mask(np.arange(6), np.arange(6), [5, 5, 9, 9, 9, 5])
    vis = np.isfinite(m)
    want = np.zeros((6, 6), dtype=bool)
    for q, k in [(0, 0), (1, 0), (1, 1), (2, 2), (3, 2), (3, 3), (4, 2), (4, 3), (4, 4), (5, 5)]:
        want[q, k] = True
    assert np.array_equal(vis, want)
    # queries at later positions (chunk after a cache)
    m2 = L.document_mask(np.array([4, 5]), np.arange(6), [5, 5, 9, 9, 9, 5])
    assert np.array_equal(np.isfinite(m2), want[4:6])


def test_one_token_documents_attend_to_themselves():
    rng = np.random.default_rng(30)
    q, k, v = _rand_qkv(rng, S=6, H=4, G=2, hd=4)
    pos = np.arange(6)
    o = L.attention(q, k, v, pos, pos, doc_ids=np.arange(6)).reshape(6, 4, 4)
    for h in range(4):
        assert np.allclose(o[:, h], v[:, h // 2], rtol=1e-13, atol=1e-13)


def test_packed_documents_equal_separate_sequences():
    # RoPE makes scores depend on relative positions only [P2 3.2], so under
    # the document mask a document packed after another gives the hidden
    # states it gives alone from position 0
    rng = np.random.default_rng(31)
    a = tiny_args(theta=500000.0, L_=2)
    layers, emb, norm_w, w_out = _tiny_model(rng, a)
    d1, d2, d3 = [3, 1, 4, 1], [5, 9, 2], [6, 5]
    packed = np.array([d1 + d2 + d3])
    docs = np.array([[0] * 4 + [1] * 3 + [0] * 2])  # the third document reuses id 0
    out = L.prefill(packed, lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a, all_hidden=True,
                    doc_ids=docs)["hidden"][0]
    off = 0
    for d in (d1, d2, d3):
        alone = L.prefill(np.array([d]), lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a,
                          all_hidden=True)["hidden"][0]
        assert np.allclose(out[off:off + len(d)], alone, rtol=1e-10, atol=1e-10)
        off += len(d)
    # and without the mask the later documents do change
    plain = L.prefill(packed, lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a, all_hidden=True)["hidden"][0]
    assert not np.allclose(plain[4:], out[4:])
