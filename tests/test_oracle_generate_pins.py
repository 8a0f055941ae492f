"""Pins of the oracle's generation loop and top-p sampler against what the
pages and the mathematics fix (no GPU).

[P2 6 "Inference"]: generate appends one model choice per position after the
prompt, greedy when the temperature is 0, else sample_top_p; it ends on the
end-of-text token or at the length limit, and the output is cut at the first
end-of-text token.  sample_top_p keeps the most probable tokens until the mass
ahead of a token exceeds p (the pages describe it as the smallest set of top
tokens whose cumulative probability passes p), renormalises and draws.
"""
import math

import numpy as np
import pytest

from oracle import brute as BR
from oracle import llama as L

from test_oracle_pins import _tiny_model, as_lists, tiny_args


# ---------------------------------------------------------------------------
# sample_top_p
# ---------------------------------------------------------------------------
def test_sampler_hand_worked_nucleus():
    # p = (0.5, 0.3, 0.15, 0.05), top_p = 0.7: masses ahead are 0, 0.5, 0.8,
    # 0.95, so tokens 2 and 3 are dropped; the nucleus {0, 1} renormalises to
    # (0.625, 0.375): u < 0.625 draws token 0, u >= 0.625 draws token 1.
    lg = np.log([0.5, 0.3, 0.15, 0.05])
    for u, want in [(0.0, 0), (0.3, 0), (0.62, 0), (0.63, 1), (0.9, 1), (0.999, 1)]:
        tok, m = L.sample_top_p(lg, 1.0, 0.7, u)
        assert tok == want, (u, tok)
    _, m = L.sample_top_p(lg, 1.0, 0.7, 0.62)
    assert m == pytest.approx(0.005, abs=1e-12)
    # p = 0.85 keeps token 2 as well (mass ahead 0.8 <= 0.85): (0.5, 0.3, 0.15) / 0.95
    # cumulative 0.5263, 0.8421, 1
    for u, want in [(0.5, 0), (0.53, 1), (0.84, 1), (0.843, 2), (0.99, 2)]:
        assert L.sample_top_p(lg, 1.0, 0.85, u)[0] == want, u


def test_sampler_full_nucleus_is_inverse_cdf_of_softmax():
    # top_p >= 1 keeps everything: the draw is the inverse CDF of softmax(l / T)
    rng = np.random.default_rng(40)
    lg = rng.normal(0, 2.0, 50)
    T = 0.7
    e = np.exp((lg - lg.max()) / T)
    cdf = np.cumsum(e / e.sum())
    for u in rng.uniform(0, 1, 40):
        want = int(np.argmax(cdf > u))
        assert L.sample_top_p(lg, T, 1.0, u)[0] == want


def test_sampler_zero_top_p_is_argmax():
    rng = np.random.default_rng(41)
    for _ in range(20):
        lg = rng.normal(0, 1.0, 30)
        for u in (0.0, 0.5, 0.99):
            assert L.sample_top_p(lg, 0.8, 0.0, u)[0] == int(np.argmax(lg))


def _shortest_prefix_nucleus(p, top_p):
    """The pages' prose: the smallest set of most probable tokens whose
    cumulative probability passes top_p (all tokens when none does)."""
    order = sorted(range(len(p)), key=lambda i: (-p[i], i))
    acc, keep = 0.0, []
    for i in order:
        keep.append(i)
        acc += p[i]
        if acc > top_p:
            break
    return sorted(keep)


@pytest.mark.parametrize("top_p", [0.1, 0.5, 0.9, 0.97])
def test_sampler_nucleus_is_shortest_prefix_passing_p(top_p):
    rng = np.random.default_rng(42)
    for _ in range(30):
        lg = rng.normal(0, 1.5, 12)
        e = np.exp(lg - lg.max())
        p = e / e.sum()
        keep = _shortest_prefix_nucleus(p.tolist(), top_p)
        # the set of tokens some u can draw is exactly the nucleus, and each is
        # drawn with probability proportional to p
        q = np.zeros_like(p)
        q[keep] = p[keep] / p[keep].sum()
        cdf = np.cumsum(q)
        for u in np.linspace(0.0005, 0.9995, 200):
            want = int(np.argmax(cdf > u))
            assert L.sample_top_p(lg, 1.0, top_p, u)[0] == want


def test_sampler_ties_keep_smaller_ids_first():
    # four equal tokens (p = 0.25 each), top_p = 0.3: the first two by id stay
    lg = np.zeros(4)
    assert [L.sample_top_p(lg, 1.0, 0.3, u)[0] for u in (0.1, 0.4, 0.6, 0.9)] == [0, 0, 1, 1]
    lg = np.array([0.0, 1.0, 0.0, 1.0, 0.0])  # ties at the top between ids 1 and 3
    assert L.sample_top_p(lg, 1.0, 0.0, 0.9)[0] == 1


def test_sampler_temperature_scales_logits():
    rng = np.random.default_rng(43)
    lg = rng.normal(0, 1.0, 40)
    for u in rng.uniform(0, 1, 20):
        assert L.sample_top_p(lg, 0.5, 0.8, u)[0] == L.sample_top_p(lg * 2.0, 1.0, 0.8, u)[0]
    # T -> 0 concentrates on the argmax
    assert L.sample_top_p(lg, 1e-4, 0.9, 0.99)[0] == int(np.argmax(lg))


# ---------------------------------------------------------------------------
# generate
# ---------------------------------------------------------------------------
def _brute_greedy(prompt, max_gen, eos, max_seq, emb, layers, norm_w, w_out, a):
    """Greedy generation by recomputing the whole sequence every step (no cache)."""
    toks = list(prompt)
    total = min(len(prompt) + max_gen, max_seq)
    while len(toks) < total:
        _, _, best = BR.forward(toks, emb.tolist(), [as_lists(lw) for lw in layers], norm_w.tolist(),
                                w_out.tolist(), a)
        toks.append(best)
        if best == eos:
            break
    return toks


def test_greedy_generate_matches_recompute_from_scratch():
    rng = np.random.default_rng(44)
    a = tiny_args(theta=500000.0)
    layers, emb, norm_w, w_out = _tiny_model(rng, a)
    prompts = [[3, 1, 4], [1, 5, 9, 2, 6], [7]]
    outs = L.generate(prompts, lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a, max_gen_len=6, eos_id=-1,
                      max_seq_len=10)
    for pr, o in zip(prompts, outs):
        want = _brute_greedy(pr, 6, -1, 10, emb, layers, norm_w, w_out, a)
        assert o["tokens"] == want
        assert len(o["tokens"]) == min(len(pr) + 6, 10)
        assert o["out_len"] == len(want)
        assert o["choices"] == want[len(pr):]


def test_generate_stops_at_eos_and_cuts_output():
    rng = np.random.default_rng(45)
    a = tiny_args(theta=500000.0)
    layers, emb, norm_w, w_out = _tiny_model(rng, a)
    prompt = [2, 7, 1]
    free = L.generate([prompt], lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a, max_gen_len=8, eos_id=-1,
                      max_seq_len=32)[0]["tokens"]
    gen = free[len(prompt):]
    eos = next(t for t in gen[1:] if t not in prompt)  # a generated token that is not in the prompt
    first = gen.index(eos)
    assert first >= 1
    o = L.generate([prompt], lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a, max_gen_len=8, eos_id=eos,
                   max_seq_len=32)[0]
    assert o["tokens"] == free[:len(prompt) + first + 1]
    assert o["out_len"] == len(prompt) + first
    # an end-of-text token inside the prompt cuts the output there but does not stop generation
    o2 = L.generate([[2, eos, 1]], lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a, max_gen_len=3,
                    eos_id=eos, max_seq_len=32)[0]
    assert o2["out_len"] == 1 and len(o2["tokens"]) >= 4 and o2["tokens"][:3] == [2, eos, 1]


def test_generate_zero_budget_and_full_context():
    rng = np.random.default_rng(46)
    a = tiny_args(theta=500000.0)
    layers, emb, norm_w, w_out = _tiny_model(rng, a)
    o = L.generate([[1, 2, 3]], lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a, max_gen_len=0, eos_id=-1,
                   max_seq_len=8)[0]
    assert o["tokens"] == [1, 2, 3] and o["choices"] == []
    o = L.generate([[1, 2, 3, 4]], lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a, max_gen_len=5,
                   eos_id=-1, max_seq_len=4)[0]
    assert o["tokens"] == [1, 2, 3, 4]


def test_forced_path_reports_choices_along_it():
    rng = np.random.default_rng(47)
    a = tiny_args(theta=500000.0)
    layers, emb, norm_w, w_out = _tiny_model(rng, a)
    prompt = [4, 4, 2]
    own = L.generate([prompt], lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a, max_gen_len=5, eos_id=-1,
                     max_seq_len=16)[0]
    forced = list(own["tokens"])
    forced[4] = (forced[4] + 1) % a["vocab_size"]  # divert the path after the second generated token
    f = L.generate([prompt], lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a, max_gen_len=5, eos_id=-1,
                   max_seq_len=16, forced=[forced])[0]
    assert f["tokens"] == forced
    assert f["choices"][:2] == own["choices"][:2]
    # after the diversion the choices follow the forced path: recompute from scratch
    _, _, best = BR.forward(forced[:5], emb.tolist(), [as_lists(lw) for lw in layers], norm_w.tolist(),
                            w_out.tolist(), a)
    assert f["choices"][2] == best


def test_sampled_generate_uses_one_uniform_per_generated_token():
    rng = np.random.default_rng(48)
    a = tiny_args(theta=500000.0)
    layers, emb, norm_w, w_out = _tiny_model(rng, a)
    prompts = [[3, 1], [5, 9, 2]]
    U = rng.uniform(0, 1, (6, 2))
    outs = L.generate(prompts, lambda r: emb[r], lambda l: layers[l], norm_w, w_out, a, max_gen_len=6, eos_id=-1,
                      max_seq_len=16, temperature=0.6, top_p=0.9, uniforms=U)
    for b, (pr, o) in enumerate(zip(prompts, outs)):
        toks = list(pr)
        for g in range(6):
            _, logits, _ = BR.forward(toks, emb.tolist(), [as_lists(lw) for lw in layers], norm_w.tolist(),
                                      w_out.tolist(), a)
            toks.append(L.sample_top_p(np.array(logits), 0.6, 0.9, U[g][b])[0])
        assert o["tokens"] == toks
