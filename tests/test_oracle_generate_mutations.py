"""Planted mistakes in the oracle's sampler and generation loop must fail at
least one pin of ``tests/test_oracle_generate_pins.py`` (CPU only)."""
import inspect

import numpy as np
import pytest

import test_oracle_generate_pins as P
from oracle import llama as L

_orig_sample = L.sample_top_p
_orig_generate = L.generate


def _sample_inclusive_cut(logits, temperature, top_p, u):
    # drops every token whose running sum INCLUDING itself exceeds top_p
    l = np.asarray(logits, dtype=np.float64).reshape(-1)
    p = L.softmax(l / float(temperature))
    order = np.argsort(-p, kind="stable")
    ps = p[order]
    ks = np.where(np.cumsum(ps) > top_p, 0.0, ps)
    if ks.sum() == 0:
        ks[0] = ps[0]
    kept = np.zeros_like(p)
    kept[order] = ks
    c = np.cumsum(kept / kept.sum())
    return min(int(np.searchsorted(c, u, side="right")), int(np.nonzero(kept)[0][-1])), 1.0


def _sample_no_renormalise(logits, temperature, top_p, u):
    l = np.asarray(logits, dtype=np.float64).reshape(-1)
    p = L.softmax(l / float(temperature))
    order = np.argsort(-p, kind="stable")
    ps = p[order]
    ks = np.where(np.cumsum(ps) - ps > top_p, 0.0, ps)
    kept = np.zeros_like(p)
    kept[order] = ks
    c = np.cumsum(kept)  # not divided by the kept mass
    return min(int(np.searchsorted(c, u, side="right")), int(np.nonzero(kept)[0][-1])), 1.0


def _sample_reversed_ids(logits, temperature, top_p, u):
    # larger ids first, both for ties and for the draw order
    l = np.asarray(logits, dtype=np.float64).reshape(-1)
    t, m = _orig_sample(l[::-1], temperature, top_p, u)
    return len(l) - 1 - t, m


def _sample_no_temperature(logits, temperature, top_p, u):
    return _orig_sample(logits, 1.0, top_p, u)


def _generate_one_short(prompts, *a, max_gen_len, **kw):
    return _orig_generate(prompts, *a, max_gen_len=max(max_gen_len - 1, 0), **kw)


def _generate_ignores_eos(prompts, embed_rows, layer, norm_w, w_out, args, max_gen_len, eos_id, max_seq_len, **kw):
    outs = _orig_generate(prompts, embed_rows, layer, norm_w, w_out, args, max_gen_len=max_gen_len, eos_id=-1,
                          max_seq_len=max_seq_len, **kw)
    for o in outs:
        o["out_len"] = o["tokens"].index(eos_id) if eos_id in o["tokens"] else len(o["tokens"])
    return outs


MUTATIONS = {
    "sample_top_p/inclusive-cut": ("sample_top_p", _sample_inclusive_cut),
    "sample_top_p/no-renormalise": ("sample_top_p", _sample_no_renormalise),
    "sample_top_p/larger-ids-first": ("sample_top_p", _sample_reversed_ids),
    "sample_top_p/no-temperature": ("sample_top_p", _sample_no_temperature),
    "generate/one-token-short": ("generate", _generate_one_short),
    "generate/ignores-eos": ("generate", _generate_ignores_eos),
}


def _pins():
    out = []
    for name, fn in inspect.getmembers(P, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if params:
            argnames = [a.strip() for a in params[0].args[0].split(",")]
            for vals in params[0].args[1]:
                vals = vals if isinstance(vals, tuple) else (vals,)
                out.append((name, fn, dict(zip(argnames, vals))))
        else:
            out.append((name, fn, {}))
    return out


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_fails_a_generation_pin(mutation, monkeypatch):
    attr, bad = MUTATIONS[mutation]
    monkeypatch.setattr(L, attr, bad)
    failed = []
    for name, fn, kw in _pins():
        try:
            fn(**kw)
        except Exception:
            failed.append(name)
    assert failed, f"no pin caught mutation {mutation}"
