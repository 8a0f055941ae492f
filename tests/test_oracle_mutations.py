"""Planted mistakes in the oracle must fail at least one pin.

CPU only.  Each mutation below is a plausible error in ``oracle.llama`` (a
dropped term, a wrong sign or index, a transposed operand, a swapped
convention).  The test patches it in, runs every pin of
``tests/test_oracle_pins.py`` and requires that at least one of them fails;
this shows the pins constrain each part of the oracle.
"""
import inspect
import math

import numpy as np
import pytest

import test_oracle_pins as P
from oracle import llama as L

_orig = {n: getattr(L, n) for n in ("rope_frequencies", "apply_rope", "attention", "causal_mask", "rms_norm",
                                    "feed_forward", "layer_forward", "argmax_first", "silu", "softmax",
                                    "ffn_hidden_dim", "lm_head", "document_mask")}


def _docmask_same_id(q_positions, k_positions, doc_ids):
    # treats equal ids as one document even when another document lies between
    doc = np.asarray(doc_ids).reshape(-1)
    qp, kp = np.asarray(q_positions), np.asarray(k_positions)
    vis = (kp[None, :] <= qp[:, None]) & (doc[kp][None, :] == doc[qp][:, None])
    return np.where(vis, 0.0, -np.inf)


def _docmask_strict_diagonal(q_positions, k_positions, doc_ids):
    # drops the query's own key
    m = _orig["document_mask"](q_positions, k_positions, doc_ids)
    qp, kp = np.asarray(q_positions), np.asarray(k_positions)
    return np.where(kp[None, :] == qp[:, None], -np.inf, m)


def _rope_freq_no_two(hd, theta):
    i = np.arange(hd // 2, dtype=np.float64)
    return 1.0 / (theta ** (i / hd))


def _rope_rotate_half(x, positions, theta):
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    rot = L.rope_rotations(positions, hd, theta)
    z = x[..., : hd // 2] + 1j * x[..., hd // 2:]
    z = z * rot[:, None, :]
    return np.concatenate([z.real, z.imag], axis=-1)


def _rope_clockwise(x, positions, theta):
    return _orig["apply_rope"](x, -np.asarray(positions), theta)


def _attention_mod_group(q, k, v, qp, kp, return_probs=False):
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    S, H, hd = q.shape
    G = k.shape[1]
    mask = L.causal_mask(qp, kp)
    out = np.empty((S, H, hd))
    probs = []
    for h in range(H):
        g = h % G
        p = L.softmax(q[:, h] @ k[:, g].T / math.sqrt(hd) + mask)
        out[:, h] = p @ v[:, g]
        probs.append(p)
    o = out.reshape(S, H * hd)
    return (o, np.stack(probs)) if return_probs else o


def _attention_no_scale(q, k, v, qp, kp, return_probs=False):
    q = np.asarray(q, dtype=np.float64) * math.sqrt(np.asarray(q).shape[-1])
    return _orig["attention"](q, k, v, qp, kp, return_probs)


def _mask_diag0(qp, kp):
    qp = np.asarray(qp)[:, None]
    kp = np.asarray(kp)[None, :]
    return np.where(kp >= qp, -np.inf, 0.0)


def _rms_eps_outside(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * np.asarray(w, dtype=np.float64)


def _rms_sum(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, dtype=np.float64)


def _ffn_swapped(xn, w1, w2, w3):
    return _orig["feed_forward"](xn, w3, w2, w1)


def _ffn_w2_transposed(xn, w1, w2, w3):
    xn = np.asarray(xn, dtype=np.float64)
    u = L.silu(xn @ np.asarray(w1).T) * (xn @ np.asarray(w3).T)
    w2 = np.asarray(w2, dtype=np.float64)
    return u @ w2.reshape(w2.shape[1], w2.shape[0])


def _layer_no_attn_residual(h, lw, args, positions, cache=None, taps=None):
    lw2 = dict(lw)
    out = _orig["layer_forward"](h, lw2, args, positions, cache=cache, taps=taps)
    # remove the residual of the attention half: out - h
    return out - np.asarray(h, dtype=np.float64)


def _argmax_last(logits):
    lg = np.asarray(logits, dtype=np.float64)
    return (lg.shape[-1] - 1 - np.argmax(lg[..., ::-1], axis=-1)).astype(np.int64)


def _silu_wrong_sign(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(x))


def _ffn_dim_no_two_thirds(dim, multiple_of, mult):
    hidden = 4 * dim
    if mult is not None:
        hidden = int(mult * hidden)
    return multiple_of * ((hidden + multiple_of - 1) // multiple_of)


def _softmax_no_max(s, axis=-1):
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s)
    return e / (np.sum(e, axis=axis, keepdims=True) + 1e-3)


MUTATIONS = {
    "rope_frequencies/no-factor-2": ("rope_frequencies", _rope_freq_no_two),
    "apply_rope/rotate-half": ("apply_rope", _rope_rotate_half),
    "apply_rope/clockwise": ("apply_rope", _rope_clockwise),
    "attention/group=h%G": ("attention", _attention_mod_group),
    "attention/no-1/sqrt(hd)": ("attention", _attention_no_scale),
    "causal_mask/diagonal-0": ("causal_mask", _mask_diag0),
    "rms_norm/eps-outside-root": ("rms_norm", _rms_eps_outside),
    "rms_norm/sum-not-mean": ("rms_norm", _rms_sum),
    "feed_forward/w1<->w3": ("feed_forward", _ffn_swapped),
    "feed_forward/w2-transposed": ("feed_forward", _ffn_w2_transposed),
    "layer_forward/no-attn-residual": ("layer_forward", _layer_no_attn_residual),
    "argmax_first/last-on-ties": ("argmax_first", _argmax_last),
    "silu/sign": ("silu", _silu_wrong_sign),
    "ffn_hidden_dim/no-2/3": ("ffn_hidden_dim", _ffn_dim_no_two_thirds),
    "softmax/biased-denominator": ("softmax", _softmax_no_max),
    "document_mask/same-id-across-documents": ("document_mask", _docmask_same_id),
    "document_mask/no-diagonal": ("document_mask", _docmask_strict_diagonal),
}


def _pins():
    out = []
    for name, fn in inspect.getmembers(P, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argnames, values = params[0].args[0], params[0].args[1]
            argnames = [a.strip() for a in argnames.split(",")]
            for vals in values:
                vals = vals if isinstance(vals, tuple) else (vals,)
                out.append((name, fn, dict(zip(argnames, vals))))
        else:
            out.append((name, fn, {}))
    return out


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(mutation, monkeypatch):
    attr, bad = MUTATIONS[mutation]
    monkeypatch.setattr(L, attr, bad)
    failed = []
    for name, fn, kw in _pins():
        try:
            fn(**kw)
        except Exception:  # AssertionError or a shape error caused by the mutation
            failed.append(name)
    assert failed, f"no pin caught mutation {mutation}"
