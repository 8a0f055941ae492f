"""Binds the fp64 oracle to the seeded inputs of ``inputs``.

TEST INFRASTRUCTURE ONLY (see ``oracle/llama.py``).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

import inputs as I
from . import llama as L


def args_of(cfg: I.Config) -> dict:
    return dict(dim=cfg.dim, n_layers=cfg.n_layers, n_heads=cfg.n_heads, n_kv_heads=cfg.n_kv_heads,
                vocab_size=cfg.vocab_size, norm_eps=cfg.norm_eps, rope_theta=cfg.rope_theta)


def model_of(cfg: I.Config) -> I.SyntheticModel:
    return I.SyntheticModel(cfg, L.ffn_hidden_dim(cfg.dim, cfg.multiple_of, cfg.ffn_dim_multiplier))


def prefill(cfg: I.Config, ids: Optional[np.ndarray] = None, n_layers: Optional[int] = None,
            all_hidden: bool = False, caches: Optional[list] = None, doc_ids: Optional[np.ndarray] = None) -> dict:
    """Oracle prefill of ``cfg`` (ids default to the seeded prompt)."""
    m = model_of(cfg)
    ids = I.prompt_ids(cfg) if ids is None else np.asarray(ids)
    a = args_of(cfg)
    if n_layers is not None:
        a["n_layers"] = n_layers
    return L.prefill(ids, lambda r: m.rows("tok_embeddings", r), m.layer, m.get("norm"), m.get("output"), a,
                     caches=caches, all_hidden=all_hidden, doc_ids=doc_ids)


def layer(cfg: I.Config, x: Optional[np.ndarray] = None, layer_index: int = 0, rows: Optional[Sequence[int]] = None,
          taps: bool = False, doc_ids: Optional[np.ndarray] = None) -> dict:
    """Oracle output of one layer on hidden states x [B, S, D] at positions 0..S-1.

    ``rows`` restricts the output to the given positions (each still attends
    to all earlier positions; later positions are not computed beyond their
    keys and values).  ``doc_ids`` [B, S] applies the document-level mask.
    """
    m = model_of(cfg)
    x = I.hidden_x(cfg) if x is None else np.asarray(x)
    lw = m.layer(layer_index)
    a = args_of(cfg)
    B, S, _ = x.shape
    outs, tap_list = [], []
    for b in range(B):
        docs = None if doc_ids is None else np.asarray(doc_ids)[b]
        if rows is None:
            t = {} if taps else None
            if docs is None:
                outs.append(L.layer_forward(x[b], lw, a, np.arange(S), taps=t))
            else:
                outs.append(L.layer_forward(x[b], lw, a, np.arange(S), taps=t, doc_ids=docs))
            tap_list.append(t)
        else:
            outs.append(_layer_rows(x[b], lw, a, rows, docs))
    res = dict(y=np.stack(outs))
    if taps:
        res["taps"] = tap_list
    return res


def _layer_rows(x: np.ndarray, lw: dict, a: dict, rows: Sequence[int], doc_ids=None) -> np.ndarray:
    """Layer outputs at the given rows only: keys/values of all earlier rows are
    computed by the oracle's own projections, then each requested row is run as
    a one-token step over that prefix (the KV-cache identity of P2 3.3)."""
    rows = list(rows)
    hi = max(rows) + 1
    H, G, D = a["n_heads"], a["n_kv_heads"], a["dim"]
    hd = D // H
    xn = L.rms_norm(x[:hi], lw["attention_norm"], a["norm_eps"])
    k = L.apply_rope((xn @ L._f64(lw["wk"]).T).reshape(hi, G, hd), np.arange(hi), a["rope_theta"])
    v = (xn @ L._f64(lw["wv"]).T).reshape(hi, G, hd)
    out = []
    for r in rows:
        cache = {"k": k[:r], "v": v[:r]}
        if doc_ids is None:
            out.append(L.layer_forward(x[r:r + 1], lw, a, np.array([r]), cache=cache)[0])
        else:
            out.append(L.layer_forward(x[r:r + 1], lw, a, np.array([r]), cache=cache, doc_ids=doc_ids[:r + 1])[0])
    return np.stack(out)


def decode(cfg: I.Config, seqs: Sequence[int], n_layers: Optional[int] = None, ids: Optional[np.ndarray] = None,
           new_kv: Optional[list] = None) -> dict:
    """Oracle decode step for the sequences ``seqs`` of a decode configuration."""
    m = model_of(cfg)
    a = args_of(cfg)
    if n_layers is not None:
        a["n_layers"] = n_layers
    all_ids = I.prompt_ids(cfg).reshape(-1) if ids is None else np.asarray(ids).reshape(-1)
    caches = []
    for b in seqs:
        per_layer = []
        for l in range(a["n_layers"]):
            per_layer.append({"k": I.kv_cache_block(cfg, l, "k", b, b + 1)[0],
                              "v": I.kv_cache_block(cfg, l, "v", b, b + 1)[0]})
        caches.append(per_layer)
    sel = np.array([all_ids[b] for b in seqs])
    return L.decode_step(sel, caches, lambda r: m.rows("tok_embeddings", r), m.layer, m.get("norm"),
                         m.get("output"), a, new_kv=new_kv)
