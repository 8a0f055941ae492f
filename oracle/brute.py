"""Brute-force scalar oracle for tiny shapes (pure Python loops, float64).

TEST INFRASTRUCTURE ONLY (see ``oracle/llama.py``).

A second, independent formulation of the same definition, used to check the
numpy oracle on tiny inputs.  Where the numpy oracle uses one formulation,
this one deliberately uses another that the pages also give:
  * RoPE as an explicit 2x2 rotation matrix per pair with cos/sin
    [P4, "RoPE as dim/2 two-dimensional rotations"], not a complex product;
  * GQA by materialising repeated K/V heads first and then running plain
    multi-head attention [P2 3.4 repeat_kv: expand a new axis after the KV
    axis, then flatten], not by indexing g = h // n_rep;
  * causality by summing only over keys j <= i [P1 7.1 "future tokens get
    no weight"], not by adding -inf;
  * every matrix product as explicit sums.
"""
from __future__ import annotations

import math
from typing import List

Vec = List[float]
Mat = List[List[float]]


def matvec(w: Mat, x: Vec) -> Vec:
    """y[o] = sum_i w[o][i] x[i] for an nn.Linear weight w of shape [out, in]."""
    return [math.fsum(w[o][i] * x[i] for i in range(len(x))) for o in range(len(w))]


def rms_norm(x: Vec, w: Vec, eps: float) -> Vec:
    ms = math.fsum(t * t for t in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [x[i] * r * w[i] for i in range(len(x))]


def rope_vec(x: Vec, pos: int, theta: float) -> Vec:
    """Rotate each pair (x[2i], x[2i+1]) by the angle pos * theta^(-2i/d)."""
    d = len(x)
    out = [0.0] * d
    for i in range(d // 2):
        ang = pos * theta ** (-(2.0 * i) / d)
        c, s = math.cos(ang), math.sin(ang)
        a, b = x[2 * i], x[2 * i + 1]
        out[2 * i] = c * a - s * b
        out[2 * i + 1] = s * a + c * b
    return out


def repeat_kv(heads: List[List[Vec]], n_rep: int) -> List[List[Vec]]:
    """[G][L][hd] -> [G*n_rep][L][hd]: each KV head repeated n_rep times in place."""
    out = []
    for g in range(len(heads)):
        for _ in range(n_rep):
            out.append(heads[g])
    return out


def silu(x: float) -> float:
    return x / (1.0 + math.exp(-x))


def layer_forward(h: List[Vec], lw: dict, args: dict, pos0: int = 0, past_k=None, past_v=None):
    """One decoder block for one sequence, positions pos0 .. pos0+S-1.

    past_k / past_v: per position, per KV head, hd-vectors of earlier positions
    (already rotated).  Returns (h_out, keys, values) where keys/values include
    the past and the new positions.
    """
    D = len(h[0])
    H, G = args["n_heads"], args["n_kv_heads"]
    hd = D // H
    eps, theta = args["norm_eps"], args["rope_theta"]
    S = len(h)
    keys = [list(p) for p in (past_k or [])]
    vals = [list(p) for p in (past_v or [])]
    qs = []
    for s in range(S):
        xn = rms_norm(h[s], lw["attention_norm"], eps)
        q = matvec(lw["wq"], xn)
        k = matvec(lw["wk"], xn)
        v = matvec(lw["wv"], xn)
        p = pos0 + s
        qs.append([rope_vec(q[j * hd:(j + 1) * hd], p, theta) for j in range(H)])
        keys.append([rope_vec(k[g * hd:(g + 1) * hd], p, theta) for g in range(G)])
        vals.append([v[g * hd:(g + 1) * hd] for g in range(G)])
    # KV heads as [G][L][hd], repeated to H heads.
    k_heads = repeat_kv([[keys[t][g] for t in range(len(keys))] for g in range(G)], H // G)
    v_heads = repeat_kv([[vals[t][g] for t in range(len(vals))] for g in range(G)], H // G)
    out = []
    for s in range(S):
        i = pos0 + s  # absolute position of this query
        o_cat: Vec = []
        for hh in range(H):
            visible = range(i + 1)  # keys 0..i only
            sc = [math.fsum(qs[s][hh][d] * k_heads[hh][j][d] for d in range(hd)) / math.sqrt(hd) for j in visible]
            m = max(sc)
            e = [math.exp(t - m) for t in sc]
            z = math.fsum(e)
            o = [math.fsum(e[j] / z * v_heads[hh][j][d] for j in visible) for d in range(hd)]
            o_cat.extend(o)
        a = matvec(lw["wo"], o_cat)
        h1 = [h[s][d] + a[d] for d in range(D)]
        xn2 = rms_norm(h1, lw["ffn_norm"], eps)
        g1 = matvec(lw["w1"], xn2)
        u3 = matvec(lw["w3"], xn2)
        f = matvec(lw["w2"], [silu(g1[t]) * u3[t] for t in range(len(g1))])
        out.append([h1[d] + f[d] for d in range(D)])
    return out, keys, vals


def forward(ids: List[int], emb: Mat, layers: List[dict], norm_w: Vec, w_out: Mat, args: dict):
    """Whole stack for one sequence; returns (last hidden, logits, argmax)."""
    h = [list(emb[t]) for t in ids]
    for lw in layers:
        h, _, _ = layer_forward(h, lw, args)
    hf = rms_norm(h[-1], norm_w, args["norm_eps"])
    logits = matvec(w_out, hf)
    best = 0
    for i in range(1, len(logits)):
        if logits[i] > logits[best]:
            best = i
    return h, logits, best
