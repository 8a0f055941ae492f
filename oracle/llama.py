"""fp64 numpy oracle of the Llama-3 decoder forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or run this module.  It
shares no code with the HIP path and never imports it.

Every function evaluates the definition on the pages directly, in float64,
with no blocking, fusion or reordering beyond what the definition states.
Inputs arrive as float32 arrays holding exactly the values the GPU receives
(bf16-representable for bf16 configurations) and are widened to float64
without rounding.  Library primitives used as steps: ``numpy.matmul``,
``numpy.exp``, ``numpy.sqrt``, complex multiplication.

Pages cited (by title and section):
  [P1] "机器学习 | 从0开发大模型—译llama3-from-scratch" (sunaigc.com)
  [P2] "Build your own Llama 3 architecture from scratch" notes (gitcode.csdn.net)
  [P3] "大语言模型实现llama3-from-scratch：输出层与预测" (agent.csdn.net)
  [P4] joto.ai blog post on the Llama architecture (GQA, RoPE, RMSNorm)

Readings where the pages are silent or disagree:
  * RoPE pairs are adjacent elements (2i, 2i+1) of a head (P1 6.6; P2 3.2),
    not the rotate-half convention.
  * theta_i = rope_theta ** (-2i / head_dim), i < head_dim/2 (P2 3.2, whose
    formula image is lost; its code and P1 6.7 agree).  Angles are exact
    float64 products p * theta_i.
  * Positions are 0-based; a decode token sits at p = current cache length
    (P2 3.4, freqs_cis sliced at start_pos).
  * Key j is visible to a query at position p iff j <= p, in prefill and in
    decode; masked scores get exactly zero probability (P1 7.1; P2 3.4).
  * Query head h reads KV head g = h // n_rep (P1 8; P2 3.4 repeat_kv).
  * RMSNorm is evaluated without intermediate rounding (P2 3.1 rounds to the
    activation type before the weight multiply; the oracle does not round).
  * Only the last position of each sequence feeds the LM head; logits are
    returned as float64 and compared as fp32 (P1 12; P3 steps 2-3).
  * argmax ties go to the smallest index.
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence

import numpy as np

F64 = np.float64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


# ---------------------------------------------------------------------------
# Configuration arithmetic
# ---------------------------------------------------------------------------
def ffn_hidden_dim(dim: int, multiple_of: int, ffn_dim_multiplier: Optional[float]) -> int:
    """SwiGLU hidden size.

    [P2 3.5 FeedForward, 3.6 TransformerBlock]: start from 4*dim, keep two
    thirds (truncating), scale by ffn_dim_multiplier when it is set
    (truncating), then round up to a multiple of multiple_of.
    """
    hidden = int(2 * (4 * dim) / 3)
    if ffn_dim_multiplier is not None:
        hidden = int(ffn_dim_multiplier * hidden)
    return multiple_of * ((hidden + multiple_of - 1) // multiple_of)


# ---------------------------------------------------------------------------
# a2, a12: RMSNorm
# ---------------------------------------------------------------------------
def rms_norm(x, w, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2 over the last axis) + eps) * w.

    [P1 5 rms_norm; P2 3.1 RMSNorm; P3 "嵌入归一化的必要性"]: eps sits inside the
    square root, the mean runs over the model dimension and the weight
    multiplies after normalizing.
    """
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(w)


# ---------------------------------------------------------------------------
# a4: rotary position embedding
# ---------------------------------------------------------------------------
def rope_frequencies(head_dim: int, theta: float) -> np.ndarray:
    """theta_i = theta ** (-2 i / head_dim) for i = 0 .. head_dim/2 - 1.

    [P2 3.2 precompute_freqs_cis; P1 6.7, where range(64)/64 equals 2i/128].
    """
    i = np.arange(head_dim // 2, dtype=F64)
    return 1.0 / (F64(theta) ** (2.0 * i / head_dim))


def rope_rotations(positions, head_dim: int, theta: float) -> np.ndarray:
    """Unit complex numbers e^{i p theta_i}, shape [len(positions), head_dim/2].

    [P1 6.7 torch.polar(ones, outer(positions, freqs)); P2 3.2].
    """
    ang = np.outer(_f64(positions), rope_frequencies(head_dim, theta))
    return np.exp(1j * ang)


def apply_rope(x, positions, theta: float) -> np.ndarray:
    """Rotate query or key vectors by their positions.

    x has shape [S, n_heads, head_dim]; positions has length S.  Adjacent
    pairs (2i, 2i+1) are read as the complex number x[2i] + i x[2i+1] and
    multiplied by e^{i p theta_i}; the product is written back as a pair
    [P1 6.8-6.9 view_as_complex / view_as_real; P2 3.2 apply_rotary_emb].
    """
    x = _f64(x)
    hd = x.shape[-1]
    rot = rope_rotations(positions, hd, theta)  # [S, hd/2]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    z = z * rot[:, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


# ---------------------------------------------------------------------------
# a6, a7: causal grouped-query attention
# ---------------------------------------------------------------------------
def causal_mask(q_positions, k_positions) -> np.ndarray:
    """0 where key position <= query position, -inf elsewhere.

    [P1 7.1: full(-inf) then triu(diagonal=1); P2 3.4 training branch].  For
    queries and keys both at 0..S-1 this is exactly that upper-triangular mask.
    """
    qp = np.asarray(q_positions)[:, None]
    kp = np.asarray(k_positions)[None, :]
    return np.where(kp > qp, -np.inf, 0.0)


def document_mask(q_positions, k_positions, doc_ids) -> np.ndarray:
    """The document-level causal mask [P2 appendix item 1; P2 1, the
    cross-document mask]: 0 where the key is at or before the query AND in
    the same document, -inf elsewhere.  Documents are concatenated into one
    sequence, so a document is a maximal run of equal ids; ``doc_ids`` gives
    the id at every absolute position up to the last query.
    """
    doc = np.asarray(doc_ids).reshape(-1)
    run = np.zeros(len(doc), dtype=np.int64)  # index of the run each position lies in
    for p in range(1, len(doc)):
        run[p] = run[p - 1] + (1 if doc[p] != doc[p - 1] else 0)
    qp = np.asarray(q_positions)
    kp = np.asarray(k_positions)
    visible = (kp[None, :] <= qp[:, None]) & (run[kp][None, :] == run[qp][:, None])
    return np.where(visible, 0.0, -np.inf)


def softmax(s, axis=-1) -> np.ndarray:
    """exp(s - max) / sum(exp(s - max)); entries at -inf get weight 0."""
    s = _f64(s)
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attention(q, k, v, q_positions, k_positions, return_probs: bool = False, doc_ids=None):
    """Causal GQA attention for one sequence (with ``doc_ids``: under the
    document-level mask, ``document_mask``).

    q: [S, H, hd]; k, v: [L, G, hd] (keys already rotated).  For head h the
    KV head is g = h // (H // G) [P1 8, `head//4`; P2 3.4 repeat_kv].
      scores = q_h k_g^T / sqrt(hd) + mask    [P1 6.11, 7.1; P2 3.4]
      P      = softmax over keys              [P1 7.1; P2 3.4]
      O_h    = P v_g                          [P1 7.4]
    Returns O with heads concatenated in order: [S, H*hd] [P1 8 torch.cat].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    S, H, hd = q.shape
    G = k.shape[1]
    n_rep = H // G
    if doc_ids is None:
        mask = causal_mask(q_positions, k_positions)
    else:
        mask = document_mask(q_positions, k_positions, doc_ids)
    out = np.empty((S, H, hd), dtype=F64)
    probs = []
    for h in range(H):
        g = h // n_rep
        s = q[:, h, :] @ k[:, g, :].T / math.sqrt(hd) + mask
        p = softmax(s, axis=-1)
        out[:, h, :] = p @ v[:, g, :]
        probs.append(p)
    o = out.reshape(S, H * hd)
    return (o, np.stack(probs)) if return_probs else o


# ---------------------------------------------------------------------------
# a9, a10: SwiGLU feed-forward
# ---------------------------------------------------------------------------
def silu(x) -> np.ndarray:
    """x * sigmoid(x) [P2 3.5]."""
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def feed_forward(xn, w1, w2, w3) -> np.ndarray:
    """w2( silu(w1 x) * w3 x ) with nn.Linear weights [out, in] [P1 9.3; P2 3.5]."""
    xn = _f64(xn)
    gate = xn @ _f64(w1).T
    up = xn @ _f64(w3).T
    return (silu(gate) * up) @ _f64(w2).T


# ---------------------------------------------------------------------------
# a2-a11: one decoder layer
# ---------------------------------------------------------------------------
def layer_forward(h, lw: dict, args: dict, positions, cache: Optional[dict] = None, taps: Optional[dict] = None,
                  doc_ids=None):
    """One pre-norm decoder block on one sequence [P2 3.6; P1 6-10].

    h: [S, D] hidden states entering the layer; positions: the S absolute
    positions.  ``cache`` (optional) holds keys/values of earlier positions,
    {"k": [P, G, hd], "v": [P, G, hd]} for positions 0..P-1 with
    P = positions[0]; the new keys/values are appended to it (in place in the
    dict) before attention [P2 3.3-3.4 inference branch].
      h1 = h  + wo( attention( rope(xn wq^T), rope(xn wk^T), xn wv^T ) ),  xn = rmsnorm(h)
      h2 = h1 + w2( silu(xn2 w1^T) * xn2 w3^T ),                          xn2 = rmsnorm(h1)
    """
    h = _f64(h)
    S, D = h.shape
    H, G = args["n_heads"], args["n_kv_heads"]
    hd = D // H
    eps, theta = args["norm_eps"], args["rope_theta"]
    positions = np.asarray(positions)

    xn = rms_norm(h, lw["attention_norm"], eps)
    q = (xn @ _f64(lw["wq"]).T).reshape(S, H, hd)
    k = (xn @ _f64(lw["wk"]).T).reshape(S, G, hd)
    v = (xn @ _f64(lw["wv"]).T).reshape(S, G, hd)
    q = apply_rope(q, positions, theta)
    k = apply_rope(k, positions, theta)
    if cache is not None:
        k_all = np.concatenate([_f64(cache["k"]), k], axis=0)
        v_all = np.concatenate([_f64(cache["v"]), v], axis=0)
        cache["k"], cache["v"] = k_all, v_all
        k_pos = np.arange(k_all.shape[0])
    else:
        k_all, v_all, k_pos = k, v, positions
    if doc_ids is None:
        o = attention(q, k_all, v_all, positions, k_pos)
    else:
        o = attention(q, k_all, v_all, positions, k_pos, doc_ids=doc_ids)
    attn_out = o @ _f64(lw["wo"]).T
    h1 = h + attn_out
    xn2 = rms_norm(h1, lw["ffn_norm"], eps)
    ffn_out = feed_forward(xn2, lw["w1"], lw["w2"], lw["w3"])
    h2 = h1 + ffn_out
    if taps is not None:
        taps.update(xn=xn, q=q, k=k, v=v, attn=o, attn_out=attn_out, h1=h1, ffn_out=ffn_out)
    return h2


# ---------------------------------------------------------------------------
# a12-a14: output head
# ---------------------------------------------------------------------------
def lm_head(hf, w_out) -> np.ndarray:
    """logits = hf @ W_out^T [P1 12; P3 3]."""
    return _f64(hf) @ _f64(w_out).T


def argmax_first(logits) -> np.ndarray:
    """Index of the largest logit per row, smallest index on ties [P1 12; P3 4]."""
    logits = _f64(logits)
    return np.argmax(logits, axis=-1).astype(np.int64)  # numpy returns the first maximum


def top2_gap(logits) -> np.ndarray:
    """Largest minus second-largest logit per row."""
    s = np.sort(_f64(logits), axis=-1)
    return s[..., -1] - s[..., -2]


# ---------------------------------------------------------------------------
# a1-a14: whole stack
# ---------------------------------------------------------------------------
LayerSource = Callable[[int], dict]


def prefill(ids, embed_rows: Callable, layer: LayerSource, norm_w, w_out, args: dict,
            caches: Optional[list] = None, all_hidden: bool = False, doc_ids=None):
    """Prefill of a batch of sequences from position 0 [P2 4 Transformer.forward; P1 4-12].

    ids: [B, S] int.  ``embed_rows(ids_1d)`` returns embedding rows;
    ``layer(l)`` returns layer l's weights (streamed, one layer at a time).
    When ``caches`` is a list of B lists (one per sequence), each layer's
    keys/values are appended to caches[b][l] (dicts with "k"/"v").
    ``doc_ids`` [B, S] (optional) applies the document-level mask.
    Returns dict(hidden=[B,S,D] or last rows, hf=[B,D], logits=[B,V], ids=[B]).
    """
    ids = np.asarray(ids)
    B, S = ids.shape
    hs = [_f64(embed_rows(ids[b])) for b in range(B)]
    positions = np.arange(S)
    for l in range(args["n_layers"]):
        lw = {k: _f64(v) for k, v in layer(l).items()}  # widen once per layer
        for b in range(B):
            cache = None
            if caches is not None:
                cache = {"k": np.zeros((0, args["n_kv_heads"], args["dim"] // args["n_heads"])),
                         "v": np.zeros((0, args["n_kv_heads"], args["dim"] // args["n_heads"]))}
            if doc_ids is None:
                hs[b] = layer_forward(hs[b], lw, args, positions, cache=cache)
            else:
                hs[b] = layer_forward(hs[b], lw, args, positions, cache=cache, doc_ids=np.asarray(doc_ids)[b])
            if caches is not None:
                caches[b].append(cache)
    last = np.stack([hs[b][-1] for b in range(B)])
    hf = rms_norm(last, norm_w, args["norm_eps"])
    logits = lm_head(hf, w_out)
    out = dict(last_hidden=last, hf=hf, logits=logits, ids=argmax_first(logits))
    if all_hidden:
        out["hidden"] = np.stack(hs)
    return out


def decode_step(ids, caches: Sequence[Sequence[dict]], embed_rows: Callable, layer: LayerSource,
                norm_w, w_out, args: dict, new_kv: Optional[list] = None, doc_ids=None):
    """One new token per sequence at position p_b = len(cache) [P2 3.3, 6 generate].

    ids: [B] token ids; caches[b][l] = {"k": [p_b, G, hd], "v": ...} (not modified).
    When ``new_kv`` is a list, it receives per (b, l) the new key/value rows.
    ``doc_ids`` (optional, per sequence the ids of positions 0..p_b, the new
    token's included) applies the document-level mask.
    """
    ids = np.asarray(ids).reshape(-1)
    B = ids.shape[0]
    hs = [_f64(embed_rows(ids[b:b + 1])) for b in range(B)]
    for l in range(args["n_layers"]):
        lw = {k: _f64(v) for k, v in layer(l).items()}  # widen once per layer
        for b in range(B):
            c = caches[b][l]
            p = c["k"].shape[0]
            cache = {"k": c["k"], "v": c["v"]}
            if doc_ids is None:
                hs[b] = layer_forward(hs[b], lw, args, np.array([p]), cache=cache)
            else:
                hs[b] = layer_forward(hs[b], lw, args, np.array([p]), cache=cache, doc_ids=doc_ids[b])
            if new_kv is not None:
                new_kv.append((b, l, cache["k"][-1], cache["v"][-1]))
    last = np.stack([hs[b][-1] for b in range(B)])
    hf = rms_norm(last, norm_w, args["norm_eps"])
    logits = lm_head(hf, w_out)
    return dict(last_hidden=last, hf=hf, logits=logits, ids=argmax_first(logits))


# ---------------------------------------------------------------------------
# Generation [P2 6 "Inference": generate, sample_top_p; P3 temperature softmax]
# ---------------------------------------------------------------------------
def sample_top_p(logits, temperature: float, top_p: float, u: float):
    """One draw from the top-p nucleus of softmax(logits / temperature).

    Steps in the pages' order [P2 6 sample_top_p]: sort the probabilities in
    descending order (ties: smaller token id first), take the running sum,
    drop every token whose mass before it exceeds top_p, renormalise, draw.
    Reading of the draw (torch.multinomial's use of its random numbers is
    not stated): inverse CDF with the given uniform u in [0, 1) over the kept
    tokens in ascending id order, i.e. the smallest id whose cumulative kept
    probability exceeds u.

    Returns (token, margin): margin is the distance, in probability, of the
    two decisions from their boundaries (the mass before the tokens next to
    the cut against top_p, and u against the chosen token's cumulative
    interval); a computation whose probabilities err by less than the margin
    makes the same choice.
    """
    l = _f64(logits).reshape(-1)
    p = softmax(l / float(temperature))
    order = np.argsort(-p, kind="stable")
    ps = p[order]
    before = np.cumsum(ps) - ps                # mass ahead of each sorted token
    removed = before > top_p
    ks = np.where(removed, 0.0, ps)
    kept = np.zeros_like(p)
    kept[order] = ks
    q = kept / kept.sum()
    c = np.cumsum(q)
    tok = int(np.searchsorted(c, u, side="right"))
    tok = min(tok, int(np.nonzero(q)[0][-1]))
    # margins
    # (the first sorted token always has zero mass before it, and the first
    # and last kept tokens have exact outer boundaries 0 and 1: no margin)
    if removed.any():
        k0 = int(np.argmax(removed))           # first removed in sorted order
        m_cut = before[k0] - top_p
        if k0 > 1:
            m_cut = min(m_cut, top_p - before[k0 - 1])
    else:
        m_cut = top_p - before[-1] if (top_p < 1.0 and len(p) > 1) else math.inf
    nz = np.nonzero(q)[0]
    m_draw = math.inf
    if tok != nz[0]:
        m_draw = min(m_draw, u - c[tok - 1])
    if tok != nz[-1]:
        m_draw = min(m_draw, c[tok] - u)
    return tok, float(min(m_cut, m_draw))


def generate(prompts, embed_rows: Callable, layer: LayerSource, norm_w, w_out, args: dict, max_gen_len: int,
             eos_id: int, max_seq_len: int, temperature: float = 0.0, top_p: float = 0.9, uniforms=None,
             forced=None):
    """Autoregressive generation of each prompt [P2 6 generate].

    For prompt b of length L the sequence runs to total = min(L + max_gen_len,
    max_seq_len) positions; position p >= L receives the model's choice from
    the logits at position p - 1 (argmax when temperature == 0, else
    ``sample_top_p`` with uniforms[p - L][b]); the sequence stops right after
    a generated eos_id (the pages' loop ends on the end-of-text token).  The
    output is cut before the first eos_id anywhere in the sequence, as the
    pages cut the decoded text.

    The prompt is fed in one forward call and each later token alone; the
    pages feed the prompt one token at a time, which yields the same cache
    and the same logits at the prompt's last position.

    ``forced`` (optional, per sequence a token list): the token appended at
    each generated position is forced[b][p] instead of the oracle's own
    choice, so that the oracle's choices can be checked along another
    implementation's path.  Returns, per sequence, dict(tokens, out_len,
    choices, margins, logits): the appended tokens, the cut length, and for
    each generated position the oracle's choice, its decision margin (top-2
    logit gap for argmax, ``sample_top_p``'s margin for sampling) and the
    logits it was taken from.
    """
    out = []
    for b, prompt in enumerate(prompts):
        prompt = [int(t) for t in prompt]
        L = len(prompt)
        total = min(L + max_gen_len, max_seq_len)
        toks = list(prompt)
        choices, margins, step_logits = [], [], []
        if total > L:
            caches = [[]]
            r = prefill(np.array([prompt]), embed_rows, layer, norm_w, w_out, args, caches=caches)
            logits = r["logits"][0]
            p = L
            while True:
                if temperature == 0.0:
                    choice = int(argmax_first(logits[None])[0])
                    margin = float(top2_gap(logits[None])[0])
                else:
                    choice, margin = sample_top_p(logits, temperature, top_p, float(uniforms[p - L][b]))
                tok = int(forced[b][p]) if forced is not None else choice
                step_logits.append(logits)
                toks.append(tok)
                choices.append(choice)
                margins.append(margin)
                if (eos_id >= 0 and tok == eos_id) or p + 1 >= total:
                    break
                new = []
                r = decode_step([tok], caches, embed_rows, layer, norm_w, w_out, args, new_kv=new)
                for (_, l, k, v) in new:
                    c = caches[0][l]
                    c["k"] = np.concatenate([c["k"], k[None]], axis=0)
                    c["v"] = np.concatenate([c["v"], v[None]], axis=0)
                logits = r["logits"][0]
                p += 1
        cut = toks.index(eos_id) if (eos_id >= 0 and eos_id in toks) else len(toks)
        out.append(dict(tokens=toks, out_len=cut, choices=choices, margins=margins, logits=step_logits))
    return out
