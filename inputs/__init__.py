"""Seeded synthetic inputs for the Llama-3 decoder forward pass.

This module is the input specification shared by the fp64 oracle (``oracle/``)
and the HIP path (``dense_decoder_only_rmsnorm_amd``).  It holds no arithmetic
of the method itself: it draws numbers, rounds them to the storage format and
lays them out.  Everything here is plain numpy on the CPU.

Generator
---------
Every tensor has a name that follows the checkpoint keys listed on the page
"llama3-from-scratch" (section 2, reading the model file): ``tok_embeddings.weight``,
``layers.{l}.attention.wq.weight`` ... ``norm.weight``, ``output.weight``, plus
``ids``, ``x`` and ``cache_k.{l}`` / ``cache_v.{l}`` for the other inputs.

A tensor is generated in chunks of ``CHUNK`` flat elements.  Chunk ``c`` of
tensor ``name`` under seed ``s`` is drawn from its own PCG64 stream, seeded by
``SeedSequence(s, spawn_key=(crc32(name), c))``.  Any chunk can therefore be
regenerated on its own, chunks can be drawn in parallel, and a slice of a
tensor (one sequence of a KV cache, one row of an embedding table) costs only
the chunks it touches.

Normal tensors are float32 standard normals times ``std`` (one float32
multiply), then rounded to bfloat16 with round-to-nearest-even when the
configuration is bf16.  Token ids are uniform integers in ``[0, vocab)``.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
import zlib
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

CHUNK = 1 << 22  # elements per independent stream
_THREADS = max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------------------
# bf16 storage format helpers (format handling, not method arithmetic)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  NaN is not expected in inputs.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Chunked, counter-addressed streams
# ----------------------------------------------------------------------------
def _stream(seed: int, name: str, chunk: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=int(seed), spawn_key=(zlib.crc32(name.encode()), int(chunk)))
    return np.random.Generator(np.random.PCG64(ss))


def _draw_chunk(kind: str, seed: int, name: str, chunk: int, n: int, param):
    g = _stream(seed, name, chunk)
    if kind == "normal":
        return g.standard_normal(n, dtype=np.float32)
    if kind == "ids":
        return g.integers(0, param, size=n, dtype=np.int32)
    if kind == "uniform":
        return g.random(n, dtype=np.float32)
    raise ValueError(kind)


def _draw(kind: str, seed: int, name: str, start: int, stop: int, param=None, dtype=np.float32,
          post=None) -> np.ndarray:
    """Elements [start, stop) of the flat stream for ``name``.

    ``post`` (optional) maps a chunk's raw draws to the stored values inside
    the worker thread (scaling, rounding); the result dtype is ``dtype``.
    """
    out = np.empty(stop - start, dtype=dtype)
    if stop <= start:
        return out
    first, last = start // CHUNK, (stop - 1) // CHUNK

    def job(c):
        lo, hi = c * CHUNK, (c + 1) * CHUNK
        a, b = max(lo, start), min(hi, stop)
        # a stream's first n draws do not depend on how many follow
        vals = _draw_chunk(kind, seed, name, c, b - lo, param)[a - lo:b - lo]
        out[a - start:b - start] = post(vals) if post is not None else vals

    chunks = range(first, last + 1)
    if len(chunks) == 1:
        job(first)
    else:
        with _cf.ThreadPoolExecutor(min(_THREADS, len(chunks))) as ex:
            list(ex.map(job, chunks))
    return out


def normal(seed: int, name: str, shape, std: float, bf16: bool, start: int = 0, stop: Optional[int] = None):
    """Normal(0, std^2) values for ``name``.

    Returns float32 values; when ``bf16`` they are exactly representable in
    bfloat16 (already rounded).  ``start``/``stop`` select a flat sub-range of
    the full tensor of ``shape`` (the result is then 1-D).
    """
    n = int(np.prod(shape))
    sub = stop is not None or start != 0
    stop = n if stop is None else stop
    sd = np.float32(std)
    if bf16:
        post = lambda v: bf16_bits_to_f32(f32_to_bf16_bits(v * sd))  # noqa: E731
    else:
        post = lambda v: v * sd  # noqa: E731
    v = _draw("normal", seed, name, start, stop, post=post)
    return v if sub else v.reshape(shape)


def normal_bits(seed: int, name: str, shape, std: float, start: int = 0, stop: Optional[int] = None) -> np.ndarray:
    """The bfloat16 bit patterns (uint16) of ``normal(seed, name, shape, std, bf16=True)``."""
    n = int(np.prod(shape))
    sub = stop is not None or start != 0
    stop = n if stop is None else stop
    sd = np.float32(std)
    v = _draw("normal", seed, name, start, stop, dtype=np.uint16, post=lambda v: f32_to_bf16_bits(v * sd))
    return v if sub else v.reshape(shape)


def token_ids(seed: int, name: str, shape, vocab: int) -> np.ndarray:
    n = int(np.prod(shape))
    return _draw("ids", seed, name, 0, n, param=vocab, dtype=np.int32).reshape(shape)


def uniform(seed: int, name: str, shape) -> np.ndarray:
    """float32 values uniform in [0, 1) (the draws a sampler consumes)."""
    n = int(np.prod(shape))
    return _draw("uniform", seed, name, 0, n).reshape(shape)


def document_ids(seed: int, name: str, batch: int, seq_len: int, max_doc: int) -> np.ndarray:
    """int32 [batch, seq_len] document ids for sequences packed from documents
    of seeded lengths uniform in [1, max_doc]: ids 0, 1, 2, ... per run."""
    out = np.empty((batch, seq_len), dtype=np.int32)
    for b in range(batch):
        lens = _draw("ids", seed, f"{name}/{b}", 0, seq_len, param=max_doc, dtype=np.int32) + 1
        ids = np.repeat(np.arange(seq_len, dtype=np.int32), lens)[:seq_len]
        out[b] = ids
    return out


# ----------------------------------------------------------------------------
# Configurations (shapes, dtypes, seeds; no derived quantities of the method)
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Config:
    key: str
    dim: int
    n_layers: int
    n_heads: int
    n_kv_heads: int
    vocab_size: int
    multiple_of: int
    ffn_dim_multiplier: Optional[float]
    norm_eps: float
    rope_theta: float
    dtype: str  # "f32" or "bf16"
    batch: int
    seq_len: int
    seed: int
    weight_std: float = 0.02
    norm_std: float = 0.0  # 0: norm weights are exactly 1.0; >0: N(1, norm_std^2)
    cache_len: int = 0  # decode: filled KV positions per sequence
    cache_cap: int = 0  # decode: KV capacity per sequence
    kind: str = "prefill"  # prefill | layer | decode

    @property
    def head_dim(self) -> int:
        return self.dim // self.n_heads

    @property
    def bf16(self) -> bool:
        return self.dtype == "bf16"

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


_8B = dict(dim=4096, n_heads=32, n_kv_heads=8, vocab_size=128256, multiple_of=1024,
           ffn_dim_multiplier=1.3, norm_eps=1e-5, rope_theta=500000.0, dtype="bf16")

CONFIGS = {
    # Tiny stack in fp32 (the page "Build your own Llama 3", section 1.2 ModelArgs).
    "c1": Config("c1", dim=512, n_layers=8, n_heads=8, n_kv_heads=4, vocab_size=68, multiple_of=256,
                 ffn_dim_multiplier=None, norm_eps=1e-5, rope_theta=500000.0, dtype="f32",
                 batch=1, seq_len=256, seed=1),
    # Small GQA stack (hidden 768, 8 heads, 2 KV heads, head_dim 96; the joto.ai page on GQA).
    "c2": Config("c2", dim=768, n_layers=4, n_heads=8, n_kv_heads=2, vocab_size=32000, multiple_of=256,
                 ffn_dim_multiplier=None, norm_eps=1e-5, rope_theta=500000.0, dtype="bf16",
                 batch=4, seq_len=1024, seed=2),
    # One 8B-shaped layer with hidden states x ~ N(0, 1) as input.
    "c3_s17": Config("c3_s17", n_layers=1, batch=1, seq_len=17, seed=3, kind="layer", **_8B),
    "c3_s2048": Config("c3_s2048", n_layers=1, batch=1, seq_len=2048, seed=3, kind="layer", **_8B),
    # Full 32-layer 8B-shaped prefill.
    "c4": Config("c4", n_layers=32, batch=1, seq_len=8192, seed=4, **_8B),
    # Batched decode step at 8B shapes over a seeded KV cache.
    "c5": Config("c5", n_layers=32, batch=64, seq_len=1, seed=5, cache_len=4096, cache_cap=4224,
                 kind="decode", **_8B),
}


# ----------------------------------------------------------------------------
# Model weights, lazily generated per tensor
# ----------------------------------------------------------------------------
LAYER_TENSORS = ("wq", "wk", "wv", "wo", "w1", "w2", "w3", "attention_norm", "ffn_norm")


def tensor_name(kind: str, layer: Optional[int] = None) -> str:
    if kind in ("wq", "wk", "wv", "wo"):
        return f"layers.{layer}.attention.{kind}.weight"
    if kind in ("w1", "w2", "w3"):
        return f"layers.{layer}.feed_forward.{kind}.weight"
    if kind in ("attention_norm", "ffn_norm"):
        return f"layers.{layer}.{kind}.weight"
    return {"tok_embeddings": "tok_embeddings.weight", "norm": "norm.weight",
            "output": "output.weight"}[kind]


class SyntheticModel:
    """Seeded random-init weights for one configuration.

    ``ffn_hidden`` is passed in by the caller (each side derives it itself).
    All arrays are float32 (bf16-exact for bf16 configurations).
    """

    def __init__(self, cfg: Config, ffn_hidden: int):
        self.cfg = cfg
        self.F = int(ffn_hidden)

    def shape(self, kind: str):
        c, F = self.cfg, self.F
        hd = c.head_dim
        return {
            "wq": (c.n_heads * hd, c.dim), "wk": (c.n_kv_heads * hd, c.dim),
            "wv": (c.n_kv_heads * hd, c.dim), "wo": (c.dim, c.n_heads * hd),
            "w1": (F, c.dim), "w3": (F, c.dim), "w2": (c.dim, F),
            "attention_norm": (c.dim,), "ffn_norm": (c.dim,), "norm": (c.dim,),
            "tok_embeddings": (c.vocab_size, c.dim), "output": (c.vocab_size, c.dim),
        }[kind]

    def get(self, kind: str, layer: Optional[int] = None) -> np.ndarray:
        c = self.cfg
        name = tensor_name(kind, layer)
        shp = self.shape(kind)
        if kind in ("attention_norm", "ffn_norm", "norm"):
            if c.norm_std == 0.0:
                return np.ones(shp, dtype=np.float32)
            v = normal(c.seed, name, shp, c.norm_std, c.bf16) + np.float32(1.0)
            return _round_like(v, c.bf16)
        return normal(c.seed, name, shp, c.weight_std, c.bf16)

    def bits(self, kind: str, layer: Optional[int] = None) -> np.ndarray:
        """bf16 bit patterns (uint16) of ``get(kind, layer)`` for a bf16 configuration."""
        c = self.cfg
        if kind in ("attention_norm", "ffn_norm", "norm"):
            return f32_to_bf16_bits(self.get(kind, layer))
        return normal_bits(c.seed, tensor_name(kind, layer), self.shape(kind), c.weight_std)

    def rows(self, kind: str, rows: np.ndarray) -> np.ndarray:
        """Selected rows of a [rows, cols] weight (embedding lookups without the full table).

        Each stream chunk the rows touch is drawn once (in parallel), however
        many of the requested rows fall into it."""
        c = self.cfg
        name = tensor_name(kind)
        nrow, ncol = self.shape(kind)
        n = nrow * ncol
        rows = np.asarray(rows, dtype=np.int64).reshape(-1)
        need = set()
        for r in np.unique(rows):
            need.update(range(int(r) * ncol // CHUNK, ((int(r) + 1) * ncol - 1) // CHUNK + 1))

        def job(ch):
            lo, hi = ch * CHUNK, min(n, (ch + 1) * CHUNK)
            return ch, normal(c.seed, name, (nrow, ncol), c.weight_std, c.bf16, start=lo, stop=hi)

        with _cf.ThreadPoolExecutor(max(1, min(_THREADS, len(need)))) as ex:
            chunks = dict(ex.map(job, sorted(need)))
        out = np.empty((len(rows), ncol), dtype=np.float32)
        for i, r in enumerate(rows):
            a, b = int(r) * ncol, (int(r) + 1) * ncol
            for ch in range(a // CHUNK, (b - 1) // CHUNK + 1):
                lo = max(a, ch * CHUNK)
                hi = min(b, (ch + 1) * CHUNK)
                out[i, lo - a:hi - a] = chunks[ch][lo - ch * CHUNK:hi - ch * CHUNK]
        return out

    def layer(self, l: int) -> dict:
        return {k: self.get(k, l) for k in LAYER_TENSORS}


def _round_like(v: np.ndarray, bf16: bool) -> np.ndarray:
    return bf16_bits_to_f32(f32_to_bf16_bits(v)) if bf16 else v.astype(np.float32)


def prompt_ids(cfg: Config) -> np.ndarray:
    """Token ids [batch, seq_len], uniform in [0, vocab)."""
    return token_ids(cfg.seed, "ids", (cfg.batch, cfg.seq_len), cfg.vocab_size)


def hidden_x(cfg: Config) -> np.ndarray:
    """Layer input x ~ N(0, 1) of shape [batch, seq_len, dim] (rounded to bf16 for bf16 configs)."""
    return normal(cfg.seed, f"x.{cfg.seq_len}", (cfg.batch, cfg.seq_len, cfg.dim), 1.0, cfg.bf16)


def kv_cache_bits(cfg: Config, layer: int, which: str) -> np.ndarray:
    """bf16 bit patterns of the whole seeded cache block of one layer, [batch, cache_len, G, hd]."""
    shape = (cfg.batch, cfg.cache_len, cfg.n_kv_heads, cfg.head_dim)
    return normal_bits(cfg.seed, f"cache_{which}.{layer}", shape, 1.0)


def kv_cache_block(cfg: Config, layer: int, which: str, b0: int = 0, b1: Optional[int] = None) -> np.ndarray:
    """Seeded KV-cache contents ~ N(0, 1) for sequences [b0, b1) of one layer.

    Shape [b1-b0, cache_len, n_kv_heads, head_dim]; positions 0..cache_len-1 are
    filled (the values stand for keys already rotated).
    """
    b1 = cfg.batch if b1 is None else b1
    per_seq = cfg.cache_len * cfg.n_kv_heads * cfg.head_dim
    shape = (cfg.batch, cfg.cache_len, cfg.n_kv_heads, cfg.head_dim)
    v = normal(cfg.seed, f"cache_{which}.{layer}", shape, 1.0, cfg.bf16, start=b0 * per_seq, stop=b1 * per_seq)
    return v.reshape(b1 - b0, cfg.cache_len, cfg.n_kv_heads, cfg.head_dim)


__all__ = [
    "CHUNK", "Config", "CONFIGS", "SyntheticModel", "LAYER_TENSORS", "tensor_name",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "normal", "normal_bits", "token_ids", "prompt_ids", "hidden_x",
    "kv_cache_block", "kv_cache_bits",
]
