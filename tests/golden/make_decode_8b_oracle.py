#!/usr/bin/env python3
"""Writes the fp64 oracle's own result for the 64-sequence decode step at 8B
shapes (32 layers, seeded KV caches of 4096 positions, one new token per
sequence at position 4096) to ``decode_8b_b64_oracle.npz`` beside this file.

TEST INFRASTRUCTURE.  This script imports only ``oracle`` and ``inputs``:
every stored value comes from the oracle alone.  Each sequence goes through
``oracle.runner.decode`` (its own seeded caches; the token at position p =
cache length attends to keys 0..p [P2 "Build your own Llama 3" 3.3-3.4 and
6 generate]; final norm, LM head, argmax [P1 "llama3-from-scratch" 11-12]).

The full logits (64 x 128256) are too large to store, so the file keeps, per
sequence, the argmax, the top-2 gap, the maximum |logit| (the scale of the
per-tensor tolerance), the 32 largest logits with their ids, and the logits
at a fixed stride of vocabulary ids; plus the new token's key and value
(after RoPE) at three layers.

  argmax    int64 [64]          top2_gap  [64]          max_abs  [64]
  top_idx   int64 [64, 32]      top_val   [64, 32]
  stride_idx int64 [Ns]         stride_val [64, Ns]
  kv_layers int64 [3]           new_k, new_v float32 [3, 64, 1024]
  ids_sha256                    hash of the 64 token ids

On this container it takes about ten minutes.  Usage:
    python tests/golden/make_decode_8b_oracle.py [--out PATH]
"""
from __future__ import annotations

import argparse
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import inputs as I  # noqa: E402
from oracle import llama as OL  # noqa: E402
from oracle import runner as OR  # noqa: E402

OUT = os.path.join(HERE, "decode_8b_b64_oracle.npz")
STRIDE = 61
TOPK = 32
KV_LAYERS = (0, 15, 31)


def summarize(logits: np.ndarray, stride_idx: np.ndarray) -> dict:
    top_idx = np.argsort(-logits, axis=1, kind="stable")[:, :TOPK]
    return dict(argmax=OL.argmax_first(logits).astype(np.int64), top2_gap=OL.top2_gap(logits),
                max_abs=np.max(np.abs(logits), axis=1), top_idx=top_idx.astype(np.int64),
                top_val=np.take_along_axis(logits, top_idx, axis=1), stride_idx=stride_idx,
                stride_val=logits[:, stride_idx])


def run(cfg: I.Config, seq_groups: int = 8, kv_layers=KV_LAYERS, log=print) -> dict:
    B = cfg.batch
    G, hd = cfg.n_kv_heads, cfg.head_dim
    stride_idx = np.arange(0, cfg.vocab_size, STRIDE, dtype=np.int64)
    logits = np.empty((B, cfg.vocab_size))
    new_k = np.zeros((len(kv_layers), B, G * hd), np.float32)
    new_v = np.zeros_like(new_k)
    per = (B + seq_groups - 1) // seq_groups
    for s0 in range(0, B, per):
        t0 = time.time()
        seqs = list(range(s0, min(B, s0 + per)))
        nk = []
        r = OR.decode(cfg, seqs, new_kv=nk)
        logits[seqs] = r["logits"]
        for (bi, l, k, v) in nk:
            if l in kv_layers:
                new_k[kv_layers.index(l), seqs[bi]] = k.reshape(-1)
                new_v[kv_layers.index(l), seqs[bi]] = v.reshape(-1)
        log(f"sequences {seqs[0]}..{seqs[-1]}: {time.time() - t0:.1f} s")
    ids = I.prompt_ids(cfg).reshape(-1).astype(np.int32)
    res = summarize(logits, stride_idx)
    res.update(kv_layers=np.array(kv_layers, dtype=np.int64), new_k=new_k, new_v=new_v,
               ids_sha256=np.array(hashlib.sha256(ids.tobytes()).hexdigest()))
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--out", default=OUT)
    args = ap.parse_args()
    t0 = time.time()
    res = run(I.CONFIGS["c5"], log=lambda s: print(s, flush=True))
    np.savez_compressed(args.out, **res)
    print(f"wrote {args.out} in {time.time() - t0:.0f} s; min top-2 gap {res['top2_gap'].min():.3e}", flush=True)


if __name__ == "__main__":
    main()
