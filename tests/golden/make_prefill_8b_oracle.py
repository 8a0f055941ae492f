#!/usr/bin/env python3
"""Writes the fp64 oracle's own result for the full 32-layer 8B-shaped prefill
(batch 1 x 8192 seeded token ids, vocabulary 128256) to
``prefill_8b_s8192_oracle.npz`` beside this file.

TEST INFRASTRUCTURE.  This script imports only ``oracle`` and ``inputs``:
the stored values come from the oracle alone, never from the HIP path.  It
runs the oracle's layer function 32 times on the whole sequence (every row,
every layer, exact fp64, no GPU-fed inputs), then the oracle's final RMSNorm,
LM head, argmax and top-2 gap on the last row, in the order of the pages'
walk-through [P1 "llama3-from-scratch" sections 10-12: all layers, final norm,
output logits, argmax; P2 section 4, Transformer.forward].

Stored (``.npz``, float64 unless noted):
  logits        [128256]   last-row logits
  argmax        int64      smallest index of the maximum
  top2_gap      scalar     largest minus second-largest logit
  hf            [4096]     final-normed last row
  rows          int64 [R]  sampled positions
  depths        int64 [K]  layer counts after which hidden rows were kept
  hidden_rows   float32 [K, R, 4096]  hidden state (residual stream) at the
                sampled rows after each depth in ``depths``; the last depth
                is 32, the stack's final hidden state
  ids_sha256    hash of the token ids, so a test can tell the inputs changed

On this container (8 cores, OpenBLAS fp64 ~370 GFLOP/s) it takes about half
an hour and ~8 GB of memory.  Usage:
    python tests/golden/make_prefill_8b_oracle.py [--out PATH]
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

OUT = os.path.join(HERE, "prefill_8b_s8192_oracle.npz")
# sampled positions: both ends, tile edges of 64/128/256, an odd interior row
ROWS = (0, 1, 63, 64, 255, 256, 1000, 4095, 5001, 8190, 8191)
DEPTHS = (1, 8, 16, 24, 32)


def ids_hash(ids: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(ids, dtype=np.int32).tobytes()).hexdigest()


def run(cfg: I.Config, rows=ROWS, depths=DEPTHS, log=print) -> dict:
    """The oracle's prefill of ``cfg`` (batch 1), keeping sampled hidden rows
    after each depth in ``depths``.  Composition identical to
    ``oracle.llama.prefill``: embedding rows, layer_forward per layer on the
    whole sequence, then the head on the last row."""
    assert cfg.batch == 1
    m = OR.model_of(cfg)
    a = OR.args_of(cfg)
    ids = I.prompt_ids(cfg)[0]
    S = ids.shape[0]
    positions = np.arange(S)
    h = OL._f64(m.rows("tok_embeddings", ids))
    kept = []
    for l in range(cfg.n_layers):
        t0 = time.time()
        lw = {k: OL._f64(v) for k, v in m.layer(l).items()}
        h = OL.layer_forward(h, lw, a, positions)
        del lw
        if l + 1 in depths:
            kept.append(h[list(rows)].astype(np.float32))
        log(f"layer {l}: {time.time() - t0:.1f} s")
    last = h[-1:]
    hf = OL.rms_norm(last, m.get("norm"), cfg.norm_eps)
    logits = OL.lm_head(hf, m.get("output"))
    return dict(logits=logits[0], argmax=np.int64(OL.argmax_first(logits)[0]),
                top2_gap=np.float64(OL.top2_gap(logits)[0]), hf=hf[0], rows=np.array(rows, dtype=np.int64),
                depths=np.array(depths, dtype=np.int64), hidden_rows=np.stack(kept),
                ids_sha256=np.array(ids_hash(ids)))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--out", default=OUT)
    args = ap.parse_args()
    cfg = I.CONFIGS["c4"]
    t0 = time.time()
    res = run(cfg, log=lambda s: print(s, flush=True))
    np.savez_compressed(args.out, **res)
    print(f"wrote {args.out} in {time.time() - t0:.0f} s: argmax {int(res['argmax'])}, "
          f"top-2 gap {float(res['top2_gap']):.4e}", flush=True)


if __name__ == "__main__":
    main()
