"""Helpers shared by the GPU parity tests (comparison against the oracle)."""
import sys

import numpy as np
import torch

from oracle import llama as OL

BF16_TOL = 2e-2   # max|gpu - ref| <= 2e-2 * max|ref| for bf16 configurations
F32_TOL = 1e-4    # ... <= 1e-4 * max|ref| for fp32 configurations
GAP_EXEMPT = 1e-3  # argmax ids may differ only where the oracle's top-2 gap is below this


def bf16_stack_tol(n_layers: int) -> float:
    """Bar for outputs of a stack of n bf16 layers (bf16 MFMA operands and
    bf16 K/V cache, as the pages store activations): BF16_TOL up to four
    layers, growing like sqrt(n) beyond.  Derived in tests/bf16_drift_model.py,
    a float32 emulation of the kernels' rounding points against the fp64
    oracle: the max-abs ratio grows like sqrt(L) (8.6e-3 after one layer,
    4.3e-2 after 32), and the bf16 K/V cache alone reaches 2.0e-2 after 32."""
    return BF16_TOL * max(1.0, (n_layers / 4.0) ** 0.5)


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got, ref, tol: float, name: str):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = float(np.max(np.abs(got - ref)))
    scale = float(np.max(np.abs(ref)))
    say(f"  {name}: max_err={err:.3e} max_ref={scale:.3e} ratio={err / max(scale, 1e-300):.3e} (tol {tol:g})")
    assert err <= tol * scale, f"{name}: max err {err:.3e} > {tol:g} * {scale:.3e}"


def assert_argmax(got_ids, ref_logits, name: str):
    ref_logits = np.atleast_2d(np.asarray(ref_logits, dtype=np.float64))
    got_ids = np.asarray(got_ids).reshape(-1)
    ref_ids = OL.argmax_first(ref_logits)
    gaps = OL.top2_gap(ref_logits)
    say(f"  {name}: ids agree {int(np.sum(got_ids == ref_ids))}/{len(ref_ids)}, min top-2 gap {gaps.min():.3e}")
    for b in range(len(ref_ids)):
        if got_ids[b] != ref_ids[b]:
            assert gaps[b] < GAP_EXEMPT, f"{name}[{b}]: gpu {got_ids[b]} vs oracle {ref_ids[b]} (gap {gaps[b]:.3e})"
            # the chosen id must itself be a near-maximum of the oracle's logits
            assert ref_logits[b, ref_ids[b]] - ref_logits[b, got_ids[b]] < GAP_EXEMPT
