"""Device-side plumbing around the C ABI: uploads seeded synthetic inputs to
the GPU, builds the argument structs and owns the workspace.

Nothing here computes any step of the forward pass; it moves bytes (bf16 bit
patterns are uploaded unchanged) and calls the entry points of the binding.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

import inputs as I

from . import (LLAMA_BF16, LLAMA_F32, kv_array, llama_decode_step, llama_ffn_hidden_dim, llama_layer_forward,
               llama_prefill, llama_workspace_bytes, lm_head_argmax, make_args, model_struct)

DEV = "cuda"


def bits_to_device(bits: np.ndarray, device: str = DEV) -> torch.Tensor:
    """Upload bf16 bit patterns (uint16) as a bfloat16 tensor."""
    return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)


def to_device(a: np.ndarray, bf16: bool, device: str = DEV) -> torch.Tensor:
    """Upload float32 values; bf16 tensors get the exact bf16 bit patterns."""
    if bf16:
        bits = I.f32_to_bf16_bits(a)
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def args_for(cfg: I.Config, max_batch: Optional[int] = None, max_seq: Optional[int] = None):
    return make_args(cfg.dim, cfg.n_layers, cfg.n_heads, cfg.n_kv_heads, cfg.vocab_size, cfg.multiple_of,
                     cfg.ffn_dim_multiplier, cfg.norm_eps, cfg.rope_theta,
                     max_batch_size=max_batch or cfg.batch, max_seq_len=max_seq or max(cfg.seq_len, cfg.cache_cap),
                     dtype=LLAMA_BF16 if cfg.bf16 else LLAMA_F32)


class DeviceModel:
    """Seeded weights of a configuration resident on the GPU."""

    def __init__(self, cfg: I.Config, n_layers: Optional[int] = None, with_head: bool = True, device: str = DEV):
        self.cfg = cfg
        self.args = args_for(cfg)
        self.F = llama_ffn_hidden_dim(self.args)
        self.syn = I.SyntheticModel(cfg, self.F)
        L = cfg.n_layers if n_layers is None else n_layers
        self.args.n_layers = L
        self.layers: List[dict] = []
        for l in range(L):
            self.layers.append({k: self._up(k, l, device) for k in I.LAYER_TENSORS})
        self.tok = self.norm = self.output = None
        if with_head:
            self.tok = self._up("tok_embeddings", None, device)
            self.norm = self._up("norm", None, device)
            self.output = self._up("output", None, device)
        self._model = None

    def _up(self, kind, layer, device):
        if self.cfg.bf16:
            return bits_to_device(self.syn.bits(kind, layer), device)
        return to_device(self.syn.get(kind, layer), False, device)

    @property
    def struct(self):
        if self._model is None:
            self._model = model_struct(self.tok, self.layers, self.norm, self.output)
        return self._model


def workspace(args, batch: int, seq_len: int, device: str = DEV) -> torch.Tensor:
    n = llama_workspace_bytes(args, batch, seq_len)
    return torch.empty(n, dtype=torch.uint8, device=device)


def kv_caches(cfg: I.Config, n_layers: int, batch: int, cap: int, device: str = DEV):
    dt = torch.bfloat16 if cfg.bf16 else torch.float32
    shape = (batch, cap, cfg.n_kv_heads, cfg.head_dim)
    return [(torch.zeros(shape, dtype=dt, device=device), torch.zeros(shape, dtype=dt, device=device))
            for _ in range(n_layers)]


__all__ = ["to_device", "args_for", "DeviceModel", "workspace", "kv_caches", "kv_array", "llama_layer_forward",
           "llama_prefill", "llama_decode_step", "lm_head_argmax"]
