"""Seeded input generator: determinism, addressability, bf16 rounding (CPU only)."""
import numpy as np
import torch

import inputs as I


def test_streams_are_deterministic_and_addressable():
    a = I.normal(7, "layers.0.attention.wq.weight", (64, 1000), 0.02, True)
    b = I.normal(7, "layers.0.attention.wq.weight", (64, 1000), 0.02, True)
    assert np.array_equal(a, b)
    # a flat sub-range equals the same slice of the full tensor, across a chunk boundary
    n = I.CHUNK + 5000
    full = I.normal(3, "cache_k.0", (n,), 1.0, True)
    part = I.normal(3, "cache_k.0", (n,), 1.0, True, start=I.CHUNK - 100, stop=I.CHUNK + 50)
    assert np.array_equal(part, full[I.CHUNK - 100:I.CHUNK + 50])
    # different names and seeds give different streams
    assert not np.array_equal(a, I.normal(7, "layers.0.attention.wk.weight", (64, 1000), 0.02, True))
    assert not np.array_equal(a, I.normal(8, "layers.0.attention.wq.weight", (64, 1000), 0.02, True))


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 1, 100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0, 65504.0], np.float32)])
    ours = I.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = I.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_distributions():
    w = I.normal(1, "w", (1 << 20,), 0.02, True)
    assert abs(w.mean()) < 1e-4 and abs(w.std() - 0.02) < 2e-4
    assert np.array_equal(w, I.bf16_bits_to_f32(I.f32_to_bf16_bits(w)))
    ids = I.token_ids(1, "ids", (4, 1024), 68)
    assert ids.dtype == np.int32 and ids.min() >= 0 and ids.max() < 68 and len(np.unique(ids)) == 68


def test_model_rows_match_full_table():
    cfg = I.CONFIGS["c1"].with_(vocab_size=50, dim=64, n_heads=4, n_kv_heads=2)
    m = I.SyntheticModel(cfg, 192)
    full = m.get("tok_embeddings")
    rows = np.array([3, 0, 49, 3])
    assert np.array_equal(m.rows("tok_embeddings", rows), full[rows])
    assert np.all(m.get("norm") == 1.0)
    m2 = I.SyntheticModel(cfg.with_(norm_std=0.1), 192)
    assert not np.all(m2.get("norm") == 1.0)


def test_kv_cache_block_slices():
    cfg = I.CONFIGS["c5"].with_(batch=3, cache_len=16, n_kv_heads=2, dim=64, n_heads=4)
    full = I.kv_cache_block(cfg, 0, "k")
    assert full.shape == (3, 16, 2, 16)
    assert np.array_equal(I.kv_cache_block(cfg, 0, "k", 1, 2)[0], full[1])


def test_bits_match_values():
    cfg = I.CONFIGS["c2"].with_(dim=128, n_heads=2, n_kv_heads=1, vocab_size=300)
    m = I.SyntheticModel(cfg, 256)
    assert np.array_equal(I.bf16_bits_to_f32(m.bits("wq", 0)), m.get("wq", 0))
    n = I.CHUNK + 77
    bits = I.normal_bits(4, "t", (n,), 0.5)
    assert np.array_equal(I.bf16_bits_to_f32(bits), I.normal(4, "t", (n,), 0.5, True))
    c5 = I.CONFIGS["c5"].with_(batch=2, cache_len=8, n_kv_heads=2, dim=128, n_heads=2)
    assert np.array_equal(I.bf16_bits_to_f32(I.kv_cache_bits(c5, 1, "v")), I.kv_cache_block(c5, 1, "v"))


def test_model_rows_across_chunk_boundaries(monkeypatch):
    # rows that straddle stream chunks are assembled from each chunk drawn once
    monkeypatch.setattr(I, "CHUNK", 1000)
    cfg = I.CONFIGS["c2"].with_(vocab_size=97, dim=96, n_heads=2, n_kv_heads=1)
    m = I.SyntheticModel(cfg, 256)
    full = m.get("tok_embeddings")
    rows = np.array([0, 10, 11, 96, 10, 41, 42])
    assert np.array_equal(m.rows("tok_embeddings", rows), full[rows])
