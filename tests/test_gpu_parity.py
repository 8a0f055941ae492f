"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  Needs an MI355X and the built library."""
import numpy as np
import pytest
import torch

import dense_decoder_only_rmsnorm_amd as M
import inputs as I
from dense_decoder_only_rmsnorm_amd import runtime as R
from gpu_util import BF16_TOL, F32_TOL, assert_argmax, assert_close, host, say
from oracle import llama as OL
from oracle import runner as OR

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def small_cfg(dtype, D, H, G, S, B=1, L=1, V=1000, norm_std=0.1, seed=11, multiple_of=64):
    return I.Config(f"small-{dtype}-{D}-{H}-{G}", dim=D, n_layers=L, n_heads=H, n_kv_heads=G, vocab_size=V,
                    multiple_of=multiple_of, ffn_dim_multiplier=None, norm_eps=1e-5, rope_theta=500000.0,
                    dtype=dtype, batch=B, seq_len=S, seed=seed, norm_std=norm_std, kind="layer")


LAYER_CASES = [
    ("bf16", 256, 4, 2, 100, 2),    # hd 64, n_rep 2, ragged tiles
    ("bf16", 384, 4, 1, 130, 1),    # hd 96, n_rep 4
    ("bf16", 512, 4, 4, 70, 1),     # hd 128, MHA
    ("bf16", 1024, 8, 1, 200, 1),   # hd 128, MQA (n_rep 8)
    ("bf16", 1024, 8, 2, 300, 2),   # hd 128, n_rep 4, several 256-row tiles
    ("bf16", 512, 4, 2, 300, 1),    # hd 128, n_rep 2
    ("bf16", 2048, 16, 1, 100, 1),  # hd 128, n_rep 16 (16 positions per block)
    ("bf16", 512, 8, 8, 90, 1),     # hd 64, MHA
    ("bf16", 512, 8, 1, 150, 1),    # hd 64, n_rep 8
    ("bf16", 1024, 16, 1, 140, 1),  # hd 64, n_rep 16 (8 positions per block)
    ("bf16", 768, 8, 1, 100, 1),    # hd 96, n_rep 8
    ("bf16", 1536, 16, 1, 70, 1),   # hd 96, n_rep 16
    ("f32", 256, 4, 2, 100, 2),
    ("f32", 384, 4, 1, 65, 1),
    ("f32", 512, 4, 4, 70, 1),
    ("f32", 512, 8, 1, 50, 1),      # fp32, n_rep 8
]


@pytest.mark.parametrize("dtype,D,H,G,S,B", LAYER_CASES)
def test_layer_forward_small(dtype, D, H, G, S, B):
    cfg = small_cfg(dtype, D, H, G, S, B)
    say(f"case layer {cfg.key} S={S} B={B}")
    dm = R.DeviceModel(cfg, with_head=False)
    x = I.hidden_x(cfg)
    xd = torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    cap = S
    kv = R.kv_caches(cfg, 1, B, cap)[0]
    args = R.args_for(cfg, max_batch=B, max_seq=cap)
    ws = R.workspace(args, B, S)
    M.llama_layer_forward(args, dm.layers[0], xd, y, B, S, 0, kv=kv, ws=ws)
    torch.cuda.synchronize()
    ref = OR.layer(cfg, x, taps=True)
    tol = BF16_TOL if cfg.bf16 else F32_TOL
    assert_close(host(y), ref["y"], tol, "layer output")
    for b in range(B):
        t = ref["taps"][b]
        assert_close(host(kv[0][b]), t["k"], tol, f"k cache (rotated) seq {b}")
        assert_close(host(kv[1][b]), t["v"], tol, f"v cache seq {b}")


# bf16 layers on at most 64 tokens take the skinny (weight-streaming) path
FEW_TOKEN_CASES = [
    (256, 4, 2, 17, 2),    # hd 64, n_rep 2, 34 tokens
    (384, 4, 1, 64, 1),    # hd 96, n_rep 4, exactly 64 tokens
    (1024, 8, 1, 9, 3),    # hd 128, n_rep 8
    (512, 4, 4, 1, 5),     # hd 128, MHA, one token per sequence
    (1152, 12, 3, 21, 1),  # hd 96, QKV of 1728 rows (ragged 128-row block)
]


@pytest.mark.parametrize("D,H,G,S,B", FEW_TOKEN_CASES)
def test_layer_forward_few_tokens(D, H, G, S, B):
    cfg = small_cfg("bf16", D, H, G, S, B)
    say(f"case layer few tokens {cfg.key} S={S} B={B}")
    dm = R.DeviceModel(cfg, with_head=False)
    x = I.hidden_x(cfg)
    xd = torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    cap = S + 3
    kv = R.kv_caches(cfg, 1, B, cap)[0]
    args = R.args_for(cfg, max_batch=B, max_seq=cap)
    ws = R.workspace(args, B, S)
    M.llama_layer_forward(args, dm.layers[0], xd, y, B, S, 0, kv=kv, ws=ws)
    torch.cuda.synchronize()
    ref = OR.layer(cfg, x, taps=True)
    assert_close(host(y), ref["y"], BF16_TOL, "layer output")
    for b in range(B):
        t = ref["taps"][b]
        assert_close(host(kv[0][b, :S]), t["k"], BF16_TOL, f"k cache (rotated) seq {b}")
        assert_close(host(kv[1][b, :S]), t["v"], BF16_TOL, f"v cache seq {b}")
    # in place (y aliases x), without a cache
    M.llama_layer_forward(args, dm.layers[0], xd, xd, B, S, 0, kv=None, ws=ws)
    torch.cuda.synchronize()
    assert_close(host(xd), ref["y"], BF16_TOL, "layer output in place")


# Sharp attention: scores peak at the diagonal, so a row's running maximum
# jumps when the tile holding its most recent keys arrives.
SHARP_CASES = [
    (512, 4, 2, 300, 1, False),  # hd 128 (eight-wave kernel), n_rep 2
    (512, 4, 2, 300, 1, True),   # the same with three documents
    (256, 4, 2, 200, 2, False),  # hd 64
]


def sharp_layer(cfg):
    """Weights and input for which the first query head of each KV group
    attends sharply to the most recent keys: wq is scaled by 4 (bf16-exact),
    each group's wk rows copy that head's wq rows, and every input row is one
    shared row plus small noise.  q_i . k_j then depends mostly on i - j and
    peaks at j = i.  Returns (layer weights as float32 arrays, x [B, S, D])."""
    lw = {k: v.copy() for k, v in OR.model_of(cfg).layer(0).items()}
    hd, rep = cfg.head_dim, cfg.n_heads // cfg.n_kv_heads
    lw["wq"] = lw["wq"] * np.float32(4.0)
    for g in range(cfg.n_kv_heads):
        lw["wk"][g * hd:(g + 1) * hd] = lw["wq"][g * rep * hd:(g * rep + 1) * hd]
    base = I.hidden_x(cfg)
    x = base[:1, :1] + np.float32(0.25) * base
    x = I.bf16_bits_to_f32(I.f32_to_bf16_bits(x))
    return lw, x


def rescales_after_first_tile(q, k, n_rep, doc=None, tile=64):
    """Rows (head, query) whose running maximum (log2 units, scale 1/sqrt(hd))
    moves by more than 8 after the row's first visible 64-key tile: where the
    attention kernels rescale their partial output mid-row."""
    S, H, hd = q.shape
    c = np.log2(np.e) / np.sqrt(hd)
    n = 0
    for h in range(H):
        s = (q[:, h] @ k[:, h // n_rep].T) * c
        for i in range(S):
            lo = 0 if doc is None else int(np.argmax(doc == doc[i]))
            m = -np.inf
            for t0 in range(lo - lo % tile, i + 1, tile):
                mx = s[i, max(t0, lo):min(t0 + tile, i + 1)].max()
                if m != -np.inf and mx > m + 8:
                    n += 1
                if mx > m + 8:
                    m = max(m, mx)
    return n


@pytest.mark.parametrize("D,H,G,S,B,docs", SHARP_CASES)
def test_layer_forward_sharp_attention(D, H, G, S, B, docs):
    cfg = small_cfg("bf16", D, H, G, S, B)
    say(f"case layer, sharp attention {cfg.key} S={S} B={B} documents={docs}")
    lw, x = sharp_layer(cfg)
    dev = {k: R.bits_to_device(I.f32_to_bf16_bits(v)) for k, v in lw.items()}
    doc = None
    if docs:
        lens = [110, 90, S - 200]
        doc = np.concatenate([np.full(n, i, np.int32) for i, n in enumerate(lens)])
        doc = np.tile(doc, (B, 1))
    xd = torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    kv = R.kv_caches(cfg, 1, B, S)[0]
    args = R.args_for(cfg, max_batch=B, max_seq=S)
    ws = R.workspace(args, B, S)
    if doc is None:
        M.llama_layer_forward(args, dev, xd, y, B, S, 0, kv=kv, ws=ws)
    else:
        M.llama_layer_forward_docs(args, dev, xd, y, B, S, 0, kv=kv, doc_ids=torch.from_numpy(doc).cuda(), ws=ws)
    torch.cuda.synchronize()
    a = OR.args_of(cfg)
    for b in range(B):
        t = {}
        if doc is None:
            ref = OL.layer_forward(x[b], lw, a, np.arange(S), taps=t)
        else:
            ref = OL.layer_forward(x[b], lw, a, np.arange(S), taps=t, doc_ids=doc[b])
        # the inputs really drive the mid-row rescale
        assert rescales_after_first_tile(t["q"], t["k"], H // G, None if doc is None else doc[b]) >= 20
        assert_close(host(y[b]), ref, BF16_TOL, f"layer output seq {b}")
        assert_close(host(kv[0][b]), t["k"], BF16_TOL, f"k cache (rotated) seq {b}")
        assert_close(host(kv[1][b]), t["v"], BF16_TOL, f"v cache seq {b}")


def test_chunked_prefill_few_tokens_per_chunk():
    # three chunks of 20, 12 and 1 positions for 2 sequences, each under 64 tokens
    chunks = [20, 12, 1]
    S = sum(chunks)
    cfg = small_cfg("bf16", 512, 8, 2, S, 2)
    say(f"case chunked prefill, few tokens per chunk {cfg.key}")
    dm = R.DeviceModel(cfg, with_head=False)
    x = I.hidden_x(cfg)
    cap = 40
    kv = R.kv_caches(cfg, 1, 2, cap)[0]
    args = R.args_for(cfg, max_batch=2, max_seq=cap)
    ws = R.workspace(args, 2, max(chunks))
    outs, p0 = [], 0
    for n in chunks:
        xc = torch.from_numpy(np.ascontiguousarray(x[:, p0:p0 + n])).cuda()
        yc = torch.empty_like(xc)
        M.llama_layer_forward(args, dm.layers[0], xc, yc, 2, n, p0, kv=kv, ws=ws)
        outs.append(yc)
        p0 += n
    torch.cuda.synchronize()
    ref = OR.layer(cfg, x)["y"]
    assert_close(np.concatenate([host(o) for o in outs], axis=1), ref, BF16_TOL, "chunked layer output")


def test_prefill_small_stack_few_tokens():
    cfg = I.CONFIGS["c2"].with_(batch=4, seq_len=16)
    say("case prefill, small GQA stack, 4 x 16 tokens (skinny path)")
    _, ids, hidden, logits, nid, _ = _run_prefill(cfg, kv_cap=24)
    ref = OR.prefill(cfg, ids, all_hidden=True)
    assert_close(host(hidden), ref["hidden"], BF16_TOL, "final hidden")
    assert_close(host(logits), ref["logits"], BF16_TOL, "logits")
    assert_argmax(nid.cpu().numpy(), ref["logits"], "argmax")


def test_layer_forward_in_place_without_cache():
    cfg = small_cfg("bf16", 512, 8, 2, 96, 1)
    say(f"case layer in-place {cfg.key}")
    dm = R.DeviceModel(cfg, with_head=False)
    x = I.hidden_x(cfg)
    xd = torch.from_numpy(x).cuda()
    args = R.args_for(cfg, max_batch=1, max_seq=96)
    ws = R.workspace(args, 1, 96)
    M.llama_layer_forward(args, dm.layers[0], xd, xd, 1, 96, 0, kv=None, ws=ws)
    torch.cuda.synchronize()
    assert_close(host(xd), OR.layer(cfg, x)["y"], BF16_TOL, "layer output (y aliases x)")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunked_prefill_with_cache(dtype):
    # two chunks: positions 0..S1-1, then S1..S1+S2-1 attending over the cache [P2 3.3]
    S1, S2 = 77, 60
    cfg = small_cfg(dtype, 512, 8, 2, S1 + S2, 2)
    say(f"case chunked prefill {cfg.key}")
    dm = R.DeviceModel(cfg, with_head=False)
    x = I.hidden_x(cfg)
    cap = 160
    kv = R.kv_caches(cfg, 1, 2, cap)[0]
    args = R.args_for(cfg, max_batch=2, max_seq=cap)
    ws = R.workspace(args, 2, S1 + S2)
    x1 = torch.from_numpy(np.ascontiguousarray(x[:, :S1])).cuda()
    x2 = torch.from_numpy(np.ascontiguousarray(x[:, S1:])).cuda()
    y1, y2 = torch.empty_like(x1), torch.empty_like(x2)
    M.llama_layer_forward(args, dm.layers[0], x1, y1, 2, S1, 0, kv=kv, ws=ws)
    M.llama_layer_forward(args, dm.layers[0], x2, y2, 2, S2, S1, kv=kv, ws=ws)
    torch.cuda.synchronize()
    ref = OR.layer(cfg, x)["y"]
    tol = BF16_TOL if cfg.bf16 else F32_TOL
    assert_close(np.concatenate([host(y1), host(y2)], axis=1), ref, tol, "chunked layer output")


def _run_prefill(cfg, n_layers=None, kv_cap=None):
    dm = R.DeviceModel(cfg, n_layers=n_layers)
    B, S = cfg.batch, cfg.seq_len
    ids = I.prompt_ids(cfg)
    idd = torch.from_numpy(ids).cuda()
    hidden = torch.empty((B, S, cfg.dim), dtype=torch.float32, device="cuda")
    logits = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device="cuda")
    nid = torch.empty(B, dtype=torch.int32, device="cuda")
    args = dm.args
    args.max_batch_size = B
    args.max_seq_len = kv_cap or S
    ws = R.workspace(args, B, S)
    kvs = None
    caches = None
    if kv_cap:
        caches = R.kv_caches(cfg, args.n_layers, B, kv_cap)
        kvs = M.kv_array(caches)
    M.llama_prefill(args, dm.struct, idd, B, S, kv=kvs, hidden=hidden, logits=logits, next_id=nid, ws=ws)
    torch.cuda.synchronize()
    return dm, ids, hidden, logits, nid, caches


def test_prefill_c1_fp32():
    cfg = I.CONFIGS["c1"]
    say("case prefill c1 (fp32, 8 layers, S=256)")
    _, ids, hidden, logits, nid, _ = _run_prefill(cfg)
    ref = OR.prefill(cfg, ids, all_hidden=True)
    assert_close(host(hidden), ref["hidden"], F32_TOL, "c1 final hidden")
    assert_close(host(logits), ref["logits"], F32_TOL, "c1 logits")
    assert_argmax(nid.cpu().numpy(), ref["logits"], "c1 argmax")


def test_prefill_c2_bf16():
    cfg = I.CONFIGS["c2"]
    say("case prefill c2 (bf16, 4 layers, 4 x 1024)")
    _, ids, hidden, logits, nid, _ = _run_prefill(cfg)
    ref = OR.prefill(cfg, ids, all_hidden=True)
    assert_close(host(hidden), ref["hidden"], BF16_TOL, "c2 final hidden")
    assert_close(host(logits), ref["logits"], BF16_TOL, "c2 logits")
    assert_argmax(nid.cpu().numpy(), ref["logits"], "c2 argmax")


@pytest.mark.parametrize("dtype,D,H,G", [("bf16", 512, 8, 2), ("f32", 512, 8, 2), ("bf16", 1024, 8, 2),
                                         ("bf16", 1024, 8, 1), ("bf16", 768, 8, 2),
                                         # hd 96: QKV has 1728 weight rows on 128-row blocks (ragged
                                         # last block), wo 128-row blocks without a K split
                                         ("bf16", 1152, 12, 3),
                                         # every decode-attention variant the argument checks admit:
                                         # hd 64/96 at n_rep 8 (MFMA, 8 heads) and 16 (vector
                                         # kernel), hd 128 at n_rep 16, fp32 at n_rep 8
                                         ("bf16", 512, 8, 1), ("bf16", 768, 8, 1), ("bf16", 1024, 16, 1),
                                         ("bf16", 1536, 16, 1), ("bf16", 2048, 16, 1), ("f32", 512, 8, 1)])
def test_decode_ragged_positions_match_oracle(dtype, D, H, G):
    # prefill S tokens into the cache, then one decode step with per-sequence positions
    cfg = small_cfg(dtype, D, H, G, 40, 3, L=2, V=3000, seed=21).with_(kind="prefill")
    say(f"case decode ragged {cfg.key}")
    S, B = cfg.seq_len, cfg.batch
    cap = 64
    dm, ids, _, _, _, caches = _run_prefill(cfg, kv_cap=cap)
    pos = np.array([S, S - 5, 17], dtype=np.int32)
    new_ids = np.array([5, 77, 2999], dtype=np.int32)
    logits = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device="cuda")
    nid = torch.empty(B, dtype=torch.int32, device="cuda")
    args = dm.args
    ws = R.workspace(args, B, S)
    M.llama_decode_step(args, dm.struct, torch.from_numpy(new_ids).cuda(), torch.from_numpy(pos).cuda(), B,
                        M.kv_array(caches), logits=logits, next_id=nid, ws=ws)
    torch.cuda.synchronize()
    # oracle: caches from the oracle's own prefill, truncated to each sequence's position
    ocaches = [[] for _ in range(B)]
    OR.prefill(cfg, ids, caches=ocaches)
    trunc = [[{"k": ocaches[b][l]["k"][:pos[b]], "v": ocaches[b][l]["v"][:pos[b]]} for l in range(cfg.n_layers)]
             for b in range(B)]
    m = OR.model_of(cfg)
    new_kv = []
    ref = OL.decode_step(new_ids, trunc, lambda r: m.rows("tok_embeddings", r), m.layer, m.get("norm"),
                         m.get("output"), OR.args_of(cfg), new_kv=new_kv)
    tol = BF16_TOL if cfg.bf16 else F32_TOL
    assert_close(host(logits), ref["logits"], tol, "decode logits")
    assert_argmax(nid.cpu().numpy(), ref["logits"], "decode argmax")
    for (b, l, kn, vn) in new_kv:
        assert_close(host(caches[l][0][b, pos[b]]), kn, tol, f"new k (seq {b}, layer {l})")
        assert_close(host(caches[l][1][b, pos[b]]), vn, tol, f"new v (seq {b}, layer {l})")


@pytest.mark.parametrize("M_rows", [1, 5, 64])
def test_lm_head_argmax_8b_vocab(M_rows):
    cfg = I.CONFIGS["c5"]
    say(f"case lm_head_argmax M={M_rows} V=128256")
    F = M.llama_ffn_hidden_dim(R.args_for(cfg))
    syn = I.SyntheticModel(cfg, F)
    w_out = syn.get("output")
    h = I.normal(99, "lm_head_test_h", (M_rows, cfg.dim), 1.0, False)
    args = R.args_for(cfg, max_batch=M_rows, max_seq=1)
    hd_ = torch.from_numpy(h).cuda()
    wd = R.to_device(w_out, True)
    nw = R.to_device(np.ones(cfg.dim, np.float32), True)
    logits = torch.empty((M_rows, cfg.vocab_size), dtype=torch.float32, device="cuda")
    am = torch.empty(M_rows, dtype=torch.int32, device="cuda")
    ws = R.workspace(args, M_rows, 1)
    M.lm_head_argmax(args, hd_, nw, wd, M_rows, logits=logits, argmax=am, ws=ws)
    torch.cuda.synchronize()
    hf = OL.rms_norm(h, np.ones(cfg.dim), cfg.norm_eps)
    ref = OL.lm_head(hf, w_out)
    assert_close(host(logits), ref, BF16_TOL, "lm head logits")
    # hi/lo activations: the logits are accurate to ~1e-5 relative, far below the exemption gap
    assert float(np.max(np.abs(host(logits) - ref))) < 1e-3
    assert_argmax(am.cpu().numpy(), ref, "lm head argmax")


def test_c3_layer_s17():
    cfg = I.CONFIGS["c3_s17"]
    say("case c3 one 8B layer, S=17")
    dm = R.DeviceModel(cfg, with_head=False)
    x = I.hidden_x(cfg)
    xd = torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    args = R.args_for(cfg, max_batch=1, max_seq=17)
    ws = R.workspace(args, 1, 17)
    M.llama_layer_forward(args, dm.layers[0], xd, y, 1, 17, 0, kv=None, ws=ws)
    torch.cuda.synchronize()
    assert_close(host(y), OR.layer(cfg, x)["y"], BF16_TOL, "c3 s17 layer output")


def test_c3_layer_s2048_sampled_rows():
    cfg = I.CONFIGS["c3_s2048"]
    say("case c3 one 8B layer, S=2048 (rows sampled)")
    dm = R.DeviceModel(cfg, with_head=False)
    x = I.hidden_x(cfg)
    xd = torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    args = R.args_for(cfg, max_batch=1, max_seq=2048)
    ws = R.workspace(args, 1, 2048)
    M.llama_layer_forward(args, dm.layers[0], xd, y, 1, 2048, 0, kv=None, ws=ws)
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 255, 1000, 1537, 2047]
    ref = OR.layer(cfg, x, rows=rows)["y"]
    assert_close(host(y)[:, rows], ref, BF16_TOL, "c3 s2048 sampled rows")


def test_decode_8b_shapes_two_layers_sampled_sequences():
    # batch 64 over seeded caches of 4096 positions at 8B shapes; two layers; sequences sampled for the oracle
    cfg = I.CONFIGS["c5"].with_(n_layers=2)
    say("case decode 8B shapes, 2 layers, B=64, cache 4096")
    dm = R.DeviceModel(cfg)
    B, P, cap = cfg.batch, cfg.cache_len, cfg.cache_cap
    caches = []
    for l in range(cfg.n_layers):
        pair = []
        for which in ("k", "v"):
            t = torch.zeros((B, cap, cfg.n_kv_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
            t[:, :P] = R.bits_to_device(I.kv_cache_bits(cfg, l, which))
            pair.append(t)
        caches.append(tuple(pair))
    ids = I.prompt_ids(cfg).reshape(-1).astype(np.int32)
    pos = torch.full((B,), P, dtype=torch.int32, device="cuda")
    logits = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device="cuda")
    nid = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = R.workspace(dm.args, B, 1)
    M.llama_decode_step(dm.args, dm.struct, torch.from_numpy(ids).cuda(), pos, B, M.kv_array(caches),
                        logits=logits, next_id=nid, ws=ws)
    torch.cuda.synchronize()
    seqs = [0, 29, 63]
    new_kv = []
    ref = OR.decode(cfg, seqs, new_kv=new_kv)
    got = host(logits)[seqs]
    assert_close(got, ref["logits"], BF16_TOL, "decode logits (sampled sequences)")
    assert float(np.max(np.abs(got - ref["logits"]))) < 1e-3 * float(np.max(np.abs(ref["logits"])))
    assert_argmax(nid.cpu().numpy()[seqs], ref["logits"], "decode argmax (sampled sequences)")
    for (bi, l, kn, vn) in new_kv:
        b = seqs[bi]
        assert_close(host(caches[l][0][b, P]), kn, BF16_TOL, f"new k seq {b} layer {l}")
        assert_close(host(caches[l][1][b, P]), vn, BF16_TOL, f"new v seq {b} layer {l}")
