#!/usr/bin/env python3
"""Prefill and decode tokens/s of the Llama-3-8B-shaped decoder on one MI355X.

Workloads (seeded synthetic inputs, random-init weights N(0, 0.02^2) in bf16):
  prefill  32 layers, dim 4096, 32 heads / 8 KV heads, FFN 14336, vocab
           128256; batch 1 x 8192 tokens; final norm, LM head and argmax of
           the last position.  One step = one llama_prefill call.
  decode   the same model; 64 sequences, each with a seeded KV cache of 4096
           positions; one new token per sequence at position 4096.  One step
           = one llama_decode_step call.

Prints ONE JSON line on stdout; progress goes to stderr.  ``value`` is the
prefill throughput (tokens/s); the decode throughput and both roofline
fractions are in the same line.  Timing: W untimed warmup steps, then K steps
bracketed by device synchronisation, timed with HIP events on the stream the
library launches on.  Per-kernel durations come from a second, instrumented
pass of K steps (llama_timing_enable), so the headline timing carries no
instrumentation.
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
# Per-kernel rocprofv3 counter figures (HBM bytes per launch from FETCH_SIZE
# and WRITE_SIZE, MFMA busy %% from SQ_VALU_MFMA_BUSY_CYCLES over
# GRBM_GUI_ACTIVE); each entry records the SHA-256 of the sources it was
# measured with and is used only while they are unchanged
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")


def measured(kernel, field):
    """``field`` of ``kernel`` from the committed counter summary, or None
    when there is none or the kernel's sources changed since it was taken."""
    try:
        with open(COUNTERS_FILE) as f:
            entry = json.load(f)["kernels"][kernel]
        value = entry[field]
    except (OSError, ValueError, KeyError):
        return None
    h = hashlib.sha256()
    for rel in entry["sources"]:
        try:
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
        except OSError:
            return None
    if h.hexdigest() != entry["sources_sha256"]:
        return None
    return None if value is None else float(value)


def measured_traffic(kernel):
    return measured(kernel, "bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", choices=["prefill", "decode"], default=None,
                    help="run one workload only (profiling); the JSON line then omits the other")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the packed-document prefill and the generation loop measurements")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the smaller configurations (tiny fp32 stack, small GQA stack, one 8B layer)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def time_steps(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def kernel_times(fn, steps, M, torch):
    torch.cuda.synchronize()
    M.llama_timing_enable(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    rep = M.llama_timing_report()
    M.llama_timing_enable(False)
    return {k: {"launches": n // steps, "ms_per_step": ms / steps, "avg_ms": ms / n} for k, (n, ms) in rep.items()}


def kernel_rooflines(kt, work, counter_keys=None):
    """Rate and roofline fraction of each timed kernel from its algorithmic
    work per launch (flop for "mfma", bytes for "hbm") and its event-timed
    average launch duration, with the counter figures where measured."""
    res = {}
    for name, (bound, amount) in work.items():
        if name not in kt:
            continue
        avg = kt[name]["avg_ms"]
        if bound == "mfma":
            ach, peak, unit = amount / (avg / 1e3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
        else:
            ach, peak, unit = amount / (avg / 1e3) / 1e9, PEAK_HBM_GBS, "GB/s"
        ck = (counter_keys or {}).get(name, name)
        res[name] = {"bound": bound, "avg_ms": round(avg, 5), "achieved": round(ach, 2), "unit": unit,
                     "frac": round(ach / peak, 4), "work_per_launch": amount,
                     "traffic": measured_traffic(ck), "mfma_busy_pct": measured(ck, "mfma_busy_pct")}
    return res


def cpu_threads():
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas = [i for i in info if i.get("user_api") == "blas"]
        if blas:
            return int(blas[0]["num_threads"])
    except Exception:
        pass
    return os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_info():
    return {"cores": cpu_threads(), "cpu": cpu_model(), "os_cpu_count": os.cpu_count(), "blas_threads": cpu_threads()}


def cpu_baseline_prefill(cfg, F):
    """fp64 oracle on a bounded sample of the prefill workload: layer 0 over
    the full 8192 positions (every row; attention's quadratic cost included),
    times the 32 layers, plus the embedding gather, final norm, LM head and
    argmax of the last row, all timed."""
    import numpy as np

    import inputs as I
    from oracle import llama as OL
    from oracle import runner as OR

    syn = I.SyntheticModel(cfg, F)
    ids = I.prompt_ids(cfg)[0]
    a = OR.args_of(cfg)
    lw32 = syn.layer(0)
    norm_w, w_out = syn.get("norm"), syn.get("output")
    table = syn.get("tok_embeddings")
    t0 = time.perf_counter()
    h = OL._f64(table[ids])
    t_embed = time.perf_counter() - t0
    t0 = time.perf_counter()
    lw = {k: OL._f64(v) for k, v in lw32.items()}
    h = OL.layer_forward(h, lw, a, np.arange(cfg.seq_len))
    t_layer = time.perf_counter() - t0
    t0 = time.perf_counter()
    hf = OL.rms_norm(h[-1:], norm_w, cfg.norm_eps)
    OL.argmax_first(OL.lm_head(hf, w_out))
    t_head = time.perf_counter() - t0
    total = t_embed + cfg.n_layers * t_layer + t_head
    return {"value": cfg.seq_len / total, "unit": "tokens/s", "kind": "oracle", **cpu_info(),
            "sample": f"fp64 oracle: layer 0 over all {cfg.seq_len} positions ({t_layer:.1f} s) x {cfg.n_layers} "
                      f"layers + embedding ({t_embed:.2f} s) + final norm, LM head and argmax of the last row "
                      f"({t_head:.2f} s); weights generated beforehand, untimed",
            "seconds": t_embed + t_layer + t_head}


def cpu_baseline_decode(cfg, F, L_s=4):
    """fp64 oracle on a bounded sample of the decode step: all 64 sequences
    through L_s of the 32 layers (every layer has the same shapes and cache
    length, so the step is 32/L_s times that), plus the final norm, LM head
    and argmax of all 64 rows, timed."""
    import numpy as np

    import inputs as I
    from oracle import llama as OL
    from oracle import runner as OR

    B = cfg.batch
    syn = I.SyntheticModel(cfg, F)
    ids = I.prompt_ids(cfg).reshape(-1)
    emb = syn.rows("tok_embeddings", ids)
    layers = [syn.layer(l) for l in range(L_s)]
    blocks = [{w: I.kv_cache_block(cfg, l, w) for w in ("k", "v")} for l in range(L_s)]
    norm_w, w_out = syn.get("norm"), syn.get("output")
    a = OR.args_of(cfg)
    hs = [OL._f64(emb[b:b + 1]) for b in range(B)]
    t0 = time.perf_counter()
    for l in range(L_s):
        lw = {k: OL._f64(v) for k, v in layers[l].items()}
        for b in range(B):
            cache = {"k": blocks[l]["k"][b], "v": blocks[l]["v"][b]}
            hs[b] = OL.layer_forward(hs[b], lw, a, np.array([cfg.cache_len]), cache=cache)
    t_layers = time.perf_counter() - t0
    t0 = time.perf_counter()
    hf = OL.rms_norm(np.concatenate(hs), norm_w, cfg.norm_eps)
    OL.argmax_first(OL.lm_head(hf, w_out))
    t_head = time.perf_counter() - t0
    total = t_layers * cfg.n_layers / L_s + t_head
    return {"value": B / total, "unit": "tokens/s", "kind": "oracle", **cpu_info(),
            "sample": f"fp64 oracle decode of all {B} sequences (cache {cfg.cache_len}) through {L_s} of the "
                      f"{cfg.n_layers} layers ({t_layers:.1f} s, x {cfg.n_layers // L_s}) + final norm, LM head and "
                      f"argmax of the {B} rows ({t_head:.2f} s); weights and caches generated beforehand, untimed",
            "seconds": t_layers + t_head}


def bench_long_layer(dm, cfg, M, I, R, torch):
    """One 8B-shaped layer prefilled over 32768 positions (causal): layer time
    and the attention kernel's rate on its unmasked pairs."""
    S = 32768
    lc = cfg.with_(key="long_layer", n_layers=1, seq_len=S)
    la = R.args_for(lc, max_batch=1, max_seq=S)
    x = torch.randn((1, S, cfg.dim), dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    ws = R.workspace(la, 1, S)

    def layer():
        M.llama_layer_forward(la, dm.layers[0], x, y, 1, S, 0, kv=None, ws=ws)

    ms = time_steps(layer, 3, 1, torch)
    kt = kernel_times(layer, 2, M, torch)
    attn_ms = kt["attn_prefill"]["avg_ms"]
    attn_flop = 4.0 * cfg.head_dim * cfg.n_heads * (S * (S + 1) / 2)
    res = {"seq_len": S, "layer_ms": round(ms, 3), "attn_prefill_ms": round(attn_ms, 3),
           "attn_tflops": round(attn_flop / (attn_ms / 1e3) / 1e12, 1)}
    log(f"one layer at S={S}: {ms:.2f} ms, attention {attn_ms:.2f} ms ({res['attn_tflops']} TFLOP/s)")
    del x, y, ws
    torch.cuda.empty_cache()
    return res


def bench_generate(dm, cfg, M, I, R, np, torch, B=64, gen=32, cap=256, lmin=96, lspan=65):
    """The generation loop: B prompts of lmin .. lmin+lspan-1 tokens (seeded
    lengths), gen new tokens each, greedy (graph replay and eager launches)
    and top-p sampled (T 0.6, p 0.9, the pages' defaults)."""
    lens = [int(x) for x in lmin + I.token_ids(cfg.seed, "bench_prompt_lengths", (B,), lspan)]
    P = max(lens)
    prompt = torch.from_numpy(I.token_ids(cfg.seed, "bench_prompts", (B, P), cfg.vocab_size)).cuda()
    ga = R.args_for(cfg, max_batch=B, max_seq=cap)
    caches = R.kv_caches(cfg, cfg.n_layers, B, cap)
    kvs = M.kv_array(caches)
    tokens = torch.empty((B, cap), dtype=torch.int32, device="cuda")
    out_len = torch.empty((B,), dtype=torch.int32, device="cuda")
    ws = torch.empty(M.llama_generate_workspace_bytes(ga, B, P), dtype=torch.uint8, device="cuda")
    u = torch.from_numpy(I.uniform(cfg.seed, "bench_uniforms", (gen, B))).cuda()
    stream = torch.cuda.Stream()
    res = {"batch": B, "prompt_tokens": sum(lens), "new_tokens_per_seq": gen}

    def run(temp, flags):
        with torch.cuda.stream(stream):
            M.llama_generate(ga, dm.struct, prompt, P, lens, B, gen, -1, temp, 0.9, u if temp > 0 else None, kvs,
                             tokens, out_len, flags, ws, stream)
        stream.synchronize()

    for name, temp, flags in (("greedy", 0.0, 0), ("greedy_graph", 0.0, M.LLAMA_GEN_GRAPH), ("top_p", 0.6, 0)):
        run(temp, flags)  # warm-up
        t0 = time.perf_counter()
        run(temp, flags)
        ms = (time.perf_counter() - t0) * 1e3
        res[name] = {"ms": round(ms, 2), "generated_tokens_per_s": round(B * gen / (ms / 1e3), 1)}
        log(f"generate {name}: {ms:.1f} ms for {B} x {gen} new tokens after {sum(lens)} prompt tokens")
    # one more greedy run with per-kernel timing (eager launches)
    M.llama_timing_enable(True)
    run(0.0, 0)
    rep = M.llama_timing_report()
    M.llama_timing_enable(False)
    res["kernel_ms_total"] = round(sum(ms for _, ms in rep.values()), 2)
    del caches, kvs, ws
    torch.cuda.empty_cache()
    return res


PEAK_FP32_TFLOPS = 157.3  # MI355X fp32 (vector and matrix)


def layer_flops(cfg, F, B, S):
    """Algorithmic flop of one layer on B x S tokens: GEMMs 2*M*N*K, attention
    4*hd*H per unmasked (query, key) pair."""
    D, Hq, Hk, T = cfg.dim, cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim, B * S
    gemm = 2.0 * T * D * (Hq + 2 * Hk) + 2.0 * T * Hq * D + 2.0 * T * D * 2 * F + 2.0 * T * F * D
    return gemm + 4.0 * cfg.head_dim * cfg.n_heads * B * (S * (S + 1) / 2)


def layer_weight_bytes(cfg, F):
    D, Hq, Hk = cfg.dim, cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    esz = 2 if cfg.bf16 else 4
    return esz * (D * (Hq + 2 * Hk) + Hq * D + 3 * D * F + 2 * D)


def bench_configs(M, I, R, np, torch, steps):
    """The smaller configurations: the tiny fp32 stack (1 x 256), the small
    GQA stack (4 x 1024), and one 8B-shaped layer at 17 and 2048 positions.
    Each is timed with HIP events over ``steps`` calls after warm-up; the
    17-position layer is also timed cold (a 1 GiB buffer written before each
    call evicts its 436 MB of weights from the 256 MB Infinity Cache)."""
    res = {}
    for key in ("c1", "c2"):
        cfg = I.CONFIGS[key]
        dm = R.DeviceModel(cfg)
        B, S = cfg.batch, cfg.seq_len
        args = dm.args
        args.max_batch_size, args.max_seq_len = B, S
        ids = torch.from_numpy(I.prompt_ids(cfg)).cuda()
        logits = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device="cuda")
        nid = torch.empty(B, dtype=torch.int32, device="cuda")
        ws = R.workspace(args, B, S)

        def run():
            M.llama_prefill(args, dm.struct, ids, B, S, kv=None, logits=logits, next_id=nid, ws=ws)

        ms = time_steps(run, steps, 3, torch)
        kt = kernel_times(run, steps, M, torch)
        flop = cfg.n_layers * layer_flops(cfg, dm.F, B, S) + 2.0 * B * cfg.dim * cfg.vocab_size
        tf = flop / (ms / 1e3) / 1e12
        peak = PEAK_BF16_TFLOPS if cfg.bf16 else PEAK_FP32_TFLOPS
        res[key] = {"workload": f"{cfg.n_layers}-layer stack dim {cfg.dim}, {cfg.n_heads}/{cfg.n_kv_heads} heads, "
                                f"vocab {cfg.vocab_size}, {cfg.dtype}; prefill {B} x {S} + LM head",
                    "ms": round(ms, 4), "tokens_per_s": round(B * S / (ms / 1e3), 1),
                    "roofline": {"bound": "mfma" if cfg.bf16 else "fp32", "achieved": round(tf, 2),
                                 "unit": "TFLOP/s", "peak": peak, "frac": round(tf / peak, 4), "flop": flop},
                    "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in
                                            sorted(kt.items(), key=lambda kv: -kv[1]["ms_per_step"])}}
        log(f"{key}: {ms:.3f} ms, {B * S / (ms / 1e3):.0f} tokens/s, {tf:.1f} TFLOP/s")
        del dm, ws, logits
    for key in ("c3_s17", "c3_s2048"):
        cfg = I.CONFIGS[key]
        dm = R.DeviceModel(cfg, with_head=False)
        S = cfg.seq_len
        args = R.args_for(cfg, max_batch=1, max_seq=S)
        x = torch.from_numpy(I.hidden_x(cfg)).cuda()
        y = torch.empty_like(x)
        ws = R.workspace(args, 1, S)

        def run():
            M.llama_layer_forward(args, dm.layers[0], x, y, 1, S, 0, kv=None, ws=ws)

        ms = time_steps(run, steps, 3, torch)
        entry = {"workload": f"one 8B-shaped layer, x ~ N(0,1) [1, {S}, 4096], bf16", "ms": round(ms, 4),
                 "tokens_per_s": round(S / (ms / 1e3), 1)}
        if key == "c3_s17":
            wb = layer_weight_bytes(cfg, dm.F)
            flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
            cold = []
            for _ in range(steps):
                flush.zero_()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                run()
                e1.record()
                torch.cuda.synchronize()
                cold.append(e0.elapsed_time(e1))
            cms = float(np.median(cold))
            del flush
            gw, gc = wb / (ms / 1e3) / 1e9, wb / (cms / 1e3) / 1e9
            entry.update(cold_ms=round(cms, 4), cold_tokens_per_s=round(S / (cms / 1e3), 1),
                         roofline={"bound": "hbm", "bytes": wb, "unit": "GB/s", "peak": PEAK_HBM_GBS,
                                   "achieved_cold": round(gc, 1), "frac_cold": round(gc / PEAK_HBM_GBS, 4),
                                   "achieved_warm": round(gw, 1), "frac_warm": round(gw / PEAK_HBM_GBS, 4)})
            log(f"{key}: warm {ms:.4f} ms, cold {cms:.4f} ms ({gc:.0f} GB/s of weights)")
        else:
            flop = layer_flops(cfg, dm.F, 1, S)
            tf = flop / (ms / 1e3) / 1e12
            entry["roofline"] = {"bound": "mfma", "achieved": round(tf, 2), "unit": "TFLOP/s",
                                 "peak": PEAK_BF16_TFLOPS, "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flop": flop}
            log(f"{key}: {ms:.4f} ms, {tf:.1f} TFLOP/s")
        res[key] = entry
        del dm, x, y, ws
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("bench.py measures one GPU only: the library runs the whole forward pass on a single MI355X "
               "and implements no multi-GPU sharding; rerun with --gpus 1")
        log(msg)
        sys.exit(2)

    import numpy as np
    import torch

    import dense_decoder_only_rmsnorm_amd as M
    import inputs as I
    from dense_decoder_only_rmsnorm_amd import runtime as R

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copy of 1 GiB done")
    c4, c5 = I.CONFIGS["c4"], I.CONFIGS["c5"]
    t0 = time.time()
    log("generating and uploading the 8B-shaped weights (seed of the prefill configuration) ...")
    dm = R.DeviceModel(c4)
    F = dm.F
    log(f"  weights ready in {time.time() - t0:.1f} s (F={F})")
    out = {}
    kern = {}

    def summarize(ktimes):
        return {k: round(v["avg_ms"], 5) for k, v in sorted(ktimes.items(), key=lambda kv: -kv[1]["ms_per_step"])}

    if args.only in (None, "prefill"):
        B, S = c4.batch, c4.seq_len
        pa = R.args_for(c4, max_batch=B, max_seq=S)
        ids = torch.from_numpy(I.prompt_ids(c4)).cuda()
        logits = torch.empty((B, c4.vocab_size), dtype=torch.float32, device="cuda")
        nid = torch.empty(B, dtype=torch.int32, device="cuda")
        ws = R.workspace(pa, B, S)

        def prefill():
            M.llama_prefill(pa, dm.struct, ids, B, S, kv=None, logits=logits, next_id=nid, ws=ws)

        ms = time_steps(prefill, args.steps, args.warmup, torch)
        kt = kernel_times(prefill, args.steps, M, torch)
        kern["prefill"] = kt
        log(f"prefill: {ms:.3f} ms/step, {B * S / (ms / 1e3):.0f} tokens/s")
        for k, v in sorted(kt.items(), key=lambda kv: -kv[1]["ms_per_step"]):
            log(f"  {k:22s} {v['launches']:5d} launches  {v['ms_per_step']:9.3f} ms/step  avg {v['avg_ms']:.4f} ms")
        # per-kernel algorithmic work per launch (GEMM 2*M*N*K; attention 4*hd*H
        # per unmasked (query, key) pair; the LM head is bound by its weight read)
        D, Hq, Hk, T = c4.dim, c4.n_heads * c4.head_dim, c4.n_kv_heads * c4.head_dim, B * S
        work = {"gemm_qkv_rope": ("mfma", 2.0 * T * D * (Hq + 2 * Hk)),
                "gemm_wo_resid": ("mfma", 2.0 * T * Hq * D),
                "gemm_w1w3_swiglu": ("mfma", 2.0 * T * D * 2 * F),
                "gemm_w2_resid": ("mfma", 2.0 * T * F * D),
                "attn_prefill": ("mfma", 4.0 * c4.head_dim * c4.n_heads * B * (S * (S + 1) / 2)),
                "lm_head": ("hbm", 2.0 * c4.vocab_size * D)}
        per_kernel = kernel_rooflines(kt, work, {"lm_head": "lm_head_prefill"})
        total_flop = c4.n_layers * sum(work[k][1] for k in work if k != "lm_head") + 2.0 * B * D * c4.vocab_size
        step_tflops = total_flop / (ms / 1e3) / 1e12
        # dominant kernel: the fused w1/w3 SwiGLU GEMM (47% of the layer FLOPs)
        dk = per_kernel["gemm_w1w3_swiglu"]
        out["prefill"] = dict(ms=ms, tok_s=B * S / (ms / 1e3), step_tflops=step_tflops, kernels=per_kernel,
                              roofline={"kernel": "gemm_w1w3_swiglu", "bound": "mfma", "achieved": dk["achieved"],
                                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": dk["frac"],
                                        "traffic": measured_traffic("gemm_w1w3_swiglu"),
                                        "mfma_busy_pct": measured("gemm_w1w3_swiglu", "mfma_busy_pct"),
                                        "flop_per_launch": work["gemm_w1w3_swiglu"][1],
                                        "avg_launch_ms": dk["avg_ms"],
                                        "step": {"achieved": round(step_tflops, 2), "unit": "TFLOP/s",
                                                 "frac": round(step_tflops / PEAK_BF16_TFLOPS, 4),
                                                 "flop": total_flop}})
        if not args.no_extras:
            # the same prefill over packed documents (document-level mask)
            docs = I.document_ids(c4.seed, "bench_documents", B, S, 2048)
            dd = torch.from_numpy(docs).cuda()

            def prefill_docs():
                M.llama_prefill_docs(pa, dm.struct, ids, dd, B, S, kv=None, logits=logits, next_id=nid, ws=ws)

            dms = time_steps(prefill_docs, max(2, args.steps // 2), 1, torch)
            dkt = kernel_times(prefill_docs, 2, M, torch)
            lens = np.bincount(docs[0])
            out["prefill_docs"] = {"ms_per_step": round(dms, 4), "tokens_per_s": round(B * S / (dms / 1e3), 1),
                                   "documents": int(len(lens)), "mean_doc_len": round(float(lens.mean()), 1),
                                   "attn_prefill_avg_ms": round(dkt["attn_prefill"]["avg_ms"], 5),
                                   "attn_prefill_causal_avg_ms": round(kt["attn_prefill"]["avg_ms"], 5)}
            log(f"prefill, packed documents: {dms:.3f} ms/step, attention {dkt['attn_prefill']['avg_ms']:.4f} ms "
                f"(causal {kt['attn_prefill']['avg_ms']:.4f} ms), {len(lens)} documents")
            del dd
        del ws, logits, ids
        torch.cuda.empty_cache()
        if not args.no_extras:
            out["long_context"] = bench_long_layer(dm, c4, M, I, R, torch)

    if args.only in (None, "decode"):
        B, P, cap = c5.batch, c5.cache_len, c5.cache_cap
        t1 = time.time()
        log("generating and uploading the seeded KV caches (32 layers x 64 x 4096 x 8 x 128, K and V) ...")
        caches = []
        for l in range(c5.n_layers):
            pair = []
            for which in ("k", "v"):
                t = torch.zeros((B, cap, c5.n_kv_heads, c5.head_dim), dtype=torch.bfloat16, device="cuda")
                t[:, :P] = R.bits_to_device(I.kv_cache_bits(c5, l, which))
                pair.append(t)
            caches.append(tuple(pair))
        log(f"  caches ready in {time.time() - t1:.1f} s")
        kvs = M.kv_array(caches)
        da = R.args_for(c5, max_batch=B, max_seq=cap)
        ids = torch.from_numpy(I.prompt_ids(c5).reshape(-1).astype(np.int32)).cuda()
        pos = torch.full((B,), P, dtype=torch.int32, device="cuda")
        logits = torch.empty((B, c5.vocab_size), dtype=torch.float32, device="cuda")
        nid = torch.empty(B, dtype=torch.int32, device="cuda")
        ws = R.workspace(da, B, 1)

        def decode():
            M.llama_decode_step(da, dm.struct, ids, pos, B, kvs, logits=logits, next_id=nid, ws=ws)

        dsteps = max(args.steps, 10)
        ms = time_steps(decode, dsteps, args.warmup, torch)
        kt = kernel_times(decode, dsteps, M, torch)
        kern["decode"] = kt
        log(f"decode: {ms:.3f} ms/step, {B / (ms / 1e3):.0f} tokens/s")
        for k, v in sorted(kt.items(), key=lambda kv: -kv[1]["ms_per_step"]):
            log(f"  {k:22s} {v['launches']:5d} launches  {v['ms_per_step']:9.3f} ms/step  avg {v['avg_ms']:.4f} ms")
        D, Hq, Hk = c5.dim, c5.n_heads * c5.head_dim, c5.n_kv_heads * c5.head_dim
        kv_bytes = 2.0 * B * (P + 1) * Hk * 2  # K and V of positions 0..P (the new one written)
        work = {"skinny_qkv": ("hbm", 2.0 * D * (Hq + 2 * Hk)), "skinny_wo": ("hbm", 2.0 * Hq * D),
                "skinny_w1w3_swiglu": ("hbm", 2.0 * 2 * F * D), "skinny_w2": ("hbm", 2.0 * F * D),
                "attn_decode": ("hbm", kv_bytes), "lm_head": ("hbm", 2.0 * c5.vocab_size * D)}
        per_kernel = kernel_rooflines(kt, work)
        w_layer = 2.0 * (D * (Hq + 2 * Hk) + Hq * D + 3 * D * F + 2 * D)
        step_bytes = c5.n_layers * (w_layer + kv_bytes) + 2.0 * c5.vocab_size * D + 2.0 * D
        dk = per_kernel["attn_decode"]
        step_gbs = step_bytes / (ms / 1e3) / 1e9
        out["decode"] = dict(ms=ms, tok_s=B / (ms / 1e3), step_gbs=step_gbs, step_frac=step_gbs / PEAK_HBM_GBS,
                             kernels=per_kernel,
                             roofline={"kernel": "attn_decode", "bound": "hbm", "achieved": dk["achieved"],
                                       "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": dk["frac"],
                                       "traffic": measured_traffic("attn_decode"), "bytes_per_launch": kv_bytes,
                                       "avg_launch_ms": dk["avg_ms"],
                                       "step": {"achieved": round(step_gbs, 1), "unit": "GB/s",
                                                "frac": round(step_gbs / PEAK_HBM_GBS, 4), "bytes": step_bytes}})
        del caches, kvs, ws
        torch.cuda.empty_cache()

        if not args.no_extras:
            out["generate"] = bench_generate(dm, c5, M, I, R, np, torch)
            # the same loop on the small 4-layer GQA stack (launch-bound steps)
            c2 = I.CONFIGS["c2"]
            dm2 = R.DeviceModel(c2)
            out["generate_small"] = bench_generate(dm2, c2, M, I, R, np, torch, B=4, gen=64, cap=256, lmin=16,
                                                   lspan=17)
            out["generate_small"]["model"] = "dim 768, 4 layers, 8 heads / 2 KV heads, vocab 32000, bf16"
            del dm2

    configs = None
    if args.only is None and not args.no_configs:
        del dm
        torch.cuda.empty_cache()
        configs = bench_configs(M, I, R, np, torch, max(args.steps, 10))

    cpu = {}
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on bounded samples (cpu_baseline) ...")
        if "prefill" in out:
            cpu["prefill"] = cpu_baseline_prefill(c4, F)
            log(f"  prefill oracle: {cpu['prefill']['value']:.2f} tokens/s ({cpu['prefill']['seconds']:.1f} s)")
        if "decode" in out:
            cpu["decode"] = cpu_baseline_decode(c5, F)
            log(f"  decode oracle: {cpu['decode']['value']:.3f} tokens/s ({cpu['decode']['seconds']:.1f} s)")

    head = "prefill" if "prefill" in out else "decode"
    res = {
        "metric": "prefill & decode tokens/s, Llama-3-8B-shaped layers, 1 MI355X; % of roofline",
        "value": round(out[head]["tok_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(out[head]["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02^2) bf16 weights, uniform token ids, N(0,1) KV cache)",
        "config": {"workload": ("llama3-8b-shape prefill B1xS8192 (value) + decode B64 over KV 4096"
                                if len(out) == 2 else f"llama3-8b-shape {head}"),
                   "prefill": {"batch": 1, "seq_len": 8192, "layers": 32, "vocab": 128256},
                   "decode": {"batch": 64, "cache_len": 4096, "layers": 32, "vocab": 128256}},
        "roofline": {k: v for k, v in out[head]["roofline"].items()},
    }
    if head == "prefill" and "decode" in out:
        d = out["decode"]
        res["decode"] = {"value": round(d["tok_s"], 1), "unit": "tokens/s", "ms_per_step": round(d["ms"], 4),
                         "step_hbm_frac": round(d["step_frac"], 4), "roofline": d["roofline"]}
    if head == "prefill":
        res["prefill_step_tflops"] = round(out["prefill"]["step_tflops"], 1)
        res["prefill_step_mfma_frac"] = round(out["prefill"]["step_tflops"] / PEAK_BF16_TFLOPS, 4)
        res["prefill_kernels"] = out["prefill"]["kernels"]
    if "decode" in out:
        res["decode_kernels"] = out["decode"]["kernels"]
    if configs:
        res["configs"] = configs
    if cpu:
        c = cpu.get(head)
        res["cpu_baseline"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in c.items() if k != "seconds"}
        if head == "prefill" and "decode" in cpu:
            res["decode"]["cpu_baseline"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                             for k, v in cpu["decode"].items() if k != "seconds"}
    for extra in ("prefill_docs", "long_context", "generate", "generate_small"):
        if extra in out:
            res[extra] = out[extra]
    res["kernels_avg_ms"] = {w: summarize(k) for w, k in kern.items()}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
