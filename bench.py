"""Throughput of one GPU's share of the 8.3B-shape tensor-parallel layer (t = 8, rank 0) on MI355X.

One step = rank 0's pre-LN layer shard, forward + backward, over one batch of 8 x 1024 synthetic
tokens (h=3072, 32 heads of 96 -> 4 per rank, ffn=12288 -> 1536 columns per rank): LN1, QKV GEMM,
causal attention, output projection, residual, LN2, MLP GEMM1 + bias + GeLU, GEMM2, residual;
the backward with the input- and weight-gradient GEMMs, the attention backward, both LN
backwards and the bias column sums. The all-reduce results rank 0 would receive (g forward,
f backward) are computed once before timing by running all 8 ranks, then handed to rank 0's
step: no collective runs inside the timed region.

value = the layer's algorithmic FLOP / the layer step's time (TFLOP/s), FLOPs counted 2 per
multiply-add, backward = 2x forward, causal attention over the visible pairs only. The rest of
the hot path, rank 0's vocabulary shard (fused logits GEMM + cross-entropy statistics and the
loss merge over 8 ranks, vocabulary 50,257 padded to 51,200), is timed on its own and reported
in "vocab_xent". "roofline" is the layer's dominant GEMM, timed live in isolation.
Prints ONE JSON line.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

B, S, H, HEADS, FFN, TP = 8, 1024, 3072, 32, 12288, 8
VOCAB, VOCAB_PAD = 50257, 51200
PEAK_BF16 = 2.5e15        # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12         # bytes/s
COPY_PROBE_BYTES = 512 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "vocab_xent_gemm_8p3b.md")
DOMINANT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "layer_dominant_gemm_8p3b.md")
KERNEL_SOURCES = ["common.h", "gemm.h", "gemm_dispatch.h", "gemm_plan.cpp", "xent.h"]
FP8_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fp8_layer_gemms_8p3b.md")
FP8_KERNEL_SOURCES = ["common.h", "gemm.h", "gemm_fp8.hip"]


def kernel_source_hash(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "tensor_transformer_layer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(path=TRAFFIC_FILE, sources=KERNEL_SOURCES):
    """HBM bytes per launch of the roofline kernel, from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources; else None."""
    try:
        text = open(path).read()
    except OSError:
        return None
    src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash(sources):
        return None
    return float(val.group(1))


def copy_probe(torch, dev):
    """One 512 MiB device-to-device copy: the reference reading for the HBM byte counters."""
    src = torch.empty(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def layer_flops(b, s, h, heads, ffn, t):
    T = b * s
    d = h // heads
    mm = 2 * T * h * (3 * h) + 2 * T * h * h + 2 * 2 * T * h * ffn          # QKV, out-proj, MLP (unsplit)
    attn = 4 * d * (s * (s + 1) // 2) * b * heads                          # QK^T and PV, visible pairs
    return 3 * (mm + attn) / t


def xent_flops(N, h, Vt):
    return 2.0 * N * Vt * h


def stage_inputs():
    import tp_synth
    w = tp_synth.WORKLOADS["layer_8p3b_t8"]
    p = tp_synth.layer_inputs(w.seed, B, S, H, FFN, "bf16")
    wx = tp_synth.WORKLOADS["xent_8p3b_t8"]
    Vt = VOCAB_PAD // TP
    xe = {"X": tp_synth.normal(wx.seed, 0, (B * S, H), 1.0, "bf16"),
          "E0": tp_synth.normal(wx.seed, 14, (Vt, H), 0.02, "bf16"),
          "targets": tp_synth.targets(wx.seed, 15, B * S, VOCAB)}
    return p, xe


def cpu_baseline(p, xe, seqs=8, heads=HEADS):
    """The float64 oracle on rank 0's layer step for `seqs` sequences (the same step, fewer tokens)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    T = seqs * S
    ht, Ft, Vt = H // TP, FFN // TP, VOCAB_PAD // TP
    x, G = p["x"][:T], p["G"][:T]
    Wqkv_r = oracle.qkv_shard(p["Wqkv"], heads, TP, 0)
    bq = oracle.qkv_shard(p["bqkv"], heads, TP, 0)
    Wo_r = oracle.wo_shard(p["Wo"], heads, TP, 0)
    A_r, b1_r, B_r = p["A"][:, :Ft], p["b1"][:Ft], p["B"][:Ft]

    def run():
        _oracle_step(oracle, p, xe, x, G, Wqkv_r, bq, Wo_r, A_r, b1_r, B_r, seqs, heads)

    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    flops = layer_flops(seqs, S, H, heads, FFN, TP)
    try:
        cores = len(os.sched_getaffinity(0))
    except Exception:
        cores = os.cpu_count()
    blas = "unknown BLAS"
    try:
        from threadpoolctl import threadpool_info
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('num_threads')} threads" for i in threadpool_info()}))
    except Exception:
        pass
    return {"value": round(flops / dt / 1e12, 4), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"rank 0's layer step (fwd+bwd) on {seqs} of {B} sequences "
                      f"({T} tokens), float64 NumPy, median of 3 runs ({', '.join(f'{t:.1f}' for t in times)} s); "
                      f"{cores} cores in the affinity mask, {blas}"}


def _oracle_step(oracle, p, xe, x, G, Wqkv_r, bq, Wo_r, A_r, b1_r, B_r, seqs, heads):
    T = seqs * S
    l1 = oracle.layernorm_fwd(x, p["ln1_g"], p["ln1_b"])
    fa = oracle.attn_shard_fwd(l1["y"], Wqkv_r, bq, Wo_r, seqs, S, heads // TP)
    x1 = x + fa["Z"] + p["bo"]                 # rank 0's partial stands in for the all-reduced sum
    l2 = oracle.layernorm_fwd(x1, p["ln2_g"], p["ln2_b"])
    fm = oracle.mlp_shard_fwd(l2["y"], A_r, b1_r, B_r)
    gm = oracle.mlp_shard_bwd(l2["y"], A_r, B_r, fm["U"], fm["Y"], G)
    b2 = oracle.layernorm_bwd(x1, p["ln2_g"], l2["mean"], l2["rstd"], gm["dX"])
    dx1 = G + b2["dx"]
    ga = oracle.attn_shard_bwd(l1["y"], Wqkv_r, Wo_r, fa, dx1, seqs, S, heads // TP)
    oracle.layernorm_bwd(x, p["ln1_g"], l1["mean"], l1["rstd"], ga["dXn"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the shader-clock sample (about 1.5 s of extra steps; for profiler runs)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="copy 512 MiB device-to-device once before the steps (calibrates HBM byte counters)")
    ap.add_argument("--vocab-bwd", action="store_true",
                    help="time the vocabulary-parallel cross-entropy backward of rank 0 instead (logits gradient "
                         "+ dX_r + dE_r GEMMs: 3 x 322 GFLOP per call) and print its own JSON line")
    ap.add_argument("--fp8", action="store_true",
                    help="time rank 0's twelve layer GEMMs (forward, input and weight gradients) in fp8 E4M3 with "
                         "per-tensor scales, each operand quantised in the step, and print their own JSON line")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="dropout probability of every site (residual sites after g with shared streams, "
                         "attention with per-rank streams); the pages train with 0.1")
    ap.add_argument("--recompute", action="store_true",
                    help="activation recompute: the step runs the layer forward again before its backward "
                         "(the recomputed forward's FLOPs are not counted)")
    ap.add_argument("--embedding", action="store_true",
                    help="add rank 0's vocabulary-parallel input-embedding lookup and its backward to the step")
    ap.add_argument("--graph", action="store_true",
                    help="capture the step into a HIP graph and time its replays (prints its own JSON line)")
    ap.add_argument("--config", type=int, default=4, choices=[1, 2, 3, 4, 5],
                    help="workload: 4 = the 8.3B layer shard (the metric, default); 1 = the fp32 MLP block (t=2), "
                         "2 = the 1.2B attention shard (t=2), 3 = the 2.5B layer shard (t=4), 5 = the 8.3B "
                         "vocabulary-parallel cross-entropy shard (t=8): rank 0's share, timed, with the worst "
                         "element-wise error against the float64 oracle and the oracle's time in cpu_baseline")
    ap.add_argument("--heads", type=int, default=HEADS,
                    help="attention heads of the layer (the pages' 8.3B head-count sweep uses 16, 24, 32; the "
                         "FLOPs and all other shapes are unchanged, heads per rank = heads / 8)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the layer; --gpus {args.gpus} is not supported "
              "(the library computes one rank's share; the multi-GPU all-reduces are not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch
    import tensor_transformer_layer_amd as tp
    from tensor_transformer_layer_amd.layer import LayerShard, rank_params

    if args.fp8:
        return bench_fp8(args, tp, torch)
    if args.config != 4:
        return bench_config(args, tp, torch)
    dev = "cuda:0"
    T = B * S
    Vt = VOCAB_PAD // TP
    p, xe = stage_inputs()

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(dev)

    x, G = d(p["x"]), d(p["G"])
    # verification run over all ranks: the sums rank 0 would receive
    heads = args.heads
    if heads % TP or H % heads:
        print(f"--heads {heads}: must be a multiple of t={TP} and divide h={H}", file=sys.stderr)
        sys.exit(2)
    if not 0.0 <= args.dropout < 1.0:
        print("--dropout must be in [0, 1)", file=sys.stderr)
        sys.exit(2)

    def rank_drop(r):
        if args.dropout == 0.0:
            return None
        return {"p": args.dropout, "seed": 20191004, "resid_streams": (0, 1), "attn_stream": 1000 + r}
    shards = [LayerShard(B, S, H, heads, FFN, TP, r, rank_params(p, heads, TP, r, dev), dev, rank_drop(r))
              for r in range(TP)]
    attn_sum = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    mlp_sum, dxn2_sum, dxn1_sum = (torch.empty_like(attn_sum) for _ in range(3))
    shards[0].combine([sh.attn_fwd(x) for sh in shards], None, None, attn_sum)
    x1 = torch.empty_like(attn_sum)
    shards[0].combine([attn_sum], shards[0].p["bo"], x, x1, shards[0].d_res1)
    shards[0].combine([sh.mlp_fwd(x1) for sh in shards], None, None, mlp_sum)
    shards[0].combine([sh.mlp_bwd(G) for sh in shards], None, None, dxn2_sum)
    dx1 = shards[0].ln2_bwd(dxn2_sum, G)
    shards[0].combine([sh.attn_bwd(dx1) for sh in shards], None, None, dxn1_sum)
    torch.cuda.synchronize()
    rank0 = shards[0]
    del shards
    torch.cuda.empty_cache()

    # rank 0's vocabulary shard; the other ranks' loss statistics are pre-staged (their values only
    # feed the merge, which reads t per-token triples)
    Xv, E0 = d(xe["X"]), d(xe["E0"])
    tg = torch.from_numpy(xe["targets"]).to(dev)
    mx, se, tv = (torch.empty(T, dtype=torch.float32, device=dev) for _ in range(3))
    am = torch.empty(T, dtype=torch.int32, device=dev)
    xws_bytes = tp.tp_vocab_xent_shard_fwd_workspace(T, H, VOCAB_PAD, TP, tp.TP_BF16)
    xws = torch.empty(xws_bytes, dtype=torch.uint8, device=dev)
    peers = [(mx, se, tv)] + [tuple(torch.empty(T, dtype=torch.float32, device=dev) for _ in range(3))
                              for _ in range(TP - 1)]
    tp.tp_vocab_xent_shard_fwd(T, H, VOCAB_PAD, VOCAB, TP, 0, tp.TP_BF16, 0, Xv, E0, tg, mx, se, tv, am, xws, xws_bytes)
    for q in peers[1:]:
        for a, b_ in zip(q, (mx, se, tv)):
            a.copy_(b_)
    loss = torch.empty(T, dtype=torch.float32, device=dev)
    mean = torch.empty(1, dtype=torch.float32, device=dev)
    # input embedding of rank 0 (the tied table's shard E0): lookup partial and its backward
    emb_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    dE0 = torch.empty((Vt, H), dtype=torch.bfloat16, device=dev)
    emb_ws_bytes = tp.tp_embedding_shard_bwd_workspace(T, VOCAB_PAD, TP)
    emb_ws = torch.empty(max(emb_ws_bytes, 256), dtype=torch.uint8, device=dev)

    stream = torch.cuda.current_stream()
    if args.vocab_bwd:
        return bench_vocab_bwd(args, tp, torch, T, Vt, Xv, E0, tg, peers, stream)
    if args.copy_probe:
        copy_probe(torch, dev)

    def layer_step():
        if args.embedding:
            tp.tp_embedding_shard_fwd(T, H, VOCAB_PAD, TP, 0, tp.TP_BF16, tg, E0, emb_out)
        rank0.step(x, G, attn_sum, mlp_sum, dxn2_sum, dxn1_sum, recompute=args.recompute)
        if args.embedding:
            tp.tp_embedding_shard_bwd(T, H, VOCAB_PAD, TP, 0, tp.TP_BF16, tg, rank0.dx, dE0, 0, emb_ws, emb_ws_bytes)

    def vocab_step():
        tp.tp_vocab_xent_shard_fwd(T, H, VOCAB_PAD, VOCAB, TP, 0, tp.TP_BF16, 0, Xv, E0, tg, mx, se, tv, am, xws,
                                   xws_bytes)
        tp.tp_vocab_xent_combine(T, TP, [q[0] for q in peers], [q[1] for q in peers], [q[2] for q in peers], loss, mean)

    def step():
        layer_step()
        vocab_step()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.graph:
        return bench_graph(args, torch, step, heads, stream)

    def timed(fn, n):
        """Mean time of fn() over n back-to-back calls, one pair of HIP events around all of them."""
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b_.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b_) / n

    # the timed region: K layer steps with no events inside (each record leaves a gap in the stream)
    ms = timed(layer_step, args.steps)
    # the rest of the hot path, timed on its own: the vocabulary shard's fused logits GEMM + CE
    # statistics and the loss merge
    xent_ms = timed(vocab_step, args.steps)
    # the unfused form of the vocabulary statistics: a pass over rank 0's materialised fp32 logits
    # (written once here, 210 MB), timed on its own (HBM-bound)
    logits = torch.empty((T, Vt), dtype=torch.float32, device=dev)
    tp.tp_vocab_logits_shard(T, H, VOCAB_PAD, TP, 0, tp.TP_BF16, Xv, E0, logits)
    ux = tuple(torch.empty(T, dtype=torch.float32, device=dev) for _ in range(3))
    uam = torch.empty(T, dtype=torch.int32, device=dev)

    def stats_pass():
        tp.tp_vocab_xent_stats_from_logits(T, VOCAB_PAD, VOCAB, TP, 0, 0, logits, Vt, tg, *ux, uam)

    stats_pass()
    pass_us = timed(stats_pass, args.steps) * 1e3
    pass_bytes = T * Vt * 4 + T * 16
    del logits
    torch.cuda.empty_cache()
    # per-step spread: a second pass of as many layer steps, each bracketed by its own events
    per_step = []
    for _ in range(args.steps):
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        layer_step()
        b_.record(stream)
        per_step.append((a, b_))
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(b_) for a, b_ in per_step])
    clock = None if args.no_clock else sample_sclk(
        lambda: [layer_step() for _ in range(max(1, int(1500 / max(ms, 1e-3))))], torch)
    roof = dominant_gemm_roofline(args, tp, torch, rank0, G, stream)

    fl_layer = layer_flops(B, S, H, heads, FFN, TP)
    fl_xent = xent_flops(T, H, Vt)
    value = fl_layer / (ms * 1e-3) / 1e12
    xent_tf = fl_xent / (xent_ms * 1e-3) / 1e12
    peak_info = rocminfo_peak()
    out = {
        "metric": "layer-shard TFLOP/s fwd+bwd (% bf16 MFMA peak), 8.3B shape t=8, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations and gradients, N(0,0.02^2) weights, uniform targets)",
        "config": {"workload": f"8.3B-shape layer shard, tp=8, rank 0, forward + backward: {B} x {S} tokens, "
                               f"hidden {H}, {heads} heads of {H // heads} ({heads // TP} per rank), ffn {FFN} "
                               f"({FFN // TP} columns per rank)"
                               + (" + input-embedding lookup fwd+bwd" if args.embedding else "")
                               + (f", dropout {args.dropout}" if args.dropout else "")
                               + (", activation recompute" if args.recompute else ""),
                   "batch": B, "seq_len": S, "hidden": H, "heads": heads, "ffn": FFN, "tp": TP,
                   "parallelism": "one rank of tp8 (all-reduce results pre-staged)",
                   "dropout": args.dropout, "recompute": args.recompute, "embedding": args.embedding},
        "pct_bf16_peak": round(100 * value * 1e12 / PEAK_BF16, 2),
        "layer_gflop": round(fl_layer / 1e9, 2),
        "step_ms_p10_p50_p90": [round(float(np.percentile(per_step, q)), 4) for q in (10, 50, 90)],
        "vocab_xent": {"what": "rank 0's vocabulary shard (6400 of 51,200 rows): fused logits GEMM + per-token "
                               "max / sum-exp / target / argmax, then the loss merge over 8 ranks; timed on its own",
                       "ms": round(xent_ms, 4), "gflop": round(fl_xent / 1e9, 2), "tflops": round(xent_tf, 2),
                       "frac": round(xent_tf * 1e12 / PEAK_BF16, 4),
                       "traffic": measured_traffic(),
                       "traffic_unit": "HBM bytes per call of the fused GEMM (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                       "copy-calibrated), from the committed counter summary; null once stale",
                       "unfused_stats_pass": {
                           "what": "the same per-token statistics from the materialised fp32 logits [8192 x 6400] "
                                   "(tp_vocab_xent_stats_from_logits): one HBM pass, the form the fusion avoids",
                           "us": round(pass_us, 2), "bytes": pass_bytes,
                           "GB_per_s": round(pass_bytes / (pass_us * 1e-6) / 1e9, 1),
                           "frac_of_8TB_per_s": round(pass_bytes / (pass_us * 1e-6) / PEAK_HBM, 4)}},
        "hot_path_ms": round(ms + xent_ms, 4),
        "roofline": roof,
        "clock": {"sclk_mhz_under_load": clock, "rocminfo": peak_info},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, xe, heads=heads)
    print(json.dumps(out), flush=True)


def rocminfo_peak():
    """Compute units and maximum engine clock of the gfx950 agent as rocminfo reports them, and
    the dense bf16 MFMA peak they imply (4096 FLOP per clock per CU)."""
    import subprocess
    try:
        text = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except Exception:
        return None
    for agent in text.split("Agent ")[1:]:
        if "gfx950" not in agent:
            continue
        cu = re.search(r"Compute Unit:\s*(\d+)", agent)
        mhz = re.search(r"Max Clock Freq\. \(MHz\):\s*(\d+)", agent)
        if cu and mhz:
            cus, f = int(cu.group(1)), int(mhz.group(1))
            return {"compute_units": cus, "max_clock_mhz": f,
                    "bf16_dense_peak_tflops": round(cus * f * 1e6 * 4096 / 1e12, 1)}
    return None


def sample_sclk(run, torch):
    """Median shader clock (MHz) that rocm-smi reports while run() keeps the GPU busy with layer
    steps for about a second and a half; None if the tool is unavailable."""
    import subprocess
    import threading
    vals, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
                m = re.search(r"sclk clock level:\s*\d+:?\s*\((\d+)Mhz\)", r.stdout)
                if m:
                    vals.append(int(m.group(1)))
            except Exception:
                return

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    run()
    torch.cuda.synchronize()
    stop.set()
    th.join(timeout=30)
    return int(np.median(vals)) if vals else None


# The layer's dominant GEMM, the weight gradient dB_r = Y_r^T G of the MLP (1536 x 3072 x 8192,
# both operands MN-contiguous): name, M, N, K, flops.
DOMINANT = ("MLP weight gradient dB_r = Y_r^T G (gemm_bf16_kernel 256x256 TN, 3 K splits, + split-K reduction)",
            FFN // TP, H, B * S)


def dominant_gemm_roofline(args, tp, torch, rank0, G, stream):
    """Average launch time of the layer's dominant GEMM, measured live: the same call the step
    makes (same shape, plan, operands and stream) through tp_gemm_bf16, K calls back to back
    between one pair of HIP events (per-call events leave gaps in the stream). Its operands (Y_r
    and G, 75 MB) then sit in the 256 MB MALL as they largely do inside the step, where the call
    takes about as long."""
    name, M, N, K = DOMINANT
    nb = tp.tp_gemm_bf16_workspace(M, N, K)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda:0")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")

    def call():
        tp.tp_gemm_bf16(M, N, K, rank0.Y, M, 1, G, N, 1, tp.TP_EPI_STORE, out, None, N, None, None, 0, ws, nb)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        call()
    b_.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b_) / args.steps * 1e3
    fl = 2.0 * M * N * K
    ach = fl / (us * 1e-6) / 1e12
    return {"bound": "mfma", "kernel": name, "M_N_K": [M, N, K], "gflop_per_launch": round(fl / 1e9, 2),
            "avg_launch_us": round(us, 2), "achieved": round(ach, 2), "peak": PEAK_BF16 / 1e12,
            "unit": "TFLOP/s", "frac": round(ach * 1e12 / PEAK_BF16, 4),
            "traffic": measured_traffic(DOMINANT_TRAFFIC_FILE, KERNEL_SOURCES),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated), from the "
                            "committed counter summary; null once the kernel sources have changed"}


def _timed_calls(torch, fn, warmup, steps):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    a.record(stream)
    for _ in range(steps):
        fn()
    b_.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b_) / steps


def _cores():
    try:
        return len(os.sched_getaffinity(0))
    except Exception:
        return os.cpu_count()


def _worst(pairs):
    """Largest of (relative L2, max|err|/max|ref|) over the named (got, ref) pairs: (name, value)."""
    worst = ("", 0.0)
    for name, got, ref in pairs:
        got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
        d = got - ref
        e = max(float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)),
                float(np.abs(d).max() / max(np.abs(ref).max(), 1e-300)))
        if e > worst[1]:
            worst = (name, e)
    return {"output": worst[0], "value": float(f"{worst[1]:.3g}")}


def bench_config(args, tp, torch):
    """Rank 0's share of one of the other workloads, timed like the default step (warm-up, then
    HIP events around K back-to-back calls), reported on its own JSON line. The oracle leg (unless
    --no-cpu-baseline) times the float64 oracle on the same work on the host cores and reports the
    worst element-wise error of the timed call's outputs against it."""
    import tp_synth
    dev = "cuda:0"

    def d(a, dt=torch.bfloat16):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)

    n = args.config
    t0 = time.perf_counter
    out = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "data": "synthetic (seeded, the workload's distributions)"}
    if n == 1:
        w = tp_synth.WORKLOADS["mlp_fp32_t2"]
        inp = tp_synth.mlp_inputs(w.seed, w.T, w.h, w.ffn, "f32")
        T, h, ffn, t = w.T, w.h, w.ffn, w.t
        Ft = ffn // t
        f32 = torch.float32
        X, G = d(inp["X"], f32), d(inp["G"], f32)
        A0, b0, B0 = d(inp["A"][:, :Ft], f32), d(inp["b1"][:Ft], f32), d(inp["B"][:Ft], f32)
        U, Y, Z = (torch.empty((T, n_), dtype=f32, device=dev) for n_ in (Ft, Ft, h))
        dX, dA, db1, dB = (torch.empty(sh, dtype=f32, device=dev) for sh in ((T, h), (h, Ft), (Ft,), (Ft, h)))
        nb = tp.tp_mlp_shard_bwd_workspace(T, h, ffn, t, tp.TP_F32)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)

        def call():
            tp.tp_mlp_shard_fwd(T, h, ffn, t, 0, tp.TP_F32, X, A0, b0, B0, U, Y, Z)
            tp.tp_mlp_shard_bwd(T, h, ffn, t, 0, tp.TP_F32, X, A0, B0, U, Y, G, dX, dA, db1, dB, 0, ws, nb)

        fl = 3 * 2.0 * 2 * T * h * Ft
        dtype, name = "f32", "MLP block shard (fp32), T=128, h=256, ffn=1024, t=2, rank 0, fwd+bwd"

        def oracle_run():
            import oracle
            f = oracle.mlp_shard_fwd(inp["X"], inp["A"][:, :Ft], inp["b1"][:Ft], inp["B"][:Ft])
            g = oracle.mlp_shard_bwd(inp["X"], inp["A"][:, :Ft], inp["B"][:Ft], f["U"], f["Y"], inp["G"])
            return [("U", U, f["U"]), ("Y", Y, f["Y"]), ("Z_0", Z, f["Z"]), ("dX_0", dX, g["dX"]),
                    ("dA_0", dA, g["dA"]), ("db1_0", db1, g["db1"]), ("dB_0", dB, g["dB"])]
    elif n == 2:
        w = tp_synth.WORKLOADS["attn_1p2b_t2"]
        inp = tp_synth.attn_inputs(w.seed, w.b, w.s, w.h, "bf16")
        b, s, h, heads, t = w.b, w.s, w.h, w.heads, w.t
        T, ht = b * s, h // t
        Xn, G = d(inp["Xn"]), d(inp["G"])
        # rank 0's [Wq | Wk | Wv] columns of its heads and its rows of Wo
        qcols = np.concatenate([np.arange(i * h, i * h + ht) for i in range(3)])
        Wq, bq, Wo = d(inp["Wqkv"][:, qcols]), d(inp["bqkv"][qcols]), d(inp["Wo"][:ht])
        QKV, O, Z = (torch.empty(sh, dtype=torch.bfloat16, device=dev) for sh in ((T, 3 * ht), (T, ht), (T, h)))
        lse = torch.empty((b, heads // t, s), dtype=torch.float32, device=dev)
        dXn, dWqkv, dbqkv, dWo = (torch.empty(sh, dtype=torch.bfloat16, device=dev)
                                  for sh in ((T, h), (h, 3 * ht), (3 * ht,), (ht, h)))
        nb = tp.tp_attn_shard_bwd_workspace(b, s, h, heads, t, tp.TP_BF16)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)

        def call():
            tp.tp_attn_shard_fwd(b, s, h, heads, t, 0, tp.TP_BF16, 1, Xn, Wq, bq, Wo, QKV, O, lse, Z)
            tp.tp_attn_shard_bwd(b, s, h, heads, t, 0, tp.TP_BF16, 1, Xn, Wq, Wo, QKV, O, lse, G, dXn, dWqkv, dbqkv,
                                 dWo, 0, ws, nb)

        d_ = h // heads
        fl = 3 * (2.0 * T * h * 3 * ht + 2.0 * T * ht * h + 4.0 * d_ * (s * (s + 1) // 2) * b * (heads // t))
        dtype, name = "bf16", "1.2B-shape attention shard, t=2, rank 0, fwd+bwd (8 x 1024 tokens, 8 heads of 96)"

        def oracle_run():
            import oracle
            Wq_, bq_, Wo_ = (oracle.qkv_shard(inp["Wqkv"], heads, t, 0), oracle.qkv_shard(inp["bqkv"], heads, t, 0),
                             oracle.wo_shard(inp["Wo"], heads, t, 0))
            f = oracle.attn_shard_fwd(inp["Xn"], Wq_, bq_, Wo_, b, s, heads // t)
            g = oracle.attn_shard_bwd(inp["Xn"], Wq_, Wo_, f, inp["G"], b, s, heads // t)
            return [("QKV", QKV, f["QKV"]), ("O", O, f["O"]), ("lse", lse, f["lse"]), ("Z_0", Z, f["Z"]),
                    ("dXn_0", dXn, g["dXn"]), ("dWqkv_0", dWqkv, g["dWqkv"]), ("dbqkv_0", dbqkv, g["dbqkv"]),
                    ("dWo_0", dWo, g["dWo"])]
    elif n == 3:
        from tensor_transformer_layer_amd.layer import LayerShard, rank_params
        w = tp_synth.WORKLOADS["layer_2p5b_t4"]
        p = tp_synth.layer_inputs(w.seed, w.b, w.s, w.h, w.ffn, "bf16")
        b, s, h, heads, ffn, t = w.b, w.s, w.h, w.heads, w.ffn, w.t
        T = b * s
        x, G = d(p["x"]), d(p["G"])
        shards = [LayerShard(b, s, h, heads, ffn, t, r, rank_params(p, heads, t, r, dev), dev) for r in range(t)]
        sums = [torch.empty((T, h), dtype=torch.bfloat16, device=dev) for _ in range(4)]
        attn_sum, mlp_sum, dxn2_sum, dxn1_sum = sums
        sh0 = shards[0]
        sh0.combine([sh.attn_fwd(x) for sh in shards], None, None, attn_sum)
        x1 = torch.empty_like(attn_sum)
        sh0.combine([attn_sum], sh0.p["bo"], x, x1)
        sh0.combine([sh.mlp_fwd(x1) for sh in shards], None, None, mlp_sum)
        sh0.combine([sh.mlp_bwd(G) for sh in shards], None, None, dxn2_sum)
        dx1 = sh0.ln2_bwd(dxn2_sum, G)
        sh0.combine([sh.attn_bwd(dx1) for sh in shards], None, None, dxn1_sum)
        torch.cuda.synchronize()
        del shards
        torch.cuda.empty_cache()

        def call():
            sh0.step(x, G, attn_sum, mlp_sum, dxn2_sum, dxn1_sum)

        fl = layer_flops(b, s, h, heads, ffn, t)
        fl_oracle = t * fl   # the oracle leg runs the whole split layer (every rank) to check rank 0's outputs
        dtype, name = "bf16", "2.5B-shape layer shard, t=4, rank 0, fwd+bwd (8 x 1024 tokens, 5 heads of 96, 1920 MLP columns)"

        def oracle_run():
            import oracle
            f = oracle.layer_split_fwd(p["x"], p, b, s, heads, t)
            gr = oracle.layer_split_bwd(p["x"], p, f, p["G"], b, s, heads, t)
            ht, Ft = h // t, ffn // t
            qcols = np.concatenate([np.arange(i * h, i * h + ht) for i in range(3)])
            return [("x2", sh0.x2, f["x2"]), ("dx", sh0.dx, gr["dx"]), ("dA_0", sh0.dA, gr["mlp"]["dA"][:, :Ft]),
                    ("dB_0", sh0.dB, gr["mlp"]["dB"][:Ft]), ("db1_0", sh0.db1, gr["mlp"]["db1"][:Ft]),
                    ("dWqkv_0", sh0.dWqkv, gr["attn"]["dWqkv"][:, qcols]), ("dWo_0", sh0.dWo, gr["attn"]["dWo"][:ht]),
                    ("dln1_g", sh0.dln1_g, gr["dln1_g"]), ("dln2_g", sh0.dln2_g, gr["dln2_g"])]
    else:
        w = tp_synth.WORKLOADS["xent_8p3b_t8"]
        inp = tp_synth.xent_inputs(w.seed, w.T, w.h, w.vocab, w.vocab_pad, "bf16")
        N, h, Vpad, Vreal, t = w.T, w.h, w.vocab_pad, w.vocab, w.t
        Vt = Vpad // t
        X, E0 = d(inp["X"]), d(inp["E"][:Vt])
        tg = torch.from_numpy(inp["targets"]).to(dev)
        mx, se, tv = (torch.empty(N, dtype=torch.float32, device=dev) for _ in range(3))
        am = torch.empty(N, dtype=torch.int32, device=dev)
        nb = tp.tp_vocab_xent_shard_fwd_workspace(N, h, Vpad, t, tp.TP_BF16)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)

        def call():
            tp.tp_vocab_xent_shard_fwd(N, h, Vpad, Vreal, t, 0, tp.TP_BF16, 0, X, E0, tg, mx, se, tv, am, ws, nb)

        fl = xent_flops(N, h, Vt)
        dtype, name = "bf16", "8.3B vocabulary shard, t=8, rank 0: fused logits GEMM + per-token max/sum-exp/target/argmax (N=8192, h=3072, V_t=6400)"

        def oracle_run():
            import oracle
            st = oracle.xent_shard_stats(inp["X"], inp["E"][:Vt], inp["targets"], t, 0, Vreal)
            return [("max", mx, st["max"]), ("sumexp", se, st["sumexp"]), ("tgt", tv, st["tgt"])]
    fl_oracle = locals().get("fl_oracle", fl)
    ms = _timed_calls(torch, call, args.warmup, args.steps)
    value = fl / (ms * 1e-3) / 1e12
    peak = PEAK_BF16 if dtype == "bf16" else 157.3e12
    out.update({"metric": f"config {n} shard TFLOP/s, 1 GPU", "value": round(value, 3), "unit": "TFLOP/s",
                "ms_per_step": round(ms, 4), "dtype": dtype, "config": {"workload": name},
                "gflop": round(fl / 1e9, 3), "pct_peak": round(100 * value * 1e12 / peak, 2),
                "peak_tflops": peak / 1e12})
    if not args.no_cpu_baseline:
        call()
        torch.cuda.synchronize()
        times = []
        for _ in range(3):
            a = t0()
            pairs = oracle_run()
            times.append(t0() - a)
        dt = float(np.median(times))
        out["worst_error_vs_oracle"] = _worst([(k, g.detach().float().cpu().numpy(), r) for k, g, r in pairs])
        what = ("the whole t-way split layer (every rank's work, to check rank 0's outputs)" if fl_oracle != fl
                else "the same rank-0 work")
        out["cpu_baseline"] = {"value": round(fl_oracle / dt / 1e12, 4), "unit": "TFLOP/s", "cores": int(_cores()),
                               "kind": "oracle", "sample": f"{what} in float64 NumPy, median of 3 runs "
                                                           f"({', '.join(f'{x:.2f}' for x in times)} s)"}
    print(json.dumps(out), flush=True)


def bench_graph(args, torch, step, heads, stream):
    """The whole hot path (layer step + vocabulary shard) captured once into a HIP graph (every
    call is a kernel launch on the captured stream) and replayed; each replay is bracketed by
    events outside the graph."""
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    ev = []
    for _ in range(args.steps):
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        graph.replay()
        b_.record(stream)
        ev.append((a, b_))
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b_) for a, b_ in ev])
    ms = float(per.mean())
    fl = layer_flops(B, S, H, heads, FFN, TP) + xent_flops(B * S, H, VOCAB_PAD // TP)
    value = fl / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "hot-path TFLOP/s (layer shard fwd+bwd + vocabulary shard xent), 8.3B shape t=8, 1 GPU, "
                  "HIP graph replay",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights, uniform targets)",
        "config": {"workload": "layer shard fwd+bwd + vocab-parallel xent shard, one graph per step",
                   "dropout": args.dropout, "recompute": args.recompute, "embedding": args.embedding},
        "pct_bf16_peak": round(100 * value * 1e12 / PEAK_BF16, 2),
        "step_ms_p10_p50_p90": [round(float(np.percentile(per, q)), 4) for q in (10, 50, 90)]}), flush=True)


def bench_vocab_bwd(args, tp, torch, T, Vt, Xv, E0, tg, peers, stream):
    """Rank 0's cross-entropy backward with the merged statistics of the (pre-staged) forward."""
    dev = "cuda:0"
    f32 = dict(dtype=torch.float32, device=dev)
    loss, M, S = torch.empty(T, **f32), torch.empty(T, **f32), torch.empty(T, **f32)
    tp.tp_vocab_xent_combine(T, TP, [q[0] for q in peers], [q[1] for q in peers], [q[2] for q in peers], loss, None,
                             M, S)
    g = torch.full((T,), 1.0 / T, **f32)
    dX = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    dE = torch.empty((Vt, H), dtype=torch.bfloat16, device=dev)
    nb = tp.tp_vocab_xent_shard_bwd_workspace(T, H, VOCAB_PAD, TP, tp.TP_BF16)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)

    def call():
        tp.tp_vocab_xent_shard_bwd(T, H, VOCAB_PAD, VOCAB, TP, 0, tp.TP_BF16, 0, Xv, E0, tg, M, S, g, dX, dE, 0, ws, nb)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    fl = 3 * xent_flops(T, H, Vt)
    value = fl / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "vocab-parallel cross-entropy backward TFLOP/s, 8.3B vocabulary shard t=8, 1 GPU",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) embedding, uniform targets)",
        "config": {"workload": "rank 0 vocab shard backward: logits gradient + dX_r + dE_r", "tokens": T,
                   "hidden": H, "vocab_padded": VOCAB_PAD, "tp": TP},
        "pct_bf16_peak": round(100 * value * 1e12 / PEAK_BF16, 2)}), flush=True)


# The twelve GEMMs of rank 0's layer step (8192 tokens, h = 3072, h/t = 384, 3h/t = 1152, ffn/t = 1536):
# (name, M, N, K, A operand, B operand, epilogue). An operand "X" is X's codes in row layout (K
# along X's rows' length), "X^T" its transposed codes (K along X's rows), as tp_gemm_fp8 takes them.
FP8_GEMMS = [
    ("qkv_fwd", 8192, 1152, 3072, "Xn", "Wqkv^T", "bias"),
    ("proj_fwd", 8192, 3072, 384, "O", "Wo^T", "store"),
    ("mlp1_fwd", 8192, 1536, 3072, "Y", "A^T", "bias_gelu"),
    ("mlp2_fwd", 8192, 3072, 1536, "Z", "B^T", "store"),
    ("dZ_dgelu", 8192, 1536, 3072, "G", "B", "dgelu"),
    ("dB_wgrad", 1536, 3072, 8192, "Z^T", "G^T", "store"),
    ("dY_dgrad", 8192, 3072, 1536, "dU", "A", "store"),
    ("dA_wgrad", 3072, 1536, 8192, "Y^T", "dU^T", "store"),
    ("dO_dgrad", 8192, 384, 3072, "G2", "Wo", "store"),
    ("dWo_wgrad", 384, 3072, 8192, "O^T", "G2^T", "store"),
    ("dXn_dgrad", 8192, 3072, 1152, "dQKV", "Wqkv", "store"),
    ("dWqkv_wgrad", 3072, 1152, 8192, "Xn^T", "dQKV^T", "store"),
]
# bf16 tensors quantised each step: (name, rows, cols, std); weights are stored [in, out] as in the layer
FP8_TENSORS = [("Xn", 8192, 3072, 1.0), ("O", 8192, 384, 1.0), ("Y", 8192, 3072, 1.0), ("Z", 8192, 1536, 1.0),
               ("G", 8192, 3072, 1e-3), ("dU", 8192, 1536, 1e-3), ("G2", 8192, 3072, 1e-3),
               ("dQKV", 8192, 1152, 1e-3), ("Wqkv", 3072, 1152, 0.02), ("Wo", 384, 3072, 0.02),
               ("A", 3072, 1536, 0.02), ("B", 1536, 3072, 0.02)]
PEAK_FP8 = 5.0e15   # MI355X dense fp8 MFMA, FLOP/s


def bench_fp8(args, tp, torch):
    """fp8 E4M3 GEMMs of rank 0's layer step, with the per-tensor quantisation of every operand
    (amax, power-of-two scale, row and transposed codes) inside the step. The weights are
    quantised in every step too, as they change after every optimizer step."""
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    T = B * S
    src, codes, codes_t, desc = {}, {}, {}, {}
    for i, (name, rows, cols, std) in enumerate(FP8_TENSORS):
        g = np.random.default_rng([9100, i])
        src[name] = torch.from_numpy((g.standard_normal((rows, cols)) * std).astype(np.float32)).to(
            torch.bfloat16).to(dev)
        codes[name] = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        codes_t[name] = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
        desc[name] = torch.empty(4, dtype=torch.float32, device=dev)
    qws = torch.empty(max(tp.tp_fp8_quantize_workspace(T, H), 256), dtype=torch.uint8, device=dev)
    bias = {n: torch.full((N,), 0.01, dtype=torch.bfloat16, device=dev) for n, M, N, K, a, b_, e in FP8_GEMMS
            if e in ("bias", "bias_gelu")}
    U = torch.randn((T, FFN // TP), device=dev).to(torch.bfloat16)   # saved pre-activation for dGeLU
    outs = {n: torch.empty((M, N), dtype=torch.bfloat16, device=dev) for n, M, N, K, a, b_, e in FP8_GEMMS}
    out2 = torch.empty((T, FFN // TP), dtype=torch.bfloat16, device=dev)
    gws_bytes = max(tp.tp_gemm_fp8_workspace(M, N, K) for n, M, N, K, a, b_, e in FP8_GEMMS)
    gws = torch.empty(max(gws_bytes, 256), dtype=torch.uint8, device=dev)

    def operand(ref):
        if ref.endswith("^T"):
            return codes_t[ref[:-2]], desc[ref[:-2]]
        return codes[ref], desc[ref]

    def quantize_all():
        for name, rows, cols, std in FP8_TENSORS:
            tp.tp_fp8_quantize(rows, cols, tp.TP_BF16, src[name], cols, codes[name], cols, codes_t[name], rows, None,
                               desc[name], qws, qws.numel())

    def gemm_call(name, M, N, K, a, b_, e):
        (ca, da), (cb, db) = operand(a), operand(b_)
        epi = {"store": tp.TP_EPI_STORE, "bias": tp.TP_EPI_STORE, "bias_gelu": tp.TP_EPI_BIAS_GELU,
               "dgelu": tp.TP_EPI_DGELU}[e]
        return lambda: tp.tp_gemm_fp8(M, N, K, ca, K, da, cb, K, db, epi, outs[name],
                                      out2 if e == "bias_gelu" else None, N, bias.get(name),
                                      U if e == "dgelu" else None, 0, gws, gws.numel())

    gemms = [(g[0], gemm_call(*g)) for g in FP8_GEMMS]

    def step():
        quantize_all()
        for _, fn in gemms:
            fn()

    def back_to_back(fn, n):
        """Mean time of fn over n calls back to back between one pair of HIP events (per-call events
        would let the host's launch rate, not the GPU, set the pace of the short kernels)."""
        fn()
        torch.cuda.synchronize()
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b_.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b_) / n

    if args.copy_probe:
        copy_probe(torch, dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the step, then each GEMM and the twelve quantisations on their own for the breakdown
    ms = back_to_back(step, args.steps)
    per = {"quantize": back_to_back(quantize_all, args.steps)}
    for name, fn in gemms:
        per[name] = back_to_back(fn, args.steps)
    gemm_fl = {n: 2.0 * M * N * K for n, M, N, K, a, b_, e in FP8_GEMMS}
    total_fl = sum(gemm_fl.values())
    value = total_fl / (ms * 1e-3) / 1e12
    gemm_ms = sum(per[n] for n in gemm_fl)
    # roofline kernel: the row-parallel second MLP GEMM (8192 x 3072 x 1536, one launch, no K split)
    dom = "mlp2_fwd"
    dom_tf = gemm_fl[dom] / (per[dom] * 1e-3) / 1e12
    # the same twelve products in bf16 through the vendor library (torch.matmul), for context
    mm = []
    for n, M, N, K, a, b_, e in FP8_GEMMS:
        mm.append((torch.randn((M, K), device=dev).to(torch.bfloat16), torch.randn((K, N), device=dev).to(torch.bfloat16)))
    for _ in range(2):
        for x_, w_ in mm:
            torch.matmul(x_, w_)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        for x_, w_ in mm:
            torch.matmul(x_, w_)
    t1.record(stream)
    torch.cuda.synchronize()
    lib_ms = t0.elapsed_time(t1) / args.steps
    print(json.dumps({
        "metric": "layer-shard GEMM TFLOP/s in fp8 E4M3 (fwd + dgrad + wgrad, quantisation included), "
                  "8.3B shape t=8, 1 GPU",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3", "data": "synthetic (seeded N(0,1) activations, N(0,1e-3^2) gradients, "
                                     "N(0,0.02^2) weights)",
        "config": {"workload": "rank 0's 12 layer GEMMs in fp8 with 12 per-tensor quantisations (row + transposed "
                               "codes) per step", "tokens": T, "hidden": H, "ffn": FFN, "tp": TP},
        "pct_fp8_peak": round(100 * value * 1e12 / PEAK_FP8, 2),
        "breakdown": {"gemm_gflop": round(total_fl / 1e9, 2), "gemm_ms": round(gemm_ms, 4),
                      "quantize_ms": round(per["quantize"], 4),
                      "gemm_tflops": round(total_fl / (gemm_ms * 1e-3) / 1e12, 2),
                      "per_gemm_us": {n: round(per[n] * 1e3, 1) for n in gemm_fl},
                      "bf16_vendor_matmul_ms_same_shapes": round(lib_ms, 4)},
        "roofline": {"bound": "mfma", "kernel": "gemm_fp8_kernel<256x192, EpiStore> of mlp2_fwd (8192 x 3072 x 1536)",
                     "achieved": round(dom_tf, 2), "peak": PEAK_FP8 / 1e12, "unit": "TFLOP/s",
                     "frac": round(dom_tf * 1e12 / PEAK_FP8, 4),
                     "traffic": measured_traffic(FP8_TRAFFIC_FILE, FP8_KERNEL_SOURCES),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"}}),
          flush=True)


if __name__ == "__main__":
    main()
