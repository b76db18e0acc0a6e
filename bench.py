"""TTT-E2E inner-loop prefill benchmark on one MI355X.

A step is one pass of the whole inner loop over one synthetic sequence of T
tokens per row from a fresh state (ttt_reset): for every chunk of b tokens,
forward with the sliding window, cross-entropy, backward into the
last-quarter MLPs, fused SGD.  Inputs (weights, token ids) are resident on the
device before the timed region; the timed region covers exactly --steps
steps between two device synchronizations.

Prints one JSON line with tokens/s, % of the bf16 MFMA peak (FLOPs counted for
forward + last-quarter backward + update), the roofline of the dominant
kernel measured live with HIP events around its launches in the timed region,
the per-class device time of one extra untimed step (events around every
launch), and the fp64 CPU oracle timed on a bounded sample of the same
workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

CONFIGS = {
    "toy": dict(n_layers=4, d_model=128, n_heads=4, d_ff=512, vocab=512, window=256, chunk=64, n_fast=1,
                rope_theta=1e4, lr=1e-2, dtype="f32", T=1024, dist="uniform"),
    "125m": dict(n_layers=12, d_model=768, n_heads=12, d_ff=2048, vocab=32000, window=8192, chunk=1024, n_fast=3,
                 rope_theta=1e6, lr=1e-3, dtype="bf16", T=32768, dist="zipf"),
    "760m": dict(n_layers=24, d_model=1536, n_heads=16, d_ff=4096, vocab=32000, window=8192, chunk=1024, n_fast=6,
                 rope_theta=1e6, lr=1e-3, dtype="bf16", T=32768, dist="zipf"),
    "3b": dict(n_layers=32, d_model=2560, n_heads=20, d_ff=6912, vocab=32000, window=8192, chunk=1024, n_fast=8,
               rope_theta=1e7, lr=1e-3, dtype="bf16", T=131072, dist="zipf"),
}
PEAK_BF16 = 2.5e15  # MI355X dense bf16 MFMA, FLOP/s
PEAK_F32 = 157.3e12
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, GB/s


def flops_per_row(c: dict, T: int) -> dict:
    """Algorithmic FLOPs (matmul = 2 M N K) of the inner loop over T tokens.  With dual_mlp the
    updated blocks also run their frozen static MLP forward (6 d f per token) and, above the
    lowest updated block, its input-gradient products (6 d f per token)."""
    L, d, f, V, k, b, Lq = c["n_layers"], c["d_model"], c["d_ff"], c["vocab"], c["window"], c["chunk"], c["n_fast"]
    out = {"fwd_gemm": 0, "fwd_attn": 0, "bwd_gemm": 0, "bwd_attn": 0, "upd": 0}
    for p0 in range(0, T, b):
        n = min(b, T - p0)
        A = sum(min(k, t + 1) for t in range(p0, p0 + n))
        I = n * (n + 1) // 2
        out["fwd_gemm"] += n * (L * (8 * d * d + 6 * d * f) + 2 * d * V)
        out["fwd_attn"] += 4 * L * d * A
        out["bwd_gemm"] += 2 * n * d * V + (Lq - 1) * n * (12 * d * f + 8 * d * d) + 8 * n * d * f
        out["bwd_attn"] += (Lq - 1) * (4 * d * A + 4 * d * I)
        out["upd"] += 6 * d * f * Lq
        if c.get("dual_mlp"):
            out["fwd_gemm"] += n * Lq * 6 * d * f
            out["bwd_gemm"] += (Lq - 1) * n * 6 * d * f
    out["total"] = sum(out.values())
    return out


def sgd_bytes_per_row(c: dict, T: int, n_steps: int = 1) -> int:
    """Algorithmic HBM bytes of the weight-gradient products with the fused SGD step over T tokens:
    per fast parameter and step the fp32 master is read and written and one bf16 copy written
    (10 B); the operands (the chunk's output gradients and the saved inputs of the three fast
    matrices, bf16) are read once.  This work is below the ridge point (about 205 FLOP/B at the
    3B shape), so it is priced against HBM bandwidth."""
    d, f, b, Lq = c["d_model"], c["d_ff"], c["chunk"], c["n_fast"]
    total = 0
    for p0 in range(0, T, b):
        n = min(b, T - p0)
        total += Lq * (3 * d * f * 10 + (3 * f + 2 * d) * n * 2)
    return total * max(1, n_steps)


HBM_CLASSES = ("gemm_sgd",)  # profile classes priced in bytes, not FLOPs


def flops_forward(c: dict, T: int) -> int:
    """Algorithmic FLOPs of the forward only (every block, lm_head) over T tokens: the comparator
    with no test-time training."""
    L, d, f, V, k, b = c["n_layers"], c["d_model"], c["d_ff"], c["vocab"], c["window"], c["chunk"]
    total = 0
    for p0 in range(0, T, b):
        n = min(b, T - p0)
        A = sum(min(k, t + 1) for t in range(p0, p0 + n))
        total += n * (L * (8 * d * d + 6 * d * f) + 2 * d * V) + 4 * L * d * A
    return total


def host_cpu() -> tuple:
    """(CPU model from lscpu, CPUs this process may run on)."""
    import subprocess
    model = "unknown"
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    return model, len(os.sched_getaffinity(0))


def cpu_baseline(c: dict, w: dict, seq: np.ndarray, sample_tokens: int) -> dict:
    """The fp64 oracle on the first `sample_tokens` positions (one chunk) of the same workload.

    At position 0 a query sees at most `sample_tokens` keys instead of the window's k, so the
    measured rate flatters the oracle; the steady-state figure scales it by the FLOPs of a token
    with a full window over the FLOPs of the sample's tokens (labelled as extrapolated)."""
    from types import SimpleNamespace

    from oracle import Oracle
    oc = SimpleNamespace(**{k: c[k] for k in ("n_layers", "d_model", "n_heads", "d_ff", "vocab", "window", "chunk",
                                              "n_fast", "rope_theta", "lr")}, batch=1, rms_eps=1e-5,
                         dual_mlp=int(c.get("dual_mlp", 0)))
    n = min(sample_tokens, c["chunk"])
    o = Oracle(oc, w, n)
    t0 = time.perf_counter()
    o.prefill_chunk(seq[:1, :n], seq[:1, 1:n + 1])
    dt = time.perf_counter() - t0
    model, nproc = host_cpu()
    threads = int(os.environ.get("OMP_NUM_THREADS", nproc))
    o.close()
    sample_flops = flops_per_row(dict(c, chunk=n), n)["total"]
    k, b = c["window"], c["chunk"]
    steady = flops_per_row(c, k + b)
    steady_tok = (steady["total"] - flops_per_row(c, k)["total"]) / b  # FLOPs of one chunk past the window fill
    rate = sample_flops / dt
    return {"value": n / dt, "unit": "tokens/s", "cores": min(threads, nproc), "kind": "oracle",
            "cpu_model": model, "nproc": nproc,
            "sample": f"positions 0..{n - 1} of the sequence as one inner-loop step (forward, backward, SGD), "
                      f"fp64, {dt:.1f} s; at position 0 each query sees <= {n} keys, not the window's {k}",
            "fp64_gflops": round(rate / 1e9, 2),
            "steady_state_extrapolated": {"value": round(rate / steady_tok, 4), "unit": "tokens/s",
                                          "basis": "the sample's fp64 FLOP rate applied to the FLOPs of a token "
                                                   f"with a full {k}-key window (extrapolated, not measured)"}}


def measured_traffic(kernel: str, cls: str, config: str):
    """HBM bytes per launch of the roofline kernel (class `cls`) from a committed rocprofv3 counter
    summary (profiles/*_hbm_traffic.txt: FETCH_SIZE and WRITE_SIZE scaled by a plain copy of known
    size), or None when there is none for this kernel and workload or the kernel's source changed
    since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_traffic.txt"))):
        kv = dict(line.split(": ", 1) for line in open(path).read().splitlines()
                  if ": " in line and not line.startswith("#"))
        if kv.get("config") != config or (kv.get("class") != cls and kv.get("kernel") != kernel):
            continue
        src = os.path.join(ROOT, kv.get("source", "-"))
        if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != kv.get("source_sha256"):
            return None
        return float(kv["traffic_bytes_per_launch"])
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="3b", choices=sorted(CONFIGS))
    ap.add_argument("--tokens", type=int, default=0, help="override T (tokens per row)")
    ap.add_argument("--window", type=int, default=0, help="override the attention window k (keys per query)")
    ap.add_argument("--cpu-sample", type=int, default=32, help="oracle sample size in tokens (0 = skip)")
    ap.add_argument("--lookahead", type=int, default=0, help="chunks per batched lower-block pass (0 = library default)")
    ap.add_argument("--workload", default="prefill", choices=("prefill", "decode", "full-attention"),
                    help="decode: greedy generation after a full window, an inner-loop update every chunk; "
                         "full-attention: forward and loss only with the window covering the whole sequence "
                         "(no test-time training), timed beside the TTT prefill step")
    ap.add_argument("--n-steps", type=int, default=0, help="SGD steps per chunk (0 = library default, one)")
    ap.add_argument("--dual-mlp", action="store_true",
                    help="static + dynamic MLP in every updated block (the dynamic one is updated)")
    ap.add_argument("--decode-tokens", type=int, default=1024, help="decode: generated tokens per step")
    ap.add_argument("--no-isolated", action="store_true",
                    help="skip the extra profiled step with the streams serialized (kernel_top_isolated)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy 3 times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4, "copies": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the inner loop of one sequence is "
              "sequential over chunks and this build runs on a single MI355X.", file=sys.stderr)
        sys.exit(2)

    import torch

    from test_token_chunk_amd import TTTConfig, TTTContext, synth

    if args.workload == "decode":
        return decode_bench(args)
    if args.workload == "full-attention":
        return full_attention_bench(args)
    c = dict(CONFIGS[args.config])
    T = args.tokens or c.pop("T")
    c.pop("T", None)
    dist = c.pop("dist")
    if args.window:
        c["window"] = args.window
    torch.cuda.set_device(0)
    t_setup = time.perf_counter()
    shape = synth.Shape(c["n_layers"], c["d_model"], c["n_heads"], c["d_ff"], c["vocab"])
    w = synth.weights(shape, bf16=c["dtype"] == "bf16")
    if args.dual_mlp:
        c["dual_mlp"] = 1
        w.update(synth.dynamic_mlp(shape, c["n_fast"], bf16=c["dtype"] == "bf16"))
    seq = synth.tokens(1, T + 1, c["vocab"], dist)
    cfg = TTTConfig(batch=1, max_positions=T + 8, lookahead=args.lookahead, n_steps=args.n_steps, **c)
    ctx = TTTContext(cfg, w)
    d_tok = torch.tensor(seq[:, :T], dtype=torch.int32, device="cuda")
    d_tgt = torch.tensor(seq[:, 1:], dtype=torch.int32, device="cuda")
    nch = (T + cfg.chunk - 1) // cfg.chunk
    d_loss = torch.zeros(nch, 1, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    print(f"setup {setup_s:.1f} s: config {args.config}, T={T}, {nch} chunks", file=sys.stderr, flush=True)

    def step():
        ctx.reset()
        ctx.prefill_device(d_tok, d_tgt, d_loss)
        ctx.sync()

    for i in range(args.warmup):
        t0 = time.perf_counter()
        step()
        print(f"warmup step {i}: {time.perf_counter() - t0:.3f} s", file=sys.stderr, flush=True)
    # per-class device time of one untimed step (HIP events around every GEMM / attention launch);
    # it picks the roofline kernel: the class with the most device time in the step
    from test_token_chunk_amd import PROFILE_KERNELS
    ctx.profile_begin()
    step()
    kstats = ctx.profile_end()
    roof_cls = max(kstats.items(), key=lambda kv: kv[1]["ms"])[0] if kstats else None

    # timed region: only the roofline kernel's launches carry events
    ctx.profile_begin([roof_cls] if roof_cls else [])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
        print(f"step {i} done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    rstats = ctx.profile_end()
    losses = d_loss[:, 0].cpu().numpy()
    ms = dt / args.steps * 1e3
    tok_s = T / (ms / 1e3)
    F = flops_per_row(c, T)
    if args.n_steps > 1:
        # each further step repeats the chunk's forward from block l0's MLP up (the attention half of
        # block l0 and everything below it is not recomputed), the lm_head, the backward and the update
        top = flops_per_row(dict(c, n_layers=c["n_fast"]), T)
        d, k, b = c["d_model"], c["window"], c["chunk"]
        l0_attn = sum(8 * d * d * min(b, T - p0) + 4 * d * sum(min(k, t + 1) for t in range(p0, min(T, p0 + b)))
                      for p0 in range(0, T, b))
        F["total"] += (args.n_steps - 1) * (top["total"] - l0_attn)
    peak = PEAK_BF16 if c["dtype"] == "bf16" else PEAK_F32

    # roofline of the class with the most device time, from its launches inside the timed region:
    # achieved = its algorithmic FLOPs (summed over the shapes it runs) / its summed duration
    hd = c["d_model"] // c["n_heads"]
    roof = None
    if roof_cls and roof_cls in rstats:
        name, st = roof_cls, rstats[roof_cls]
        flops_per_launch = st["flops"] / max(st["count"], 1)
        avg_s = st["ms"] / max(st["count"], 1) / 1e3
        achieved = flops_per_launch / avg_s / 1e12
        kname = PROFILE_KERNELS[name][0].replace("hd", str(hd))
        roof = {"kernel": kname, "class": name, "bound": "mfma", "achieved": round(achieved, 1),
                "peak": peak / 1e12, "unit": "TFLOP/s", "frac": round(achieved / (peak / 1e12), 4),
                "traffic": measured_traffic(kname, name, args.config),
                "avg_launch_us": round(avg_s * 1e6, 2), "launches_per_step": st["count"] // args.steps,
                "gflop_per_launch": round(flops_per_launch / 1e9, 3),
                "share_of_device_time": round(kstats[name]["ms"] / sum(v["ms"] for v in kstats.values()), 4)}
        if name in HBM_CLASSES:
            # bytes per launch: the step's algorithmic bytes of the class over its launches per step
            bytes_per_launch = sgd_bytes_per_row(c, T, args.n_steps) / max(st["count"] // args.steps, 1)
            gbs = bytes_per_launch / avg_s / 1e9
            roof.update({"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "mb_per_launch": round(bytes_per_launch / 1e6, 2),
                         "mfma_tflops": round(achieved, 1)})
    total_dev = sum(v["ms"] for v in kstats.values())
    top = sorted(kstats.items(), key=lambda kv: -kv[1]["ms"])[:6]
    kernel_top = [{"class": k, "kernels": PROFILE_KERNELS[k][0].replace("hd", str(hd)),
                   "ms_per_step": round(v["ms"], 2), "share": round(v["ms"] / total_dev, 4),
                   "tflops": round(v["flops"] / max(v["ms"], 1e-9) / 1e9, 1),
                   "frac": round(v["flops"] / max(v["ms"], 1e-9) / 1e9 / (peak / 1e12), 4)} for k, v in top]
    for e in kernel_top:
        if e["class"] in HBM_CLASSES:
            gbs = sgd_bytes_per_row(c, T, args.n_steps) / (e["ms_per_step"] / 1e3) / 1e9
            e.update({"bound": "hbm", "gbps": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
                      "mfma_frac": e["frac"]})
    iso = None
    if not args.no_isolated:
        # One more (untimed) step in a fresh context with every launch on one stream: per-class
        # device time of each kernel alone on the GPU.  In the measured step the three streams
        # time-slice the CUs, so a class's event time there includes the other streams' kernels.
        ctx.close()
        saved = {k: os.environ.get(k) for k in ("TTT_NO_SIDE", "TTT_NO_BOTTOM_OVERLAP")}
        os.environ.update(TTT_NO_SIDE="1", TTT_NO_BOTTOM_OVERLAP="1")
        try:
            ctx = TTTContext(cfg, w)
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
        ctx.profile_begin()
        t0 = time.perf_counter()
        step()
        iso_ms = (time.perf_counter() - t0) * 1e3
        istats = ctx.profile_end()
        ctx.close()
        iso_top = sorted(istats.items(), key=lambda kv: -kv[1]["ms"])[:8]
        iso = {"step_ms_serial_with_events": round(iso_ms, 1),
               "device_ms_per_step": round(sum(v["ms"] for v in istats.values()), 1), "classes": []}
        for k, v in iso_top:
            e = {"class": k, "ms_per_step": round(v["ms"], 2),
                 "tflops": round(v["flops"] / max(v["ms"], 1e-9) / 1e9, 1),
                 "frac": round(v["flops"] / max(v["ms"], 1e-9) / 1e9 / (peak / 1e12), 4)}
            if k in HBM_CLASSES:
                gbs = sgd_bytes_per_row(c, T, args.n_steps) / (v["ms"] / 1e3) / 1e9
                e.update({"bound": "hbm", "gbps": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
                          "mfma_frac": e["frac"]})
            iso["classes"].append(e)
    out = {
        "metric": "TTT prefill tokens/s (fwd+inner-loop bwd+update) and % bf16 MFMA peak",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 2), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": c["dtype"], "data": "synthetic",
        "config": {"workload": f"ttt-prefill-{args.config}" + (f"-k{c['window']}" if args.window else "") +
                   (f"-steps{args.n_steps}" if args.n_steps > 1 else "") + ("-dual-mlp" if args.dual_mlp else ""),
                   "layers": c["n_layers"],
                   "d_model": c["d_model"], "tokens": T, "window": c["window"], "chunk": c["chunk"],
                   "fast_blocks": c["n_fast"], "batch": 1, "token_dist": dist,
                   "sgd_steps_per_chunk": max(1, args.n_steps), "dual_mlp": bool(args.dual_mlp)},
        "flops_per_step": F["total"], "mfma_peak_frac": round(F["total"] / (ms / 1e3) / peak, 4),
        "final_chunk_loss": float(losses[-1]), "first_chunk_loss": float(losses[0]),
        "roofline": roof,
        "kernel_top": kernel_top,
        "kernel_classes": {k: {"ms_per_step": round(v["ms"], 3), "tflops": round(
            v["flops"] / max(v["ms"], 1e-9) / 1e9, 1)} for k, v in kstats.items()},
        "device_ms_per_step_all_streams": round(total_dev, 1),
        "kernel_top_isolated": iso,
    }
    if args.cpu_sample > 0:
        out["cpu_baseline"] = cpu_baseline(c, w, seq, args.cpu_sample)
    print(json.dumps(out))


def full_attention_bench(args):
    """The comparator of the pages' latency claim: the same model and sequence with the window
    covering every position (full causal attention) and no test-time training -- forward and
    loss only (ttt_score_device) -- timed beside the TTT prefill step at the configuration's
    window.  value = tokens/s of the full-attention forward; ttt_over_full = the TTT step's time
    over the full-attention forward's."""
    import torch

    from test_token_chunk_amd import TTTConfig, TTTContext, synth

    c = dict(CONFIGS[args.config])
    T = args.tokens or c.pop("T")
    c.pop("T", None)
    dist = c.pop("dist")
    if args.window:
        c["window"] = args.window
    torch.cuda.set_device(0)
    w = synth.weights(synth.Shape(c["n_layers"], c["d_model"], c["n_heads"], c["d_ff"], c["vocab"]),
                      bf16=c["dtype"] == "bf16")
    seq = synth.tokens(1, T + 1, c["vocab"], dist)
    d_tok = torch.tensor(seq[:, :T], dtype=torch.int32, device="cuda")
    d_tgt = torch.tensor(seq[:, 1:], dtype=torch.int32, device="cuda")
    nch = (T + c["chunk"] - 1) // c["chunk"]
    d_loss = torch.zeros(nch, 1, dtype=torch.float32, device="cuda")

    def timed(ctx, fn, label):
        def step():
            ctx.reset()
            fn(ctx)
            ctx.sync()
        for i in range(args.warmup):
            step()
            print(f"{label} warmup step {i} done", file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step()
            print(f"{label} step {i} done", file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps

    full = dict(c, window=T)
    ctx = TTTContext(TTTConfig(batch=1, max_positions=T + 8, lookahead=args.lookahead, **full), w)
    t_full = timed(ctx, lambda x: x.score_device(d_tok, d_tgt, d_loss), "full-attention")
    full_losses = d_loss[:, 0].cpu().numpy()
    ctx.close()
    del ctx
    torch.cuda.empty_cache()
    ctx = TTTContext(TTTConfig(batch=1, max_positions=T + 8, lookahead=args.lookahead, **c), w)
    t_ttt = timed(ctx, lambda x: x.prefill_device(d_tok, d_tgt, d_loss), "ttt")
    ttt_losses = d_loss[:, 0].cpu().numpy()
    ctx.close()
    F_full = flops_forward(full, T)
    F_ttt = flops_per_row(c, T)["total"]
    out = {
        "metric": "full-attention forward tokens/s (no test-time training) and TTT/full latency ratio",
        "value": round(T / t_full, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t_full * 1e3, 2), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": c["dtype"], "data": "synthetic",
        "config": {"workload": f"full-attention-vs-ttt-{args.config}", "layers": c["n_layers"],
                   "d_model": c["d_model"], "tokens": T, "ttt_window": c["window"], "chunk": c["chunk"],
                   "fast_blocks": c["n_fast"], "batch": 1, "token_dist": dist},
        "full_attention": {"ms": round(t_full * 1e3, 2), "flops": F_full,
                           "mfma_peak_frac": round(F_full / t_full / PEAK_BF16, 4),
                           "mean_chunk_loss": float(full_losses.mean())},
        "ttt_prefill": {"ms": round(t_ttt * 1e3, 2), "flops": F_ttt, "mfma_peak_frac": round(F_ttt / t_ttt / PEAK_BF16, 4),
                        "mean_chunk_loss": float(ttt_losses.mean())},
        "ttt_over_full_latency": round(t_ttt / t_full, 4),
        "ttt_over_full_flops": round(F_ttt / F_full, 4),
    }
    print(json.dumps(out))


def decode_bench(args):
    """Greedy generation of one row with test-time training: the window is filled by a prefill of
    window + chunk tokens, then a step generates --decode-tokens tokens with an inner-loop update
    after every chunk of them (forward of those positions again, loss, backward, SGD).  The roofline
    kernel is the attention of the single query over its window blocks, bound by reading the
    window's keys and values from HBM."""
    import torch

    from test_token_chunk_amd import PROFILE_KERNELS, TTTConfig, TTTContext, synth

    c = dict(CONFIGS[args.config])
    c.pop("T")
    dist = c.pop("dist")
    if args.window:
        c["window"] = args.window
    n_new, b, k = args.decode_tokens, c["chunk"], c["window"]
    P = k + b
    upd = min(b, n_new)
    torch.cuda.set_device(0)
    w = synth.weights(synth.Shape(c["n_layers"], c["d_model"], c["n_heads"], c["d_ff"], c["vocab"]),
                      bf16=c["dtype"] == "bf16")
    seq = synth.tokens(1, P + 1, c["vocab"], dist)
    max_pos = P + (max(args.warmup, args.steps) + args.steps + 1) * n_new + 8
    ctx = TTTContext(TTTConfig(batch=1, max_positions=max_pos, **c), w)
    ctx.prefill(seq[:, :P], seq[:, 1:])
    last = seq[:, P]
    print(f"decode: config {args.config}, window filled by {P} tokens, {n_new} tokens per step, update every {upd}",
          file=sys.stderr, flush=True)
    # warm-up steps run with the attention launches timed as well, at least as many as the timed
    # steps, so that the library's pool already holds every event the timed region records
    ctx.profile_begin(["swa_decode"])
    for i in range(max(args.warmup, args.steps)):
        toks, _ = ctx.generate(last, n_new, upd)
        last = toks[:, -1]
        print(f"warmup step {i} done", file=sys.stderr, flush=True)
    ctx.profile_end()
    ctx.profile_begin(["swa_decode"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    losses = []
    for i in range(args.steps):
        toks, ul = ctx.generate(last, n_new, upd)
        last = toks[:, -1]
        losses.append(float(ul[0, -1]) if ul.size else None)
        print(f"step {i} done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st = ctx.profile_end().get("swa_decode")
    ms = dt / args.steps * 1e3
    H, hd = c["n_heads"], c["d_model"] // c["n_heads"]
    roof = None
    if st and st["count"]:
        # algorithmic bytes of one launch (position >= window - 1, so every query sees k keys): the
        # window's keys and values (bf16), the query, and the fp32 parts of S = k/128 blocks per head
        S = -(-k // 128)
        byts = 2 * k * H * hd * 2 + H * hd * 2 + S * H * (hd + 2) * 4
        avg_s = st["ms"] / st["count"] / 1e3
        roof = {"kernel": PROFILE_KERNELS["swa_decode"][0].replace("hd", str(hd)), "class": "swa_decode",
                "bound": "hbm", "achieved": round(byts / avg_s / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(byts / avg_s / 8e12, 4), "traffic": None, "avg_launch_us": round(avg_s * 1e6, 2),
                "launches_per_step": st["count"] // args.steps, "mb_per_launch": round(byts / 1e6, 2)}
    out = {
        "metric": "TTT greedy decode tokens/s (update every chunk)", "value": round(args.steps * n_new / dt, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 2),
        "ms_per_token": round(ms / n_new, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": c["dtype"], "data": "synthetic",
        "config": {"workload": f"ttt-decode-{args.config}" + (f"-k{k}" if args.window else ""), "layers": c["n_layers"],
                   "d_model": c["d_model"],
                   "window": k, "chunk": b, "fast_blocks": c["n_fast"], "batch": 1, "tokens_per_step": n_new,
                   "update_every": upd, "prefill_tokens": P, "token_dist": dist},
        "last_update_loss": losses[-1], "roofline": roof,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
