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


def flops_per_row(c: dict, T: int) -> dict:
    """Algorithmic FLOPs (matmul = 2 M N K) of the inner loop over T tokens."""
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
    out["total"] = sum(out.values())
    return out


def cpu_baseline(c: dict, w: dict, seq: np.ndarray, sample_tokens: int) -> dict:
    """The fp64 oracle on the first `sample_tokens` positions (one chunk) of the same workload."""
    from types import SimpleNamespace

    from oracle import Oracle
    oc = SimpleNamespace(**{k: c[k] for k in ("n_layers", "d_model", "n_heads", "d_ff", "vocab", "window", "chunk",
                                              "n_fast", "rope_theta", "lr")}, batch=1, rms_eps=1e-5)
    n = min(sample_tokens, c["chunk"])
    o = Oracle(oc, w, n)
    t0 = time.perf_counter()
    o.prefill_chunk(seq[:1, :n], seq[:1, 1:n + 1])
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    o.close()
    return {"value": n / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n} positions of the sequence as one inner-loop step (forward, backward, SGD), "
                      f"fp64, {dt:.1f} s"}


def measured_traffic(kernel: str, config: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, or None when
    there is none for this kernel and workload or the kernel's source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "k_swa_fwd_3b_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = dict(line.split(": ", 1) for line in open(path).read().splitlines()
              if ": " in line and not line.startswith("#"))
    src = os.path.join(ROOT, kv.get("source", "-"))
    if kv.get("kernel") != kernel or kv.get("config") != config or not os.path.exists(src):
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != kv.get("source_sha256"):
        return None
    return float(kv["traffic_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="3b", choices=sorted(CONFIGS))
    ap.add_argument("--tokens", type=int, default=0, help="override T (tokens per row)")
    ap.add_argument("--cpu-sample", type=int, default=32, help="oracle sample size in tokens (0 = skip)")
    ap.add_argument("--lookahead", type=int, default=0, help="chunks per batched lower-block pass (0 = library default)")
    ap.add_argument("--workload", default="prefill", choices=("prefill", "decode"),
                    help="decode: greedy generation after a full window, an inner-loop update every chunk")
    ap.add_argument("--decode-tokens", type=int, default=1024, help="decode: generated tokens per step")
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
    c = dict(CONFIGS[args.config])
    T = args.tokens or c.pop("T")
    c.pop("T", None)
    dist = c.pop("dist")
    torch.cuda.set_device(0)
    t_setup = time.perf_counter()
    w = synth.weights(synth.Shape(c["n_layers"], c["d_model"], c["n_heads"], c["d_ff"], c["vocab"]),
                      bf16=c["dtype"] == "bf16")
    seq = synth.tokens(1, T + 1, c["vocab"], dist)
    cfg = TTTConfig(batch=1, max_positions=T + 8, lookahead=args.lookahead, **c)
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
    # it picks the roofline kernel: the one-kernel class with the most device time
    from test_token_chunk_amd import PROFILE_KERNELS
    ctx.profile_begin()
    step()
    kstats = ctx.profile_end()
    single = {k: v for k, v in kstats.items() if PROFILE_KERNELS.get(k, ("", False))[1]}
    roof_cls = max(single.items(), key=lambda kv: kv[1]["ms"])[0] if single else None

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
    peak = PEAK_BF16 if c["dtype"] == "bf16" else PEAK_F32

    # roofline of the dominant single kernel, from its launches inside the timed region
    roof = None
    if roof_cls and roof_cls in rstats:
        name, st = roof_cls, rstats[roof_cls]
        flops_per_launch = st["flops"] / max(st["count"], 1)
        avg_s = st["ms"] / max(st["count"], 1) / 1e3
        achieved = flops_per_launch / avg_s / 1e12
        kname = PROFILE_KERNELS[name][0].replace("hd", str(c["d_model"] // c["n_heads"]))
        roof = {"kernel": kname, "class": name, "bound": "mfma", "achieved": round(achieved, 1),
                "peak": peak / 1e12, "unit": "TFLOP/s", "frac": round(achieved / (peak / 1e12), 4),
                "traffic": measured_traffic(kname, args.config),
                "avg_launch_us": round(avg_s * 1e6, 2), "launches_per_step": st["count"] // args.steps,
                "gflop_per_launch": round(flops_per_launch / 1e9, 3)}
    out = {
        "metric": "TTT prefill tokens/s (fwd+inner-loop bwd+update) and % bf16 MFMA peak",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 2), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": c["dtype"], "data": "synthetic",
        "config": {"workload": f"ttt-prefill-{args.config}", "layers": c["n_layers"], "d_model": c["d_model"],
                   "tokens": T, "window": c["window"], "chunk": c["chunk"], "fast_blocks": c["n_fast"], "batch": 1,
                   "token_dist": dist},
        "flops_per_step": F["total"], "mfma_peak_frac": round(F["total"] / (ms / 1e3) / peak, 4),
        "final_chunk_loss": float(losses[-1]), "first_chunk_loss": float(losses[0]),
        "roofline": roof,
        "kernel_classes": {k: {"ms_per_step": round(v["ms"], 3), "tflops": round(
            v["flops"] / max(v["ms"], 1e-9) / 1e9, 1)} for k, v in kstats.items()},
    }
    if args.cpu_sample > 0:
        out["cpu_baseline"] = cpu_baseline(c, w, seq, args.cpu_sample)
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
                "bound": "hbm", "achieved": round(byts / avg_s / 1e9, 1), "peak": 8000.0, "unit": "GB/s",
                "frac": round(byts / avg_s / 8e12, 4), "traffic": None, "avg_launch_us": round(avg_s * 1e6, 2),
                "launches_per_step": st["count"] // args.steps, "mb_per_launch": round(byts / 1e6, 2)}
    out = {
        "metric": "TTT greedy decode tokens/s (update every chunk)", "value": round(args.steps * n_new / dt, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 2),
        "ms_per_token": round(ms / n_new, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": c["dtype"], "data": "synthetic",
        "config": {"workload": f"ttt-decode-{args.config}", "layers": c["n_layers"], "d_model": c["d_model"],
                   "window": k, "chunk": b, "fast_blocks": c["n_fast"], "batch": 1, "tokens_per_step": n_new,
                   "update_every": upd, "prefill_tokens": P, "token_dist": dist},
        "last_update_loss": losses[-1], "roofline": roof,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
