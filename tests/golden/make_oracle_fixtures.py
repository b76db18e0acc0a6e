"""Write the oracle's expected values for the engine tests at the model shapes.

TEST INFRASTRUCTURE.  Calls only the fp64 oracle (oracle/) and the seeded
input generator (test_token_chunk_amd/synth, which holds no arithmetic of the
method); nothing here touches the HIP library.

For each workload the file holds, for one batch row:
  losses        [chunks]      pre-update chunk losses (fp64)
  phi_absmax    [3 * n_fast]  max |W_ref| of every fast tensor after the last chunk
  dw_absmax     [3 * n_fast]  max |W_ref - W_0| of every fast tensor
  dw_argmax     [3 * n_fast]  flat index where that maximum is reached
  dw_at_argmax  [3 * n_fast]  W_ref - W_0 there
  dw_samples    [3 * n_fast, S]  W_ref - W_0 at the sample indices of sample_indices()
plus the configuration, the token recipe and the SHA-256 of the oracle source.
Fast tensors are numbered block by block in ascending order, gate, up, down.

Workloads (the model shapes of the target statement; the first m = k/b + 2
chunks for 3B, where the window has filled and the chunk after it is done):
  125m  12 layers, d 768, 32 chunks of 1024 over 32768 Zipf(1.1) tokens
  3b    32 layers, d 2560, the first 10 chunks of the 131072-token sequence
The 3B run needs about 47 GB of host memory and several hours on 8 cores.

    python tests/golden/make_oracle_fixtures.py 125m
    python tests/golden/make_oracle_fixtures.py 3b
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from types import SimpleNamespace

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from tests.cfgs import M125, M3B  # noqa: E402
from test_token_chunk_amd import synth  # noqa: E402

SAMPLES = 4096          # sampled elements per fast tensor
SAMPLE_SEED = 7         # stream t of this seed picks the samples of fast tensor t
TOKEN_SEED = 1

WORKLOADS = {
    "125m": dict(cfg=M125, chunks=32),
    "3b": dict(cfg=M3B, chunks=10),
}


def fixture_path(name: str) -> str:
    return os.path.join(HERE, f"oracle_{name}.npz")


def fast_tensor_sizes(c) -> list:
    f, d = c["d_ff"], c["d_model"]
    return [f * d] * (3 * c["n_fast"])


def sample_indices(tensor: int, size: int, n: int = SAMPLES) -> np.ndarray:
    """Seeded flat indices into fast tensor number `tensor` (uniform, with repeats)."""
    u = synth.uniform(SAMPLE_SEED, tensor, n)
    return np.minimum((u * size).astype(np.int64), size - 1)


def initial_fast(w: dict, c) -> list:
    L, nf = c["n_layers"], c["n_fast"]
    out = []
    for l in range(L - nf, L):
        out += [w["w_gate"][l].ravel(), w["w_up"][l].ravel(), w["w_down"][l].ravel()]
    return out


def sequence(c, chunks: int) -> np.ndarray:
    T = chunks * c["chunk"]
    return synth.tokens(1, T + 1, c["vocab"], "zipf", seed=TOKEN_SEED)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("workload", choices=sorted(WORKLOADS))
    args = ap.parse_args(argv)
    from oracle import Oracle
    with open(os.path.join(ROOT, "oracle", "ttt_oracle.c"), "rb") as fh:  # the source the library is built from
        sha = hashlib.sha256(fh.read()).hexdigest()
    spec = WORKLOADS[args.workload]
    c = dict(spec["cfg"])
    chunks, b = spec["chunks"], c["chunk"]
    T = chunks * b
    ns = SimpleNamespace(**c)
    t0 = time.time()
    w = synth.weights(synth.Shape(c["n_layers"], c["d_model"], c["n_heads"], c["d_ff"], c["vocab"]),
                      bf16=c["dtype"] == "bf16")
    seq = sequence(c, chunks)
    o = Oracle(ns, w, T)
    losses = []
    for k in range(chunks):
        tc = time.time()
        loss = o.prefill_chunk(seq[:, k * b:(k + 1) * b], seq[:, k * b + 1:(k + 1) * b + 1])
        losses.append(float(loss[0]))
        print(f"{args.workload} chunk {k}: loss {loss[0]:.10f} ({time.time() - tc:.1f} s)", flush=True)
    fast = o.get_fast_flat(0)
    o.close()
    w0 = initial_fast(w, c)
    sizes = fast_tensor_sizes(c)
    nt = len(sizes)
    phi_absmax = np.zeros(nt)
    dw_absmax = np.zeros(nt)
    dw_argmax = np.zeros(nt, dtype=np.int64)
    dw_at_argmax = np.zeros(nt)
    dw_samples = np.zeros((nt, SAMPLES))
    off = 0
    for t in range(nt):
        ref = fast[off:off + sizes[t]]
        dw = ref - w0[t].astype(np.float64)
        phi_absmax[t] = np.max(np.abs(ref))
        i = int(np.argmax(np.abs(dw)))
        dw_argmax[t], dw_at_argmax[t], dw_absmax[t] = i, dw[i], abs(dw[i])
        dw_samples[t] = dw[sample_indices(t, sizes[t])]
        off += sizes[t]
    meta = dict(workload=args.workload, config=c, chunks=chunks, tokens=T, token_dist="zipf",
                token_seed=TOKEN_SEED, weight_seed=synth.WEIGHT_SEED, samples=SAMPLES, sample_seed=SAMPLE_SEED,
                oracle_sha256=sha, oracle_seconds=round(time.time() - t0, 1))
    path = fixture_path(args.workload)
    np.savez_compressed(path, meta=np.array(json.dumps(meta, sort_keys=True)), losses=np.array(losses),
                        phi_absmax=phi_absmax, dw_absmax=dw_absmax, dw_argmax=dw_argmax,
                        dw_at_argmax=dw_at_argmax, dw_samples=dw_samples)
    print(f"wrote {path} ({os.path.getsize(path)} bytes, {time.time() - t0:.0f} s)")
    return 0


if __name__ == "__main__":
    sys.exit(main())
