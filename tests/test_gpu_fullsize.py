"""Parity at the full sizes of the 3B workload (d=2560, 20 heads of 128, f=6912, V=32000,
window 8192, chunk 1024, 32 chunks per batched lower-block pass), in the launch
configuration the benchmark uses, on sampled outputs that fp64 recomputes one by one:

- every GEMM shape of the step through the C ABI (wide tiles, K-split sums included),
  sampled output elements against fp64 dot products of the same bf16 operands;
- sliding-window attention forward for the batched pass (32768 queries) and for one chunk
  (1024 queries, split key range), sampled queries against the window definition in fp64;
- attention backward for one chunk, sampled dq rows and dk/dv rows against fp64;
- whole-engine properties that hold at any size: the batched lower-block pass is exact
  (lookahead 1 vs 32 agree to the bf16 tolerance) and runs repeat bit for bit.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

D, H, HD, F, V = 2560, 20, 128, 6912, 32000
WINDOW, CHUNK, G = 8192, 1024, 32


def _torch():
    import torch
    assert torch.cuda.is_available()
    return torch


GEMMS = [  # (M, N, K): rows = tokens of a pass or model dims of a weight gradient
    (G * CHUNK, 3 * D, D),      # q|k|v projection, batched pass
    (G * CHUNK, D, F),          # down projection + residual, batched pass
    (CHUNK, 2 * F, D),          # gate|up projection of a chunk
    (CHUNK, V, D),              # LM head
    (CHUNK, D, V),              # d logits -> d hidden (K split)
    (CHUNK, D, 2 * F),          # d(gate|up) -> d hidden (K split)
    (D, F, CHUNK),              # dW_down
    (2 * F, D, CHUNK),          # dW_gate|up
]


@pytest.mark.parametrize("M,N,K", GEMMS)
def test_gemm_full_size_sampled(M, N, K):
    torch = _torch()
    from test_token_chunk_amd import gemm
    print(f"case gemm {M}x{N}x{K}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(M + 7 * N + 13 * K)
    A = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
    B = torch.randn(N, K, device="cuda", generator=g).to(torch.bfloat16)
    ws = torch.empty(8 * CHUNK * (D + 2 * H), dtype=torch.float32, device="cuda")  # the engine's workspace size
    C = gemm(A, B, ws=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M + N + K)
    ms = rng.integers(0, M, 2048)
    ns = rng.integers(0, N, 2048)
    ms[:4], ns[:4] = [0, M - 1, 0, M - 1], [0, 0, N - 1, N - 1]
    a = A[torch.as_tensor(ms, device="cuda")].double().cpu().numpy()
    b = B[torch.as_tensor(ns, device="cuda")].double().cpu().numpy()
    ref = np.einsum("sk,sk->s", a, b)
    got = C[torch.as_tensor(ms, device="cuda"), torch.as_tensor(ns, device="cuda")].double().cpu().numpy()
    # fp32 accumulation of K exact bf16 products (rms ~1): rounding grows like sqrt(K) ulps of
    # partial sums of size ~sqrt(K); K * 1e-6 bounds it with margin, while a dropped or doubled
    # K slice would be off by ~sqrt(K)
    tol = 1e-6 * K * np.sqrt(np.mean(a ** 2) * np.mean(b ** 2))
    err = np.max(np.abs(got - ref))
    print(f"gemm {M}x{N}x{K}: max abs err {err:.3e} (tol {tol:.3e})")
    assert err <= tol


def _attn_inputs(torch, n, R, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn(1, H, n, HD, device="cuda", generator=g).to(torch.bfloat16)
    kr = torch.randn(1, H, R, HD, device="cuda", generator=g).to(torch.bfloat16)
    vr = torch.randn(1, H, R, HD, device="cuda", generator=g).to(torch.bfloat16)
    return q, kr, vr, vr.transpose(2, 3).contiguous()


def _ref_query(q, kr, vr, h, t, pos0, R):
    """fp64 attention of one query over its window: output [HD] and lse."""
    pt = pos0 + t
    keys = np.arange(max(0, pt - WINDOW + 1), pt + 1)
    slots = torch_index(keys % R)
    qv = q[0, h, t].double().cpu().numpy()
    K = kr[0, h, slots].double().cpu().numpy()
    Vv = vr[0, h, slots].double().cpu().numpy()
    s = K @ qv / np.sqrt(HD)
    m = s.max()
    p = np.exp(s - m)
    return (p / p.sum()) @ Vv, m + np.log(p.sum())


def torch_index(a):
    import torch
    return torch.as_tensor(a, device="cuda")


@pytest.mark.parametrize("n,pos0", [(G * CHUNK, 65536), (CHUNK, 130048)])
def test_attention_forward_full_size_sampled(n, pos0):
    """Batched lower-block pass (32 chunks) and one chunk at the end of a 131072-token
    sequence (key-range split); the ring holds window + 32 chunks of slots, as in the engine."""
    torch = _torch()
    from test_token_chunk_amd import swa_fwd
    print(f"case attention fwd n={n} pos0={pos0}", flush=True)
    R = WINDOW + G * CHUNK
    q, kr, vr, vtr = _attn_inputs(torch, n, R, seed=n + pos0)
    o = torch.empty(n, H * HD, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, H, n, dtype=torch.float32, device="cuda")
    ws = torch.empty(8 * CHUNK * (D + 2 * H), dtype=torch.float32, device="cuda")
    swa_fwd(q, kr, vr, vtr, o, lse, pos0, WINDOW, ws=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(n)
    samples = [(int(rng.integers(H)), int(rng.integers(n))) for _ in range(48)] + [(0, 0), (H - 1, n - 1)]
    worst_o = worst_l = 0.0
    for h, t in samples:
        ro, rl = _ref_query(q, kr, vr, h, t, pos0, R)
        go = o[t, h * HD:(h + 1) * HD].double().cpu().numpy()
        worst_o = max(worst_o, np.max(np.abs(go - ro)) / np.max(np.abs(ro)))
        worst_l = max(worst_l, abs(float(lse[0, h, t]) - rl) / abs(rl))
    print(f"attention fwd n={n}: worst O rel err {worst_o:.3e}, lse rel err {worst_l:.3e}")
    assert worst_o <= 2e-2 and worst_l <= 1e-2


def test_attention_backward_full_size_sampled():
    """One chunk (1024 queries) at the end of a 131072-token sequence: sampled dq rows and
    dk/dv rows of the chunk's own keys (earlier keys are constants)."""
    torch = _torch()
    from test_token_chunk_amd import swa_bwd, swa_fwd
    print("case attention bwd full size", flush=True)
    n, pos0 = CHUNK, 130048
    R = WINDOW + G * CHUNK
    q, kr, vr, vtr = _attn_inputs(torch, n, R, seed=5)
    # the chunk's own keys sit in the ring at their slots (the forward wrote them)
    g = torch.Generator(device="cuda").manual_seed(6)
    dO = torch.randn(n, H * HD, device="cuda", generator=g).to(torch.bfloat16)
    o = torch.empty(n, H * HD, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, H, n, dtype=torch.float32, device="cuda")
    ws = torch.empty(8 * CHUNK * (D + 2 * H), dtype=torch.float32, device="cuda")
    swa_fwd(q, kr, vr, vtr, o, lse, pos0, WINDOW, ws=ws)
    dq = torch.empty(n, H * HD, dtype=torch.float32, device="cuda")
    dk, dv = torch.empty_like(dq), torch.empty_like(dq)
    dvec = torch.empty(1, H, n, dtype=torch.float32, device="cuda")
    swa_bwd(q, q.transpose(2, 3).contiguous(), kr, vr, vtr, o, dO, lse, dvec, dq, dk, dv, pos0, WINDOW, ws=ws,
            ktr=kr.transpose(2, 3).contiguous(), dot=torch.empty_like(dO))
    torch.cuda.synchronize()
    sc = 1 / np.sqrt(HD)
    rng = np.random.default_rng(7)
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for h in (0, H - 1):
        # fp64 probabilities of every chunk query over its window (keys pos0+t-8191 .. pos0+t)
        keys = np.arange(pos0 - WINDOW + 1, pos0 + n)            # all keys any chunk query sees
        Kk = kr[0, h, torch_index(keys % R)].double().cpu().numpy()
        Vk = vr[0, h, torch_index(keys % R)].double().cpu().numpy()
        Q = q[0, h].double().cpu().numpy()
        dOh = dO[:, h * HD:(h + 1) * HD].double().cpu().numpy()
        S = (Q @ Kk.T) * sc                                       # [n, len(keys)]
        t_pos = pos0 + np.arange(n)[:, None]
        vis = (keys[None, :] <= t_pos) & (keys[None, :] > t_pos - WINDOW)
        S = np.where(vis, S, -np.inf)
        P = np.exp(S - S.max(1, keepdims=True))
        P /= P.sum(1, keepdims=True)
        dP = dOh @ Vk.T
        Dv = (P * dP).sum(1, keepdims=True)
        dS = P * (dP - Dv)
        for t in list(rng.integers(0, n, 12)) + [0, n - 1]:
            ref = dS[t] @ Kk * sc
            got = dq[t, h * HD:(h + 1) * HD].double().cpu().numpy()
            worst["dq"] = max(worst["dq"], np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
        own = keys >= pos0                                        # the chunk's keys: column index
        for s in list(rng.integers(0, n, 12)) + [0, n - 1]:
            col = np.nonzero(own)[0][s]
            rk = dS[:, col] @ Q * sc
            rv = P[:, col] @ dOh
            gk = dk[s, h * HD:(h + 1) * HD].double().cpu().numpy()
            gv = dv[s, h * HD:(h + 1) * HD].double().cpu().numpy()
            worst["dk"] = max(worst["dk"], np.max(np.abs(gk - rk)) / np.max(np.abs(rk)))
            worst["dv"] = max(worst["dv"], np.max(np.abs(gv - rv)) / np.max(np.abs(rv)))
    print("attention bwd worst rel err", {k: f"{v:.3e}" for k, v in worst.items()})
    assert all(v <= 3e-2 for v in worst.values()), worst


def _ctx3b(torch, w, lookahead, T):
    from test_token_chunk_amd import TTTConfig, TTTContext
    cfg = TTTConfig(n_layers=32, d_model=D, n_heads=H, d_ff=F, vocab=V, window=WINDOW, chunk=CHUNK, n_fast=8,
                    batch=1, rope_theta=1e7, lr=1e-3, dtype="bf16", max_positions=T + 8, lookahead=lookahead)
    return TTTContext(cfg, w)


def test_engine_full_size_lookahead_exact_and_repeatable():
    """The 3B configuration on 4 chunks: batched lower blocks (lookahead 32, the default)
    against one chunk at a time, and a second run after reset repeating bit for bit."""
    torch = _torch()
    from test_token_chunk_amd import synth
    print("case engine 3B 4 chunks", flush=True)
    T = 4 * CHUNK
    w = synth.weights(synth.Shape(32, D, H, F, V), bf16=True)
    seq = synth.tokens(1, T + 1, V, "zipf", seed=3)
    a = _ctx3b(torch, w, 0, T)
    la = a.prefill(seq[:, :T], seq[:, 1:])
    fa = a.fast_weights_flat(0)
    a.reset()
    la2 = a.prefill(seq[:, :T], seq[:, 1:])
    fa2 = a.fast_weights_flat(0)
    assert np.array_equal(la, la2) and np.array_equal(fa, fa2)
    b = _ctx3b(torch, w, 1, T)
    lb = b.prefill(seq[:, :T], seq[:, 1:])
    fb = b.fast_weights_flat(0)
    assert np.all(np.isfinite(la))
    rel = np.max(np.abs(la - lb) / np.abs(lb))
    w0 = np.concatenate([np.concatenate([w["w_gate"][l].ravel(), w["w_up"][l].ravel(), w["w_down"][l].ravel()])
                         for l in range(24, 32)])
    du = np.max(np.abs((fa - w0) - (fb - w0))) / np.max(np.abs(fb - w0))
    print(f"3B lookahead 32 vs 1: loss rel {rel:.3e}, update rel {du:.3e}")
    assert rel <= 2e-2 and du <= 3e-2
