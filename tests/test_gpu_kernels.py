"""Kernel-level parity (include/ttt_kernels.h) against fp64 references.

GEMM: exact fp64 products of the same bf16/fp32 inputs.  Attention: the
window definition written out in fp64 (query t sees keys t-k < s <= t).
The window-set recovery test is bit-exact: with q = 0 every key in the
window gets the same weight, and with V_s = e_(s mod hd) the output times
|S_t| recovers how many window keys fall in each residue class.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    assert torch.cuda.is_available()
    return torch


GEMM_SHAPES = [(128, 128, 64), (300, 200, 72), (1, 512, 128), (1000, 384, 40), (257, 129, 1000), (64, 96, 8),
               (1024, 2560, 256), (1000, 384, 4100), (256, 640, 2056),
               # wide tiles: 128-row (small grid), 128-row split K, 256-row (large grid)
               (512, 512, 256), (512, 1024, 2048), (4096, 4096, 256),
               # a handful of rows (decode): the matrix-vector kernel, K in whole and partial 512-element steps
               (1, 7680, 2560), (2, 300, 520), (3, 1000, 2056), (5, 129, 40), (8, 2560, 6912), (2, 32000, 2560)]


def _workspace(torch, use):
    return torch.zeros(1 << 24, dtype=torch.float32, device="cuda") if use else None


@pytest.mark.parametrize("use_ws", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_matches_fp64(dtype, M, N, K, use_ws):
    """bf16 with a workspace also covers the split-K path (small grids, K >= 1024)."""
    torch = _torch()
    from test_token_chunk_amd import gemm
    g = torch.Generator(device="cpu").manual_seed(M * 7 + N * 3 + K)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    A = torch.randn(M, K, generator=g).to(dt)
    B = torch.randn(N, K, generator=g).to(dt)
    C = gemm(A.cuda(), B.cuda(), ws=_workspace(torch, use_ws))
    torch.cuda.synchronize()
    ref = A.double().numpy() @ B.double().numpy().T
    err = np.max(np.abs(C.cpu().numpy() - ref)) / max(np.max(np.abs(ref)), 1e-30)
    assert err < 2e-6 * max(1.0, np.sqrt(K / 64)), err


def ring_inputs(torch, B, H, hd, n, R, window, pos0, dt, seed=0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn(B, H, n, hd, generator=g).to(dt)
    kr = torch.randn(B, H, R, hd, generator=g).to(dt)
    vr = torch.randn(B, H, R, hd, generator=g).to(dt)
    return q, kr, vr


def ref_attention(q, kr, vr, pos0, window):
    """fp64 sliding-window attention over ring slots; returns O [B,H,n,hd], lse [B,H,n]."""
    B, H, n, hd = q.shape
    R = kr.shape[2]
    O = np.zeros((B, H, n, hd))
    lse = np.zeros((B, H, n))
    for t in range(n):
        pt = pos0 + t
        keys = np.arange(max(0, pt - window + 1), pt + 1)
        slots = keys % R
        s = np.einsum("bhd,bhkd->bhk", q[:, :, t], kr[:, :, slots]) / np.sqrt(hd)
        m = s.max(axis=-1, keepdims=True)
        p = np.exp(s - m)
        den = p.sum(axis=-1, keepdims=True)
        O[:, :, t] = np.einsum("bhk,bhkd->bhd", p / den, vr[:, :, slots])
        lse[:, :, t] = (m + np.log(den))[..., 0]
    return O, lse


ATTN_CASES = [
    # B, H, hd, n, window, pos0, R   (R >= window + n - 1; pos0 > R exercises the wrap)
    (1, 2, 32, 64, 256, 0, 320),
    (1, 2, 32, 64, 256, 1000, 320),
    (2, 3, 64, 100, 130, 517, 256),
    (1, 2, 128, 130, 200, 331, 336),
    (1, 1, 128, 1, 64, 5000, 128),
    (1, 2, 96, 70, 150, 77, 224),
    (1, 2, 128, 300, 1024, 2000, 1344),
    # one query per head (decode): blocks of 128 window keys (6, 16, 3 and 64 here), merged
    (1, 2, 128, 1, 1000, 700, 1100),
    (2, 3, 128, 1, 2048, 5000, 2100),
    (1, 2, 64, 1, 300, 1234, 320),
    (1, 4, 128, 1, 8192, 20000, 9216),
    # more window blocks than one round of the merge holds (64 parts at head dim 128, 128 at
    # 64), so the running maximum is rescaled across rounds: windows of 32768 and 20000 keys
    (1, 2, 128, 1, 32768, 40000, 33024),
    (1, 2, 64, 1, 20000, 30000, 20480),
]


@pytest.mark.parametrize("use_ws", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,H,hd,n,window,pos0,R", ATTN_CASES)
def test_swa_fwd_matches_fp64(dtype, B, H, hd, n, window, pos0, R, use_ws):
    """bf16 with a workspace also covers the split key range (small grids, long windows)."""
    torch = _torch()
    from test_token_chunk_amd import swa_fwd
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, kr, vr = ring_inputs(torch, B, H, hd, n, R, window, pos0, dt)
    vtr = vr.transpose(2, 3).contiguous()
    o = torch.empty(B * n, H * hd, dtype=dt, device="cuda")
    lse = torch.empty(B, H, n, dtype=torch.float32, device="cuda")
    swa_fwd(q.cuda(), kr.cuda(), vr.cuda(), vtr.cuda(), o, lse, pos0, window, ws=_workspace(torch, use_ws))
    torch.cuda.synchronize()
    O, L = ref_attention(q.double().numpy(), kr.double().numpy(), vr.double().numpy(), pos0, window)
    got = o.float().cpu().numpy().reshape(B, n, H, hd).transpose(0, 2, 1, 3)
    tol = 2e-2 if dtype == "bf16" else 1e-5
    assert np.max(np.abs(got - O)) <= tol * np.max(np.abs(O))
    assert np.max(np.abs(lse.cpu().numpy() - L)) <= (1e-2 if dtype == "bf16" else 1e-5) * np.max(np.abs(L))


@pytest.mark.parametrize("trend", ["growing", "shrinking", "spiky"])
def test_swa_fwd_score_trends(trend):
    """Scores that grow along the window (the reference max must move many times), shrink
    (later keys underflow against an early max) or jump by far more than 2^8 at single keys."""
    torch = _torch()
    from test_token_chunk_amd import swa_fwd
    B, H, hd, n, window, pos0, R = 1, 2, 128, 256, 1024, 3000, 1344
    q, kr, vr = ring_inputs(torch, B, H, hd, n, R, window, pos0, torch.float32, seed=11)
    pos = torch.arange(R, dtype=torch.float32)
    # the absolute position of each ring slot over the range the chunk reads
    slot_pos = torch.zeros(R)
    for s_ in range(pos0 - window + 1, pos0 + n):
        slot_pos[s_ % R] = s_
    rel = (slot_pos - (pos0 - window)) / (window + n)
    if trend == "growing":
        scale = 0.5 + 6.0 * rel
    elif trend == "shrinking":
        scale = 6.5 - 6.0 * rel
    else:
        scale = torch.ones(R)
        scale[torch.arange(0, R, 97)] = 12.0
    kr = kr * scale[None, None, :, None]
    q, kr, vr = q.to(torch.bfloat16), kr.to(torch.bfloat16), vr.to(torch.bfloat16)
    o = torch.empty(B * n, H * hd, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, H, n, dtype=torch.float32, device="cuda")
    swa_fwd(q.cuda(), kr.cuda(), vr.cuda(), vr.transpose(2, 3).contiguous().cuda(), o, lse, pos0, window,
            ws=_workspace(torch, True))
    torch.cuda.synchronize()
    O, L = ref_attention(q.double().numpy(), kr.double().numpy(), vr.double().numpy(), pos0, window)
    got = o.float().cpu().numpy().reshape(B, n, H, hd).transpose(0, 2, 1, 3)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - O)) <= 2e-2 * np.max(np.abs(O))
    assert np.max(np.abs(lse.cpu().numpy() - L)) <= 1e-2 * np.max(np.abs(L))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hd,n,window,pos0,R", [(128, 256, 8192, 20000, 9216), (32, 64, 256, 960, 320),
                                                 (64, 96, 100, 5, 200)])
def test_window_set_recovery_bit_exact(dtype, hd, n, window, pos0, R):
    torch = _torch()
    from test_token_chunk_amd import swa_fwd
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, H = 1, 1
    q = torch.zeros(B, H, n, hd, dtype=dt)
    kr = torch.randn(B, H, R, hd, generator=torch.Generator().manual_seed(1)).to(dt)
    vr = torch.zeros(B, H, R, hd, dtype=dt)
    # slot of absolute position s holds e_(s mod hd); positions reachable are pos0-window+1 .. pos0+n-1
    for s in range(max(0, pos0 - window + 1), pos0 + n):
        vr[0, 0, s % R] = 0
        vr[0, 0, s % R, s % hd] = 1
    vtr = vr.transpose(2, 3).contiguous()
    o = torch.empty(n, hd, dtype=dt, device="cuda")
    swa_fwd(q.cuda(), kr.cuda(), vr.cuda(), vtr.cuda(), o, None, pos0, window)
    torch.cuda.synchronize()
    O = o.float().cpu().numpy().astype(np.float64)
    for t in range(n):
        pt = pos0 + t
        keys = np.arange(max(0, pt - window + 1), pt + 1)
        cnt = np.bincount(keys % hd, minlength=hd)
        got = np.rint(O[t] * len(keys)).astype(np.int64)
        assert np.array_equal(got, cnt), t


def ref_attention_bwd(q, kr, vr, dO, pos0, window):
    """fp64 gradients; keys before pos0 are constants (dk, dv only for the chunk's keys)."""
    B, H, n, hd = q.shape
    R = kr.shape[2]
    dq = np.zeros_like(q)
    dk = np.zeros_like(q)
    dv = np.zeros_like(q)
    sc = 1 / np.sqrt(hd)
    for t in range(n):
        pt = pos0 + t
        keys = np.arange(max(0, pt - window + 1), pt + 1)
        slots = keys % R
        s = np.einsum("bhd,bhkd->bhk", q[:, :, t], kr[:, :, slots]) * sc
        p = np.exp(s - s.max(-1, keepdims=True))
        p /= p.sum(-1, keepdims=True)
        dp = np.einsum("bhd,bhkd->bhk", dO[:, :, t], vr[:, :, slots])
        ds = p * (dp - (p * dp).sum(-1, keepdims=True))
        dq[:, :, t] = np.einsum("bhk,bhkd->bhd", ds, kr[:, :, slots]) * sc
        own = keys >= pos0
        for j in np.nonzero(own)[0]:
            kk = keys[j] - pos0
            dk[:, :, kk] += ds[:, :, j, None] * q[:, :, t] * sc
            dv[:, :, kk] += p[:, :, j, None] * dO[:, :, t]
    return dq, dk, dv


@pytest.mark.parametrize("tr", [False, True])
@pytest.mark.parametrize("use_ws", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,H,hd,n,window,pos0,R", [(1, 2, 32, 64, 256, 1000, 320), (2, 2, 64, 100, 130, 517, 256),
                                                    (1, 2, 128, 130, 200, 331, 336), (1, 2, 128, 200, 1536, 3000, 1736),
                                                    (2, 3, 96, 136, 300, 4000, 440),
                                                    # whole 64-query tiles at head dim 128 (the direct-to-LDS dK/dV
                                                    # form): a half-empty last key block, and two rows of 3 heads
                                                    (1, 2, 128, 192, 512, 3000, 704), (2, 3, 128, 256, 1024, 5000, 1280),
                                                    (1, 2, 64, 192, 512, 3000, 704), (2, 3, 64, 128, 300, 4000, 448)])
def test_swa_bwd_matches_fp64(dtype, B, H, hd, n, window, pos0, R, use_ws, tr):
    """tr: the transposed key ring and a dO^T scratch are passed (16-byte tile copies when n % 8 == 0)."""
    torch = _torch()
    if tr and dtype == "f32":
        pytest.skip("transposed operands only feed the bf16 matrix-core path")
    from test_token_chunk_amd import swa_bwd, swa_fwd
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, kr, vr = ring_inputs(torch, B, H, hd, n, R, window, pos0, dt, seed=3)
    dO = torch.randn(B, n, H, hd, generator=torch.Generator().manual_seed(4)).to(dt)
    cu = lambda x: x.contiguous().cuda()
    o = torch.empty(B * n, H * hd, dtype=dt, device="cuda")
    lse = torch.empty(B, H, n, dtype=torch.float32, device="cuda")
    ws = _workspace(torch, use_ws)
    swa_fwd(cu(q), cu(kr), cu(vr), cu(vr.transpose(2, 3)), o, lse, pos0, window, ws=ws)
    dq = torch.empty(B * n, H * hd, dtype=torch.float32, device="cuda")
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    dvec = torch.empty(B, H, n, dtype=torch.float32, device="cuda")
    ktr = cu(kr.transpose(2, 3)) if tr else None
    dot = torch.full((B * n * H * hd,), float("nan"), dtype=dt, device="cuda") if tr else None
    swa_bwd(cu(q), cu(q.transpose(2, 3)), cu(kr), cu(vr), cu(vr.transpose(2, 3)), o, cu(dO.reshape(B * n, H * hd)),
            lse, dvec, dq, dk, dv, pos0, window, ws=ws, ktr=ktr, dot=dot)
    torch.cuda.synchronize()
    rq, rk, rv = ref_attention_bwd(q.double().numpy(), kr.double().numpy(), vr.double().numpy(),
                                   dO.double().numpy().transpose(0, 2, 1, 3), pos0, window)
    tol = 3e-2 if dtype == "bf16" else 1e-5
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        g = got.cpu().numpy().reshape(B, n, H, hd).transpose(0, 2, 1, 3)
        assert np.max(np.abs(g - ref)) <= tol * np.max(np.abs(ref))
