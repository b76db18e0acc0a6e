"""tttk_swa_fwd_noalloc (include/ttt_kernels.h) against tttk_swa_fwd given a workspace of the
same size: the same kernels with the same split, so outputs must match bit for bit -- on
consecutive calls with shrinking inputs (the static array keeps the previous call's parts), on
the decode form, and a call whose split would not fit is refused before any launch."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

# B, H, hd, n, window, pos0, R: a 3B-shaped chunk (3 key-range parts of 2.66 M floats, about
# the whole array), then smaller calls (8 parts of one head; the decode form with 64 parts)
CASES = [(1, 20, 128, 1024, 8192, 20000, 9216), (1, 4, 64, 256, 1024, 3000, 1280),
         (2, 3, 128, 1, 8192, 9000, 8448)]


def _inputs(torch, B, H, hd, n, R, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn(B, H, n, hd, generator=g).to(torch.bfloat16).cuda()
    kr = torch.randn(B, H, R, hd, generator=g).to(torch.bfloat16).cuda()
    vr = torch.randn(B, H, R, hd, generator=g).to(torch.bfloat16).cuda()
    return q, kr, vr, vr.transpose(2, 3).contiguous()


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    import torch
    from test_token_chunk_amd import NOALLOC_SCRATCH_FLOATS, swa_fwd, swa_fwd_noalloc
    assert torch.cuda.is_available()
    ws = torch.empty(NOALLOC_SCRATCH_FLOATS, dtype=torch.float32, device="cuda")
    for i, (B, H, hd, n, window, pos0, R) in enumerate(CASES):
        print(f"case noalloc {i}: B={B} H={H} hd={hd} n={n} window={window} pos0={pos0}", flush=True)
        q, kr, vr, vtr = _inputs(torch, B, H, hd, n, R, seed=20 + i)
        o1 = torch.full((B * n, H * hd), float("nan"), dtype=torch.bfloat16, device="cuda")
        l1 = torch.full((B, H, n), float("nan"), dtype=torch.float32, device="cuda")
        o2, l2 = o1.clone(), l1.clone()
        swa_fwd(q, kr, vr, vtr, o1, l1, pos0, window, ws=ws)
        swa_fwd_noalloc(q, kr, vr, vtr, o2, l2, pos0, window)
        torch.cuda.synchronize()
        assert torch.isfinite(o2.float()).all() and torch.isfinite(l2).all()
        assert torch.equal(o1, o2), i
        assert torch.equal(l1, l2), i


def test_noalloc_refuses_a_split_beyond_the_scratch():
    """16 heads of 128 over a 1024-query chunk would split into 4 parts of 2.13 M floats."""
    import torch
    from test_token_chunk_amd import TTT_EINVAL, TTTError, swa_fwd_noalloc
    B, H, hd, n, window, pos0, R = 1, 16, 128, 1024, 8192, 20000, 9216
    q, kr, vr, vtr = _inputs(torch, B, H, hd, n, R, seed=30)
    o = torch.zeros(B * n, H * hd, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(B, H, n, dtype=torch.float32, device="cuda")
    with pytest.raises(TTTError) as ei:
        swa_fwd_noalloc(q, kr, vr, vtr, o, lse, pos0, window)
    assert ei.value.code == TTT_EINVAL
    torch.cuda.synchronize()
    assert not o.any()
