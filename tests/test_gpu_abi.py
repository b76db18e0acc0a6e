"""The error contract of the C ABI on a live context (include/ttt.h, Conventions).

* Argument errors are caught before any device work and leave the context
  unchanged (position, fast weights, later results).
* A device-side error (a bad id in device input) or a non-finite loss poisons
  the context: later calls return TTT_ESTATE until ttt_reset.
* An allocation hook that returns NULL makes ttt_create fail with TTT_ENOMEM
  and release everything it had allocated.
* A snapshot is refused by a context whose configuration differs in anything
  the stored keys depend on (here the RoPE base).
"""
import ctypes

import numpy as np
import pytest

import test_token_chunk_amd as ttt
from oracle import Oracle
from tests.cfgs import TOY, cfg as mkcfg
from test_token_chunk_amd import synth

pytestmark = pytest.mark.gpu

T = 256


def _torch():
    import torch
    assert torch.cuda.is_available()
    return torch


def _toy(**over):
    c = mkcfg(**dict(TOY, **over))
    w = synth.weights(synth.Shape(c.n_layers, c.d_model, c.n_heads, c.d_ff, c.vocab), bf16=False)
    seq = synth.tokens(1, T + 1, c.vocab, "uniform")
    return c, w, seq


def _ctx(c, w, **over):
    tc = ttt.TTTConfig.from_dict(vars(c), max_positions=T + 8, **over)
    return ttt.TTTContext(tc, w)


def _code(fn, *a):
    with pytest.raises(ttt.TTTError) as ei:
        fn(*a)
    return ei.value.code


def test_bad_ids_leave_context_unchanged():
    """Out-of-range token or target ids (host entry points): TTT_EINVAL before any device work;
    position, fast weights and the results of later calls are as if the call never happened."""
    _torch()
    c, w, seq = _toy()
    ref = _ctx(c, w)
    ref_l = ref.prefill(seq[:, :2 * 64], seq[:, 1:2 * 64 + 1])
    ctx = _ctx(c, w)
    l0 = ctx.prefill(seq[:, :64], seq[:, 1:65])
    pos, fast = ctx.position, ctx.fast_weights_flat(0).copy()
    bad_tok = seq[:, 64:128].copy()
    bad_tok[0, 5] = c.vocab
    bad_tgt = seq[:, 65:129].copy()
    bad_tgt[0, 7] = -2
    neg_tok = seq[:, 64:128].copy()
    neg_tok[0, 0] = -1                      # -1 is only allowed as a target
    for tok, tgt in ((bad_tok, seq[:, 65:129]), (seq[:, 64:128], bad_tgt), (neg_tok, seq[:, 65:129])):
        assert _code(ctx.prefill, tok, tgt) == ttt.TTT_EINVAL
        assert _code(ctx.prefill_chunk, tok, tgt) == ttt.TTT_EINVAL
    assert _code(ctx.prefill_chunk, seq[:, 64:64 + 65], seq[:, 65:65 + 65]) == ttt.TTT_EINVAL  # n > chunk
    assert _code(ctx.generate, np.array([c.vocab], dtype=np.int32), 4, 4) == ttt.TTT_EINVAL
    assert _code(ctx.generate, seq[:, 64], 4, 65) == ttt.TTT_EINVAL                           # update_every > b
    assert ctx.position == pos
    assert np.array_equal(ctx.fast_weights_flat(0), fast)
    l1 = ctx.prefill(seq[:, 64:128], seq[:, 65:129])
    assert np.array_equal(np.concatenate([l0, l1], axis=1), ref_l)
    assert np.array_equal(ctx.fast_weights_flat(0), ref.fast_weights_flat(0))


def test_device_error_poisons_until_reset():
    """A bad id in device input is found on the device: ttt_sync reports TTT_EINVAL and poisons
    the context; every later call returns TTT_ESTATE (a snapshot is refused too) until
    ttt_reset, after which the context runs as a fresh one."""
    torch = _torch()
    c, w, seq = _toy()
    ctx = _ctx(c, w)
    tok = torch.tensor(seq[:, :64], dtype=torch.int32, device="cuda")
    tok[0, 3] = c.vocab + 5
    tgt = torch.tensor(seq[:, 1:65], dtype=torch.int32, device="cuda")
    ctx.prefill_device(tok, tgt)
    assert _code(ctx.sync) == ttt.TTT_EINVAL
    assert _code(ctx.prefill, seq[:, :64], seq[:, 1:65]) == ttt.TTT_ESTATE
    assert _code(ctx.generate, seq[:, 0], 4, 4) == ttt.TTT_ESTATE
    assert _code(ctx.save_state) == ttt.TTT_ESTATE
    assert _code(ctx.set_fast_weights_flat, 0, ctx.fast_weights_flat(0)) == ttt.TTT_ESTATE
    ctx.reset()
    assert ctx.position == 0
    got = ctx.prefill(seq[:, :T], seq[:, 1:])
    fresh = _ctx(c, w).prefill(seq[:, :T], seq[:, 1:])
    assert np.array_equal(got, fresh)


def test_snapshot_of_poisoned_device_work_is_refused():
    """ttt_save_state right after device work with a bad id: the error is reported (and the
    context poisoned) before anything is written, instead of travelling inside the snapshot."""
    torch = _torch()
    c, w, seq = _toy()
    ctx = _ctx(c, w)
    tok = torch.tensor(seq[:, :64], dtype=torch.int32, device="cuda")
    tok[0, 0] = -7
    tgt = torch.tensor(seq[:, 1:65], dtype=torch.int32, device="cuda")
    ctx.prefill_device(tok, tgt)
    assert _code(ctx.save_state) == ttt.TTT_EINVAL
    assert _code(ctx.save_state) == ttt.TTT_ESTATE


def test_non_finite_loss_poisons():
    """A NaN in the weights makes the chunk loss non-finite: TTT_ENONFINITE, then TTT_ESTATE
    until ttt_reset (which clears the poisoning; the weights stay what they were)."""
    _torch()
    c, w, seq = _toy()
    w = dict(w)
    w["lm_head"] = w["lm_head"].copy()
    w["lm_head"][3, 7] = np.nan
    ctx = _ctx(c, w)
    assert _code(ctx.prefill, seq[:, :64], seq[:, 1:65]) == ttt.TTT_ENONFINITE
    assert _code(ctx.prefill, seq[:, :64], seq[:, 1:65]) == ttt.TTT_ESTATE
    ctx.reset()
    assert ctx.position == 0
    assert _code(ctx.prefill, seq[:, :64], seq[:, 1:65]) == ttt.TTT_ENONFINITE


def test_allocation_failure_reports_enomem_and_releases_everything():
    """An allocation hook that returns NULL after a number of successful allocations (each one
    through PyTorch's caching allocator): ttt_create returns TTT_ENOMEM, gives back no context
    and frees every allocation it made."""
    torch = _torch()
    c, w, seq = _toy()
    lib = ttt.load_library()
    ttt._install_torch_allocator(lib)
    live = {}

    def run(limit):
        calls = [0]

        def alloc(nbytes, _user):
            calls[0] += 1
            if calls[0] > limit:
                return None
            p = torch.cuda.caching_allocator_alloc(int(nbytes), torch.cuda.current_device(),
                                                   torch.cuda.current_stream())
            live[p] = nbytes
            return p

        def free(ptr, _user):
            live.pop(ptr)
            torch.cuda.caching_allocator_delete(ptr)

        hooks = (ttt._ALLOC_FN(alloc), ttt._FREE_FN(free))
        assert lib.ttt_set_allocator(hooks[0], hooks[1], None) == ttt.TTT_OK
        try:
            with pytest.raises(ttt.TTTError) as ei:
                ttt.TTTContext(ttt.TTTConfig.from_dict(vars(c), max_positions=T + 8), w, use_torch_allocator=False)
        finally:
            assert lib.ttt_set_allocator(ttt._hooks[0], ttt._hooks[1], None) == ttt.TTT_OK
        return ei.value.code, calls[0]

    for limit in (0, 1, 7, 40):
        code, calls = run(limit)
        assert code == ttt.TTT_ENOMEM, (limit, code)
        assert calls == limit + 1
        assert not live, f"{len(live)} allocations left after a failed create (limit {limit})"
    # the restored hook works
    ctx = _ctx(c, w)
    assert np.all(np.isfinite(ctx.prefill(seq[:, :64], seq[:, 1:65])))


def test_snapshot_refused_by_other_rope_base():
    """Ring keys are stored rotated, so a snapshot taken with one RoPE base is refused by a
    context with another (same sizes), and accepted by one with the same base."""
    _torch()
    c, w, seq = _toy()
    a = _ctx(c, w)
    a.prefill(seq[:, :128], seq[:, 1:129])
    blob = a.save_state()
    other = _ctx(c, w, rope_theta=c.rope_theta * 2)
    assert _code(other.load_state, blob) == ttt.TTT_EINVAL
    assert other.position == 0
    same = _ctx(c, w)
    same.load_state(blob)
    assert same.position == 128
    assert np.array_equal(same.fast_weights_flat(0), a.fast_weights_flat(0))


def test_all_ignored_chunk_gives_zero_loss_and_no_update():
    """A chunk whose targets are all -1 (bf16 path, d = 256): loss 0 and the fast weights bit for
    bit unchanged, as in the oracle; the chunks around it match the oracle."""
    from tests.cfgs import MID
    c = mkcfg(**MID)
    w = synth.weights(synth.Shape(c.n_layers, c.d_model, c.n_heads, c.d_ff, c.vocab), bf16=True)
    n = 3 * c.chunk
    seq = synth.tokens(1, n + 1, c.vocab, "zipf")
    tg = seq[:, 1:].copy()
    tg[:, c.chunk:2 * c.chunk] = -1
    ctx = ttt.TTTContext(ttt.TTTConfig.from_dict(vars(c), max_positions=n + 8), w)
    l0 = ctx.prefill_chunk(seq[:, :c.chunk], tg[:, :c.chunk])
    before = ctx.fast_weights_flat(0).copy()
    l1 = ctx.prefill_chunk(seq[:, c.chunk:2 * c.chunk], tg[:, c.chunk:2 * c.chunk])
    assert l1[0] == 0.0
    assert np.array_equal(ctx.fast_weights_flat(0), before)
    l2 = ctx.prefill_chunk(seq[:, 2 * c.chunk:n], tg[:, 2 * c.chunk:n])
    o = Oracle(c, w, n + 8)
    ref = [o.prefill_chunk(seq[:, s:s + c.chunk], tg[:, s:s + c.chunk])[0] for s in range(0, n, c.chunk)]
    assert ref[1] == 0.0
    got = [l0[0], l1[0], l2[0]]
    assert abs(got[0] - ref[0]) <= 2e-2 * abs(ref[0]) and abs(got[2] - ref[2]) <= 2e-2 * abs(ref[2])
