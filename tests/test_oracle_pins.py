"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself:
finite differences, library routines (PyTorch fp64 attention / RMSNorm /
cross-entropy / autograd), closed forms and invariances.
"""
import math

import os

import numpy as np
import pytest
import torch

from oracle import Oracle, rmsnorm, rope
from tests import torch_pin as tp
from tests.cfgs import cfg
from test_token_chunk_amd import synth


def tiny_weights(c, std=0.3, seed=7):
    w = synth.weights(synth.Shape(c.n_layers, c.d_model, c.n_heads, c.d_ff, c.vocab), bf16=False, seed=seed, std=std)
    # non-trivial norm gains so that the gain enters every check
    rng = np.random.default_rng(seed)
    for key in ("attn_norm", "mlp_norm"):
        w[key] = [(1.0 + 0.2 * rng.standard_normal(c.d_model)).astype(np.float32) for _ in range(c.n_layers)]
    w["final_norm"] = (1.0 + 0.2 * rng.standard_normal(c.d_model)).astype(np.float32)
    return w


def seq_for(c, T, seed=3):
    return synth.tokens(c.batch, T + 1, c.vocab, "uniform", seed=seed)


# ------------------------------------------------------------------ gradient

@pytest.mark.parametrize("n_fast", [1, 2, 3])
def test_gradient_matches_central_differences(n_fast):
    """Chunk-loss gradient w.r.t. the fast weights equals central finite
    differences of the chunk loss with earlier keys/values frozen; the chunk
    sits after two updated chunks so the store holds cached entries that
    the window reaches (T=12, k=5, b=4)."""
    c = cfg(n_fast=n_fast, lr=0.1)
    w = tiny_weights(c)
    seq = seq_for(c, 12)
    o = Oracle(c, w, 16)
    for ch in range(2):
        o.prefill_chunk(seq[:, ch * 4:(ch + 1) * 4], seq[:, ch * 4 + 1:(ch + 1) * 4 + 1])
    toks, tgts = seq[:, 8:12], seq[:, 9:13]
    _, g = o.eval_chunk(toks, tgts, grad=True)
    g = g[0]
    phi = o.get_fast_flat(0)
    rng = np.random.default_rng(0)
    idx = rng.choice(phi.size, size=min(phi.size, 400), replace=False)
    h = 1e-5
    fd = np.empty(idx.size)
    for j, i in enumerate(idx):
        p = phi.copy()
        p[i] += h
        o.set_fast_flat(0, p)
        lp, _ = o.eval_chunk(toks, tgts)
        p[i] -= 2 * h
        o.set_fast_flat(0, p)
        lm, _ = o.eval_chunk(toks, tgts)
        fd[j] = (lp[0] - lm[0]) / (2 * h)
    o.set_fast_flat(0, phi)
    err = np.max(np.abs(fd - g[idx])) / np.max(np.abs(g[idx]))
    assert err < 1e-6, err
    assert np.max(np.abs(g)) > 1e-4  # the check is not vacuous


# ----------------------------------------------------------- forward / window

def test_full_window_equals_textbook_causal_attention():
    """k >= T and lr = 0: chunked losses equal the per-chunk mean CE of a
    one-shot causal transformer built from library routines."""
    c = cfg(window=16, chunk=4, lr=0.0, n_fast=2)
    w = tiny_weights(c)
    seq = seq_for(c, 12)
    o = Oracle(c, w, 16)
    losses = o.prefill(seq)[0]
    W = tp.Weights(w, c)
    logits = tp.forward_full(W, seq[0, :12], causal_only=True)
    tgt = torch.as_tensor(seq[0, 1:13], dtype=torch.long)
    ref = [float(torch.nn.functional.cross_entropy(logits[s:s + 4], tgt[s:s + 4])) for s in range(0, 12, 4)]
    np.testing.assert_allclose(losses, ref, rtol=1e-12, atol=0)


@pytest.mark.parametrize("window,chunk", [(5, 4), (4, 4), (7, 3)])
def test_lr0_chunked_equals_one_shot_sliding_window(window, chunk):
    """lr = 0: the chunked loop with its key/value store gives the losses of
    a one-shot sliding-window forward with an explicit band mask."""
    c = cfg(window=window, chunk=chunk, lr=0.0, n_fast=2)
    w = tiny_weights(c)
    T = 13
    seq = seq_for(c, T)
    o = Oracle(c, w, 16)
    losses = o.prefill(seq)[0]
    W = tp.Weights(w, c)
    logits = tp.forward_full(W, seq[0, :T])
    tgt = torch.as_tensor(seq[0, 1:T + 1], dtype=torch.long)
    ref = [float(torch.nn.functional.cross_entropy(logits[s:s + chunk], tgt[s:s + chunk])) for s in range(0, T, chunk)]
    np.testing.assert_allclose(losses, ref, rtol=1e-12, atol=0)
    # lr = 0 leaves the fast weights bit-unchanged
    phi0 = np.concatenate([np.concatenate([w["w_gate"][l].ravel(), w["w_up"][l].ravel(), w["w_down"][l].ravel()])
                           for l in range(c.n_layers - c.n_fast, c.n_layers)]).astype(np.float64)
    assert np.array_equal(o.get_fast_flat(0), phi0)


# --------------------------------------------------------------------- update

def test_single_chunk_update_equals_autograd_sgd_step():
    """b = T: exactly one update, equal to phi - lr * autograd gradient of the
    plain sliding-window mean CE."""
    c = cfg(window=12, chunk=12, lr=0.05, n_fast=2)  # k >= b (b = T)
    w = tiny_weights(c)
    seq = seq_for(c, 12)
    o = Oracle(c, w, 16)
    loss = o.prefill(seq)[0]
    W = tp.Weights(w, c)
    logits = tp.forward_full(W, seq[0, :12])
    L = torch.nn.functional.cross_entropy(logits, torch.as_tensor(seq[0, 1:13], dtype=torch.long))
    params = [p for blk in W.fast for p in blk]
    grads = torch.autograd.grad(L, params)
    np.testing.assert_allclose(loss, [float(L)], rtol=1e-12)
    got = o.get_fast(0)
    for j in range(c.n_fast):
        for a in range(3):
            ref = (params[3 * j + a] - c.lr * grads[3 * j + a]).detach().numpy()
            delta_ref = -c.lr * grads[3 * j + a].numpy()
            delta_got = got[j][a] - params[3 * j + a].detach().numpy()
            np.testing.assert_allclose(got[j][a], ref, rtol=1e-12, atol=1e-15)
            assert np.max(np.abs(delta_got - delta_ref)) <= 1e-9 * np.max(np.abs(delta_ref))


@pytest.mark.parametrize("n_fast", [1, 2])
def test_chunk_loop_equals_autograd_chunk_loop(n_fast):
    """Several chunks with lr > 0 (window smaller than the history): losses and
    final fast weights equal a chunk loop driven by autograd with detached
    earlier keys/values."""
    c = cfg(window=6, chunk=4, lr=0.2, n_fast=n_fast)
    w = tiny_weights(c)
    seq = seq_for(c, 16)
    o = Oracle(c, w, 20)
    losses = o.prefill(seq)[0]
    W = tp.Weights(w, c)
    ref_losses, _ = tp.chunk_loop(W, seq[0], c.lr, c.chunk)
    np.testing.assert_allclose(losses, ref_losses, rtol=1e-11)
    got = o.get_fast(0)
    ref = tp.fast_numpy(W)
    w0 = [(w["w_gate"][l], w["w_up"][l], w["w_down"][l]) for l in range(c.n_layers - n_fast, c.n_layers)]
    for j in range(n_fast):
        for a in range(3):
            d_ref = ref[j][a] - w0[j][a]
            d_got = got[j][a] - w0[j][a]
            assert np.max(np.abs(d_got - d_ref)) <= 1e-9 * np.max(np.abs(d_ref))


@pytest.mark.parametrize("n_fast,n_steps", [(1, 2), (2, 3)])
def test_several_sgd_steps_per_chunk_equal_autograd_chunk_loop(n_fast, n_steps):
    """n SGD steps per chunk (forward at the weights the previous step left, loss, gradient,
    step; first loss reported; the chunk's keys/values from its last forward) against the
    autograd chunk loop doing the same with library routines."""
    c = cfg(window=6, chunk=4, lr=0.2, n_fast=n_fast, n_steps=n_steps)
    w = tiny_weights(c)
    seq = seq_for(c, 14)
    o = Oracle(c, w, 20)
    losses = o.prefill(seq)[0]
    W = tp.Weights(w, c)
    ref_losses, _ = tp.chunk_loop(W, seq[0], c.lr, c.chunk, n_steps=n_steps)
    np.testing.assert_allclose(losses, ref_losses, rtol=1e-11)
    got, ref = o.get_fast(0), tp.fast_numpy(W)
    w0 = [(w["w_gate"][l], w["w_up"][l], w["w_down"][l]) for l in range(c.n_layers - n_fast, c.n_layers)]
    for j in range(n_fast):
        for a in range(3):
            d_ref = ref[j][a] - w0[j][a]
            assert np.max(np.abs((got[j][a] - w0[j][a]) - d_ref)) <= 1e-9 * np.max(np.abs(d_ref))
    # more steps move the weights further than one step does
    one = Oracle(cfg(window=6, chunk=4, lr=0.2, n_fast=n_fast), w, 20)
    one.prefill(seq)
    assert not np.allclose(one.get_fast_flat(0), o.get_fast_flat(0))


def test_one_step_is_the_default_and_lr0_steps_change_nothing():
    """n_steps = 1 is exactly the single-step loop; with lr = 0 three steps report the same
    losses as one and leave the fast weights bit for bit unchanged."""
    c = cfg(window=6, chunk=4, lr=0.2, n_fast=2)
    w = tiny_weights(c)
    seq = seq_for(c, 12)
    a, b = Oracle(c, w, 16), Oracle(cfg(window=6, chunk=4, lr=0.2, n_fast=2, n_steps=1), w, 16)
    np.testing.assert_array_equal(a.prefill(seq), b.prefill(seq))
    np.testing.assert_array_equal(a.get_fast_flat(0), b.get_fast_flat(0))
    z1, z3 = Oracle(cfg(window=6, chunk=4, lr=0.0, n_fast=2), w, 16), \
        Oracle(cfg(window=6, chunk=4, lr=0.0, n_fast=2, n_steps=3), w, 16)
    np.testing.assert_array_equal(z1.prefill(seq), z3.prefill(seq))
    np.testing.assert_array_equal(z3.get_fast_flat(0), z1.get_fast_flat(0))


def test_ignored_targets_and_empty_chunk():
    """Targets -1 are left out of the mean; a chunk with none valid has loss 0
    and leaves the fast weights unchanged."""
    c = cfg(window=5, chunk=4, lr=0.1, n_fast=2)
    w = tiny_weights(c)
    seq = seq_for(c, 8)
    o = Oracle(c, w, 16)
    tg = seq[:, 1:5].copy()
    tg[0, 1] = -1
    tg[0, 3] = -1
    loss = o.prefill_chunk(seq[:, 0:4], tg)
    W = tp.Weights(w, c)
    logits = tp.forward_full(W, seq[0, :4])
    ref = torch.nn.functional.cross_entropy(logits, torch.as_tensor(tg[0], dtype=torch.long), ignore_index=-1)
    np.testing.assert_allclose(loss, [float(ref)], rtol=1e-12)
    phi = o.get_fast_flat(0)
    loss2 = o.prefill_chunk(seq[:, 4:8], np.full((1, 4), -1))
    assert loss2[0] == 0.0
    assert np.array_equal(o.get_fast_flat(0), phi)


# ------------------------------------------------------------------- batch rows

def test_row_permutation_equivariance():
    """Unrelated batch rows: permuting them permutes per-row losses and fast
    weights exactly, and the batch-mean loss is unchanged."""
    c = cfg(window=5, chunk=4, lr=0.1, n_fast=2, batch=3)
    w = tiny_weights(c)
    seq = synth.tokens(3, 13, c.vocab, "uniform", seed=11)
    perm = [2, 0, 1]
    a = Oracle(c, w, 16)
    la = a.prefill(seq)
    b = Oracle(c, w, 16)
    lb = b.prefill(seq[perm])
    assert np.array_equal(lb, la[perm])
    for i, p in enumerate(perm):
        assert np.array_equal(b.get_fast_flat(i), a.get_fast_flat(p))
    assert la.mean() == pytest.approx(lb.mean(), rel=1e-15)
    # a row on its own gives the same results as inside the batch
    c1 = cfg(window=5, chunk=4, lr=0.1, n_fast=2, batch=1)
    s = Oracle(c1, w, 16)
    ls = s.prefill(seq[1:2])
    assert np.array_equal(ls[0], la[1])


# ------------------------------------------------------------------ closed forms

@pytest.mark.parametrize("V", [11, 512])
def test_zero_lm_head_gives_log_vocab(V):
    """W_lm = 0: every logit is 0, so every chunk loss is ln V exactly and no
    gradient reaches the fast weights."""
    c = cfg(vocab=V, window=5, chunk=4, lr=0.1, n_fast=2)
    w = synth.weights(synth.Shape(c.n_layers, c.d_model, c.n_heads, c.d_ff, V), bf16=False, zero_lm_head=True)
    seq = seq_for(c, 12)
    o = Oracle(c, w, 16)
    phi = o.get_fast_flat(0)
    losses = o.prefill(seq)[0]
    np.testing.assert_allclose(losses, math.log(V), rtol=1e-15)
    assert np.array_equal(o.get_fast_flat(0), phi)


def test_rope_properties():
    rng = np.random.default_rng(1)
    hd, theta = 32, 1e4
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    assert np.array_equal(rope(q, 0, theta), q)  # position 0 is the identity
    for p in (1, 17, 131071):
        np.testing.assert_allclose(np.linalg.norm(rope(q, p, theta)), np.linalg.norm(q), rtol=1e-14)
        np.testing.assert_allclose(rope(rope(q, p, theta), p, theta, inverse=True), q, rtol=0, atol=1e-13)
    # <R(q, m), R(k, n)> depends only on m - n
    a = rope(q, 100, theta) @ rope(k, 93, theta)
    b = rope(q, 7, theta) @ rope(k, 0, theta)
    np.testing.assert_allclose(a, b, rtol=1e-12)
    # against the complex-rotation form
    ref = tp.rope_complex(torch.as_tensor(q[None, :]), torch.tensor([37]), theta)[0].numpy()
    np.testing.assert_allclose(rope(q, 37, theta), ref, rtol=0, atol=1e-14)


def test_rmsnorm_matches_library_and_scale_invariance():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 24))
    g = (1 + 0.1 * rng.standard_normal(24)).astype(np.float32)
    y = rmsnorm(x, g, 1e-5)
    ref = torch.nn.functional.rms_norm(torch.as_tensor(x), (24,), weight=torch.as_tensor(g, dtype=torch.float64),
                                       eps=1e-5).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-15)
    y0 = rmsnorm(x, g, 0.0)
    np.testing.assert_allclose(rmsnorm(37.5 * x, g, 0.0), y0, rtol=1e-14)


# ------------------------------------------------------------------- decode

def test_generate_equals_chunk_loop_on_extended_sequence():
    """Greedy generation with an update every b tokens is the chunk loop run
    over the prompt followed by the generated tokens: each generated token is
    the argmax of that loop's logits, and each update loss is its chunk loss."""
    c = cfg(window=6, chunk=4, lr=0.2, n_fast=2, vocab=11)
    w = tiny_weights(c)
    T, n_new = 8, 8
    seq = seq_for(c, T)
    o = Oracle(c, w, 32)
    o.prefill(seq)
    toks, upd, _ = o.generate(seq[:, T], n_new, update_every=4)
    ext = np.concatenate([seq[0, :T + 1], toks[0]])  # x_0..x_T, g_0..g_{n-1}
    W = tp.Weights(w, c)
    losses, logits = tp.chunk_loop(W, ext, c.lr, c.chunk)
    lg = torch.cat(logits[T // 4:], dim=0).numpy()  # positions T .. T+n_new-1
    assert np.array_equal(lg.argmax(axis=1), toks[0])
    np.testing.assert_allclose(upd[0], losses[T // 4:], rtol=1e-11)
    # replaying its own tokens reproduces the same state evolution
    o2 = Oracle(c, w, 32)
    o2.prefill(seq)
    toks2, upd2, _ = o2.generate(seq[:, T], n_new, update_every=4, forced=toks)
    assert np.array_equal(toks2, toks) and np.array_equal(upd2, upd)
    assert np.array_equal(o2.get_fast_flat(0), o.get_fast_flat(0))


def test_rejects_bad_ids_and_window_smaller_than_chunk():
    c = cfg(window=3, chunk=4)
    w = tiny_weights(cfg())
    with pytest.raises(ValueError):
        Oracle(c, w, 16)
    o = Oracle(cfg(), w, 16)
    with pytest.raises(ValueError):
        o.prefill_chunk(np.array([[0, 1, 11, 2]]), np.array([[1, 2, 3, 4]]))
    with pytest.raises(ValueError):
        o.prefill_chunk(np.array([[0, 1, 2, 3]]), np.array([[1, 2, -2, 4]]))


def test_fast_set_is_the_last_quarter_of_the_blocks():
    """tests/golden/fast_set.txt (the pages' fast-set rule, cited there): every configuration of the
    tests and the benchmark updates the MLPs of its last max(1, L/4) blocks, and the fast parameter
    count is 3 d f of each of them."""
    from tests import cfgs
    rows = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "fast_set.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                name, L, d, f, nf, npar = line.split()
                rows[name] = tuple(int(x) for x in (L, d, f, nf, npar))
    assert set(rows) == {"toy", "125M", "760M", "3B"}
    for name, (L, d, f, nf, npar) in rows.items():
        assert nf == max(1, L // 4), name
        assert npar == 3 * d * f * nf, name
    for name, c in (("toy", cfgs.TOY), ("125M", cfgs.M125), ("760M", cfgs.M760), ("3B", cfgs.M3B)):
        L, d, f, nf, _ = rows[name]
        assert (c["n_layers"], c["d_model"], c["d_ff"], c["n_fast"]) == (L, d, f, nf), name



# ------------------------------------------------- static + dynamic MLP (dual)

def dual_weights(c, std=0.3, seed=7, static_down_zero=False, dyn_from_static=False):
    """tiny_weights plus the dynamic MLPs of the updated blocks (their own seeded draws)."""
    w = tiny_weights(c, std=std, seed=seed)
    shape = synth.Shape(c.n_layers, c.d_model, c.n_heads, c.d_ff, c.vocab)
    w.update(synth.dynamic_mlp(shape, c.n_fast, bf16=False, seed=seed + 1, std=std))
    l0 = c.n_layers - c.n_fast
    if dyn_from_static:
        for j in range(c.n_fast):
            w["dyn_gate"][j] = w["w_gate"][l0 + j].copy()
            w["dyn_up"][j] = w["w_up"][l0 + j].copy()
    if static_down_zero:
        for l in range(l0, c.n_layers):
            w["w_down"][l] = np.zeros_like(w["w_down"][l])
    return w


@pytest.mark.parametrize("n_fast", [1, 2])
def test_dual_mlp_equals_autograd_chunk_loop(n_fast):
    """Static + dynamic MLP in the updated blocks (the static one frozen, the dynamic one
    updated; one RMSNorm feeds both, their outputs add): losses and final dynamic weights of a
    several-chunk loop equal the autograd chunk loop of the same model."""
    c = cfg(window=6, chunk=4, lr=0.2, n_fast=n_fast, dual_mlp=1)
    w = dual_weights(c)
    seq = seq_for(c, 14)
    o = Oracle(c, w, 20)
    losses = o.prefill(seq)[0]
    W = tp.Weights(w, c)
    ref_losses, _ = tp.chunk_loop(W, seq[0], c.lr, c.chunk)
    np.testing.assert_allclose(losses, ref_losses, rtol=1e-11)
    got, ref = o.get_fast(0), tp.fast_numpy(W)
    for j in range(n_fast):
        for a, key in enumerate(("dyn_gate", "dyn_up", "dyn_down")):
            d_ref = ref[j][a] - w[key][j]
            assert np.max(np.abs((got[j][a] - w[key][j]) - d_ref)) <= 1e-9 * np.max(np.abs(d_ref))


def test_dual_mlp_with_shared_gate_up_equals_single_mlp_with_summed_down():
    """SwiGLU is linear in its down projection: when every dynamic MLP has the static one's
    gate and up weights, the model equals the single-MLP model whose down projection is the sum
    of the two.  So the losses agree, and the gradient w.r.t. the dynamic W_down equals the
    single model's gradient w.r.t. its W_down in every updated block -- in the lower one only if
    the static MLP's input gradient reaches the blocks below."""
    c2 = cfg(window=6, chunk=4, lr=0.0, n_fast=2, dual_mlp=1)
    c1 = cfg(window=6, chunk=4, lr=0.0, n_fast=2)
    w = dual_weights(c2, dyn_from_static=True)
    l0 = c2.n_layers - c2.n_fast
    # both down projections on a grid of 2^-12 (|w| < 2), so their sum is exact in fp32
    for j in range(c2.n_fast):
        w["w_down"][l0 + j] = (np.round(w["w_down"][l0 + j] * 4096) / 4096).astype(np.float32)
        w["dyn_down"][j] = (np.round(w["dyn_down"][j] * 4096) / 4096).astype(np.float32)
    w1 = {k: (list(v) if isinstance(v, list) else v) for k, v in w.items()}
    for j in range(c2.n_fast):
        s64 = w["w_down"][l0 + j].astype(np.float64) + w["dyn_down"][j].astype(np.float64)
        w1["w_down"][l0 + j] = s64.astype(np.float32)
        assert np.array_equal(w1["w_down"][l0 + j].astype(np.float64), s64)
    seq = seq_for(c2, 12)
    od, os_ = Oracle(c2, w, 16), Oracle(c1, w1, 16)
    np.testing.assert_allclose(od.prefill(seq, 2), os_.prefill(seq, 2), rtol=1e-12)
    toks, tgts = seq[:, 8:12], seq[:, 9:13]
    ld, gd = od.eval_chunk(toks, tgts, grad=True)
    ls, gs = os_.eval_chunk(toks, tgts, grad=True)
    np.testing.assert_allclose(ld, ls, rtol=1e-12)
    fd = c2.d_ff * c2.d_model
    for j in range(c2.n_fast):
        dn = slice(j * 3 * fd + 2 * fd, (j + 1) * 3 * fd)
        err = np.max(np.abs(gd[0, dn] - gs[0, dn])) / np.max(np.abs(gs[0, dn]))
        assert err < 1e-10, (j, err)
        assert np.max(np.abs(gs[0, dn])) > 1e-4


def test_dual_mlp_with_zero_static_down_equals_single_mlp():
    """With the static MLPs' down projections zero the static branch adds nothing and passes
    no gradient: the dual model equals the single-MLP model whose updated MLPs start at the
    dynamic weights, losses and updated weights alike over several updated chunks."""
    c2 = cfg(window=6, chunk=4, lr=0.2, n_fast=2, dual_mlp=1)
    c1 = cfg(window=6, chunk=4, lr=0.2, n_fast=2)
    w = dual_weights(c2, static_down_zero=True)
    l0 = c2.n_layers - c2.n_fast
    w1 = {k: (list(v) if isinstance(v, list) else v) for k, v in w.items()}
    for j in range(c2.n_fast):
        w1["w_gate"][l0 + j], w1["w_up"][l0 + j], w1["w_down"][l0 + j] = \
            w["dyn_gate"][j], w["dyn_up"][j], w["dyn_down"][j]
    seq = seq_for(c2, 14)
    od, os_ = Oracle(c2, w, 20), Oracle(c1, w1, 20)
    np.testing.assert_allclose(od.prefill(seq), os_.prefill(seq), rtol=1e-12)
    np.testing.assert_allclose(od.get_fast_flat(0), os_.get_fast_flat(0), rtol=0, atol=1e-13)
    assert not np.allclose(od.get_fast_flat(0), np.concatenate(
        [np.concatenate([w[k][j].ravel() for k in ("dyn_gate", "dyn_up", "dyn_down")]) for j in range(2)]))


def test_dual_mlp_gradient_matches_central_differences():
    """Chunk-loss gradient w.r.t. the dynamic MLPs against central finite differences (two
    updated blocks, cached keys/values from two earlier updated chunks)."""
    c = cfg(n_fast=2, lr=0.1, dual_mlp=1)
    w = dual_weights(c)
    seq = seq_for(c, 12)
    o = Oracle(c, w, 16)
    for ch in range(2):
        o.prefill_chunk(seq[:, ch * 4:(ch + 1) * 4], seq[:, ch * 4 + 1:(ch + 1) * 4 + 1])
    toks, tgts = seq[:, 8:12], seq[:, 9:13]
    _, g = o.eval_chunk(toks, tgts, grad=True)
    g = g[0]
    phi = o.get_fast_flat(0)
    idx = np.random.default_rng(1).choice(phi.size, size=300, replace=False)
    h = 1e-5
    fd = np.empty(idx.size)
    for j, i in enumerate(idx):
        p = phi.copy()
        p[i] += h
        o.set_fast_flat(0, p)
        lp, _ = o.eval_chunk(toks, tgts)
        p[i] -= 2 * h
        o.set_fast_flat(0, p)
        lm, _ = o.eval_chunk(toks, tgts)
        fd[j] = (lp[0] - lm[0]) / (2 * h)
    o.set_fast_flat(0, phi)
    err = np.max(np.abs(fd - g[idx])) / np.max(np.abs(g[idx]))
    assert err < 1e-6, err


def test_dual_mlp_requires_the_dynamic_weights():
    c = cfg(n_fast=2, dual_mlp=1)
    w = tiny_weights(c)
    w.update({"dyn_gate": [], "dyn_up": [], "dyn_down": []})
    with pytest.raises(AssertionError):
        Oracle(c, w, 16)
