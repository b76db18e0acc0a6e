"""Library-routine formulation of the model, used only to pin the oracle.

Built from PyTorch primitives in fp64 on the CPU -- torch.nn.functional's
rms_norm, scaled_dot_product_attention (causal flag or an explicit band
mask), silu and cross_entropy, autograd for gradients, and RoPE written as a
complex rotation -- so that it shares nothing with the oracle's hand-written
loops and backward.  Not used by the product path.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

DT = torch.float64


def t64(a) -> torch.Tensor:
    return torch.as_tensor(np.asarray(a), dtype=DT)


def rope_complex(x: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    """x [..., T, hd]; element i is paired with i + hd/2 and the pair, read as
    a complex number, is multiplied by exp(i * pos * theta^(-2i/hd))."""
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-2.0 * torch.arange(half, dtype=DT) / hd)
    ang = pos.to(DT)[:, None] * inv[None, :]
    z = torch.complex(x[..., :half], x[..., half:]) * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1)


class Weights:
    def __init__(self, w: dict, cfg, fast=None):
        self.cfg = cfg
        self.E = t64(w["embed"])
        self.gf = t64(w["final_norm"])
        self.Wlm = t64(w["lm_head"])
        L = cfg.n_layers
        self.layers = []
        for l in range(L):
            self.layers.append({k: t64(w[k][l]) for k in
                                ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")})
        l0 = L - cfg.n_fast
        # dual: blocks l0..L-1 keep their own MLP frozen (static) and add a dynamic one
        self.dual = bool(getattr(cfg, "dual_mlp", 0))
        # fast weights as leaf tensors (the updated MLP matrices of blocks l0..L-1)
        self.fast = []
        for j, l in enumerate(range(l0, L)):
            if fast is not None:
                src = fast[j]
            elif self.dual:
                src = (w["dyn_gate"][j], w["dyn_up"][j], w["dyn_down"][j])
            else:
                src = (w["w_gate"][l], w["w_up"][l], w["w_down"][l])
            self.fast.append([t64(a).clone().requires_grad_(True) for a in src])
        self.l0 = l0

    def mlp(self, l):
        if l >= self.l0:
            return self.fast[l - self.l0]
        lay = self.layers[l]
        return lay["w_gate"], lay["w_up"], lay["w_down"]


def _block_attn_inputs(W: Weights, l: int, h: torch.Tensor, pos: torch.Tensor):
    cfg = W.cfg
    H, d = cfg.n_heads, cfg.d_model
    hd = d // H
    lay = W.layers[l]
    u = F.rms_norm(h, (d,), weight=lay["attn_norm"], eps=cfg.rms_eps)
    T = h.shape[0]
    q = (u @ lay["wq"].T).view(T, H, hd).transpose(0, 1)
    k = (u @ lay["wk"].T).view(T, H, hd).transpose(0, 1)
    v = (u @ lay["wv"].T).view(T, H, hd).transpose(0, 1)
    return rope_complex(q, pos, cfg.rope_theta), rope_complex(k, pos, cfg.rope_theta), v


def _block_rest(W: Weights, l: int, h: torch.Tensor, att: torch.Tensor):
    cfg = W.cfg
    T = h.shape[0]
    lay = W.layers[l]
    hm = h + att.transpose(0, 1).reshape(T, cfg.d_model) @ lay["wo"].T
    m = F.rms_norm(hm, (cfg.d_model,), weight=lay["mlp_norm"], eps=cfg.rms_eps)
    wg, wu, wd = W.mlp(l)
    y = (F.silu(m @ wg.T) * (m @ wu.T)) @ wd.T
    if W.dual and l >= W.l0:
        y = y + (F.silu(m @ lay["w_gate"].T) * (m @ lay["w_up"].T)) @ lay["w_down"].T
    return hm + y


def band_mask(q_pos: torch.Tensor, k_pos: torch.Tensor, window: int) -> torch.Tensor:
    """True where key position s is visible from query position t: t-window < s <= t."""
    t = q_pos[:, None]
    s = k_pos[None, :]
    return (s <= t) & (s > t - window)


def forward_full(W: Weights, ids, causal_only: bool = False) -> torch.Tensor:
    """One-shot forward over a whole sequence; logits [T, V]."""
    cfg = W.cfg
    ids = torch.as_tensor(np.asarray(ids), dtype=torch.long)
    T = ids.shape[0]
    pos = torch.arange(T)
    h = W.E[ids]
    for l in range(cfg.n_layers):
        q, k, v = _block_attn_inputs(W, l, h, pos)
        if causal_only:
            att = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        else:
            att = F.scaled_dot_product_attention(q, k, v, attn_mask=band_mask(pos, pos, cfg.window))
        h = _block_rest(W, l, h, att)
    hf = F.rms_norm(h, (cfg.d_model,), weight=W.gf, eps=cfg.rms_eps)
    return hf @ W.Wlm.T


def chunk_loop(W: Weights, seq, lr: float, chunk: int, n_steps: int = 1):
    """TTT chunk loop with autograd: keys/values of earlier chunks are kept
    (detached) and attended to through the band mask; per chunk, n_steps times:
    forward at the current fast weights, mean CE, gradient w.r.t. the fast
    weights, one SGD step.  The keys/values cached for the chunk are those of
    its last forward; the loss reported is that of its first.  Returns
    (losses [C], per-chunk logits of the first forward)."""
    cfg = W.cfg
    seq = torch.as_tensor(np.asarray(seq), dtype=torch.long)
    T = seq.shape[0] - 1
    cacheK = [None] * cfg.n_layers
    cacheV = [None] * cfg.n_layers
    losses, all_logits = [], []
    params = [p for blk in W.fast for p in blk]
    for p0 in range(0, T, chunk):
        p1 = min(T, p0 + chunk)
        ids, tgt = seq[p0:p1], seq[p0 + 1:p1 + 1]
        pos = torch.arange(p0, p1)
        for step in range(n_steps):
            h = W.E[ids]
            newK, newV = [], []
            for l in range(cfg.n_layers):
                q, k, v = _block_attn_inputs(W, l, h, pos)
                Kall = k if cacheK[l] is None else torch.cat([cacheK[l], k], dim=1)
                Vall = v if cacheV[l] is None else torch.cat([cacheV[l], v], dim=1)
                mask = band_mask(pos, torch.arange(0, p1), cfg.window)
                att = F.scaled_dot_product_attention(q, Kall, Vall, attn_mask=mask)
                newK.append(k.detach())
                newV.append(v.detach())
                h = _block_rest(W, l, h, att)
            hf = F.rms_norm(h, (cfg.d_model,), weight=W.gf, eps=cfg.rms_eps)
            logits = hf @ W.Wlm.T
            loss = F.cross_entropy(logits, tgt, ignore_index=-1)
            grads = torch.autograd.grad(loss, params)
            with torch.no_grad():
                for p, g in zip(params, grads):
                    p -= lr * g
            if step == 0:
                losses.append(float(loss))
                all_logits.append(logits.detach())
        for l in range(cfg.n_layers):
            cacheK[l] = newK[l] if cacheK[l] is None else torch.cat([cacheK[l], newK[l]], dim=1)
            cacheV[l] = newV[l] if cacheV[l] is None else torch.cat([cacheV[l], newV[l]], dim=1)
    return np.array(losses), all_logits


def fast_numpy(W: Weights) -> list:
    return [tuple(p.detach().numpy() for p in blk) for blk in W.fast]
