"""Seeded synthetic inputs for the TTT-E2E inner loop.

Both the HIP path and the oracle receive the very same arrays produced here,
so this module holds none of the method's arithmetic: only seeds -> arrays.

* Weights: every matrix (embedding, attention projections, MLP matrices,
  lm_head) ~ N(0, 0.02^2), drawn by fp64 Box-Muller from SplitMix64; norm
  gains are 1.  For bf16 workloads each value is rounded to nearest-even bf16
  *before* it is handed out, so both sides see bf16-representable weights.
* Tokens: T+1 ids per batch row, so that every position of the T-token
  sequence has a next-token target.  Uniform over the vocabulary, or
  Zipf(1.1) over ranks (id = rank - 1), one independent stream per row.

The long documents the pages train and test on (Books, DCLM, PG-19) are not
available; these draws stand in for them with the same shapes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

WEIGHT_SEED = 0
TOKEN_SEED = 1
WEIGHT_STD = 0.02


def build_lib(force: bool = False) -> str:
    """Compile libsynth.so with the host C compiler (plain C + OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        src = os.path.join(_HERE, "synth.c")
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build_lib()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        lib.synth_normal.argtypes = [u64, u64, dbl, ctypes.c_int, ctypes.c_void_p, i64]
        lib.synth_normal.restype = None
        lib.synth_uniform.argtypes = [u64, u64, ctypes.c_void_p, i64]
        lib.synth_uniform.restype = None
        lib.synth_tokens_uniform.argtypes = [u64, u64, i32, ctypes.c_void_p, i64]
        lib.synth_tokens_uniform.restype = None
        lib.synth_tokens_zipf.argtypes = [u64, u64, i32, dbl, ctypes.c_void_p, i64]
        lib.synth_tokens_zipf.restype = ctypes.c_int
        lib.synth_splitmix64_at.argtypes = [u64, u64]
        lib.synth_splitmix64_at.restype = u64
        _lib = lib
    return _lib


def splitmix64_at(key: int, i: int) -> int:
    return int(_load().synth_splitmix64_at(key, i))


def normal(seed: int, stream: int, shape, std: float = WEIGHT_STD, bf16: bool = False) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().synth_normal(seed, stream, std, int(bf16), out.ctypes.data, out.size)
    return out


def uniform(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform(seed, stream, out.ctypes.data, n)
    return out


def tokens(batch: int, n: int, vocab: int, dist: str = "uniform", seed: int = TOKEN_SEED,
           zipf_s: float = 1.1) -> np.ndarray:
    """[batch, n] int32 token ids; row r uses stream r."""
    out = np.empty((batch, n), dtype=np.int32)
    lib = _load()
    for r in range(batch):
        row = out[r]
        if dist == "uniform":
            lib.synth_tokens_uniform(seed, r, vocab, row.ctypes.data, n)
        elif dist == "zipf":
            if lib.synth_tokens_zipf(seed, r, vocab, zipf_s, row.ctypes.data, n) != 0:
                raise MemoryError("zipf table")
        else:
            raise ValueError(f"unknown token distribution {dist!r}")
    return out


@dataclass
class Shape:
    n_layers: int
    d_model: int
    n_heads: int
    d_ff: int
    vocab: int


def weight_stream(name: str, layer: int = -1) -> int:
    """Stream id of one weight tensor (fixed numbering, independent of shape)."""
    glob = {"embed": 0, "lm_head": 1}
    per = {"wq": 0, "wk": 1, "wv": 2, "wo": 3, "w_gate": 4, "w_up": 5, "w_down": 6}
    if layer < 0:
        return glob[name]
    return 16 + 8 * layer + per[name]


def dynamic_mlp_stream(name: str, block: int) -> int:
    """Stream id of a dynamic-MLP tensor of updated block `block` (0 = the lowest updated block)."""
    return (1 << 20) + 4 * block + {"dyn_gate": 0, "dyn_up": 1, "dyn_down": 2}[name]


def dynamic_mlp(shape, n_fast: int, bf16: bool, seed: int = WEIGHT_SEED, std: float = WEIGHT_STD) -> dict:
    """Initial weights of the dynamic MLPs of the n_fast updated blocks, for the variant with a
    static and a dynamic MLP in each of them: {"dyn_gate": [f, d] x n_fast, "dyn_up": [f, d] x
    n_fast, "dyn_down": [d, f] x n_fast}, N(0, std) from streams of their own."""
    d, f = shape.d_model, shape.d_ff
    return {"dyn_gate": [normal(seed, dynamic_mlp_stream("dyn_gate", j), (f, d), std, bf16) for j in range(n_fast)],
            "dyn_up": [normal(seed, dynamic_mlp_stream("dyn_up", j), (f, d), std, bf16) for j in range(n_fast)],
            "dyn_down": [normal(seed, dynamic_mlp_stream("dyn_down", j), (d, f), std, bf16) for j in range(n_fast)]}


def weights(shape, bf16: bool, seed: int = WEIGHT_SEED, std: float = WEIGHT_STD,
            zero_lm_head: bool = False) -> dict:
    """All model weights as fp32 numpy arrays, row-major [out, in]."""
    L, d, f, V = shape.n_layers, shape.d_model, shape.d_ff, shape.vocab
    w = {
        "embed": normal(seed, weight_stream("embed"), (V, d), std, bf16),
        "final_norm": np.ones(d, dtype=np.float32),
        "lm_head": (np.zeros((V, d), dtype=np.float32) if zero_lm_head
                    else normal(seed, weight_stream("lm_head"), (V, d), std, bf16)),
    }
    for key in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"):
        w[key] = []
    for l in range(L):
        w["attn_norm"].append(np.ones(d, dtype=np.float32))
        w["mlp_norm"].append(np.ones(d, dtype=np.float32))
        for key in ("wq", "wk", "wv", "wo"):
            w[key].append(normal(seed, weight_stream(key, l), (d, d), std, bf16))
        w["w_gate"].append(normal(seed, weight_stream("w_gate", l), (f, d), std, bf16))
        w["w_up"].append(normal(seed, weight_stream("w_up", l), (f, d), std, bf16))
        w["w_down"].append(normal(seed, weight_stream("w_down", l), (d, f), std, bf16))
    return w
