"""ctypes loader for the fp64 CPU oracle of the TTT-E2E inner loop.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use it.  The product path never imports this package; the
oracle shares no code with the HIP path.

The configuration is any object with the attributes n_layers, d_model,
n_heads, d_ff, vocab, window, chunk, n_fast, batch, rope_theta, rms_eps, lr
(and optionally n_steps, SGD steps per chunk, default 1, and dual_mlp, a static
plus a dynamic MLP in every updated block, default 0).
Weights are the dict of fp32 numpy arrays produced by the seeded generator
(row-major [out, in]); with dual_mlp it also holds dyn_gate, dyn_up, dyn_down,
lists of n_fast arrays (the dynamic MLPs' initial weights).  They must stay
alive as long as the Oracle does.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libttt_oracle.so")
_lib = None


def build_lib(force: bool = False) -> str:
    if force or not os.path.exists(_LIB_PATH):
        src = os.path.join(_HERE, "ttt_oracle.c")
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-shared", "-fPIC", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_layers", "d_model", "n_heads", "d_ff", "vocab", "window", "chunk", "n_fast", "batch", "n_steps",
                "dual_mlp")] + \
               [("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_double), ("lr", ctypes.c_double)]


_FP = ctypes.POINTER(ctypes.c_float)
_FPP = ctypes.POINTER(_FP)


class _W(ctypes.Structure):
    _fields_ = [("embed", _FP), ("final_norm", _FP), ("lm_head", _FP)] + \
               [(n, _FPP) for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down",
                                    "dyn_gate", "dyn_up", "dyn_down")]


def _load():
    global _lib
    if _lib is None:
        build_lib()
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.oracle_create.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_W), i64]
        lib.oracle_create.restype = vp
        lib.oracle_destroy.argtypes = [vp]
        lib.oracle_destroy.restype = None
        lib.oracle_fast_size.argtypes = [vp]
        lib.oracle_fast_size.restype = i64
        lib.oracle_get_pos.argtypes = [vp, ctypes.c_int]
        lib.oracle_get_pos.restype = i64
        lib.oracle_get_fast.argtypes = [vp, ctypes.c_int, vp]
        lib.oracle_set_fast.argtypes = [vp, ctypes.c_int, vp]
        lib.oracle_eval_chunk.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp]
        lib.oracle_prefill_chunk.argtypes = [vp, vp, vp, ctypes.c_int, vp]
        lib.oracle_generate.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp]
        lib.oracle_rope.argtypes = [vp, ctypes.c_int, i64, ctypes.c_double, ctypes.c_int, vp]
        lib.oracle_rope.restype = None
        lib.oracle_rmsnorm.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, ctypes.c_double, vp, vp]
        lib.oracle_rmsnorm.restype = None
        _lib = lib
    return _lib


def _fp(a: np.ndarray):
    assert a.dtype == np.float32 and a.flags.c_contiguous
    return a.ctypes.data_as(_FP)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def rope(x: np.ndarray, pos: int, theta: float, inverse: bool = False) -> np.ndarray:
    """Rotate-half RoPE of one head vector (fp64)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    _load().oracle_rope(x.ctypes.data, x.size, pos, theta, -1 if inverse else 1, y.ctypes.data)
    return y


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float32)
    n, d = x.shape
    y = np.empty_like(x)
    _load().oracle_rmsnorm(x.ctypes.data, n, d, g.ctypes.data, eps, y.ctypes.data, None)
    return y


class Oracle:
    def __init__(self, cfg, weights: dict, max_positions: int):
        lib = _load()
        self.cfg = cfg
        self.L = cfg.n_layers
        c = _Cfg(*(int(getattr(cfg, n)) for n in
                   ("n_layers", "d_model", "n_heads", "d_ff", "vocab", "window", "chunk", "n_fast", "batch")),
                 int(getattr(cfg, "n_steps", 1)), int(getattr(cfg, "dual_mlp", 0)), float(cfg.rope_theta),
                 float(cfg.rms_eps), float(cfg.lr))
        self._keep = []
        arrs = {}
        for key in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"):
            lst = [np.ascontiguousarray(a, dtype=np.float32) for a in weights[key]]
            self._keep.extend(lst)
            arr = (_FP * self.L)(*[_fp(a) for a in lst])
            self._keep.append(arr)
            arrs[key] = ctypes.cast(arr, _FPP)
        if int(getattr(cfg, "dual_mlp", 0)):
            nf = int(cfg.n_fast)
            for key in ("dyn_gate", "dyn_up", "dyn_down"):
                lst = [np.ascontiguousarray(a, dtype=np.float32) for a in weights[key]]
                assert len(lst) == nf, f"{key}: {len(lst)} arrays for {nf} updated blocks"
                self._keep.extend(lst)
                arr = (_FP * nf)(*[_fp(a) for a in lst])
                self._keep.append(arr)
                arrs[key] = ctypes.cast(arr, _FPP)
        glob = {k: np.ascontiguousarray(weights[k], dtype=np.float32) for k in ("embed", "final_norm", "lm_head")}
        self._keep.extend(glob.values())
        w = _W(_fp(glob["embed"]), _fp(glob["final_norm"]), _fp(glob["lm_head"]), **arrs)
        self._h = lib.oracle_create(ctypes.byref(c), ctypes.byref(w), int(max_positions))
        if not self._h:
            raise ValueError("oracle_create rejected the configuration (or out of memory)")
        self.fast_size = lib.oracle_fast_size(self._h)

    def close(self):
        if getattr(self, "_h", None):
            _load().oracle_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @property
    def pos(self) -> int:
        return int(_load().oracle_get_pos(self._h, 0))

    def eval_chunk(self, tokens, targets, grad: bool = False):
        tokens, targets = _i32(tokens), _i32(targets)
        B, n = tokens.shape
        loss = np.zeros(B, dtype=np.float64)
        g = np.zeros((B, self.fast_size), dtype=np.float64) if grad else None
        rc = _load().oracle_eval_chunk(self._h, tokens.ctypes.data, targets.ctypes.data, n, loss.ctypes.data,
                                       g.ctypes.data if grad else None)
        if rc:
            raise ValueError(f"oracle_eval_chunk failed ({rc})")
        return loss, g

    def prefill_chunk(self, tokens, targets) -> np.ndarray:
        tokens, targets = _i32(tokens), _i32(targets)
        B, n = tokens.shape
        loss = np.zeros(B, dtype=np.float64)
        rc = _load().oracle_prefill_chunk(self._h, tokens.ctypes.data, targets.ctypes.data, n, loss.ctypes.data)
        if rc:
            raise ValueError(f"oracle_prefill_chunk failed ({rc})")
        return loss

    def prefill(self, seq, n_chunks: int | None = None) -> np.ndarray:
        """seq: [B, T+1] ids; runs the chunk loop over T tokens; losses [B, chunks]."""
        seq = _i32(seq)
        T = seq.shape[1] - 1
        b = self.cfg.chunk
        total = (T + b - 1) // b
        if n_chunks is None:
            n_chunks = total
        out = []
        for c in range(n_chunks):
            s, e = c * b, min(T, (c + 1) * b)
            out.append(self.prefill_chunk(seq[:, s:e], seq[:, s + 1:e + 1]))
        return np.stack(out, axis=1)

    def generate(self, first_input, n_new: int, update_every: int, forced=None, want_logits: bool = False):
        first_input = _i32(first_input)
        B = first_input.shape[0]
        toks = np.zeros((B, n_new), dtype=np.int32)
        nu = n_new // update_every
        losses = np.zeros((B, max(nu, 1)), dtype=np.float64)
        logits = np.zeros((B, n_new, self.cfg.vocab), dtype=np.float64) if want_logits else None
        forced_arr = _i32(forced) if forced is not None else None
        rc = _load().oracle_generate(self._h, first_input.ctypes.data, n_new, update_every,
                                     forced_arr.ctypes.data if forced_arr is not None else None,
                                     toks.ctypes.data, losses.ctypes.data,
                                     logits.ctypes.data if want_logits else None)
        if rc:
            raise ValueError(f"oracle_generate failed ({rc})")
        return toks, losses[:, :nu], logits

    def get_fast_flat(self, row: int) -> np.ndarray:
        out = np.empty(self.fast_size, dtype=np.float64)
        if _load().oracle_get_fast(self._h, row, out.ctypes.data):
            raise IndexError(row)
        return out

    def set_fast_flat(self, row: int, flat: np.ndarray):
        flat = np.ascontiguousarray(flat, dtype=np.float64)
        assert flat.size == self.fast_size
        if _load().oracle_set_fast(self._h, row, flat.ctypes.data):
            raise IndexError(row)

    def get_fast(self, row: int) -> list:
        """[(W_gate [f,d], W_up [f,d], W_down [d,f]) for each fast block, ascending]"""
        flat = self.get_fast_flat(row)
        f, d = self.cfg.d_ff, self.cfg.d_model
        out = []
        for j in range(self.cfg.n_fast):
            blk = flat[j * 3 * f * d:(j + 1) * 3 * f * d]
            out.append((blk[:f * d].reshape(f, d), blk[f * d:2 * f * d].reshape(f, d),
                        blk[2 * f * d:].reshape(d, f)))
        return out
