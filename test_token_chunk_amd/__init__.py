"""MI355X-native TTT-E2E inner loop: Python binding of the C ABI (include/ttt.h).

Argument marshalling only: every step of the inner loop runs in the HIP
kernels of libttt.so.  PyTorch provides device memory (its caching allocator
is installed as the library's allocator) and the stream.  There is no CPU
fallback: without the built library, or without a gfx950 GPU, calls fail.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import weakref
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libttt.so")

TTT_OK, TTT_EINVAL, TTT_ENOMEM, TTT_EDEVICE, TTT_ESTATE, TTT_ENONFINITE, TTT_ENODEV = 0, -1, -2, -3, -4, -5, -6
TTT_F32, TTT_BF16 = 0, 1
_NAMES = {-1: "TTT_EINVAL", -2: "TTT_ENOMEM", -3: "TTT_EDEVICE", -4: "TTT_ESTATE", -5: "TTT_ENONFINITE",
          -6: "TTT_ENODEV"}

# every symbol include/ttt.h declares
EXPORTS = ("ttt_set_allocator", "ttt_create", "ttt_prefill_chunk", "ttt_prefill", "ttt_prefill_device", "ttt_sync",
           "ttt_generate", "ttt_get_fast_weights", "ttt_reset", "ttt_position", "ttt_destroy", "ttt_last_error",
           "ttt_profile_enable", "ttt_profile_read", "ttt_set_fast_weights", "ttt_state_size", "ttt_save_state",
           "ttt_load_state", "ttt_score", "ttt_score_device")
PROFILE_CLASSES = ("gemm_f32out", "gemm_bf16out", "gemm_resid", "gemm_swiglu", "gemm_swiglu_bwd", "gemm_sgd",
                   "gemm_splitk", "swa_fwd", "swa_fwd_split", "swa_bwd", "swa_decode", "gemm_qkv_rope",
                   "gemm_lm_ce")
# kernels behind each class (rocprofv3 names); classes marked single=True are one kernel
PROFILE_KERNELS = {  # class: (kernels, one kernel per launch)
    "gemm_f32out": ("k_gemm_wide<256|128, 0, false> (k_gemm_dl / k_gemm_mfma off the wide-tile shapes)", False),
    "gemm_bf16out": ("k_gemm_wide<256|128, 1, false> (k_gemm_dl / k_gemm_mfma off the wide-tile shapes)", False),
    "gemm_resid": ("k_gemm_wide<256|128, 2, false> (k_gemm_mfma off the wide-tile shapes)", False),
    "gemm_swiglu": ("k_gemm_wide<256|128, 7, false> (k_gemm_dl / k_gemm_mfma off the wide-tile shapes)", False),
    "gemm_swiglu_bwd": ("k_gemm_wide<128, 4, false> (k_gemm_mfma off the wide-tile shapes)", False),
    "gemm_sgd": ("k_gemm_dl<*, 5, false> (K <= 1024) / k_gemm_wide<256|128, 5, false> on the side stream "
                 "(overlapped)", False),
    "gemm_splitk": ("k_gemm_wide<128, 0, true> + k_splitk_reduce4<0>", False),
    "swa_fwd": ("k_swa_fwd<hd, 8, false>", True),
    "swa_fwd_split": ("k_swa_fwd<hd, 8, true> + k_swa_combine", False),
    "swa_bwd": ("k_swa_dq2<hd, *> (k_dvec + k_swa_dq<hd, 8, *> off hd 128) + k_swa_dkv3<hd> (k_swa_dkv<hd, *> off "
                "hd 128 / 64 with whole 64-query tiles); split parts "
                "are summed by k_rope_bwd_pack4 outside the class", False),
    "swa_decode": ("k_swa_decode<hd>", True),
    "gemm_qkv_rope": ("k_gemm_wide<256|128, 6, false> (q|k|v product, RoPE and ring writes in the epilogue; "
                      "k_gemv for a handful of rows)", False),
    "gemm_lm_ce": ("k_gemm_wide<256|128, 8, false> (lm_head, vocabulary-tile softmax statistics in the epilogue)",
                   False),
}


class TTTError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_layers", "d_model", "n_heads", "d_ff", "vocab", "window", "chunk", "n_fast", "batch", "dtype",
                 "lookahead", "n_steps")] + \
               [("max_positions", ctypes.c_int64), ("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_double),
                ("lr", ctypes.c_float), ("dual_mlp", ctypes.c_int32)]


_FP = ctypes.POINTER(ctypes.c_float)
_FPP = ctypes.POINTER(_FP)


class _Weights(ctypes.Structure):
    _fields_ = [("embed", _FP), ("final_norm", _FP), ("lm_head", _FP)] + \
               [(n, _FPP) for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down",
                                    "dyn_gate", "dyn_up", "dyn_down")]


_ALLOC_FN = ctypes.CFUNCTYPE(ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p)
_FREE_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_void_p)

_lib = None
_hooks = None


def load_library():
    """Load libttt.so (built by __graft_entry__.build() / build_lib.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run test_token_chunk_amd/build_lib.py")
    # torch first: it carries its own HIP runtime, and the library's HIP dependency must resolve
    # to the runtime torch's memory and streams belong to (opened the other way round, the
    # library saw no device)
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.ttt_set_allocator.argtypes = [_ALLOC_FN, _FREE_FN, vp]
    lib.ttt_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Weights), vp, ctypes.POINTER(vp)]
    lib.ttt_prefill_chunk.argtypes = [vp, vp, vp, i32, vp]
    lib.ttt_prefill.argtypes = [vp, vp, vp, i64, vp]
    lib.ttt_prefill_device.argtypes = [vp, vp, vp, i64, vp]
    lib.ttt_score.argtypes = [vp, vp, vp, i64, vp]
    lib.ttt_score_device.argtypes = [vp, vp, vp, i64, vp]
    lib.ttt_sync.argtypes = [vp]
    lib.ttt_generate.argtypes = [vp, vp, i32, i32, vp, vp]
    lib.ttt_get_fast_weights.argtypes = [vp, i32, vp, i64]
    lib.ttt_reset.argtypes = [vp]
    lib.ttt_position.argtypes = [vp]
    lib.ttt_position.restype = i64
    lib.ttt_destroy.argtypes = [vp]
    lib.ttt_destroy.restype = None
    lib.ttt_set_fast_weights.argtypes = [vp, i32, vp, i64]
    lib.ttt_state_size.argtypes = [vp]
    lib.ttt_state_size.restype = i64
    lib.ttt_save_state.argtypes = [vp, vp, i64]
    lib.ttt_load_state.argtypes = [vp, vp, i64]
    lib.ttt_profile_enable.argtypes = [vp, i32]
    lib.ttt_profile_read.argtypes = [vp, i32, vp, vp, vp]
    lib.ttt_last_error.argtypes = [vp]
    lib.ttt_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _install_torch_allocator(lib):
    """Route the library's device allocations through PyTorch's caching allocator."""
    global _hooks
    if _hooks is not None:
        return
    import torch

    def _alloc(nbytes, _user):
        try:
            return torch.cuda.caching_allocator_alloc(int(nbytes), torch.cuda.current_device(),
                                                      torch.cuda.current_stream())
        except Exception:  # out of memory: the library reports TTT_ENOMEM
            return None

    def _free(ptr, _user):
        torch.cuda.caching_allocator_delete(ptr)

    _hooks = (_ALLOC_FN(_alloc), _FREE_FN(_free))
    rc = lib.ttt_set_allocator(_hooks[0], _hooks[1], None)
    if rc:
        raise TTTError(rc, "ttt_set_allocator")


# Contexts still open when the interpreter exits are destroyed by an exit handler, while the
# allocator callbacks and torch are intact: at finalization, a context held in a module global
# would otherwise free its memory through callbacks whose objects may already be gone.  The
# handler is registered with the first context, after torch is imported, so it runs before
# torch's own exit handlers.
_LIVE = weakref.WeakSet()
_exit_hook = False


def _close_live():
    for ctx in list(_LIVE):
        ctx.close()


def _track(ctx):
    global _exit_hook
    if not _exit_hook:
        atexit.register(_close_live)
        _exit_hook = True
    _LIVE.add(ctx)


@dataclass
class TTTConfig:
    n_layers: int
    d_model: int
    n_heads: int
    d_ff: int
    vocab: int
    window: int
    chunk: int
    n_fast: int = 0
    batch: int = 1
    dtype: str = "bf16"  # "bf16" or "f32"
    lookahead: int = 0
    n_steps: int = 0  # SGD steps per chunk (0 = 1)
    dual_mlp: int = 0  # 1: static + dynamic MLP in every updated block (weights dyn_gate/dyn_up/dyn_down)
    max_positions: int = 1 << 17
    rope_theta: float = 1e4
    rms_eps: float = 1e-5
    lr: float = 1e-3

    @classmethod
    def from_dict(cls, d: dict, **over):
        kw = {k: v for k, v in d.items() if k in cls.__dataclass_fields__}
        kw.update(over)
        return cls(**kw)

    def _c(self) -> _Config:
        return _Config(self.n_layers, self.d_model, self.n_heads, self.d_ff, self.vocab, self.window, self.chunk,
                       self.n_fast, self.batch, TTT_BF16 if self.dtype == "bf16" else TTT_F32, self.lookahead,
                       self.n_steps,
                       self.max_positions, self.rope_theta, self.rms_eps, self.lr, int(self.dual_mlp))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


class TTTContext:
    """One inner-loop state (fast weights, key/value window, position) on the GPU."""

    def __init__(self, cfg: TTTConfig, weights: dict, stream=None, use_torch_allocator: bool = True):
        lib = load_library()
        import torch
        if use_torch_allocator:
            _install_torch_allocator(lib)
        self.cfg = cfg
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        L = cfg.n_layers
        keep = []

        def fp(a):
            a = np.ascontiguousarray(a, dtype=np.float32)
            keep.append(a)
            return a.ctypes.data_as(_FP)

        arrs = {}
        for key in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"):
            arr = (_FP * L)(*[fp(x) for x in weights[key]])
            keep.append(arr)
            arrs[key] = ctypes.cast(arr, _FPP)
        if cfg.dual_mlp:  # the dynamic MLPs of the updated blocks, n_fast arrays each
            nf = cfg.n_fast or max(1, L // 4)
            for key in ("dyn_gate", "dyn_up", "dyn_down"):
                if len(weights[key]) != nf:
                    raise ValueError(f"{key}: {len(weights[key])} arrays for {nf} updated blocks")
                arr = (_FP * nf)(*[fp(x) for x in weights[key]])
                keep.append(arr)
                arrs[key] = ctypes.cast(arr, _FPP)
        w = _Weights(fp(weights["embed"]), fp(weights["final_norm"]), fp(weights["lm_head"]), **arrs)
        h = ctypes.c_void_p()
        self._c = cfg._c()
        rc = lib.ttt_create(ctypes.byref(self._c), ctypes.byref(w), ctypes.c_void_p(self.stream.cuda_stream),
                            ctypes.byref(h))
        if rc:
            raise TTTError(rc, lib.ttt_last_error(None).decode())
        self._h = h
        self._lib = lib
        self.n_fast = cfg.n_fast or max(1, L // 4)
        _track(self)

    def _check(self, rc):
        if rc:
            raise TTTError(rc, self._lib.ttt_last_error(self._h).decode())

    def close(self):
        if getattr(self, "_h", None) is not None and self._h:
            self._lib.ttt_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def position(self) -> int:
        return int(self._lib.ttt_position(self._h))

    def prefill_chunk(self, tokens, targets) -> np.ndarray:
        tokens, targets = _i32(tokens), _i32(targets)
        B, n = tokens.shape
        loss = np.zeros(B, dtype=np.float32)
        self._check(self._lib.ttt_prefill_chunk(self._h, tokens.ctypes.data, targets.ctypes.data, n,
                                                loss.ctypes.data))
        return loss

    def prefill(self, tokens, targets) -> np.ndarray:
        """Host arrays [B, n_tokens]; returns losses [B, n_chunks]."""
        tokens, targets = _i32(tokens), _i32(targets)
        B, n = tokens.shape
        nch = (n + self.cfg.chunk - 1) // self.cfg.chunk
        losses = np.zeros((B, nch), dtype=np.float32)
        self._check(self._lib.ttt_prefill(self._h, tokens.ctypes.data, targets.ctypes.data, n, losses.ctypes.data))
        return losses

    def prefill_seq(self, seq) -> np.ndarray:
        """seq [B, T+1]: inputs seq[:, :T], targets seq[:, 1:]."""
        seq = _i32(seq)
        return self.prefill(seq[:, :-1], seq[:, 1:])

    def prefill_device(self, d_tokens, d_targets, d_losses=None):
        """torch int32 CUDA tensors [B, n_tokens] (contiguous); d_losses fp32 [n_chunks, B] or None. Async."""
        n = d_tokens.shape[1]
        self._check(self._lib.ttt_prefill_device(self._h, ctypes.c_void_p(d_tokens.data_ptr()),
                                                 ctypes.c_void_p(d_targets.data_ptr()), n,
                                                 ctypes.c_void_p(d_losses.data_ptr()) if d_losses is not None
                                                 else None))

    def score(self, tokens, targets) -> np.ndarray:
        """Forward and loss only (no update): host arrays [B, n_tokens]; losses [B, n_chunks]."""
        tokens, targets = _i32(tokens), _i32(targets)
        B, n = tokens.shape
        nch = (n + self.cfg.chunk - 1) // self.cfg.chunk
        losses = np.zeros((B, nch), dtype=np.float32)
        self._check(self._lib.ttt_score(self._h, tokens.ctypes.data, targets.ctypes.data, n, losses.ctypes.data))
        return losses

    def score_device(self, d_tokens, d_targets, d_losses=None):
        """As prefill_device, forward and loss only (no update). Async."""
        n = d_tokens.shape[1]
        self._check(self._lib.ttt_score_device(self._h, ctypes.c_void_p(d_tokens.data_ptr()),
                                               ctypes.c_void_p(d_targets.data_ptr()), n,
                                               ctypes.c_void_p(d_losses.data_ptr()) if d_losses is not None
                                               else None))

    def sync(self):
        self._check(self._lib.ttt_sync(self._h))

    def generate(self, first_input, n_new: int, update_every: int):
        first_input = _i32(first_input)
        B = first_input.shape[0]
        toks = np.zeros((B, n_new), dtype=np.int32)
        nu = n_new // update_every
        losses = np.zeros((B, max(nu, 1)), dtype=np.float32)
        self._check(self._lib.ttt_generate(self._h, first_input.ctypes.data, n_new, update_every, toks.ctypes.data,
                                           losses.ctypes.data))
        return toks, losses[:, :nu]

    def fast_weights_flat(self, row: int = 0) -> np.ndarray:
        n = 3 * self.cfg.d_model * self.cfg.d_ff * self.n_fast
        out = np.zeros(n, dtype=np.float32)
        self._check(self._lib.ttt_get_fast_weights(self._h, row, out.ctypes.data, n))
        return out

    def set_fast_weights_flat(self, row: int, flat) -> None:
        """fp32 fast weights of `row` in the layout of fast_weights_flat."""
        flat = np.ascontiguousarray(flat, dtype=np.float32)
        self._check(self._lib.ttt_set_fast_weights(self._h, row, flat.ctypes.data, flat.size))

    def save_state(self) -> np.ndarray:
        """Snapshot of fast weights, window and position (bytes, see ttt_state_size)."""
        n = int(self._lib.ttt_state_size(self._h))
        buf = np.empty(n, dtype=np.uint8)
        self._check(self._lib.ttt_save_state(self._h, buf.ctypes.data, n))
        return buf

    def load_state(self, blob) -> None:
        blob = np.ascontiguousarray(blob, dtype=np.uint8)
        self._check(self._lib.ttt_load_state(self._h, blob.ctypes.data, blob.size))

    def fast_weights(self, row: int = 0) -> list:
        """[(W_gate [f,d], W_up [f,d], W_down [d,f]) per fast block, ascending]"""
        flat = self.fast_weights_flat(row)
        f, d = self.cfg.d_ff, self.cfg.d_model
        out = []
        for j in range(self.n_fast):
            blk = flat[j * 3 * f * d:(j + 1) * 3 * f * d]
            out.append((blk[:f * d].reshape(f, d), blk[f * d:2 * f * d].reshape(f, d), blk[2 * f * d:].reshape(d, f)))
        return out

    def reset(self):
        self._check(self._lib.ttt_reset(self._h))

    def profile_begin(self, classes=None):
        """Start timing the launches of `classes` (names of PROFILE_CLASSES; None = all) with HIP events."""
        mask = -1 if classes is None else sum(1 << PROFILE_CLASSES.index(k) for k in classes)
        self._check(self._lib.ttt_profile_enable(self._h, mask))
        return True

    def profile_end(self, _token=None) -> dict:
        """Stop timing; {class: {"ms", "count", "flops"}} since profile_begin."""
        n = len(PROFILE_CLASSES)
        ms = np.zeros(n, dtype=np.float64)
        cnt = np.zeros(n, dtype=np.int64)
        fl = np.zeros(n, dtype=np.float64)
        self._check(self._lib.ttt_profile_read(self._h, n, ms.ctypes.data, cnt.ctypes.data, fl.ctypes.data))
        self._check(self._lib.ttt_profile_enable(self._h, 0))
        return {name: {"ms": float(ms[i]), "count": int(cnt[i]), "flops": float(fl[i])}
                for i, name in enumerate(PROFILE_CLASSES) if cnt[i] > 0}


# ---------------------------------------------------------------- kernel level
KERNEL_EXPORTS = ("tttk_gemm", "tttk_swa_fwd", "tttk_swa_bwd", "tttk_swa_fwd_noalloc")
NOALLOC_SCRATCH_FLOATS = 8 * 1024 * 1024  # TTTK_NOALLOC_SCRATCH_FLOATS of include/ttt_kernels.h


def _klib():
    lib = load_library()
    if not getattr(lib, "_k_ready", False):
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.tttk_gemm.argtypes = [ctypes.c_int, vp, i64, vp, i64, vp, i64, i32, i32, i32, vp, i64, vp]
        lib.tttk_swa_fwd.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64, vp, i64,
                                     vp]
        lib.tttk_swa_bwd.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     i32, i32, i32, i32, i32, i32, i64, vp, i64, vp]
        lib.tttk_swa_fwd_noalloc.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64,
                                             vp]
        lib._k_ready = True
    return lib


def _dt(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return TTT_BF16
    if t.dtype == torch.float32:
        return TTT_F32
    raise TypeError(t.dtype)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ws(ws):
    return (_p(ws), ws.numel()) if ws is not None else (None, 0)


def gemm(A, B, C=None, ws=None):
    """C (fp32) = A @ B.T for CUDA tensors A [M,K], B [N,K] (bf16 or fp32, row-major); ws: fp32 workspace."""
    import torch
    M, K = A.shape
    N = B.shape[0]
    if C is None:
        C = torch.empty(M, N, dtype=torch.float32, device=A.device)
    rc = _klib().tttk_gemm(_dt(A), _p(A), A.stride(0), _p(B), B.stride(0), _p(C), C.stride(0), M, N, K, *_ws(ws),
                           _stream())
    if rc:
        raise TTTError(rc, "tttk_gemm")
    return C


def swa_fwd(q, kr, vr, vtr, o, lse, pos0: int, window: int, ws=None):
    """Kernel-level sliding-window attention (see include/ttt_kernels.h)."""
    B, H, n, hd = q.shape
    R = kr.shape[2]
    rc = _klib().tttk_swa_fwd(_dt(q), _p(q), _p(kr), _p(vr), _p(vtr), _p(o), _p(lse), B, H, hd, n, R, window, pos0,
                              *_ws(ws), _stream())
    if rc:
        raise TTTError(rc, "tttk_swa_fwd")


def swa_fwd_noalloc(q, kr, vr, vtr, o, lse, pos0: int, window: int):
    """tttk_swa_fwd_noalloc: as swa_fwd, with the split parts in the library's static scratch."""
    B, H, n, hd = q.shape
    R = kr.shape[2]
    rc = _klib().tttk_swa_fwd_noalloc(_dt(q), _p(q), _p(kr), _p(vr), _p(vtr), _p(o), _p(lse), B, H, hd, n, R, window,
                                      pos0, _stream())
    if rc:
        raise TTTError(rc, "tttk_swa_fwd_noalloc")


def swa_bwd(q, qt, kr, vr, vtr, o, dout, lse, dvec, dq, dk, dv, pos0: int, window: int, ws=None, ktr=None,
            dot=None):
    B, H, n, hd = q.shape
    R = kr.shape[2]
    rc = _klib().tttk_swa_bwd(_dt(q), _p(q), _p(qt), _p(kr), _p(vr), _p(vtr), _p(ktr), _p(o), _p(dout), _p(lse),
                              _p(dvec), _p(dq), _p(dk), _p(dv), _p(dot), B, H, hd, n, R, window, pos0, *_ws(ws),
                              _stream())
    if rc:
        raise TTTError(rc, "tttk_swa_bwd")
