"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/ttt.h declares, and rejects bad arguments before touching a
device (a valid configuration without a gfx950 device gives TTT_ENODEV)."""
import ctypes
import os
import re

import numpy as np
import pytest

import test_token_chunk_amd as ttt
from test_token_chunk_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = set()
    for hdr in sorted(os.listdir(os.path.join(ROOT, "include"))):
        src = open(os.path.join(ROOT, "include", hdr)).read()
        names |= set(re.findall(r"^\s*(?:int|void|int64_t|const char\*)\s+(tttk?_\w+)\s*\(", src, re.M))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = ttt.load_library()
    declared = header_functions()
    assert len(declared) >= 12
    assert sorted(ttt.EXPORTS + ttt.KERNEL_EXPORTS) == declared
    for name in declared:
        assert hasattr(lib, name), name


def _create(**over):
    lib = ttt.load_library()
    c = ttt.TTTConfig(n_layers=2, d_model=16, n_heads=2, d_ff=24, vocab=11, window=8, chunk=4, dtype="f32",
                      max_positions=64)
    for k, v in over.items():
        setattr(c, k, v)
    w = synth.weights(synth.Shape(2, 16, 2, 24, 11), bf16=False)
    keep = []

    def fp(a):
        a = np.ascontiguousarray(a, dtype=np.float32)
        keep.append(a)
        return a.ctypes.data_as(ttt._FP)

    arrs = {}
    for key in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"):
        arr = (ttt._FP * 2)(*[fp(x) for x in w[key]])
        keep.append(arr)
        arrs[key] = ctypes.cast(arr, ttt._FPP)
    ws = ttt._Weights(fp(w["embed"]), fp(w["final_norm"]), fp(w["lm_head"]), **arrs)
    h = ctypes.c_void_p()
    cc = c._c()
    rc = lib.ttt_create(ctypes.byref(cc), ctypes.byref(ws), None, ctypes.byref(h))
    return rc, lib.ttt_last_error(None).decode(), h


@pytest.mark.parametrize("over,msg", [
    (dict(window=3), "window"),          # k < b (the pages require k >= b)
    (dict(chunk=0), "window"),
    (dict(d_model=15), "multiple"),
    (dict(n_fast=3), "n_fast"),
    (dict(max_positions=0), "max_positions"),
])
def test_create_rejects_bad_config(over, msg):
    rc, err, _ = _create(**over)
    assert rc == ttt.TTT_EINVAL and msg in err


def test_create_without_gpu_reports_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc, err, h = _create()
    assert rc == ttt.TTT_ENODEV and not h.value


def test_null_arguments():
    lib = ttt.load_library()
    assert lib.ttt_create(None, None, None, None) == ttt.TTT_EINVAL
    assert lib.ttt_prefill(None, None, None, 1, None) == ttt.TTT_EINVAL
    assert lib.ttt_reset(None) == ttt.TTT_EINVAL
    assert lib.ttt_position(None) == -1
