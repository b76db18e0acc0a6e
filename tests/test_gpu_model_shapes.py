"""The HIP path at the model shapes of the target workloads against oracle values stored by
tests/golden/make_oracle_fixtures.py (that script calls only the fp64 oracle and the seeded
input generator).

* 125M shape: all 32 chunks of a 32768-token Zipf(1.1) sequence.
* 3B shape: the first 10 chunks of the 131072-token sequence.  The 8192-key window fills during
  chunk 8, so chunks 8 and 9 see it full, and the 32-chunk batched lower-block pass of the
  library's default lookahead covers them all.

The engine runs at its defaults (bf16, fp32 master fast weights, default lookahead).  Checked
against the bf16 tolerances:
* every chunk loss within 2e-2 relative;
* per fast tensor, the fast weights at the stored samples and at the element where |dW_ref| is
  largest, within 3e-2 of the tensor's max |W_ref|;
* the update dW = W_T - W_0 at the same elements, within 3e-2 of the tensor's max |dW_ref|.
"""
import json
import os

import numpy as np
import pytest

from tests.cfgs import M125, M3B
from tests.golden import make_oracle_fixtures as fx
from test_token_chunk_amd import synth

pytestmark = pytest.mark.gpu

LOSS_TOL, W_TOL = 2e-2, 3e-2


def _load(name):
    path = fx.fixture_path(name)
    if not os.path.exists(path):
        pytest.skip(f"{os.path.basename(path)} has not been generated (tests/golden/make_oracle_fixtures.py {name})")
    with np.load(path, allow_pickle=False) as z:
        data = {k: z[k] for k in z.files}
    data["meta"] = json.loads(str(data["meta"]))
    return data


def _run_engine(c, chunks):
    import torch
    from test_token_chunk_amd import TTTConfig, TTTContext
    assert torch.cuda.is_available()
    T = chunks * c["chunk"]
    w = synth.weights(synth.Shape(c["n_layers"], c["d_model"], c["n_heads"], c["d_ff"], c["vocab"]), bf16=True)
    seq = fx.sequence(c, chunks)
    ctx = TTTContext(TTTConfig.from_dict(c, max_positions=T + 8), w)
    losses = ctx.prefill(seq[:, :T], seq[:, 1:])[0]
    fast = ctx.fast_weights_flat(0)
    w0 = fx.initial_fast(w, c)
    ctx.close()
    return losses, fast, w0


@pytest.mark.parametrize("name,cfg", [("125m", M125), ("3b", M3B)])
def test_engine_matches_oracle_at_model_shape(name, cfg):
    ref = _load(name)
    meta = ref["meta"]
    c = dict(cfg)
    assert meta["config"] == c, "fixture written for another configuration"
    chunks = meta["chunks"]
    print(f"case model shape {name}: {chunks} chunks of {c['chunk']}", flush=True)
    losses, fast, w0 = _run_engine(c, chunks)
    rel = np.abs(losses - ref["losses"]) / np.abs(ref["losses"])
    print(f"{name}: chunk loss rel err max {rel.max():.3e} (chunk {int(rel.argmax())})")
    assert rel.max() <= LOSS_TOL, rel
    sizes = fx.fast_tensor_sizes(c)
    off, worst_w, worst_d = 0, 0.0, 0.0
    for t, size in enumerate(sizes):
        idx = np.concatenate([fx.sample_indices(t, size), [ref["dw_argmax"][t]]])
        want_dw = np.concatenate([ref["dw_samples"][t], [ref["dw_at_argmax"][t]]])
        got_w = fast[off + idx].astype(np.float64)
        base = w0[t][idx].astype(np.float64)
        ew = np.max(np.abs(got_w - (base + want_dw))) / ref["phi_absmax"][t]
        ed = np.max(np.abs((got_w - base) - want_dw)) / ref["dw_absmax"][t]
        worst_w, worst_d = max(worst_w, ew), max(worst_d, ed)
        off += size
    print(f"{name}: fast-weight rel err {worst_w:.3e}, update rel err {worst_d:.3e} "
          f"({len(sizes)} tensors x {fx.SAMPLES + 1} elements)")
    assert worst_w <= W_TOL and worst_d <= W_TOL
