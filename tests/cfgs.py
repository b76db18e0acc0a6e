"""Model/loop configurations used by the tests (plain attribute bags)."""
from types import SimpleNamespace


def cfg(**kw):
    base = dict(n_layers=4, d_model=16, n_heads=2, d_ff=24, vocab=11, window=5, chunk=4, n_fast=1, batch=1,
                rope_theta=1e4, rms_eps=1e-5, lr=0.1, dtype="f32", n_steps=1, dual_mlp=0)
    base.update(kw)
    return SimpleNamespace(**base)


# the pages' toy workload: 4 layers, d=128, 4 heads, SwiGLU 512, vocab 512,
# T=1024, window 256, chunk 64, last block's MLP fast, SGD lr 1e-2, fp32
TOY = dict(n_layers=4, d_model=128, n_heads=4, d_ff=512, vocab=512, window=256, chunk=64, n_fast=1, batch=1,
           rope_theta=1e4, rms_eps=1e-5, lr=1e-2, dtype="f32")
TOY_T = 1024

M125 = dict(n_layers=12, d_model=768, n_heads=12, d_ff=2048, vocab=32000, window=8192, chunk=1024, n_fast=3,
            batch=1, rope_theta=1e6, rms_eps=1e-5, lr=1e-3, dtype="bf16")
M125_T = 32768

M760 = dict(n_layers=24, d_model=1536, n_heads=16, d_ff=4096, vocab=32000, window=8192, chunk=1024, n_fast=6,
            batch=1, rope_theta=1e6, rms_eps=1e-5, lr=1e-3, dtype="bf16")
M760_T = 32768

M3B = dict(n_layers=32, d_model=2560, n_heads=20, d_ff=6912, vocab=32000, window=8192, chunk=1024, n_fast=8,
           batch=1, rope_theta=1e7, rms_eps=1e-5, lr=1e-3, dtype="bf16")
M3B_T = 131072

# matrix-core tile coverage: every GEMM of the engine meets the wide-tile shape rules
# (rows % 128, columns % 256, K % 64), and the per-chunk N = d GEMMs with K >= 1024 split K
MID = dict(n_layers=4, d_model=256, n_heads=2, d_ff=1024, vocab=1024, window=256, chunk=128, n_fast=2, batch=1,
           rope_theta=1e4, rms_eps=1e-5, lr=1e-2, dtype="bf16")
MID_T = 680

# d = 1024 (8 heads of 128): the per-chunk N = d products with K >= 1024 -- attention output
# projection (bf16 output) and its input gradient, down projection (residual add), the
# d(gate|up) -> d hidden product -- take the K-split path with the fused ordered sum
MIDK = dict(n_layers=2, d_model=1024, n_heads=8, d_ff=1024, vocab=512, window=256, chunk=128, n_fast=1, batch=1,
            rope_theta=1e4, rms_eps=1e-5, lr=1e-2, dtype="bf16")
MIDK_T = 256
# the same width with two fast blocks: the upper block's attention backward runs, its dO comes
# from the K-split W_o^T product (parts summed together with dO's per-head transpose) and the
# RMSNorm backward kernels sum K-split parts
MIDK2 = dict(MIDK, n_layers=3, n_fast=2)
