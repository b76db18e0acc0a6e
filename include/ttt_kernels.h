/*
 * ttt_kernels.h -- kernel-level entry points of the MI355X TTT-E2E library,
 * for unit tests and micro-benchmarks of single kernels.  All pointers are
 * DEVICE pointers owned by the caller, 16-byte aligned (as hipMalloc and torch
 * allocations are); every call is asynchronous on
 * `stream` (hipStream_t, may be NULL) and returns 0 or a negative TTT_E* code
 * (include/ttt.h) for a bad argument or a launch failure.  dtype is TTT_F32
 * (fp32 operands, SIMT kernels) or TTT_BF16 (bf16 operands, matrix cores).
 */
#ifndef TTT_KERNELS_H
#define TTT_KERNELS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every call takes an optional fp32 workspace (ws, ws_floats; NULL/0 for none): with
 * one, launches whose grid would under-fill the GPU split their reduction dimension
 * (K of a GEMM, the key range of attention) over more blocks and sum the parts in a
 * fixed order afterwards.  Calls that share a workspace must not overlap. */

/* C[m][n] = sum_k A[m][k] * B[n][k]  (y = x W^T with W stored [out, in]);
 * A [M][lda], B [N][ldb] row-major in dtype, C fp32 [M][ldc]. */
int tttk_gemm(int dtype, const void* A, int64_t lda, const void* B, int64_t ldb, float* C, int64_t ldc, int32_t M,
              int32_t N, int32_t K, float* ws, int64_t ws_floats, void* stream);

/* Sliding-window attention of n queries per (row, head) at absolute
 * positions pos0 .. pos0+n-1 over the key/value ring (page "TTT-E2E 如何让大模型
 * 边用边学", §4.2: the key/value cache holds only the window): query t sees
 * keys t-window < s <= t, s >= 0, key s at ring slot s mod R.
 * q [B][H][n][hd] (rotated), kr, vr [B][H][R][hd], vtr [B][H][hd][R] (V
 * transposed), o [B*n][H*hd], lse [B][H][n] fp32 (natural log) or NULL.
 * Scale 1/sqrt(hd).  Every ring slot must hold finite values: slots next to
 * a query's window are read with the tile and weighted by exactly zero. */
int tttk_swa_fwd(int dtype, const void* q, const void* kr, const void* vr, const void* vtr, void* o, float* lse,
                 int32_t B, int32_t H, int32_t hd, int32_t n, int32_t R, int32_t window, int64_t pos0, float* ws,
                 int64_t ws_floats, void* stream);

/* tttk_swa_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops, harnesses that forbid allocation): no workspace
 * argument, and the call allocates nothing.  Where tttk_swa_fwd would split the
 * key range (small grids, bf16), the parts go to a static fp32 array of the
 * library, TTTK_NOALLOC_SCRATCH_FLOATS floats (32 MiB) per device, which every
 * device the library runs on holds until the process ends.  Results are those of
 * tttk_swa_fwd with a workspace of that many floats.  TTT_EINVAL (nothing is
 * launched) when the split the call would take needs more floats than that, e.g.
 * one 1024-query chunk of 16 heads of 128 (4 parts of 2.1 M floats); the
 * smaller-split forms are not substituted.  Every call on a device shares that
 * device's array and leaves its parts there: calls that overlap on one device
 * (on different streams, or from different threads) race. */
#define TTTK_NOALLOC_SCRATCH_FLOATS (8 * 1024 * 1024)
int tttk_swa_fwd_noalloc(int dtype, const void* q, const void* kr, const void* vr, const void* vtr, void* o,
                         float* lse, int32_t B, int32_t H, int32_t hd, int32_t n, int32_t R, int32_t window,
                         int64_t pos0, void* stream);

/* Backward of tttk_swa_fwd for a chunk whose keys are ring slots of
 * positions pos0 .. pos0+n-1; keys before pos0 are constants (same page,
 * §8 Q1).  qt [B][H][hd][n] (q transposed), o, dout [B*n][H*hd] in dtype,
 * lse from the forward, dvec scratch [B][H][n]; outputs dq, dk, dv fp32
 * [B*n][H*hd] (dk, dv for the chunk's own keys only).  Optional (may be NULL):
 * ktr, the ring of keys transposed [B][H][hd][R], and dot, a scratch of
 * B*n*H*hd elements of dtype for dout transposed; with both (and n % 8 == 0)
 * the matrix-core kernels read transposed tiles instead of transposing in LDS. */
int tttk_swa_bwd(int dtype, const void* q, const void* qt, const void* kr, const void* vr, const void* vtr,
                 const void* ktr, const void* o, const void* dout, const float* lse, float* dvec, float* dq, float* dk,
                 float* dv, void* dot, int32_t B, int32_t H, int32_t hd, int32_t n, int32_t R, int32_t window,
                 int64_t pos0, float* ws, int64_t ws_floats, void* stream);

#ifdef __cplusplus
}
#endif
#endif
