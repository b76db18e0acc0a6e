// Kernel launchers of the HIP path (gfx950).  All pointers are device pointers;
// every launcher enqueues on `s` and returns the launch status.
#pragma once
#include "common.h"

// ------------------------------------------------------------------ GEMM
// C[b][m][n] = sum_k A[b][m][k] * B[b][n][k]   (both operands K-contiguous,
// i.e. y = x W^T with W stored [out, in]), fp32 accumulation, then an
// epilogue applied per output element.
enum EpiKind {
  EPI_F32 = 0,     // c (fp32) = acc
  EPI_T = 1,       // c (T) = acc
  EPI_ADD_F32 = 2, // c (fp32) += acc           (residual stream)
  EPI_SWIGLU = 3,  // dual: act = silu(acc_g) * acc_u -> c (T); zg, zu (T) and act^T (T) optional
  EPI_SWIGLU_BWD = 4, // acc = d act: dz_g, dz_u -> c = dz (T, [m][2f]) and dz^T (T, [2f][ldt])
  EPI_SGD = 5,     // acc = gradient: master (fp32) -= lr * acc; shadow (T) and shadow^T (T) refreshed
  EPI_QKV_ROPE = 6, // acc = [q|k|v] row (N = 3 H hd, row m = token m % n of batch row m / n): RoPE of q, k
                    // at pos0 + m % n; q (q^T) and the ring slots of k (K^T), v, V^T written as in
                    // rope_qkv_f32in; the matrix-vector kernel (gemv_ok) or, with pair-interleaved
                    // q/k columns (rr.perm), the wide matrix-core tiles (gemm_mfma_fuses_qkv_rope)
  EPI_SWIGLU_IL = 7, // single operand with gate/up rows interleaved in groups of 32 (see swiglu_il_row):
                    // columns 64g..64g+31 are gate rows 32g.., 64g+32..64g+63 the matching up rows;
                    // outputs as EPI_SWIGLU with N = 2f (act, z_g, z_u [m][f], act^T)
  EPI_LM_CE = 8     // acc = logits z [m][v] of the lm_head (wide tiles, batch 1, N % 256 == 0): the
                    // softmax statistics of each row over each 256-column vocabulary tile (max m_t
                    // and sum of exp(z - m_t): ce_part [N/256][2][M]), exp(z - m_t) as T in c, and the
                    // target's logit z[m][y_m] in ce_zt [M] (targets tgt [B][ldtg], rows of rpb);
                    // ce_finalize turns c into dlogits in place
};

// row of the interleaved [gate; up] weight that holds row r (< 2f) of the stacked [W_gate; W_up]
__host__ __device__ inline int64_t swiglu_il_row(int64_t r, int64_t f) {
  const int64_t u = r >= f ? 1 : 0, rr = r - u * f;
  return 64 * (rr / 32) + 32 * u + rr % 32;
}

struct RopeRing {
  const float* cos_t;  // [max_pos][hd/2]
  const float* sin_t;
  int64_t pos0;        // absolute position of local row 0 (same for every batch row)
  int n;               // tokens per batch row in this call
  int H, hd, R;        // heads, head dim, ring slots
  void* q;             // [B][H][n][hd] T (rotated queries)
  void* qt;            // [B][H][hd][n] T or null
  void* kr;            // ring K [B][H][R][hd] T
  void* vr;            // ring V [B][H][R][hd] T
  void* vtr;           // ring V^T [B][H][hd][R] T
  void* ktr = nullptr; // ring K^T [B][H][hd][R] T, or null (needed only where the backward runs)
  // 1: the q and k columns of the [q|k|v] product are pair-interleaved within each head (the
  // weight rows are stored that way): column 2i of a head holds dim i, column 2i + 1 holds dim
  // i + hd/2, so a RoPE pair sits in adjacent columns; the v columns keep their natural order
  int perm = 0;
};
// weight row that holds natural row r (< 3 d) of [W_q; W_k; W_v] when the q and k rows are
// pair-interleaved within each head of hd rows (RopeRing::perm)
__host__ __device__ inline int64_t qkv_perm_row(int64_t r, int64_t d, int hd) {
  const int64_t part = r / d, c = r % d, h = c / hd, dim = c % hd, half = hd / 2;
  if (part == 2) return r;
  return part * d + h * hd + (dim < half ? 2 * dim : 2 * (dim - half) + 1);
}

struct Epi {
  int kind = EPI_F32;
  void* c = nullptr;
  int64_t ldc = 0, sc = 0;  // row stride and batch stride of c
  // SWIGLU / SWIGLU_BWD extras
  void* zg = nullptr;
  void* zu = nullptr;
  int64_t ldz = 0, sz = 0;
  void* t = nullptr;  // transposed output ([n][ldt] per batch)
  int64_t ldt = 0, st = 0;
  int f = 0;
  // SGD extras
  float* master = nullptr;
  int64_t ldm = 0, sm = 0;
  void* sh = nullptr;
  int64_t ldsh = 0, ssh = 0;
  void* shT = nullptr;
  int64_t ldshT = 0, sshT = 0;
  float lr = 0.f;
  int64_t il_f = 0;  // EPI_SGD: > 0 writes the row-major shadow with gate/up rows interleaved (f = il_f)
  RopeRing rr;
  // EPI_LM_CE extras
  const int32_t* tgt = nullptr;
  int64_t ldtg = 0;
  int rpb = 0;
  float* ce_part = nullptr;
  float* ce_zt = nullptr;
};

struct GemmArgs {
  const void* A = nullptr;
  int64_t lda = 0, sA = 0;
  const void* B = nullptr;
  int64_t ldb = 0, sB = 0;
  int M = 0, N = 0, K = 0, batch = 1;
  int64_t dual_off = 0;  // EPI_SWIGLU: the "up" operand starts dual_off rows after the "gate" rows
  Epi e;
  float* ws = nullptr;    // optional fp32 workspace: lets small-grid GEMMs split K (EPI_F32/EPI_T/EPI_ADD_F32)
  int64_t ws_floats = 0;
  bool defer = false;     // a K split leaves its fp32 parts in ws ([S][batch][M][N]) for the caller to sum
  // runs on a side stream beside latency-bound work: take the form that holds fewer resources per
  // CU (the fused-SGD 128 x 128 loop with three LDS stages: one block per CU instead of two)
  bool background = false;
  // input rows normalized inside the product (matrix-vector form only, see gemv_ok): with nx set,
  // input row m of batch b is RMSNorm(x; ng, neps) of the fp32 row x = nx + (b * M + m) * ldnx
  // (K elements), and A is not read
  const float* nx = nullptr;
  const float* ng = nullptr;
  int64_t ldnx = 0;
  float neps = 0.f;
};

hipError_t gemm_simt_f32(const GemmArgs& g, hipStream_t s);   // fp32 operands
hipError_t gemm_simt_bf16(const GemmArgs& g, hipStream_t s);  // bf16 operands, SIMT
hipError_t gemm_mfma_bf16(const GemmArgs& g, hipStream_t s);  // bf16 operands, MFMA
int gemm_mfma_splits(const GemmArgs& g, int* ks_out);          // split-K parts gemm_mfma_bf16 would use
// whether gemm_mfma_bf16 runs this EPI_QKV_ROPE product in one kernel (matrix-vector form for a
// handful of rows; wide tiles with rr.perm, d % 256 == 0, n, pos0 and R multiples of 8, hd % 4 == 0)
bool gemm_mfma_fuses_qkv_rope(const GemmArgs& g);
// M <= 8 rows per batch (decode), bf16 operands: one read of the weight rows per product;
// kinds EPI_F32, EPI_T, EPI_ADD_F32 and the SwiGLU kinds without z_g / z_u / act^T outputs,
// K % 8 == 0, 16-byte aligned operands and 8-element strides (gemv_ok); gemm_mfma_bf16 takes
// it by itself for such products; with g.nx it normalizes the input rows itself (the product
// of the RMSNorm of a handful of residual-stream rows, in one kernel)
bool gemv_ok(const GemmArgs& g);
hipError_t gemv_bf16(const GemmArgs& g, hipStream_t s);

// ------------------------------------------------------------------ elementwise
// Token arrays are [B][ld] int32 (row stride ld); activations are [B*n][d] rows.
template <typename T>
hipError_t embed_gather_ld(const int32_t* ids, int64_t ld, int B, int n, const T* E, int d, int V, float* h,
                           int* err, hipStream_t s);
// y = g * x / sqrt(mean(x^2) + eps) as T (optional), rstd (optional), transposed copy yT [B][d][ldT] (optional),
// a copy of x itself (optional)
template <typename T>
hipError_t rmsnorm_fwd(const float* x, int64_t M, int d, const float* g, float eps, T* y, float* rstd, T* yT,
                       int rows_per_batch, int64_t ldT, float* xcopy, hipStream_t s);
// out = resid + RMSNorm-backward(dy) (resid may be null, out may alias resid); outT: T copy of out (optional)
template <typename T>
hipError_t rmsnorm_bwd(const float* x, const float* rstd, int64_t M, int d, const float* g, const float* dy,
                       const float* resid, float* out, T* outT, hipStream_t s);
// consumers of a K-split GEMM's fp32 parts ([S][M][d], plane = M * d floats apart), summed
// in order in the row kernel: h += sum, then RMSNorm forward (as rmsnorm_fwd); RMSNorm
// backward with dy = sum (as rmsnorm_bwd).  d % 4 == 0, d <= 4096 (row_parts_ok), 16-byte
// aligned rows; hipErrorInvalidValue otherwise.
bool row_parts_ok(int d);
template <typename T>
hipError_t add_rmsnorm_fwd_parts(float* h, const float* parts, int S, int64_t plane, int64_t M, int d, const float* g,
                                 float eps, T* y, float* rstd, T* yT, int rows_per_batch, int64_t ldT, float* xcopy,
                                 hipStream_t s);
template <typename T>
hipError_t rmsnorm_bwd_parts(const float* x, const float* rstd, int64_t M, int d, const float* g, const float* parts,
                             int S, int64_t plane, const float* resid, float* out, T* outT, hipStream_t s);
// the sum of a K-split GEMM's fp32 parts ([S][M][d], plane = M * d floats apart, summed in
// order) as y [M][d] and, transposed per batch of rpb rows, yT [M/rpb][d][rpb] (bf16 only;
// d % 4 == 0, rpb % 8 == 0, 16-byte aligned; hipErrorInvalidValue otherwise)
template <typename T>
hipError_t parts_rows_t(const float* parts, int S, int64_t plane, int64_t M, int d, int rpb, T* y, T* yT,
                        hipStream_t s);
// fp32 [B*n][d] -> T copy [B*n][d] (optional) and transposed T [B][d][ldT] (optional)
template <typename T>
hipError_t convert_rows(const float* x, int64_t M, int d, T* y, T* yT, int rows_per_batch, int64_t ldT,
                        hipStream_t s);
// yT = y (T [M][d] in batches of rpb rows) transposed per batch into [d][ldT]; hipErrorNotSupported
// (nothing launched) for shapes the 16-byte transposing kernel does not take (fp32, rpb % 8 ...)
template <typename T>
hipError_t transpose_rows_checked(const T* y, T* yT, int64_t M, int d, int rpb, int64_t ldT, hipStream_t s);
hipError_t count_valid_ld(const int32_t* tgt, int64_t ld, int B, int n, int* nvalid, hipStream_t s);
// whether gemm_mfma_bf16 runs this lm_head product with the EPI_LM_CE epilogue
bool gemm_mfma_fuses_lm_ce(const GemmArgs& g);
// the rest of the vocabulary-tiled cross-entropy after an EPI_LM_CE product: per row, merges the
// tiles' (max, exp-sum) into logsumexp (online softmax), loss_tok[m] = lse - z[m][y] (0 for an
// ignored target), and turns the row of exp(z - m_t) in e into dlogits = (softmax - onehot) /
// nvalid in place (e == nullptr: the losses only)
template <typename T>
hipError_t ce_finalize(const float* part, const float* zt, int64_t M, int V, const int32_t* tgt, int64_t ld,
                       const int* nvalid, int rows_per_batch, float* loss_tok, T* e, int* err, hipStream_t s);
// cross-entropy of full logit rows: loss_tok[m] and dlogits = (softmax - onehot) / nvalid (T;
// dlogits == nullptr: the losses only)
template <typename T>
hipError_t ce_rows_ld(const float* logits, int64_t M, int V, const int32_t* tgt, int64_t ld, const int* nvalid,
                      int rows_per_batch, float* loss_tok, T* dlogits, int* err, hipStream_t s);
hipError_t reduce_loss(const float* loss_tok, const int* nvalid, int B, int n, float* loss_out, hipStream_t s);
hipError_t argmax_rows_ld(const float* logits, int B, int V, int32_t* out, int64_t ld_out, int32_t* out2,
                          int64_t ld_out2, hipStream_t s);
hipError_t copy_rows(const float* src, int64_t src_batch_stride, float* dst, int B, int n, int d, hipStream_t s);

// ------------------------------------------------------------------ attention
struct AttnArgs {
  const void* q;    // [B][H][n][hd] rotated queries
  const void* kr;   // ring K [B][H][R][hd]
  const void* vr;   // ring V [B][H][R][hd]
  const void* vtr;  // ring V^T [B][H][hd][R]
  void* o;          // [B*n][H*hd] output (T)
  float* lse;       // [B][H][n] or null
  int B, H, hd, n, R, window;
  int64_t pos0;     // absolute position of query 0
  float* ws = nullptr;  // optional fp32 workspace: lets small grids split the key range
  int64_t ws_floats = 0;
};
template <typename T>
hipError_t swa_fwd_simt(const AttnArgs& a, hipStream_t s);
hipError_t swa_fwd_mfma(const AttnArgs& a, hipStream_t s);  // bf16
int swa_fwd_mfma_splits(const AttnArgs& a);                  // key-range parts it would use
// fp32 workspace floats the split it prefers takes when the workspace does not limit it (0: none)
int64_t swa_fwd_mfma_ws_need(const AttnArgs& a);
// the two launches swa_fwd_mfma makes for one query per (row, head) (n == 1, hd 64 or 128):
// S blocks of 128 window keys per (row, head) (S = swa_decode_splits, 0 when that form does
// not apply; parts in ws when S > 1), then their merge into o and lse
int swa_decode_splits(const AttnArgs& a);
hipError_t swa_decode_blocks(const AttnArgs& a, int S, hipStream_t s);
hipError_t swa_decode_merge(const AttnArgs& a, int S, hipStream_t s);

struct AttnBwdArgs {
  const void* q;    // [B][H][n][hd]
  const void* qt;   // [B][H][hd][n]
  const void* kr;   // ring K
  const void* vr;   // ring V
  const void* vtr;  // ring V^T
  const void* ktr;  // ring K^T [B][H][hd][R] or null (then K^T tiles are transposed in LDS)
  const void* o;    // [B*n][H*hd] forward output (T)
  const void* dout; // [B*n][H*hd] gradient of the output (T)
  const float* lse; // [B][H][n]
  float* dvec;      // [B][H][n] scratch: rowsum(dO * O)
  float* dq;        // [B*n][H*hd] fp32 (rotated frame)
  float* dk;        // [B*n][H*hd] fp32 (rotated frame), in-chunk keys only
  float* dv;        // [B*n][H*hd] fp32
  void* dot;        // scratch for dO^T [B][H][hd][n] (T), or null (then dO^T is transposed in LDS)
  int B, H, hd, n, R, window;
  int64_t pos0;
  float* ws = nullptr;  // optional fp32 workspace: lets small grids split the key range of dq
  int64_t ws_floats = 0;
  bool dot_ready = false;  // dot already holds dO^T (written by the producer of dout)
};
template <typename T>
hipError_t swa_bwd_simt(const AttnBwdArgs& a, hipStream_t s);
// where a backward left dQ, dK, dV: sq (pkv) fp32 parts, plane floats apart, that the consumer
// sums in order from zero; a count of 1 means the arrays hold the finished sums
struct AttnBwdParts {
  const float* dq = nullptr;
  int sq = 1;
  const float* dk = nullptr;
  const float* dv = nullptr;
  int pkv = 1;
  int64_t plane = 0;
};
// bf16; with parts != null, split sums are not taken but described in *parts (dK/dV parts
// are placed after the dQ parts in ws)
hipError_t swa_bwd_mfma(const AttnBwdArgs& a, hipStream_t s, AttnBwdParts* parts = nullptr);

// RoPE of q, k from a fp32 [B*n][3d] projection; q -> rr.q (and rr.qt), k, v -> rings
hipError_t rope_qkv_f32in(const float* qkv, int B, const RopeRing& rr, int is_bf16, hipStream_t s);

// RoPE backward of dq, dk (fp32, rotated frame; each the ordered sum of its parts) and
// packing [dq | dk | dv] into T [B*n][3d]
template <typename T>
hipError_t rope_bwd_pack(const AttnBwdParts& g, const float* cos_t, const float* sin_t, int64_t pos0, int B, int n,
                         int H, int hd, T* dqkv, hipStream_t s);
