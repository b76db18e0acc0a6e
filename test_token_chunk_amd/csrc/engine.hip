// Host engine of the TTT-E2E inner loop and the C ABI (include/ttt.h).
//
// Per chunk of b tokens (page "TTT-E2E 如何让大模型边用边学", §4.4): forward
// with the sliding window over the key/value rings, mean next-token
// cross-entropy, backward into the MLPs of the last n_fast blocks only (keys
// and values of earlier chunks are constants, same page §8 Q1), one SGD step
// on fp32 master weights, then the next chunk.
//
// Exact reordering used here: blocks 0 .. l0-1 and the attention half of
// block l0 (l0 = L - n_fast) never see the fast weights, so their forward for
// up to `lookahead` consecutive chunks runs as one large batch before the
// per-chunk loop over the upper blocks.  Every row of every kernel computes
// the same values as it would chunk by chunk.
#include <string.h>

#include <algorithm>
#include <cmath>
#include <string>
#include <type_traits>
#include <vector>

#include "kernels.h"
#include "ttt.h"

hipError_t refresh_shadows(const float* master, int rows, int cols, int batch, int64_t sm, void* sh, int64_t ssh,
                           void* shT, int64_t sshT, int is_bf16, int64_t il_f, hipStream_t s);

namespace {

ttt_alloc_fn g_alloc = nullptr;
ttt_free_fn g_free = nullptr;
void* g_user = nullptr;
thread_local std::string g_create_err;

enum Mode { FULL = 0, ATTN_ONLY = 1, MLP_ONLY = 2 };

struct LayerW {
  float* attn_norm = nullptr;
  float* mlp_norm = nullptr;
  void* wqkv = nullptr;   // [3d][d]
  void* wo = nullptr;     // [d][d]
  void* wgu = nullptr;    // [2f][d]  (frozen blocks)
  void* wd = nullptr;     // [d][f]   (frozen blocks)
  void* wqkvT = nullptr;  // [d][3d]  (blocks above l0)
  void* woT = nullptr;    // [d][d]   (blocks above l0)
  void* kr = nullptr;     // ring K [B][H][R][hd]
  void* vr = nullptr;     // ring V [B][H][R][hd]
  void* vtr = nullptr;    // ring V^T [B][H][hd][R]
  void* ktr = nullptr;    // ring K^T [B][H][hd][R] (bf16 blocks whose attention runs backward)
};

struct FastW {
  float* master = nullptr;  // [B][ W_gate f*d | W_up f*d | W_down d*f ] fp32
  void* wgu = nullptr;      // [B][2f][d]  shadow (T)
  void* wguT = nullptr;     // [B][d][2f]
  void* wd = nullptr;       // [B][d][f]
  void* wdT = nullptr;      // [B][f][d]
};

struct TopActs {
  float *h_in = nullptr, *rstd1 = nullptr, *h_mid = nullptr, *rstd2 = nullptr, *lse = nullptr;
  void *q = nullptr, *qt = nullptr, *o = nullptr, *mT = nullptr, *zg = nullptr, *zu = nullptr, *actT = nullptr;
  void *zg_s = nullptr, *zu_s = nullptr;  // static MLP pre-activations (dual MLP, blocks above l0)
};

}  // namespace

struct ttt_ctx {
  ttt_config cfg;
  int L, d, H, hd, f, V, k, b, Lq, l0, B, R, G;
  int n_steps = 1;  // SGD steps per chunk
  // static + dynamic MLP in every fast block: sw holds the frozen static MLPs in the fast
  // weights' layouts (one copy, all rows share it), fw the dynamic ones
  bool dual = false;
  bool bf16;
  size_t es;  // element size of T
  bool mfma = true;
  bool overlap = true;  // weight-gradient GEMMs on the side stream (TTT_NO_SIDE=1: on the main stream)
  bool il = false;  // gate/up rows interleaved for the single-operand SwiGLU GEMM (bf16 matrix-core path)
  // q/k rows of the forward W_qkv pair-interleaved within each head (RopeRing::perm), so the
  // projection's epilogue applies RoPE and writes q and the rings (bf16 matrix-core path)
  bool rope_perm = false;
  hipStream_t stream = nullptr;
  // second stream for the fused-SGD weight-gradient GEMMs, which only the next chunk depends on
  hipStream_t side = nullptr;
  hipEvent_t ev_m2s = nullptr, ev_s2m = nullptr;
  // the batched lower-block pass of the next lookahead group runs on its own stream beside the
  // current group's chunks, with its own scratch buffers and an h' buffer per group parity
  // (TTT_NO_BOTTOM_OVERLAP=1: in line on the main stream)
  bool bot_overlap = true;
  hipStream_t bstream = nullptr;
  hipEvent_t ev_bdone[2] = {nullptr, nullptr}, ev_cdone[2] = {nullptr, nullptr}, ev_c2b = nullptr;
  float *hb2 = nullptr, *b_qkvb = nullptr, *b_rstd = nullptr, *b_ws = nullptr;
  void *b_ub = nullptr, *b_qb = nullptr, *b_ob = nullptr, *b_actb = nullptr;
  ttt_free_fn free_fn = nullptr;
  void* free_user = nullptr;
  std::vector<void*> allocs;
  bool alloc_failed = false;

  std::vector<LayerW> lw;
  std::vector<FastW> fw;
  std::vector<FastW> sw;  // dual MLP: static MLPs of the fast blocks (batch 1, master kept)
  std::vector<TopActs> acts;
  void *embed = nullptr, *lm_head = nullptr, *lm_headT = nullptr;
  float* final_norm = nullptr;
  float *cos_t = nullptr, *sin_t = nullptr;
  float* fast_init = nullptr;  // [Lq][3fd]

  // work buffers
  float *hb = nullptr, *qkvb = nullptr, *rstd_tmp = nullptr;
  void *ub = nullptr, *qb = nullptr, *ob = nullptr, *actb = nullptr;
  float *htop = nullptr, *rstdf = nullptr, *logits = nullptr, *loss_tok = nullptr;
  float *ce_part = nullptr, *ce_zt = nullptr;  // vocabulary-tile softmax statistics, target logits
  void *hf = nullptr, *dlogits = nullptr;
  int* nvalid = nullptr;
  float *dh = nullptr, *tmpf = nullptr, *dq = nullptr, *dk = nullptr, *dv = nullptr, *dvec = nullptr;
  void *dyN = nullptr, *dz = nullptr, *dhT = nullptr, *dO = nullptr, *dOT = nullptr, *dqkv = nullptr;
  void* dzT_s = nullptr;  // dual MLP: transposed dz of the static MLP's backward (written, never read)
  // dual MLP: the static MLP's activations when both MLPs read the residual stream directly
  // (decode, norm inside the products): [B * chunk][f]
  void* act_s = nullptr;
  std::vector<void*> dyT, dzT;  // per fast block: inputs of its weight-gradient GEMMs (side stream)
  int* err_dev = nullptr;
  float* ws = nullptr;  // split-K / split-key workspace (used by one launch at a time)
  int64_t ws_floats = 0;        // what GEMM splits and the attention forward may use
  int64_t ws_alloc_floats = 0;  // allocated: also dQ and dK/dV parts of the attention backward side by side
  int32_t* d_tok = nullptr;
  int64_t d_tok_cap = 0;
  float* d_loss = nullptr;
  int64_t d_loss_cap = 0;
  float* loss_later = nullptr;  // [B]: losses of a chunk's steps after the first (not reported)

  int64_t pos = 0;
  bool poisoned = false;
  std::string err;
  float* pending_loss = nullptr;  // device losses of async work, checked by ttt_sync
  int64_t pending_n = 0;
  // K-split parts of the last residual-stream GEMM left in ws, summed into the residual
  // stream by the next RMSNorm forward (0: none)
  int pend_parts = 0;

  // per-kernel-class device time (HIP events around each launch) while profiling is on
  uint32_t prof = 0;  // bit i: time launches of class i
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
  struct ProfRec {
    int cls;
    double flops;
    hipEvent_t a, b;
  };
  std::vector<ProfRec> prof_recs;

  // the streams and events this context created (null ones skipped)
  void destroy_streams() {
    for (hipEvent_t* e : {&ev_m2s, &ev_s2m, &ev_c2b, &ev_bdone[0], &ev_bdone[1], &ev_cdone[0], &ev_cdone[1]})
      if (*e) {
        (void)hipEventDestroy(*e);
        *e = nullptr;
      }
    for (hipStream_t* st : {&side, &bstream})
      if (*st) {
        (void)hipStreamDestroy(*st);
        *st = nullptr;
      }
  }

  void* alloc(size_t bytes) {
    if (bytes == 0) bytes = 256;
    void* p = nullptr;
    if (g_alloc) {
      p = g_alloc(bytes, g_user);
    } else if (hipMalloc(&p, bytes) != hipSuccess) {
      p = nullptr;
    }
    if (!p) {
      alloc_failed = true;
      return nullptr;
    }
    allocs.push_back(p);
    return p;
  }
  void release_all() {
    for (void* p : allocs) {
      if (free_fn)
        free_fn(p, free_user);
      else
        (void)hipFree(p);
    }
    allocs.clear();
  }
};

namespace {

int fail(ttt_ctx* c, int code, const std::string& msg) {
  c->err = msg;
  if (code == TTT_EDEVICE || code == TTT_ENONFINITE || code == TTT_ENOMEM) c->poisoned = true;
  return code;
}

#define CK(expr)                                                                                   \
  do {                                                                                             \
    hipError_t e_ = (expr);                                                                        \
    if (e_ != hipSuccess) return fail(c, TTT_EDEVICE, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

// ------------------------------------------------------------------ profiling
// Classes: GEMMs without split by epilogue kind (EPI_F32 .. EPI_SGD; one kernel each),
// split-K GEMMs (kernel + ordered reduce), attention forward (one kernel), split-key
// attention forward (kernel + combine), attention backward (dvec + dq + dk/dv)
enum {
  PC_GEMM_SPLITK = 6, PC_SWA_FWD = 7, PC_SWA_FWD_SPLIT = 8, PC_SWA_BWD = 9, PC_SWA_DEC = 10, PC_QKV_ROPE = 11,
  PC_LM_CE = 12, PC_N = 13
};

hipEvent_t next_event(ttt_ctx* c) {
  if (c->ev_used == c->ev_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    c->ev_pool.push_back(e);
  }
  return c->ev_pool[c->ev_used++];
}

// run `launch` (returns hipError_t); with profiling on, bracket it with events
template <typename F>
hipError_t timed(ttt_ctx* c, int cls, double flops, hipStream_t st, F&& launch) {
  if (!(c->prof & (1u << cls))) return launch();
  hipEvent_t a = next_event(c), b = next_event(c);
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, st);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, st);
  c->prof_recs.push_back({cls, flops, a, b});
  return e;
}

double attn_pairs(const ttt_ctx* c, int n, int64_t p0) {
  double s = 0;
  for (int t = 0; t < n; ++t) s += (double)std::min<int64_t>(c->k, p0 + t + 1);
  return s;
}

// ------------------------------------------------------------------ dispatch

template <typename T>
struct Ops;

double gemm_flops(const GemmArgs& g) {
  return 2.0 * g.M * g.N * g.K * g.batch * (g.e.kind == EPI_SWIGLU ? 2 : 1);
}

template <>
struct Ops<float> {
  static hipError_t gemm(ttt_ctx* c, const GemmArgs& g, hipStream_t st = nullptr) {
    if (!st) st = c->stream;
    return timed(c, g.e.kind, gemm_flops(g), st, [&] { return gemm_simt_f32(g, st); });
  }
  static hipError_t gemm_parts(ttt_ctx* c, const GemmArgs& g, int rpb, int& S) {
    (void)rpb;
    S = 1;
    return gemm(c, g);
  }
  static hipError_t fwd(ttt_ctx* c, const AttnArgs& a) {
    double fl = 4.0 * a.hd * a.H * a.B * attn_pairs(c, a.n, a.pos0);
    return timed(c, PC_SWA_FWD, fl, c->stream, [&] { return swa_fwd_simt<float>(a, c->stream); });
  }
  static hipError_t bwd(ttt_ctx* c, const AttnBwdArgs& a, AttnBwdParts* parts) {
    *parts = AttnBwdParts{a.dq, 1, a.dk, a.dv, 1, (int64_t)a.B * a.n * a.H * a.hd};
    double fl = 4.0 * a.hd * a.H * a.B * (attn_pairs(c, a.n, a.pos0) + 0.5 * a.n * (a.n + 1.0));
    return timed(c, PC_SWA_BWD, fl, c->stream, [&] { return swa_bwd_simt<float>(a, c->stream); });
  }
};

// the bf16 kernels may use the context's workspace to split under-filled grids
template <>
struct Ops<bf16> {
  // st: the side stream (no workspace there: the split workspace belongs to the main stream)
  static hipError_t gemm(ttt_ctx* c, const GemmArgs& g0, hipStream_t st = nullptr) {
    if (c->pend_parts && !st) return hipErrorIllegalState;  // the workspace still holds parts to sum
    GemmArgs g = g0;
    g.ws = st ? nullptr : c->ws;
    g.ws_floats = st ? 0 : c->ws_floats;
    if (!st) st = c->stream;
    // one SwiGLU class; the products with the RoPE and cross-entropy epilogues have their own
    const int kind_cls = g.e.kind == EPI_SWIGLU_IL  ? (int)EPI_SWIGLU
                         : g.e.kind == EPI_QKV_ROPE ? (int)PC_QKV_ROPE
                         : g.e.kind == EPI_LM_CE    ? (int)PC_LM_CE
                                                    : g.e.kind;
    const int cls = (c->mfma && gemm_mfma_splits(g, nullptr) > 1) ? PC_GEMM_SPLITK : kind_cls;
    return timed(c, cls, gemm_flops(g), st,
                 [&] { return c->mfma ? gemm_mfma_bf16(g, st) : gemm_simt_bf16(g, st); });
  }
  // a GEMM whose fp32 result [M][N] (batches of rpb rows) feeds a row kernel next: if it
  // splits K, its S parts stay in the workspace for that kernel to sum (S > 1); otherwise it
  // writes g.e.c (S = 1).  The consumers' transposed copies move 8-row groups into rows of
  // rpb (dO^T) or of the chunk length b (the MLP input of the weight gradients): both % 8 == 0.
  static hipError_t gemm_parts(ttt_ctx* c, const GemmArgs& g0, int rpb, int& S) {
    GemmArgs g = g0;
    g.ws = c->ws;
    g.ws_floats = c->ws_floats;
    S = (c->mfma && rpb % 8 == 0 && c->b % 8 == 0 && (int64_t)g.M * g.batch >= 128 && row_parts_ok(g.N) &&
         g.e.ldc == g.N &&
         g.e.sc == (g.batch > 1 ? (int64_t)g.M * g.N : g.e.sc))
            ? gemm_mfma_splits(g, nullptr)
            : 1;
    g.defer = S > 1;
    return gemm(c, g);
  }
  static hipError_t fwd(ttt_ctx* c, const AttnArgs& a0) {
    if (c->pend_parts) return hipErrorIllegalState;
    AttnArgs a = a0;
    a.ws = c->ws;
    a.ws_floats = c->ws_floats;
    double fl = 4.0 * a.hd * a.H * a.B * attn_pairs(c, a.n, a.pos0);
    if (c->mfma) {
      // one query per head (decode): the window-block kernel is timed on its own, the merge after it
      if (const int S = swa_decode_splits(a)) {
        hipError_t e = timed(c, PC_SWA_DEC, fl, c->stream,
                             [&] { return swa_decode_blocks(a, S, c->stream); });
        return e != hipSuccess ? e : swa_decode_merge(a, S, c->stream);
      }
    }
    const int cls = (c->mfma && swa_fwd_mfma_splits(a) > 1) ? PC_SWA_FWD_SPLIT : PC_SWA_FWD;
    return timed(c, cls, fl, c->stream,
                 [&] { return c->mfma ? swa_fwd_mfma(a, c->stream) : swa_fwd_simt<bf16>(a, c->stream); });
  }
  // the split sums of dQ, dK, dV are left to the consumer as described in *parts
  static hipError_t bwd(ttt_ctx* c, const AttnBwdArgs& a0, AttnBwdParts* parts) {
    if (c->pend_parts) return hipErrorIllegalState;
    AttnBwdArgs a = a0;
    a.ws = c->ws;
    a.ws_floats = c->ws_alloc_floats;
    *parts = AttnBwdParts{a.dq, 1, a.dk, a.dv, 1, (int64_t)a.B * a.n * a.H * a.hd};
    double fl = 4.0 * a.hd * a.H * a.B * (attn_pairs(c, a.n, a.pos0) + 0.5 * a.n * (a.n + 1.0));
    return timed(c, PC_SWA_BWD, fl, c->stream,
                 [&] { return c->mfma ? swa_bwd_mfma(a, c->stream, parts) : swa_bwd_simt<bf16>(a, c->stream); });
  }
};

GemmArgs mk(const void* A, int64_t lda, const void* B, int64_t ldb, int M, int N, int K) {
  GemmArgs g;
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.M = M;
  g.N = N;
  g.K = K;
  return g;
}

template <typename T>
T* tp(void* p, int64_t off = 0) {
  return (T*)p + off;
}

// forward of block l over n tokens per row at positions [p0, p0+n); h is the
// fp32 residual stream [B*n][d], updated in place.
// RMSNorm forward of the residual stream h [M][d]; parts of a preceding K-split GEMM that
// are still in the workspace are added to h first (in order, in the same kernel)
template <typename T>
hipError_t norm_fwd(ttt_ctx* c, float* h, int64_t M, const float* g, T* y, float* rstd, T* yT, int rpb, int64_t ldT,
                    float* xcopy) {
  const float eps = (float)c->cfg.rms_eps;
  if (c->pend_parts > 1) {
    const int S = c->pend_parts;
    c->pend_parts = 0;
    return add_rmsnorm_fwd_parts<T>(h, c->ws, S, M * c->d, M, c->d, g, eps, y, rstd, yT, rpb, ldT, xcopy, c->stream);
  }
  return rmsnorm_fwd<T>(h, M, c->d, g, eps, y, rstd, yT, rpb, ldT, xcopy, c->stream);
}

// RMSNorm backward with dy from a GEMM that may have left S > 1 K-split parts in the workspace
template <typename T>
hipError_t norm_bwd(ttt_ctx* c, int S, const float* x, const float* rstd, int64_t M, const float* g, const float* dy,
                    const float* resid, float* out, T* outT) {
  if (S > 1) return rmsnorm_bwd_parts<T>(x, rstd, M, c->d, g, c->ws, S, M * c->d, resid, out, outT, c->stream);
  return rmsnorm_bwd<T>(x, rstd, M, c->d, g, dy, resid, out, outT, c->stream);
}

// lm_head over M rows of x (rows of rpb per batch row, targets tgt [B][ld]) and the chunk's
// cross-entropy per row into loss_tok, with dlogits (T [M][V]) when dl != nullptr; nvalid must
// be counted.  bf16 matrix cores: one GEMM whose epilogue keeps the softmax statistics of each
// 256-column vocabulary tile and exp(z - tile max) in dl (or the logits buffer), then a per-row
// merge that writes the loss and rescales dl in place; otherwise fp32 logits and a row pass.
template <typename T>
hipError_t lmhead_ce(ttt_ctx* c, const void* x, int64_t M, const int32_t* tgt, int64_t ld, int rpb, T* dl) {
  const int d = c->d, V = c->V;
  GemmArgs gl = mk(x, d, c->lm_head, d, (int)M, V, d);
  if (c->mfma && c->bf16) {
    GemmArgs gf = gl;
    gf.e.kind = EPI_LM_CE;
    gf.e.c = dl ? (void*)dl : c->logits;  // exp(z - m_t) as bf16 (the fp32 logits buffer is big enough)
    gf.e.ldc = V;
    gf.e.tgt = tgt;
    gf.e.ldtg = ld;
    gf.e.rpb = rpb;
    gf.e.ce_part = c->ce_part;
    gf.e.ce_zt = c->ce_zt;
    if (gemm_mfma_fuses_lm_ce(gf)) {
      hipError_t e = Ops<T>::gemm(c, gf);
      if (e != hipSuccess) return e;
      return ce_finalize<T>(c->ce_part, c->ce_zt, M, V, tgt, ld, c->nvalid, rpb, c->loss_tok, dl, c->err_dev,
                            c->stream);
    }
  }
  gl.e.kind = EPI_F32;
  gl.e.c = c->logits;
  gl.e.ldc = V;
  hipError_t e = Ops<T>::gemm(c, gl);
  if (e != hipSuccess) return e;
  return ce_rows_ld<T>(c->logits, M, V, tgt, ld, c->nvalid, rpb, c->loss_tok, dl, c->err_dev, c->stream);
}

// A product whose input rows are RMSNorm(h; gain): with a handful of rows (decode) and nothing
// of the norm to keep for a backward, the matrix-vector kernel normalizes the fp32 rows itself;
// returns whether g now reads h that way (else g is unchanged and the norm must run first).
bool norm_in_product(ttt_ctx* c, const TopActs* sv, GemmArgs& g, const float* h, const float* gain) {
  static int off = -1;  // tuning switch TTT_NO_NORM_IN_PRODUCT=1: separate norm kernels
  if (off < 0) {
    const char* e = getenv("TTT_NO_NORM_IN_PRODUCT");
    off = e && e[0] == '1' ? 1 : 0;
  }
  if (off || sv || !c->bf16 || !c->mfma || c->pend_parts) return false;
  GemmArgs t = g;
  t.A = nullptr;
  t.nx = h;
  t.ng = gain;
  t.ldnx = c->d;
  t.neps = (float)c->cfg.rms_eps;
  if (!gemv_ok(t)) return false;
  g = t;
  return true;
}

template <typename T>
int layer_fwd(ttt_ctx* c, int l, float* h, int n, int64_t p0, int mode, TopActs* sv) {
  const int B = c->B, d = c->d, f = c->f;
  const int64_t M = (int64_t)B * n;
  const LayerW& w = c->lw[l];
  if (mode != MLP_ONLY) {
    GemmArgs g = mk(c->ub, d, w.wqkv, d, (int)M, 3 * d, d);
    g.e.kind = EPI_F32;
    g.e.c = c->qkvb;
    g.e.ldc = 3 * d;
    RopeRing rr;
    rr.cos_t = c->cos_t;
    rr.sin_t = c->sin_t;
    rr.pos0 = p0;
    rr.n = n;
    rr.H = c->H;
    rr.hd = c->hd;
    rr.R = c->R;
    rr.q = sv ? sv->q : c->qb;
    rr.qt = sv ? sv->qt : nullptr;
    rr.kr = w.kr;
    rr.vr = w.vr;
    rr.vtr = w.vtr;
    rr.ktr = w.ktr;
    rr.perm = c->rope_perm ? 1 : 0;
    // RoPE and the ring writes in the product's epilogue: the matrix-vector kernel for a handful
    // of rows (decode), the wide matrix-core tiles for chunks whose shape allows it; otherwise
    // an fp32 product and a separate RoPE pass
    GemmArgs gr = g;
    gr.e.kind = EPI_QKV_ROPE;
    gr.e.rr = rr;
    // (decode: the attention norm inside the product)
    if (!norm_in_product(c, sv, gr, h, w.attn_norm))
      CK(norm_fwd<T>(c, h, M, w.attn_norm, tp<T>(c->ub), sv ? sv->rstd1 : c->rstd_tmp, (T*)nullptr, n, 0,
                     sv ? sv->h_in : nullptr));
    if (c->mfma && c->bf16 && (gr.nx || gemm_mfma_fuses_qkv_rope(gr))) {
      CK(Ops<T>::gemm(c, gr));
    } else {
      CK(Ops<T>::gemm(c, g));
      CK(rope_qkv_f32in(c->qkvb, B, rr, c->bf16 ? 1 : 0, c->stream));
    }
    AttnArgs a;
    a.q = rr.q;
    a.kr = w.kr;
    a.vr = w.vr;
    a.vtr = w.vtr;
    a.o = sv ? sv->o : c->ob;
    a.lse = sv ? sv->lse : nullptr;
    a.B = B;
    a.H = c->H;
    a.hd = c->hd;
    a.n = n;
    a.R = c->R;
    a.window = c->k;
    a.pos0 = p0;
    CK(Ops<T>::fwd(c, a));
    GemmArgs go = mk(a.o, d, w.wo, d, (int)M, d, d);
    go.e.kind = EPI_ADD_F32;
    go.e.c = h;
    go.e.ldc = d;
    if (mode == ATTN_ONLY) {
      CK(Ops<T>::gemm(c, go));
      return TTT_OK;
    }
    int So = 1;  // the MLP norm below sums a K split of the output projection
    CK(Ops<T>::gemm_parts(c, go, n, So));
    c->pend_parts = So > 1 ? So : 0;
  }
  // the MLP products that read the normed rows m: the static and the dynamic MLP (fast blocks,
  // dual MLP), the fast MLP (batched over rows: each row has its own weights) or the frozen one
  const bool fast = l >= c->l0;
  GemmArgs gs, gu;
  if (fast && c->dual) {
    const FastW& st = c->sw[l - c->l0];
    gs = mk(c->ub, d, st.wgu, d, (int)M, c->il ? 2 * f : f, d);
    gs.dual_off = c->il ? 0 : f;
    gs.e.kind = c->il ? EPI_SWIGLU_IL : EPI_SWIGLU;
    gs.e.c = c->actb;
    gs.e.ldc = f;
    if (sv && sv->zg_s) {  // pre-activations for the backward of blocks above l0
      gs.e.zg = sv->zg_s;
      gs.e.zu = sv->zu_s;
      gs.e.ldz = f;
    }
  }
  if (fast) {
    const FastW& fw = c->fw[l - c->l0];
    gu = mk(c->ub, d, fw.wgu, d, n, c->il ? 2 * f : f, d);
    gu.batch = B;
    gu.sA = (int64_t)n * d;
    gu.sB = 2LL * f * d;
    gu.dual_off = c->il ? 0 : f;
    gu.e.kind = c->il ? EPI_SWIGLU_IL : EPI_SWIGLU;
    gu.e.c = c->actb;
    gu.e.ldc = f;
    gu.e.sc = (int64_t)n * f;
    if (sv) {
      gu.e.zg = sv->zg;
      gu.e.zu = sv->zu;
      gu.e.ldz = f;
      gu.e.sz = (int64_t)n * f;
      gu.e.t = sv->actT;
      gu.e.ldt = c->b;
      gu.e.st = (int64_t)f * c->b;
    }
  } else {
    gu = mk(c->ub, d, w.wgu, d, (int)M, c->il ? 2 * f : f, d);
    gu.dual_off = c->il ? 0 : f;
    gu.e.kind = c->il ? EPI_SWIGLU_IL : EPI_SWIGLU;
    gu.e.c = c->actb;
    gu.e.ldc = f;
  }
  // (decode: the MLP norm inside those products when all of them take it)
  bool in_product = false;
  {
    GemmArgs ts = gs, tu = gu;
    const bool both = fast && c->dual;
    if (norm_in_product(c, sv, tu, h, w.mlp_norm) && (!both || norm_in_product(c, sv, ts, h, w.mlp_norm))) {
      gu = tu;
      gs = ts;
      in_product = true;
    } else {
      CK(norm_fwd<T>(c, h, M, w.mlp_norm, tp<T>(c->ub), sv ? sv->rstd2 : c->rstd_tmp,
                     sv ? tp<T>(sv->mT) : (T*)nullptr, n, c->b, sv ? sv->h_mid : nullptr));
    }
  }
  if (fast) {
    if (c->dual) {
      // the frozen static MLP on the same normed input, all rows at once; its output is added to
      // the residual stream after the dynamic MLP's gate/up product has read that stream (when
      // the norm runs inside the products, both read h itself: the static activations go to
      // their own buffer), else right away
      const FastW& st = c->sw[l - c->l0];
      GemmArgs gds = mk(in_product ? c->act_s : c->actb, f, st.wd, f, (int)M, d, f);
      gds.e.kind = EPI_ADD_F32;
      gds.e.c = h;
      gds.e.ldc = d;
      if (in_product) {
        gs.e.c = c->act_s;
        CK(Ops<T>::gemm(c, gs));
        CK(Ops<T>::gemm(c, gu));
        CK(Ops<T>::gemm(c, gds));
      } else {
        CK(Ops<T>::gemm(c, gs));
        CK(Ops<T>::gemm(c, gds));
        CK(Ops<T>::gemm(c, gu));
      }
    } else {
      CK(Ops<T>::gemm(c, gu));
    }
    const FastW& fw = c->fw[l - c->l0];
    GemmArgs gd = mk(c->actb, f, fw.wd, f, n, d, f);
    gd.batch = B;
    gd.sA = (int64_t)n * f;
    gd.sB = (int64_t)d * f;
    gd.e.kind = EPI_ADD_F32;
    gd.e.c = h;
    gd.e.ldc = d;
    gd.e.sc = (int64_t)n * d;
    int Sd = 1;  // summed by the next norm forward (next block's attention norm or the final norm)
    CK(Ops<T>::gemm_parts(c, gd, n, Sd));
    c->pend_parts = Sd > 1 ? Sd : 0;
  } else {
    CK(Ops<T>::gemm(c, gu));
    GemmArgs gd = mk(c->actb, f, w.wd, f, (int)M, d, f);
    gd.e.kind = EPI_ADD_F32;
    gd.e.c = h;
    gd.e.ldc = d;
    int Sd = 1;
    CK(Ops<T>::gemm_parts(c, gd, n, Sd));
    c->pend_parts = Sd > 1 ? Sd : 0;
  }
  return TTT_OK;
}

// fast-weight-independent forward of g tokens per row: blocks 0..l0-1 and the
// attention half of block l0; leaves h' of block l0 in c->hb ([B][g][d]).
template <typename T>
int bottom_pass(ttt_ctx* c, const int32_t* tok, int64_t ld, int g, int64_t p0) {
  CK(embed_gather_ld<T>(tok, ld, c->B, g, tp<T>(c->embed), c->d, c->V, c->hb, c->err_dev, c->stream));
  for (int l = 0; l < c->l0; ++l) {
    int rc = layer_fwd<T>(c, l, c->hb, g, p0, FULL, nullptr);
    if (rc) return rc;
  }
  return layer_fwd<T>(c, c->l0, c->hb, g, p0, ATTN_ONLY, nullptr);
}

// upper blocks of one chunk: forward, loss, backward, SGD.  hsrc: h' of block
// l0 for this chunk (row r at hsrc + r*hsrc_bs).
template <typename T>
int top_chunk(ttt_ctx* c, const int32_t* tgt, int64_t ld, const float* hsrc, int64_t hsrc_bs, int n, int64_t p0,
              float* loss_dev) {
  const int B = c->B, d = c->d, f = c->f, V = c->V, b = c->b;
  const int64_t M = (int64_t)B * n;
  CK(copy_rows(hsrc, hsrc_bs, c->htop, B, n, d, c->stream));
  int rc = layer_fwd<T>(c, c->l0, c->htop, n, p0, MLP_ONLY, &c->acts[0]);
  if (rc) return rc;
  for (int j = 1; j < c->Lq; ++j) {
    rc = layer_fwd<T>(c, c->l0 + j, c->htop, n, p0, FULL, &c->acts[j]);
    if (rc) return rc;
  }
  CK(norm_fwd<T>(c, c->htop, M, c->final_norm, tp<T>(c->hf), c->rstdf, (T*)nullptr, n, 0, nullptr));
  CK(count_valid_ld(tgt, ld, B, n, c->nvalid, c->stream));
  CK(lmhead_ce<T>(c, c->hf, M, tgt, ld, n, tp<T>(c->dlogits)));
  CK(reduce_loss(c->loss_tok, c->nvalid, B, n, loss_dev, c->stream));

  // backward
  GemmArgs gx = mk(c->dlogits, V, c->lm_headT, V, (int)M, d, V);
  gx.e.kind = EPI_F32;
  gx.e.c = c->tmpf;
  gx.e.ldc = d;
  int Sx = 1;
  CK(Ops<T>::gemm_parts(c, gx, n, Sx));
  // (dh and its T copy dy for the first block's products)
  CK(norm_bwd<T>(c, Sx, c->htop, c->rstdf, M, c->final_norm, c->tmpf, nullptr, c->dh, tp<T>(c->dyN)));
  const float lr = c->cfg.lr;
  const int64_t fsz = 3LL * f * d;
  for (int j = c->Lq - 1; j >= 0; --j) {
    const int l = c->l0 + j;
    TopActs& a = c->acts[j];
    FastW& w = c->fw[j];
    void* dyT = c->dyT[j];
    void* dzT = c->dzT[j];
    // dy in T (written by the norm backward that produced dh) and transposed for the weight gradients
    const hipError_t te = transpose_rows_checked<T>(tp<T>(c->dyN), tp<T>(dyT), M, d, n, b, c->stream);
    if (te == hipErrorNotSupported)
      CK(convert_rows<T>(c->dh, M, d, tp<T>(c->dyN), tp<T>(dyT), n, b, c->stream));
    else
      CK(te);
    // d act = dy W_down  ->  dz_g, dz_u
    GemmArgs g1 = mk(c->dyN, d, w.wdT, d, n, f, d);
    g1.batch = B;
    g1.sA = (int64_t)n * d;
    g1.sB = (int64_t)f * d;
    g1.e.kind = EPI_SWIGLU_BWD;
    g1.e.zg = a.zg;
    g1.e.zu = a.zu;
    g1.e.ldz = f;
    g1.e.sz = (int64_t)n * f;
    g1.e.c = c->dz;
    g1.e.ldc = 2 * f;
    g1.e.sc = (int64_t)n * 2 * f;
    g1.e.t = dzT;
    g1.e.ldt = b;
    g1.e.st = 2LL * f * b;
    g1.e.f = f;
    CK(Ops<T>::gemm(c, g1));
    int S3 = 1;   // K-split parts of dm left for the MLP norm's backward
    if (j > 0) {  // dm = dz_g W_gate + dz_u W_up  (before W_gate/W_up change)
      GemmArgs g3 = mk(c->dz, 2 * f, w.wguT, 2 * f, n, d, 2 * f);
      g3.batch = B;
      g3.sA = (int64_t)n * 2 * f;
      g3.sB = 2LL * d * f;
      g3.e.kind = EPI_F32;
      g3.e.c = c->tmpf;
      g3.e.ldc = d;
      g3.e.sc = (int64_t)n * d;
      if (c->dual)
        CK(Ops<T>::gemm(c, g3));  // the static MLP's part is added to tmpf below
      else
        CK(Ops<T>::gemm_parts(c, g3, n, S3));
    }
    // The weight gradients of this block with the fused SGD step run on the side stream,
    // overlapping the rest of the backward: their inputs (dy^T, dz^T of this block, act^T,
    // m^T) stay untouched until the next chunk, and the GEMMs above that read the old
    // W_down^T and W_gu^T have been enqueued before them.
    // (the lowest block's update is the chunk's critical path: it runs on the main stream,
    // next to the side stream's remaining updates)
    const bool on_side = c->overlap && j > 0;
    hipStream_t sg = on_side ? c->side : c->stream;
    if (on_side) {
      CK(hipEventRecord(c->ev_m2s, c->stream));
      CK(hipStreamWaitEvent(c->side, c->ev_m2s, 0));
    }
    // dW_down = dy^T act, fused SGD step on W_down
    GemmArgs g2 = mk(dyT, b, a.actT, b, d, f, n);
    g2.batch = B;
    g2.sA = (int64_t)d * b;
    g2.sB = (int64_t)f * b;
    g2.e.kind = EPI_SGD;
    g2.e.master = w.master + 2LL * f * d;
    g2.e.ldm = f;
    g2.e.sm = fsz;
    g2.e.sh = w.wd;
    g2.e.ldsh = f;
    g2.e.ssh = (int64_t)d * f;
    g2.e.shT = w.wdT;
    g2.e.ldshT = d;
    g2.e.sshT = (int64_t)f * d;
    g2.e.lr = lr;
    g2.background = on_side;
    CK(Ops<T>::gemm(c, g2, sg));
    // [dW_gate; dW_up] = dz^T m, fused SGD step
    GemmArgs g4 = mk(dzT, b, a.mT, b, 2 * f, d, n);
    g4.batch = B;
    g4.sA = 2LL * f * b;
    g4.sB = (int64_t)d * b;
    g4.e.kind = EPI_SGD;
    g4.e.master = w.master;
    g4.e.ldm = d;
    g4.e.sm = fsz;
    g4.e.sh = w.wgu;
    g4.e.ldsh = d;
    g4.e.ssh = 2LL * f * d;
    g4.e.shT = w.wguT;
    g4.e.ldshT = 2 * f;
    g4.e.sshT = 2LL * d * f;
    g4.e.lr = lr;
    g4.e.il_f = c->il ? f : 0;
    g4.background = on_side;
    CK(Ops<T>::gemm(c, g4, sg));
    if (j == 0) break;
    if (c->dual) {
      // the frozen static MLP passes its input gradient on as well: d act_s = dy W_down_s ->
      // dz_s, then dm += dz_s,g W_gate_s + dz_s,u W_up_s (c->dz is free again: the dynamic dm
      // product that read it is ahead on this stream, the SGD products read dzT)
      const FastW& st = c->sw[j];
      GemmArgs s1 = mk(c->dyN, d, st.wdT, d, (int)M, f, d);
      s1.e.kind = EPI_SWIGLU_BWD;
      s1.e.zg = a.zg_s;
      s1.e.zu = a.zu_s;
      s1.e.ldz = f;
      s1.e.c = c->dz;
      s1.e.ldc = 2 * f;
      s1.e.t = c->dzT_s;
      s1.e.ldt = (int64_t)M;
      s1.e.f = f;
      CK(Ops<T>::gemm(c, s1));
      GemmArgs s3 = mk(c->dz, 2 * f, st.wguT, 2 * f, (int)M, d, 2 * f);
      s3.e.kind = EPI_ADD_F32;
      s3.e.c = c->tmpf;
      s3.e.ldc = d;
      CK(Ops<T>::gemm(c, s3));
    }
    const LayerW& lw = c->lw[l];
    // through the MLP norm and the residual: dh <- d h_mid
    CK(norm_bwd<T>(c, S3, a.h_mid, a.rstd2, M, lw.mlp_norm, c->tmpf, c->dh, c->dh, tp<T>(c->dhT)));
    // attention output projection
    GemmArgs g5 = mk(c->dhT, d, lw.woT, d, (int)M, d, d);
    g5.e.kind = EPI_T;
    g5.e.c = c->dO;
    g5.e.ldc = d;
    // one pass sums K-split parts into dO and its per-head transpose for the backward
    int S5 = 1;
    CK(Ops<T>::gemm_parts(c, g5, n, S5));
    AttnBwdArgs ab;
    if (S5 > 1) {
      CK(parts_rows_t<T>(c->ws, S5, M * d, M, d, n, tp<T>(c->dO), tp<T>(c->dOT), c->stream));
      ab.dot_ready = true;
    }
    ab.q = a.q;
    ab.qt = a.qt;
    ab.kr = lw.kr;
    ab.vr = lw.vr;
    ab.vtr = lw.vtr;
    ab.ktr = lw.ktr;
    ab.dot = c->dOT;
    ab.o = a.o;
    ab.dout = c->dO;
    ab.lse = a.lse;
    ab.dvec = c->dvec;
    ab.dq = c->dq;
    ab.dk = c->dk;
    ab.dv = c->dv;
    ab.B = B;
    ab.H = c->H;
    ab.hd = c->hd;
    ab.n = n;
    ab.R = c->R;
    ab.window = c->k;
    ab.pos0 = p0;
    AttnBwdParts bp;
    CK(Ops<T>::bwd(c, ab, &bp));
    CK(rope_bwd_pack<T>(bp, c->cos_t, c->sin_t, p0, B, n, c->H, c->hd, tp<T>(c->dqkv), c->stream));
    GemmArgs g6 = mk(c->dqkv, 3 * d, lw.wqkvT, 3 * d, (int)M, d, 3 * d);
    g6.e.kind = EPI_F32;
    g6.e.c = c->tmpf;
    g6.e.ldc = d;
    int S6 = 1;
    CK(Ops<T>::gemm_parts(c, g6, n, S6));
    CK(norm_bwd<T>(c, S6, a.h_in, a.rstd1, M, lw.attn_norm, c->tmpf, c->dh, c->dh, tp<T>(c->dyN)));
  }
  // the next chunk reads the updated fast weights and rewrites the saved activations
  if (c->overlap) {
    CK(hipEventRecord(c->ev_s2m, c->side));
    CK(hipStreamWaitEvent(c->stream, c->ev_s2m, 0));
  }
  return TTT_OK;
}

// the chunk loop over n_tokens tokens per row, starting at c->pos
// While alive, the context's stream, scratch buffers and workspace are those of the batched
// pass, and c->hb is the given h' buffer; the destructor restores them.
struct BottomScope {
  ttt_ctx* c;
  float* hb_main;
  BottomScope(ttt_ctx* c_, float* hbuf) : c(c_), hb_main(c_->hb) {
    swap_all();
    c->hb = hbuf;
  }
  ~BottomScope() {
    c->hb = hb_main;
    swap_all();
  }
  void swap_all() {
    std::swap(c->stream, c->bstream);
    std::swap(c->qkvb, c->b_qkvb);
    std::swap(c->rstd_tmp, c->b_rstd);
    std::swap(c->ws, c->b_ws);
    std::swap(c->ub, c->b_ub);
    std::swap(c->qb, c->b_qb);
    std::swap(c->ob, c->b_ob);
    std::swap(c->actb, c->b_actb);
  }
};

// Lookahead groups of G chunks: the batched pass of group i + 1 (batched stream, h' buffer
// (i + 1) % 2) is issued before the chunks of group i (main stream, buffer i % 2), so the two
// run side by side; events order each buffer's writer after its previous readers.
template <typename T>
int run_tokens_overlap(ttt_ctx* c, const int32_t* tok, const int32_t* tgt, int64_t ld, int64_t n_tokens,
                       float* loss_dev) {
  const int64_t gmax = (int64_t)c->G * c->b;
  const int ng = (int)((n_tokens + gmax - 1) / gmax);
  float* hbuf[2] = {c->hb, c->hb2};
  auto group_len = [&](int gi) { return (int)std::min<int64_t>(n_tokens - gi * gmax, gmax); };
  auto bottom = [&](int gi) -> int {
    BottomScope scope(c, hbuf[gi & 1]);
    int rc = bottom_pass<T>(c, tok + gi * gmax, ld, group_len(gi), c->pos + gi * gmax);
    if (rc) return rc;
    CK(hipEventRecord(c->ev_bdone[gi & 1], c->stream));  // (the batched stream in this scope)
    return TTT_OK;
  };
  // the batched stream starts after the main stream's earlier work, which may still read h'
  CK(hipEventRecord(c->ev_c2b, c->stream));
  CK(hipStreamWaitEvent(c->bstream, c->ev_c2b, 0));
  int rc = bottom(0);
  if (rc) return rc;
  int64_t ci = 0;
  for (int gi = 0; gi < ng; ++gi) {
    if (gi + 1 < ng) {
      // buffer (gi + 1) % 2 was last read by the chunks of group gi - 1
      if (gi >= 1) CK(hipStreamWaitEvent(c->bstream, c->ev_cdone[(gi + 1) & 1], 0));
      rc = bottom(gi + 1);
      if (rc) return rc;
    }
    CK(hipStreamWaitEvent(c->stream, c->ev_bdone[gi & 1], 0));
    const int g = group_len(gi);
    const int64_t s = gi * gmax;
    for (int cs = 0; cs < g; cs += c->b) {
      const int n = std::min(c->b, g - cs);
      for (int st = 0; st < c->n_steps; ++st) {
        rc = top_chunk<T>(c, tgt + s + cs, ld, hbuf[gi & 1] + (int64_t)cs * c->d, (int64_t)g * c->d, n,
                          c->pos + s + cs, st == 0 ? loss_dev + ci * c->B : c->loss_later);
        if (rc) return rc;
      }
      ++ci;
    }
    CK(hipEventRecord(c->ev_cdone[gi & 1], c->stream));
  }
  c->pos += n_tokens;
  return TTT_OK;
}

template <typename T>
int run_tokens(ttt_ctx* c, const int32_t* tok, const int32_t* tgt, int64_t ld, int64_t n_tokens, float* loss_dev) {
  if (c->bot_overlap) return run_tokens_overlap<T>(c, tok, tgt, ld, n_tokens, loss_dev);
  int64_t done = 0, ci = 0;
  const int64_t gmax = (int64_t)c->G * c->b;
  while (done < n_tokens) {
    int g = (int)std::min<int64_t>(n_tokens - done, gmax);
    int rc = bottom_pass<T>(c, tok + done, ld, g, c->pos + done);
    if (rc) return rc;
    for (int cs = 0; cs < g; cs += c->b) {
      int n = std::min(c->b, g - cs);
      for (int st = 0; st < c->n_steps; ++st) {
        rc = top_chunk<T>(c, tgt + done + cs, ld, c->hb + (int64_t)cs * c->d, (int64_t)g * c->d, n,
                          c->pos + done + cs, st == 0 ? loss_dev + ci * c->B : c->loss_later);
        if (rc) return rc;
      }
      ++ci;
    }
    done += g;
  }
  c->pos += n_tokens;
  return TTT_OK;
}

// Forward and loss only over n_tokens tokens per row from c->pos (no backward, no update):
// while nothing changes the fast weights every block is frozen, so all L blocks run over
// groups of up to G chunks at once; then final norm, lm_head and the cross-entropy of each
// chunk (the loss a prefill of the same chunk would report).  The window's keys and values
// are written as by a prefill.
template <typename T>
int run_score(ttt_ctx* c, const int32_t* tok, const int32_t* tgt, int64_t ld, int64_t n_tokens, float* loss_dev) {
  const int B = c->B, d = c->d, V = c->V, b = c->b;
  const int64_t gmax = (int64_t)c->G * b;
  int64_t done = 0, ci = 0;
  while (done < n_tokens) {
    const int g = (int)std::min<int64_t>(n_tokens - done, gmax);
    CK(embed_gather_ld<T>(tok + done, ld, B, g, tp<T>(c->embed), d, V, c->hb, c->err_dev, c->stream));
    for (int l = 0; l < c->L; ++l) {
      int rc = layer_fwd<T>(c, l, c->hb, g, c->pos + done, FULL, nullptr);
      if (rc) return rc;
    }
    // final norm of the whole group into ub ([B][g][d]); sums K-split parts still pending
    CK(norm_fwd<T>(c, c->hb, (int64_t)B * g, c->final_norm, tp<T>(c->ub), c->rstd_tmp, (T*)nullptr, g, 0, nullptr));
    for (int cs = 0; cs < g; cs += b) {
      const int n = std::min(b, g - cs);
      const int32_t* t0 = tgt + done + cs;
      CK(count_valid_ld(t0, ld, B, n, c->nvalid, c->stream));
      if (B == 1) {  // the chunk's rows are contiguous: lm_head and the tiled cross-entropy in one product
        CK(lmhead_ce<T>(c, tp<T>(c->ub, (int64_t)cs * d), n, t0, ld, n, (T*)nullptr));
      } else {
        GemmArgs gl = mk(tp<T>(c->ub, (int64_t)cs * d), d, c->lm_head, d, n, V, d);
        gl.batch = B;
        gl.sA = (int64_t)g * d;
        gl.sB = 0;
        gl.e.kind = EPI_F32;
        gl.e.c = c->logits;
        gl.e.ldc = V;
        gl.e.sc = (int64_t)n * V;
        CK(Ops<T>::gemm(c, gl));
        CK(ce_rows_ld<T>(c->logits, (int64_t)B * n, V, t0, ld, c->nvalid, n, c->loss_tok, (T*)nullptr, c->err_dev,
                         c->stream));
      }
      CK(reduce_loss(c->loss_tok, c->nvalid, B, n, loss_dev + ci * B, c->stream));
      ++ci;
    }
    done += g;
  }
  c->pos += n_tokens;
  return TTT_OK;
}

// one greedy decode step: input tok[r*ld], output arg-max to tok[r*ld + 1]
template <typename T>
int decode_step(ttt_ctx* c, int32_t* tok, int64_t ld) {
  const int B = c->B, d = c->d;
  CK(embed_gather_ld<T>(tok, ld, B, 1, tp<T>(c->embed), d, c->V, c->hb, c->err_dev, c->stream));
  for (int l = 0; l < c->L; ++l) {
    int rc = layer_fwd<T>(c, l, c->hb, 1, c->pos, FULL, nullptr);
    if (rc) return rc;
  }
  GemmArgs gl = mk(c->hf, d, c->lm_head, d, B, c->V, d);
  gl.e.kind = EPI_F32;
  gl.e.c = c->logits;
  gl.e.ldc = c->V;
  // (the final norm inside the lm_head product when it takes it)
  if (!norm_in_product(c, nullptr, gl, c->hb, c->final_norm))
    CK(norm_fwd<T>(c, c->hb, B, c->final_norm, tp<T>(c->hf), c->rstd_tmp, (T*)nullptr, 1, 0, nullptr));
  CK(Ops<T>::gemm(c, gl));
  CK(argmax_rows_ld(c->logits, B, c->V, tok + 1, ld, nullptr, 0, c->stream));
  c->pos += 1;
  return TTT_OK;
}

int ensure_tok(ttt_ctx* c, int64_t n) {
  if (n <= c->d_tok_cap) return TTT_OK;
  void* p = c->alloc((size_t)n * 4);
  if (!p) return fail(c, TTT_ENOMEM, "token buffer allocation failed");
  c->d_tok = (int32_t*)p;
  c->d_tok_cap = n;
  return TTT_OK;
}

int ensure_loss(ttt_ctx* c, int64_t n) {
  if (n <= c->d_loss_cap) return TTT_OK;
  void* p = c->alloc((size_t)n * 4);
  if (!p) return fail(c, TTT_ENOMEM, "loss buffer allocation failed");
  c->d_loss = (float*)p;
  c->d_loss_cap = n;
  return TTT_OK;
}

int check_ids(const ttt_ctx* c, const int32_t* x, int64_t cnt, bool allow_ignore) {
  for (int64_t i = 0; i < cnt; ++i) {
    if (x[i] >= c->V) return 0;
    if (x[i] < 0 && !(allow_ignore && x[i] == -1)) return 0;
  }
  return 1;
}

int sync_and_check(ttt_ctx* c, const float* dloss, int64_t nloss, float* host_copy) {
  std::vector<float> tmp;
  if (dloss && nloss > 0) {
    tmp.resize(nloss);
    CK(hipMemcpyAsync(tmp.data(), dloss, nloss * 4, hipMemcpyDeviceToHost, c->stream));
  }
  int herr = 0;
  CK(hipMemcpyAsync(&herr, c->err_dev, 4, hipMemcpyDeviceToHost, c->stream));
  CK(hipStreamSynchronize(c->stream));
  if (herr) {
    c->poisoned = true;
    return fail(c, TTT_EINVAL, "token id out of range in device input");
  }
  for (int64_t i = 0; i < nloss; ++i)
    if (!std::isfinite(tmp[i])) return fail(c, TTT_ENONFINITE, "non-finite chunk loss");
  if (host_copy && nloss > 0) memcpy(host_copy, tmp.data(), nloss * 4);
  return TTT_OK;
}

int run_dispatch(ttt_ctx* c, const int32_t* tok, const int32_t* tgt, int64_t ld, int64_t n, float* loss_dev) {
  return c->bf16 ? run_tokens<bf16>(c, tok, tgt, ld, n, loss_dev) : run_tokens<float>(c, tok, tgt, ld, n, loss_dev);
}

int score_dispatch(ttt_ctx* c, const int32_t* tok, const int32_t* tgt, int64_t ld, int64_t n, float* loss_dev) {
  return c->bf16 ? run_score<bf16>(c, tok, tgt, ld, n, loss_dev) : run_score<float>(c, tok, tgt, ld, n, loss_dev);
}

int decode_dispatch(ttt_ctx* c, int32_t* tok, int64_t ld) {
  return c->bf16 ? decode_step<bf16>(c, tok, ld) : decode_step<float>(c, tok, ld);
}

// host fp32 -> device T
int upload(ttt_ctx* c, void* dst, const float* src, int64_t cnt) {
  if (!c->bf16) {
    CK(hipMemcpy(dst, src, cnt * 4, hipMemcpyHostToDevice));
    return TTT_OK;
  }
  std::vector<bf16> tmp(cnt);
  for (int64_t i = 0; i < cnt; ++i) tmp[i] = f2bf(src[i]);
  CK(hipMemcpy(dst, tmp.data(), cnt * 2, hipMemcpyHostToDevice));
  return TTT_OK;
}

// host fp32 [rows][cols] -> device T transposed [cols][rows]
int upload_t(ttt_ctx* c, void* dst, const float* src, int64_t rows, int64_t cols) {
  std::vector<float> t(rows * cols);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t q = 0; q < cols; ++q) t[q * rows + r] = src[r * cols + q];
  return upload(c, dst, t.data(), rows * cols);
}

int build(ttt_ctx* c, const ttt_weights* w) {
  const int L = c->L, d = c->d, f = c->f, V = c->V, B = c->B, H = c->H, hd = c->hd, b = c->b, R = c->R;
  const size_t es = c->es;
  const int64_t rows_bot = (int64_t)B * c->G * b, rows_top = (int64_t)B * b;
#define AL(ptr, bytes)                                                           \
  do {                                                                           \
    (ptr) = (std::remove_reference_t<decltype(ptr)>)c->alloc((size_t)(bytes));   \
    if (!(ptr)) return fail(c, TTT_ENOMEM, "device allocation failed: " #ptr);  \
  } while (0)
  AL(c->embed, (int64_t)V * d * es);
  AL(c->lm_head, (int64_t)V * d * es);
  AL(c->lm_headT, (int64_t)V * d * es);
  AL(c->final_norm, d * 4);
  int rc;
  if ((rc = upload(c, c->embed, w->embed, (int64_t)V * d))) return rc;
  if ((rc = upload(c, c->lm_head, w->lm_head, (int64_t)V * d))) return rc;
  if ((rc = upload_t(c, c->lm_headT, w->lm_head, V, d))) return rc;
  CK(hipMemcpy(c->final_norm, w->final_norm, d * 4, hipMemcpyHostToDevice));
  c->lw.resize(L);
  const int64_t ring = (int64_t)B * H * R * hd * es;
  std::vector<float> qkv((size_t)3 * d * d);
  for (int l = 0; l < L; ++l) {
    LayerW& lw = c->lw[l];
    AL(lw.attn_norm, d * 4);
    AL(lw.mlp_norm, d * 4);
    CK(hipMemcpy(lw.attn_norm, w->attn_norm[l], d * 4, hipMemcpyHostToDevice));
    CK(hipMemcpy(lw.mlp_norm, w->mlp_norm[l], d * 4, hipMemcpyHostToDevice));
    memcpy(qkv.data(), w->wq[l], (size_t)d * d * 4);
    memcpy(qkv.data() + (size_t)d * d, w->wk[l], (size_t)d * d * 4);
    memcpy(qkv.data() + 2 * (size_t)d * d, w->wv[l], (size_t)d * d * 4);
    AL(lw.wqkv, 3LL * d * d * es);
    AL(lw.wo, (int64_t)d * d * es);
    if (c->rope_perm) {  // forward copy with the q/k rows of each head pair-interleaved
      std::vector<float> perm((size_t)3 * d * d);
      for (int64_t r = 0; r < 3LL * d; ++r)
        memcpy(perm.data() + qkv_perm_row(r, d, hd) * d, qkv.data() + r * d, (size_t)d * 4);
      if ((rc = upload(c, lw.wqkv, perm.data(), 3LL * d * d))) return rc;
    } else if ((rc = upload(c, lw.wqkv, qkv.data(), 3LL * d * d))) {
      return rc;
    }
    if ((rc = upload(c, lw.wo, w->wo[l], (int64_t)d * d))) return rc;
    if (l > c->l0) {
      AL(lw.wqkvT, 3LL * d * d * es);
      AL(lw.woT, (int64_t)d * d * es);
      if ((rc = upload_t(c, lw.wqkvT, qkv.data(), 3LL * d, d))) return rc;
      if ((rc = upload_t(c, lw.woT, w->wo[l], d, d))) return rc;
    }
    if (l < c->l0) {
      AL(lw.wgu, 2LL * f * d * es);
      AL(lw.wd, (int64_t)d * f * es);
      if (c->il) {  // [W_gate; W_up] rows placed at swiglu_il_row
        std::vector<float> gu((size_t)2 * f * d);
        for (int64_t r = 0; r < 2LL * f; ++r) {
          const float* src = r < f ? w->w_gate[l] + r * d : w->w_up[l] + (r - f) * d;
          memcpy(gu.data() + swiglu_il_row(r, f) * d, src, (size_t)d * 4);
        }
        if ((rc = upload(c, lw.wgu, gu.data(), 2LL * f * d))) return rc;
      } else {
        if ((rc = upload(c, lw.wgu, w->w_gate[l], (int64_t)f * d))) return rc;
        if ((rc = upload(c, (char*)lw.wgu + (int64_t)f * d * es, w->w_up[l], (int64_t)f * d))) return rc;
      }
      if ((rc = upload(c, lw.wd, w->w_down[l], (int64_t)d * f))) return rc;
    }
    AL(lw.kr, ring);
    AL(lw.vr, ring);
    AL(lw.vtr, ring);
    CK(hipMemset(lw.kr, 0, ring));
    CK(hipMemset(lw.vr, 0, ring));
    CK(hipMemset(lw.vtr, 0, ring));
    if (c->bf16 && l > c->l0) {
      AL(lw.ktr, ring);
      CK(hipMemset(lw.ktr, 0, ring));
    }
  }
  // fast weights: fp32 masters per row plus T shadows in both layouts
  const int64_t fsz = 3LL * f * d;
  AL(c->fast_init, fsz * c->Lq * 4);
  c->fw.resize(c->Lq);
  for (int j = 0; j < c->Lq; ++j) {
    int l = c->l0 + j;
    float* init = c->fast_init + j * fsz;
    // the updated MLP: the block's own, or (dual MLP) its dynamic one
    const float* gsrc = c->dual ? w->dyn_gate[j] : w->w_gate[l];
    const float* usrc = c->dual ? w->dyn_up[j] : w->w_up[l];
    const float* dsrc = c->dual ? w->dyn_down[j] : w->w_down[l];
    CK(hipMemcpy(init, gsrc, (size_t)f * d * 4, hipMemcpyHostToDevice));
    CK(hipMemcpy(init + (int64_t)f * d, usrc, (size_t)f * d * 4, hipMemcpyHostToDevice));
    CK(hipMemcpy(init + 2LL * f * d, dsrc, (size_t)d * f * 4, hipMemcpyHostToDevice));
    FastW& fw = c->fw[j];
    AL(fw.master, fsz * B * 4);
    AL(fw.wgu, 2LL * f * d * B * es);
    AL(fw.wguT, 2LL * f * d * B * es);
    AL(fw.wd, (int64_t)d * f * B * es);
    AL(fw.wdT, (int64_t)d * f * B * es);
  }
  // dual MLP: the static MLPs of the fast blocks, frozen, in the same layouts as the dynamic
  // ones (the transposed copies serve the backward of the blocks above l0)
  if (c->dual) {
    c->sw.resize(c->Lq);
    for (int j = 0; j < c->Lq; ++j) {
      const int l = c->l0 + j;
      FastW& sw = c->sw[j];
      AL(sw.master, fsz * 4);
      CK(hipMemcpy(sw.master, w->w_gate[l], (size_t)f * d * 4, hipMemcpyHostToDevice));
      CK(hipMemcpy(sw.master + (int64_t)f * d, w->w_up[l], (size_t)f * d * 4, hipMemcpyHostToDevice));
      CK(hipMemcpy(sw.master + 2LL * f * d, w->w_down[l], (size_t)d * f * 4, hipMemcpyHostToDevice));
      AL(sw.wgu, 2LL * f * d * es);
      AL(sw.wguT, 2LL * f * d * es);
      AL(sw.wd, (int64_t)d * f * es);
      AL(sw.wdT, (int64_t)d * f * es);
      CK(refresh_shadows(sw.master, 2 * f, d, 1, fsz, sw.wgu, 2LL * f * d, sw.wguT, 2LL * f * d, c->bf16,
                         c->il ? f : 0, c->stream));
      CK(refresh_shadows(sw.master + 2LL * f * d, d, f, 1, fsz, sw.wd, (int64_t)d * f, sw.wdT, (int64_t)d * f,
                         c->bf16, 0, c->stream));
    }
    CK(hipStreamSynchronize(c->stream));
  }
  // RoPE table in fp64 on the host, stored fp32: angle = pos * theta^(-2i/hd)
  const int half = hd / 2;
  const int64_t P = c->cfg.max_positions;
  {
    std::vector<float> cs((size_t)P * half), sn((size_t)P * half);
    std::vector<double> inv(half);
    for (int i = 0; i < half; ++i) inv[i] = std::pow(c->cfg.rope_theta, -2.0 * i / hd);
    for (int64_t p = 0; p < P; ++p)
      for (int i = 0; i < half; ++i) {
        double a = (double)p * inv[i];
        cs[(size_t)p * half + i] = (float)std::cos(a);
        sn[(size_t)p * half + i] = (float)std::sin(a);
      }
    AL(c->cos_t, P * half * 4);
    AL(c->sin_t, P * half * 4);
    CK(hipMemcpy(c->cos_t, cs.data(), (size_t)P * half * 4, hipMemcpyHostToDevice));
    CK(hipMemcpy(c->sin_t, sn.data(), (size_t)P * half * 4, hipMemcpyHostToDevice));
  }
  // work buffers
  AL(c->hb, rows_bot * d * 4);
  if (c->bot_overlap) {
    AL(c->hb2, rows_bot * d * 4);
    AL(c->b_qkvb, rows_bot * 3 * d * 4);
    AL(c->b_rstd, rows_bot * 4);
    AL(c->b_ub, rows_bot * d * es);
    AL(c->b_qb, rows_bot * d * es);
    AL(c->b_ob, rows_bot * d * es);
    AL(c->b_actb, rows_bot * f * es);
  }
  AL(c->qkvb, rows_bot * 3 * d * 4);
  AL(c->rstd_tmp, rows_bot * 4);
  AL(c->ub, rows_bot * d * es);
  AL(c->qb, rows_bot * d * es);
  AL(c->ob, rows_bot * d * es);
  AL(c->actb, rows_bot * f * es);
  AL(c->htop, rows_top * d * 4);
  AL(c->rstdf, rows_top * 4);
  AL(c->logits, rows_top * V * 4);
  AL(c->loss_tok, rows_top * 4);
  AL(c->hf, rows_top * d * es);
  AL(c->dlogits, rows_top * V * es);
  AL(c->ce_part, rows_top * 2 * cdiv(V, 256) * 4);
  AL(c->ce_zt, rows_top * 4);
  AL(c->nvalid, B * 4);
  AL(c->loss_later, B * 4);
  AL(c->dh, rows_top * d * 4);
  AL(c->tmpf, rows_top * d * 4);
  AL(c->dq, rows_top * d * 4);
  AL(c->dk, rows_top * d * 4);
  AL(c->dv, rows_top * d * 4);
  AL(c->dvec, rows_top * H * 4);
  AL(c->dyN, rows_top * d * es);
  c->dyT.resize(c->Lq);
  c->dzT.resize(c->Lq);
  for (int j = 0; j < c->Lq; ++j) {
    AL(c->dyT[j], rows_top * d * es);
    AL(c->dzT[j], rows_top * 2 * f * es);
  }
  AL(c->dz, rows_top * 2 * f * es);
  if (c->dual) {
    AL(c->dzT_s, rows_top * 2 * f * es);
    AL(c->act_s, rows_top * f * es);
  }
  AL(c->dhT, rows_top * d * es);
  AL(c->dO, rows_top * d * es);
  if (c->bf16) AL(c->dOT, rows_top * d * es);
  AL(c->dqkv, rows_top * 3 * d * es);
  AL(c->err_dev, 256);
  c->ws_floats = 8 * rows_top * (int64_t)(d + 2 * H);
  c->ws_alloc_floats = 2 * c->ws_floats;
  AL(c->ws, c->ws_alloc_floats * 4);
  if (c->bot_overlap) AL(c->b_ws, c->ws_alloc_floats * 4);
  CK(hipMemset(c->err_dev, 0, 4));
  c->acts.resize(c->Lq);
  for (int j = 0; j < c->Lq; ++j) {
    TopActs& a = c->acts[j];
    AL(a.h_in, rows_top * d * 4);
    AL(a.h_mid, rows_top * d * 4);
    AL(a.rstd1, rows_top * 4);
    AL(a.rstd2, rows_top * 4);
    AL(a.lse, rows_top * H * 4);
    AL(a.q, rows_top * d * es);
    AL(a.qt, rows_top * d * es);
    AL(a.o, rows_top * d * es);
    AL(a.mT, rows_top * d * es);
    AL(a.zg, rows_top * f * es);
    AL(a.zu, rows_top * f * es);
    AL(a.actT, rows_top * f * es);
    if (c->dual && j > 0) {
      AL(a.zg_s, rows_top * f * es);
      AL(a.zu_s, rows_top * f * es);
    }
  }
#undef AL
  return TTT_OK;
}

// bf16 copies (row-major, transposed, interleaved gate/up) of every row's fp32 fast weights
hipError_t refresh_fast_shadows(ttt_ctx* c) {
  const int64_t fsz = 3LL * c->f * c->d;
  for (int j = 0; j < c->Lq; ++j) {
    FastW& fw = c->fw[j];
    hipError_t e = refresh_shadows(fw.master, 2 * c->f, c->d, c->B, fsz, fw.wgu, 2LL * c->f * c->d, fw.wguT,
                                   2LL * c->f * c->d, c->bf16, c->il ? c->f : 0, c->stream);
    if (e != hipSuccess) return e;
    e = refresh_shadows(fw.master + 2LL * c->f * c->d, c->d, c->f, c->B, fsz, fw.wd, (int64_t)c->d * c->f, fw.wdT,
                        (int64_t)c->d * c->f, c->bf16, 0, c->stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

constexpr int64_t STATE_MAGIC = 0x5354544E49545454LL, STATE_VERSION = 3, STATE_HDR = 17;

// Everything a snapshot's contents depend on: the ring keys are stored RoPE-rotated at their
// absolute positions (theta) in slots pos mod R, so window, chunk and theta must match as well
// as the array sizes, and the fast weights are the dynamic MLPs' when dual_mlp is set; slot 11
// is the position.
void state_header(const ttt_ctx* c, int64_t* h) {
  int64_t theta_bits = 0;
  memcpy(&theta_bits, &c->cfg.rope_theta, 8);
  const int64_t v[STATE_HDR] = {STATE_MAGIC, STATE_VERSION, c->B, c->L, c->H, c->hd, c->R, (int64_t)c->es, c->Lq, c->f,
                                c->d, c->pos, c->k, c->b, c->V, theta_bits, c->dual ? 1 : 0};
  for (int i = 0; i < STATE_HDR; ++i) h[i] = v[i];
}

// the device arrays of a snapshot after the header, in order: fast weights, then each layer's rings
template <typename F>
hipError_t for_state_arrays(ttt_ctx* c, F&& f) {
  const int64_t fsz = 3LL * c->f * c->d, ring = (int64_t)c->B * c->H * c->R * c->hd * c->es;
  for (int j = 0; j < c->Lq; ++j) {
    hipError_t e = f((void*)c->fw[j].master, fsz * c->B * 4);
    if (e != hipSuccess) return e;
  }
  for (int l = 0; l < c->L; ++l) {
    void* arr[4] = {c->lw[l].kr, c->lw[l].vr, c->lw[l].vtr, c->lw[l].ktr};
    for (void* p : arr) {
      if (!p) continue;
      hipError_t e = f(p, ring);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// the batched and side streams finished (a failed call may leave work in flight there)
hipError_t sync_aux(ttt_ctx* c) {
  if (c->bstream) {
    hipError_t e = hipStreamSynchronize(c->bstream);
    if (e != hipSuccess) return e;
  }
  return c->side ? hipStreamSynchronize(c->side) : hipSuccess;
}

int reset_state(ttt_ctx* c) {
  // (a failed call may have left a batched pass or updates in flight on the other streams)
  CK(sync_aux(c));
  c->pend_parts = 0;
  const int64_t fsz = 3LL * c->f * c->d;
  for (int j = 0; j < c->Lq; ++j) {
    FastW& fw = c->fw[j];
    for (int r = 0; r < c->B; ++r)
      CK(hipMemcpyAsync(fw.master + r * fsz, c->fast_init + j * fsz, fsz * 4, hipMemcpyDeviceToDevice, c->stream));
    CK(refresh_shadows(fw.master, 2 * c->f, c->d, c->B, fsz, fw.wgu, 2LL * c->f * c->d, fw.wguT, 2LL * c->f * c->d,
                       c->bf16, c->il ? c->f : 0, c->stream));
    CK(refresh_shadows(fw.master + 2LL * c->f * c->d, c->d, c->f, c->B, fsz, fw.wd, (int64_t)c->d * c->f, fw.wdT,
                       (int64_t)c->d * c->f, c->bf16, 0, c->stream));
  }
  // The key/value rings need no clearing: a query at position t reads only slots of positions
  // max(0, t - window + 1) .. t, all written by the new sequence before; the other slots of a
  // 64-key tile are masked to probability 0, which needs only that they hold finite values, as
  // the previous sequence leaves them (they are zero from creation).  After a failure (the context
  // was poisoned: a non-finite value may sit in a ring), or when the last asynchronous call was
  // never checked by ttt_sync, they are cleared.
  if (c->poisoned || c->pending_loss) {
    const int64_t ring = (int64_t)c->B * c->H * c->R * c->hd * c->es;
    for (int l = 0; l < c->L; ++l) {
      CK(hipMemsetAsync(c->lw[l].kr, 0, ring, c->stream));
      CK(hipMemsetAsync(c->lw[l].vr, 0, ring, c->stream));
      CK(hipMemsetAsync(c->lw[l].vtr, 0, ring, c->stream));
      if (c->lw[l].ktr) CK(hipMemsetAsync(c->lw[l].ktr, 0, ring, c->stream));
    }
  }
  CK(hipMemsetAsync(c->err_dev, 0, 4, c->stream));
  CK(hipStreamSynchronize(c->stream));
  c->pos = 0;
  c->poisoned = false;
  c->pending_loss = nullptr;
  c->pending_n = 0;
  return TTT_OK;
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

int ttt_set_allocator(ttt_alloc_fn alloc, ttt_free_fn free_fn, void* user) {
  if ((alloc == nullptr) != (free_fn == nullptr)) return TTT_EINVAL;
  g_alloc = alloc;
  g_free = free_fn;
  g_user = user;
  return TTT_OK;
}

const char* ttt_last_error(const ttt_ctx* ctx) { return ctx ? ctx->err.c_str() : g_create_err.c_str(); }

int ttt_create(const ttt_config* cfg, const ttt_weights* w, void* hip_stream, ttt_ctx** out) {
  g_create_err.clear();
  if (!cfg || !w || !out) {
    g_create_err = "NULL argument";
    return TTT_EINVAL;
  }
  *out = nullptr;
  ttt_config c0 = *cfg;
  if (c0.n_fast == 0) c0.n_fast = std::max(1, c0.n_layers / 4);
  // default: 32 chunks per batched lower-block pass (large GEMM and attention grids fill the
  // 256 CUs in whole rounds), no more than the positions the context will see
  if (c0.lookahead <= 0 && c0.chunk > 0) {
    const int64_t need = c0.max_positions > 0 ? (c0.max_positions + c0.chunk - 1) / c0.chunk : 32;
    c0.lookahead = (int32_t)std::max<int64_t>(1, std::min<int64_t>(32, need));
  }
  auto bad = [&](const char* m) {
    g_create_err = m;
    return TTT_EINVAL;
  };
  if (c0.n_layers <= 0 || c0.d_model <= 0 || c0.n_heads <= 0 || c0.d_ff <= 0 || c0.vocab <= 0 || c0.batch <= 0)
    return bad("sizes must be positive");
  if (c0.d_model % c0.n_heads) return bad("d_model must be a multiple of n_heads");
  int hd = c0.d_model / c0.n_heads;
  if (hd % 2 || hd > 128) return bad("head_dim must be even and at most 128");
  if (c0.chunk <= 0 || c0.window < c0.chunk) return bad("window must be >= chunk >= 1");
  if (c0.n_fast < 1 || c0.n_fast > c0.n_layers) return bad("n_fast out of range");
  if (c0.dtype != TTT_F32 && c0.dtype != TTT_BF16) return bad("dtype must be TTT_F32 or TTT_BF16");
  if (c0.max_positions <= 0) return bad("max_positions must be positive");
  if (c0.n_steps < 0) return bad("n_steps must be >= 0");
  if (!(c0.rope_theta > 0) || !(c0.rms_eps >= 0) || !std::isfinite(c0.lr)) return bad("bad theta/eps/lr");
  if (c0.dual_mlp != 0 && c0.dual_mlp != 1) return bad("dual_mlp must be 0 or 1");
  if (c0.dual_mlp) {
    if (!w->dyn_gate || !w->dyn_up || !w->dyn_down) return bad("dual_mlp needs the dyn_* weight arrays");
    for (int j = 0; j < c0.n_fast; ++j)
      if (!w->dyn_gate[j] || !w->dyn_up[j] || !w->dyn_down[j]) return bad("NULL dynamic MLP weight pointer");
  }
  if (!w->embed || !w->final_norm || !w->lm_head || !w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo ||
      !w->mlp_norm || !w->w_gate || !w->w_up || !w->w_down)
    return bad("NULL weight pointer");
  for (int l = 0; l < c0.n_layers; ++l)
    if (!w->attn_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] || !w->mlp_norm[l] || !w->w_gate[l] ||
        !w->w_up[l] || !w->w_down[l])
      return bad("NULL per-layer weight pointer");
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) {
    g_create_err = "no HIP device";
    return TTT_ENODEV;
  }
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
      strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    g_create_err = "device is not gfx950";
    return TTT_ENODEV;
  }
  ttt_ctx* c = new ttt_ctx();
  c->cfg = c0;
  c->L = c0.n_layers;
  c->d = c0.d_model;
  c->H = c0.n_heads;
  c->hd = hd;
  c->f = c0.d_ff;
  c->V = c0.vocab;
  c->k = c0.window;
  c->b = c0.chunk;
  c->Lq = c0.n_fast;
  c->l0 = c0.n_layers - c0.n_fast;
  c->B = c0.batch;
  c->G = c0.lookahead;
  c->n_steps = std::max(1, c0.n_steps);
  c->dual = c0.dual_mlp == 1;
  c->R = c0.window + c0.lookahead * c0.chunk;
  c->bf16 = c0.dtype == TTT_BF16;
  c->es = c->bf16 ? 2 : 4;
  c->stream = (hipStream_t)hip_stream;
  c->free_fn = g_free;
  c->free_user = g_user;
  const char* simt = getenv("TTT_SIMT");
  c->mfma = !(simt && simt[0] == '1');
  const char* noside = getenv("TTT_NO_SIDE");
  c->overlap = !(noside && noside[0] == '1');
  c->il = c->bf16 && c->mfma && c0.d_ff % 32 == 0 && c0.d_model % 8 == 0;
  c->rope_perm = c->bf16 && c->mfma;
  const char* nobot = getenv("TTT_NO_BOTTOM_OVERLAP");
  c->bot_overlap = !(nobot && nobot[0] == '1');
  bool ok = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&c->ev_m2s, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&c->ev_s2m, hipEventDisableTiming) == hipSuccess;
  if (ok && c->bot_overlap) {
    ok = hipStreamCreateWithFlags(&c->bstream, hipStreamNonBlocking) == hipSuccess &&
         hipEventCreateWithFlags(&c->ev_c2b, hipEventDisableTiming) == hipSuccess;
    for (int i = 0; i < 2 && ok; ++i)
      ok = hipEventCreateWithFlags(&c->ev_bdone[i], hipEventDisableTiming) == hipSuccess &&
           hipEventCreateWithFlags(&c->ev_cdone[i], hipEventDisableTiming) == hipSuccess;
  }
  if (!ok) {
    g_create_err = "stream/event creation failed";
    c->destroy_streams();
    delete c;
    return TTT_EDEVICE;
  }
  int rc = build(c, w);
  if (rc == TTT_OK) rc = reset_state(c);
  if (rc != TTT_OK) {
    g_create_err = c->err;
    c->release_all();
    c->destroy_streams();
    delete c;
    return rc;
  }
  *out = c;
  return TTT_OK;
}

int ttt_profile_enable(ttt_ctx* c, int32_t on) {
  if (!c) return TTT_EINVAL;
  CK(hipStreamSynchronize(c->stream));
  c->prof = (uint32_t)on & ((1u << PC_N) - 1);
  c->prof_recs.clear();
  c->ev_used = 0;
  return TTT_OK;
}

int ttt_profile_read(ttt_ctx* c, int32_t n_classes, double* ms, int64_t* counts, double* flops) {
  if (!c || n_classes < 0 || (n_classes > 0 && (!ms || !counts || !flops))) return TTT_EINVAL;
  CK(hipStreamSynchronize(c->stream));
  for (int i = 0; i < n_classes; ++i) {
    ms[i] = 0;
    counts[i] = 0;
    flops[i] = 0;
  }
  for (const auto& r : c->prof_recs) {
    if (r.cls >= n_classes) continue;
    float t = 0.f;
    CK(hipEventElapsedTime(&t, r.a, r.b));
    ms[r.cls] += t;
    counts[r.cls] += 1;
    flops[r.cls] += r.flops;
  }
  return TTT_OK;
}

void ttt_destroy(ttt_ctx* c) {
  if (!c) return;
  (void)hipStreamSynchronize(c->stream);
  for (hipEvent_t e : c->ev_pool) (void)hipEventDestroy(e);
  (void)hipStreamSynchronize(c->side);
  if (c->bstream) (void)hipStreamSynchronize(c->bstream);
  c->destroy_streams();
  c->release_all();
  delete c;
}

int64_t ttt_position(const ttt_ctx* c) { return c ? c->pos : -1; }

int ttt_reset(ttt_ctx* c) {
  if (!c) return TTT_EINVAL;
  return reset_state(c);
}

int ttt_prefill(ttt_ctx* c, const int32_t* tokens, const int32_t* targets, int64_t n_tokens, float* losses) {
  if (!c) return TTT_EINVAL;
  if (c->poisoned) return fail(c, TTT_ESTATE, "context poisoned; call ttt_reset");
  if (!tokens || !targets || n_tokens <= 0) return fail(c, TTT_EINVAL, "NULL tokens/targets or n_tokens <= 0");
  if (c->pos + n_tokens > c->cfg.max_positions) return fail(c, TTT_EINVAL, "beyond max_positions");
  const int64_t cnt = (int64_t)c->B * n_tokens;
  if (!check_ids(c, tokens, cnt, false)) return fail(c, TTT_EINVAL, "token id out of range");
  if (!check_ids(c, targets, cnt, true)) return fail(c, TTT_EINVAL, "target id out of range");
  const int64_t nch = (n_tokens + c->b - 1) / c->b;
  int rc;
  if ((rc = ensure_tok(c, 2 * cnt))) return rc;
  if ((rc = ensure_loss(c, nch * c->B))) return rc;
  CK(hipMemcpyAsync(c->d_tok, tokens, cnt * 4, hipMemcpyHostToDevice, c->stream));
  CK(hipMemcpyAsync(c->d_tok + cnt, targets, cnt * 4, hipMemcpyHostToDevice, c->stream));
  rc = run_dispatch(c, c->d_tok, c->d_tok + cnt, n_tokens, n_tokens, c->d_loss);
  if (rc) return rc;
  std::vector<float> tmp(nch * c->B);
  rc = sync_and_check(c, c->d_loss, nch * c->B, tmp.data());
  if (rc) return rc;
  if (losses)
    for (int64_t ch = 0; ch < nch; ++ch)
      for (int r = 0; r < c->B; ++r) losses[(int64_t)r * nch + ch] = tmp[ch * c->B + r];
  return TTT_OK;
}

int ttt_score(ttt_ctx* c, const int32_t* tokens, const int32_t* targets, int64_t n_tokens, float* losses) {
  if (!c) return TTT_EINVAL;
  if (c->poisoned) return fail(c, TTT_ESTATE, "context poisoned; call ttt_reset");
  if (!tokens || !targets || n_tokens <= 0) return fail(c, TTT_EINVAL, "NULL tokens/targets or n_tokens <= 0");
  if (c->pos + n_tokens > c->cfg.max_positions) return fail(c, TTT_EINVAL, "beyond max_positions");
  const int64_t cnt = (int64_t)c->B * n_tokens;
  if (!check_ids(c, tokens, cnt, false)) return fail(c, TTT_EINVAL, "token id out of range");
  if (!check_ids(c, targets, cnt, true)) return fail(c, TTT_EINVAL, "target id out of range");
  const int64_t nch = (n_tokens + c->b - 1) / c->b;
  int rc;
  if ((rc = ensure_tok(c, 2 * cnt))) return rc;
  if ((rc = ensure_loss(c, nch * c->B))) return rc;
  CK(sync_aux(c));
  CK(hipMemcpyAsync(c->d_tok, tokens, cnt * 4, hipMemcpyHostToDevice, c->stream));
  CK(hipMemcpyAsync(c->d_tok + cnt, targets, cnt * 4, hipMemcpyHostToDevice, c->stream));
  rc = score_dispatch(c, c->d_tok, c->d_tok + cnt, n_tokens, n_tokens, c->d_loss);
  if (rc) return rc;
  std::vector<float> tmp(nch * c->B);
  rc = sync_and_check(c, c->d_loss, nch * c->B, tmp.data());
  if (rc) return rc;
  if (losses)
    for (int64_t ch = 0; ch < nch; ++ch)
      for (int r = 0; r < c->B; ++r) losses[(int64_t)r * nch + ch] = tmp[ch * c->B + r];
  return TTT_OK;
}

int ttt_score_device(ttt_ctx* c, const int32_t* d_tokens, const int32_t* d_targets, int64_t n_tokens,
                     float* d_losses) {
  if (!c) return TTT_EINVAL;
  if (c->poisoned) return fail(c, TTT_ESTATE, "context poisoned; call ttt_reset");
  if (!d_tokens || !d_targets || n_tokens <= 0) return fail(c, TTT_EINVAL, "NULL tokens/targets or n_tokens <= 0");
  if (c->pos + n_tokens > c->cfg.max_positions) return fail(c, TTT_EINVAL, "beyond max_positions");
  const int64_t nch = (n_tokens + c->b - 1) / c->b;
  if (!d_losses) {
    int rc = ensure_loss(c, nch * c->B);
    if (rc) return rc;
    d_losses = c->d_loss;
  }
  // (a batched pass of an earlier prefill may still be writing the shared buffers)
  if (c->bstream) {
    CK(hipEventRecord(c->ev_c2b, c->bstream));
    CK(hipStreamWaitEvent(c->stream, c->ev_c2b, 0));
  }
  int rc = score_dispatch(c, d_tokens, d_targets, n_tokens, n_tokens, d_losses);
  if (rc) return rc;
  c->pending_loss = d_losses;
  c->pending_n = nch * c->B;
  return TTT_OK;
}

int ttt_prefill_chunk(ttt_ctx* c, const int32_t* tokens, const int32_t* targets, int32_t n, float* loss_out) {
  if (!c) return TTT_EINVAL;
  if (n <= 0 || n > c->b) return fail(c, TTT_EINVAL, "n must be in 1..chunk");
  return ttt_prefill(c, tokens, targets, n, loss_out);
}

int ttt_prefill_device(ttt_ctx* c, const int32_t* d_tokens, const int32_t* d_targets, int64_t n_tokens,
                       float* d_losses) {
  if (!c) return TTT_EINVAL;
  if (c->poisoned) return fail(c, TTT_ESTATE, "context poisoned; call ttt_reset");
  if (!d_tokens || !d_targets || n_tokens <= 0) return fail(c, TTT_EINVAL, "NULL tokens/targets or n_tokens <= 0");
  if (c->pos + n_tokens > c->cfg.max_positions) return fail(c, TTT_EINVAL, "beyond max_positions");
  const int64_t nch = (n_tokens + c->b - 1) / c->b;
  if (!d_losses) {
    int rc = ensure_loss(c, nch * c->B);
    if (rc) return rc;
    d_losses = c->d_loss;
  }
  int rc = run_dispatch(c, d_tokens, d_targets, n_tokens, n_tokens, d_losses);
  if (rc) return rc;
  c->pending_loss = d_losses;
  c->pending_n = nch * c->B;
  return TTT_OK;
}

int ttt_sync(ttt_ctx* c) {
  if (!c) return TTT_EINVAL;
  if (c->poisoned) return fail(c, TTT_ESTATE, "context poisoned; call ttt_reset");
  int rc = sync_and_check(c, c->pending_loss, c->pending_n, nullptr);
  c->pending_loss = nullptr;
  c->pending_n = 0;
  return rc;
}

int ttt_generate(ttt_ctx* c, const int32_t* first_input, int32_t n_new, int32_t update_every, int32_t* out_tokens,
                 float* update_losses) {
  if (!c) return TTT_EINVAL;
  if (c->poisoned) return fail(c, TTT_ESTATE, "context poisoned; call ttt_reset");
  if (!first_input || !out_tokens || n_new < 0) return fail(c, TTT_EINVAL, "bad generate arguments");
  if (update_every < 1 || update_every > c->b) return fail(c, TTT_EINVAL, "update_every must be in 1..chunk");
  if (c->pos + n_new > c->cfg.max_positions) return fail(c, TTT_EINVAL, "beyond max_positions");
  if (!check_ids(c, first_input, c->B, false)) return fail(c, TTT_EINVAL, "first_input id out of range");
  if (n_new == 0) return TTT_OK;
  const int64_t ld = (int64_t)n_new + 1;
  const int nu = n_new / update_every;
  int rc;
  if ((rc = ensure_tok(c, ld * c->B))) return rc;
  if ((rc = ensure_loss(c, (int64_t)std::max(nu, 1) * c->B))) return rc;
  CK(hipMemcpy2DAsync(c->d_tok, ld * 4, first_input, 4, 4, c->B, hipMemcpyHostToDevice, c->stream));
  int upd = 0;
  for (int j = 0; j < n_new; ++j) {
    rc = decode_dispatch(c, c->d_tok + j, ld);
    if (rc) return rc;
    if ((j + 1) % update_every == 0) {
      const int j0 = j + 1 - update_every;
      c->pos -= update_every;
      rc = run_dispatch(c, c->d_tok + j0, c->d_tok + j0 + 1, ld, update_every, c->d_loss + (int64_t)upd * c->B);
      if (rc) return rc;
      ++upd;
    }
  }
  std::vector<float> tmp((size_t)std::max(nu, 1) * c->B);
  rc = sync_and_check(c, c->d_loss, (int64_t)nu * c->B, tmp.data());
  if (rc) return rc;
  std::vector<int32_t> all((size_t)ld * c->B);
  CK(hipMemcpy(all.data(), c->d_tok, ld * c->B * 4, hipMemcpyDeviceToHost));
  for (int r = 0; r < c->B; ++r)
    for (int j = 0; j < n_new; ++j) out_tokens[(int64_t)r * n_new + j] = all[(size_t)r * ld + j + 1];
  if (update_losses)
    for (int u = 0; u < nu; ++u)
      for (int r = 0; r < c->B; ++r) update_losses[(int64_t)r * nu + u] = tmp[(size_t)u * c->B + r];
  return TTT_OK;
}

int ttt_set_fast_weights(ttt_ctx* c, int32_t row, const float* src, int64_t n_floats) {
  if (!c) return TTT_EINVAL;
  if (c->poisoned) return fail(c, TTT_ESTATE, "context poisoned; call ttt_reset");
  if (!src || row < 0 || row >= c->B) return fail(c, TTT_EINVAL, "bad row or NULL src");
  const int64_t fsz = 3LL * c->f * c->d;
  if (n_floats != fsz * c->Lq) return fail(c, TTT_EINVAL, "n_floats must be 3*d*f*n_fast");
  CK(sync_aux(c));
  for (int j = 0; j < c->Lq; ++j)
    CK(hipMemcpyAsync(c->fw[j].master + row * fsz, src + j * fsz, fsz * 4, hipMemcpyHostToDevice, c->stream));
  CK(refresh_fast_shadows(c));
  CK(hipStreamSynchronize(c->stream));
  return TTT_OK;
}

int64_t ttt_state_size(const ttt_ctx* c) {
  if (!c) return -1;
  int64_t n = STATE_HDR * 8;
  (void)for_state_arrays(const_cast<ttt_ctx*>(c), [&](void*, int64_t bytes) {
    n += bytes;
    return hipSuccess;
  });
  return n;
}

int ttt_save_state(ttt_ctx* c, void* dst, int64_t nbytes) {
  if (!c) return TTT_EINVAL;
  if (c->poisoned) return fail(c, TTT_ESTATE, "context poisoned; call ttt_reset");
  if (!dst || nbytes < ttt_state_size(c)) return fail(c, TTT_EINVAL, "NULL dst or nbytes below ttt_state_size");
  CK(sync_aux(c));
  // device-side errors of earlier asynchronous work (a bad id, a non-finite loss) poison the
  // context here instead of travelling inside the snapshot
  {
    int rc = sync_and_check(c, c->pending_loss, c->pending_n, nullptr);
    c->pending_loss = nullptr;
    c->pending_n = 0;
    if (rc) return rc;
  }
  state_header(c, (int64_t*)dst);
  char* p = (char*)dst + STATE_HDR * 8;
  CK(for_state_arrays(c, [&](void* a, int64_t bytes) {
    hipError_t e = hipMemcpy(p, a, bytes, hipMemcpyDeviceToHost);
    p += bytes;
    return e;
  }));
  return TTT_OK;
}

int ttt_load_state(ttt_ctx* c, const void* src, int64_t nbytes) {
  if (!c) return TTT_EINVAL;
  if (!src || nbytes < ttt_state_size(c)) return fail(c, TTT_EINVAL, "NULL src or nbytes below ttt_state_size");
  int64_t want[STATE_HDR];
  state_header(c, want);
  const int64_t* got = (const int64_t*)src;
  for (int i = 0; i < STATE_HDR; ++i)
    if (i != 11 && got[i] != want[i]) return fail(c, TTT_EINVAL, "snapshot of another configuration");
  if (got[11] < 0 || got[11] > c->cfg.max_positions) return fail(c, TTT_EINVAL, "snapshot position out of range");
  CK(sync_aux(c));
  CK(hipStreamSynchronize(c->stream));
  const char* p = (const char*)src + STATE_HDR * 8;
  CK(for_state_arrays(c, [&](void* a, int64_t bytes) {
    hipError_t e = hipMemcpy(a, p, bytes, hipMemcpyHostToDevice);
    p += bytes;
    return e;
  }));
  CK(refresh_fast_shadows(c));
  CK(hipMemsetAsync(c->err_dev, 0, 4, c->stream));
  CK(hipStreamSynchronize(c->stream));
  c->pos = got[11];
  c->pend_parts = 0;
  c->poisoned = false;
  c->pending_loss = nullptr;
  c->pending_n = 0;
  return TTT_OK;
}

int ttt_get_fast_weights(ttt_ctx* c, int32_t row, float* dst, int64_t n_floats) {
  if (!c) return TTT_EINVAL;
  if (!dst || row < 0 || row >= c->B) return fail(c, TTT_EINVAL, "bad row or NULL dst");
  const int64_t fsz = 3LL * c->f * c->d;
  if (n_floats != fsz * c->Lq) return fail(c, TTT_EINVAL, "n_floats must be 3*d*f*n_fast");
  CK(hipStreamSynchronize(c->stream));
  for (int j = 0; j < c->Lq; ++j)
    CK(hipMemcpy(dst + j * fsz, c->fw[j].master + row * fsz, fsz * 4, hipMemcpyDeviceToHost));
  return TTT_OK;
}

}  // extern "C"
