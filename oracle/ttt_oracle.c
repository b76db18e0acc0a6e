/*
 * ORACLE for the TTT-E2E inner loop -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU implementation of what the inner loop computes.
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * may load this library; the product path never calls it, and it shares no
 * code, header or table with the HIP path.
 *
 * What it follows (page title, then section):
 *  - "TTT-E2E 如何让大模型边用边学" §4.4 (pseudo-code): the text is read in
 *    non-overlapping chunks of b tokens; for each chunk the model runs with a
 *    sliding window, the next-token cross-entropy of the chunk is taken (mean
 *    reduction, the default of a cross-entropy call), back-propagated, and one
 *    optimizer step touches only the MLPs of the last quarter of the blocks.
 *  - same page §4.2: b = 1k, only the last 1/4 of the layers' MLPs change, the
 *    key/value cache covers only the window.
 *  - same page §8 Q1: history activations are not kept, so keys/values of
 *    earlier chunks enter as constants (no gradient into them).
 *  - same page §8 Q4: the window k must be at least b.
 *  - "突破大语言模型上下文限制的新范式" §2.1: one gradient step per update,
 *    on mlp_layers[-len//4:] only; §2.2: during generation an update follows
 *    every ~1000 generated tokens.
 *  - "测试时训练：长上下文的持续学习" §2.1.2: the training signal is
 *    -log p(x_{t+1} | x_<=t) and the step is theta <- theta - eta * grad.
 *  - "从KV Cache到权重压缩：大模型持续学习的新范式" §2.2: 1-3 gradient steps per
 *    update (n_steps), and optionally two MLPs in each updated block, a static
 *    one that keeps what pretraining stored and a dynamic one that adapts
 *    (dual_mlp: both read the block's MLP RMSNorm output and their outputs
 *    add; only the dynamic one is updated).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  window = k keys including the query itself (t-k < s <= t); Llama-style
 *  pre-norm block (RMSNorm, rotate-half RoPE, MHA, SwiGLU MLP, untied
 *  lm_head, no biases); attention scale 1/sqrt(head_dim); plain SGD without
 *  momentum, weight decay or clipping; targets equal to -1 are ignored, a
 *  chunk without valid targets has loss 0 and leaves the weights unchanged;
 *  the reported loss is the one before the chunk's update; cached keys and
 *  values are not recomputed after an update; batch rows are independent
 *  sequences, each with its own fast weights and key/value history.
 *
 * Every function computes its definition directly, in fp64, in the order the
 * definition states.  Frozen weights are read as given (fp32 arrays that hold
 * bf16-representable values for bf16 workloads; widening to fp64 is exact).
 * The fast weights and the key/value store are fp64.  The store keeps every
 * position by its absolute index (no ring).  The frozen weight arrays are
 * referenced, not copied: the caller keeps them alive until oracle_destroy.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t n_layers, d_model, n_heads, d_ff, vocab, window, chunk, n_fast, batch;
  int32_t n_steps; /* SGD steps per chunk; 0 and 1 both mean one */
  int32_t dual_mlp; /* 1: static + dynamic MLP in every updated block */
  double rope_theta, rms_eps, lr;
} oracle_cfg;

typedef struct {
  const float* embed;      /* [V, d] */
  const float* final_norm; /* [d] */
  const float* lm_head;    /* [V, d] */
  const float* const* attn_norm; /* L x [d] */
  const float* const* wq;        /* L x [d, d] */
  const float* const* wk;
  const float* const* wv;
  const float* const* wo;
  const float* const* mlp_norm;  /* L x [d] */
  const float* const* w_gate;    /* L x [f, d] */
  const float* const* w_up;      /* L x [f, d] */
  const float* const* w_down;    /* L x [d, f] */
  /* dual_mlp only: initial weights of the dynamic MLP of updated block j (layer L - n_fast + j),
     n_fast entries each; the static MLP of those blocks is w_gate / w_up / w_down above */
  const float* const* dyn_gate;  /* n_fast x [f, d] */
  const float* const* dyn_up;    /* n_fast x [f, d] */
  const float* const* dyn_down;  /* n_fast x [d, f] */
} oracle_weights;

/* saved activations of one layer for the current chunk */
typedef struct {
  double *h_in, *u, *rstd1, *q, *k, *v, *att, *h_mid, *m, *rstd2, *zg, *zu, *act;
  double *zg_s, *zu_s; /* static MLP of an updated block (dual_mlp), else NULL */
} layer_acts;

typedef struct {
  double* fast;  /* Lq blocks x [W_gate f*d | W_up f*d | W_down d*f] */
  double* kst;   /* L x [max_pos, d]  rotated keys by absolute position */
  double* vst;   /* L x [max_pos, d]  values by absolute position */
  int64_t pos;
} row_state;

typedef struct {
  oracle_cfg c;
  oracle_weights w;
  const float** ptrs; /* storage for the per-layer pointer arrays */
  int64_t max_pos;
  row_state* rows;
  double* fast0; /* initial fast weights (shared by all rows) */
} oracle_state;

static int L_(const oracle_state* s) { return s->c.n_layers; }
static int64_t fast_block(const oracle_cfg* c) { return 3 * (int64_t)c->d_ff * c->d_model; }
static int l0_of(const oracle_cfg* c) { return c->n_layers - c->n_fast; }

/* ---------------------------------------------------------------- primitives */

/* Y[t][o] = sum_i X[t][i] * W[o][i]   (y = x W^T), W fp32 */
static void mm_xwt_f(const double* X, int n, int din, const float* W, int dout, double* Y) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int t = 0; t < n; ++t)
    for (int o = 0; o < dout; ++o) {
      const double* x = X + (int64_t)t * din;
      const float* w = W + (int64_t)o * din;
      double acc = 0.0;
      for (int i = 0; i < din; ++i) acc += x[i] * (double)w[i];
      Y[(int64_t)t * dout + o] = acc;
    }
}

/* same with fp64 W */
static void mm_xwt_d(const double* X, int n, int din, const double* W, int dout, double* Y) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int t = 0; t < n; ++t)
    for (int o = 0; o < dout; ++o) {
      const double* x = X + (int64_t)t * din;
      const double* w = W + (int64_t)o * din;
      double acc = 0.0;
      for (int i = 0; i < din; ++i) acc += x[i] * w[i];
      Y[(int64_t)t * dout + o] = acc;
    }
}

/* dX[t][i] = sum_o dY[t][o] * W[o][i]   (gradient of y = x W^T w.r.t. x), W fp32 */
static void mm_dyw_f(const double* dY, int n, int dout, const float* W, int din, double* dX) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < n; ++t) {
    double* dx = dX + (int64_t)t * din;
    for (int i = 0; i < din; ++i) dx[i] = 0.0;
    for (int o = 0; o < dout; ++o) {
      double g = dY[(int64_t)t * dout + o];
      const float* w = W + (int64_t)o * din;
      for (int i = 0; i < din; ++i) dx[i] += g * (double)w[i];
    }
  }
}

static void mm_dyw_d(const double* dY, int n, int dout, const double* W, int din, double* dX) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < n; ++t) {
    double* dx = dX + (int64_t)t * din;
    for (int i = 0; i < din; ++i) dx[i] = 0.0;
    for (int o = 0; o < dout; ++o) {
      double g = dY[(int64_t)t * dout + o];
      const double* w = W + (int64_t)o * din;
      for (int i = 0; i < din; ++i) dx[i] += g * w[i];
    }
  }
}

/* dW[o][i] = sum_t dY[t][o] * X[t][i]   (gradient of y = x W^T w.r.t. W) */
static void mm_dw(const double* dY, const double* X, int n, int dout, int din, double* dW) {
#pragma omp parallel for schedule(static)
  for (int o = 0; o < dout; ++o) {
    double* dw = dW + (int64_t)o * din;
    for (int i = 0; i < din; ++i) dw[i] = 0.0;
    for (int t = 0; t < n; ++t) {
      double g = dY[(int64_t)t * dout + o];
      const double* x = X + (int64_t)t * din;
      for (int i = 0; i < din; ++i) dw[i] += g * x[i];
    }
  }
}

/* RMSNorm(x; g) = g * x / sqrt(mean(x^2) + eps); rstd saved per row */
void oracle_rmsnorm(const double* X, int n, int d, const float* g, double eps, double* Y, double* rstd) {
  for (int t = 0; t < n; ++t) {
    const double* x = X + (int64_t)t * d;
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss / d + eps);
    if (rstd) rstd[t] = r;
    for (int i = 0; i < d; ++i) Y[(int64_t)t * d + i] = (double)g[i] * x[i] * r;
  }
}

/* gradient of RMSNorm: given dy, returns dx (overwrites) with
   dx_i = r g_i dy_i - x_i r^3 (1/d) sum_j g_j dy_j x_j */
static void rmsnorm_bwd(const double* X, const double* rstd, int n, int d, const float* g, const double* dY,
                        double* dX) {
  for (int t = 0; t < n; ++t) {
    const double* x = X + (int64_t)t * d;
    const double* dy = dY + (int64_t)t * d;
    double r = rstd[t], dot = 0.0;
    for (int i = 0; i < d; ++i) dot += (double)g[i] * dy[i] * x[i];
    for (int i = 0; i < d; ++i) dX[(int64_t)t * d + i] = r * (double)g[i] * dy[i] - x[i] * r * r * r * dot / d;
  }
}

/* rotate-half RoPE of one head vector at absolute position pos:
   pairs (i, i + hd/2), angle = pos * theta^(-2i/hd).  sign = +1 forward,
   -1 applies the inverse rotation (which is also the gradient map). */
void oracle_rope(const double* x, int hd, int64_t pos, double theta, int sign, double* y) {
  int half = hd / 2;
  for (int i = 0; i < half; ++i) {
    double inv_freq = pow(theta, -2.0 * i / hd);
    double ang = (double)pos * inv_freq;
    double c = cos(ang), s = sin(ang) * sign;
    double a = x[i], b = x[i + half];
    y[i] = a * c - b * s;
    y[i + half] = b * c + a * s;
  }
}

static double silu(double z) { return z / (1.0 + exp(-z)); }
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* ------------------------------------------------------------------ state */

static void* xcalloc(size_t n, size_t sz) { return calloc(n ? n : 1, sz); }

oracle_state* oracle_create(const oracle_cfg* cfg, const oracle_weights* w, int64_t max_positions) {
  if (!cfg || !w || max_positions <= 0) return NULL;
  const oracle_cfg c = *cfg;
  if (c.n_layers <= 0 || c.d_model <= 0 || c.n_heads <= 0 || c.d_model % c.n_heads || (c.d_model / c.n_heads) % 2 ||
      c.d_ff <= 0 || c.vocab <= 0 || c.chunk <= 0 || c.window < c.chunk || c.n_fast < 1 || c.n_fast > c.n_layers ||
      c.batch <= 0 || c.n_steps < 0 || c.dual_mlp < 0 || c.dual_mlp > 1)
    return NULL;
  if (c.dual_mlp && (!w->dyn_gate || !w->dyn_up || !w->dyn_down)) return NULL;
  oracle_state* s = (oracle_state*)xcalloc(1, sizeof(oracle_state));
  s->c = c;
  s->max_pos = max_positions;
  int L = c.n_layers;
  s->ptrs = (const float**)xcalloc((size_t)9 * L, sizeof(float*));
  const float** p = s->ptrs;
  const float* const* src[9] = {w->attn_norm, w->wq, w->wk, w->wv, w->wo, w->mlp_norm, w->w_gate, w->w_up, w->w_down};
  for (int a = 0; a < 9; ++a)
    for (int l = 0; l < L; ++l) p[a * L + l] = src[a][l];
  s->w.embed = w->embed;
  s->w.final_norm = w->final_norm;
  s->w.lm_head = w->lm_head;
  s->w.attn_norm = p + 0 * L;
  s->w.wq = p + 1 * L;
  s->w.wk = p + 2 * L;
  s->w.wv = p + 3 * L;
  s->w.wo = p + 4 * L;
  s->w.mlp_norm = p + 5 * L;
  s->w.w_gate = p + 6 * L;
  s->w.w_up = p + 7 * L;
  s->w.w_down = p + 8 * L;
  s->w.dyn_gate = w->dyn_gate;
  s->w.dyn_up = w->dyn_up;
  s->w.dyn_down = w->dyn_down;

  int64_t fd = (int64_t)c.d_ff * c.d_model, blk = fast_block(&c);
  s->fast0 = (double*)xcalloc((size_t)(blk * c.n_fast), sizeof(double));
  for (int j = 0; j < c.n_fast; ++j) {
    /* the updated MLP: the block's own, or its dynamic one */
    int l = l0_of(&c) + j;
    const float* gsrc = c.dual_mlp ? w->dyn_gate[j] : w->w_gate[l];
    const float* usrc = c.dual_mlp ? w->dyn_up[j] : w->w_up[l];
    const float* dsrc = c.dual_mlp ? w->dyn_down[j] : w->w_down[l];
    double* dst = s->fast0 + j * blk;
    for (int64_t i = 0; i < fd; ++i) {
      dst[i] = gsrc[i];
      dst[fd + i] = usrc[i];
      dst[2 * fd + i] = dsrc[i];
    }
  }
  s->rows = (row_state*)xcalloc((size_t)c.batch, sizeof(row_state));
  for (int r = 0; r < c.batch; ++r) {
    row_state* rs = &s->rows[r];
    rs->fast = (double*)xcalloc((size_t)(blk * c.n_fast), sizeof(double));
    memcpy(rs->fast, s->fast0, sizeof(double) * (size_t)(blk * c.n_fast));
    rs->kst = (double*)xcalloc((size_t)(L * max_positions * c.d_model), sizeof(double));
    rs->vst = (double*)xcalloc((size_t)(L * max_positions * c.d_model), sizeof(double));
    if (!rs->fast || !rs->kst || !rs->vst) return NULL;
    rs->pos = 0;
  }
  return s;
}

void oracle_destroy(oracle_state* s) {
  if (!s) return;
  for (int r = 0; r < s->c.batch; ++r) {
    free(s->rows[r].fast);
    free(s->rows[r].kst);
    free(s->rows[r].vst);
  }
  free(s->rows);
  free(s->fast0);
  free(s->ptrs);
  free(s);
}

int64_t oracle_get_pos(const oracle_state* s, int row) { return s->rows[row].pos; }
int64_t oracle_fast_size(const oracle_state* s) { return fast_block(&s->c) * s->c.n_fast; }

int oracle_get_fast(const oracle_state* s, int row, double* dst) {
  if (row < 0 || row >= s->c.batch) return -1;
  memcpy(dst, s->rows[row].fast, sizeof(double) * (size_t)oracle_fast_size(s));
  return 0;
}

int oracle_set_fast(oracle_state* s, int row, const double* src) {
  if (row < 0 || row >= s->c.batch) return -1;
  memcpy(s->rows[row].fast, src, sizeof(double) * (size_t)oracle_fast_size(s));
  return 0;
}

/* fast weights of layer l (l >= l0) for a row */
static double* fast_gate(const oracle_state* s, row_state* rs, int l) {
  return rs->fast + (int64_t)(l - l0_of(&s->c)) * fast_block(&s->c);
}

/* ---------------------------------------------------------- one chunk, one row */

typedef struct {
  int n;                 /* positions in this chunk */
  int64_t p0;            /* absolute position of the first */
  layer_acts* acts;      /* per layer */
  double *h_final, *hf, *rstdf, *logits;
} chunk_work;

static void acts_alloc(layer_acts* a, int n, int d, int f, int dual) {
  a->h_in = xcalloc((size_t)n * d, 8);
  a->u = xcalloc((size_t)n * d, 8);
  a->rstd1 = xcalloc((size_t)n, 8);
  a->q = xcalloc((size_t)n * d, 8);
  a->k = xcalloc((size_t)n * d, 8);
  a->v = xcalloc((size_t)n * d, 8);
  a->att = xcalloc((size_t)n * d, 8);
  a->h_mid = xcalloc((size_t)n * d, 8);
  a->m = xcalloc((size_t)n * d, 8);
  a->rstd2 = xcalloc((size_t)n, 8);
  a->zg = xcalloc((size_t)n * f, 8);
  a->zu = xcalloc((size_t)n * f, 8);
  a->act = xcalloc((size_t)n * f, 8);
  a->zg_s = dual ? xcalloc((size_t)n * f, 8) : NULL;
  a->zu_s = dual ? xcalloc((size_t)n * f, 8) : NULL;
}

static void acts_free(layer_acts* a) {
  free(a->h_in); free(a->u); free(a->rstd1); free(a->q); free(a->k); free(a->v); free(a->att);
  free(a->h_mid); free(a->m); free(a->rstd2); free(a->zg); free(a->zu); free(a->act);
  free(a->zg_s); free(a->zu_s);
}

/* first key position visible from query position t: window of k keys incl. t */
static int64_t first_key(int64_t t, int k) { return t - k + 1 > 0 ? t - k + 1 : 0; }

/* Forward of positions [p0, p0+n) of one row.  Writes rotated keys and values
   of these positions into the row's store (overwriting), and fills work. */
static void forward_chunk(const oracle_state* s, row_state* rs, const int32_t* ids, chunk_work* wk) {
  const oracle_cfg* c = &s->c;
  int n = wk->n, d = c->d_model, f = c->d_ff, H = c->n_heads, hd = d / H, L = c->n_layers, V = c->vocab;
  int l0 = l0_of(c);
  int64_t p0 = wk->p0;
  double scale = 1.0 / sqrt((double)hd);
  double* h = xcalloc((size_t)n * d, 8);
  for (int t = 0; t < n; ++t)
    for (int i = 0; i < d; ++i) h[(int64_t)t * d + i] = s->w.embed[(int64_t)ids[t] * d + i];
  double* tmp = xcalloc((size_t)n * (d > f ? d : f), 8);
  for (int l = 0; l < L; ++l) {
    layer_acts* a = &wk->acts[l];
    memcpy(a->h_in, h, sizeof(double) * (size_t)n * d);
    oracle_rmsnorm(h, n, d, s->w.attn_norm[l], c->rms_eps, a->u, a->rstd1);
    mm_xwt_f(a->u, n, d, s->w.wq[l], d, tmp);
    for (int t = 0; t < n; ++t)
      for (int hh = 0; hh < H; ++hh)
        oracle_rope(tmp + (int64_t)t * d + hh * hd, hd, p0 + t, c->rope_theta, +1, a->q + (int64_t)t * d + hh * hd);
    mm_xwt_f(a->u, n, d, s->w.wk[l], d, tmp);
    for (int t = 0; t < n; ++t)
      for (int hh = 0; hh < H; ++hh)
        oracle_rope(tmp + (int64_t)t * d + hh * hd, hd, p0 + t, c->rope_theta, +1, a->k + (int64_t)t * d + hh * hd);
    mm_xwt_f(a->u, n, d, s->w.wv[l], d, a->v);
    double* ks = rs->kst + (int64_t)l * s->max_pos * d;
    double* vs = rs->vst + (int64_t)l * s->max_pos * d;
    memcpy(ks + p0 * d, a->k, sizeof(double) * (size_t)n * d);
    memcpy(vs + p0 * d, a->v, sizeof(double) * (size_t)n * d);
    /* attention over S_t = {first_key(t) .. t} */
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int t = 0; t < n; ++t)
      for (int hh = 0; hh < H; ++hh) {
        int64_t pt = p0 + t, s0 = first_key(pt, c->window);
        int64_t cnt = pt - s0 + 1;
        double* sc = malloc(sizeof(double) * (size_t)cnt);
        const double* qv = a->q + (int64_t)t * d + hh * hd;
        double mx = -INFINITY;
        for (int64_t j = 0; j < cnt; ++j) {
          const double* kv = ks + (s0 + j) * d + hh * hd;
          double dot = 0.0;
          for (int i = 0; i < hd; ++i) dot += qv[i] * kv[i];
          sc[j] = dot * scale;
          if (sc[j] > mx) mx = sc[j];
        }
        double den = 0.0;
        for (int64_t j = 0; j < cnt; ++j) { sc[j] = exp(sc[j] - mx); den += sc[j]; }
        double* o = a->att + (int64_t)t * d + hh * hd;
        for (int i = 0; i < hd; ++i) o[i] = 0.0;
        for (int64_t j = 0; j < cnt; ++j) {
          double pj = sc[j] / den;
          const double* vv = vs + (s0 + j) * d + hh * hd;
          for (int i = 0; i < hd; ++i) o[i] += pj * vv[i];
        }
        free(sc);
      }
    mm_xwt_f(a->att, n, d, s->w.wo[l], d, tmp);
    for (int64_t i = 0; i < (int64_t)n * d; ++i) a->h_mid[i] = h[i] + tmp[i];
    oracle_rmsnorm(a->h_mid, n, d, s->w.mlp_norm[l], c->rms_eps, a->m, a->rstd2);
    if (l >= l0) {
      double* wg = fast_gate(s, rs, l);
      int64_t fd = (int64_t)f * d;
      mm_xwt_d(a->m, n, d, wg, f, a->zg);
      mm_xwt_d(a->m, n, d, wg + fd, f, a->zu);
      for (int64_t i = 0; i < (int64_t)n * f; ++i) a->act[i] = silu(a->zg[i]) * a->zu[i];
      mm_xwt_d(a->act, n, f, wg + 2 * fd, d, tmp);
      if (c->dual_mlp) {
        /* the static MLP reads the same normed input; the two outputs add */
        double* act_s = xcalloc((size_t)n * f, 8);
        double* y_s = xcalloc((size_t)n * d, 8);
        mm_xwt_f(a->m, n, d, s->w.w_gate[l], f, a->zg_s);
        mm_xwt_f(a->m, n, d, s->w.w_up[l], f, a->zu_s);
        for (int64_t i = 0; i < (int64_t)n * f; ++i) act_s[i] = silu(a->zg_s[i]) * a->zu_s[i];
        mm_xwt_f(act_s, n, f, s->w.w_down[l], d, y_s);
        for (int64_t i = 0; i < (int64_t)n * d; ++i) tmp[i] += y_s[i];
        free(act_s);
        free(y_s);
      }
    } else {
      mm_xwt_f(a->m, n, d, s->w.w_gate[l], f, a->zg);
      mm_xwt_f(a->m, n, d, s->w.w_up[l], f, a->zu);
      for (int64_t i = 0; i < (int64_t)n * f; ++i) a->act[i] = silu(a->zg[i]) * a->zu[i];
      mm_xwt_f(a->act, n, f, s->w.w_down[l], d, tmp);
    }
    for (int64_t i = 0; i < (int64_t)n * d; ++i) h[i] = a->h_mid[i] + tmp[i];
  }
  memcpy(wk->h_final, h, sizeof(double) * (size_t)n * d);
  oracle_rmsnorm(h, n, d, s->w.final_norm, c->rms_eps, wk->hf, wk->rstdf);
  mm_xwt_f(wk->hf, n, d, s->w.lm_head, V, wk->logits);
  free(tmp);
  free(h);
}

/* mean next-token cross-entropy over valid targets; dlogits if requested */
static double chunk_loss(const oracle_cfg* c, const double* logits, const int32_t* tgt, int n, double* dlogits) {
  int V = c->vocab, nvalid = 0;
  for (int t = 0; t < n; ++t) nvalid += tgt[t] >= 0;
  double loss = 0.0;
  for (int t = 0; t < n; ++t) {
    const double* z = logits + (int64_t)t * V;
    double mx = -INFINITY;
    for (int v = 0; v < V; ++v) if (z[v] > mx) mx = z[v];
    double se = 0.0;
    for (int v = 0; v < V; ++v) se += exp(z[v] - mx);
    double lse = mx + log(se);
    if (tgt[t] >= 0) loss += lse - z[tgt[t]];
    if (dlogits) {
      double* dz = dlogits + (int64_t)t * V;
      for (int v = 0; v < V; ++v) {
        if (tgt[t] < 0) { dz[v] = 0.0; continue; }
        double p = exp(z[v] - lse);
        dz[v] = (p - (v == tgt[t] ? 1.0 : 0.0)) / nvalid;
      }
    }
  }
  return nvalid ? loss / nvalid : 0.0;
}

/* Hand-written backward of the chunk loss w.r.t. the row's fast weights.
   Keys/values stored for positions before p0 are constants. */
static void backward_chunk(const oracle_state* s, row_state* rs, const chunk_work* wk, const double* dlogits,
                           double* grad) {
  const oracle_cfg* c = &s->c;
  int n = wk->n, d = c->d_model, f = c->d_ff, H = c->n_heads, hd = d / H, L = c->n_layers, V = c->vocab;
  int l0 = l0_of(c);
  int64_t p0 = wk->p0, fd = (int64_t)f * d, blk = fast_block(c);
  double scale = 1.0 / sqrt((double)hd);
  double* dh = xcalloc((size_t)n * d, 8);
  double* tmp = xcalloc((size_t)n * d, 8);
  double* dact = xcalloc((size_t)n * f, 8);
  double* dzg = xcalloc((size_t)n * f, 8);
  double* dzu = xcalloc((size_t)n * f, 8);
  double* dq = xcalloc((size_t)n * d, 8);
  double* dk = xcalloc((size_t)n * d, 8);
  double* dv = xcalloc((size_t)n * d, 8);
  double* dmid = xcalloc((size_t)n * d, 8);

  /* through lm_head and the final norm */
  mm_dyw_f(dlogits, n, V, s->w.lm_head, d, tmp);
  rmsnorm_bwd(wk->h_final, wk->rstdf, n, d, s->w.final_norm, tmp, dh);

  for (int l = L - 1; l >= l0; --l) {
    const layer_acts* a = &wk->acts[l];
    double* wg = fast_gate(s, rs, l);
    double* g = grad + (int64_t)(l - l0) * blk;
    /* MLP: h_out = h_mid + act W_down^T, act = silu(zg) * zu, zg = m Wg^T, zu = m Wu^T */
    mm_dw(dh, a->act, n, d, f, g + 2 * fd);          /* dW_down */
    mm_dyw_d(dh, n, d, wg + 2 * fd, f, dact);       /* d act */
    for (int64_t i = 0; i < (int64_t)n * f; ++i) {
      double sg = sigmoid(a->zg[i]);
      dzu[i] = dact[i] * a->zg[i] * sg;
      dzg[i] = dact[i] * a->zu[i] * sg * (1.0 + a->zg[i] * (1.0 - sg));
    }
    mm_dw(dzg, a->m, n, f, d, g);                    /* dW_gate */
    mm_dw(dzu, a->m, n, f, d, g + fd);               /* dW_up */
    if (l == l0) break;                              /* nothing below has fast weights */
    /* dm = dzg Wg + dzu Wu; then RMSNorm backward; residual */
    mm_dyw_d(dzg, n, f, wg, d, tmp);
    mm_dyw_d(dzu, n, f, wg + fd, d, dmid);
    for (int64_t i = 0; i < (int64_t)n * d; ++i) tmp[i] += dmid[i];
    if (c->dual_mlp) {
      /* the frozen static MLP passes its input gradient on too (its weights get none) */
      mm_dyw_f(dh, n, d, s->w.w_down[l], f, dact);
      for (int64_t i = 0; i < (int64_t)n * f; ++i) {
        double sg = sigmoid(a->zg_s[i]);
        dzu[i] = dact[i] * a->zg_s[i] * sg;
        dzg[i] = dact[i] * a->zu_s[i] * sg * (1.0 + a->zg_s[i] * (1.0 - sg));
      }
      mm_dyw_f(dzg, n, f, s->w.w_gate[l], d, dmid);
      for (int64_t i = 0; i < (int64_t)n * d; ++i) tmp[i] += dmid[i];
      mm_dyw_f(dzu, n, f, s->w.w_up[l], d, dmid);
      for (int64_t i = 0; i < (int64_t)n * d; ++i) tmp[i] += dmid[i];
    }
    rmsnorm_bwd(a->h_mid, a->rstd2, n, d, s->w.mlp_norm[l], tmp, dmid);
    for (int64_t i = 0; i < (int64_t)n * d; ++i) dmid[i] += dh[i]; /* d h_mid */
    /* attention: h_mid = h_in + att W_o^T */
    mm_dyw_f(dmid, n, d, s->w.wo[l], d, tmp);        /* d att */
    const double* ks = rs->kst + (int64_t)l * s->max_pos * d;
    const double* vs = rs->vst + (int64_t)l * s->max_pos * d;
    memset(dq, 0, sizeof(double) * (size_t)n * d);
    memset(dk, 0, sizeof(double) * (size_t)n * d);
    memset(dv, 0, sizeof(double) * (size_t)n * d);
    /* per head; queries processed in order so the in-chunk key sums are sequential */
#pragma omp parallel for schedule(static)
    for (int hh = 0; hh < H; ++hh) {
      for (int t = 0; t < n; ++t) {
        int64_t pt = p0 + t, s0 = first_key(pt, c->window), cnt = pt - s0 + 1;
        double* P = malloc(sizeof(double) * (size_t)cnt);
        double* dP = malloc(sizeof(double) * (size_t)cnt);
        const double* qv = a->q + (int64_t)t * d + hh * hd;
        const double* dO = tmp + (int64_t)t * d + hh * hd;
        double mx = -INFINITY;
        for (int64_t j = 0; j < cnt; ++j) {
          const double* kv = ks + (s0 + j) * d + hh * hd;
          double dot = 0.0;
          for (int i = 0; i < hd; ++i) dot += qv[i] * kv[i];
          P[j] = dot * scale;
          if (P[j] > mx) mx = P[j];
        }
        double den = 0.0;
        for (int64_t j = 0; j < cnt; ++j) { P[j] = exp(P[j] - mx); den += P[j]; }
        for (int64_t j = 0; j < cnt; ++j) P[j] /= den;
        double rowdot = 0.0;
        for (int64_t j = 0; j < cnt; ++j) {
          const double* vv = vs + (s0 + j) * d + hh * hd;
          double dd = 0.0;
          for (int i = 0; i < hd; ++i) dd += dO[i] * vv[i];
          dP[j] = dd;
          rowdot += P[j] * dd;
        }
        double* dqt = dq + (int64_t)t * d + hh * hd;
        for (int64_t j = 0; j < cnt; ++j) {
          int64_t sp = s0 + j;
          double dS = P[j] * (dP[j] - rowdot);
          const double* kv = ks + sp * d + hh * hd;
          for (int i = 0; i < hd; ++i) dqt[i] += dS * scale * kv[i];
          if (sp >= p0) { /* key of this chunk: a function of the fast weights */
            double* dks = dk + (sp - p0) * d + hh * hd;
            double* dvs = dv + (sp - p0) * d + hh * hd;
            for (int i = 0; i < hd; ++i) {
              dks[i] += dS * scale * qv[i];
              dvs[i] += P[j] * dO[i];
            }
          }
        }
        free(P);
        free(dP);
      }
    }
    /* RoPE backward: inverse rotation */
    for (int t = 0; t < n; ++t)
      for (int hh = 0; hh < H; ++hh) {
        double buf[1024];
        double* x = dq + (int64_t)t * d + hh * hd;
        oracle_rope(x, hd, p0 + t, c->rope_theta, -1, buf);
        memcpy(x, buf, sizeof(double) * hd);
        x = dk + (int64_t)t * d + hh * hd;
        oracle_rope(x, hd, p0 + t, c->rope_theta, -1, buf);
        memcpy(x, buf, sizeof(double) * hd);
      }
    /* du = dq Wq + dk Wk + dv Wv */
    double* du = xcalloc((size_t)n * d, 8);
    mm_dyw_f(dq, n, d, s->w.wq[l], d, du);
    mm_dyw_f(dk, n, d, s->w.wk[l], d, tmp);
    for (int64_t i = 0; i < (int64_t)n * d; ++i) du[i] += tmp[i];
    mm_dyw_f(dv, n, d, s->w.wv[l], d, tmp);
    for (int64_t i = 0; i < (int64_t)n * d; ++i) du[i] += tmp[i];
    rmsnorm_bwd(a->h_in, a->rstd1, n, d, s->w.attn_norm[l], du, dh);
    for (int64_t i = 0; i < (int64_t)n * d; ++i) dh[i] += dmid[i]; /* d h_in */
    free(du);
  }
  free(dh); free(tmp); free(dact); free(dzg); free(dzu); free(dq); free(dk); free(dv); free(dmid);
}

static void work_alloc(const oracle_cfg* c, chunk_work* wk, int n) {
  int d = c->d_model, f = c->d_ff, V = c->vocab;
  wk->n = n;
  wk->acts = (layer_acts*)xcalloc((size_t)c->n_layers, sizeof(layer_acts));
  for (int l = 0; l < c->n_layers; ++l) acts_alloc(&wk->acts[l], n, d, f, c->dual_mlp && l >= l0_of(c));
  wk->h_final = xcalloc((size_t)n * d, 8);
  wk->hf = xcalloc((size_t)n * d, 8);
  wk->rstdf = xcalloc((size_t)n, 8);
  wk->logits = xcalloc((size_t)n * V, 8);
}

static void work_free(const oracle_cfg* c, chunk_work* wk) {
  for (int l = 0; l < c->n_layers; ++l) acts_free(&wk->acts[l]);
  free(wk->acts); free(wk->h_final); free(wk->hf); free(wk->rstdf); free(wk->logits);
}

static int ids_ok(const oracle_cfg* c, const int32_t* x, int n, int allow_ignore) {
  for (int t = 0; t < n; ++t) {
    if (x[t] >= c->vocab) return 0;
    if (x[t] < 0 && !(allow_ignore && x[t] == -1)) return 0;
  }
  return 1;
}

/*
 * Loss of one chunk for every row (and optionally its gradient w.r.t. the
 * fast weights), evaluated at the row's current fast weights and position,
 * without updating anything except the key/value store entries of the
 * chunk's own positions.  tokens/targets: [batch, n].  grad: [batch, fast].
 */
int oracle_eval_chunk(oracle_state* s, const int32_t* tokens, const int32_t* targets, int n, double* loss_out,
                      double* grad_out) {
  const oracle_cfg* c = &s->c;
  if (n <= 0 || n > c->chunk) return -1;
  for (int r = 0; r < c->batch; ++r) {
    if (!ids_ok(c, tokens + (int64_t)r * n, n, 0) || !ids_ok(c, targets + (int64_t)r * n, n, 1)) return -1;
    if (s->rows[r].pos + n > s->max_pos) return -2;
  }
  for (int r = 0; r < c->batch; ++r) {
    row_state* rs = &s->rows[r];
    chunk_work wk;
    work_alloc(c, &wk, n);
    wk.p0 = rs->pos;
    forward_chunk(s, rs, tokens + (int64_t)r * n, &wk);
    double* dlog = grad_out ? xcalloc((size_t)n * c->vocab, 8) : NULL;
    double loss = chunk_loss(c, wk.logits, targets + (int64_t)r * n, n, dlog);
    if (loss_out) loss_out[r] = loss;
    if (grad_out) {
      double* g = grad_out + (int64_t)r * oracle_fast_size(s);
      memset(g, 0, sizeof(double) * (size_t)oracle_fast_size(s));
      backward_chunk(s, rs, &wk, dlog, g);
      free(dlog);
    }
    work_free(c, &wk);
  }
  return 0;
}

/*
 * One step of the inner loop for every row: chunk loss at the current fast
 * weights, its gradient, one SGD step  phi <- phi - lr * grad, pos += n.
 * loss_out[batch] receives the loss before the step.
 *
 * With n_steps > 1 (page "从KV Cache到权重压缩：大模型持续学习的新范式", §2.2:
 * one to three gradient steps on what has been read before the next
 * prediction) the chunk is processed n_steps times in a row, each time as
 * above at the weights the previous step left: loss, gradient, SGD.  The
 * chunk's own key/value entries are those of its last forward; loss_out is
 * the loss of the first.
 */
int oracle_prefill_chunk(oracle_state* s, const int32_t* tokens, const int32_t* targets, int n, double* loss_out) {
  int64_t F = oracle_fast_size(s);
  const int steps = s->c.n_steps > 1 ? s->c.n_steps : 1;
  double* grad = xcalloc((size_t)(F * s->c.batch), 8);
  int rc = 0;
  for (int st = 0; st < steps && rc == 0; ++st) {
    rc = oracle_eval_chunk(s, tokens, targets, n, st == 0 ? loss_out : NULL, grad);
    if (rc == 0) {
      for (int r = 0; r < s->c.batch; ++r) {
        double* phi = s->rows[r].fast;
        const double* g = grad + (int64_t)r * F;
        for (int64_t i = 0; i < F; ++i) phi[i] -= s->c.lr * g[i];
      }
    }
  }
  if (rc == 0)
    for (int r = 0; r < s->c.batch; ++r) s->rows[r].pos += n;
  free(grad);
  return rc;
}

/*
 * Greedy generation with a TTT update after every `update_every` generated
 * tokens.  Step j feeds input x (first_input, then the previous output) at
 * the next position, stores its keys/values, and outputs argmax of the
 * logits (lowest id on ties) -- or forced[r][j] when `forced` is given, which
 * lets a caller replay another implementation's tokens.  After every
 * `update_every` steps the chunk of those positions (inputs = what was fed,
 * targets = what was output) is processed again as one inner-loop step:
 * forward recomputed with earlier keys/values as constants, its own store
 * entries overwritten, loss, gradient, SGD.
 * out_tokens [batch, n_new]; update_losses [batch, n_new / update_every] or
 * NULL; step_logits [batch, n_new, V] or NULL.
 */
int oracle_generate(oracle_state* s, const int32_t* first_input, int n_new, int update_every,
                    const int32_t* forced, int32_t* out_tokens, double* update_losses, double* step_logits) {
  const oracle_cfg* c = &s->c;
  int B = c->batch, V = c->vocab;
  if (n_new < 0 || update_every < 1 || update_every > c->chunk) return -1;
  if (!ids_ok(c, first_input, B, 0)) return -1;
  if (forced && !ids_ok(c, forced, B * n_new, 0)) return -1;
  for (int r = 0; r < B; ++r)
    if (s->rows[r].pos + n_new > s->max_pos) return -2;
  int32_t* in_buf = xcalloc((size_t)B * update_every, 4);
  int32_t* tg_buf = xcalloc((size_t)B * update_every, 4);
  int32_t* cur = xcalloc((size_t)B, 4);
  memcpy(cur, first_input, sizeof(int32_t) * B);
  int nbuf = 0, nupd = 0;
  for (int j = 0; j < n_new; ++j) {
    for (int r = 0; r < B; ++r) {
      row_state* rs = &s->rows[r];
      chunk_work wk;
      work_alloc(c, &wk, 1);
      wk.p0 = rs->pos;
      forward_chunk(s, rs, &cur[r], &wk);
      int32_t best = 0;
      for (int v = 1; v < V; ++v)
        if (wk.logits[v] > wk.logits[best]) best = v;
      if (step_logits) memcpy(step_logits + ((int64_t)r * n_new + j) * V, wk.logits, sizeof(double) * V);
      int32_t out = forced ? forced[(int64_t)r * n_new + j] : best;
      out_tokens[(int64_t)r * n_new + j] = out;
      in_buf[(int64_t)r * update_every + nbuf] = cur[r];
      tg_buf[(int64_t)r * update_every + nbuf] = out;
      cur[r] = out;
      rs->pos += 1;
      work_free(c, &wk);
    }
    ++nbuf;
    if (nbuf == update_every) {
      for (int r = 0; r < B; ++r) s->rows[r].pos -= update_every;
      double* l = xcalloc((size_t)B, 8);
      int rc = oracle_prefill_chunk(s, in_buf, tg_buf, update_every, l);
      if (rc) { free(l); free(in_buf); free(tg_buf); free(cur); return rc; }
      if (update_losses) {
        int nu = n_new / update_every;
        for (int r = 0; r < B; ++r) update_losses[(int64_t)r * nu + nupd] = l[r];
      }
      free(l);
      ++nupd;
      nbuf = 0;
    }
  }
  free(in_buf); free(tg_buf); free(cur);
  return 0;
}
