/*
 * Drives every entry point of the fp64 oracle on a tiny batched model, for a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitizers.py).  TEST INFRASTRUCTURE: the oracle source is
 * compiled into this program as one translation unit, so the structures it
 * uses are the oracle's own.
 *
 * Covered: creation (and the rejected configurations), chunks of the full size,
 * a ragged last chunk and chunks with ignored targets, two SGD steps per chunk,
 * the static + dynamic MLP variant,
 * the gradient of one chunk, greedy generation with an update and per-step
 * logits, teacher forcing, reading and writing fast weights, the RoPE and
 * RMSNorm helpers.  Exit status 0 when every call returned what it should.
 */
#include "../../oracle/ttt_oracle.c"

#include <stdio.h>

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

/* test data only: a 64-bit LCG mapped to [-scale, scale) */
static uint64_t lcg_state = 0x9e3779b97f4a7c15ull;
static float next_uniform(float scale) {
  lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
  return scale * (2.0f * (float)((lcg_state >> 40) * (1.0 / 16777216.0)) - 1.0f);
}

static float* filled(size_t n, float scale, float offset) {
  float* p = (float*)malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = offset + next_uniform(scale);
  return p;
}

enum { L = 4, D = 16, H = 2, F = 24, V = 11, K = 5, B = 4, ROWS = 2, MAXPOS = 16 };

typedef struct {
  float *embed, *final_norm, *lm_head;
  float* per_layer[9][L];
  const float* ptrs[9][L];
  float* dyn[3][2];           /* dynamic MLPs of the two updated blocks */
  const float* dyn_ptrs[3][2];
} weights;

static void make_weights(weights* w) {
  w->embed = filled((size_t)V * D, 0.5f, 0.f);
  w->final_norm = filled(D, 0.1f, 1.f);
  w->lm_head = filled((size_t)V * D, 0.3f, 0.f);
  const size_t sizes[9] = {D, D * D, D * D, D * D, D * D, D, (size_t)F * D, (size_t)F * D, (size_t)D * F};
  for (int a = 0; a < 9; ++a)
    for (int l = 0; l < L; ++l) {
      const int gain = a == 0 || a == 5;
      w->per_layer[a][l] = filled(sizes[a], gain ? 0.1f : 0.3f, gain ? 1.f : 0.f);
      w->ptrs[a][l] = w->per_layer[a][l];
    }
  for (int a = 0; a < 3; ++a)
    for (int j = 0; j < 2; ++j) {
      w->dyn[a][j] = filled((size_t)F * D, 0.3f, 0.f);
      w->dyn_ptrs[a][j] = w->dyn[a][j];
    }
}

static void free_weights(weights* w) {
  free(w->embed);
  free(w->final_norm);
  free(w->lm_head);
  for (int a = 0; a < 9; ++a)
    for (int l = 0; l < L; ++l) free(w->per_layer[a][l]);
  for (int a = 0; a < 3; ++a)
    for (int j = 0; j < 2; ++j) free(w->dyn[a][j]);
}

static oracle_weights view(const weights* w) {
  oracle_weights o;
  memset(&o, 0, sizeof(o));
  o.embed = w->embed;
  o.final_norm = w->final_norm;
  o.lm_head = w->lm_head;
  o.attn_norm = w->ptrs[0];
  o.wq = w->ptrs[1];
  o.wk = w->ptrs[2];
  o.wv = w->ptrs[3];
  o.wo = w->ptrs[4];
  o.mlp_norm = w->ptrs[5];
  o.w_gate = w->ptrs[6];
  o.w_up = w->ptrs[7];
  o.w_down = w->ptrs[8];
  o.dyn_gate = w->dyn_ptrs[0];
  o.dyn_up = w->dyn_ptrs[1];
  o.dyn_down = w->dyn_ptrs[2];
  return o;
}

static oracle_cfg base_cfg(void) {
  oracle_cfg c;
  memset(&c, 0, sizeof(c));
  c.n_layers = L;
  c.d_model = D;
  c.n_heads = H;
  c.d_ff = F;
  c.vocab = V;
  c.window = K;
  c.chunk = B;
  c.n_fast = 2;
  c.batch = ROWS;
  c.n_steps = 1;
  c.rope_theta = 1e4;
  c.rms_eps = 1e-5;
  c.lr = 0.1;
  return c;
}

static int finite_all(const double* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) return 0;
  return 1;
}

/* T = 11 positions: chunks of 4, 4 and a ragged 3; row 1 ignores some targets */
static void run_prefill(oracle_state* s) {
  int32_t tok[ROWS * 11], tgt[ROWS * 11];
  for (int i = 0; i < ROWS * 11; ++i) {
    tok[i] = (i * 7 + 3) % V;
    tgt[i] = (i * 5 + 1) % V;
  }
  tgt[11 + 2] = -1;
  tgt[11 + 5] = -1;
  for (int i = 4; i < 8; ++i) tgt[i] = -1; /* row 0: an all-ignored chunk */
  int p0 = 0;
  while (p0 < 11) {
    const int n = p0 + B <= 11 ? B : 11 - p0;
    int32_t ct[ROWS * B], cg[ROWS * B];
    for (int r = 0; r < ROWS; ++r)
      for (int i = 0; i < n; ++i) {
        ct[r * n + i] = tok[r * 11 + p0 + i];
        cg[r * n + i] = tgt[r * 11 + p0 + i];
      }
    double loss[ROWS];
    CHECK(oracle_prefill_chunk(s, ct, cg, n, loss) == 0);
    CHECK(finite_all(loss, ROWS));
    if (p0 == 4) CHECK(loss[0] == 0.0);
    p0 += n;
  }
  CHECK(oracle_get_pos(s, 0) == 11 && oracle_get_pos(s, 1) == 11);
}

int main(void) {
  weights w;
  make_weights(&w);
  oracle_weights ow = view(&w);

  /* rejected configurations */
  oracle_cfg bad = base_cfg();
  bad.window = B - 1;
  CHECK(oracle_create(&bad, &ow, MAXPOS) == NULL);
  bad = base_cfg();
  bad.d_model = 15;
  CHECK(oracle_create(&bad, &ow, MAXPOS) == NULL);
  bad = base_cfg();
  bad.n_fast = L + 1;
  CHECK(oracle_create(&bad, &ow, MAXPOS) == NULL);
  CHECK(oracle_create(NULL, &ow, MAXPOS) == NULL);
  CHECK(oracle_create(&bad, &ow, 0) == NULL);

  /* a dual configuration without its dynamic weights is refused */
  bad = base_cfg();
  bad.dual_mlp = 1;
  oracle_weights nodyn = ow;
  nodyn.dyn_up = NULL;
  CHECK(oracle_create(&bad, &nodyn, MAXPOS) == NULL);

  /* one SGD step, two SGD steps, static + dynamic MLP */
  for (int variant = 0; variant < 3; ++variant) {
    oracle_cfg c = base_cfg();
    c.n_steps = variant == 1 ? 2 : 1;
    c.dual_mlp = variant == 2;
    oracle_state* s = oracle_create(&c, &ow, MAXPOS);
    CHECK(s != NULL);
    if (!s) break;
    const int64_t nf = oracle_fast_size(s);
    CHECK(nf == 2 * 3 * F * D);

    /* gradient of a first chunk (no state change), then the chunk loop */
    int32_t ct[ROWS * B], cg[ROWS * B];
    for (int i = 0; i < ROWS * B; ++i) {
      ct[i] = (3 * i + 1) % V;
      cg[i] = (5 * i + 2) % V;
    }
    double loss[ROWS];
    double* grad = (double*)calloc((size_t)(ROWS * nf), sizeof(double));
    CHECK(oracle_eval_chunk(s, ct, cg, B, loss, grad) == 0);
    CHECK(finite_all(loss, ROWS) && finite_all(grad, ROWS * nf));
    CHECK(oracle_get_pos(s, 0) == 0);
    free(grad);

    /* argument errors */
    ct[0] = V;
    CHECK(oracle_prefill_chunk(s, ct, cg, B, loss) != 0);
    ct[0] = 0;
    CHECK(oracle_prefill_chunk(s, ct, cg, B + 1, loss) != 0);

    run_prefill(s);

    /* fast weights: read, write back, out-of-range rows */
    double* fast = (double*)malloc(sizeof(double) * (size_t)nf);
    CHECK(oracle_get_fast(s, 1, fast) == 0);
    CHECK(finite_all(fast, nf));
    CHECK(oracle_set_fast(s, 0, fast) == 0);
    CHECK(oracle_get_fast(s, ROWS, fast) != 0);
    CHECK(oracle_set_fast(s, -1, fast) != 0);
    free(fast);

    /* generation: 4 tokens with an update after them, logits of every step; then past the end */
    int32_t first[ROWS] = {1, 2}, out[ROWS * 4];
    double ul[ROWS];
    double* logits = (double*)malloc(sizeof(double) * ROWS * 4 * V);
    CHECK(oracle_generate(s, first, 4, 4, NULL, out, ul, logits) == 0);
    CHECK(finite_all(ul, ROWS) && finite_all(logits, ROWS * 4 * V));
    for (int i = 0; i < ROWS * 4; ++i) CHECK(out[i] >= 0 && out[i] < V);
    int32_t forced[ROWS * 4];
    for (int i = 0; i < ROWS * 4; ++i) forced[i] = i % V;
    CHECK(oracle_generate(s, first, 4, 4, forced, out, ul, NULL) == -2); /* 15 + 4 > MAXPOS */
    free(logits);
    oracle_destroy(s);
  }

  /* helpers */
  double x[8], y[8], z[8], rstd[2];
  for (int i = 0; i < 8; ++i) x[i] = next_uniform(1.f);
  oracle_rope(x, 8, 5, 1e4, 1, y);
  oracle_rope(y, 8, 5, 1e4, -1, z);
  for (int i = 0; i < 8; ++i) CHECK(fabs(z[i] - x[i]) < 1e-12);
  float g[4] = {1.f, 0.5f, 2.f, 1.f};
  oracle_rmsnorm(x, 2, 4, g, 1e-5, y, rstd);
  CHECK(finite_all(y, 8) && finite_all(rstd, 2));

  free_weights(&w);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle driver: all checks passed\n");
  return 0;
}
