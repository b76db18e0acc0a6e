// Row-wise and element-wise kernels: embedding gather, RMSNorm forward and
// backward, conversions/transposes, RoPE (+ key/value window write) and its
// backward, cross-entropy with its logit gradient, loss reduction, arg-max.
#include "kernels.h"

namespace {

template <typename T>
__global__ void k_embed(const int32_t* ids, int64_t ld, int n, const T* E, int d, int V, float* h, int* err) {
  int64_t m = blockIdx.x;
  int b = (int)(m / n), t = (int)(m % n);
  int id = ids[b * ld + t];
  if (id < 0 || id >= V) {
    if (threadIdx.x == 0) atomicOr(err, 1);
    id = 0;
  }
  const T* e = E + (int64_t)id * d;
  float* o = h + m * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) o[i] = to_f<T>(e[i]);
}

template <typename T>
__global__ void k_rmsnorm_fwd(const float* x, int d, const float* g, float eps, T* y, float* rstd, T* yT, int rpb,
                              int64_t ldT) {
  __shared__ float sh[16];
  int64_t m = blockIdx.x;
  const float* xr = x + m * d;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += blockDim.x) ss += xr[i] * xr[i];
  ss = block_sum(ss, sh);
  float r = 1.f / sqrtf(ss / (float)d + eps);
  if (threadIdx.x == 0 && rstd) rstd[m] = r;
  int b = (int)(m / rpb), t = (int)(m % rpb);
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    float v = g[i] * xr[i] * r;
    if (y) y[m * d + i] = from_f<T>(v);
    if (yT) yT[(int64_t)b * d * ldT + (int64_t)i * ldT + t] = from_f<T>(v);
  }
}

template <typename T>
__global__ void k_rmsnorm_bwd(const float* x, const float* rstd, int d, const float* g, const float* dy,
                              const float* resid, float* out, T* outT) {
  __shared__ float sh[16];
  int64_t m = blockIdx.x;
  const float* xr = x + m * d;
  const float* dyr = dy + m * d;
  float dot = 0.f;
  for (int i = threadIdx.x; i < d; i += blockDim.x) dot += g[i] * dyr[i] * xr[i];
  dot = block_sum(dot, sh);
  float r = rstd[m];
  float c = r * r * r * dot / (float)d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    float v = r * g[i] * dyr[i] - xr[i] * c;
    if (resid) v += resid[m * d + i];
    out[m * d + i] = v;
    if (outT) outT[m * d + i] = from_f<T>(v);
  }
}

template <typename T>
__global__ void k_convert(const float* x, int d, T* y, T* yT, int rpb, int64_t ldT) {
  int64_t m = blockIdx.x;
  int b = (int)(m / rpb), t = (int)(m % rpb);
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    float v = x[m * d + i];
    if (y) y[m * d + i] = from_f<T>(v);
    if (yT) yT[(int64_t)b * d * ldT + (int64_t)i * ldT + t] = from_f<T>(v);
  }
}

__global__ void k_count_valid(const int32_t* tgt, int64_t ld, int n, int* nvalid) {
  __shared__ float sh[16];
  int b = blockIdx.x;
  float c = 0.f;
  for (int t = threadIdx.x; t < n; t += blockDim.x) c += tgt[b * ld + t] >= 0 ? 1.f : 0.f;
  c = block_sum(c, sh);
  if (threadIdx.x == 0) nvalid[b] = (int)c;
}

template <typename T>
__global__ void k_ce_rows(const float* logits, int V, const int32_t* tgt, int64_t ld, const int* nvalid, int rpb,
                          float* loss_tok, T* dlogits, int* err) {
  __shared__ float sh[16];
  int64_t m = blockIdx.x;
  int b = (int)(m / rpb), t = (int)(m % rpb);
  int y = tgt[b * ld + t];
  if (y < -1 || y >= V) {
    if (threadIdx.x == 0) atomicOr(err, 2);
    y = -1;
  }
  const float* z = logits + m * V;
  float mx = -INFINITY;
  for (int v = threadIdx.x; v < V; v += blockDim.x) mx = fmaxf(mx, z[v]);
  mx = block_max(mx, sh);
  float se = 0.f;
  for (int v = threadIdx.x; v < V; v += blockDim.x) se += expf(z[v] - mx);
  se = block_sum(se, sh);
  float lse = mx + logf(se);
  int nv = nvalid[b];
  float inv = nv > 0 ? 1.f / (float)nv : 0.f;
  if (threadIdx.x == 0) loss_tok[m] = (y >= 0) ? lse - z[y] : 0.f;
  T* dz = dlogits + m * V;
  for (int v = threadIdx.x; v < V; v += blockDim.x) {
    float p = (y >= 0) ? (expf(z[v] - lse) - (v == y ? 1.f : 0.f)) * inv : 0.f;
    dz[v] = from_f<T>(p);
  }
}

__global__ void k_reduce_loss(const float* loss_tok, const int* nvalid, int n, float* out) {
  __shared__ float sh[16];
  int b = blockIdx.x;
  float s = 0.f;
  for (int t = threadIdx.x; t < n; t += blockDim.x) s += loss_tok[(int64_t)b * n + t];
  s = block_sum(s, sh);
  if (threadIdx.x == 0) out[b] = nvalid[b] > 0 ? s / (float)nvalid[b] : 0.f;
}

// arg-max of each row, lowest index on ties; written to out[b*ld_out] and out2[b*ld_out2] (if given)
__global__ void k_argmax(const float* logits, int V, int32_t* out, int64_t ld_out, int32_t* out2, int64_t ld_out2) {
  __shared__ float sv[1024];
  __shared__ int si[1024];
  int b = blockIdx.x;
  const float* z = logits + (int64_t)b * V;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int v = threadIdx.x; v < V; v += blockDim.x) {
    float x = z[v];
    if (x > bv || (x == bv && v < bi)) { bv = x; bi = v; }
  }
  sv[threadIdx.x] = bv;
  si[threadIdx.x] = bi;
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      float x = sv[threadIdx.x + o];
      int i = si[threadIdx.x + o];
      if (x > sv[threadIdx.x] || (x == sv[threadIdx.x] && i < si[threadIdx.x])) {
        sv[threadIdx.x] = x;
        si[threadIdx.x] = i;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int r = si[0] == 0x7fffffff ? 0 : si[0];
    out[b * ld_out] = r;
    if (out2) out2[b * ld_out2] = r;
  }
}

__global__ void k_copy_rows(const float* src, int64_t sbs, float* dst, int n, int d) {
  int64_t m = blockIdx.x;
  int b = (int)(m / n), t = (int)(m % n);
  const float* s = src + b * sbs + (int64_t)t * d;
  float* o = dst + m * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) o[i] = s[i];
}

// RoPE (rotate-half pairs (i, i+hd/2)) of q and k from a fp32 [B*n][3d] projection,
// and the write of rotated keys and values into the window ring at slot = pos mod R.
// One block handles 64 consecutive tokens of one (row, head); the transposed outputs
// (V^T ring, optional q^T) go through LDS so that each of their rows is written as 64
// consecutive tokens.
constexpr int RT = 64;  // tokens per block
template <typename T>
__global__ __launch_bounds__(256) void k_rope_qkv(const float* __restrict__ qkv, RopeRing rr) {
  __shared__ T vt[128][RT + 2];  // [dim][token]
  __shared__ T qs[128][RT + 2];
  constexpr bool KTR = sizeof(T) == 2;  // transposed key ring (bf16 contexts only)
  __shared__ T ks[KTR ? 128 : 1][RT + 2];
  const int h = blockIdx.y, b = blockIdx.z;
  const int t0 = blockIdx.x * RT;
  const int hd = rr.hd, half = hd / 2, d = rr.H * hd;
  const int nt = min(RT, rr.n - t0);
  const int64_t bh = (int64_t)b * rr.H + h;
  T* Q = (T*)rr.q;
  T* Kr = (T*)rr.kr;
  T* Vr = (T*)rr.vr;
  // rotated q, k and plain v: thread -> (token, pair) over 64 x hd/2
  for (int e = threadIdx.x; e < RT * half; e += blockDim.x) {
    const int tt = e / half, i = e % half;
    if (tt >= nt) continue;
    const int t = t0 + tt;
    const int64_t pos = rr.pos0 + t;
    const int slot = (int)(pos % rr.R);
    const float* row = qkv + ((int64_t)b * rr.n + t) * 3 * d + h * hd;
    const float c = rr.cos_t[pos * half + i], s = rr.sin_t[pos * half + i];
    float a = row[i], bb = row[i + half];
    const float q0 = a * c - bb * s, q1 = bb * c + a * s;
    T* qrow = Q + (bh * rr.n + t) * hd;
    qrow[i] = from_f<T>(q0);
    qrow[i + half] = from_f<T>(q1);
    qs[i][tt] = from_f<T>(q0);
    qs[i + half][tt] = from_f<T>(q1);
    a = row[d + i];
    bb = row[d + i + half];
    T* krow = Kr + (bh * rr.R + slot) * hd;
    const T k0 = from_f<T>(a * c - bb * s), k1 = from_f<T>(bb * c + a * s);
    krow[i] = k0;
    krow[i + half] = k1;
    if constexpr (KTR) {
      ks[i][tt] = k0;
      ks[i + half][tt] = k1;
    }
    const float v0 = row[2 * d + i], v1 = row[2 * d + i + half];
    T* vrow = Vr + (bh * rr.R + slot) * hd;
    vrow[i] = from_f<T>(v0);
    vrow[i + half] = from_f<T>(v1);
    vt[i][tt] = from_f<T>(v0);
    vt[i + half][tt] = from_f<T>(v1);
  }
  __syncthreads();
  // V^T (and K^T) ring rows: [dim][slot], consecutive tokens -> consecutive slots (mod R)
  T* Vt = (T*)rr.vtr + bh * hd * rr.R;
  T* Kt = (KTR && rr.ktr) ? (T*)rr.ktr + bh * hd * rr.R : nullptr;
  T* Qt = rr.qt ? (T*)rr.qt + bh * hd * rr.n : nullptr;
  for (int e = threadIdx.x; e < hd * RT; e += blockDim.x) {
    const int dim = e / RT, tt = e % RT;
    if (tt >= nt) continue;
    const int t = t0 + tt;
    const int slot = (int)((rr.pos0 + t) % rr.R);
    Vt[(int64_t)dim * rr.R + slot] = vt[dim][tt];
    if constexpr (KTR)
      if (Kt) Kt[(int64_t)dim * rr.R + slot] = ks[dim][tt];
    if (Qt) Qt[(int64_t)dim * rr.n + t] = qs[dim][tt];
  }
}

// inverse rotation of dq, dk (gradients w.r.t. rotated q, k) and packing [dq|dk|dv]
template <typename T>
__global__ void k_rope_bwd_pack(const float* dq, const float* dk, const float* dv, const float* cos_t,
                                const float* sin_t, int64_t pos0, int n, int H, int hd, T* dqkv) {
  int64_t m = blockIdx.x;
  int h = blockIdx.y;
  int t = (int)(m % n);
  int half = hd / 2, d = H * hd;
  int64_t pos = pos0 + t;
  const float* q = dq + m * d + h * hd;
  const float* k = dk + m * d + h * hd;
  const float* v = dv + m * d + h * hd;
  T* o = dqkv + m * 3 * d + h * hd;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    float c = cos_t[pos * half + i], s = sin_t[pos * half + i];
    float a = q[i], bb = q[i + half];
    o[i] = from_f<T>(a * c + bb * s);
    o[i + half] = from_f<T>(bb * c - a * s);
    a = k[i];
    bb = k[i + half];
    o[d + i] = from_f<T>(a * c + bb * s);
    o[d + i + half] = from_f<T>(bb * c - a * s);
    o[2 * d + i] = from_f<T>(v[i]);
    o[2 * d + i + half] = from_f<T>(v[i + half]);
  }
}

// shadow copies of fp32 master weights: sh = T(master) [rows][cols], shT = T(master)^T [cols][rows]
template <typename T>
__global__ void k_shadow(const float* master, int rows, int cols, int64_t sm, T* sh, int64_t ssh, T* shT,
                         int64_t sshT, int64_t il_f) {
  __shared__ float tile[32][33];
  int bz = blockIdx.z;
  int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const float* src = master + bz * sm;
  for (int i = threadIdx.y; i < 32; i += blockDim.y) {
    int r = r0 + i, q = c0 + threadIdx.x;
    if (r < rows && q < cols) {
      float v = src[(int64_t)r * cols + q];
      tile[i][threadIdx.x] = v;
      sh[bz * ssh + (il_f ? swiglu_il_row(r, il_f) : (int64_t)r) * cols + q] = from_f<T>(v);
    }
  }
  __syncthreads();
  for (int i = threadIdx.y; i < 32; i += blockDim.y) {
    int q = c0 + i, r = r0 + threadIdx.x;
    if (r < rows && q < cols) shT[bz * sshT + (int64_t)q * rows + r] = from_f<T>(tile[threadIdx.x][i]);
  }
}

int row_threads(int d) { return d >= 1024 ? 256 : (d >= 256 ? 128 : 64); }

}  // namespace

template <typename T>
hipError_t embed_gather_ld(const int32_t* ids, int64_t ld, int B, int n, const T* E, int d, int V, float* h, int* err,
                           hipStream_t s) {
  if (B * n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_embed<T>, dim3(B * n), dim3(row_threads(d)), 0, s, ids, ld, n, E, d, V, h, err);
  return hipGetLastError();
}

template <typename T>
hipError_t rmsnorm_fwd(const float* x, int64_t M, int d, const float* g, float eps, T* y, float* rstd, T* yT, int rpb,
                       int64_t ldT, hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm_fwd<T>, dim3(M), dim3(row_threads(d)), 0, s, x, d, g, eps, y, rstd, yT, rpb, ldT);
  return hipGetLastError();
}

template <typename T>
hipError_t rmsnorm_bwd(const float* x, const float* rstd, int64_t M, int d, const float* g, const float* dy,
                       const float* resid, float* out, T* outT, hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm_bwd<T>, dim3(M), dim3(row_threads(d)), 0, s, x, rstd, d, g, dy, resid, out, outT);
  return hipGetLastError();
}

template <typename T>
hipError_t convert_rows(const float* x, int64_t M, int d, T* y, T* yT, int rpb, int64_t ldT, hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(k_convert<T>, dim3(M), dim3(row_threads(d)), 0, s, x, d, y, yT, rpb, ldT);
  return hipGetLastError();
}

hipError_t count_valid_ld(const int32_t* tgt, int64_t ld, int B, int n, int* nvalid, hipStream_t s) {
  hipLaunchKernelGGL(k_count_valid, dim3(B), dim3(256), 0, s, tgt, ld, n, nvalid);
  return hipGetLastError();
}

template <typename T>
hipError_t ce_rows_ld(const float* logits, int64_t M, int V, const int32_t* tgt, int64_t ld, const int* nvalid,
                      int rpb, float* loss_tok, T* dlogits, int* err, hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(k_ce_rows<T>, dim3(M), dim3(256), 0, s, logits, V, tgt, ld, nvalid, rpb, loss_tok, dlogits, err);
  return hipGetLastError();
}

hipError_t reduce_loss(const float* loss_tok, const int* nvalid, int B, int n, float* loss_out, hipStream_t s) {
  hipLaunchKernelGGL(k_reduce_loss, dim3(B), dim3(256), 0, s, loss_tok, nvalid, n, loss_out);
  return hipGetLastError();
}

hipError_t argmax_rows_ld(const float* logits, int B, int V, int32_t* out, int64_t ld_out, int32_t* out2,
                          int64_t ld_out2, hipStream_t s) {
  hipLaunchKernelGGL(k_argmax, dim3(B), dim3(1024), 0, s, logits, V, out, ld_out, out2, ld_out2);
  return hipGetLastError();
}

hipError_t copy_rows(const float* src, int64_t src_batch_stride, float* dst, int B, int n, int d, hipStream_t s) {
  if (B * n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy_rows, dim3(B * n), dim3(row_threads(d)), 0, s, src, src_batch_stride, dst, n, d);
  return hipGetLastError();
}

hipError_t rope_qkv_f32in(const float* qkv, int B, const RopeRing& rr, int is_bf16, hipStream_t s) {
  if (B * rr.n == 0) return hipSuccess;
  if (rr.hd > 128) return hipErrorInvalidValue;
  dim3 grid(cdiv(rr.n, RT), rr.H, B);
  if (is_bf16)
    hipLaunchKernelGGL(k_rope_qkv<bf16>, grid, dim3(256), 0, s, qkv, rr);
  else
    hipLaunchKernelGGL(k_rope_qkv<float>, grid, dim3(256), 0, s, qkv, rr);
  return hipGetLastError();
}

template <typename T>
hipError_t rope_bwd_pack(const float* dq, const float* dk, const float* dv, const float* cos_t, const float* sin_t,
                         int64_t pos0, int B, int n, int H, int hd, T* dqkv, hipStream_t s) {
  if (B * n == 0) return hipSuccess;
  int th = hd / 2 >= 64 ? 64 : 32;
  hipLaunchKernelGGL(k_rope_bwd_pack<T>, dim3(B * n, H), dim3(th), 0, s, dq, dk, dv, cos_t, sin_t, pos0, n, H, hd,
                     dqkv);
  return hipGetLastError();
}

hipError_t refresh_shadows(const float* master, int rows, int cols, int batch, int64_t sm, void* sh, int64_t ssh,
                           void* shT, int64_t sshT, int is_bf16, int64_t il_f, hipStream_t s) {
  dim3 grid(cdiv(cols, 32), cdiv(rows, 32), batch), block(32, 8);
  if (is_bf16)
    hipLaunchKernelGGL(k_shadow<bf16>, grid, block, 0, s, master, rows, cols, sm, (bf16*)sh, ssh, (bf16*)shT, sshT,
                       il_f);
  else
    hipLaunchKernelGGL(k_shadow<float>, grid, block, 0, s, master, rows, cols, sm, (float*)sh, ssh, (float*)shT,
                       sshT, il_f);
  return hipGetLastError();
}

#define INST(T)                                                                                                      \
  template hipError_t embed_gather_ld<T>(const int32_t*, int64_t, int, int, const T*, int, int, float*, int*,       \
                                         hipStream_t);                                                              \
  template hipError_t rmsnorm_fwd<T>(const float*, int64_t, int, const float*, float, T*, float*, T*, int, int64_t, \
                                     hipStream_t);                                                                  \
  template hipError_t rmsnorm_bwd<T>(const float*, const float*, int64_t, int, const float*, const float*,          \
                                     const float*, float*, T*, hipStream_t);                                        \
  template hipError_t convert_rows<T>(const float*, int64_t, int, T*, T*, int, int64_t, hipStream_t);               \
  template hipError_t ce_rows_ld<T>(const float*, int64_t, int, const int32_t*, int64_t, const int*, int, float*,   \
                                    T*, int*, hipStream_t);                                                         \
  template hipError_t rope_bwd_pack<T>(const float*, const float*, const float*, const float*, const float*,        \
                                       int64_t, int, int, int, int, T*, hipStream_t);
INST(float)
INST(bf16)
