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

// 4 consecutive values -> T: one 16-byte (fp32) or 8-byte (bf16) store
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *(float4*)p = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, float a, float b, float c, float d) {
  *(uint2*)p = make_uint2(bf16pair(a, b), bf16pair(c, d));
}

// Vector forms of the row kernels above: one 256-thread block per row, 16-byte access
// (d % 4 == 0, d <= 4096, 16-byte aligned rows); transposed outputs are written by
// k_transpose_rows afterwards.  With `parts`, the S fp32 parts of a K-split GEMM
// ([S][M][d], plane = M * d floats apart) are summed in order inside the row kernel
// instead of by a separate pass: the forward adds them to h (and rewrites h), the backward
// uses their sum as dy.
template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm_fwd_row(float* h, const float* __restrict__ parts, int S, int64_t plane,
                                                         int d, const float* __restrict__ g, float eps,
                                                         T* __restrict__ y, float* __restrict__ rstd,
                                                         float* __restrict__ xcopy) {
  __shared__ float sh[16];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x, d4 = d / 4;
  float4* hr = (float4*)(h + m * d);
  float4 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid + 256 * k;
    if (i < d4) v[k] = hr[i];
  }
  if (parts) {
    const float4* pr = (const float4*)(parts + m * d);
    const int64_t pl4 = plane / 4;
    // up to four parts' loads in flight at once, then added in order (an absent part adds 0)
    for (int sp0 = 0; sp0 < S; sp0 += 4) {
      float4 q[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = tid + 256 * k;
          q[u][k] = (sp0 + u < S && i < d4) ? pr[(sp0 + u) * pl4 + i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[k].x += q[u][k].x;
          v[k].y += q[u][k].y;
          v[k].z += q[u][k].z;
          v[k].w += q[u][k].w;
        }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid + 256 * k;
    if (i < d4) {
      if (parts) hr[i] = v[k];
      if (xcopy) ((float4*)(xcopy + m * d))[i] = v[k];
      ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
    }
  }
  ss = block_sum(ss, sh);
  const float r = 1.f / sqrtf(ss / (float)d + eps);
  if (tid == 0 && rstd) rstd[m] = r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid + 256 * k;
    if (i < d4) {
      const float4 w = ((const float4*)g)[i];
      store4<T>(y + m * d + 4 * i, w.x * v[k].x * r, w.y * v[k].y * r, w.z * v[k].z * r, w.w * v[k].w * r);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd_row(const float* __restrict__ x, const float* __restrict__ rstd,
                                                         int d, const float* __restrict__ g, const float* dy,
                                                         const float* __restrict__ parts, int S, int64_t plane,
                                                         const float* resid, float* out, T* outT) {
  __shared__ float sh[16];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x, d4 = d / 4;
  const float4* xr = (const float4*)(x + m * d);
  const float4* g4 = (const float4*)g;
  const float4* er = (const float4*)((parts ? parts : dy) + m * d);
  float4 e[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid + 256 * k;
    if (i < d4) e[k] = er[i];
  }
  if (parts) {
    const int64_t pl4 = plane / 4;
    // (parts 1.. as in the forward kernel: four parts' loads in flight, added in order)
    for (int sp0 = 1; sp0 < S; sp0 += 4) {
      float4 q[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = tid + 256 * k;
          q[u][k] = (sp0 + u < S && i < d4) ? er[(sp0 + u) * pl4 + i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          e[k].x += q[u][k].x;
          e[k].y += q[u][k].y;
          e[k].z += q[u][k].z;
          e[k].w += q[u][k].w;
        }
    }
  }
  float dot = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid + 256 * k;
    if (i < d4) {
      const float4 v = xr[i], w = g4[i];
      dot += w.x * e[k].x * v.x + w.y * e[k].y * v.y + w.z * e[k].z * v.z + w.w * e[k].w * v.w;
    }
  }
  dot = block_sum(dot, sh);
  const float r = rstd[m];
  const float c = r * r * r * dot / (float)d;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid + 256 * k;
    if (i < d4) {
      const float4 v = xr[i], w = g4[i];
      float4 o = make_float4(r * w.x * e[k].x - v.x * c, r * w.y * e[k].y - v.y * c, r * w.z * e[k].z - v.z * c,
                             r * w.w * e[k].w - v.w * c);
      if (resid) {
        const float4 q = ((const float4*)(resid + m * d))[i];
        o.x += q.x;
        o.y += q.y;
        o.z += q.z;
        o.w += q.w;
      }
      ((float4*)(out + m * d))[i] = o;
      if (outT) store4<T>(outT + m * d + 4 * i, o.x, o.y, o.z, o.w);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_convert4(const float* x, int64_t M, int d, T* y) {
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const int lane = threadIdx.x & 63, d4 = d / 4;
  for (int i = lane; i < d4; i += 64) {
    const float4 v = ((const float4*)(x + m * d))[i];
    store4<T>(y + m * d + 4 * i, v.x, v.y, v.z, v.w);
  }
}

// y [B][n][d] (bf16) -> yT [B][d][ldt]: yT[b][c][t] = y[b][t][c] for t < n, through a 64 x 64
// LDS tile, 16-byte loads and stores (d % 8 == 0, n % 8 == 0, ldt % 8 == 0)
__global__ __launch_bounds__(256) void k_transpose_rows(const bf16* __restrict__ y, bf16* __restrict__ yt, int n,
                                                        int d, int64_t ldt) {
  __shared__ __align__(16) uint16_t tile[64][72];  // [token][column]
  const int t0 = blockIdx.x * 64, c0 = blockIdx.y * 64, b = blockIdx.z;
  for (int e = threadIdx.x; e < 64 * 8; e += 256) {
    const int r = e >> 3, ch = (e & 7) * 8, t = t0 + r, c = c0 + ch;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t < n && c < d) v = *(const uint4*)(y + ((int64_t)b * n + t) * d + c);
    *(uint4*)&tile[r][ch] = v;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 8; e += 256) {
    const int cr = e >> 3, tch = (e & 7) * 8, c = c0 + cr, t = t0 + tch;
    if (c < d && t < n) {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = (uint32_t)tile[tch + 2 * k][cr] | ((uint32_t)tile[tch + 2 * k + 1][cr] << 16);
      *(uint4*)(yt + ((int64_t)b * d + c) * ldt + t) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// sum of S fp32 parts [S][B*n][d] (plane floats apart, in order) -> y [B][n][d] and
// yT [B][d][n] (bf16), 64 rows x 64 columns per block through the same LDS tile as above
// (d % 4 == 0, n % 8 == 0)
__global__ __launch_bounds__(256) void k_parts_rows_t(const float* __restrict__ parts, int S, int64_t plane, int n,
                                                      int d, bf16* __restrict__ y, bf16* __restrict__ yt) {
  __shared__ __align__(16) uint16_t tile[64][72];  // [token][column]
  const int t0 = blockIdx.x * 64, c0 = blockIdx.y * 64, b = blockIdx.z;
  const int tid = threadIdx.x, c4 = tid & 15, r0 = tid >> 4, c = c0 + 4 * c4;
  float4 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  // up to four parts' loads in flight at once, then added in order (an absent part adds 0)
  for (int sp0 = 0; sp0 < S; sp0 += 4) {
    float4 v[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int t = t0 + r0 + 16 * k;
        v[u][k] = (sp0 + u < S && t < n && c < d)
                      ? *(const float4*)(parts + (sp0 + u) * plane + ((int64_t)b * n + t) * d + c)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[k].x += v[u][k].x;
        acc[k].y += v[u][k].y;
        acc[k].z += v[u][k].z;
        acc[k].w += v[u][k].w;
      }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = r0 + 16 * k, t = t0 + r;
    const uint2 w = make_uint2(bf16pair(acc[k].x, acc[k].y), bf16pair(acc[k].z, acc[k].w));
    if (t < n && c < d) *(uint2*)(y + ((int64_t)b * n + t) * d + c) = w;
    *(uint2*)&tile[r][4 * c4] = w;
  }
  __syncthreads();
  for (int e = tid; e < 64 * 8; e += 256) {
    const int cr = e >> 3, tch = (e & 7) * 8, cc = c0 + cr, t = t0 + tch;
    if (cc < d && t < n) {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = (uint32_t)tile[tch + 2 * k][cr] | ((uint32_t)tile[tch + 2 * k + 1][cr] << 16);
      *(uint4*)(yt + ((int64_t)b * d + cc) * n + t) = make_uint4(w[0], w[1], w[2], w[3]);
    }
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
  if (!dlogits) return;  // loss only (scoring without an update)
  T* dz = dlogits + m * V;
  for (int v = threadIdx.x; v < V; v += blockDim.x) {
    float p = (y >= 0) ? (expf(z[v] - lse) - (v == y ? 1.f : 0.f)) * inv : 0.f;
    dz[v] = from_f<T>(p);
  }
}

// Same result for V % 4 == 0 with 16-byte logit loads and one pass fewer: each thread keeps a
// running (max, sum of exp) over its elements; the block merges them (sum_i s_i e^(m_i - M)).
template <typename T>
__global__ __launch_bounds__(512) void k_ce_rows4(const float* logits, int V, const int32_t* tgt, int64_t ld,
                                                  const int* nvalid, int rpb, float* loss_tok, T* dlogits, int* err) {
  __shared__ float sh[16];
  const int64_t m = blockIdx.x;
  const int b = (int)(m / rpb), t = (int)(m % rpb);
  int y = tgt[b * ld + t];
  if (y < -1 || y >= V) {
    if (threadIdx.x == 0) atomicOr(err, 2);
    y = -1;
  }
  const float4* z4 = (const float4*)(logits + m * V);
  const int V4 = V / 4;
  float mx = -INFINITY, se = 0.f;
  for (int v = threadIdx.x; v < V4; v += blockDim.x) {
    const float4 z = z4[v];
    const float zm = fmaxf(fmaxf(z.x, z.y), fmaxf(z.z, z.w));
    if (zm > mx) {
      se *= __expf(mx - zm);
      mx = zm;
    }
    se += __expf(z.x - mx) + __expf(z.y - mx) + __expf(z.z - mx) + __expf(z.w - mx);
  }
  const float M = block_max(mx, sh);
  const float ssum = block_sum(mx == -INFINITY ? 0.f : se * __expf(mx - M), sh);
  const float lse = M + logf(ssum);
  const int nv = nvalid[b];
  const float inv = nv > 0 ? 1.f / (float)nv : 0.f;
  if (threadIdx.x == 0) loss_tok[m] = (y >= 0) ? lse - logits[m * V + y] : 0.f;
  if (!dlogits) return;  // loss only (scoring without an update)
  T* dz = dlogits + m * V;
  for (int v = threadIdx.x; v < V4; v += blockDim.x) {
    const float4 z = z4[v];
    float p[4] = {__expf(z.x - lse), __expf(z.y - lse), __expf(z.z - lse), __expf(z.w - lse)};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (4 * v + k == y) p[k] -= 1.f;
      p[k] = (y >= 0) ? p[k] * inv : 0.f;
    }
    if constexpr (sizeof(T) == 2) {
      *(uint2*)(dz + 4 * v) = make_uint2(bf16pair(p[0], p[1]), bf16pair(p[2], p[3]));
    } else {
      *(float4*)(dz + 4 * v) = make_float4(p[0], p[1], p[2], p[3]);
    }
  }
}

// Rest of the vocabulary-tiled cross-entropy of one row (after an EPI_LM_CE lm_head product):
// merge the tiles' statistics (maxima m_t, sums s_t of exp(z - m_t)) into lse = M + log sum_t
// s_t e^(m_t - M), loss = lse - z_y, and rescale the row's exp(z - m_t) in place into
// dlogits = (e^(z - lse) - [v == y]) / nvalid.  Grid: one block per row.
template <typename T>
__global__ __launch_bounds__(256) void k_ce_finalize(const float* part, const float* zt, int64_t M, int V,
                                                     const int32_t* tgt, int64_t ld, const int* nvalid, int rpb,
                                                     float* loss_tok, T* e, int* err) {
  __shared__ float sh[16];
  __shared__ float scale[1024];  // e^(m_t - lse) / nvalid per vocabulary tile
  const int64_t m = blockIdx.x;
  const int b = (int)(m / rpb), t = (int)(m % rpb);
  const int ntile = (V + 255) / 256;
  int y = tgt[b * ld + t];
  if (y < -1 || y >= V) {
    if (threadIdx.x == 0) atomicOr(err, 2);
    y = -1;
  }
  float mx = -INFINITY;
  for (int i = threadIdx.x; i < ntile; i += blockDim.x) mx = fmaxf(mx, part[(int64_t)i * 2 * M + m]);
  const float Mx = block_max(mx, sh);
  float sm = 0.f;
  for (int i = threadIdx.x; i < ntile; i += blockDim.x)
    sm += part[(int64_t)i * 2 * M + M + m] * __expf(part[(int64_t)i * 2 * M + m] - Mx);
  const float lse = Mx + logf(block_sum(sm, sh));
  if (threadIdx.x == 0) loss_tok[m] = y >= 0 ? lse - zt[m] : 0.f;
  if (!e) return;
  const int nv = nvalid[b];
  const float inv = nv > 0 ? 1.f / (float)nv : 0.f;
  for (int i = threadIdx.x; i < ntile; i += blockDim.x)
    scale[i] = y >= 0 ? __expf(part[(int64_t)i * 2 * M + m] - lse) * inv : 0.f;
  __syncthreads();
  T* row = e + m * V;
  for (int v = 8 * threadIdx.x; v < V; v += 8 * blockDim.x) {  // 8 columns of one tile (V % 8 == 0)
    const float sc = scale[v / 256];
    const uint4 in = *(const uint4*)(row + v);
    const uint32_t w[4] = {in.x, in.y, in.z, in.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float x0 = bf2f(bf16{(uint16_t)(w[k] & 0xffff)}) * sc, x1 = bf2f(bf16{(uint16_t)(w[k] >> 16)}) * sc;
      if (v + 2 * k == y) x0 -= inv;
      if (v + 2 * k + 1 == y) x1 -= inv;
      o[k] = bf16pair(x0, x1);
    }
    *(uint4*)(row + v) = make_uint4(o[0], o[1], o[2], o[3]);
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
// arg-max of each logits row (ties to the lowest id; NaNs are never taken): 16-byte loads, each
// thread keeping its running best in id order, then a shuffle reduction per wave and one across
// the block's waves
__device__ __forceinline__ void argmax_merge(float& bv, int& bi, float x, int i) {
  if (x > bv || (x == bv && i < bi)) {
    bv = x;
    bi = i;
  }
}

__global__ __launch_bounds__(1024) void k_argmax(const float* logits, int V, int32_t* out, int64_t ld_out,
                                                 int32_t* out2, int64_t ld_out2) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, nw = blockDim.x >> 6;
  const float* z = logits + (int64_t)b * V;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if (V % 4 == 0 && ((uintptr_t)z & 15) == 0) {
    for (int v = 4 * tid; v < V; v += 4 * blockDim.x) {
      const float4 x = *(const float4*)(z + v);
      argmax_merge(bv, bi, x.x, v);
      argmax_merge(bv, bi, x.y, v + 1);
      argmax_merge(bv, bi, x.z, v + 2);
      argmax_merge(bv, bi, x.w, v + 3);
    }
  } else {
    for (int v = tid; v < V; v += blockDim.x) argmax_merge(bv, bi, z[v], v);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) argmax_merge(bv, bi, __shfl_xor(bv, o, 64), __shfl_xor(bi, o, 64));
  if (lane == 0) {
    sv[wid] = bv;
    si[wid] = bi;
  }
  __syncthreads();
  if (wid == 0) {
    bv = lane < nw ? sv[lane] : -INFINITY;
    bi = lane < nw ? si[lane] : 0x7fffffff;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) argmax_merge(bv, bi, __shfl_xor(bv, o, 64), __shfl_xor(bi, o, 64));
    if (lane == 0) {
      const int r = bi == 0x7fffffff ? 0 : bi;
      out[b * ld_out] = r;
      if (out2) out2[b * ld_out2] = r;
    }
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
    // dims i and i + half: natural columns, or adjacent ones when q/k are pair-interleaved
    const int ca = rr.perm ? 2 * i : i, cb = rr.perm ? 2 * i + 1 : i + half;
    float a = row[ca], bb = row[cb];
    const float q0 = a * c - bb * s, q1 = bb * c + a * s;
    T* qrow = Q + (bh * rr.n + t) * hd;
    qrow[i] = from_f<T>(q0);
    qrow[i + half] = from_f<T>(q1);
    qs[i][tt] = from_f<T>(q0);
    qs[i + half][tt] = from_f<T>(q1);
    a = row[d + ca];
    bb = row[d + cb];
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

// Vector form of k_rope_qkv (hd % 8 == 0, 16-byte aligned projection rows and tables):
// each thread rotates 4 consecutive pairs with 16-byte loads and 8- or 16-byte stores; the
// transposed rows are written 4 tokens per store where the 4 ring slots are consecutive.
template <typename T>
__global__ __launch_bounds__(256) void k_rope_qkv4(const float* __restrict__ qkv, RopeRing rr) {
  __shared__ T vt[128][RT + 2];  // [dim][token]
  __shared__ T qs[128][RT + 2];
  constexpr bool KTR = sizeof(T) == 2;
  __shared__ T ks[KTR ? 128 : 1][RT + 2];
  const int h = blockIdx.y, b = blockIdx.z;
  const int t0 = blockIdx.x * RT;
  const int hd = rr.hd, half = hd / 2, q4 = half / 4, d = rr.H * hd;
  const int nt = min(RT, rr.n - t0);
  const int64_t bh = (int64_t)b * rr.H + h;
  T* Q = (T*)rr.q;
  T* Kr = (T*)rr.kr;
  T* Vr = (T*)rr.vr;
  for (int e = threadIdx.x; e < RT * q4; e += blockDim.x) {
    const int tt = e / q4, i = (e % q4) * 4;
    if (tt >= nt) continue;
    const int t = t0 + tt;
    const int64_t pos = rr.pos0 + t;
    const int slot = (int)(pos % rr.R);
    const float* row = qkv + ((int64_t)b * rr.n + t) * 3 * d + h * hd;
    const float4 c = *(const float4*)(rr.cos_t + pos * half + i), sn = *(const float4*)(rr.sin_t + pos * half + i);
    const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {sn.x, sn.y, sn.z, sn.w};
    float lo[4], hi[4];
    // dims i..i+3 and i+half..i+half+3 of a q or k head (natural columns, or pair-interleaved:
    // columns 2i..2i+7 hold dim i, i+half, i+1, i+1+half, ...)
    auto pairs4 = [&](const float* hrow, float4& lo4, float4& hi4) {
      if (rr.perm) {
        const float4 x0 = *(const float4*)(hrow + 2 * i), x1 = *(const float4*)(hrow + 2 * i + 4);
        lo4 = make_float4(x0.x, x0.z, x1.x, x1.z);
        hi4 = make_float4(x0.y, x0.w, x1.y, x1.w);
      } else {
        lo4 = *(const float4*)(hrow + i);
        hi4 = *(const float4*)(hrow + half + i);
      }
    };
    // q
    float4 a, bb;
    pairs4(row, a, bb);
    float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[j] = av[j] * cc[j] - bv[j] * ss[j];
      hi[j] = bv[j] * cc[j] + av[j] * ss[j];
      qs[i + j][tt] = from_f<T>(lo[j]);
      qs[i + j + half][tt] = from_f<T>(hi[j]);
    }
    T* qrow = Q + (bh * rr.n + t) * hd;
    store4<T>(qrow + i, lo[0], lo[1], lo[2], lo[3]);
    store4<T>(qrow + half + i, hi[0], hi[1], hi[2], hi[3]);
    // k
    pairs4(row + d, a, bb);
    av[0] = a.x; av[1] = a.y; av[2] = a.z; av[3] = a.w;
    bv[0] = bb.x; bv[1] = bb.y; bv[2] = bb.z; bv[3] = bb.w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[j] = av[j] * cc[j] - bv[j] * ss[j];
      hi[j] = bv[j] * cc[j] + av[j] * ss[j];
      if constexpr (KTR) {
        ks[i + j][tt] = from_f<T>(lo[j]);
        ks[i + j + half][tt] = from_f<T>(hi[j]);
      }
    }
    T* krow = Kr + (bh * rr.R + slot) * hd;
    store4<T>(krow + i, lo[0], lo[1], lo[2], lo[3]);
    store4<T>(krow + half + i, hi[0], hi[1], hi[2], hi[3]);
    // v
    a = *(const float4*)(row + 2 * d + i);
    bb = *(const float4*)(row + 2 * d + half + i);
    T* vrow = Vr + (bh * rr.R + slot) * hd;
    store4<T>(vrow + i, a.x, a.y, a.z, a.w);
    store4<T>(vrow + half + i, bb.x, bb.y, bb.z, bb.w);
    vt[i][tt] = from_f<T>(a.x);
    vt[i + 1][tt] = from_f<T>(a.y);
    vt[i + 2][tt] = from_f<T>(a.z);
    vt[i + 3][tt] = from_f<T>(a.w);
    vt[i + half][tt] = from_f<T>(bb.x);
    vt[i + half + 1][tt] = from_f<T>(bb.y);
    vt[i + half + 2][tt] = from_f<T>(bb.z);
    vt[i + half + 3][tt] = from_f<T>(bb.w);
  }
  __syncthreads();
  T* Vt = (T*)rr.vtr + bh * hd * rr.R;
  T* Kt = (KTR && rr.ktr) ? (T*)rr.ktr + bh * hd * rr.R : nullptr;
  T* Qt = rr.qt ? (T*)rr.qt + bh * hd * rr.n : nullptr;
  const bool qt4 = rr.n % 4 == 0;
  for (int e = threadIdx.x; e < hd * (RT / 4); e += blockDim.x) {
    const int dim = e / (RT / 4), tt = (e % (RT / 4)) * 4;
    if (tt >= nt) continue;
    const int t = t0 + tt;
    const int slot = (int)((rr.pos0 + t) % rr.R);
    if (tt + 4 <= nt && slot % 4 == 0 && slot + 4 <= rr.R && rr.R % 4 == 0) {
      store4<T>(Vt + (int64_t)dim * rr.R + slot, to_f<T>(vt[dim][tt]), to_f<T>(vt[dim][tt + 1]),
                to_f<T>(vt[dim][tt + 2]), to_f<T>(vt[dim][tt + 3]));
      if constexpr (KTR)
        if (Kt)
          store4<T>(Kt + (int64_t)dim * rr.R + slot, to_f<T>(ks[dim][tt]), to_f<T>(ks[dim][tt + 1]),
                    to_f<T>(ks[dim][tt + 2]), to_f<T>(ks[dim][tt + 3]));
    } else {
      for (int u = 0; u < 4 && tt + u < nt; ++u) {
        const int sl = (int)((rr.pos0 + t + u) % rr.R);
        Vt[(int64_t)dim * rr.R + sl] = vt[dim][tt + u];
        if constexpr (KTR)
          if (Kt) Kt[(int64_t)dim * rr.R + sl] = ks[dim][tt + u];
      }
    }
    if (Qt) {
      if (qt4 && tt + 4 <= nt) {
        store4<T>(Qt + (int64_t)dim * rr.n + t, to_f<T>(qs[dim][tt]), to_f<T>(qs[dim][tt + 1]),
                  to_f<T>(qs[dim][tt + 2]), to_f<T>(qs[dim][tt + 3]));
      } else {
        for (int u = 0; u < 4 && tt + u < nt; ++u) Qt[(int64_t)dim * rr.n + t + u] = qs[dim][tt + u];
      }
    }
  }
}

// the ordered sums from zero of cnt parts (plane floats apart) of the float4s at p and
// p + half, with up to four parts' loads in flight
__device__ inline void sum_parts_pair(const float* p, int half, int cnt, int64_t plane, float4& x, float4& y) {
  x = make_float4(0.f, 0.f, 0.f, 0.f);
  y = x;
  for (int i = 0; i < cnt; i += 4) {
    float4 u[4], v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i + j < cnt) {
        u[j] = *(const float4*)(p + (i + j) * plane);
        v[j] = *(const float4*)(p + (i + j) * plane + half);
      }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i + j < cnt) {
        x.x += u[j].x; x.y += u[j].y; x.z += u[j].z; x.w += u[j].w;
        y.x += v[j].x; y.y += v[j].y; y.z += v[j].z; y.w += v[j].w;
      }
  }
}

// vector form of k_rope_bwd_pack: 4 consecutive pairs per thread (hd % 8 == 0, aligned rows
// and planes)
template <typename T>
__global__ __launch_bounds__(256) void k_rope_bwd_pack4(AttnBwdParts g, const float* cos_t, const float* sin_t,
                                                        int64_t pos0, int64_t M, int n, int H, int hd, T* dqkv) {
  const int half = hd / 2, q4 = half / 4, d = H * hd;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= M * H * q4) return;
  const int64_t m = e / (H * q4);
  const int h = (int)((e / q4) % H), i = (int)(e % q4) * 4;
  const int64_t pos = pos0 + m % n, off = m * d + h * hd + i;
  const float4 c = *(const float4*)(cos_t + pos * half + i), sn = *(const float4*)(sin_t + pos * half + i);
  const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {sn.x, sn.y, sn.z, sn.w};
  T* o = dqkv + m * 3 * d + h * hd;
  const float* src[2] = {g.dq + off, g.dk + off};
  const int cnt[2] = {g.sq, g.pkv};
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    float4 a, bb;
    sum_parts_pair(src[w], half, cnt[w], g.plane, a, bb);
    const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {bb.x, bb.y, bb.z, bb.w};
    float lo[4], hi[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[j] = av[j] * cc[j] + bv[j] * ss[j];
      hi[j] = bv[j] * cc[j] - av[j] * ss[j];
    }
    store4<T>(o + w * d + i, lo[0], lo[1], lo[2], lo[3]);
    store4<T>(o + w * d + half + i, hi[0], hi[1], hi[2], hi[3]);
  }
  float4 a, bb;
  sum_parts_pair(g.dv + off, half, g.pkv, g.plane, a, bb);
  store4<T>(o + 2 * d + i, a.x, a.y, a.z, a.w);
  store4<T>(o + 2 * d + half + i, bb.x, bb.y, bb.z, bb.w);
}

// inverse rotation of dq, dk (gradients w.r.t. rotated q, k) and packing [dq|dk|dv]
template <typename T>
__global__ void k_rope_bwd_pack(AttnBwdParts g, const float* cos_t, const float* sin_t, int64_t pos0, int n, int H,
                                int hd, T* dqkv) {
  int64_t m = blockIdx.x;
  int h = blockIdx.y;
  int t = (int)(m % n);
  int half = hd / 2, d = H * hd;
  int64_t pos = pos0 + t;
  const int64_t off = m * d + h * hd;
  auto sum = [&](const float* p, int cnt) {
    float acc = 0.f;
    for (int j = 0; j < cnt; ++j) acc += p[j * g.plane];
    return acc;
  };
  T* o = dqkv + m * 3 * d + h * hd;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    float c = cos_t[pos * half + i], s = sin_t[pos * half + i];
    float a = sum(g.dq + off + i, g.sq), bb = sum(g.dq + off + i + half, g.sq);
    o[i] = from_f<T>(a * c + bb * s);
    o[i + half] = from_f<T>(bb * c - a * s);
    a = sum(g.dk + off + i, g.pkv);
    bb = sum(g.dk + off + i + half, g.pkv);
    o[d + i] = from_f<T>(a * c + bb * s);
    o[d + i + half] = from_f<T>(bb * c - a * s);
    o[2 * d + i] = from_f<T>(sum(g.dv + off + i, g.pkv));
    o[2 * d + i + half] = from_f<T>(sum(g.dv + off + i + half, g.pkv));
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

namespace {
bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// the bf16 transposed copy [B][d][ldT] of a row-major [B*rpb][d] bf16 matrix
template <typename T>
bool transpose_ok(const T* y, const T* yT, int64_t M, int d, int rpb, int64_t ldT) {
  return sizeof(T) == 2 && y && rpb > 0 && M % rpb == 0 && rpb % 8 == 0 && ldT % 8 == 0 && d % 8 == 0 && al16(y) &&
         al16(yT);
}

template <typename T>
hipError_t transpose_rows(const T* y, T* yT, int64_t M, int d, int rpb, int64_t ldT, hipStream_t s) {
  hipLaunchKernelGGL(k_transpose_rows, dim3(cdiv(rpb, 64), cdiv(d, 64), (unsigned)(M / rpb)), dim3(256), 0, s,
                     (const bf16*)y, (bf16*)yT, rpb, d, ldT);
  return hipGetLastError();
}
}  // namespace

template <typename T>
hipError_t transpose_rows_checked(const T* y, T* yT, int64_t M, int d, int rpb, int64_t ldT, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (!transpose_ok(y, yT, M, d, rpb, ldT)) return hipErrorNotSupported;
  return transpose_rows(y, yT, M, d, rpb, ldT, s);
}

template <typename T>
hipError_t rmsnorm_fwd(const float* x, int64_t M, int d, const float* g, float eps, T* y, float* rstd, T* yT, int rpb,
                       int64_t ldT, float* xcopy, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (y && d % 4 == 0 && d <= 4096 && al16(x) && al16(g) && al16(y) && al16(xcopy) &&
      (!yT || transpose_ok(y, yT, M, d, rpb, ldT))) {
    hipLaunchKernelGGL(k_rmsnorm_fwd_row<T>, dim3((unsigned)M), dim3(256), 0, s, const_cast<float*>(x), nullptr, 0,
                       (int64_t)0, d, g, eps, y, rstd, xcopy);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !yT) return e;
    return transpose_rows(y, yT, M, d, rpb, ldT, s);
  }
  if (xcopy) {
    hipError_t e = hipMemcpyAsync(xcopy, x, (size_t)M * d * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_rmsnorm_fwd<T>, dim3(M), dim3(row_threads(d)), 0, s, x, d, g, eps, y, rstd, yT, rpb, ldT);
  return hipGetLastError();
}

template <typename T>
hipError_t rmsnorm_bwd(const float* x, const float* rstd, int64_t M, int d, const float* g, const float* dy,
                       const float* resid, float* out, T* outT, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (d % 4 == 0 && d <= 4096 && al16(x) && al16(g) && al16(dy) && al16(resid) && al16(out) && al16(outT)) {
    hipLaunchKernelGGL(k_rmsnorm_bwd_row<T>, dim3((unsigned)M), dim3(256), 0, s, x, rstd, d, g, dy, nullptr, 0,
                       (int64_t)0, resid, out, outT);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_rmsnorm_bwd<T>, dim3(M), dim3(row_threads(d)), 0, s, x, rstd, d, g, dy, resid, out, outT);
  return hipGetLastError();
}

static bool parts_ok(int d, const void* a, const void* b, const void* c2, const void* d2, const void* e2) {
  return d % 4 == 0 && d <= 4096 && al16(a) && al16(b) && al16(c2) && al16(d2) && al16(e2);
}

template <typename T>
hipError_t add_rmsnorm_fwd_parts(float* h, const float* parts, int S, int64_t plane, int64_t M, int d, const float* g,
                                 float eps, T* y, float* rstd, T* yT, int rpb, int64_t ldT, float* xcopy,
                                 hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (!(y && parts_ok(d, h, parts, g, y, xcopy) && plane % 4 == 0 && (!yT || transpose_ok(y, yT, M, d, rpb, ldT))))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rmsnorm_fwd_row<T>, dim3((unsigned)M), dim3(256), 0, s, h, parts, S, plane, d, g, eps, y, rstd,
                     xcopy);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !yT) return e;
  return transpose_rows(y, yT, M, d, rpb, ldT, s);
}

template <typename T>
hipError_t rmsnorm_bwd_parts(const float* x, const float* rstd, int64_t M, int d, const float* g, const float* parts,
                             int S, int64_t plane, const float* resid, float* out, T* outT, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (!(parts_ok(d, x, g, parts, resid, out) && al16(outT) && plane % 4 == 0)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rmsnorm_bwd_row<T>, dim3((unsigned)M), dim3(256), 0, s, x, rstd, d, g, nullptr, parts, S,
                     plane, resid, out, outT);
  return hipGetLastError();
}

bool row_parts_ok(int d) { return d % 4 == 0 && d <= 4096; }

template <typename T>
hipError_t convert_rows(const float* x, int64_t M, int d, T* y, T* yT, int rpb, int64_t ldT, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (y && d % 4 == 0 && al16(x) && al16(y) && (!yT || transpose_ok(y, yT, M, d, rpb, ldT))) {
    hipLaunchKernelGGL(k_convert4<T>, dim3(cdiv(M, 4)), dim3(256), 0, s, x, M, d, y);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !yT) return e;
    return transpose_rows(y, yT, M, d, rpb, ldT, s);
  }
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
  if (V % 4 == 0 && ((uintptr_t)logits % 16) == 0 && ((uintptr_t)dlogits % 16) == 0)
    hipLaunchKernelGGL(k_ce_rows4<T>, dim3(M), dim3(512), 0, s, logits, V, tgt, ld, nvalid, rpb, loss_tok, dlogits,
                       err);
  else
    hipLaunchKernelGGL(k_ce_rows<T>, dim3(M), dim3(256), 0, s, logits, V, tgt, ld, nvalid, rpb, loss_tok, dlogits,
                       err);
  return hipGetLastError();
}

template <typename T>
hipError_t ce_finalize(const float* part, const float* zt, int64_t M, int V, const int32_t* tgt, int64_t ld,
                       const int* nvalid, int rpb, float* loss_tok, T* e, int* err, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (sizeof(T) != 2 || V % 8 != 0 || (V + 255) / 256 > 1024 || (e && !al16(e))) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_ce_finalize<T>, dim3((unsigned)M), dim3(256), 0, s, part, zt, M, V, tgt, ld, nvalid, rpb,
                     loss_tok, e, err);
  return hipGetLastError();
}
template hipError_t ce_finalize<bf16>(const float*, const float*, int64_t, int, const int32_t*, int64_t, const int*,
                                      int, float*, bf16*, int*, hipStream_t);
template hipError_t ce_finalize<float>(const float*, const float*, int64_t, int, const int32_t*, int64_t,
                                       const int*, int, float*, float*, int*, hipStream_t);

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
  const bool vec = rr.hd % 8 == 0 && al16(qkv) && al16(rr.cos_t) && al16(rr.sin_t) && al16(rr.q) && al16(rr.kr) &&
                   al16(rr.vr) && al16(rr.vtr) && al16(rr.ktr) && al16(rr.qt);
  if (is_bf16)
    hipLaunchKernelGGL(vec ? k_rope_qkv4<bf16> : k_rope_qkv<bf16>, grid, dim3(256), 0, s, qkv, rr);
  else
    hipLaunchKernelGGL(vec ? k_rope_qkv4<float> : k_rope_qkv<float>, grid, dim3(256), 0, s, qkv, rr);
  return hipGetLastError();
}

template <typename T>
hipError_t rope_bwd_pack(const AttnBwdParts& g, const float* cos_t, const float* sin_t, int64_t pos0, int B, int n,
                         int H, int hd, T* dqkv, hipStream_t s) {
  if (B * n == 0) return hipSuccess;
  if (g.sq < 1 || g.pkv < 1 || ((g.sq > 1 || g.pkv > 1) && g.plane < (int64_t)B * n * H * hd))
    return hipErrorInvalidValue;
  if (hd % 8 == 0 && g.plane % 4 == 0 && al16(g.dq) && al16(g.dk) && al16(g.dv) && al16(cos_t) && al16(sin_t) &&
      al16(dqkv)) {
    const int64_t M = (int64_t)B * n, items = M * H * (hd / 8);
    hipLaunchKernelGGL(k_rope_bwd_pack4<T>, dim3(cdiv(items, 256)), dim3(256), 0, s, g, cos_t, sin_t, pos0, M, n, H,
                       hd, dqkv);
    return hipGetLastError();
  }
  int th = hd / 2 >= 64 ? 64 : 32;
  hipLaunchKernelGGL(k_rope_bwd_pack<T>, dim3(B * n, H), dim3(th), 0, s, g, cos_t, sin_t, pos0, n, H, hd, dqkv);
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

template <typename T>
hipError_t parts_rows_t(const float* parts, int S, int64_t plane, int64_t M, int d, int rpb, T* y, T* yT,
                        hipStream_t s) {
  if (sizeof(T) != 2 || S < 1 || rpb <= 0 || M % rpb != 0 || rpb % 8 != 0 || d % 4 != 0 || plane % 4 != 0 ||
      !al16(parts) || !al16(y) || !al16(yT))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_parts_rows_t, dim3(cdiv(rpb, 64), cdiv(d, 64), (unsigned)(M / rpb)), dim3(256), 0, s, parts,
                     S, plane, rpb, d, (bf16*)y, (bf16*)yT);
  return hipGetLastError();
}

#define INST(T)                                                                                                      \
  template hipError_t embed_gather_ld<T>(const int32_t*, int64_t, int, int, const T*, int, int, float*, int*,       \
                                         hipStream_t);                                                              \
  template hipError_t rmsnorm_fwd<T>(const float*, int64_t, int, const float*, float, T*, float*, T*, int, int64_t, \
                                     float*, hipStream_t);                                                                  \
  template hipError_t add_rmsnorm_fwd_parts<T>(float*, const float*, int, int64_t, int64_t, int, const float*,  \
                                               float, T*, float*, T*, int, int64_t, float*, hipStream_t);         \
  template hipError_t rmsnorm_bwd_parts<T>(const float*, const float*, int64_t, int, const float*, const float*,  \
                                           int, int64_t, const float*, float*, T*, hipStream_t);                   \
  template hipError_t rmsnorm_bwd<T>(const float*, const float*, int64_t, int, const float*, const float*,          \
                                     const float*, float*, T*, hipStream_t);                                        \
  template hipError_t convert_rows<T>(const float*, int64_t, int, T*, T*, int, int64_t, hipStream_t);               \
  template hipError_t transpose_rows_checked<T>(const T*, T*, int64_t, int, int, int64_t, hipStream_t);             \
  template hipError_t parts_rows_t<T>(const float*, int, int64_t, int64_t, int, int, T*, T*, hipStream_t);          \
  template hipError_t ce_rows_ld<T>(const float*, int64_t, int, const int32_t*, int64_t, const int*, int, float*,   \
                                    T*, int*, hipStream_t);                                                         \
  template hipError_t rope_bwd_pack<T>(const AttnBwdParts&, const float*, const float*, int64_t, int, int, int, int, \
                                       T*, hipStream_t);
INST(float)
INST(bf16)
