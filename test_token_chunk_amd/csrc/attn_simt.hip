// Sliding-window attention over the key/value ring, SIMT version (one
// wavefront per query and head).  It is the fp32 path and the reference
// layout for the MFMA kernels.  Window: a query at absolute position t sees
// keys t-k < s <= t (and s >= 0); key s lives in ring slot s mod R.
#include "kernels.h"

namespace {

template <typename T>
__device__ __forceinline__ float exp_(float x) {
  if constexpr (sizeof(T) == 4)
    return expf(x);
  else
    return __expf(x);
}

// grid (n, H, B), block 64
template <typename T>
__global__ __launch_bounds__(64) void k_swa_fwd_simt(AttnArgs a) {
  __shared__ float qs[256];
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int hd = a.hd;
  const int64_t bh = (int64_t)b * a.H + h;
  const T* q = (const T*)a.q + (bh * a.n + t) * hd;
  const T* K = (const T*)a.kr + bh * a.R * hd;
  const T* Vv = (const T*)a.vr + bh * a.R * hd;
  for (int i = lane; i < hd; i += 64) qs[i] = to_f<T>(q[i]);
  __syncthreads();
  const float scale = 1.f / sqrtf((float)hd);
  const int64_t pt = a.pos0 + t;
  const int64_t s0 = pt - a.window + 1 > 0 ? pt - a.window + 1 : 0;
  float mx = -INFINITY, l = 0.f;
  float o0 = 0.f, o1 = 0.f;  // dims lane and lane + 64
  for (int64_t j0 = s0; j0 <= pt; j0 += 64) {
    int64_t sp = j0 + lane;
    float sc = -INFINITY;
    if (sp <= pt) {
      const T* kv = K + (sp % a.R) * hd;
      float dot = 0.f;
      for (int i = 0; i < hd; ++i) dot += qs[i] * to_f<T>(kv[i]);
      sc = dot * scale;
    }
    float mnew = fmaxf(mx, warp_max(sc));
    float p = (sp <= pt) ? exp_<T>(sc - mnew) : 0.f;
    float corr = exp_<T>(mx - mnew);
    l = l * corr + warp_sum(p);
    o0 *= corr;
    o1 *= corr;
    int cnt = (int)((pt - j0 + 1) < 64 ? (pt - j0 + 1) : 64);
    for (int j = 0; j < cnt; ++j) {
      float pj = __shfl(p, j, 64);
      const T* vv = Vv + ((j0 + j) % a.R) * hd;
      if (lane < hd) o0 += pj * to_f<T>(vv[lane]);
      if (lane + 64 < hd) o1 += pj * to_f<T>(vv[lane + 64]);
    }
    mx = mnew;
  }
  T* o = (T*)a.o + ((int64_t)b * a.n + t) * (a.H * hd) + h * hd;
  float inv = 1.f / l;
  if (lane < hd) o[lane] = from_f<T>(o0 * inv);
  if (lane + 64 < hd) o[lane + 64] = from_f<T>(o1 * inv);
  if (a.lse && lane == 0) a.lse[bh * a.n + t] = mx + logf(l);
}

// D[t] = sum_i dO[t][i] * O[t][i]; grid (n, H, B), block 64
template <typename T>
__global__ void k_dvec(AttnBwdArgs a) {
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int64_t off = ((int64_t)b * a.n + t) * (a.H * a.hd) + h * a.hd;
  float s = 0.f;
  for (int i = lane; i < a.hd; i += 64) s += to_f<T>(((const T*)a.dout)[off + i]) * to_f<T>(((const T*)a.o)[off + i]);
  s = warp_sum(s);
  if (lane == 0) a.dvec[((int64_t)b * a.H + h) * a.n + t] = s;
}

// dq over the whole window; grid (n, H, B), block 64
template <typename T>
__global__ __launch_bounds__(64) void k_swa_dq_simt(AttnBwdArgs a) {
  __shared__ float qs[256];
  __shared__ float dos[256];
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int hd = a.hd, d = a.H * hd;
  const int64_t bh = (int64_t)b * a.H + h;
  const T* q = (const T*)a.q + (bh * a.n + t) * hd;
  const T* dO = (const T*)a.dout + ((int64_t)b * a.n + t) * d + h * hd;
  const T* K = (const T*)a.kr + bh * a.R * hd;
  const T* Vv = (const T*)a.vr + bh * a.R * hd;
  for (int i = lane; i < hd; i += 64) {
    qs[i] = to_f<T>(q[i]);
    dos[i] = to_f<T>(dO[i]);
  }
  __syncthreads();
  const float scale = 1.f / sqrtf((float)hd);
  const float lse = a.lse[bh * a.n + t], D = a.dvec[bh * a.n + t];
  const int64_t pt = a.pos0 + t;
  const int64_t s0 = pt - a.window + 1 > 0 ? pt - a.window + 1 : 0;
  float g0 = 0.f, g1 = 0.f;
  for (int64_t j0 = s0; j0 <= pt; j0 += 64) {
    int64_t sp = j0 + lane;
    float ds = 0.f;
    if (sp <= pt) {
      const T* kv = K + (sp % a.R) * hd;
      const T* vv = Vv + (sp % a.R) * hd;
      float dot = 0.f, dp = 0.f;
      for (int i = 0; i < hd; ++i) {
        dot += qs[i] * to_f<T>(kv[i]);
        dp += dos[i] * to_f<T>(vv[i]);
      }
      float p = exp_<T>(dot * scale - lse);
      ds = p * (dp - D) * scale;
    }
    int cnt = (int)((pt - j0 + 1) < 64 ? (pt - j0 + 1) : 64);
    for (int j = 0; j < cnt; ++j) {
      float dj = __shfl(ds, j, 64);
      const T* kv = K + ((j0 + j) % a.R) * hd;
      if (lane < hd) g0 += dj * to_f<T>(kv[lane]);
      if (lane + 64 < hd) g1 += dj * to_f<T>(kv[lane + 64]);
    }
  }
  float* o = a.dq + ((int64_t)b * a.n + t) * d + h * hd;
  if (lane < hd) o[lane] = g0;
  if (lane + 64 < hd) o[lane + 64] = g1;
}

// dk, dv of the chunk's own keys (cached keys are constants); grid (n, H, B), block 64
template <typename T>
__global__ __launch_bounds__(64) void k_swa_dkv_simt(AttnBwdArgs a) {
  __shared__ float ks[256];
  __shared__ float vs[256];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;  // key j of the chunk
  const int hd = a.hd, d = a.H * hd;
  const int64_t bh = (int64_t)b * a.H + h;
  const int64_t sp = a.pos0 + j;
  const T* kv = (const T*)a.kr + (bh * a.R + sp % a.R) * hd;
  const T* vv = (const T*)a.vr + (bh * a.R + sp % a.R) * hd;
  for (int i = lane; i < hd; i += 64) {
    ks[i] = to_f<T>(kv[i]);
    vs[i] = to_f<T>(vv[i]);
  }
  __syncthreads();
  const float scale = 1.f / sqrtf((float)hd);
  float gk0 = 0.f, gk1 = 0.f, gv0 = 0.f, gv1 = 0.f;
  // queries t of the chunk with t >= j and pos_t - pos_j < window
  int tend = a.n;
  if ((int64_t)j + a.window < (int64_t)tend) tend = j + a.window;
  for (int t0 = j; t0 < tend; t0 += 64) {
    int t = t0 + lane;
    float p = 0.f, ds = 0.f;
    if (t < tend) {
      const T* q = (const T*)a.q + (bh * a.n + t) * hd;
      const T* dO = (const T*)a.dout + ((int64_t)b * a.n + t) * d + h * hd;
      float dot = 0.f, dp = 0.f;
      for (int i = 0; i < hd; ++i) {
        dot += to_f<T>(q[i]) * ks[i];
        dp += to_f<T>(dO[i]) * vs[i];
      }
      p = exp_<T>(dot * scale - a.lse[bh * a.n + t]);
      ds = p * (dp - a.dvec[bh * a.n + t]) * scale;
    }
    int cnt = tend - t0 < 64 ? tend - t0 : 64;
    for (int u = 0; u < cnt; ++u) {
      float pu = __shfl(p, u, 64), du = __shfl(ds, u, 64);
      const T* q = (const T*)a.q + (bh * a.n + t0 + u) * hd;
      const T* dO = (const T*)a.dout + ((int64_t)b * a.n + t0 + u) * d + h * hd;
      if (lane < hd) {
        gk0 += du * to_f<T>(q[lane]);
        gv0 += pu * to_f<T>(dO[lane]);
      }
      if (lane + 64 < hd) {
        gk1 += du * to_f<T>(q[lane + 64]);
        gv1 += pu * to_f<T>(dO[lane + 64]);
      }
    }
  }
  float* ok = a.dk + ((int64_t)b * a.n + j) * d + h * hd;
  float* ov = a.dv + ((int64_t)b * a.n + j) * d + h * hd;
  if (lane < hd) {
    ok[lane] = gk0;
    ov[lane] = gv0;
  }
  if (lane + 64 < hd) {
    ok[lane + 64] = gk1;
    ov[lane + 64] = gv1;
  }
}

}  // namespace

template <typename T>
hipError_t swa_fwd_simt(const AttnArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  if (a.hd > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_swa_fwd_simt<T>, dim3(a.n, a.H, a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t swa_bwd_simt(const AttnBwdArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  if (a.hd > 128) return hipErrorInvalidValue;
  dim3 grid(a.n, a.H, a.B);
  hipLaunchKernelGGL(k_dvec<T>, grid, dim3(64), 0, s, a);
  hipLaunchKernelGGL(k_swa_dq_simt<T>, grid, dim3(64), 0, s, a);
  hipLaunchKernelGGL(k_swa_dkv_simt<T>, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t swa_dvec_bf16(const AttnBwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_dvec<bf16>, dim3(a.n, a.H, a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

template hipError_t swa_fwd_simt<float>(const AttnArgs&, hipStream_t);
template hipError_t swa_fwd_simt<bf16>(const AttnArgs&, hipStream_t);
template hipError_t swa_bwd_simt<float>(const AttnBwdArgs&, hipStream_t);
template hipError_t swa_bwd_simt<bf16>(const AttnBwdArgs&, hipStream_t);
