// Tiled SIMT GEMM (fp32 FMA) with the shared epilogues.  It is the fp32 path
// (where MFMA bf16 would not meet fp32 accuracy) and the generic fallback for
// shapes the MFMA kernel does not take.
#include "epilogue.h"

namespace {

constexpr int BM = 64, BN = 64, BK = 16;

template <typename T, bool DUAL>
__global__ __launch_bounds__(256) void gemm_simt_kernel(GemmArgs g) {
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  __shared__ float Us[DUAL ? BK : 1][DUAL ? BN + 4 : 1];
  const int bz = blockIdx.z;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const T* A = (const T*)g.A + bz * g.sA;
  const T* B = (const T*)g.B + bz * g.sB;
  const T* U = DUAL ? B + g.dual_off * g.ldb : nullptr;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  float accu[DUAL ? 4 : 1][DUAL ? 4 : 1] = {};
  for (int k0 = 0; k0 < g.K; k0 += BK) {
    // each thread loads 4 elements of A and of B (64 x 16 tiles)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = threadIdx.x + i * 256;
      int r = e / BK, kk = e % BK;
      int gm = m0 + r, gn = n0 + r, gk = k0 + kk;
      As[kk][r] = (gm < g.M && gk < g.K) ? to_f<T>(A[(int64_t)gm * g.lda + gk]) : 0.f;
      Bs[kk][r] = (gn < g.N && gk < g.K) ? to_f<T>(B[(int64_t)gn * g.ldb + gk]) : 0.f;
      if constexpr (DUAL) Us[kk][r] = (gn < g.N && gk < g.K) ? to_f<T>(U[(int64_t)gn * g.ldb + gk]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4], u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty * 4 + i];
        b[i] = Bs[kk][tx * 4 + i];
        if constexpr (DUAL) u[i] = Us[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if constexpr (DUAL) accu[i][j] = fmaf(a[i], u[j], accu[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < g.M && n < g.N) {
        if constexpr (DUAL)
          epi_apply2<T>(g.e, bz, m, n, acc[i][j], accu[i][j]);
        else
          epi_apply<T>(g.e, bz, m, n, acc[i][j]);
      }
    }
}

template <typename T>
hipError_t launch(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  dim3 grid(cdiv(g.N, BN), cdiv(g.M, BM), g.batch);
  if (g.e.kind == EPI_SWIGLU)
    hipLaunchKernelGGL((gemm_simt_kernel<T, true>), grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_simt_kernel<T, false>), grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

// (rows normalized inside the product are a matrix-vector-kernel feature only)
hipError_t gemm_simt_f32(const GemmArgs& g, hipStream_t s) { return g.nx ? hipErrorInvalidValue : launch<float>(g, s); }
hipError_t gemm_simt_bf16(const GemmArgs& g, hipStream_t s) { return g.nx ? hipErrorInvalidValue : launch<bf16>(g, s); }
