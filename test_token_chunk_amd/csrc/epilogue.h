// Per-element GEMM epilogues shared by the SIMT and MFMA GEMM kernels.
#pragma once
#include "kernels.h"

// exp: the accurate libm routine on the fp32 path, the hardware exp2 based one on bf16
template <typename T>
__device__ __forceinline__ float epi_exp(float x) {
  if constexpr (sizeof(T) == 4)
    return expf(x);
  else
    return __expf(x);
}

template <typename T, int KIND>
__device__ __forceinline__ void epi_apply_k(const Epi& e, int bz, int m, int n, float acc) {
  switch (KIND) {
    case EPI_F32:
      ((float*)e.c)[bz * e.sc + (int64_t)m * e.ldc + n] = acc;
      break;
    case EPI_T:
      ((T*)e.c)[bz * e.sc + (int64_t)m * e.ldc + n] = from_f<T>(acc);
      break;
    case EPI_ADD_F32: {
      float* p = (float*)e.c + bz * e.sc + (int64_t)m * e.ldc + n;
      *p = *p + acc;
      break;
    }
    case EPI_SWIGLU_BWD: {
      // acc = d act at (m, n); act = silu(zg) * zu
      float zg = to_f<T>(((const T*)e.zg)[bz * e.sz + (int64_t)m * e.ldz + n]);
      float zu = to_f<T>(((const T*)e.zu)[bz * e.sz + (int64_t)m * e.ldz + n]);
      float sg = 1.f / (1.f + epi_exp<T>(-zg));
      float dzu = acc * zg * sg;
      float dzg = acc * zu * sg * (1.f + zg * (1.f - sg));
      T* c = (T*)e.c + bz * e.sc + (int64_t)m * e.ldc;
      c[n] = from_f<T>(dzg);
      c[e.f + n] = from_f<T>(dzu);
      if (e.t) {
        T* t = (T*)e.t + bz * e.st;
        t[(int64_t)n * e.ldt + m] = from_f<T>(dzg);
        t[(int64_t)(e.f + n) * e.ldt + m] = from_f<T>(dzu);
      }
      break;
    }
    case EPI_SGD: {
      float* p = e.master + bz * e.sm + (int64_t)m * e.ldm + n;
      float w = *p - e.lr * acc;
      *p = w;
      // (il_f > 0: the row-major shadow keeps gate/up rows interleaved, as the SwiGLU
      // epilogue of the forward reads them)
      const int64_t shrow = e.il_f ? swiglu_il_row(m, e.il_f) : (int64_t)m;
      ((T*)e.sh)[bz * e.ssh + shrow * e.ldsh + n] = from_f<T>(w);
      ((T*)e.shT)[bz * e.sshT + (int64_t)n * e.ldshT + m] = from_f<T>(w);
      break;
    }
    default:
      break;
  }
}

template <typename T>
__device__ __forceinline__ void epi_apply(const Epi& e, int bz, int m, int n, float acc) {
  switch (e.kind) {
    case EPI_F32: epi_apply_k<T, EPI_F32>(e, bz, m, n, acc); break;
    case EPI_T: epi_apply_k<T, EPI_T>(e, bz, m, n, acc); break;
    case EPI_ADD_F32: epi_apply_k<T, EPI_ADD_F32>(e, bz, m, n, acc); break;
    case EPI_SWIGLU_BWD: epi_apply_k<T, EPI_SWIGLU_BWD>(e, bz, m, n, acc); break;
    case EPI_SGD: epi_apply_k<T, EPI_SGD>(e, bz, m, n, acc); break;
    default: break;
  }
}

// dual-operand epilogue (EPI_SWIGLU): accg = gate pre-activation, accu = up
template <typename T>
__device__ __forceinline__ void epi_apply2(const Epi& e, int bz, int m, int n, float accg, float accu) {
  float act = accg / (1.f + epi_exp<T>(-accg)) * accu;
  ((T*)e.c)[bz * e.sc + (int64_t)m * e.ldc + n] = from_f<T>(act);
  if (e.zg) {
    ((T*)e.zg)[bz * e.sz + (int64_t)m * e.ldz + n] = from_f<T>(accg);
    ((T*)e.zu)[bz * e.sz + (int64_t)m * e.ldz + n] = from_f<T>(accu);
  }
  if (e.t) ((T*)e.t)[bz * e.st + (int64_t)n * e.ldt + m] = from_f<T>(act);
}
