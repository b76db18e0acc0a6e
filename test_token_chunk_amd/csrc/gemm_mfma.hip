// bf16 GEMM on the CDNA4 matrix cores: C = A B^T with A [M][K], B [N][K]
// (both K-contiguous), fp32 accumulation in v_mfma_f32_32x32x16_bf16, then the
// shared per-element epilogues (residual add, SwiGLU, SwiGLU backward, fused
// SGD step, ...).
//
// Block tile BM x BN, K step 64, 256 threads = 4 waves in a 2 x 2 grid, each
// wave WM x WN made of 32 x 32 MFMA tiles.  Global -> register -> LDS double
// buffering (one barrier per K step); LDS rows padded by 16 bytes so the
// 16-byte operand reads of a wave spread over all banks.
//
// MFMA 32x32x16 bf16 lane layout (checked on the device): lane l holds
// A[row l%32][k 8*(l/32) .. +7], B[col l%32][k 8*(l/32) .. +7], and
// C[row 8j + 4*(l/32) + i][col l%32] in acc[4j + i].
#include "epilogue.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (elements)

template <int BM, int BN, bool DUAL>
struct Smem {
  bf16 a[2][BM][LDK];
  bf16 b[2][BN][LDK];
  bf16 u[DUAL ? 2 : 1][DUAL ? BN : 1][LDK];
};

// load 16 bytes (8 elements along K) with per-element zero fill past K
// (no address of a local is taken, so everything stays in registers)
__device__ __forceinline__ uint32_t pair(const uint16_t* q, int i, int valid) {
  uint32_t lo = i < valid ? (uint32_t)q[i] : 0u;
  uint32_t hi = i + 1 < valid ? (uint32_t)q[i + 1] : 0u;
  return lo | (hi << 16);
}

__device__ __forceinline__ uint4 ldg16_tail(const bf16* p, int valid) {
  if (valid >= 8) return *(const uint4*)p;
  if (valid <= 0) return make_uint4(0, 0, 0, 0);
  const uint16_t* q = (const uint16_t*)p;
  return make_uint4(pair(q, 0, valid), pair(q, 2, valid), pair(q, 4, valid), pair(q, 6, valid));
}

template <int BM, int BN, int WM, int WN, bool DUAL, int EK>
__global__ __launch_bounds__(256) void k_gemm_mfma(GemmArgs g) {
  constexpr int TM = WM / 32, TN = WN / 32;        // MFMA tiles per wave
  constexpr int A_CH = BM * BK / 8 / 256;          // 16-byte chunks per thread
  constexpr int B_CH = BN * BK / 8 / 256;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem<BM, BN, DUAL>& sm = *reinterpret_cast<Smem<BM, BN, DUAL>*>(smem_raw);

  const int bz = blockIdx.z;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const bf16* A = (const bf16*)g.A + bz * g.sA;
  const bf16* B = (const bf16*)g.B + bz * g.sB;
  const bf16* U = DUAL ? B + g.dual_off * g.ldb : nullptr;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm0 = (wid >> 1) * WM, wn0 = (wid & 1) * WN;
  const int nk = (g.K + BK - 1) / BK;

  uint4 ra[A_CH], rb[B_CH], ru[DUAL ? B_CH : 1];
  auto load = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      int c = tid + i * 256, r = c >> 3, kc = (c & 7) * 8;
      int gm = m0 + r, gk = k0 + kc;
      ra[i] = (gm < g.M) ? ldg16_tail(A + (int64_t)gm * g.lda + gk, g.K - gk) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      int c = tid + i * 256, r = c >> 3, kc = (c & 7) * 8;
      int gn = n0 + r, gk = k0 + kc;
      rb[i] = (gn < g.N) ? ldg16_tail(B + (int64_t)gn * g.ldb + gk, g.K - gk) : make_uint4(0, 0, 0, 0);
      if constexpr (DUAL)
        ru[i] = (gn < g.N) ? ldg16_tail(U + (int64_t)gn * g.ldb + gk, g.K - gk) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      int c = tid + i * 256, r = c >> 3, kc = (c & 7) * 8;
      *(uint4*)&sm.a[buf][r][kc] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      int c = tid + i * 256, r = c >> 3, kc = (c & 7) * 8;
      *(uint4*)&sm.b[buf][r][kc] = rb[i];
      if constexpr (DUAL) *(uint4*)&sm.u[buf][r][kc] = ru[i];
    }
  };

  f32x16 acc[TM][TN];
  f32x16 accu[DUAL ? TM : 1][DUAL ? TN : 1];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      acc[i][j] = f32x16{};
      if constexpr (DUAL) accu[i][j] = f32x16{};
    }

  load(0);
  store(0);
  __syncthreads();
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[TM], bfr[TN], uf[DUAL ? TN : 1];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *(const bf16x8*)&sm.a[cur][wm0 + i * 32 + lr][kk + lk];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        bfr[j] = *(const bf16x8*)&sm.b[cur][wn0 + j * 32 + lr][kk + lk];
        if constexpr (DUAL) uf[j] = *(const bf16x8*)&sm.u[cur][wn0 + j * 32 + lr][kk + lk];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
          if constexpr (DUAL) accu[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], uf[j], accu[i][j], 0, 0, 0);
        }
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  // epilogue: C[row 8q + 4*(l/32) + i][col l%32] = acc[4q + i]
  const int hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn0 + j * 32 + lr;
      if (n >= g.N) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm0 + i * 32 + 8 * q + 4 * hi + r;
          if (m < g.M) {
            if constexpr (DUAL)
              epi_apply2<bf16>(g.e, bz, m, n, acc[i][j][4 * q + r], accu[i][j][4 * q + r]);
            else
              epi_apply_k<bf16, EK>(g.e, bz, m, n, acc[i][j][4 * q + r]);
          }
        }
    }
}

template <int BM, int BN, int WM, int WN, bool DUAL, int EK>
hipError_t launch(const GemmArgs& g, hipStream_t s) {
  auto kern = k_gemm_mfma<BM, BN, WM, WN, DUAL, EK>;
  size_t shm = sizeof(Smem<BM, BN, DUAL>);
  static bool attr_set = false;  // one-time opt-in to more than 64 KB of LDS
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid(cdiv(g.N, BN), cdiv(g.M, BM), g.batch);
  hipLaunchKernelGGL(kern, grid, dim3(256), shm, s, g);
  return hipGetLastError();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

hipError_t gemm_mfma_bf16(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  // 16-byte vector loads need 8-element aligned rows and batch strides
  bool ok = aligned16(g.A) && aligned16(g.B) && g.lda % 8 == 0 && g.ldb % 8 == 0 && g.sA % 8 == 0 &&
            g.sB % 8 == 0 && (g.dual_off * g.ldb) % 8 == 0 && g.K >= 1;
  if (!ok) return gemm_simt_bf16(g, s);
  switch (g.e.kind) {
    case EPI_SWIGLU: return launch<128, 128, 64, 64, true, EPI_SWIGLU>(g, s);
    case EPI_F32: return launch<128, 128, 64, 64, false, EPI_F32>(g, s);
    case EPI_T: return launch<128, 128, 64, 64, false, EPI_T>(g, s);
    case EPI_ADD_F32: return launch<128, 128, 64, 64, false, EPI_ADD_F32>(g, s);
    case EPI_SWIGLU_BWD: return launch<128, 128, 64, 64, false, EPI_SWIGLU_BWD>(g, s);
    case EPI_SGD: return launch<128, 128, 64, 64, false, EPI_SGD>(g, s);
    default: return hipErrorInvalidValue;
  }
}
