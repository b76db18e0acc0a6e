// Products with a handful of rows (decode: one token per sequence), gfx950.
//
// y[b][m][j] = sum_k A[b][m][k] * W[b][j][k] for M <= 8 rows is bound by reading W once
// from HBM; a matrix-core tile of 128 rows would leave 127 of them empty.  One wave
// computes NR output columns: each of the 64 lanes takes 8-element (16-byte) pieces of
// every weight row of those columns, 512 elements per step and up to four steps of loads in
// flight, multiplies them with the matching pieces of the M input rows (bf16 pairs into fp32
// with v_dot2c_f32_bf16) and the wave sums its lanes at the end.  The epilogues are those of
// the matrix-core GEMM (fp32, bf16, residual add, SwiGLU with separate or interleaved gate/up
// rows) and, for the q|k|v projection, RoPE with the writes into the key/value ring
// (EPI_QKV_ROPE: a wave takes the column pair i, i + hd/2 of one head).
#include "kernels.h"

namespace {

constexpr int GW = 4;  // waves per block

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a), __builtin_bit_cast(bf16x2v, b), c, false);
}

__device__ __forceinline__ float dot8(const uint4& a, const uint4& b, float c) {
  c = dot2(a.x, b.x, c);
  c = dot2(a.y, b.y, c);
  c = dot2(a.z, b.z, c);
  return dot2(a.w, b.w, c);
}

__device__ __forceinline__ float sigmoid_g(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// RoPE of the pair (x0, x1) = columns (i, i + hd/2) of head h in part `part` (0 q, 1 k, 2 v) of
// product row m, and its writes: q (and q^T), ring K (and K^T), ring V and V^T
__device__ __forceinline__ void qkv_rope_store(const RopeRing& rr, int part, int h, int i, int m, float x0,
                                               float x1) {
  const int half = rr.hd / 2, b = m / rr.n, t = m % rr.n;
  const int64_t pos = rr.pos0 + t, bh = (int64_t)b * rr.H + h, slot = pos % rr.R;
  float lo = x0, hi = x1;
  if (part < 2) {
    const float c = rr.cos_t[pos * half + i], sn = rr.sin_t[pos * half + i];
    lo = x0 * c - x1 * sn;
    hi = x1 * c + x0 * sn;
  }
  const bf16 l16 = f2bf(lo), h16 = f2bf(hi);
  if (part == 0) {
    bf16* q = (bf16*)rr.q + (bh * rr.n + t) * rr.hd;
    q[i] = l16;
    q[i + half] = h16;
    if (rr.qt) {
      bf16* qt = (bf16*)rr.qt + bh * rr.hd * rr.n + t;
      qt[(int64_t)i * rr.n] = l16;
      qt[(int64_t)(i + half) * rr.n] = h16;
    }
    return;
  }
  bf16* row = (bf16*)(part == 1 ? rr.kr : rr.vr) + (bh * rr.R + slot) * rr.hd;
  row[i] = l16;
  row[i + half] = h16;
  bf16* tr = (bf16*)(part == 1 ? rr.ktr : rr.vtr);
  if (tr) {
    tr += bh * rr.hd * rr.R + slot;
    tr[(int64_t)i * rr.R] = l16;
    tr[(int64_t)(i + half) * rr.R] = h16;
  }
}

template <int MR, int NR, int KIND>
__global__ __launch_bounds__(256) void k_gemv(GemmArgs g, int ncols, int f) {
  constexpr bool SW = KIND == EPI_SWIGLU || KIND == EPI_SWIGLU_IL;
  constexpr bool RP = KIND == EPI_QKV_ROPE;  // NR == 2: the pair (i, i + hd/2); ncols = pairs
  constexpr int RW = SW ? 2 * NR : NR;  // weight rows per wave
  constexpr int U = MR <= 2 ? 4 : 2;    // 512-element steps per trip
  const int lane = threadIdx.x & 63;
  const int64_t wv = (int64_t)blockIdx.x * GW + (threadIdx.x >> 6);
  const int64_t j0 = RP ? wv : wv * NR;
  if (j0 >= ncols) return;
  const int64_t bz = blockIdx.y;
  const bf16* A = (const bf16*)g.A + bz * g.sA;
  const bf16* W = (const bf16*)g.B + bz * g.sB;
  const bf16* wr[RW];
  int part = 0, ph = 0, pi = 0;
  if constexpr (RP) {
    const int half = g.e.rr.hd / 2, hpart = g.e.rr.H * half;
    part = (int)(j0 / hpart);
    ph = (int)(j0 % hpart) / half;
    pi = (int)(j0 % hpart) % half;
    const int64_t c0 = (int64_t)part * g.e.rr.H * g.e.rr.hd + (int64_t)ph * g.e.rr.hd + pi;
    wr[0] = W + c0 * g.ldb;
    wr[1] = W + (c0 + half) * g.ldb;
  }
  if constexpr (!RP) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int64_t j = min(j0 + r, (int64_t)ncols - 1);  // a clamped column is read again, not stored
      if constexpr (KIND == EPI_SWIGLU) {
        wr[2 * r] = W + j * g.ldb;
        wr[2 * r + 1] = W + (j + g.dual_off) * g.ldb;
      } else if constexpr (KIND == EPI_SWIGLU_IL) {
        wr[2 * r] = W + swiglu_il_row(j, f) * g.ldb;
        wr[2 * r + 1] = W + swiglu_il_row(j + f, f) * g.ldb;
      } else {
        wr[r] = W + j * g.ldb;
      }
    }
  }
  const int M = g.M, K = g.K;
  float acc[RW][MR];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[r][m] = 0.f;
  for (int k0 = 8 * lane; k0 < K; k0 += 512 * U) {
    uint4 wv[U][RW], xv[U][MR];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + 512 * u;
      // rows m >= M repeat row M - 1 (their sums are not stored); pieces past K add zero
#pragma unroll
      for (int r = 0; r < RW; ++r) wv[u][r] = k < K ? *(const uint4*)(wr[r] + k) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int m = 0; m < MR; ++m)
        xv[u][m] = k < K ? *(const uint4*)(A + (int64_t)(m < M ? m : M - 1) * g.lda + k) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[r][m] = dot8(wv[u][r], xv[u][m], acc[r][m]);
  }
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[r][m] = warp_sum(acc[r][m]);
  if (lane != 0) return;
  const Epi& e = g.e;
  if constexpr (RP) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
      if (m < M) qkv_rope_store(e.rr, part, ph, pi, m, acc[0][m], acc[1][m]);
    return;
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int64_t j = j0 + r;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (j >= ncols || m >= M) continue;
      const int64_t o = bz * e.sc + (int64_t)m * e.ldc + j;
      if constexpr (SW) {
        const float x = acc[2 * r][m], u = acc[2 * r + 1][m];
        ((bf16*)e.c)[o] = f2bf(x * sigmoid_g(x) * u);
      } else if constexpr (KIND == EPI_F32) {
        ((float*)e.c)[o] = acc[r][m];
      } else if constexpr (KIND == EPI_T) {
        ((bf16*)e.c)[o] = f2bf(acc[r][m]);
      } else {
        ((float*)e.c)[o] += acc[r][m];
      }
    }
  }
}

template <int MR, int NR, int KIND>
hipError_t launch_gemv(const GemmArgs& g, int ncols, int f, hipStream_t s) {
  // one wave per NR columns, or per column pair (ncols counts pairs) with RoPE
  const int64_t waves = KIND == EPI_QKV_ROPE ? ncols : (ncols + NR - 1) / NR;
  hipLaunchKernelGGL((k_gemv<MR, NR, KIND>), dim3((unsigned)((waves + GW - 1) / GW), (unsigned)g.batch),
                     dim3(64 * GW), 0, s, g, ncols, f);
  return hipGetLastError();
}

template <int KIND>
hipError_t gemv_kind(const GemmArgs& g, hipStream_t s) {
  if constexpr (KIND == EPI_QKV_ROPE) {
    const int pairs = g.N / 2;
    if (g.M == 1) return launch_gemv<1, 2, KIND>(g, pairs, 0, s);
    if (g.M == 2) return launch_gemv<2, 2, KIND>(g, pairs, 0, s);
    if (g.M <= 4) return launch_gemv<4, 2, KIND>(g, pairs, 0, s);
    return launch_gemv<8, 2, KIND>(g, pairs, 0, s);
  }
  const bool sw = KIND == EPI_SWIGLU || KIND == EPI_SWIGLU_IL;
  const int ncols = KIND == EPI_SWIGLU_IL ? g.N / 2 : g.N;
  const int f = sw ? ncols : 0;
  // columns per wave: enough waves to fill the chip, more loads in flight per wave for wide outputs
  const int nr = g.M > 2 ? 1 : (ncols >= 16384 ? 4 : (ncols >= 4096 ? 2 : 1));
  if (g.M == 1) {
    if (nr == 4) return launch_gemv<1, 4, KIND>(g, ncols, f, s);
    if (nr == 2) return launch_gemv<1, 2, KIND>(g, ncols, f, s);
    return launch_gemv<1, 1, KIND>(g, ncols, f, s);
  }
  if (g.M == 2) {
    if (nr == 4) return launch_gemv<2, 4, KIND>(g, ncols, f, s);
    if (nr == 2) return launch_gemv<2, 2, KIND>(g, ncols, f, s);
    return launch_gemv<2, 1, KIND>(g, ncols, f, s);
  }
  if (g.M <= 4) return launch_gemv<4, 1, KIND>(g, ncols, f, s);
  return launch_gemv<8, 1, KIND>(g, ncols, f, s);
}

bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

bool gemv_ok(const GemmArgs& g) {
  const int k = g.e.kind;
  if (g.M < 1 || g.M > 8 || g.N < 1 || g.K < 8 || g.K % 8 != 0 || g.batch < 1) return false;
  if (k == EPI_QKV_ROPE) {
    const RopeRing& r = g.e.rr;
    return g.batch == 1 && r.hd > 0 && r.hd % 2 == 0 && r.H > 0 && g.N == 3 * r.H * r.hd && r.n > 0 &&
           g.M % r.n == 0 && r.R > 0 && r.q && r.kr && r.vr && r.cos_t && r.sin_t && al16(g.A) && al16(g.B) &&
           g.lda % 8 == 0 && g.ldb % 8 == 0;
  }
  if (k != EPI_F32 && k != EPI_T && k != EPI_ADD_F32 && k != EPI_SWIGLU && k != EPI_SWIGLU_IL) return false;
  if ((k == EPI_SWIGLU || k == EPI_SWIGLU_IL) && (g.e.zg || g.e.zu || g.e.t)) return false;
  if (k == EPI_SWIGLU_IL && (g.N % 64 != 0 || g.dual_off != 0)) return false;
  return g.e.c && al16(g.A) && al16(g.B) && g.lda % 8 == 0 && g.ldb % 8 == 0 && g.sA % 8 == 0 && g.sB % 8 == 0 &&
         (g.dual_off * g.ldb) % 8 == 0;
}

hipError_t gemv_bf16(const GemmArgs& g, hipStream_t s) {
  if (!gemv_ok(g)) return hipErrorInvalidValue;
  switch (g.e.kind) {
    case EPI_F32: return gemv_kind<EPI_F32>(g, s);
    case EPI_T: return gemv_kind<EPI_T>(g, s);
    case EPI_ADD_F32: return gemv_kind<EPI_ADD_F32>(g, s);
    case EPI_SWIGLU: return gemv_kind<EPI_SWIGLU>(g, s);
    case EPI_SWIGLU_IL: return gemv_kind<EPI_SWIGLU_IL>(g, s);
    case EPI_QKV_ROPE: return gemv_kind<EPI_QKV_ROPE>(g, s);
    default: return hipErrorInvalidValue;
  }
}
