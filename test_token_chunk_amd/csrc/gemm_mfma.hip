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
#include <algorithm>

#include "epilogue.h"

namespace {

// 1 / (1 + e^-x), the logistic function, with the hardware reciprocal (v_rcp_f32, about 1 ulp):
// the bf16 outputs of the matrix-core epilogues do not resolve the difference from a correctly
// rounded division, which takes about ten instructions.  Large negative x: e^-x = inf, 1/inf = 0.
__device__ __forceinline__ float sigmoid_fast(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

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

// Epilogue shared by the GEMM main loops: C[row 8q + 4*(l/32) + i][col l%32] = acc[4q + i]
// of each 32 x 32 tile.  smem_raw (free once the main loop has ended with a barrier) stages
// outputs that are stored transposed.
template <int BM, int BN, int WM, int WN, bool DUAL, int EK, bool SPLIT, int TM = WM / 32, int TN = WN / 32>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, f32x16 (&acc)[TM][TN],
                                              f32x16 (&accu)[DUAL ? TM : 1][DUAL ? TN : 1],
                                              unsigned char* smem_raw, int m0, int n0, int wm0, int wn0, int tid,
                                              int bz, int split, int S) {
  const int lane = tid & 63, lr = lane & 31;
  // Outputs stored transposed ([n][m]: the refreshed W^T shadow of the fused SGD step,
  // act^T, dz^T) are staged through LDS and written as 16-byte row segments.
  constexpr bool TR = (EK == EPI_SGD) || (EK == EPI_SWIGLU_BWD) || DUAL || (EK == EPI_SWIGLU_IL);
  static_assert(EK != EPI_SWIGLU_IL || TN % 2 == 0, "interleaved SwiGLU pairs 32-column halves of a wave");
  constexpr int TLD = BM + 8;
  bf16* tr0 = reinterpret_cast<bf16*>(smem_raw);  // [BN][TLD]
  bf16* tr1 = tr0 + BN * TLD;                     // second tile (dz_u^T)
  static_assert(!TR || (EK == EPI_SWIGLU_BWD ? 2 : 1) * BN * TLD * 2 <= (int)sizeof(Smem<BM, BN, DUAL>),
                "transpose staging fits in the operand buffers");
  const bool want_t = TR && ((EK != EPI_SWIGLU && EK != EPI_SWIGLU_IL) || g.e.t != nullptr);
  const int hi = lane >> 5;
  const Epi& e = g.e;
  // Epilogues that read memory (fp32 master, residual stream) first load every element of
  // a 32-row group of the wave into registers, then compute and store: interleaving a load
  // with the stores of earlier elements would serialize each element on a full memory
  // round trip (the stores may alias the loads).
  constexpr bool READS = (EK == EPI_SGD) || (EK == EPI_ADD_F32);
  if constexpr (EK == EPI_SWIGLU_IL) {
    // lane holds gate column (j = 2p) and up column (j = 2p + 1) of hidden unit fi
#pragma unroll
    for (int jp = 0; jp < TN / 2; ++jp) {
      const int fl = wn0 / 2 + jp * 32 + lr, fi = n0 / 2 + fl;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int ml = wm0 + i * 32 + 8 * q + 4 * hi + r, m = m0 + ml;
            const float x = acc[i][2 * jp][4 * q + r], u = acc[i][2 * jp + 1][4 * q + r];
            const float act = x * sigmoid_fast(x) * u;
            if (m < g.M && 2 * fi < g.N) {
              ((bf16*)e.c)[bz * e.sc + (int64_t)m * e.ldc + fi] = f2bf(act);
              if (e.zg) {
                ((bf16*)e.zg)[bz * e.sz + (int64_t)m * e.ldz + fi] = f2bf(x);
                ((bf16*)e.zu)[bz * e.sz + (int64_t)m * e.ldz + fi] = f2bf(u);
              }
            }
            tr0[fl * TLD + ml] = f2bf(act);
          }
    }
  } else
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float pre0[READS ? TN * 16 : 1];
    if constexpr (READS) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn0 + j * 32 + lr;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = m0 + wm0 + i * 32 + 8 * q + 4 * hi + r;
            const bool in = m < g.M && n < g.N;
            float v = 0.f;
            if constexpr (EK == EPI_SGD) {
              if (in) v = e.master[bz * e.sm + (int64_t)m * e.ldm + n];
            } else {
              if (in) v = ((const float*)e.c)[bz * e.sc + (int64_t)m * e.ldc + n];
            }
            pre0[j * 16 + 4 * q + r] = v;
          }
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int nl = wn0 + j * 32 + lr, n = n0 + nl;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ml = wm0 + i * 32 + 8 * q + 4 * hi + r, m = m0 + ml;
          const int idx = j * 16 + 4 * q + r;
          const bool in = m < g.M && n < g.N;
          const float x = acc[i][j][4 * q + r];
          if constexpr (DUAL) {
            const float u = accu[i][j][4 * q + r];
            const float act = x * sigmoid_fast(x) * u;
            if (in) {
              ((bf16*)e.c)[bz * e.sc + (int64_t)m * e.ldc + n] = f2bf(act);
              if (e.zg) {
                ((bf16*)e.zg)[bz * e.sz + (int64_t)m * e.ldz + n] = f2bf(x);
                ((bf16*)e.zu)[bz * e.sz + (int64_t)m * e.ldz + n] = f2bf(u);
              }
            }
            tr0[nl * TLD + ml] = f2bf(act);
          } else if constexpr (EK == EPI_SGD) {
            if (in) {
              const float w = pre0[idx] - e.lr * x;
              e.master[bz * e.sm + (int64_t)m * e.ldm + n] = w;
              const int64_t shrow = e.il_f ? swiglu_il_row(m, e.il_f) : m;
              ((bf16*)e.sh)[bz * e.ssh + shrow * e.ldsh + n] = f2bf(w);
              tr0[nl * TLD + ml] = f2bf(w);
            }
          } else if constexpr (EK == EPI_SWIGLU_BWD) {
            if (in) {
              const float zg = bf2f(((const bf16*)e.zg)[bz * e.sz + (int64_t)m * e.ldz + n]);
              const float zu = bf2f(((const bf16*)e.zu)[bz * e.sz + (int64_t)m * e.ldz + n]);
              const float sg = sigmoid_fast(zg);
              const float dzu = x * zg * sg;
              const float dzg = x * zu * sg * (1.f + zg * (1.f - sg));
              bf16* c = (bf16*)e.c + bz * e.sc + (int64_t)m * e.ldc;
              c[n] = f2bf(dzg);
              c[e.f + n] = f2bf(dzu);
              tr0[nl * TLD + ml] = f2bf(dzg);
              tr1[nl * TLD + ml] = f2bf(dzu);
            }
          } else if constexpr (EK == EPI_ADD_F32) {
            if (in) ((float*)e.c)[bz * e.sc + (int64_t)m * e.ldc + n] = pre0[idx] + x;
          } else if constexpr (SPLIT) {
            if (in) g.ws[(((int64_t)split * g.batch + bz) * g.M + m) * g.N + n] = x;
          } else {
            if (in) epi_apply_k<bf16, EK>(e, bz, m, n, x);
          }
        }
    }
  }
  if constexpr (TR) {
    if (!want_t) return;
    __syncthreads();
    // tile rows nl (output rows n0+nl) hold BM consecutive m values
    bf16* dst0;
    bf16* dst1 = nullptr;
    int64_t ld;
    if constexpr (EK == EPI_SGD) {
      dst0 = (bf16*)e.shT + bz * e.sshT;
      ld = e.ldshT;
    } else {
      dst0 = (bf16*)e.t + bz * e.st;
      ld = e.ldt;
      if constexpr (EK == EPI_SWIGLU_BWD) dst1 = dst0 + (int64_t)e.f * e.ldt;
    }
    const bool vec = (ld % 8) == 0 && (((uintptr_t)dst0) & 15) == 0;
    constexpr int CH = BM / 8;  // 16-byte chunks per tile row
    constexpr int ROWS = EK == EPI_SWIGLU_IL ? BN / 2 : BN;
    const int row0 = EK == EPI_SWIGLU_IL ? n0 / 2 : n0;
    const int nrows = EK == EPI_SWIGLU_IL ? g.N / 2 : g.N;
    for (int cidx = tid; cidx < ROWS * CH; cidx += 256) {
      const int nl = cidx / CH, ml = (cidx % CH) * 8;
      const int n = row0 + nl, m = m0 + ml;
      if (n >= nrows || m >= g.M) continue;
#pragma unroll
      for (int t = 0; t < (EK == EPI_SWIGLU_BWD ? 2 : 1); ++t) {
        const bf16* srow = (t ? tr1 : tr0) + nl * TLD + ml;
        bf16* drow = (t ? dst1 : dst0) + (int64_t)n * ld + m;
        if (vec && m + 8 <= g.M) {
          *(uint4*)drow = *(const uint4*)srow;
        } else {
          for (int x = 0; x < 8 && m + x < g.M; ++x) drow[x] = srow[x];
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, bool DUAL, int EK, bool SPLIT = false>
__global__ __launch_bounds__(256) void k_gemm_mfma(GemmArgs g) {
  constexpr int TM = WM / 32, TN = WN / 32;        // MFMA tiles per wave
  constexpr int A_CH = BM * BK / 8 / 256;          // 16-byte chunks per thread
  constexpr int B_CH = BN * BK / 8 / 256;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem<BM, BN, DUAL>& sm = *reinterpret_cast<Smem<BM, BN, DUAL>*>(smem_raw);

  // SPLIT: blockIdx.z = batch * S + split; split covers K range [split*Ks, (split+1)*Ks)
  // (S and Ks travel in e.ldt / e.st) and writes fp32 partials to ws[split][batch][M][N].
  const int S = SPLIT ? (int)g.e.ldt : 1;
  const int bz = SPLIT ? blockIdx.z / S : blockIdx.z;
  const int split = SPLIT ? blockIdx.z % S : 0;
  const int kbeg = SPLIT ? split * (int)g.e.st : 0;
  const int kend = SPLIT ? min(g.K, kbeg + (int)g.e.st) : g.K;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const bf16* A = (const bf16*)g.A + bz * g.sA;
  const bf16* B = (const bf16*)g.B + bz * g.sB;
  const bf16* U = DUAL ? B + g.dual_off * g.ldb : nullptr;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm0 = (wid >> 1) * WM, wn0 = (wid & 1) * WN;
  const int nk = (kend - kbeg + BK - 1) / BK;

  uint4 ra[A_CH], rb[B_CH], ru[DUAL ? B_CH : 1];
  // Interior tiles (the common case) load with straight-line 16-byte loads; only tiles
  // that cross M, N or the end of K take the guarded path (a block-uniform branch, so
  // the fast path has no per-load control flow or waits between loads).
  const bool interior_mn = m0 + BM <= g.M && n0 + BN <= g.N;
  auto load = [&](int kt) {
    const int k0 = kbeg + kt * BK;
    if (interior_mn && k0 + BK <= kend) {
#pragma unroll
      for (int i = 0; i < A_CH; ++i) {
        const int c = tid + i * 256, r = c >> 3, kc = (c & 7) * 8;
        ra[i] = *(const uint4*)(A + (int64_t)(m0 + r) * g.lda + k0 + kc);
      }
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = tid + i * 256, r = c >> 3, kc = (c & 7) * 8;
        rb[i] = *(const uint4*)(B + (int64_t)(n0 + r) * g.ldb + k0 + kc);
        if constexpr (DUAL) ru[i] = *(const uint4*)(U + (int64_t)(n0 + r) * g.ldb + k0 + kc);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      int c = tid + i * 256, r = c >> 3, kc = (c & 7) * 8;
      int gm = m0 + r, gk = k0 + kc;
      ra[i] = (gm < g.M) ? ldg16_tail(A + (int64_t)gm * g.lda + gk, kend - gk) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      int c = tid + i * 256, r = c >> 3, kc = (c & 7) * 8;
      int gn = n0 + r, gk = k0 + kc;
      rb[i] = (gn < g.N) ? ldg16_tail(B + (int64_t)gn * g.ldb + gk, kend - gk) : make_uint4(0, 0, 0, 0);
      if constexpr (DUAL)
        ru[i] = (gn < g.N) ? ldg16_tail(U + (int64_t)gn * g.ldb + gk, kend - gk) : make_uint4(0, 0, 0, 0);
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

  gemm_epilogue<BM, BN, WM, WN, DUAL, EK, SPLIT>(g, acc, accu, smem_raw, m0, n0, wm0, wn0, tid, bz, split, S);
}


// ------------------------------------------------------------------ direct-to-LDS main loop
// Same tile (128 x 128, K step 64, 4 waves of 64 x 64) with the operand tiles copied
// straight from global memory into LDS (global_load_lds_dwordx4: lane L of a wave writes
// 16 bytes at the wave's LDS address + 16 L) through a ring of STAGES buffers, so loads run
// STAGES-1 K steps ahead without staging registers.  LDS rows are 128 bytes with the
// 16-byte chunks XOR-swizzled by (row / 2) % 8: a 16-byte fragment read serves 16 lanes (16
// consecutive rows) per pass, and rows 2t and 2t + 1 fall into the two 128-byte halves of the
// banks, so the 16 rows take 16 distinct (half, chunk) places -- no bank conflicts (with
// row % 8, rows r and r + 8 collided).  Requires M, N multiples of 128 and a K range that is a
// multiple of 64.

constexpr int DL_TILE_BYTES = (128 + 128) * BK * 2;  // one stage: A and B tiles

// Tile of a block of the 128 x 128 loop (grid: n tiles, m tiles, batch).  Consecutive
// workgroups of a launch go round-robin to the 8 XCDs, each with its own 4 MB L2: block b of a
// z slice takes logical tile (b % 8) * (nt / 8) + b / 8, so an XCD works through a contiguous
// run of logical tiles, and the logical order walks groups of 8 m tiles column by column, so
// the 64 blocks an XCD holds at a time (two per CU) cover about 8 x 8 tiles and share 8 panels
// of each operand in its L2 instead of fetching a panel per tile.
__device__ __forceinline__ void dl_tile(int& m0, int& n0) {
  const int ntn = gridDim.x, ntm = gridDim.y, nt = ntn * ntm;
  const int lin = blockIdx.y * ntn + blockIdx.x;
  const int lg = nt % 8 == 0 ? (lin % 8) * (nt / 8) + lin / 8 : lin;
  const int GM = min(8, ntm);
  const int grp = lg / (GM * ntn), first = grp * GM, gm = min(ntm - first, GM);
  const int rr = lg - grp * GM * ntn;
  m0 = (first + rr % gm) * 128;
  n0 = (rr / gm) * 128;
}

// Fused SGD step of the 128 x 128 loop with the MFMA operands swapped (lane = output row m,
// four consecutive columns n per register group): the fp32 master values of the tile are
// loaded into registers before the main loop (their latency hides behind it), then
// master -= lr * acc, its row-major bf16 shadow and the transposed shadow go through LDS and
// leave as whole rows (the master and the shadow a quarter of the tile at a time), with
// non-temporal stores: the next chunk reads them, so they need not displace the operand panels
// (and what the kernels of the other streams hold) from the L2s.
typedef float nt_f4 __attribute__((ext_vector_type(4)));
typedef unsigned nt_u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void dl_sgd_prefetch(const GemmArgs& g, float4 (&pre)[2][2][4], int m0, int n0, int wm0,
                                                int wn0, int lane, int bz) {
  const int lr = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm0 + i * 32 + lr, n = n0 + wn0 + j * 32 + 8 * q + 4 * hi;
        pre[i][j][q] = *(const float4*)(g.e.master + bz * g.e.sm + (int64_t)m * g.e.ldm + n);
      }
}

__device__ __forceinline__ void dl_sgd_epilogue(const GemmArgs& g, f32x16 (&acc)[2][2], const float4 (&pre)[2][2][4],
                                                unsigned char* smem_raw, int m0, int n0, int wm0, int wn0, int tid,
                                                int bz) {
  constexpr int BM = 128, BN = 128, TLD = BM + 8, SLD = BN + 4, BLD = BN + 8;
  const int lane = tid & 63, lr = lane & 31, hi = lane >> 5;
  const Epi& e = g.e;
  // LDS: the transposed shadow tile [BN][TLD], then one quarter (32 rows) of the updated master
  // [32][SLD] and of the row-major shadow [32][BLD]; a quarter leaves LDS as whole rows
  bf16* tr = reinterpret_cast<bf16*>(smem_raw);
  float* sq = reinterpret_cast<float*>(smem_raw + BN * TLD * 2);
  bf16* sb = reinterpret_cast<bf16*>(smem_raw + BN * TLD * 2 + 32 * SLD * 4);
#pragma unroll
  for (int Q = 0; Q < 4; ++Q) {
    if (Q > 0) __syncthreads();  // the previous quarter has left LDS
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (wm0 + 32 * i != 32 * Q) continue;  // (wave-uniform)
      const int ml = wm0 + i * 32 + lr;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wn0 + j * 32 + 8 * q + 4 * hi;
          const float4 w = make_float4(pre[i][j][q].x - e.lr * acc[i][j][4 * q], pre[i][j][q].y - e.lr * acc[i][j][4 * q + 1],
                                       pre[i][j][q].z - e.lr * acc[i][j][4 * q + 2],
                                       pre[i][j][q].w - e.lr * acc[i][j][4 * q + 3]);
          const uint32_t p01 = bf16pair(w.x, w.y), p23 = bf16pair(w.z, w.w);
          *(float4*)(sq + lr * SLD + nl) = w;
          *(uint2*)(sb + lr * BLD + nl) = make_uint2(p01, p23);
          tr[(nl + 0) * TLD + ml] = bf16{(uint16_t)p01};
          tr[(nl + 1) * TLD + ml] = bf16{(uint16_t)(p01 >> 16)};
          tr[(nl + 2) * TLD + ml] = bf16{(uint16_t)p23};
          tr[(nl + 3) * TLD + ml] = bf16{(uint16_t)(p23 >> 16)};
        }
    }
    __syncthreads();
    for (int c = tid; c < 32 * (BN / 4); c += 256) {
      const int r = c / (BN / 4), c4 = (c % (BN / 4)) * 4, m = m0 + 32 * Q + r;
      __builtin_nontemporal_store(*(const nt_f4*)(sq + r * SLD + c4), (nt_f4*)(e.master + bz * e.sm + (int64_t)m * e.ldm + n0 + c4));
    }
    for (int c = tid; c < 32 * (BN / 8); c += 256) {
      const int r = c / (BN / 8), c8 = (c % (BN / 8)) * 8, m = m0 + 32 * Q + r;
      const int64_t shrow = e.il_f ? swiglu_il_row(m, e.il_f) : m;
      __builtin_nontemporal_store(*(const nt_u4*)(sb + r * BLD + c8), (nt_u4*)((bf16*)e.sh + bz * e.ssh + shrow * e.ldsh + n0 + c8));
    }
  }
  __syncthreads();
  bf16* dst = (bf16*)e.shT + bz * e.sshT;
  constexpr int CH = BM / 8;
  for (int c = tid; c < BN * CH; c += 256) {
    const int nl = c / CH, ml = (c % CH) * 8;
    __builtin_nontemporal_store(*(const nt_u4*)(tr + nl * TLD + ml), (nt_u4*)(dst + (int64_t)(n0 + nl) * e.ldshT + m0 + ml));
  }
}

static_assert(128 * 136 * 2 + 32 * 132 * 4 + 32 * 136 * 2 <= 2 * DL_TILE_BYTES, "SGD epilogue staging fits two stages");

template <int EK, int STAGES, bool SPLIT>
__global__ __launch_bounds__(256) void k_gemm_dl(GemmArgs g) {
  constexpr int BM = 128, BN = 128, WM = 64, WN = 64, TM = 2, TN = 2;
  constexpr int LPT = (BM + BN) * BK * 2 / 16 / 256;  // 16-byte loads per thread per tile
  static_assert(STAGES >= 2 && STAGES <= 4, "pipeline depth");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int S = SPLIT ? (int)g.e.ldt : 1;
  const int bz = SPLIT ? blockIdx.z / S : blockIdx.z;
  const int split = SPLIT ? blockIdx.z % S : 0;
  const int kbeg = SPLIT ? split * (int)g.e.st : 0;
  const int kend = SPLIT ? min(g.K, kbeg + (int)g.e.st) : g.K;
  int m0, n0;
  dl_tile(m0, n0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS addresses stay scalar
  const int wm0 = (wid >> 1) * WM, wn0 = (wid & 1) * WN;
  const int nk = (kend - kbeg) / BK;

  // 1 KB blocks i = 0..3 of the A and B tiles of step kt (8 rows each).  The 128-row operand
  // panels are buffers: each lane keeps the byte offsets of its rows and chunks, a K step
  // moves only the scalar offset.
  const __amdgpu_buffer_rsrc_t ra = buf_rsrc((const bf16*)g.A + bz * g.sA + (int64_t)m0 * g.lda, (uint32_t)(BM * g.lda * 2));
  const __amdgpu_buffer_rsrc_t rb = buf_rsrc((const bf16*)g.B + bz * g.sB + (int64_t)n0 * g.ldb, (uint32_t)(BN * g.ldb * 2));
  int va[4], vb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (wid * 4 + i) * 8 + (lane >> 3);  // tile row of this lane
    const int c = (lane & 7) ^ ((r >> 1) & 7);      // logical chunk that lands at physical chunk lane & 7
    va[i] = (r * g.lda + c * 8) * 2;
    vb[i] = (r * g.ldb + c * 8) * 2;
  }
  auto issue_one = [&](int kt, int i) {
    unsigned char* base = smem_raw + (kt % STAGES) * DL_TILE_BYTES;
    const int k0b = (kbeg + kt * BK) * 2;
    const int blk = wid * 4 + i;  // 8-row block of the tile (1 KB)
    buf_lds16(ra, base + blk * 1024, va[i], k0b);
    buf_lds16(rb, base + BM * BK * 2 + blk * 1024, vb[i], k0b);
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_one(kt, i);
  };

  f32x16 acc[TM][TN];
  f32x16 accu[1][1];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  // fused SGD step (no K split): the master values of the tile, loaded ahead of the main loop
  constexpr bool SGD = EK == EPI_SGD && !SPLIT;
  float4 pre[SGD ? 2 : 1][SGD ? 2 : 1][SGD ? 4 : 1];
  if constexpr (SGD) dl_sgd_prefetch(g, pre, m0, n0, wm0, wn0, lane, bz);

  const int lr = lane & 31, lk = (lane >> 5) * 8, sw = (lr >> 1) & 7;  // (wm0 + 32 i keeps the swizzle)
  for (int st = 0; st < STAGES - 1 && st < nk; ++st) issue(st);
  for (int kt = 0; kt < nk; ++kt) {
    const int later = min(STAGES - 2, nk - 1 - kt);  // tiles issued after tile kt
    if (later >= 2)
      WAIT_VM(2 * LPT);
    else if (later == 1)
      WAIT_VM(LPT);
    else
      WAIT_VM(0);
    __builtin_amdgcn_s_barrier();  // tile kt is in LDS for all waves; stage of tile kt-1 is free
    // the DMA of tile kt + STAGES - 1 goes out between the MFMAs of this step, a block pair per
    // 16-deep slice (in one burst the vector-memory queue stalls the wave in front of them)
    const bool pend = kt + STAGES - 1 < nk;
    const unsigned char* a_base = smem_raw + (kt % STAGES) * DL_TILE_BYTES;
    const unsigned char* b_base = a_base + BM * BK * 2;
    // fragments of the 16-deep slice kk (logical chunk (kk + lk) / 8 at its swizzled place);
    // those of the next slice are read while the MFMAs of this one run
    auto frags = [&](int kk, bf16x8 (&af)[TM], bf16x8 (&bfr)[TN]) {
      const int p = (((kk + lk) >> 3) ^ sw) << 4;
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *(const bf16x8*)(a_base + (wm0 + i * 32 + lr) * 128 + p);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = *(const bf16x8*)(b_base + (wn0 + j * 32 + lr) * 128 + p);
    };
    bf16x8 af0[TM], bf0[TN], af1[TM], bf1[TN];
    frags(0, af0, bf0);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 (&af)[TM] = (kk / 16) % 2 ? af1 : af0;
      bf16x8 (&bfr)[TN] = (kk / 16) % 2 ? bf1 : bf0;
      if (kk + 16 < BK) {
        if ((kk / 16) % 2) frags(kk + 16, af0, bf0);
        else frags(kk + 16, af1, bf1);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = SGD ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0)
                          : __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      // (with 2 stages the next tile is waited for at the top of the next step: its DMA goes
      // out over the first half of this one)
      if (pend) {
        if constexpr (STAGES == 2) {
          if (kk < BK / 2) {
            issue_one(kt + 1, 2 * (kk / 16));
            issue_one(kt + 1, 2 * (kk / 16) + 1);
          }
        } else {
          issue_one(kt + STAGES - 1, kk / 16);
        }
      }
    }
  }
  WAIT_VM_LDS(0);
  __builtin_amdgcn_s_barrier();  // every wave is done with the operand buffers
  if constexpr (SGD)
    dl_sgd_epilogue(g, acc, pre, smem_raw, m0, n0, wm0, wn0, tid, bz);
  else
    gemm_epilogue<BM, BN, WM, WN, false, EK, SPLIT>(g, acc, accu, smem_raw, m0, n0, wm0, wn0, tid, bz, split, S);
}

// ------------------------------------------------------------------ wide tiles
// BM x 256 block tile, 8 waves in a 2 x 4 grid, each wave (BM/2) x 64 = (BM/64) x 2 MFMA
// tiles, one block (two waves per SIMD) per CU (NW = 4, a 2 x 2 grid of (BM/2) x 128 wave
// tiles at one wave per SIMD, halves the LDS reads per MFMA but measured no faster: LDS
// reads are conflict-free and rarely waited on).  Two configurations:
//   BM = 256: K steps of 32 through a ring of 4 stages (32 KB each; 5 measured no faster);
//   BM = 128: K steps of 64 through a ring of 3 stages (48 KB each).
//
// Operands go straight from global memory to LDS (global_load_lds), WST - 2 steps ahead of
// the step being published.  LDS rows hold one K step of one operand row (64 or 128 bytes) with the
// 16-byte chunks XOR-swizzled by (row / 4) % 4 or (row / 2) % 8, which puts the 16 rows read
// by a quarter-wave on distinct banks.  Inside a step the fragments of the next 16-deep
// slice are read while the MFMAs of the current one run, across the step boundary too:
// the barrier that publishes step kt + 1 sits inside step kt.
//
// The MFMA takes the B fragment as its first operand, so a lane's accumulators hold one
// output row m and four consecutive columns n per 4-register group: the epilogues store
// 16-byte (fp32) or 8-byte (bf16) row segments.
//
// XCD-aware tile order: workgroups are dispatched round-robin over the 8 XCDs, each with
// its own L2.  Block b (1-D grid of 8 * per blocks) takes logical tile (b % 8) * per + b / 8,
// so every XCD walks a contiguous range of logical tiles; logical tiles run down groups of
// up to 8 row tiles before moving to the next column, so the tiles an XCD has in flight
// form a compact rectangle whose operand panels are shared in its L2.
// Requires M % BM == 0, N % 256 == 0 and a K range that is a multiple of the K step.
template <int BM>
struct WideCfg {
  static constexpr int BK = BM == 256 ? 32 : 64;     // K step
  static constexpr int ST = BM == 256 ? 4 : 3;       // ring stages
  static constexpr int RB = BK * 2;                  // LDS row bytes
  static constexpr int SBYTES = (BM + 256) * RB;     // one stage
};

template <int BM, int EK>
constexpr size_t wide_lds_bytes() {
  const size_t ops = (size_t)WideCfg<BM>::ST * WideCfg<BM>::SBYTES;
  const int ntr = EK == EPI_SWIGLU_BWD ? 2 : (EK == EPI_SGD || EK == EPI_QKV_ROPE) ? 1 : 0;
  // (EPI_LM_CE reduces through 2 x 4 x BM floats, well within the operand ring)
  // EPI_SWIGLU_IL: the transposed activations (128 rows of BM + 8) and the activation rows
  // (BM rows of 128 + 8) side by side
  // EPI_ADD_F32: 128 rows of 256 + 4 floats (the residual rows are updated 128 at a time)
  const size_t trb = EK == EPI_SWIGLU_IL ? (size_t)128 * (BM + 8) * 2 + (size_t)BM * 136 * 2
                     : EK == EPI_ADD_F32 ? (size_t)128 * 260 * 4
                                         : (size_t)ntr * 256 * (BM + 8) * 2;
  return ops > trb ? ops : trb;
}

template <int BK>
__device__ __forceinline__ int wide_swz(int row) {
  return BK == 32 ? (row >> 2) & 3 : (row >> 1) & 7;
}

// Epilogue of the wide tiles: lane holds C[m][n .. n+3] with m = m0 + wm0 + 32 i + (l % 32),
// n = n0 + wn0 + 32 j + 8 q + 4 (l / 32) in acc[i][j][4q .. 4q+3].
template <int BM, int EK, bool SPLIT, int TM, int TN, int NT>
__device__ __forceinline__ void wide_epilogue(const GemmArgs& g, f32x16 (&acc)[TM][TN], unsigned char* smem_raw,
                                              int m0, int n0, int wm0, int wn0, int tid, int bz, int split) {
  constexpr int BN = 256;
  const int lane = tid & 63, lr = lane & 31, hi = lane >> 5;
  const Epi& e = g.e;
  constexpr bool TR = EK == EPI_SGD || EK == EPI_SWIGLU_IL || EK == EPI_SWIGLU_BWD;
  constexpr int TLD = BM + 8;
  bf16* tr0 = reinterpret_cast<bf16*>(smem_raw);  // [BN][TLD] (IL: [BN/2][TLD])
  bf16* tr1 = tr0 + BN * TLD;                     // SwiGLU backward: dz_u^T
  auto pk4 = [](float a, float b, float c, float d) {
    return make_uint2(bf16pair(a, b), bf16pair(c, d));
  };
  if constexpr (SPLIT) {
    // fp32 part of a K split: the tile goes through LDS (rows of BN + 4 floats) so that each
    // wave stores whole 1 KB rows instead of 32-byte pieces of 32 rows
    static_assert(BM * (BN + 4) * 4 <= wide_lds_bytes<BM, EK>(), "staged part fits the operand ring");
    constexpr int SLD = BN + 4;
    float* st = reinterpret_cast<float*>(smem_raw);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(float4*)(st + (wm0 + i * 32 + lr) * SLD + wn0 + j * 32 + 8 * q + 4 * hi) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
    __syncthreads();
    float* part = g.ws + (((int64_t)split * g.batch + bz) * g.M + m0) * g.N + n0;
    for (int c = tid; c < BM * (BN / 4); c += NT) {
      const int r = c / (BN / 4), c4 = (c % (BN / 4)) * 4;
      *(float4*)(part + (int64_t)r * g.N + c4) = *(const float4*)(st + r * SLD + c4);
    }
    return;
  }
  if constexpr (EK == EPI_ADD_F32) {
    // residual update c += acc, 128 rows at a time through LDS: each wave reads and writes whole
    // 1 KB rows of c instead of 32-byte pieces of 32 rows
    constexpr int SLD = BN + 4, HR = BM < 128 ? BM : 128;
    float* st = reinterpret_cast<float*>(smem_raw);
    float* cb = (float*)e.c + bz * e.sc + (int64_t)m0 * e.ldc + n0;
#pragma unroll
    for (int h0 = 0; h0 < BM; h0 += HR) {
      if (h0 > 0) __syncthreads();  // the previous rows have been read out of LDS
      if (wm0 >= h0 && wm0 < h0 + HR) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *(float4*)(st + (wm0 - h0 + i * 32 + lr) * SLD + wn0 + j * 32 + 8 * q + 4 * hi) =
                  make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
      __syncthreads();
      for (int c = tid; c < HR * (BN / 4); c += NT) {
        const int r = c / (BN / 4), c4 = (c % (BN / 4)) * 4;
        float* p = cb + (int64_t)(h0 + r) * e.ldc + c4;
        const float4 v = *(const float4*)(st + r * SLD + c4), o = *(const float4*)p;
        *(float4*)p = make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w);
      }
    }
    return;
  }
  if constexpr (EK == EPI_LM_CE) {
    // Vocabulary tile n0 / 256 of the lm_head logits: for each row the maximum m_t of its 256
    // columns and the sum of exp(z - m_t) (fp32, reduced over the lane pair and the 4 column
    // waves through LDS), exp(z - m_t) stored as T, and the fp32 logit of the row's target if
    // it falls in this tile.  Waves: wid / 4 picks the row half, wid % 4 the 64-column group.
    static_assert(NT == 512, "2 x 4 waves");
    float* red = reinterpret_cast<float*>(smem_raw);  // [2][4][BM]: column-group maxima, then sums
    const int wc = wn0 / 64, tn = n0 / BN;
    float mx[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float v = -INFINITY;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) v = fmaxf(v, acc[i][j][r]);
      v = fmaxf(v, __shfl_xor(v, 32, 64));
      if (hi == 0) red[wc * BM + wm0 + i * 32 + lr] = v;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int ml = wm0 + i * 32 + lr, m = m0 + ml;
      mx[i] = fmaxf(fmaxf(red[ml], red[BM + ml]), fmaxf(red[2 * BM + ml], red[3 * BM + ml]));
      const int y = e.tgt[(int64_t)(m / e.rpb) * e.ldtg + m % e.rpb];
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn0 + j * 32 + 8 * q + 4 * hi;
          float x[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float z = acc[i][j][4 * q + r];
            x[r] = __expf(z - mx[i]);
            sum += x[r];
            if (n + r == y) e.ce_zt[m] = z;
          }
          *(uint2*)((bf16*)e.c + (int64_t)m * e.ldc + n) = pk4(x[0], x[1], x[2], x[3]);
        }
      sum += __shfl_xor(sum, 32, 64);
      if (hi == 0) red[4 * BM + wc * BM + ml] = sum;
    }
    __syncthreads();
    if (wc == 0 && hi == 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int ml = wm0 + i * 32 + lr, m = m0 + ml;
        const float sm = (red[4 * BM + ml] + red[5 * BM + ml]) + (red[6 * BM + ml] + red[7 * BM + ml]);
        e.ce_part[(int64_t)tn * 2 * g.M + m] = mx[i];
        e.ce_part[(int64_t)tn * 2 * g.M + g.M + m] = sm;
      }
    }
    return;
  }
  if constexpr (EK == EPI_QKV_ROPE) {
    // [q|k|v] product with pair-interleaved q/k columns (a tile lies in one part): a lane's four
    // columns of a q or k head are dims (i, i + hd/2, i + 1, i + 1 + hd/2), rotated in registers at
    // the row's position; v columns are natural.  Rows go to q [B][H][n][hd] or to ring slot
    // pos % R of K / V [B][H][R][hd]; the transposed copy (q^T, K^T, V^T, where wanted) is staged
    // through LDS by tile column and stored as 8-token segments.  When the tile holds whole heads
    // (hd divides 256) the rows are staged through LDS too and stored as 16-byte segments of whole
    // rows (written directly, a 128-byte line of a q or k row would collect 4-byte pieces from two
    // waves: partial-line writes that the L2 fetches and writes back).
    const RopeRing& rr = e.rr;
    const int hd = rr.hd, half = hd / 2, dm = rr.H * hd;
    const int part = n0 / dm;
    bf16* const rows = (bf16*)(part == 0 ? rr.q : part == 1 ? rr.kr : rr.vr);
    bf16* const tdst = (bf16*)(part == 0 ? rr.qt : part == 1 ? rr.ktr : rr.vtr);
    const int s0 = (int)(rr.pos0 % rr.R);
    const bool staged = BN % hd == 0;
    constexpr int SLD = BN + 8;
    bf16* const st = reinterpret_cast<bf16*>(smem_raw);  // staged rows [BM][SLD], by natural tile column
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int ml = wm0 + i * 32 + lr, m = m0 + ml;
      const int b = m / rr.n, t = m % rr.n;
      const int64_t pos = rr.pos0 + t;
      const int slot = s0 + t >= rr.R ? s0 + t - rr.R : s0 + t;  // t < n <= R
      const float* cs = rr.cos_t + pos * half;
      const float* sn = rr.sin_t + pos * half;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wn0 + j * 32 + 8 * q + 4 * hi, c = n0 + nl - part * dm;
          const int h = c / hd, jj = c % hd;
          float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          if (part < 2) {  // rotate; the pairs become (lo0, hi0, lo1, hi1), kept in acc for the transposed copy
            const int i0 = jj / 2;
            const float2 cc = *(const float2*)(cs + i0), ss = *(const float2*)(sn + i0);
            const float lo0 = v[0] * cc.x - v[1] * ss.x, hi0 = v[1] * cc.x + v[0] * ss.x;
            const float lo1 = v[2] * cc.y - v[3] * ss.y, hi1 = v[3] * cc.y + v[2] * ss.y;
            v[0] = lo0;
            v[1] = hi0;
            v[2] = lo1;
            v[3] = hi1;
            acc[i][j][4 * q] = lo0;
            acc[i][j][4 * q + 1] = hi0;
            acc[i][j][4 * q + 2] = lo1;
            acc[i][j][4 * q + 3] = hi1;
          }
          const uint32_t plo = bf16pair(v[0], v[2]);
          const uint32_t phi = bf16pair(v[1], v[3]);
          if (staged) {
            bf16* srow = st + ml * SLD + (nl - jj);
            if (part < 2) {
              *(uint32_t*)(srow + jj / 2) = plo;
              *(uint32_t*)(srow + jj / 2 + half) = phi;
            } else {
              *(uint2*)(srow + jj) = pk4(v[0], v[1], v[2], v[3]);
            }
          } else {
            const int64_t bh = (int64_t)b * rr.H + h;
            bf16* row = rows + (part == 0 ? bh * rr.n + t : bh * rr.R + slot) * hd;
            if (part < 2) {
              *(uint32_t*)(row + jj / 2) = plo;
              *(uint32_t*)(row + jj / 2 + half) = phi;
            } else {
              *(uint2*)(row + jj) = pk4(v[0], v[1], v[2], v[3]);
            }
          }
        }
    }
    if (staged) {
      __syncthreads();
      constexpr int SEG = BN / 8;  // 16-byte segments per staged row
      const int h0 = (n0 - part * dm) / hd;
      for (int cidx = tid; cidx < BM * SEG; cidx += NT) {
        const int ml = cidx / SEG, cs8 = (cidx % SEG) * 8;
        const int m = m0 + ml, b = m / rr.n, t = m % rr.n;
        const int sl = s0 + t >= rr.R ? s0 + t - rr.R : s0 + t;
        const int64_t bh = (int64_t)b * rr.H + h0 + cs8 / hd;
        bf16* row = rows + (part == 0 ? bh * rr.n + t : bh * rr.R + sl) * hd + cs8 % hd;
        *(uint4*)row = *(const uint4*)(st + ml * SLD + cs8);
      }
    }
    if (!tdst) return;  // (the same for the whole block)
    if (staged) __syncthreads();  // the staged rows have been read: the LDS takes the transposed tile
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int ml = wm0 + i * 32 + lr;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wn0 + j * 32 + 8 * q + 4 * hi;
#pragma unroll
          for (int r = 0; r < 4; ++r) tr0[(nl + r) * TLD + ml] = f2bf(acc[i][j][4 * q + r]);  // pair-interleaved order
        }
    }
    __syncthreads();
    constexpr int CH = BM / 8;
    for (int cidx = tid; cidx < BN * CH; cidx += NT) {
      const int lc = cidx / CH, ml = (cidx % CH) * 8;
      const int c = n0 + lc - part * dm, h = c / hd, jj = c % hd;
      const int dim = part < 2 ? ((jj & 1) ? jj / 2 + half : jj / 2) : jj;
      const int m = m0 + ml, b = m / rr.n, t = m % rr.n;
      const int64_t bh = (int64_t)b * rr.H + h;
      const int sl = s0 + t >= rr.R ? s0 + t - rr.R : s0 + t;
      const int64_t off = part == 0 ? (bh * hd + dim) * rr.n + t : (bh * hd + dim) * rr.R + sl;
      *(uint4*)(tdst + off) = *(const uint4*)(tr0 + lc * TLD + ml);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int ml = wm0 + i * 32 + lr, m = m0 + ml;
    if constexpr (EK == EPI_SWIGLU_IL) {
      static_assert(TN % 2 == 0, "gate and up halves of 64-column groups");
#pragma unroll
      for (int pq = 0; pq < 2 * TN; ++pq) {
        // column group pq / 4 of the wave: accumulators 2 (pq / 4) (gate) and 2 (pq / 4) + 1 (up)
        const int q = pq % 4, jg = 2 * (pq / 4);
        const int fl = (wn0 + 32 * jg) / 2 + 8 * q + 4 * hi, fi = n0 / 2 + fl;
        float x[4], u[4], a[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = acc[i][jg][4 * q + r];
          u[r] = acc[i][jg + 1][4 * q + r];
          a[r] = x[r] * sigmoid_fast(x[r]) * u[r];
        }
        const uint2 ab = pk4(a[0], a[1], a[2], a[3]);
        if (e.t) {
          tr0[(fl + 0) * TLD + ml] = bf16{(uint16_t)ab.x};
          tr0[(fl + 1) * TLD + ml] = bf16{(uint16_t)(ab.x >> 16)};
          tr0[(fl + 2) * TLD + ml] = bf16{(uint16_t)ab.y};
          tr0[(fl + 3) * TLD + ml] = bf16{(uint16_t)(ab.y >> 16)};
        }
        *(uint2*)(tr0 + (BN / 2) * TLD + ml * 136 + fl) = ab;  // activation rows, stored below
        if (e.zg) {
          *(uint2*)((bf16*)e.zg + bz * e.sz + (int64_t)m * e.ldz + fi) = pk4(x[0], x[1], x[2], x[3]);
          *(uint2*)((bf16*)e.zu + bz * e.sz + (int64_t)m * e.ldz + fi) = pk4(u[0], u[1], u[2], u[3]);
        }
      }
    } else {
      // epilogues that read memory load the row group first (stores could alias the loads)
      constexpr bool READS = EK == EPI_SGD || EK == EPI_ADD_F32;
      float4 pre[READS ? TN * 4 : 1];
      uint2 zgp[EK == EPI_SWIGLU_BWD ? TN * 4 : 1], zup[EK == EPI_SWIGLU_BWD ? TN * 4 : 1];
      if constexpr (EK == EPI_SWIGLU_BWD) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn0 + j * 32 + 8 * q + 4 * hi;
            zgp[j * 4 + q] = *(const uint2*)((const bf16*)e.zg + bz * e.sz + (int64_t)m * e.ldz + n);
            zup[j * 4 + q] = *(const uint2*)((const bf16*)e.zu + bz * e.sz + (int64_t)m * e.ldz + n);
          }
      }
      if constexpr (READS) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn0 + j * 32 + 8 * q + 4 * hi;
            pre[j * 4 + q] = EK == EPI_SGD ? *(const float4*)(e.master + bz * e.sm + (int64_t)m * e.ldm + n)
                                           : *(const float4*)((const float*)e.c + bz * e.sc + (int64_t)m * e.ldc + n);
          }
      }
      const int64_t shrow = (EK == EPI_SGD && e.il_f) ? swiglu_il_row(m, e.il_f) : m;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wn0 + j * 32 + 8 * q + 4 * hi, n = n0 + nl;
          const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1], v2 = acc[i][j][4 * q + 2],
                      v3 = acc[i][j][4 * q + 3];
          if constexpr (EK == EPI_F32) {
            *(float4*)((float*)e.c + bz * e.sc + (int64_t)m * e.ldc + n) = make_float4(v0, v1, v2, v3);
          } else if constexpr (EK == EPI_T) {
            *(uint2*)((bf16*)e.c + bz * e.sc + (int64_t)m * e.ldc + n) = pk4(v0, v1, v2, v3);
          } else if constexpr (EK == EPI_ADD_F32) {
            const float4 p = pre[j * 4 + q];
            *(float4*)((float*)e.c + bz * e.sc + (int64_t)m * e.ldc + n) =
                make_float4(p.x + v0, p.y + v1, p.z + v2, p.w + v3);
          } else if constexpr (EK == EPI_SWIGLU_BWD) {
            // dz_g = dact * u * s(1 + g(1 - s)), dz_u = dact * g * s with s = sigmoid(g)
            const uint2 zg2 = zgp[j * 4 + q], zu2 = zup[j * 4 + q];
            const float zg[4] = {bf2f(bf16{(uint16_t)zg2.x}), bf2f(bf16{(uint16_t)(zg2.x >> 16)}),
                                 bf2f(bf16{(uint16_t)zg2.y}), bf2f(bf16{(uint16_t)(zg2.y >> 16)})};
            const float zu[4] = {bf2f(bf16{(uint16_t)zu2.x}), bf2f(bf16{(uint16_t)(zu2.x >> 16)}),
                                 bf2f(bf16{(uint16_t)zu2.y}), bf2f(bf16{(uint16_t)(zu2.y >> 16)})};
            const float x[4] = {v0, v1, v2, v3};
            float dg[4], du[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float sg = sigmoid_fast(zg[r]);
              du[r] = x[r] * zg[r] * sg;
              dg[r] = x[r] * zu[r] * sg * (1.f + zg[r] * (1.f - sg));
              tr0[(nl + r) * TLD + ml] = f2bf(dg[r]);
              tr1[(nl + r) * TLD + ml] = f2bf(du[r]);
            }
            bf16* crow = (bf16*)e.c + bz * e.sc + (int64_t)m * e.ldc;
            *(uint2*)(crow + n) = pk4(dg[0], dg[1], dg[2], dg[3]);
            *(uint2*)(crow + e.f + n) = pk4(du[0], du[1], du[2], du[3]);
          } else if constexpr (EK == EPI_SGD) {
            const float4 p = pre[j * 4 + q];
            const float w0 = p.x - e.lr * v0, w1 = p.y - e.lr * v1, w2 = p.z - e.lr * v2, w3 = p.w - e.lr * v3;
            *(float4*)(e.master + bz * e.sm + (int64_t)m * e.ldm + n) = make_float4(w0, w1, w2, w3);
            const uint2 wb = pk4(w0, w1, w2, w3);
            *(uint2*)((bf16*)e.sh + bz * e.ssh + shrow * e.ldsh + n) = wb;
            tr0[(nl + 0) * TLD + ml] = bf16{(uint16_t)wb.x};
            tr0[(nl + 1) * TLD + ml] = bf16{(uint16_t)(wb.x >> 16)};
            tr0[(nl + 2) * TLD + ml] = bf16{(uint16_t)wb.y};
            tr0[(nl + 3) * TLD + ml] = bf16{(uint16_t)(wb.y >> 16)};
          }
        }
    }
  }
  if constexpr (EK == EPI_SWIGLU_IL) {
    // the activation tile (BM rows of 128) leaves LDS as whole 256-byte row segments
    __syncthreads();
    const bf16* sa = tr0 + (BN / 2) * TLD;
    bf16* cb = (bf16*)e.c + bz * e.sc + (int64_t)m0 * e.ldc + n0 / 2;
    for (int c = tid; c < BM * 16; c += NT) {
      const int r = c / 16, s8 = (c % 16) * 8;
      *(uint4*)(cb + (int64_t)r * e.ldc + s8) = *(const uint4*)(sa + r * 136 + s8);
    }
  }
  if constexpr (TR) {
    if (EK == EPI_SWIGLU_IL && e.t == nullptr) return;
    __syncthreads();
    // tile rows (output rows of the transposed matrix) hold BM consecutive m values
    bf16* dst = EK == EPI_SGD ? (bf16*)e.shT + bz * e.sshT : (bf16*)e.t + bz * e.st;
    const int64_t ld = EK == EPI_SGD ? e.ldshT : e.ldt;
    constexpr int CH = BM / 8;
    constexpr int ROWS = EK == EPI_SWIGLU_IL ? BN / 2 : BN;
    const int row0 = EK == EPI_SWIGLU_IL ? n0 / 2 : n0;
    for (int c = tid; c < ROWS * CH; c += NT) {
      const int rl = c / CH, ml = (c % CH) * 8;
      *(uint4*)(dst + (int64_t)(row0 + rl) * ld + m0 + ml) = *(const uint4*)(tr0 + rl * TLD + ml);
      if constexpr (EK == EPI_SWIGLU_BWD)
        *(uint4*)(dst + (int64_t)e.f * ld + (int64_t)(row0 + rl) * ld + m0 + ml) = *(const uint4*)(tr1 + rl * TLD + ml);
    }
  }
}

template <int BM, int EK, bool SPLIT, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void k_gemm_wide(GemmArgs g) {
  using C = WideCfg<BM>;
  constexpr int BN = 256, BK = C::BK, WST = C::ST, RB = C::RB, SBYTES = C::SBYTES;
  // NW = 8: 2 x 4 waves of (BM / 2) x 64; NW = 4: 2 x 2 waves of (BM / 2) x 128 (half the
  // fragment reads from LDS per MFMA, one wave per SIMD)
  constexpr int WM = BM / 2, WN = 2 * BN / NW, TM = WM / 32, TN = WN / 32;
  constexpr int RPB = 1024 / RB, CPR = RB / 16, NH = BK / 16;
  constexpr int ABYTES = BM * RB, ABLK = BM / RPB / NW, BBLK = BN / RPB / NW;
  constexpr int LPT = ABLK + BBLK;  // 1 KB DMA blocks per wave per step
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int S = SPLIT ? (int)g.e.ldt : 1;
  const int tiles_m = g.M / BM, tiles_n = g.N / BN, tiles = tiles_m * tiles_n;
  const int per = gridDim.x / 8;
  const int t = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (t >= tiles * g.batch * S) return;  // padding block of the last XCD range (uniform, before any barrier)
  const int zz = t / tiles, r = t % tiles;
  const int GM = min(8, tiles_m);
  const int grp = r / (GM * tiles_n), first_m = grp * GM, gm = min(tiles_m - first_m, GM);
  const int rr = r - grp * GM * tiles_n;
  const int m0 = (first_m + rr % gm) * BM, n0 = (rr / gm) * BN;
  const int bz = SPLIT ? zz / S : zz;
  const int split = SPLIT ? zz % S : 0;
  const int kbeg = SPLIT ? split * (int)g.e.st : 0;
  const int kend = SPLIT ? min(g.K, kbeg + (int)g.e.st) : g.K;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS addresses stay scalar
  const int wm0 = (wid / (NW / 2)) * WM, wn0 = (wid % (NW / 2)) * WN;
  const int nk = (kend - kbeg) / BK;
  // 1 KB DMA block = RPB rows; lane L lands at row L / CPR, physical chunk L % CPR and
  // fetches the logical chunk the swizzle puts there.  Wave w copies A blocks
  // [w ABLK, (w+1) ABLK) and B blocks [w BBLK, (w+1) BBLK).  The operand panels (BM rows of A
  // from m0, 256 rows of B from n0) are buffers: each lane keeps the byte offsets of its rows and
  // chunks, and a K step only moves the scalar offset.
  const int lrow = lane / CPR, lpc = lane % CPR;
  const int arow = wid * ABLK * RPB + lrow, brow = wid * BBLK * RPB + lrow;
  const __amdgpu_buffer_rsrc_t ra = buf_rsrc((const bf16*)g.A + bz * g.sA + (int64_t)m0 * g.lda, (uint32_t)(BM * g.lda * 2));
  const __amdgpu_buffer_rsrc_t rb = buf_rsrc((const bf16*)g.B + bz * g.sB + (int64_t)n0 * g.ldb, (uint32_t)(BN * g.ldb * 2));
  int voff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    if (i < ABLK) {
      const int r = arow + i * RPB;
      voff[i] = (r * g.lda + (lpc ^ wide_swz<BK>(r)) * 8) * 2;
    } else {
      const int r = brow + (i - ABLK) * RPB;
      voff[i] = (r * g.ldb + (lpc ^ wide_swz<BK>(r)) * 8) * 2;
    }
  }

  // DMA block i (0 .. LPT-1: A blocks, then B blocks) of step kt
  auto issue_one = [&](int kt, int i) {
    unsigned char* base = smem_raw + (kt % WST) * SBYTES;
    const int k0b = (kbeg + kt * BK) * 2;
    if (i < ABLK) buf_lds16(ra, base + (wid * ABLK + i) * 1024, voff[i], k0b);
    else buf_lds16(rb, base + ABYTES + (wid * BBLK + (i - ABLK)) * 1024, voff[i], k0b);
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) issue_one(kt, i);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  const int lr = lane & 31, lk = lane >> 5, sw = wide_swz<BK>(lr);
  const int a_off = (wm0 + lr) * RB, b_off = ABYTES + (wn0 + lr) * RB;
  bf16x8 f0a[TM], f0b[TN], f1a[TM], f1b[TN];
  // fragments of 16-deep slice h of step kt: logical chunk 2h + lk of the row
#define FRAGS(fa, fb, kt, h)                                                                   \
  {                                                                                            \
    const unsigned char* sb = smem_raw + ((kt) % WST) * SBYTES;                                \
    const int p = ((2 * (h) + lk) ^ sw) << 4;                                                  \
    _Pragma("unroll") for (int i = 0; i < TM; ++i) fa[i] = *(const bf16x8*)(sb + a_off + i * 32 * RB + p); \
    _Pragma("unroll") for (int j = 0; j < TN; ++j) fb[j] = *(const bf16x8*)(sb + b_off + j * 32 * RB + p); \
  }
#define MFMA_ROWS(fa, fb, i0, i1)                                                              \
  _Pragma("unroll") for (int i = (i0); i < (i1); ++i)                                          \
    _Pragma("unroll") for (int j = 0; j < TN; ++j)                                             \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
#define SB() __builtin_amdgcn_sched_barrier(0)
  // The DMA of step kt + WST - 1 is spread over the MFMA rows that follow the barrier (2 TM - 1
  // slots: rows 1 .. TM-1 of half-step NH-2, rows 0 .. TM-1 of half-step NH-1): issued in one
  // burst, the queue of vector-memory instructions stalls the wave in front of its MFMAs.
  // DMA block i goes after slot i (2 TM - 1) / LPT.
  constexpr int NSLOT = 2 * TM - 1;
#define DMA_SLOT(slot)                                                                         \
  if (pend) {                                                                                  \
    _Pragma("unroll") for (int i = 0; i < LPT; ++i) if (i * NSLOT / LPT == (slot)) issue_one(kt + WST - 1, i); \
  }
  // waits until at most `later` steps of DMA are outstanding (later <= 3 here)
#define WAIT_STEPS(later)                                                                      \
  {                                                                                            \
    if ((later) >= 3) WAIT_VM(3 * LPT);                                                        \
    else if ((later) == 2) WAIT_VM(2 * LPT);                                                   \
    else if ((later) == 1) WAIT_VM(LPT);                                                       \
    else WAIT_VM(0);                                                                           \
  }
  static_assert(WST - 2 <= 3 && WST >= 3, "ring depth");

  // prologue: steps 0 .. WST-2 in flight, step 0 published, its first slice in registers
  for (int st = 0; st < WST - 1 && st < nk; ++st) issue(st);
  if (nk > 0) {
    WAIT_STEPS(min(WST - 2, nk - 1));
    __builtin_amdgcn_s_barrier();
    FRAGS(f0a, f0b, 0, 0)
  }
  SB();
  for (int kt = 0; kt < nk; ++kt) {
    // invariant: f0 holds slice 0 of step kt; step kt is published; every wave has finished
    // reading step kt - 1
    const bool more = kt + 1 < nk;
    const bool pend = kt + WST - 1 < nk;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      // the fragments of the next slice are read before this slice's MFMAs, so all TM rows of
      // MFMAs cover the LDS latency
      if ((h & 1) == 0) {
        if (h + 1 < NH) FRAGS(f1a, f1b, kt, h + 1)
        SB();
        MFMA_ROWS(f0a, f0b, 0, 1)
        SB();
        if (h == NH - 2 && more) {
          // publish step kt + 1 (issued WST - 2 steps ago) for every wave; the barrier also
          // tells that every wave is past its reads of step kt - 1, whose stage is reused next
          WAIT_STEPS(min(WST - 3, nk - 2 - kt));
          __builtin_amdgcn_s_barrier();
        }
        SB();
        _Pragma("unroll") for (int r = 1; r < TM; ++r) {
          MFMA_ROWS(f0a, f0b, r, r + 1)
          SB();
          if (h == NH - 2) DMA_SLOT(r - 1)
          SB();
        }
      } else {
        if (h + 1 < NH) {
          FRAGS(f0a, f0b, kt, h + 1)
        } else if (more) {
          FRAGS(f0a, f0b, kt + 1, 0)
        }
        SB();
        MFMA_ROWS(f1a, f1b, 0, 1)
        SB();
        if (h == NH - 1) DMA_SLOT(TM - 1)
        SB();
        _Pragma("unroll") for (int r = 1; r < TM; ++r) {
          MFMA_ROWS(f1a, f1b, r, r + 1)
          SB();
          if (h == NH - 1) DMA_SLOT(TM - 1 + r)
          SB();
        }
      }
    }
  }
#undef FRAGS
#undef MFMA_ROWS
#undef DMA_SLOT
#undef SB
#undef WAIT_STEPS
  WAIT_VM_LDS(0);
  __syncthreads();  // every wave is done with the operand buffers
  wide_epilogue<BM, EK, SPLIT, TM, TN, 64 * NW>(g, acc, smem_raw, m0, n0, wm0, wn0, tid, bz, split);
}

template <int BM, int EK, bool SPLIT, int NW = 8>
hipError_t launch_wide(const GemmArgs& g, int S, hipStream_t s) {
  auto kern = k_gemm_wide<BM, EK, SPLIT, NW>;
  constexpr size_t shm = wide_lds_bytes<BM, EK>();
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t tiles = (int64_t)(g.M / BM) * (g.N / 256) * g.batch * S;
  hipLaunchKernelGGL(kern, dim3((unsigned)(8 * cdiv(tiles, 8))), dim3(64 * NW), shm, s, g);
  return hipGetLastError();
}

template <int EK>
hipError_t launch_wide_bm(const GemmArgs& g, int bm, hipStream_t s) {
  return bm == 256 ? launch_wide<256, EK, false>(g, 1, s) : launch_wide<128, EK, false>(g, 1, s);
}

template <int EK, bool SPLIT, int STAGES>
hipError_t launch_dl_st(const GemmArgs& g, int S, hipStream_t s) {
  auto kern = k_gemm_dl<EK, STAGES, SPLIT>;
  const size_t shm = std::max<size_t>(STAGES * DL_TILE_BYTES, sizeof(Smem<128, 128, false>));
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid(cdiv(g.N, 128), cdiv(g.M, 128), g.batch * S);
  hipLaunchKernelGGL(kern, grid, dim3(256), shm, s, g);
  return hipGetLastError();
}

template <int EK, bool SPLIT>
hipError_t launch_dl(const GemmArgs& g, int S, hipStream_t s) {
  static int stages = -1;  // TTT_GEMM_STAGES (tuning switch) or 0 = by role
  if (stages < 0) {
    const char* e = getenv("TTT_GEMM_STAGES");
    stages = e ? atoi(e) : 0;
  }
  // background work: three stages (96 KB of LDS, one block per CU), which leaves the other
  // half of each CU's block slots to the latency-bound kernels of the main stream (3B step, same
  // box: 2016 -> 1970 ms although the weight-gradient GEMMs themselves take twice as long)
  if (stages == 0 && g.background) return launch_dl_st<EK, SPLIT, 3>(g, S, s);
  if (stages == 4) return launch_dl_st<EK, SPLIT, 4>(g, S, s);
  if (stages == 3) return launch_dl_st<EK, SPLIT, 3>(g, S, s);
  return launch_dl_st<EK, SPLIT, 2>(g, S, s);
}

// shapes the direct-to-LDS loop takes
bool dl_ok(const GemmArgs& g, int Ks) {
  const char* off = getenv("TTT_GEMM_NO_DL");
  if (off && off[0] == '1') return false;
  return g.M % 128 == 0 && g.N % 128 == 0 && g.K % BK == 0 && Ks % BK == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
         g.e.kind != EPI_SWIGLU &&
         // 128-row operand panels are buffers with 32-bit byte offsets
         (int64_t)128 * g.lda * 2 < (1LL << 31) && (int64_t)128 * g.ldb * 2 < (1LL << 31);
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

// out = epilogue(sum_s ws[s]) for the split-K parts; the sum runs over s in order
template <int EK>
__global__ void k_splitk_reduce(GemmArgs g, int S) {
  const int64_t per = (int64_t)g.M * g.N;
  const int64_t total = per * g.batch;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    float acc = 0.f;
    for (int sidx = 0; sidx < S; ++sidx) acc += g.ws[sidx * total + i];
    const int bz = (int)(i / per);
    const int64_t r = i % per;
    epi_apply_k<bf16, EK>(g.e, bz, (int)(r / g.N), (int)(r % g.N), acc);
  }
}

// the same four elements of a row at a time (N, ldc, the batch stride and c are multiples of
// four elements / 16 bytes): 16-byte part reads, 16-byte fp32 or 8-byte bf16 stores
template <int EK>
__global__ __launch_bounds__(256) void k_splitk_reduce4(GemmArgs g, int S) {
  const int64_t per = (int64_t)g.M * g.N;
  const int64_t total = per * g.batch, total4 = total / 4;
  const Epi& e = g.e;
  for (int64_t i4 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i4 < total4; i4 += (int64_t)gridDim.x * blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sidx = 0; sidx < S; ++sidx) {
      const float4 v = *(const float4*)(g.ws + sidx * total + 4 * i4);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const int64_t i = 4 * i4;
    const int64_t bz = i / per, r = i % per, m = r / g.N, n = r % g.N;
    if constexpr (EK == EPI_F32) {
      *(float4*)((float*)e.c + bz * e.sc + m * e.ldc + n) = acc;
    } else if constexpr (EK == EPI_T) {
      const uint2 w = make_uint2(bf16pair(acc.x, acc.y), bf16pair(acc.z, acc.w));
      *(uint2*)((bf16*)e.c + bz * e.sc + m * e.ldc + n) = w;
    } else {
      float* c = (float*)e.c + bz * e.sc + m * e.ldc + n;
      const float4 p = *(const float4*)c;
      *(float4*)c = make_float4(p.x + acc.x, p.y + acc.y, p.z + acc.z, p.w + acc.w);
    }
  }
}

hipError_t launch_splitk(const GemmArgs& g0, int S, int Ks, bool wide, hipStream_t s) {
  GemmArgs g = g0;
  g.e.ldt = S;   // carried to the kernel
  g.e.st = Ks;
  if (wide) {
    hipError_t e = launch_wide<128, EPI_F32, true>(g, S, s);
    if (e != hipSuccess) return e;
  } else if (dl_ok(g, Ks)) {
    hipError_t e = launch_dl<EPI_F32, true>(g, S, s);
    if (e != hipSuccess) return e;
  } else {
    auto kern = k_gemm_mfma<128, 128, 64, 64, false, EPI_F32, true>;
    static bool attr_set = false;
    const size_t shm = sizeof(Smem<128, 128, false>);
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    dim3 grid(cdiv(g.N, 128), cdiv(g.M, 128), g.batch * S);
    hipLaunchKernelGGL(kern, grid, dim3(256), shm, s, g);
  }
  if (g0.defer) return hipGetLastError();  // the caller sums the parts
  const int64_t total = (int64_t)g.batch * g.M * g.N;
  const bool vec = g.N % 4 == 0 && g.e.ldc % 4 == 0 && g.e.sc % 4 == 0 && ((uintptr_t)g.e.c % 16) == 0 &&
                   ((uintptr_t)g.ws % 16) == 0;
  if (vec) {
    dim3 rg4((unsigned)std::min<int64_t>(cdiv(total / 4, 256), 8192));
    switch (g0.e.kind) {
      case EPI_F32: hipLaunchKernelGGL(k_splitk_reduce4<EPI_F32>, rg4, dim3(256), 0, s, g0, S); break;
      case EPI_T: hipLaunchKernelGGL(k_splitk_reduce4<EPI_T>, rg4, dim3(256), 0, s, g0, S); break;
      case EPI_ADD_F32: hipLaunchKernelGGL(k_splitk_reduce4<EPI_ADD_F32>, rg4, dim3(256), 0, s, g0, S); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  dim3 rg((unsigned)std::min<int64_t>(cdiv(total, 256), 4096));
  switch (g0.e.kind) {
    case EPI_F32: hipLaunchKernelGGL(k_splitk_reduce<EPI_F32>, rg, dim3(256), 0, s, g0, S); break;
    case EPI_T: hipLaunchKernelGGL(k_splitk_reduce<EPI_T>, rg, dim3(256), 0, s, g0, S); break;
    case EPI_ADD_F32: hipLaunchKernelGGL(k_splitk_reduce<EPI_ADD_F32>, rg, dim3(256), 0, s, g0, S); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

namespace {

// Which main loop runs a GEMM, with how many K parts.
//   kern 3 / 2: wide tiles with BM = 256 / 128; 1: 128 x 128 direct-to-LDS; 0: 128 x 128
//   register-staged (any shape).
// Small grids with a long K (the N = d GEMMs of the per-chunk upper blocks) split K over
// several blocks into an fp32 workspace; one pass then sums the parts in a fixed order and
// applies the epilogue.
struct GemmPlan {
  int kern, S, Ks;
};

bool al(const void* p, int bytes) { return ((uintptr_t)p % bytes) == 0; }

bool wide_ok(const GemmArgs& g) {
  static int off = -1;
  if (off < 0) {
    const char* e = getenv("TTT_GEMM_NO_WIDE");
    off = e && e[0] == '1';
  }
  if (off) return false;
  if (!(g.M % 128 == 0 && g.N % 256 == 0 && g.K % 64 == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0)) return false;
  // operand panels of 256 rows are addressed as buffers with 32-bit byte offsets
  if ((int64_t)256 * g.lda * 2 >= (1LL << 31) || (int64_t)256 * g.ldb * 2 >= (1LL << 31)) return false;
  // the epilogues store 4-element row segments (and 8-element transposed segments)
  const Epi& e = g.e;
  switch (e.kind) {
    case EPI_F32:
    case EPI_ADD_F32: return e.ldc % 4 == 0 && e.sc % 4 == 0 && al(e.c, 16);
    case EPI_T: return e.ldc % 4 == 0 && e.sc % 4 == 0 && al(e.c, 8);
    case EPI_SWIGLU_IL:
      return e.ldc % 8 == 0 && e.sc % 8 == 0 && al(e.c, 16) &&
             (!e.zg || (e.ldz % 4 == 0 && e.sz % 4 == 0 && al(e.zg, 8) && al(e.zu, 8))) &&
             (!e.t || (e.ldt % 8 == 0 && e.st % 8 == 0 && al(e.t, 16)));
    case EPI_SGD:
      return e.ldm % 4 == 0 && e.sm % 4 == 0 && al(e.master, 16) && e.ldsh % 4 == 0 && e.ssh % 4 == 0 &&
             al(e.sh, 8) && e.ldshT % 8 == 0 && e.sshT % 8 == 0 && al(e.shT, 16);
    case EPI_SWIGLU_BWD:
      return e.ldc % 4 == 0 && e.sc % 4 == 0 && e.f % 4 == 0 && al(e.c, 8) && e.ldz % 4 == 0 && e.sz % 4 == 0 &&
             al(e.zg, 8) && al(e.zu, 8) && e.t && e.ldt % 8 == 0 && e.st % 8 == 0 && al(e.t, 16);
    case EPI_LM_CE:
      return g.batch == 1 && e.ldc % 4 == 0 && al(e.c, 8) && e.tgt && e.rpb > 0 && g.M % e.rpb == 0 && e.ce_part &&
             e.ce_zt;
    case EPI_QKV_ROPE: {
      // a 256-column tile inside one of q, k, v; RoPE pairs in a lane's 4-column group; 8-token
      // groups of a tile inside one batch row and one run of ring slots (16-byte transposed stores)
      const RopeRing& r = e.rr;
      const int64_t dm = (int64_t)r.H * r.hd;
      return g.batch == 1 && r.perm && r.hd % 4 == 0 && r.hd <= 256 && dm % 256 == 0 && g.N == 3 * dm && r.n > 0 &&
             r.n % 8 == 0 && g.M % r.n == 0 && r.n <= r.R && r.pos0 % 8 == 0 && r.R % 8 == 0 && r.q && r.kr &&
             r.vr && r.vtr && r.cos_t && r.sin_t && al(r.q, 8) && al(r.kr, 8) && al(r.vr, 8) && al(r.vtr, 16) &&
             al(r.ktr, 16) && al(r.qt, 16) && al(r.cos_t, 8) && al(r.sin_t, 8);
    }
    default: return false;
  }
}

GemmPlan gemm_plan(const GemmArgs& g) {
  // a handful of rows: the matrix-vector kernel, one pass over the weights, no K split
  if (gemv_ok(g)) return {4, 1, g.K};
  const bool splittable = g.e.kind == EPI_F32 || g.e.kind == EPI_T || g.e.kind == EPI_ADD_F32;
  // short K (the weight gradients over one chunk): the prologue and the epilogue weigh as much as
  // the main loop, and two 128 x 128 blocks per CU overlap them better than one wide block
  if (g.K <= 1024 && g.e.kind == EPI_SGD && dl_ok(g, g.K)) return {1, 1, g.K};
  if (wide_ok(g)) {
    const int64_t t128 = (int64_t)(g.M / 128) * (g.N / 256) * g.batch;
    // (the SwiGLU backward's two transposed tiles fit beside 128-row tiles only)
    const int64_t t256 =
        g.M % 256 == 0 && g.e.kind != EPI_SWIGLU_BWD ? (int64_t)(g.M / 256) * (g.N / 256) * g.batch : 0;
    if (g.ws && splittable && t128 < 192 && g.K >= 1024 && al(g.ws, 16)) {
      int S = (int)std::min<int64_t>(8, std::max<int64_t>(2, 256 / t128));
      S = std::min(S, g.K / 256);
      const int Ks = (int)cdiv(cdiv(g.K, S), 64) * 64;
      S = (int)cdiv(g.K, Ks);
      if (S >= 2 && (int64_t)S * g.batch * g.M * g.N <= g.ws_floats) return {2, S, Ks};
    }
    // one block per CU: rounds of 256 tiles; a 128-row tile costs a little over half a 256-row one
    const double c256 = t256 ? (double)cdiv(t256, 256) : 1e30;
    const double c128 = 0.55 * (double)cdiv(t128, 256);
    return {c256 <= c128 ? 3 : 2, 1, g.K};
  }
  const int64_t tiles = (int64_t)cdiv(g.M, 128) * cdiv(g.N, 128) * g.batch;
  if (g.ws && tiles < 384 && g.K >= 1024 && splittable) {
    int S = (int)std::min<int64_t>(8, (640 + tiles - 1) / tiles);
    S = std::min(S, g.K / 256);
    const int Ks = (int)cdiv(cdiv(g.K, S), BK) * BK;
    S = (int)cdiv(g.K, Ks);
    if (S >= 2 && (int64_t)S * g.batch * g.M * g.N <= g.ws_floats) return {dl_ok(g, Ks) ? 1 : 0, S, Ks};
  }
  return {dl_ok(g, g.K) ? 1 : 0, 1, g.K};
}

}  // namespace

bool gemm_mfma_fuses_lm_ce(const GemmArgs& g) {
  if (g.e.kind != EPI_LM_CE || g.M <= 0) return false;
  if (!(aligned16(g.A) && aligned16(g.B) && g.lda % 8 == 0 && g.ldb % 8 == 0)) return false;
  return wide_ok(g);
}

bool gemm_mfma_fuses_qkv_rope(const GemmArgs& g) {
  if (g.e.kind != EPI_QKV_ROPE || g.M <= 0) return false;
  if (g.nx) return gemv_ok(g);
  if (!(aligned16(g.A) && aligned16(g.B) && g.lda % 8 == 0 && g.ldb % 8 == 0)) return false;
  return gemv_ok(g) || wide_ok(g);
}

// split-K parts for this GEMM (1: no split)
int gemm_mfma_splits(const GemmArgs& g, int* ks_out) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return 1;
  const GemmPlan p = gemm_plan(g);
  if (ks_out) *ks_out = p.Ks;
  return p.S;
}

hipError_t gemm_mfma_bf16(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  // rows normalized in the kernel: only the matrix-vector form does that
  if (g.nx) return gemv_ok(g) ? gemv_bf16(g, s) : hipErrorInvalidValue;
  // 16-byte vector loads need 8-element aligned rows and batch strides
  bool ok = aligned16(g.A) && aligned16(g.B) && g.lda % 8 == 0 && g.ldb % 8 == 0 && g.sA % 8 == 0 &&
            g.sB % 8 == 0 && (g.dual_off * g.ldb) % 8 == 0 && g.K >= 1;
  if (!ok) return g.e.kind == EPI_SWIGLU_IL ? hipErrorInvalidValue : gemm_simt_bf16(g, s);
  if (g.e.kind == EPI_SWIGLU_IL && (g.N % 64 != 0)) return hipErrorInvalidValue;
  const GemmPlan p = gemm_plan(g);
  if (p.kern == 4) return gemv_bf16(g, s);
  if (p.S > 1) return launch_splitk(g, p.S, p.Ks, p.kern >= 2, s);
  if (p.kern >= 2) {
    const int bm = p.kern == 3 ? 256 : 128;
    switch (g.e.kind) {
      case EPI_SWIGLU_IL: return launch_wide_bm<EPI_SWIGLU_IL>(g, bm, s);
      case EPI_F32: return launch_wide_bm<EPI_F32>(g, bm, s);
      case EPI_T: return launch_wide_bm<EPI_T>(g, bm, s);
      case EPI_ADD_F32: return launch_wide_bm<EPI_ADD_F32>(g, bm, s);
      case EPI_SGD: return launch_wide_bm<EPI_SGD>(g, bm, s);
      case EPI_SWIGLU_BWD: return launch_wide<128, EPI_SWIGLU_BWD, false>(g, 1, s);
      case EPI_QKV_ROPE: return launch_wide_bm<EPI_QKV_ROPE>(g, bm, s);
      case EPI_LM_CE: return launch_wide_bm<EPI_LM_CE>(g, bm, s);
      default: break;
    }
  }
  // (gemm_mfma_fuses_qkv_rope / gemm_mfma_fuses_lm_ce said no)
  if (g.e.kind == EPI_QKV_ROPE || g.e.kind == EPI_LM_CE) return hipErrorInvalidValue;
  if (p.kern == 1) {
    switch (g.e.kind) {
      case EPI_SWIGLU_IL: return launch_dl<EPI_SWIGLU_IL, false>(g, 1, s);
      case EPI_F32: return launch_dl<EPI_F32, false>(g, 1, s);
      case EPI_T: return launch_dl<EPI_T, false>(g, 1, s);
      // EPI_ADD_F32 stays on the register-staged loop: its two-phase epilogue needs many
      // registers and the lower occupancy costs more than the direct loads gain
      case EPI_SWIGLU_BWD: return launch_dl<EPI_SWIGLU_BWD, false>(g, 1, s);
      case EPI_SGD: return launch_dl<EPI_SGD, false>(g, 1, s);
      default: break;
    }
  }
  switch (g.e.kind) {
    case EPI_SWIGLU: return launch<128, 128, 64, 64, true, EPI_SWIGLU>(g, s);
    case EPI_SWIGLU_IL: return launch<128, 128, 64, 64, false, EPI_SWIGLU_IL>(g, s);
    case EPI_F32: return launch<128, 128, 64, 64, false, EPI_F32>(g, s);
    case EPI_T: return launch<128, 128, 64, 64, false, EPI_T>(g, s);
    case EPI_ADD_F32: return launch<128, 128, 64, 64, false, EPI_ADD_F32>(g, s);
    case EPI_SWIGLU_BWD: return launch<128, 128, 64, 64, false, EPI_SWIGLU_BWD>(g, s);
    case EPI_SGD: return launch<128, 128, 64, 64, false, EPI_SGD>(g, s);
    default: return hipErrorInvalidValue;
  }
}
