// Sliding-window attention on the CDNA4 matrix cores (bf16 in, fp32
// accumulate), flash-style with an online softmax over 64-key tiles of the
// key/value ring.  Window (page "TTT-E2E 如何让大模型边用边学", §4.2/§4.4): a
// query at absolute position t sees keys t-k < s <= t; key s lives in ring
// slot s mod R.
//
// Formulation per wave (32 queries): S^T = K Q^T (M = keys, N = queries,
// v_mfma_f32_32x32x16_bf16), so each lane owns one query and 16 keys of a
// 32-key tile; the softmax row statistics need one exchange with lane l^32.
// The probabilities then feed O^T += V^T P^T directly from registers: the
// MFMA's k index is permuted so that k-slot e of lane group g (= l/32) of
// the 16-key step h is key 16h + 8(e/4) + 4g + e%4, which is exactly the C
// register 8h + e of S^T.  V^T tiles come from the transposed value ring.
#include "kernels.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int KT = 64;   // keys per tile
constexpr int NW = 4;    // waves per block
constexpr int QW = 32;   // queries per wave
constexpr int BQ = NW * QW;

template <int HD>
struct FwdSmem {
  bf16 k[2][KT][HD + 8];   // K tile, row = key
  bf16 vt[2][HD][KT + 8];  // V^T tile, row = head dim
};

__device__ __forceinline__ uint32_t pk2(float a, float b) {
  return (uint32_t)f2bf(a).x | ((uint32_t)f2bf(b).x << 16);
}

template <int HD>
__global__ __launch_bounds__(256) void k_swa_fwd(AttnArgs a) {
  constexpr int KS = HD / 16;               // MFMA k-steps over the head dim
  constexpr int HM = HD / 32;               // 32-row tiles of the head dim
  constexpr int KCH = KT * HD / 8 / 256;    // 16-byte chunks of the K tile per thread
  constexpr int VCH = HD * KT / 8 / 256;    // same for the V^T tile
  static_assert(KCH <= 4 && VCH <= 4 && KT * HD % 2048 == 0, "tile staging covers HD <= 128");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  FwdSmem<HD>& sm = *reinterpret_cast<FwdSmem<HD>*>(smem_raw);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.z, h = blockIdx.y;
  const int64_t bh = (int64_t)b * a.H + h;
  const int R = a.R;
  const int t0 = blockIdx.x * BQ;               // first local query of the block
  const int tq = t0 + wid * QW + (lane & 31);   // this lane's query
  const bool qok = tq < a.n;
  const int64_t qpos = a.pos0 + tq;
  const int g = lane >> 5;

  const bf16* Kr = (const bf16*)a.kr + bh * R * HD;
  const bf16* Vt = (const bf16*)a.vtr + bh * HD * R;

  // Q fragments (B operand of S^T = K Q^T): query lane%32, head dims 16*ks + 8g .. +7.
  // Kept in named registers (an array here ends up in scratch memory).
  bf16x8 q0, q1, q2, q3, q4, q5, q6, q7;
  {
    const bf16* q = (const bf16*)a.q + (bh * a.n + (qok ? tq : 0)) * HD + g * 8;
    auto ldq = [&](int ks) {
      uint4 v = qok ? *(const uint4*)(q + ks * 16) : make_uint4(0, 0, 0, 0);
      return __builtin_bit_cast(bf16x8, v);
    };
    q0 = ldq(0);
    q1 = ldq(1);
    if constexpr (KS > 2) { q2 = ldq(2); q3 = ldq(3); }
    if constexpr (KS > 4) { q4 = ldq(4); q5 = ldq(5); }
    if constexpr (KS > 6) { q6 = ldq(6); q7 = ldq(7); }
  }

  // key range of the block: [max(0, first query - k + 1), last query], tiles aligned to 64 positions
  const int tlast = min(t0 + BQ, a.n) - 1;
  const int64_t kbeg = max((int64_t)0, a.pos0 + t0 - a.window + 1);
  const int64_t kend = a.pos0 + tlast;
  const int64_t ktile0 = (kbeg / KT) * KT;
  const int ntiles = (int)((kend - ktile0) / KT) + 1;

  // global -> register staging of the next tile (named registers: at most 4 + 4 chunks)
  uint4 rk0, rk1, rk2, rk3, rv0, rv1, rv2, rv3;
  const int sbase = (int)(ktile0 % R);  // ring slot of the first tile's first key
  // K tile: chunk c -> key row c / (HD/8), head dims (c % (HD/8)) * 8 .. +7
  // V^T tile: chunk c -> head-dim row c / 8, keys (c % 8) * 8 .. +7 (contiguous: 64-aligned
  // tiles and R % 8 == 0 keep every 8-key group inside the ring)
#define LOADK(i, dst)                                                              \
  if constexpr (KCH > i) {                                                         \
    const int c = tid + i * 256, r = c / (HD / 8), col = (c % (HD / 8)) * 8;       \
    dst = *(const uint4*)(Kr + (int64_t)((slot0 + r) % R) * HD + col);            \
  }
#define LOADV(i, dst)                                                              \
  if constexpr (VCH > i) {                                                         \
    const int c = tid + i * 256, r = c / (KT / 8), col = (c % (KT / 8)) * 8;       \
    dst = *(const uint4*)(Vt + (int64_t)r * R + (slot0 + col) % R);               \
  }
#define LOAD_TILE(it_)                                                             \
  {                                                                                \
    const int slot0 = (sbase + (it_) * KT) % R;                                    \
    LOADK(0, rk0) LOADK(1, rk1) LOADK(2, rk2) LOADK(3, rk3)                        \
    LOADV(0, rv0) LOADV(1, rv1) LOADV(2, rv2) LOADV(3, rv3)                        \
  }
#define STK(i, src)                                                                \
  if constexpr (KCH > i) {                                                         \
    const int c = tid + i * 256, r = c / (HD / 8), col = (c % (HD / 8)) * 8;       \
    *(uint4*)&sm.k[buf][r][col] = src;                                             \
  }
#define STV(i, src)                                                                \
  if constexpr (VCH > i) {                                                         \
    const int c = tid + i * 256, r = c / (KT / 8), col = (c % (KT / 8)) * 8;       \
    *(uint4*)&sm.vt[buf][r][col] = src;                                            \
  }
#define STORE_TILE(buf_)                                                           \
  {                                                                                \
    const int buf = (buf_);                                                        \
    STK(0, rk0) STK(1, rk1) STK(2, rk2) STK(3, rk3)                                \
    STV(0, rv0) STV(1, rv1) STV(2, rv2) STV(3, rv3)                                \
  }

  f32x16 o[HM];
#pragma unroll
  for (int i = 0; i < HM; ++i) o[i] = f32x16{};
  float mrun = -INFINITY, lrun = 0.f;
  const float sl2 = 1.4426950408889634f / sqrtf((float)HD);  // log2(e) / sqrt(hd)

  LOAD_TILE(0)
  STORE_TILE(0)
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    if (it + 1 < ntiles) LOAD_TILE(it + 1)
    const int64_t kp0 = ktile0 + (int64_t)it * KT;
    // S^T for the two 32-key halves of the tile
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    {
      const bf16* k0p = &sm.k[cur][(lane & 31)][g * 8];
      const bf16* k1p = &sm.k[cur][32 + (lane & 31)][g * 8];
#define SSTEP(ks, qv)                                                         \
  if constexpr (KS > ks) {                                                    \
    bf16x8 k0 = *(const bf16x8*)(k0p + ks * 16);                              \
    bf16x8 k1 = *(const bf16x8*)(k1p + ks * 16);                              \
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qv, s0, 0, 0, 0);       \
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qv, s1, 0, 0, 0);       \
  }
      SSTEP(0, q0) SSTEP(1, q1) SSTEP(2, q2) SSTEP(3, q3) SSTEP(4, q4) SSTEP(5, q5) SSTEP(6, q6) SSTEP(7, q7)
#undef SSTEP
    }
    // mask + scale; register 4j+i of half mt holds key kp0 + 32 mt + 8 j + 4 g + i.
    // Visible: qpos - window < key <= qpos, i.e. lo < off <= hi with off = key - kp0.
    const int64_t hi64 = qpos - kp0, lo64 = qpos - a.window - kp0;
    const int hi = qok ? (int)min<int64_t>(max<int64_t>(hi64, -1), 64) : -1;
    const int lo = (int)min<int64_t>(max<int64_t>(lo64, -2), 64);
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = 8 * (r >> 2) + 4 * g + (r & 3);
      float v0 = (off <= hi && off > lo) ? s0[r] * sl2 : -INFINITY;
      float v1 = (off + 32 <= hi && off + 32 > lo) ? s1[r] * sl2 : -INFINITY;
      s0[r] = v0;
      s1[r] = v1;
      tmax = fmaxf(tmax, fmaxf(v0, v1));
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mnew = fmaxf(mrun, tmax);
    const float msafe = mnew == -INFINITY ? 0.f : mnew;
    const float corr = exp2f(mrun - msafe);
    float psum = 0.f;
    uint32_t pa[8], pb[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float p0 = exp2f(s0[r] - msafe), p1 = exp2f(s0[r + 1] - msafe);
      float q0 = exp2f(s1[r] - msafe), q1 = exp2f(s1[r + 1] - msafe);
      psum += (p0 + p1) + (q0 + q1);
      pa[r >> 1] = pk2(p0, p1);
      pb[r >> 1] = pk2(q0, q1);
    }
    psum += __shfl_xor(psum, 32, 64);
    lrun = lrun * corr + psum;
    mrun = mnew;
#pragma unroll
    for (int i = 0; i < HM; ++i) o[i] *= corr;
    // O^T += V^T P^T, four 16-key steps (keys 0-15, 16-31 of each half)
    const bf16x8 pf[4] = {__builtin_bit_cast(bf16x8, make_uint4(pa[0], pa[1], pa[2], pa[3])),
                          __builtin_bit_cast(bf16x8, make_uint4(pa[4], pa[5], pa[6], pa[7])),
                          __builtin_bit_cast(bf16x8, make_uint4(pb[0], pb[1], pb[2], pb[3])),
                          __builtin_bit_cast(bf16x8, make_uint4(pb[4], pb[5], pb[6], pb[7]))};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kc = st * 16 + 4 * g;
#pragma unroll
      for (int hm = 0; hm < HM; ++hm) {
        const bf16* vrow = &sm.vt[cur][hm * 32 + (lane & 31)][0];
        uint2 lo2 = *(const uint2*)(vrow + kc);
        uint2 hi2 = *(const uint2*)(vrow + kc + 8);
        bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
        o[hm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[st], o[hm], 0, 0, 0);
      }
    }
    if (it + 1 < ntiles) STORE_TILE(cur ^ 1)
    __syncthreads();
  }

#undef LOADK
#undef LOADV
#undef LOAD_TILE
#undef STK
#undef STV
#undef STORE_TILE
  if (!qok) return;
  const float inv = 1.f / lrun;
  bf16* out = (bf16*)a.o + ((int64_t)b * a.n + tq) * ((int64_t)a.H * HD) + (int64_t)h * HD;
#pragma unroll
  for (int hm = 0; hm < HM; ++hm)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = hm * 32 + 8 * j + 4 * g;
      uint2 w = make_uint2(pk2(o[hm][4 * j] * inv, o[hm][4 * j + 1] * inv),
                           pk2(o[hm][4 * j + 2] * inv, o[hm][4 * j + 3] * inv));
      *(uint2*)(out + d0) = w;
    }
  if (a.lse && g == 0) a.lse[bh * a.n + tq] = (mrun + log2f(lrun)) * 0.6931471805599453f;
}

template <int HD>
hipError_t launch_fwd(const AttnArgs& a, hipStream_t s) {
  auto kern = k_swa_fwd<HD>;
  size_t shm = sizeof(FwdSmem<HD>);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    attr = true;
  }
  dim3 grid(cdiv(a.n, BQ), a.H, a.B);
  hipLaunchKernelGGL(kern, grid, dim3(256), shm, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t swa_fwd_mfma(const AttnArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  // 64-key tiles read 8-key groups of the transposed value ring: R % 8 == 0
  if (a.R % 8 != 0) return swa_fwd_simt<bf16>(a, s);
  switch (a.hd) {
    case 32: return launch_fwd<32>(a, s);
    case 64: return launch_fwd<64>(a, s);
    case 96: return launch_fwd<96>(a, s);
    case 128: return launch_fwd<128>(a, s);
    default: return swa_fwd_simt<bf16>(a, s);
  }
}

hipError_t swa_bwd_mfma(const AttnBwdArgs& a, hipStream_t s) { return swa_bwd_simt<bf16>(a, s); }
