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
#include <algorithm>

#include "kernels.h"

hipError_t swa_dvec_bf16(const AttnBwdArgs& a, hipStream_t s);

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
  // V^T tile, row = head dim (ring of 3: read one and two tiles late).  Rows are 34 dwords
  // apart: the 8-byte fragment reads of 32 lanes (32 consecutive rows, one column) then fall
  // on 32 distinct bank pairs (17 r mod 32 is a permutation), where a 36-dword stride repeats
  // every 16 rows and conflicts two ways.
  bf16 vt[3][HD][KT + 4];
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk2(float a, float b) { return bf16pair(a, b); }

// 2^x with one v_exp_f32 (results below 2^-126 flush to zero, which no probability here
// resolves anyway); exp2f adds a denormal-range fix-up of five more instructions
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// ring slot s0 + r for a slot s0 < R and an offset 0 <= r < R, without a division
__device__ __forceinline__ int ring_add(int s0, int r, int R) {
  const int s = s0 + r;
  return s >= R ? s - R : s;
}

// SPLIT: blockIdx.z = b * S + split; the block covers only its share of the key tiles
// and writes unnormalized O, the reference max (raw score units) and the exp-sum to the
// workspace: O [S][B][H][n][hd], m [S][B][H][n], l [S][B][H][n].
template <int HD, int NW, bool SPLIT = false>
__global__ __launch_bounds__(NW * 64) void k_swa_fwd(AttnArgs a, int S) {
  constexpr int NT = NW * 64;  // threads per block
  constexpr int BQ = NW * QW;  // queries per block
  constexpr int KS = HD / 16;               // MFMA k-steps over the head dim
  constexpr int HM = HD / 32;               // 32-row tiles of the head dim
  constexpr int KCH = (KT * HD / 8 + NT - 1) / NT;  // 16-byte chunks of the K tile per thread
  constexpr int VCH = (HD * KT / 8 + NT - 1) / NT;  // same for the V^T tile
  static_assert(KCH <= 4 && VCH <= 4, "tile staging covers HD <= 128");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  FwdSmem<HD>& sm = *reinterpret_cast<FwdSmem<HD>*>(smem_raw);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = SPLIT ? blockIdx.z / S : blockIdx.z, h = blockIdx.y;
  const int sp = SPLIT ? blockIdx.z % S : 0;
  const int64_t bh = (int64_t)b * a.H + h;
  const int R = a.R;
  const int t0 = blockIdx.x * BQ;               // first local query of the block
  const int tq = t0 + wid * QW + (lane & 31);   // this lane's query
  const bool qok = tq < a.n;
  const int64_t qpos = a.pos0 + tq;
  const int g = lane >> 5;
  const int tw0 = t0 + wid * QW;                  // first query of this wave
  const bool wfull = tw0 + QW <= a.n;             // all 32 queries of the wave exist
  const int64_t wpos_lo = a.pos0 + tw0, wpos_hi = wpos_lo + QW - 1;

  const bf16* Kr = (const bf16*)a.kr + bh * R * HD;
  const bf16* Vt = (const bf16*)a.vtr + bh * HD * R;

  // Q fragments (B operand of S^T = K Q^T): query lane%32, head dims 16*ks + 8g .. +7,
  // pre-multiplied by log2(e)/sqrt(hd) (rounded to bf16) so that S^T comes out in log2
  // units.  Kept in named registers (an array here ends up in scratch memory).
  const float sl2 = 1.4426950408889634f / sqrtf((float)HD);  // log2(e) / sqrt(hd)
  bf16x8 q0, q1, q2, q3, q4, q5, q6, q7;
  {
    const bf16* q = (const bf16*)a.q + (bh * a.n + (qok ? tq : 0)) * HD + g * 8;
    auto ldq = [&](int ks) {
      uint4 v = qok ? *(const uint4*)(q + ks * 16) : make_uint4(0, 0, 0, 0);
      bf16x8 x = __builtin_bit_cast(bf16x8, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (__bf16)((float)x[e] * sl2);
      return x;
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
  const int ntiles_all = (int)((kend - ktile0) / KT) + 1;
  const int per = SPLIT ? (ntiles_all + S - 1) / S : ntiles_all;
  const int it_beg = SPLIT ? min(ntiles_all, sp * per) : 0;
  const int ntiles = SPLIT ? min(ntiles_all, it_beg + per) : ntiles_all;  // loop end

  // global -> register staging of the next tile (named registers: at most 4 + 4 chunks)
  uint4 rk0, rk1, rk2, rk3, rv0, rv1, rv2, rv3;
  const int sbase = (int)(ktile0 % R);  // ring slot of the first tile's first key
  // K tile: chunk c -> key row c / (HD/8), head dims (c % (HD/8)) * 8 .. +7
  // V^T tile: chunk c -> head-dim row c / 8, keys (c % 8) * 8 .. +7 (contiguous: 64-aligned
  // tiles and R % 8 == 0 keep every 8-key group inside the ring)
#define LOADK(i, dst)                                                              \
  if constexpr (KCH > i) {                                                         \
    const int c = tid + i * NT, r = c / (HD / 8), col = (c % (HD / 8)) * 8;        \
    if (c < KT * HD / 8) dst = *(const uint4*)(Kr + (int64_t)ring_add(slot0, r, R) * HD + col); \
  }
#define LOADV(i, dst)                                                              \
  if constexpr (VCH > i) {                                                         \
    const int c = tid + i * NT, r = c / (KT / 8), col = (c % (KT / 8)) * 8;        \
    if (c < KT * HD / 8) dst = *(const uint4*)(Vt + (int64_t)r * R + ring_add(slot0, col, R)); \
  }
#define LOAD_TILE(it_)                                                             \
  {                                                                                \
    const int slot0 = (sbase + (it_) * KT) % R;                                    \
    LOADK(0, rk0) LOADK(1, rk1) LOADK(2, rk2) LOADK(3, rk3)                        \
    LOADV(0, rv0) LOADV(1, rv1) LOADV(2, rv2) LOADV(3, rv3)                        \
  }
#define STK(i, src)                                                                \
  if constexpr (KCH > i) {                                                         \
    const int c = tid + i * NT, r = c / (HD / 8), col = (c % (HD / 8)) * 8;        \
    if (c < KT * HD / 8) *(uint4*)&sm.k[buf][r][col] = src;                        \
  }
#define STV(i, src)                                                                \
  if constexpr (VCH > i) {                                                         \
    const int c = tid + i * NT, r = c / (KT / 8), col = (c % (KT / 8)) * 8;        \
    if (c < KT * HD / 8) { /* rows are 8-byte aligned only */                      \
      uint2* d = (uint2*)&sm.vt[vbuf][r][col];                                     \
      d[0] = make_uint2(src.x, src.y);                                             \
      d[1] = make_uint2(src.z, src.w);                                             \
    }                                                                              \
  }
#define STORE_TILE(buf_, vbuf_)                                                    \
  {                                                                                \
    const int buf = (buf_), vbuf = (vbuf_);                                        \
    STK(0, rk0) STK(1, rk1) STK(2, rk2) STK(3, rk3)                                \
    STV(0, rv0) STV(1, rv1) STV(2, rv2) STV(3, rv3)                                \
  }

  f32x16 o[HM];
#pragma unroll
  for (int i = 0; i < HM; ++i) o[i] = f32x16{};
  float mref = -INFINITY, lrun = 0.f;  // reference max (log2 units), this lane's row sum
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

  // Two wave groups in counter-phase.  The waves of a block move in lockstep between the
  // per-tile barriers, and the two waves that share a SIMD (w and w + NW/2) are in different
  // groups: group A runs S^T, softmax, PV for tile it; group B runs PV for tile it-1 (its
  // probabilities kept in registers), then S^T and softmax for tile it.  So while one wave of
  // a SIMD works through its softmax on the vector ALUs, the other issues MFMAs.  V^T tiles
  // live in a ring of 3 (group B reads them one iteration late).
  const bool late = wid >= NW / 2;
  if (it_beg < ntiles) {
    LOAD_TILE(it_beg)
    STORE_TILE(it_beg & 1, it_beg % 3)
  }
  __syncthreads();
#define PV(vb, PA_, PB_)                                                                             \
  {                                                                                              \
    const bf16x8 pf0 = __builtin_bit_cast(bf16x8, make_uint4(PA_[0], PA_[1], PA_[2], PA_[3]));           \
    const bf16x8 pf1 = __builtin_bit_cast(bf16x8, make_uint4(PA_[4], PA_[5], PA_[6], PA_[7]));           \
    const bf16x8 pf2 = __builtin_bit_cast(bf16x8, make_uint4(PB_[0], PB_[1], PB_[2], PB_[3]));           \
    const bf16x8 pf3 = __builtin_bit_cast(bf16x8, make_uint4(PB_[4], PB_[5], PB_[6], PB_[7]));           \
    _Pragma("unroll") for (int st = 0; st < 4; ++st) {                                           \
      const int kc = st * 16 + 4 * g;                                                            \
      const bf16x8 pf = st == 0 ? pf0 : st == 1 ? pf1 : st == 2 ? pf2 : pf3;                     \
      _Pragma("unroll") for (int hm = 0; hm < HM; ++hm) {                                        \
        const bf16* vrow = &sm.vt[vb][hm * 32 + (lane & 31)][0];                                 \
        uint2 lo2 = *(const uint2*)(vrow + kc);                                                  \
        uint2 hi2 = *(const uint2*)(vrow + kc + 8);                                              \
        bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));          \
        o[hm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[hm], 0, 0, 0);                 \
      }                                                                                          \
    }                                                                                            \
  }
#define SSTEP(ks, qv)                                                         \
  if constexpr (KS > ks) {                                                    \
    bf16x8 k0 = *(const bf16x8*)(k0p + ks * 16);                              \
    bf16x8 k1 = *(const bf16x8*)(k1p + ks * 16);                              \
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qv, s0, 0, 0, 0);       \
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qv, s1, 0, 0, 0);       \
  }
#define EXP_TILE(PA, PB) \
_Pragma("unroll") \
    for (int r = 0; r < 16; r += 2) { \
      PA[r >> 1] = pk2(ex2(s0[r]), ex2(s0[r + 1])); \
      PB[r >> 1] = pk2(ex2(s1[r]), ex2(s1[r + 1])); \
      psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, PA[r >> 1]), ones, psum, false); \
      psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, PB[r >> 1]), ones, psum, false); \
    }
#define FWD_TILE(it, PA, PB, QA, QB) \
  { \
    const int cur = it & 1; \
    if (it + 1 < ntiles) LOAD_TILE(it + 1) \
    const int64_t kp0 = ktile0 + (int64_t)it * KT; \
    if (late && it > it_beg) PV((it - 1) % 3, QA, QB) \
    /* S^T - reference for the two 32-key halves of the tile: the accumulators start at */ \
    /* minus this lane's (this query's) reference, so the exponent needs no extra operation */ \
    const float nb0 = mref == -INFINITY ? 0.f : -mref; \
    f32x16 s0, s1; \
_Pragma("unroll") \
    for (int r = 0; r < 16; ++r) { \
      s0[r] = nb0; \
      s1[r] = nb0; \
    } \
    { \
      const bf16* k0p = &sm.k[cur][(lane & 31)][g * 8]; \
      const bf16* k1p = &sm.k[cur][32 + (lane & 31)][g * 8]; \
      SSTEP(0, q0) SSTEP(1, q1) SSTEP(2, q2) SSTEP(3, q3) SSTEP(4, q4) SSTEP(5, q5) SSTEP(6, q6) SSTEP(7, q7) \
    } \
    /* register 4j+i of half mt holds key kp0 + 32 mt + 8 j + 4 g + i.  Visible keys: */ \
    /* qpos - window < key <= qpos.  Only tiles that cut a window edge for some query of */ \
    /* this wave (or waves with out-of-range queries) need the per-element mask. */ \
    const bool full = wfull && kp0 >= wpos_hi - a.window + 1 && kp0 + KT - 1 <= wpos_lo; \
    if (!full) { \
      const int64_t hi64 = qpos - kp0, lo64 = qpos - a.window - kp0; \
      const int hi = !qok ? -1 : hi64 < -1 ? -1 : hi64 > 64 ? 64 : (int)hi64; \
      const int lo = lo64 < -2 ? -2 : lo64 > 64 ? 64 : (int)lo64; \
_Pragma("unroll") \
      for (int r = 0; r < 16; ++r) { \
        const int off = 8 * (r >> 2) + 4 * g + (r & 3); \
        if (!(off <= hi && off > lo)) s0[r] = -INFINITY; \
        if (!(off + 32 <= hi && off + 32 > lo)) s1[r] = -INFINITY; \
      } \
    } \
    /* probabilities against the current reference, and their row sums: dot products of the */ \
    /* bf16 values that feed the PV product, per lane (the pair's sums are added at the end) */ \
    float psum = 0.f; \
    EXP_TILE(PA, PB) \
    /* lazy reference max (log2 units): it stays while every lane's sum of the tile's */ \
    /* probabilities is at most 2^12 (so each is), which needs no maximum over the tile; */ \
    /* otherwise (and on the first tile, with no reference yet) the tile's maximum moves it */ \
    /* when it passes the reference by more than 8, O is rescaled and the probabilities */ \
    /* are redone.  The result does not depend on the reference; the pair of lanes of a */ \
    /* query shares it. */ \
    float corr = 1.f; \
    if (__any(!(psum <= 4096.f) || mref == -INFINITY)) { \
      float tmax = -INFINITY; \
_Pragma("unroll") \
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, fmaxf(s0[r], s1[r])); \
      /* what the accumulators had subtracted */ \
      const float base = mref == -INFINITY ? 0.f : mref; \
      const float pmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) + base; \
      const float mnew = (mref == -INFINITY || pmax > mref + 8.f) ? pmax : mref; \
      corr = mnew == mref ? 1.f : exp2f(mref - mnew); \
      mref = mnew; \
      const float shift = mnew == -INFINITY ? 0.f : base - mnew; \
_Pragma("unroll") \
      for (int r = 0; r < 16; ++r) { \
        s0[r] += shift; \
        s1[r] += shift; \
      } \
_Pragma("unroll") \
      for (int i = 0; i < HM; ++i) o[i] *= corr; \
      psum = 0.f; \
      EXP_TILE(PA, PB) \
    } \
    lrun = lrun * corr + psum; \
    if (!late) PV(it % 3, PA, PB) \
    if (it + 1 < ntiles) STORE_TILE(cur ^ 1, (it + 1) % 3) \
    __syncthreads(); \
  }
  // P of a tile in (pa, pb) or (qa, qb), alternating, so that group B keeps the previous
  // tile's probabilities without copying them
  uint32_t pa[8], pb[8], qa[8], qb[8];
  for (int it2 = it_beg; it2 < ntiles; it2 += 2) {
    {
      const int it = it2;
      FWD_TILE(it, pa, pb, qa, qb)
    }
    if (it2 + 1 < ntiles) {
      const int it = it2 + 1;
      FWD_TILE(it, qa, qb, pa, pb)
    }
  }
#undef FWD_TILE
#undef EXP_TILE
#undef SSTEP
  if (late && it_beg < ntiles) {
    if ((ntiles - it_beg) & 1)
      PV((ntiles - 1) % 3, pa, pb)
    else
      PV((ntiles - 1) % 3, qa, qb)
  }
#undef PV

#undef LOADK
#undef LOADV
#undef LOAD_TILE
#undef STK
#undef STV
#undef STORE_TILE
  lrun += __shfl_xor(lrun, 32, 64);
  // The block's output rows leave through LDS as whole rows (queries past the chunk end are not
  // written): every wave is done with the K and V^T tiles first.
  __syncthreads();
  const int qr = wid * QW + (lane & 31);  // the lane's query row in the block
  if constexpr (SPLIT) {
    // fp32 part [S][B][H][n][HD] of this key range (the block's rows are consecutive), half the
    // block's queries at a time; the reference and the row sum per query beside it
    constexpr int SLD = HD + 4, HQ = BQ / 2;
    static_assert(HQ * SLD * 4 <= sizeof(FwdSmem<HD>), "staged part rows fit");
    float* st = reinterpret_cast<float*>(smem_raw);
    const int64_t row0 = ((int64_t)sp * a.B * a.H + bh) * a.n + t0;
    float* pm = a.ws + (int64_t)S * a.B * a.H * a.n * HD;
    float* pl = pm + (int64_t)S * a.B * a.H * a.n;
    if (qok && g == 0) {
      pm[row0 + qr] = mref == -INFINITY ? -INFINITY : mref / sl2;  // raw score units
      pl[row0 + qr] = lrun;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half > 0) __syncthreads();  // the first half's rows have left LDS
      if (qr / HQ == half) {
#pragma unroll
        for (int hm = 0; hm < HM; ++hm)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d0 = hm * 32 + 8 * j + 4 * g;
            *(float4*)(st + (qr - half * HQ) * SLD + d0) = make_float4(o[hm][4 * j], o[hm][4 * j + 1], o[hm][4 * j + 2], o[hm][4 * j + 3]);
          }
      }
      __syncthreads();
      float* po = a.ws + (row0 + half * HQ) * HD;
      for (int c = tid; c < HQ * (HD / 4); c += NT) {
        const int r = c / (HD / 4), c4 = (c % (HD / 4)) * 4;
        if (t0 + half * HQ + r < a.n) *(float4*)(po + (int64_t)r * HD + c4) = *(const float4*)(st + r * SLD + c4);
      }
    }
    return;
  }
  // bf16 rows of O [B n][H HD] (head h's HD columns), all BQ queries at once
  constexpr int OLD = HD + 8;
  static_assert(BQ * OLD * 2 <= sizeof(FwdSmem<HD>), "staged output rows fit");
  bf16* so = reinterpret_cast<bf16*>(smem_raw);
  const float inv = 1.f / lrun;
#pragma unroll
  for (int hm = 0; hm < HM; ++hm)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = hm * 32 + 8 * j + 4 * g;
      *(uint2*)(so + qr * OLD + d0) = make_uint2(pk2(o[hm][4 * j] * inv, o[hm][4 * j + 1] * inv),
                                                 pk2(o[hm][4 * j + 2] * inv, o[hm][4 * j + 3] * inv));
    }
  if (a.lse && qok && g == 0) a.lse[bh * a.n + tq] = (mref + log2f(lrun)) * 0.6931471805599453f;
  __syncthreads();
  bf16* ob = (bf16*)a.o + ((int64_t)b * a.n + t0) * ((int64_t)a.H * HD) + (int64_t)h * HD;
  for (int c = tid; c < BQ * (HD / 8); c += NT) {
    const int r = c / (HD / 8), c8 = (c % (HD / 8)) * 8;
    if (t0 + r < a.n) *(uint4*)(ob + (int64_t)r * (a.H * HD) + c8) = *(const uint4*)(so + r * OLD + c8);
  }
}

// merge the key-range parts of a split forward: O = sum_s w_s O_s / sum_s w_s l_s with
// w_s = 2^((m_s - max m) * sl2); grid (n, H, B), one thread per head dim
__global__ __launch_bounds__(256) void k_swa_combine(AttnArgs a, int S) {
  // one wave per (query, head); lane l covers head dims 2l, 2l+1
  const int64_t plane = (int64_t)a.B * a.H * a.n;
  const int64_t qh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b*H + h)*n + t
  if (qh >= plane) return;
  const int lane = threadIdx.x & 63, hd = a.hd;
  const int64_t bh = qh / a.n;
  const int t = (int)(qh % a.n), h = (int)(bh % a.H), b = (int)(bh / a.H);
  const float* pm = a.ws + (int64_t)S * plane * hd;
  const float* pl = pm + (int64_t)S * plane;
  const float sl2 = 1.4426950408889634f / sqrtf((float)hd);
  float M = -INFINITY;
  float L = 0.f;
  float2 acc = make_float2(0.f, 0.f);
  const bool act = 2 * lane < hd;
  constexpr int SMAX = 8;  // (the split takes at most 8 parts): every load of the row in one round
  if (S <= SMAX) {
    float pmv[SMAX], plv[SMAX];
    float2 vv[SMAX];
#pragma unroll
    for (int sidx = 0; sidx < SMAX; ++sidx) {
      pmv[sidx] = -INFINITY;
      plv[sidx] = 0.f;
      vv[sidx] = make_float2(0.f, 0.f);
      if (sidx < S) {
        const int64_t row = sidx * plane + qh;
        pmv[sidx] = pm[row];
        plv[sidx] = pl[row];
        if (act) vv[sidx] = *(const float2*)(a.ws + row * hd + 2 * lane);
      }
    }
#pragma unroll
    for (int sidx = 0; sidx < SMAX; ++sidx) M = fmaxf(M, pmv[sidx]);
#pragma unroll
    for (int sidx = 0; sidx < SMAX; ++sidx) {
      const float w = pmv[sidx] == -INFINITY ? 0.f : exp2f((pmv[sidx] - M) * sl2);
      L += w * plv[sidx];
      acc.x += w * vv[sidx].x;
      acc.y += w * vv[sidx].y;
    }
  } else {
    for (int sidx = 0; sidx < S; ++sidx) M = fmaxf(M, pm[sidx * plane + qh]);
    for (int sidx = 0; sidx < S; ++sidx) {
      const int64_t row = sidx * plane + qh;
      const float w = pm[row] == -INFINITY ? 0.f : exp2f((pm[row] - M) * sl2);
      L += w * pl[row];
      if (act) {
        const float2 v = *(const float2*)(a.ws + row * hd + 2 * lane);
        acc.x += w * v.x;
        acc.y += w * v.y;
      }
    }
  }
  if (act) {
    const uint32_t pkd = (uint32_t)f2bf(acc.x / L).x | ((uint32_t)f2bf(acc.y / L).x << 16);
    *(uint32_t*)((bf16*)a.o + ((int64_t)b * a.n + t) * ((int64_t)a.H * hd) + (int64_t)h * hd + 2 * lane) = pkd;
  }
  if (a.lse && lane == 0) a.lse[qh] = M * (sl2 * 0.6931471805599453f) + logf(L);
}

template <int HD, int NW, bool SPLIT>
hipError_t launch_fwd_nw(const AttnArgs& a, int S, hipStream_t s) {
  auto kern = k_swa_fwd<HD, NW, SPLIT>;
  size_t shm = sizeof(FwdSmem<HD>);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    attr = true;
  }
  dim3 grid(cdiv(a.n, NW * QW), a.H, a.B * S);
  hipLaunchKernelGGL(kern, grid, dim3(NW * 64), shm, s, a, S);
  if (SPLIT) hipLaunchKernelGGL(k_swa_combine, dim3(cdiv((int64_t)a.B * a.H * a.n, 4)), dim3(256), 0, s, a, S);
  return hipGetLastError();
}

// parts of a split that give about one round of blocks on the 256 CUs (one 8-wave block per
// CU): floor(256 / blocks), at most 8, at least 8 key tiles per part, within the workspace
int attn_splits(int64_t blocks, int64_t ntiles, int64_t need_per_split, const float* ws, int64_t ws_floats) {
  if (!ws || blocks >= 128) return 1;
  int S = (int)std::min<int64_t>(8, 256 / blocks);
  S = (int)std::min<int64_t>(S, std::max<int64_t>(1, ntiles / 8));
  while (S > 1 && S * need_per_split > ws_floats) --S;
  return std::max(S, 1);
}

// key-range parts of the forward
int fwd_splits(const AttnArgs& a) {
  const int64_t blocks = (int64_t)cdiv(a.n, 8 * QW) * a.H * a.B;
  const int64_t ntiles = (std::min<int64_t>(a.window, a.pos0 + 1) + 8 * QW) / KT + 1;
  const int64_t need = (int64_t)a.B * a.H * a.n * (a.hd + 2);
  static int force_s = -1;  // TTT_FWD_SPLITS (tuning switch): key-range parts of a small-grid forward
  if (force_s < 0) {
    const char* ev = getenv("TTT_FWD_SPLITS");
    force_s = ev ? std::max(0, atoi(ev)) : 0;
  }
  if (force_s > 0 && a.ws && blocks < 128 && force_s * need <= a.ws_floats) return force_s;
  return attn_splits(blocks, ntiles, need, a.ws, a.ws_floats);
}

template <int HD>
hipError_t launch_fwd(const AttnArgs& a, hipStream_t s) {
  const int S = fwd_splits(a);
  if (S > 1) return launch_fwd_nw<HD, 8, true>(a, S, s);
  return launch_fwd_nw<HD, 8, false>(a, 1, s);
}


// ---------------------------------------------------------------- backward
//
// dQ kernel: per wave 32 queries, loop over the 64-key tiles of the window
// (cached keys included, as constants).  S^T = K Q^T and dP^T = V dO^T put
// one query per lane; dS^T = P^T (dP^T - D) then feeds dQ^T += K^T dS^T from
// registers with the same permuted k index as the forward's P V product.
// TR: K^T tiles are 16-byte copies from the transposed key ring; otherwise
// K^T is produced in LDS by a transposing store of the K tile.
template <int HD>
struct DqSmem {
  bf16 k[2][KT][HD + 8];
  bf16 v[2][KT][HD + 8];
  bf16 kt[2][HD][KT + 8];
};

// SPLIT: blockIdx.z = b * S + split over the key tiles; partial dq to ws[S][B*n][H*hd]
template <int HD, int NW, bool SPLIT, bool TR>
__global__ __launch_bounds__(NW * 64) void k_swa_dq(AttnBwdArgs a, int S) {
  constexpr int NT = NW * 64, BQn = NW * QW;
  constexpr int KS = HD / 16, HM = HD / 32;
  constexpr int KCH = (KT * HD / 8 + NT - 1) / NT;
  static_assert(KCH <= 4, "tile staging covers HD <= 128");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  DqSmem<HD>& sm = *reinterpret_cast<DqSmem<HD>*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 5;
  const int b = SPLIT ? blockIdx.z / S : blockIdx.z, h = blockIdx.y;
  const int sp = SPLIT ? blockIdx.z % S : 0;
  const int64_t bh = (int64_t)b * a.H + h;
  const int R = a.R, d = a.H * HD;
  const int t0 = blockIdx.x * BQn;
  const int tq = t0 + wid * QW + (lane & 31);
  const bool qok = tq < a.n;
  const int64_t qpos = a.pos0 + tq;
  const int tw0 = t0 + wid * QW;
  const bool wfull = tw0 + QW <= a.n;
  const int64_t wpos_lo = a.pos0 + tw0, wpos_hi = wpos_lo + QW - 1;
  const bf16* Kr = (const bf16*)a.kr + bh * R * HD;
  const bf16* Vr = (const bf16*)a.vr + bh * R * HD;
  const bf16* Kt = TR ? (const bf16*)a.ktr + bh * HD * R : nullptr;

  bf16x8 q0, q1, q2, q3, q4, q5, q6, q7, e0, e1, e2, e3, e4, e5, e6, e7;
  {
    const bf16* q = (const bf16*)a.q + (bh * a.n + (qok ? tq : 0)) * HD + g * 8;
    const bf16* dO = (const bf16*)a.dout + ((int64_t)b * a.n + (qok ? tq : 0)) * d + (int64_t)h * HD + g * 8;
    auto ld8 = [&](const bf16* p, int ks) {
      uint4 v = qok ? *(const uint4*)(p + ks * 16) : make_uint4(0, 0, 0, 0);
      return __builtin_bit_cast(bf16x8, v);
    };
    q0 = ld8(q, 0); q1 = ld8(q, 1); e0 = ld8(dO, 0); e1 = ld8(dO, 1);
    if constexpr (KS > 2) { q2 = ld8(q, 2); q3 = ld8(q, 3); e2 = ld8(dO, 2); e3 = ld8(dO, 3); }
    if constexpr (KS > 4) { q4 = ld8(q, 4); q5 = ld8(q, 5); e4 = ld8(dO, 4); e5 = ld8(dO, 5); }
    if constexpr (KS > 6) { q6 = ld8(q, 6); q7 = ld8(q, 7); e6 = ld8(dO, 6); e7 = ld8(dO, 7); }
  }
  const float LOG2E = 1.4426950408889634f;
  const float sl2 = LOG2E / sqrtf((float)HD);
  const float nlse2 = qok ? -a.lse[bh * a.n + tq] * LOG2E : 0.f;
  const float Dq = qok ? a.dvec[bh * a.n + tq] : 0.f;

  const int tlast = min(t0 + BQn, a.n) - 1;
  const int64_t kbeg = max((int64_t)0, a.pos0 + t0 - a.window + 1);
  const int64_t kend = a.pos0 + tlast;
  const int64_t ktile0 = (kbeg / KT) * KT;
  const int ntiles_all = (int)((kend - ktile0) / KT) + 1;
  const int per = SPLIT ? (ntiles_all + S - 1) / S : ntiles_all;
  const int it_beg = SPLIT ? min(ntiles_all, sp * per) : 0;
  const int ntiles = SPLIT ? min(ntiles_all, it_beg + per) : ntiles_all;
  const int sbase = (int)(ktile0 % R);

  f32x16 acc[HM];
#pragma unroll
  for (int i = 0; i < HM; ++i) acc[i] = f32x16{};

  uint4 rk0, rk1, rk2, rk3, rv0, rv1, rv2, rv3, rt0, rt1, rt2, rt3;
  // K^T chunk c (TR): head-dim row c / 8, keys (c % 8) * 8 .. +7 -- contiguous, since
  // tiles start at multiples of 64 positions and R % 8 == 0
#define LD(i, dk, dv, dt)                                                                \
  if constexpr (KCH > i) {                                                               \
    const int c = tid + i * NT, r = c / (HD / 8), col = (c % (HD / 8)) * 8;              \
    if (c < KT * HD / 8) {                                                               \
      const int64_t off = (int64_t)ring_add(slot0, r, R) * HD + col;                         \
      dk = *(const uint4*)(Kr + off);                                                    \
      dv = *(const uint4*)(Vr + off);                                                    \
      if constexpr (TR)                                                                  \
        dt = *(const uint4*)(Kt + (int64_t)(c / (KT / 8)) * R + ring_add(slot0, (c % (KT / 8)) * 8, R)); \
    }                                                                                    \
  }
#define LOAD_TILE(it_)                                                                   \
  {                                                                                      \
    const int slot0 = (sbase + (it_) * KT) % R;                                          \
    LD(0, rk0, rv0, rt0) LD(1, rk1, rv1, rt1) LD(2, rk2, rv2, rt2) LD(3, rk3, rv3, rt3)  \
  }
#define ST(i, sk, sv, st_)                                                               \
  if constexpr (KCH > i) {                                                               \
    const int c = tid + i * NT, r = c / (HD / 8), col = (c % (HD / 8)) * 8;              \
    if (c < KT * HD / 8) {                                                               \
      *(uint4*)&sm.k[buf][r][col] = sk;                                                  \
      *(uint4*)&sm.v[buf][r][col] = sv;                                                  \
      if constexpr (TR) {                                                                \
        *(uint4*)&sm.kt[buf][c / (KT / 8)][(c % (KT / 8)) * 8] = st_;                    \
      } else {                                                                           \
        const uint32_t w0 = sk.x, w1 = sk.y, w2 = sk.z, w3 = sk.w;                       \
        sm.kt[buf][col + 0][r].x = (uint16_t)w0;                                         \
        sm.kt[buf][col + 1][r].x = (uint16_t)(w0 >> 16);                                 \
        sm.kt[buf][col + 2][r].x = (uint16_t)w1;                                         \
        sm.kt[buf][col + 3][r].x = (uint16_t)(w1 >> 16);                                 \
        sm.kt[buf][col + 4][r].x = (uint16_t)w2;                                         \
        sm.kt[buf][col + 5][r].x = (uint16_t)(w2 >> 16);                                 \
        sm.kt[buf][col + 6][r].x = (uint16_t)w3;                                         \
        sm.kt[buf][col + 7][r].x = (uint16_t)(w3 >> 16);                                 \
      }                                                                                  \
    }                                                                                    \
  }
#define STORE_TILE(buf_)                                                                 \
  {                                                                                      \
    const int buf = (buf_);                                                              \
    ST(0, rk0, rv0, rt0) ST(1, rk1, rv1, rt1) ST(2, rk2, rv2, rt2) ST(3, rk3, rv3, rt3)  \
  }
  if (it_beg < ntiles) {
    LOAD_TILE(it_beg)
    STORE_TILE(it_beg & 1)
  }
  __syncthreads();
  for (int it = it_beg; it < ntiles; ++it) {
    const int cur = it & 1;
    if (it + 1 < ntiles) LOAD_TILE(it + 1)
    const int64_t kp0 = ktile0 + (int64_t)it * KT;
    // masked keys get score -inf (p = 0); only tiles that cut a window edge need it
    const bool full = wfull && kp0 >= wpos_hi - a.window + 1 && kp0 + KT - 1 <= wpos_lo;
    const int64_t hi64 = qpos - kp0, lo64 = qpos - a.window - kp0;
    const int hi = !qok ? -1 : hi64 < -1 ? -1 : hi64 > 64 ? 64 : (int)hi64;
    const int lo = lo64 < -2 ? -2 : lo64 > 64 ? 64 : (int)lo64;
    // the 64-key tile in two halves of 32 keys (keeps the score registers to one half)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x16 s0 = f32x16{}, p0 = f32x16{};
      const bf16* k0p = &sm.k[cur][hf * 32 + (lane & 31)][g * 8];
      const bf16* v0p = &sm.v[cur][hf * 32 + (lane & 31)][g * 8];
#define SSTEP(ks, qv, ev)                                                                          \
  if constexpr (KS > ks) {                                                                         \
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(k0p + ks * 16), qv, s0, 0, 0, 0); \
    p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(v0p + ks * 16), ev, p0, 0, 0, 0); \
  }
      SSTEP(0, q0, e0) SSTEP(1, q1, e1) SSTEP(2, q2, e2) SSTEP(3, q3, e3)
      SSTEP(4, q4, e4) SSTEP(5, q5, e5) SSTEP(6, q6, e6) SSTEP(7, q7, e7)
#undef SSTEP
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = hf * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (!(off <= hi && off > lo)) s0[r] = -INFINITY;
        }
      }
      uint32_t da[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float x0 = ex2(fmaf(s0[r], sl2, nlse2)) * (p0[r] - Dq);
        const float x1 = ex2(fmaf(s0[r + 1], sl2, nlse2)) * (p0[r + 1] - Dq);
        da[r >> 1] = pk2(x0, x1);
      }
      const bf16x8 ds0 = __builtin_bit_cast(bf16x8, make_uint4(da[0], da[1], da[2], da[3]));
      const bf16x8 ds1 = __builtin_bit_cast(bf16x8, make_uint4(da[4], da[5], da[6], da[7]));
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int kc = hf * 32 + st * 16 + 4 * g;
#pragma unroll
        for (int hm = 0; hm < HM; ++hm) {
          const bf16* row = &sm.kt[cur][hm * 32 + (lane & 31)][0];
          uint2 lo2 = *(const uint2*)(row + kc);
          uint2 hi2 = *(const uint2*)(row + kc + 8);
          bf16x8 kf = __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
          acc[hm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, st ? ds1 : ds0, acc[hm], 0, 0, 0);
        }
      }
    }
    if (it + 1 < ntiles) STORE_TILE((it + 1) & 1)
    __syncthreads();
  }
#undef LD
#undef LOAD_TILE
#undef ST
#undef STORE_TILE
  if (!qok) return;
  const float sc = 1.f / sqrtf((float)HD);
  float* out = (SPLIT ? a.ws + (int64_t)sp * a.B * a.n * d : a.dq) + ((int64_t)b * a.n + tq) * d + (int64_t)h * HD;
#pragma unroll
  for (int hm = 0; hm < HM; ++hm)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = hm * 32 + 8 * j + 4 * g;
      *(float4*)(out + d0) = make_float4(acc[hm][4 * j] * sc, acc[hm][4 * j + 1] * sc, acc[hm][4 * j + 2] * sc,
                                         acc[hm][4 * j + 3] * sc);
    }
}

// dK/dV kernel for the chunk's own keys (keys before pos0 are constants and get
// nothing): per wave 32 keys, loop over 64-query tiles of the chunk.  S = Q K^T
// and dP = dO V^T put one key per lane; dV^T += dO^T P and dK^T += Q^T dS with
// the permuted k index over queries.  TR: Q^T and dO^T tiles are 16-byte copies
// of the transposed rows [B][H][hd][n] (n % 8 == 0); otherwise they come from
// transposing LDS stores.
template <int HD>
struct DkvSmem {
  bf16 q[KT][HD + 8];
  bf16 o[KT][HD + 8];   // dO
  bf16 qt[HD][KT + 8];
  bf16 ot[HD][KT + 8];  // dO^T
  float lse2[KT];
  float dd[KT];
};

// P > 1: the block covers part `part` of its key block's query tiles and writes partial
// dK / dV to ws[part] / ws[P + part] (each [B*n][H*hd]).
template <int HD, bool TR>
__global__ __launch_bounds__(256) void k_swa_dkv(AttnBwdArgs a, int P) {
  constexpr int KS = HD / 16, HM = HD / 32;
  constexpr int KCH = KT * HD / 8 / 256;
  static_assert(KCH <= 4, "tile staging covers HD <= 128");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  DkvSmem<HD>& sm = *reinterpret_cast<DkvSmem<HD>*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 5;
  // blockIdx.y = key block * P + part: blocks are dispatched head-fastest in that order, so the
  // early key blocks (the longest query ranges) start first and the short ones fill in behind
  const int b = blockIdx.z, h = blockIdx.x, part = blockIdx.y % P;
  const int64_t bh = (int64_t)b * a.H + h;
  const int R = a.R, d = a.H * HD;
  const int s0blk = (blockIdx.y / P) * BQ;
  const int sk = s0blk + wid * QW + (lane & 31);  // this lane's key (chunk-local)
  const bool kok = sk < a.n;
  const int wsk_hi = s0blk + wid * QW + QW - 1;    // last key of this wave
  const bool wkok = wsk_hi < a.n;                   // all 32 keys of the wave exist
  const float LOG2E = 1.4426950408889634f;
  const float sl2 = LOG2E / sqrtf((float)HD);

  bf16x8 k0, k1, k2, k3, k4, k5, k6, k7, v0, v1, v2, v3, v4, v5, v6, v7;
  {
    const int slot = (int)((a.pos0 + (kok ? sk : 0)) % R);
    const bf16* kp = (const bf16*)a.kr + (bh * R + slot) * HD + g * 8;
    const bf16* vp = (const bf16*)a.vr + (bh * R + slot) * HD + g * 8;
    auto ld8 = [&](const bf16* p, int ks) {
      uint4 v = kok ? *(const uint4*)(p + ks * 16) : make_uint4(0, 0, 0, 0);
      return __builtin_bit_cast(bf16x8, v);
    };
    k0 = ld8(kp, 0); k1 = ld8(kp, 1); v0 = ld8(vp, 0); v1 = ld8(vp, 1);
    if constexpr (KS > 2) { k2 = ld8(kp, 2); k3 = ld8(kp, 3); v2 = ld8(vp, 2); v3 = ld8(vp, 3); }
    if constexpr (KS > 4) { k4 = ld8(kp, 4); k5 = ld8(kp, 5); v4 = ld8(vp, 4); v5 = ld8(vp, 5); }
    if constexpr (KS > 6) { k6 = ld8(kp, 6); k7 = ld8(kp, 7); v6 = ld8(vp, 6); v7 = ld8(vp, 7); }
  }
  f32x16 dk[HM], dv[HM];
#pragma unroll
  for (int i = 0; i < HM; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }
  // queries t >= first key of the block, up to the end of the chunk; part `part` of them
  const int tfirst = (s0blk / KT) * KT;
  const int ntq = (a.n - tfirst + KT - 1) / KT;
  const int per = (ntq + P - 1) / P;
  const int tbeg = tfirst + part * per * KT;
  const int tstop = min(a.n, tfirst + (part + 1) * per * KT);
  // the next query tile is loaded into registers while the current one is computed
  uint4 rq0, rq1, rq2, rq3, ro0, ro1, ro2, ro3, tq_0, tq_1, tq_2, tq_3, to_0, to_1, to_2, to_3;
  float nl2 = 0.f, ndd = 0.f;
  // Q^T / dO^T chunk c (TR): head-dim row c / 8, queries (c % 8) * 8 .. +7
#define LD(i, dq_, do_, tq_, to_)                                                           \
  if constexpr (KCH > i) {                                                                  \
    const int c = tid + i * 256, r = c / (HD / 8), col = (c % (HD / 8)) * 8;                \
    const int t = tl0 + r;                                                                  \
    if (t < a.n) {                                                                          \
      dq_ = *(const uint4*)((const bf16*)a.q + (bh * a.n + t) * HD + col);                  \
      do_ = *(const uint4*)((const bf16*)a.dout + ((int64_t)b * a.n + t) * d + (int64_t)h * HD + col); \
    } else {                                                                                \
      dq_ = make_uint4(0, 0, 0, 0);                                                         \
      do_ = make_uint4(0, 0, 0, 0);                                                         \
    }                                                                                       \
    if constexpr (TR) {                                                                     \
      const int tt = tl0 + (c % (KT / 8)) * 8;                                              \
      const int64_t toff = (bh * HD + c / (KT / 8)) * a.n + tt;                             \
      if (tt < a.n) {                                                                       \
        tq_ = *(const uint4*)((const bf16*)a.qt + toff);                                    \
        to_ = *(const uint4*)((const bf16*)a.dot + toff);                                   \
      } else {                                                                              \
        tq_ = make_uint4(0, 0, 0, 0);                                                       \
        to_ = make_uint4(0, 0, 0, 0);                                                       \
      }                                                                                     \
    }                                                                                       \
  }
#define LOAD_QTILE(T)                                                                       \
  {                                                                                         \
    const int tl0 = (T);                                                                    \
    LD(0, rq0, ro0, tq_0, to_0) LD(1, rq1, ro1, tq_1, to_1) LD(2, rq2, ro2, tq_2, to_2)     \
    LD(3, rq3, ro3, tq_3, to_3)                                                             \
    if (tid < KT) {                                                                         \
      const int t = tl0 + tid;                                                              \
      nl2 = t < a.n ? a.lse[bh * a.n + t] * LOG2E : 0.f;                                    \
      ndd = t < a.n ? a.dvec[bh * a.n + t] : 0.f;                                           \
    }                                                                                       \
  }
  if (tbeg < tstop) LOAD_QTILE(tbeg)
  for (int tq0 = tbeg; tq0 < tstop; tq0 += KT) {
    __syncthreads();  // the previous tile's reads of LDS are done
#define ST(i, sq, so, tq_, to_)                                                             \
  if constexpr (KCH > i) {                                                                  \
    const int c = tid + i * 256, r = c / (HD / 8), col = (c % (HD / 8)) * 8;                \
    *(uint4*)&sm.q[r][col] = sq;                                                            \
    *(uint4*)&sm.o[r][col] = so;                                                            \
    if constexpr (TR) {                                                                     \
      *(uint4*)&sm.qt[c / (KT / 8)][(c % (KT / 8)) * 8] = tq_;                              \
      *(uint4*)&sm.ot[c / (KT / 8)][(c % (KT / 8)) * 8] = to_;                              \
    } else {                                                                                \
      const uint16_t* eq = (const uint16_t*)&sq;                                            \
      const uint16_t* eo = (const uint16_t*)&so;                                            \
      _Pragma("unroll") for (int x = 0; x < 8; ++x) {                                       \
        sm.qt[col + x][r].x = eq[x];                                                        \
        sm.ot[col + x][r].x = eo[x];                                                        \
      }                                                                                     \
    }                                                                                       \
  }
    ST(0, rq0, ro0, tq_0, to_0) ST(1, rq1, ro1, tq_1, to_1) ST(2, rq2, ro2, tq_2, to_2) ST(3, rq3, ro3, tq_3, to_3)
#undef ST
    if (tid < KT) {
      sm.lse2[tid] = nl2;
      sm.dd[tid] = ndd;
    }
    __syncthreads();
    if (tq0 + KT < tstop) LOAD_QTILE(tq0 + KT)
    // the 64-query tile in two halves of 32 queries (keeps the score registers to one half)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x16 s0 = f32x16{}, p0 = f32x16{};
      const bf16* q0p = &sm.q[hf * 32 + (lane & 31)][g * 8];
      const bf16* o0p = &sm.o[hf * 32 + (lane & 31)][g * 8];
#define SSTEP(ks, kv, vv)                                                                          \
  if constexpr (KS > ks) {                                                                         \
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(q0p + ks * 16), kv, s0, 0, 0, 0); \
    p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(o0p + ks * 16), vv, p0, 0, 0, 0); \
  }
      SSTEP(0, k0, v0) SSTEP(1, k1, v1) SSTEP(2, k2, v2) SSTEP(3, k3, v3)
      SSTEP(4, k4, v4) SSTEP(5, k5, v5) SSTEP(6, k6, v6) SSTEP(7, k7, v7)
#undef SSTEP
      // rows = queries tq0 + 32 hf + 8 j + 4 g + i; visible iff sk <= t < n and t - sk < window
      // (window >= n here, so the last condition always holds).  Only halves that reach the
      // chunk end or the diagonal of this wave's keys need the per-element test.
      const int th0 = tq0 + hf * 32;
      const bool full = wkok && th0 + 31 < a.n && th0 >= wsk_hi;
      uint32_t pa[8], da[8];
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const float4 l4 = *(const float4*)&sm.lse2[hf * 32 + 8 * j4 + 4 * g];
        const float4 d4 = *(const float4*)&sm.dd[hf * 32 + 8 * j4 + 4 * g];
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dvv[4] = {d4.x, d4.y, d4.z, d4.w};
        float pv[4], dsv[4];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int rr = 4 * j4 + i4;
          const int t = th0 + 8 * j4 + 4 * g + i4;
          const bool ok = full || (kok && t < a.n && t >= sk);
          const float p = ok ? ex2(fmaf(s0[rr], sl2, -lv[i4])) : 0.f;
          pv[i4] = p;
          dsv[i4] = p * (p0[rr] - dvv[i4]);
        }
        pa[2 * j4] = pk2(pv[0], pv[1]);
        pa[2 * j4 + 1] = pk2(pv[2], pv[3]);
        da[2 * j4] = pk2(dsv[0], dsv[1]);
        da[2 * j4 + 1] = pk2(dsv[2], dsv[3]);
      }
      const bf16x8 pf0 = __builtin_bit_cast(bf16x8, make_uint4(pa[0], pa[1], pa[2], pa[3]));
      const bf16x8 pf1 = __builtin_bit_cast(bf16x8, make_uint4(pa[4], pa[5], pa[6], pa[7]));
      const bf16x8 df0 = __builtin_bit_cast(bf16x8, make_uint4(da[0], da[1], da[2], da[3]));
      const bf16x8 df1 = __builtin_bit_cast(bf16x8, make_uint4(da[4], da[5], da[6], da[7]));
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int kc = hf * 32 + st * 16 + 4 * g;
#pragma unroll
        for (int hm = 0; hm < HM; ++hm) {
          const bf16* orow = &sm.ot[hm * 32 + (lane & 31)][0];
          const bf16* qrow = &sm.qt[hm * 32 + (lane & 31)][0];
          uint2 ol = *(const uint2*)(orow + kc), oh = *(const uint2*)(orow + kc + 8);
          uint2 ql = *(const uint2*)(qrow + kc), qh = *(const uint2*)(qrow + kc + 8);
          bf16x8 of = __builtin_bit_cast(bf16x8, make_uint4(ol.x, ol.y, oh.x, oh.y));
          bf16x8 qf = __builtin_bit_cast(bf16x8, make_uint4(ql.x, ql.y, qh.x, qh.y));
          dv[hm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(of, st ? pf1 : pf0, dv[hm], 0, 0, 0);
          dk[hm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, st ? df1 : df0, dk[hm], 0, 0, 0);
        }
      }
    }
  }
#undef LD
#undef LOAD_QTILE
  // dK (scaled) and then dV of the block's keys leave through LDS as whole rows of HD floats
  // (keys past the chunk end hold zeros and are not written)
  const float sc = 1.f / sqrtf((float)HD);
  const int64_t plane = (int64_t)a.B * a.n * d;
  constexpr int SLD = HD + 4;
  static_assert(BQ * SLD * 4 <= sizeof(DkvSmem<HD>), "staged dK / dV rows fit");
  float* st = reinterpret_cast<float*>(smem_raw);
  const int kr = wid * QW + (lane & 31);  // the lane's key row in the block
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    __syncthreads();  // the last tile's (then the dK rows') reads of LDS are done
#pragma unroll
    for (int hm = 0; hm < HM; ++hm)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = hm * 32 + 8 * j + 4 * g;
        *(float4*)(st + kr * SLD + d0) =
            which == 0 ? make_float4(dk[hm][4 * j] * sc, dk[hm][4 * j + 1] * sc, dk[hm][4 * j + 2] * sc, dk[hm][4 * j + 3] * sc)
                       : make_float4(dv[hm][4 * j], dv[hm][4 * j + 1], dv[hm][4 * j + 2], dv[hm][4 * j + 3]);
      }
    __syncthreads();
    float* base = (P > 1 ? a.ws + (which * P + part) * plane : (which ? a.dv : a.dk)) + ((int64_t)b * a.n + s0blk) * d +
                  (int64_t)h * HD;
    for (int c = tid; c < BQ * (HD / 4); c += 256) {
      const int r = c / (HD / 4), c4 = (c % (HD / 4)) * 4;
      if (s0blk + r < a.n) *(float4*)(base + (int64_t)r * d + c4) = *(const float4*)(st + r * SLD + c4);
    }
  }
}

// One stage of the direct-to-LDS dK/dV kernel below: the Q and dO tiles [64 queries][hd] (the
// 16-byte chunks of a row XOR-swizzled by row % 16 at hd 128, by (row / 2) % 8 at hd 64), the
// transposed Q^T and dO^T tiles [hd][64 queries] (chunks swizzled by (row / 2) % 8), and the tile's
// 64 log-sum-exp and D values (1 KB each).
template <int HD>
constexpr int dkv2_stage_bytes() { return 4 * KT * HD * 2 + 2 * 1024; }

// dK/dV for the chunk's own keys with the query tiles copied straight from global memory into
// LDS (buffer loads to LDS, two stages, per-lane offsets precomputed, no per-row bounds tests:
// every query tile of the chunk is whole, n % 64 == 0; head dim 128 or 64; 32-bit byte offsets
// within a head's arrays), 16 keys per wave on the 16 x 16 x 32 matrix instructions: 8 waves
// (two per SIMD at hd 128) cover the 128 keys of a block, and the two waves of a SIMD hide each
// other's latencies (a 32-key wave needs about 400 registers, one wave per SIMD).  The fragments
// of a phase are read in one group before its MFMAs, and the next tile's copies go out after the
// tile's last LDS read.  Otherwise as k_swa_dkv (TR form).  In
// the 16 x 16 x 32 product a lane supplies row (or column) l % 16 and k indices 8 (l / 16) .. +7,
// and holds rows 4 (l / 16) .. +3 of column l % 16 of the result; P and dS feed the dV and dK
// products from registers with the k index over the 32 queries of a half-tile permuted so that
// k slot e of lane group G is query 16 (e / 4) + 4 G + e % 4 -- the rows the lane holds.
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int HD>
__global__ __launch_bounds__(512) void k_swa_dkv3(AttnBwdArgs a, int P) {
  constexpr int NWV = 8, KW = 16;          // waves, keys per wave
  constexpr int KS = HD / 32, HB = HD / 16;
  constexpr int CPR = HD / 8;
  constexpr int RPK = 1024 / (HD * 2);
  constexpr int TB = KT * HD * 2 / 1024;
  constexpr int TBW = TB / NWV;
  constexpr int SB = dkv2_stage_bytes<HD>();
  constexpr int OOFF = KT * HD * 2, QTOFF = 2 * KT * HD * 2, OTOFF = 3 * KT * HD * 2;
  constexpr int LOFF = 4 * KT * HD * 2, DOFF = LOFF + 1024;
  static_assert(TB % NWV == 0 && (CPR == 16 || CPR == 8) && KT == 64 && NWV * KW == BQ, "tile copy layout");
  auto qswz = [](int row) { return CPR == 16 ? row % 16 : (row >> 1) & 7; };
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, l16 = lane & 15;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.z, h = blockIdx.x, part = blockIdx.y % P;
  const int64_t bh = (int64_t)b * a.H + h;
  const int R = a.R, d = a.H * HD, n = a.n;
  const int s0blk = (blockIdx.y / P) * BQ;
  const int sk = s0blk + wid * KW + l16;  // this lane's key (chunk-local)
  const bool kok = sk < n;
  const int wsk_hi = s0blk + wid * KW + KW - 1;
  const bool wkok = wsk_hi < n;
  const float LOG2E = 1.4426950408889634f;
  const float sl2 = LOG2E / sqrtf((float)HD);

  // K (pre-multiplied by log2(e)/sqrt(hd)) and V fragments of this lane's key: head dims
  // 32 ks + 8 G .. +7
  bf16x8 kf[KS], vf[KS];
  {
    const int slot = (int)((a.pos0 + (kok ? sk : 0)) % R);
    const bf16* kp = (const bf16*)a.kr + (bh * R + slot) * HD + G * 8;
    const bf16* vp = (const bf16*)a.vr + (bh * R + slot) * HD + G * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = __builtin_bit_cast(bf16x8, kok ? *(const uint4*)(kp + ks * 32) : make_uint4(0, 0, 0, 0));
      vf[ks] = __builtin_bit_cast(bf16x8, kok ? *(const uint4*)(vp + ks * 32) : make_uint4(0, 0, 0, 0));
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[ks][e] = (__bf16)((float)kf[ks][e] * sl2);
    }
  }
  f32x4 dk[HB], dv[HB];
#pragma unroll
  for (int i = 0; i < HB; ++i) {
    dk[i] = f32x4{};
    dv[i] = f32x4{};
  }
  const int tfirst = (s0blk / KT) * KT;
  const int ntq = (n - tfirst + KT - 1) / KT;
  const int per = (ntq + P - 1) / P;
  const int tbeg = tfirst + part * per * KT;
  const int tstop = min(n, tfirst + (part + 1) * per * KT);

  const __amdgpu_buffer_rsrc_t rq = buf_rsrc((const bf16*)a.q + bh * n * HD, (uint32_t)(n * HD * 2));
  const __amdgpu_buffer_rsrc_t rqt = buf_rsrc((const bf16*)a.qt + bh * HD * n, (uint32_t)(n * HD * 2));
  const __amdgpu_buffer_rsrc_t rot = buf_rsrc((const bf16*)a.dot + bh * HD * n, (uint32_t)(n * HD * 2));
  const __amdgpu_buffer_rsrc_t ro =
      buf_rsrc((const bf16*)a.dout + (int64_t)b * n * d + (int64_t)h * HD, (uint32_t)((int64_t)n * d * 2));
  const __amdgpu_buffer_rsrc_t rl = buf_rsrc(a.lse + bh * n, (uint32_t)(n * 4));
  const __amdgpu_buffer_rsrc_t rd = buf_rsrc(a.dvec + bh * n, (uint32_t)(n * 4));
  int oq[TBW], oo[TBW], ot[TBW];
#pragma unroll
  for (int u = 0; u < TBW; ++u) {
    const int j = wid * TBW + u;
    const int row = j * RPK + lane / CPR, c = (lane % CPR) ^ qswz(row);
    oq[u] = (row * HD + c * 8) * 2;
    oo[u] = (row * d + c * 8) * 2;
    const int trow = j * 8 + (lane >> 3), tc = (lane & 7) ^ ((trow >> 1) & 7);
    ot[u] = (trow * n + tc * 8) * 2;
  }
  const int ol = (lane & 15) * 16;
  auto issue = [&](int t0, int st) {
    unsigned char* base = smem_raw + st * SB;
#pragma unroll
    for (int u = 0; u < TBW; ++u) {
      const int j = wid * TBW + u;
      buf_lds16(rq, base + j * 1024, oq[u], t0 * HD * 2);
      buf_lds16(ro, base + OOFF + j * 1024, oo[u], t0 * d * 2);
      buf_lds16(rqt, base + QTOFF + j * 1024, ot[u], t0 * 2);
      buf_lds16(rot, base + OTOFF + j * 1024, ot[u], t0 * 2);
    }
    if (wid == 0) {
      buf_lds16(rl, base + LOFF, ol, t0 * 4);
      buf_lds16(rd, base + DOFF, ol, t0 * 4);
    }
  };
  const int xr = qswz(l16), xt = (l16 >> 1) & 7;  // (rows r * 16 + l16 keep the swizzle of l16)
  if (tbeg < tstop) issue(tbeg, 0);
  WAIT_VM_LDS(0);
  __syncthreads();
  int it = 0;
  for (int tq0 = tbeg; tq0 < tstop; tq0 += KT, ++it) {
    const int cur = it & 1;
    const unsigned char* stg = smem_raw + cur * SB;
    const float* lse_t = reinterpret_cast<const float*>(stg + LOFF);
    const float* dd_t = reinterpret_cast<const float*>(stg + DOFF);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      // S and dP of the half-tile's two 16-query row blocks, started at minus the row's
      // log-sum-exp (log2 units) and minus its D
      f32x4 sc[2], pc[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float4 l4 = *(const float4*)&lse_t[hf * 32 + rb * 16 + 4 * G];
        const float4 d4 = *(const float4*)&dd_t[hf * 32 + rb * 16 + 4 * G];
        sc[rb] = f32x4{-LOG2E * l4.x, -LOG2E * l4.y, -LOG2E * l4.z, -LOG2E * l4.w};
        pc[rb] = f32x4{-d4.x, -d4.y, -d4.z, -d4.w};
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const unsigned char* qrow = stg + (hf * 32 + rb * 16 + l16) * (HD * 2);
        bf16x8 aq[KS], ao[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int co = (((4 * ks + G) ^ xr) << 4);
          aq[ks] = *(const bf16x8*)(qrow + co);
          ao[ks] = *(const bf16x8*)(qrow + OOFF + co);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          sc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[ks], kf[ks], sc[rb], 0, 0, 0);
          pc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao[ks], vf[ks], pc[rb], 0, 0, 0);
        }
      }
      // rows = queries tq0 + 32 hf + 16 rb + 4 G + i; visible iff sk <= t (window >= n here)
      const int th0 = tq0 + hf * 32;
      const bool full = wkok && th0 >= wsk_hi;
      uint32_t pa[4], da[4];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float pv[4], dsv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = th0 + rb * 16 + 4 * G + i;
          float x = sc[rb][i];
          if (!full) x = (kok && t >= sk) ? x : -INFINITY;
          const float pp = ex2(x);
          pv[i] = pp;
          dsv[i] = pp * pc[rb][i];
        }
        pa[2 * rb] = pk2(pv[0], pv[1]);
        pa[2 * rb + 1] = pk2(pv[2], pv[3]);
        da[2 * rb] = pk2(dsv[0], dsv[1]);
        da[2 * rb + 1] = pk2(dsv[2], dsv[3]);
      }
      const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(pa[0], pa[1], pa[2], pa[3]));
      const bf16x8 df = __builtin_bit_cast(bf16x8, make_uint4(da[0], da[1], da[2], da[3]));
      // dV^T += dO^T P, dK^T += Q^T dS over the half's 32 queries: the A fragments are queries
      // 32 hf + 4 G .. +3 and 32 hf + 16 + 4 G .. +3 of head-dim row 16 hb + l16
      const int c0 = hf * 4 + (G >> 1), c1 = c0 + 2, bo = 8 * (G & 1);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const unsigned char* trow = stg + QTOFF + (hb * 16 + l16) * (KT * 2) + bo;
        const unsigned char* orow = stg + OTOFF + (hb * 16 + l16) * (KT * 2) + bo;
        const uint2 ql = *(const uint2*)(trow + ((c0 ^ xt) << 4));
        const uint2 qh = *(const uint2*)(trow + ((c1 ^ xt) << 4));
        const uint2 olo = *(const uint2*)(orow + ((c0 ^ xt) << 4));
        const uint2 ohi = *(const uint2*)(orow + ((c1 ^ xt) << 4));
        const bf16x8 ofr = __builtin_bit_cast(bf16x8, make_uint4(olo.x, olo.y, ohi.x, ohi.y));
        const bf16x8 qfr = __builtin_bit_cast(bf16x8, make_uint4(ql.x, ql.y, qh.x, qh.y));
        dv[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ofr, pf, dv[hb], 0, 0, 0);
        dk[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qfr, df, dk[hb], 0, 0, 0);
      }
      // the next tile's copies go out after this tile's last LDS reads (an LDS read issued
      // after them would wait for them)
      __builtin_amdgcn_sched_barrier(0);
      if (hf == 1 && tq0 + KT < tstop) issue(tq0 + KT, cur ^ 1);
    }
    WAIT_VM_LDS(0);
    __syncthreads();  // the next tile is in LDS; every wave is done with this one
  }
  // dK (scaled) and then dV leave through LDS as whole rows of HD floats: the lane holds head
  // dims 16 hb + 4 G .. +3 of key wid * 16 + l16
  const float scl = 1.f / sqrtf((float)HD);
  const int64_t plane = (int64_t)a.B * n * d;
  constexpr int SLD = HD + 4;
  static_assert(BQ * SLD * 4 <= 2 * SB, "staged dK / dV rows fit");
  float* stf = reinterpret_cast<float*>(smem_raw);
  const int kr = wid * KW + l16;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    if (which > 0) __syncthreads();
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const f32x4 v = which == 0 ? dk[hb] * scl : dv[hb];
      *(float4*)(stf + kr * SLD + hb * 16 + 4 * G) = make_float4(v[0], v[1], v[2], v[3]);
    }
    __syncthreads();
    float* base = (P > 1 ? a.ws + (which * P + part) * plane : (which ? a.dv : a.dk)) + ((int64_t)b * n + s0blk) * d +
                  (int64_t)h * HD;
    for (int c = tid; c < BQ * (HD / 4); c += NWV * 64) {
      const int r = c / (HD / 4), c4 = (c % (HD / 4)) * 4;
      if (s0blk + r < n) *(float4*)(base + (int64_t)r * d + c4) = *(const float4*)(stf + r * SLD + c4);
    }
  }
}

template <int HD>
hipError_t launch_dkv3(const AttnBwdArgs& a, int P, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k_swa_dkv3<HD>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       2 * dkv2_stage_bytes<HD>());
    if (e != hipSuccess) return e;
    attr = true;
  }
  if ((int64_t)cdiv(a.n, BQ) * P > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_swa_dkv3<HD>), dim3(a.H, cdiv(a.n, BQ) * P, a.B), dim3(512), 2 * dkv2_stage_bytes<HD>(), s,
                     a, P);
  return hipGetLastError();
}

template <typename Smem, typename K>
hipError_t set_lds(K kern) {
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(Smem));
}

// dk = sum_p ws[p], dv = sum_p ws[P + p], in order (4 elements per thread; total % 4 == 0)
__global__ __launch_bounds__(256) void k_dkv_reduce(const float* ws, int P, int64_t total, float* dk, float* dv) {
  for (int64_t i = 4 * (blockIdx.x * (int64_t)blockDim.x + threadIdx.x); i < total;
       i += 4 * (int64_t)gridDim.x * blockDim.x) {
    float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
    for (int p = 0; p < P; ++p) {
      const float4 a = *(const float4*)(ws + p * total + i);
      const float4 c = *(const float4*)(ws + (P + p) * total + i);
      sk.x += a.x; sk.y += a.y; sk.z += a.z; sk.w += a.w;
      sv.x += c.x; sv.y += c.y; sv.z += c.z; sv.w += c.w;
    }
    *(float4*)(dk + i) = sk;
    *(float4*)(dv + i) = sv;
  }
}

// dq = sum over the key-range parts, in order (4 elements per thread; total % 4 == 0)
__global__ __launch_bounds__(256) void k_dq_reduce(const float* ws, int S, int64_t total, float* dq) {
  for (int64_t i = 4 * (blockIdx.x * (int64_t)blockDim.x + threadIdx.x); i < total;
       i += 4 * (int64_t)gridDim.x * blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sidx = 0; sidx < S; ++sidx) {
      const float4 v = *(const float4*)(ws + sidx * total + i);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *(float4*)(dq + i) = acc;
  }
}

// dO [B*n][H*hd] -> dO^T [B][H][hd][n], 64 x 64 tiles through LDS with 16-byte global
// loads and stores (H*hd % 8 == 0 and n % 8 == 0)
__global__ __launch_bounds__(256) void k_heads_transpose(const bf16* __restrict__ x, bf16* __restrict__ xt, int n,
                                                         int H, int hd) {
  __shared__ __align__(16) uint16_t tile[64][72];  // [token][column]
  const int d = H * hd, t0 = blockIdx.x * 64, c0 = blockIdx.y * 64, b = blockIdx.z;
  for (int e = threadIdx.x; e < 64 * 8; e += 256) {
    const int r = e >> 3, ch = (e & 7) * 8, t = t0 + r, c = c0 + ch;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t < n && c < d) v = *(const uint4*)(x + ((int64_t)b * n + t) * d + c);
    *(uint4*)&tile[r][ch] = v;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 8; e += 256) {
    const int cr = e >> 3, tch = (e & 7) * 8, c = c0 + cr, t = t0 + tch;
    if (c < d && t < n) {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = (uint32_t)tile[tch + 2 * k][cr] | ((uint32_t)tile[tch + 2 * k + 1][cr] << 16);
      *(uint4*)(xt + ((int64_t)b * d + c) * n + t) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// dQ with the K, V and K^T tiles copied straight from global memory into LDS
// (global_load_lds: lane L of a wave writes 16 bytes at the wave's LDS address + 16 L), two
// stages, no staging registers.  Rows are unpadded; the 16-byte chunks of a K or V row are
// XOR-swizzled by row % (hd/8) and those of a K^T row by (row / 2) % 8, which keeps the fragment
// reads of a wave on distinct banks.  Needs the transposed key ring; otherwise as k_swa_dq.
template <int HD>
constexpr int dq2_stage_bytes() { return 3 * KT * HD * 2; }

template <int HD, bool SPLIT>
__global__ __launch_bounds__(512) void k_swa_dq2(AttnBwdArgs a, int S) {
  constexpr int NW = 8, BQn = NW * QW;
  constexpr int KS = HD / 16, HM = HD / 32;
  constexpr int CPR = HD / 8;              // 16-byte chunks per K / V row
  constexpr int RPK = 1024 / (HD * 2);     // K / V rows per 1 KB copy
  constexpr int TB = KT * HD * 2 / 1024;   // 1 KB copies per tile (K, V and K^T each)
  constexpr int TBW = TB / NW;             // per wave
  constexpr int SB = dq2_stage_bytes<HD>();
  constexpr int VOFF = KT * HD * 2, TOFF = 2 * KT * HD * 2;
  static_assert(TB % NW == 0 && CPR * 16 == HD * 2 && 32 % CPR == 0, "tile copy layout");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS addresses stay scalar
  const int b = SPLIT ? blockIdx.z / S : blockIdx.z, h = blockIdx.y;
  const int sp = SPLIT ? blockIdx.z % S : 0;
  const int64_t bh = (int64_t)b * a.H + h;
  const int R = a.R, d = a.H * HD;
  const int t0 = blockIdx.x * BQn;
  const int tq = t0 + wid * QW + l32;
  const bool qok = tq < a.n;
  const int64_t qpos = a.pos0 + tq;
  const int tw0 = t0 + wid * QW;
  const bool wfull = tw0 + QW <= a.n;
  const int64_t wpos_lo = a.pos0 + tw0, wpos_hi = wpos_lo + QW - 1;
  const bf16* Kr = (const bf16*)a.kr + bh * R * HD;
  const bf16* Vr = (const bf16*)a.vr + bh * R * HD;
  const bf16* Kt = (const bf16*)a.ktr + bh * HD * R;

  bf16x8 q0, q1, q2, q3, q4, q5, q6, q7, e0, e1, e2, e3, e4, e5, e6, e7;
  {
    const bf16* q = (const bf16*)a.q + (bh * a.n + (qok ? tq : 0)) * HD + g * 8;
    const bf16* dO = (const bf16*)a.dout + ((int64_t)b * a.n + (qok ? tq : 0)) * d + (int64_t)h * HD + g * 8;
    auto ld8 = [&](const bf16* p, int ks) {
      uint4 v = qok ? *(const uint4*)(p + ks * 16) : make_uint4(0, 0, 0, 0);
      return __builtin_bit_cast(bf16x8, v);
    };
    q0 = ld8(q, 0); q1 = ld8(q, 1); e0 = ld8(dO, 0); e1 = ld8(dO, 1);
    if constexpr (KS > 2) { q2 = ld8(q, 2); q3 = ld8(q, 3); e2 = ld8(dO, 2); e3 = ld8(dO, 3); }
    if constexpr (KS > 4) { q4 = ld8(q, 4); q5 = ld8(q, 5); e4 = ld8(dO, 4); e5 = ld8(dO, 5); }
    if constexpr (KS > 6) { q6 = ld8(q, 6); q7 = ld8(q, 7); e6 = ld8(dO, 6); e7 = ld8(dO, 7); }
  }
  const float LOG2E = 1.4426950408889634f;
  const float sl2 = LOG2E / sqrtf((float)HD);
  const float nlse2 = qok ? -a.lse[bh * a.n + tq] * LOG2E : 0.f;
  // D = rowsum(dO * O) of this lane's query from its own dO fragments and the matching O
  // fragments (the lane pair holds the two halves of the head dim); written for the dK/dV
  // kernel by the first key-range part
  float Dq;
  {
    const bf16* op = (const bf16*)a.o + ((int64_t)b * a.n + (qok ? tq : 0)) * d + (int64_t)h * HD + g * 8;
    float part = 0.f;
    auto dot8 = [&](const bf16x8& e, int ks) {
      const bf16x8 o = __builtin_bit_cast(bf16x8, qok ? *(const uint4*)(op + ks * 16) : make_uint4(0, 0, 0, 0));
#pragma unroll
      for (int u = 0; u < 8; ++u) part = fmaf((float)e[u], (float)o[u], part);
    };
    dot8(e0, 0); dot8(e1, 1);
    if constexpr (KS > 2) { dot8(e2, 2); dot8(e3, 3); }
    if constexpr (KS > 4) { dot8(e4, 4); dot8(e5, 5); }
    if constexpr (KS > 6) { dot8(e6, 6); dot8(e7, 7); }
    Dq = part + __shfl_xor(part, 32, 64);
    if (qok && g == 0 && sp == 0) a.dvec[bh * a.n + tq] = Dq;
  }

  const int tlast = min(t0 + BQn, a.n) - 1;
  const int64_t kbeg = max((int64_t)0, a.pos0 + t0 - a.window + 1);
  const int64_t kend = a.pos0 + tlast;
  const int64_t ktile0 = (kbeg / KT) * KT;
  const int ntiles_all = (int)((kend - ktile0) / KT) + 1;
  const int per = SPLIT ? (ntiles_all + S - 1) / S : ntiles_all;
  const int it_beg = SPLIT ? min(ntiles_all, sp * per) : 0;
  const int ntiles = SPLIT ? min(ntiles_all, it_beg + per) : ntiles_all;
  const int sbase = (int)(ktile0 % R);

  // copies of tile it_ into stage st: K and V rows by ring slot, K^T rows (head dims) of
  // 64 consecutive slots (tiles start at multiples of 64 positions and R % 8 == 0, so an
  // 8-key chunk never wraps)
  // the head's K, V and K^T rings are buffers (32-bit byte offsets, checked at launch)
  const __amdgpu_buffer_rsrc_t rk = buf_rsrc(Kr, (uint32_t)(R * HD * 2)), rv = buf_rsrc(Vr, (uint32_t)(R * HD * 2)),
                               rt = buf_rsrc(Kt, (uint32_t)(R * HD * 2));
  auto issue = [&](int it_, int st) {
    const int slot0 = (sbase + it_ * KT) % R;
    unsigned char* base = smem_raw + st * SB;
#pragma unroll
    for (int u = 0; u < TBW; ++u) {
      const int j = wid * TBW + u;
      const int row = j * RPK + lane / CPR, c = (lane % CPR) ^ (row % CPR);
      const int off = (ring_add(slot0, row, R) * HD + c * 8) * 2;
      buf_lds16(rk, base + j * 1024, off, 0);
      buf_lds16(rv, base + VOFF + j * 1024, off, 0);
      const int trow = j * 8 + (lane >> 3), tc = (lane & 7) ^ ((trow >> 1) & 7);
      buf_lds16(rt, base + TOFF + j * 1024, (trow * R + ring_add(slot0, tc * 8, R)) * 2, 0);
    }
  };

  f32x16 acc[HM];
#pragma unroll
  for (int i = 0; i < HM; ++i) acc[i] = f32x16{};
  const int xr = l32 % CPR, xt = (l32 >> 1) & 7;
  if (it_beg < ntiles) issue(it_beg, it_beg & 1);
  WAIT_VM_LDS(0);
  __syncthreads();
  for (int it = it_beg; it < ntiles; ++it) {
    const int cur = it & 1;
    if (it + 1 < ntiles) issue(it + 1, cur ^ 1);
    const unsigned char* stg = smem_raw + cur * SB;
    const int64_t kp0 = ktile0 + (int64_t)it * KT;
    const bool full = wfull && kp0 >= wpos_hi - a.window + 1 && kp0 + KT - 1 <= wpos_lo;
    const int64_t hi64 = qpos - kp0, lo64 = qpos - a.window - kp0;
    const int hi = !qok ? -1 : hi64 < -1 ? -1 : hi64 > 64 ? 64 : (int)hi64;
    const int lo = lo64 < -2 ? -2 : lo64 > 64 ? 64 : (int)lo64;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x16 s0 = f32x16{}, p0 = f32x16{};
      const unsigned char* krow = stg + (hf * 32 + l32) * (HD * 2);
#define SSTEP(ks, qv, ev)                                                                          \
  if constexpr (KS > ks) {                                                                         \
    const int co = (((2 * ks + g) ^ xr) << 4);                                                     \
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(krow + co), qv, s0, 0, 0, 0);    \
    p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(krow + VOFF + co), ev, p0, 0, 0, 0); \
  }
      SSTEP(0, q0, e0) SSTEP(1, q1, e1) SSTEP(2, q2, e2) SSTEP(3, q3, e3)
      SSTEP(4, q4, e4) SSTEP(5, q5, e5) SSTEP(6, q6, e6) SSTEP(7, q7, e7)
#undef SSTEP
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = hf * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (!(off <= hi && off > lo)) s0[r] = -INFINITY;
        }
      }
      uint32_t da[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float x0 = ex2(fmaf(s0[r], sl2, nlse2)) * (p0[r] - Dq);
        const float x1 = ex2(fmaf(s0[r + 1], sl2, nlse2)) * (p0[r + 1] - Dq);
        da[r >> 1] = pk2(x0, x1);
      }
      const bf16x8 ds0 = __builtin_bit_cast(bf16x8, make_uint4(da[0], da[1], da[2], da[3]));
      const bf16x8 ds1 = __builtin_bit_cast(bf16x8, make_uint4(da[4], da[5], da[6], da[7]));
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int ch = hf * 4 + st * 2;  // 16-byte chunk of keys hf*32 + st*16 .. +7
#pragma unroll
        for (int hm = 0; hm < HM; ++hm) {
          const unsigned char* trow = stg + TOFF + (hm * 32 + l32) * (KT * 2) + 8 * g;
          const uint2 lo2 = *(const uint2*)(trow + ((ch ^ xt) << 4));
          const uint2 hi2 = *(const uint2*)(trow + (((ch + 1) ^ xt) << 4));
          const bf16x8 kf = __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
          acc[hm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, st ? ds1 : ds0, acc[hm], 0, 0, 0);
        }
      }
    }
    WAIT_VM_LDS(0);
    __syncthreads();
  }
  // dQ rows leave through LDS as whole rows of HD floats, half the block's queries at a time
  // (queries past the chunk end hold zeros and are not written)
  const float sc = 1.f / sqrtf((float)HD);
  constexpr int SLD = HD + 4, HQ = BQn / 2;
  static_assert(HQ * SLD * 4 <= 2 * SB, "staged dQ rows fit");
  float* st = reinterpret_cast<float*>(smem_raw);
  float* outb = (SPLIT ? a.ws + (int64_t)sp * a.B * a.n * d : a.dq) + ((int64_t)b * a.n + t0) * d + (int64_t)h * HD;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (half > 0) __syncthreads();  // the first half's rows have left LDS
    if (wid / (NW / 2) == half) {
      const int r = (wid % (NW / 2)) * QW + l32;
#pragma unroll
      for (int hm = 0; hm < HM; ++hm)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d0 = hm * 32 + 8 * j + 4 * g;
          *(float4*)(st + r * SLD + d0) = make_float4(acc[hm][4 * j] * sc, acc[hm][4 * j + 1] * sc,
                                                      acc[hm][4 * j + 2] * sc, acc[hm][4 * j + 3] * sc);
        }
    }
    __syncthreads();
    for (int c = tid; c < HQ * (HD / 4); c += NW * 64) {
      const int r = c / (HD / 4), c4 = (c % (HD / 4)) * 4, tq_ = half * HQ + r;
      if (t0 + tq_ < a.n) *(float4*)(outb + (int64_t)tq_ * d + c4) = *(const float4*)(st + r * SLD + c4);
    }
  }
}

template <int HD, bool SPLIT>
hipError_t launch_dq2(const AttnBwdArgs& a, int S, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k_swa_dq2<HD, SPLIT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       2 * dq2_stage_bytes<HD>());
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((k_swa_dq2<HD, SPLIT>), dim3(cdiv(a.n, 8 * QW), a.H, a.B * S), dim3(512),
                     2 * dq2_stage_bytes<HD>(), s, a, S);
  return hipGetLastError();
}

template <int HD, int NW, bool SPLIT, bool TR>
hipError_t launch_dq(const AttnBwdArgs& a, int S, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = set_lds<DqSmem<HD>>(k_swa_dq<HD, NW, SPLIT, TR>);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((k_swa_dq<HD, NW, SPLIT, TR>), dim3(cdiv(a.n, NW * QW), a.H, a.B * S), dim3(NW * 64),
                     sizeof(DqSmem<HD>), s, a, S);
  return hipGetLastError();
}

template <int HD, bool TR>
hipError_t launch_dkv(const AttnBwdArgs& a, int P, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = set_lds<DkvSmem<HD>>(k_swa_dkv<HD, TR>);
    if (e != hipSuccess) return e;
    attr = true;
  }
  if ((int64_t)cdiv(a.n, BQ) * P > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_swa_dkv<HD, TR>), dim3(a.H, cdiv(a.n, BQ) * P, a.B), dim3(256), sizeof(DkvSmem<HD>), s, a,
                     P);
  return hipGetLastError();
}

// TTT_NO_DKV2=1 (tuning switch): the register-staged dK/dV kernel everywhere (not the direct-to-LDS one)
bool dkv2_off() {
  static int off = -1;
  if (off < 0) {
    const char* e = getenv("TTT_NO_DKV2");
    off = e && atoi(e) ? 1 : 0;
  }
  return off == 1;
}

template <int HD>
hipError_t launch_bwd(const AttnBwdArgs& a, hipStream_t s, AttnBwdParts* parts) {
  // the direct-to-LDS dQ form (head dim 128, transposed key ring) computes D = rowsum(dO * O)
  // itself and stores it for dK/dV; otherwise a separate pass does
  // (the direct-to-LDS dQ form addresses a head's ring with 32-bit byte offsets)
  const bool tr = a.ktr && a.dot && a.R % 8 == 0 && a.n % 8 == 0 && (a.H * HD) % 8 == 0 &&
                  (int64_t)a.R * HD * 2 < (1LL << 31);
  constexpr bool DQ2 = HD == 128;
  hipError_t e = hipSuccess;
  if (!(DQ2 && tr)) {
    e = swa_dvec_bf16(a, s);
    if (e != hipSuccess) return e;
  }
  // transposed tiles are read with 16-byte copies when the caller provides the
  // transposed key ring and a dO^T scratch, 8-key groups stay inside the ring
  // (R % 8 == 0) and 8-query groups inside the chunk (n % 8 == 0)
  if (tr && !a.dot_ready)
    hipLaunchKernelGGL(k_heads_transpose, dim3(cdiv(a.n, 64), cdiv(a.H * HD, 64), a.B), dim3(256), 0, s,
                       (const bf16*)a.dout, (bf16*)a.dot, a.n, a.H, HD);
  const int64_t blocks8 = (int64_t)cdiv(a.n, 8 * QW) * a.H * a.B;
  const int64_t ntiles = (std::min<int64_t>(a.window, a.pos0 + 1) + 8 * QW) / KT + 1;
  const int64_t total = (int64_t)a.B * a.n * a.H * HD;
  int S = attn_splits(blocks8, ntiles, total, a.ws, a.ws_floats);
  static int force_s = -1;  // TTT_DQ_SPLITS (tuning switch): key-range parts of dQ
  if (force_s < 0) {
    const char* ev = getenv("TTT_DQ_SPLITS");
    force_s = ev ? std::max(0, atoi(ev)) : 0;
  }
  if (force_s > 0 && a.ws && (int64_t)force_s * total <= a.ws_floats / 2) S = force_s;
  // (the direct-to-LDS dQ form: measured faster at head dim 128, slower at 64)
  if (S > 1) {
    if constexpr (DQ2) e = tr ? launch_dq2<HD, true>(a, S, s) : launch_dq<HD, 8, true, false>(a, S, s);
    else e = tr ? launch_dq<HD, 8, true, true>(a, S, s) : launch_dq<HD, 8, true, false>(a, S, s);
    if (e != hipSuccess) return e;
    if (!parts)
      hipLaunchKernelGGL(k_dq_reduce, dim3((unsigned)std::min<int64_t>(cdiv(total / 4, 256), 8192)), dim3(256), 0, s,
                         a.ws, S, total, a.dq);
  } else {
    if constexpr (DQ2) e = tr ? launch_dq2<HD, false>(a, 1, s) : launch_dq<HD, 8, false, false>(a, 1, s);
    else e = tr ? launch_dq<HD, 8, false, true>(a, 1, s) : launch_dq<HD, 8, false, false>(a, 1, s);
    if (e != hipSuccess) return e;
  }
  // dK/dV: split each key block's query range when the grid is small (ordered sum after);
  // one 4-wave block per CU, so pick the P <= 4 with the fewest rounds of 256 blocks per part.
  // Parts left to the caller go after the dQ parts in the workspace.
  AttnBwdArgs kv = a;
  if (parts && S > 1) {
    kv.ws = a.ws + S * total;
    kv.ws_floats = a.ws_floats - S * total;
  }
  const int64_t kblocks = (int64_t)cdiv(a.n, BQ) * a.H * a.B;
  int P = 1;
  static int force_p = -1;  // TTT_DKV_PARTS (tuning switch): query-range parts of dK/dV
  if (force_p < 0) {
    const char* ev = getenv("TTT_DKV_PARTS");
    force_p = ev ? std::max(0, atoi(ev)) : 0;
  }
  if (force_p > 0 && kv.ws && 2LL * force_p * total <= kv.ws_floats) {
    P = std::min(force_p, (int)cdiv(a.n, KT));
  } else if (kv.ws && kblocks < 256) {
    double best = 1e30;
    for (int p = 1; p <= std::min(4, (int)cdiv(a.n, KT)); ++p) {
      if (p > 1 && 2LL * p * total > kv.ws_floats) break;
      const double cost = (double)cdiv(kblocks * p, 256) / p;
      if (cost < best - 1e-9) {
        best = cost;
        P = p;
      }
    }
  }
  // the direct-to-LDS dK/dV form: head dim 128 or 64, transposed tiles, whole 64-query tiles, a head's
  // arrays and the row's dO within 32-bit byte offsets.  It takes at most two parts: at the 3B
  // chunk shape (160 key blocks) two parts beat the three that the model above picks, inside the
  // step (1828 against 1837 ms, same box; one part 1828), where fewer parts also mean fewer fp32
  // planes written here and summed by the consumer
  const bool dkv2 = (HD == 128 || HD == 64) && tr && a.n % KT == 0 && (int64_t)a.n * a.H * HD * 2 < (1LL << 31) &&
                    !dkv2_off();
  if (dkv2 && force_p == 0) P = std::min(P, 2);
  if constexpr (HD == 128 || HD == 64) {
    if (dkv2) e = launch_dkv3<HD>(kv, P, s);
  }
  if (!dkv2) e = tr ? launch_dkv<HD, true>(kv, P, s) : launch_dkv<HD, false>(kv, P, s);
  if (e != hipSuccess) return e;
  if (parts) {
    parts->dq = S > 1 ? a.ws : a.dq;
    parts->sq = S;
    parts->dk = P > 1 ? kv.ws : a.dk;
    parts->dv = P > 1 ? kv.ws + P * total : a.dv;
    parts->pkv = P;
    parts->plane = total;
  } else if (P > 1) {
    hipLaunchKernelGGL(k_dkv_reduce, dim3((unsigned)std::min<int64_t>(cdiv(total / 4, 256), 8192)), dim3(256), 0, s,
                       a.ws, P, total, a.dk, a.dv);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- decode
//
// One query per (row, head) at position pos0 (n == 1), as in greedy generation: the window's
// keys and values are read once, so the kernel is bound by HBM.  A block takes 128 keys of
// the window (32 per wave) and the grid covers the window with S blocks per (row, head); the
// parts are merged by k_swa_dec_combine.  The HD/8 lanes of one key row each load a 16-byte piece
// (a wave load covers 64/(HD/8) whole rows), the piece's dot product with the query (bf16 pairs
// into fp32) is summed over those lanes with DPP moves, so every lane holds the scores of the
// keys whose value pieces it loads; softmax weights use the wave's maximum, and the four waves
// merge through LDS.

typedef __bf16 bf16x2d __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dec_dot8(const uint4& a, const uint4& b) {
  auto d2 = [](uint32_t x, uint32_t y, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2d, x), __builtin_bit_cast(bf16x2d, y), c, false);
  };
  return d2(a.w, b.w, d2(a.z, b.z, d2(a.y, b.y, d2(a.x, b.x, 0.f))));
}

// sum over the LPK (8 or 16) adjacent lanes of a key row: quad swaps, then the mirrored half
// rows and rows of 16 (each step pairs lanes whose partial sums cover disjoint lanes)
template <int LPK>
__device__ __forceinline__ float dec_sum_lanes(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)); // half-row mirror
  if constexpr (LPK == 16)
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));  // row mirror
  return v;
}

constexpr int DEC_KB = 128;  // keys per block (measured: 128 beats 256 and 64)

template <int HD>
__global__ __launch_bounds__(256) void k_swa_decode(AttnArgs a, int S) {
  constexpr int LPK = HD / 8;       // lanes per key row
  constexpr int KPR = 64 / LPK;     // keys per load round
  constexpr int ROUNDS = 32 / KPR;  // rounds per wave (32 keys)
  __shared__ float sm_o[4][HD];
  __shared__ float sm_m[4], sm_l[4];
  const int sp = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, dg = lane % LPK, sub = lane / LPK;
  const int64_t pos = a.pos0;
  const int64_t lo = pos - a.window + 1 > 0 ? pos - a.window + 1 : 0;
  const int64_t blo = lo + (int64_t)sp * DEC_KB;
  const int64_t bhi = blo + DEC_KB < pos + 1 ? blo + DEC_KB : pos + 1;  // this block's keys [blo, bhi)
  const int64_t bh = (int64_t)b * a.H + h;
  const uint4 qv = *(const uint4*)((const bf16*)a.q + bh * HD + dg * 8);
  const bf16* Kb = (const bf16*)a.kr + bh * a.R * HD + dg * 8;
  const bf16* Vb = (const bf16*)a.vr + bh * a.R * HD + dg * 8;
  const int64_t wlo = blo + 32 * w;  // this wave's first key
  const int s0 = (int)(wlo % a.R);    // its ring slot; 64 <= R, so one wrap at most
  uint4 kv[ROUNDS], vv[ROUNDS];
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i) {
    const int kk = i * KPR + sub;
    int slot = s0 + kk;
    if (slot >= a.R) slot -= a.R;
    // every slot is a valid ring row, so the loads are unconditional (a branch per load, with
    // zeros on the other path, made the wave wait for the loads in flight before issuing the
    // next); keys past the block are left out of the maximum and get weight 0, which needs only
    // that their slots hold finite values
    kv[i] = *(const uint4*)(Kb + (int64_t)slot * HD);
    vv[i] = *(const uint4*)(Vb + (int64_t)slot * HD);
  }
  __builtin_amdgcn_sched_barrier(0);  // all of the wave's loads go out before its first product
  float sc[ROUNDS];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i) {
    sc[i] = dec_sum_lanes<LPK>(dec_dot8(kv[i], qv));
    if (wlo + i * KPR + sub < bhi) mx = fmaxf(mx, sc[i]);
  }
#pragma unroll
  for (int o = LPK; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  const float sl2 = 1.4426950408889634f / sqrtf((float)HD);
  float l = 0.f, o8[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o8[j] = 0.f;
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i) {
    const float pw = wlo + i * KPR + sub < bhi ? exp2f((sc[i] - mx) * sl2) : 0.f;
    l += pw;
    const uint32_t u[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o8[2 * j] += pw * __uint_as_float(u[j] << 16);
      o8[2 * j + 1] += pw * __uint_as_float(u[j] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int o = LPK; o < 64; o <<= 1) {
    l += __shfl_xor(l, o, 64);
#pragma unroll
    for (int j = 0; j < 8; ++j) o8[j] += __shfl_xor(o8[j], o, 64);
  }
  if (sub == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) sm_o[w][dg * 8 + j] = o8[j];
  }
  if (lane == 0) {
    sm_m[w] = mx;
    sm_l[w] = l;
  }
  __syncthreads();
  if (threadIdx.x >= HD) return;
  const int d = threadIdx.x;
  float M = fmaxf(fmaxf(sm_m[0], sm_m[1]), fmaxf(sm_m[2], sm_m[3]));
  float L = 0.f, O = 0.f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float wt = sm_m[v] == -INFINITY ? 0.f : exp2f((sm_m[v] - M) * sl2);
    L += wt * sm_l[v];
    O += wt * sm_o[v][d];
  }
  if (S == 1) {
    ((bf16*)a.o)[(int64_t)b * a.H * HD + (int64_t)h * HD + d] = f2bf(O / L);
    if (a.lse && d == 0) a.lse[bh] = M * (sl2 * 0.6931471805599453f) + logf(L);
    return;
  }
  const int64_t plane = (int64_t)a.B * a.H;  // n == 1
  const int64_t row = (int64_t)sp * plane + bh;
  a.ws[row * HD + d] = O;
  if (d == 0) {
    float* pm = a.ws + (int64_t)S * plane * HD;
    pm[row] = M;
    pm[(int64_t)S * plane + row] = L;
  }
}

// merge of the S key-block parts of one (row, head): a block per (row, head); thread t takes parts
// t / (HD/8) + k * 256 / (HD/8) and dims (t % (HD/8)) * 8 ..+8, issues the loads of four parts at
// once and merges them against its own running maximum, so a window of up to 64 parts costs one
// round of loads; the threads' results are rescaled to the block maximum and summed through LDS
template <int HD>
__global__ __launch_bounds__(256) void k_swa_dec_combine(AttnArgs a, int S) {
  constexpr int DG = HD / 8, PS = 256 / DG;
  __shared__ float red[PS][HD];
  __shared__ float sh[16];
  const int64_t bh = blockIdx.x, plane = (int64_t)a.B * a.H;
  const float* pm = a.ws + (int64_t)S * plane * HD;
  const float* pl = pm + (int64_t)S * plane;
  const int t = threadIdx.x, dg = t % DG, ps = t / DG;
  const float sl2 = 1.4426950408889634f / sqrtf((float)HD);
  float mt = -INFINITY, lt = 0.f, o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = 0.f;
  for (int base = ps; base < S; base += 4 * PS) {
    float pmv[4], plv[4];
    float4 xa[4], xb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sp = base + u * PS;
      const int64_t row = (int64_t)(sp < S ? sp : 0) * plane + bh;
      // an absent part reads part 0 and gets maximum -inf (its weight is 0); written as an add so
      // the load stays unconditional (a select made it a branch that serialized the load groups)
      pmv[u] = pm[row] + (sp < S ? 0.f : -INFINITY);
      plv[u] = pl[row];
      xa[u] = *(const float4*)(a.ws + row * HD + dg * 8);
      xb[u] = *(const float4*)(a.ws + row * HD + dg * 8 + 4);
    }
    __builtin_amdgcn_sched_barrier(0);  // the group's loads all go out before the first wait
    float mn = mt;
#pragma unroll
    for (int u = 0; u < 4; ++u) mn = fmaxf(mn, pmv[u]);
    // (no early exit when every maximum is -inf: then nothing was accumulated, the scale and the
    // weights are 0 and the sums stay 0, and all loads of the group stay unconditional)
    const float sc = mt == -INFINITY ? 0.f : exp2f((mt - mn) * sl2);
    lt *= sc;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] *= sc;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = pmv[u] == -INFINITY ? 0.f : exp2f((pmv[u] - mn) * sl2);
      lt += w * plv[u];
      o[0] += w * xa[u].x; o[1] += w * xa[u].y; o[2] += w * xa[u].z; o[3] += w * xa[u].w;
      o[4] += w * xb[u].x; o[5] += w * xb[u].y; o[6] += w * xb[u].z; o[7] += w * xb[u].w;
    }
    mt = mn;
  }
  const float M = block_max(mt, sh);
  const float f = mt == -INFINITY ? 0.f : exp2f((mt - M) * sl2);
#pragma unroll
  for (int j = 0; j < 8; ++j) red[ps][dg * 8 + j] = o[j] * f;
  const float L = block_sum(dg == 0 ? lt * f : 0.f, sh);  // (its barriers also order the LDS writes above)
  if (t >= HD) return;
  float O = 0.f;
#pragma unroll
  for (int p = 0; p < PS; ++p) O += red[p][t];
  const int64_t b = bh / a.H, h = bh % a.H;
  ((bf16*)a.o)[b * a.H * HD + h * HD + t] = f2bf(O / L);
  if (a.lse && t == 0) a.lse[bh] = M * (sl2 * 0.6931471805599453f) + logf(L);
}

template <int HD>
hipError_t launch_decode(const AttnArgs& a, int S, hipStream_t s) {
  hipLaunchKernelGGL(k_swa_decode<HD>, dim3(S, a.H, a.B), dim3(256), 0, s, a, S);
  if (S > 1) hipLaunchKernelGGL(k_swa_dec_combine<HD>, dim3(a.B * a.H), dim3(256), 0, s, a, S);
  return hipGetLastError();
}

// blocks of DEC_KB keys over the window of the single query, or 0 when the decode kernel does not apply
int decode_splits(const AttnArgs& a) {
  if (a.n != 1 || (a.hd != 64 && a.hd != 128) || a.R < 64 || a.window < 1) return 0;
  if (((uintptr_t)a.q | (uintptr_t)a.kr | (uintptr_t)a.vr) & 15) return 0;
  const int64_t nkeys = std::min<int64_t>(a.window, a.pos0 + 1);
  const int S = (int)cdiv(nkeys, DEC_KB);
  if (S > 1 && (!a.ws || (int64_t)S * a.B * a.H * (a.hd + 2) > a.ws_floats)) return 0;
  return S;
}

}  // namespace

// key-range parts the forward would use for this call (1: single kernel)
int swa_fwd_mfma_splits(const AttnArgs& a) {
  if (const int S = decode_splits(a)) return S;
  if (a.n == 0 || a.R % 8 != 0 || (a.hd != 32 && a.hd != 64 && a.hd != 96 && a.hd != 128)) return 1;
  return fwd_splits(a);
}

int swa_decode_splits(const AttnArgs& a) { return decode_splits(a); }

int64_t swa_fwd_mfma_ws_need(const AttnArgs& a0) {
  if (a0.n == 0) return 0;
  AttnArgs a = a0;
  a.ws = reinterpret_cast<float*>(static_cast<uintptr_t>(256));  // any non-null workspace: only sizes are computed
  a.ws_floats = INT64_MAX;
  if (const int S = decode_splits(a)) return S > 1 ? (int64_t)S * a.B * a.H * (a.hd + 2) : 0;
  if (a.R % 8 != 0 || (a.hd != 32 && a.hd != 64 && a.hd != 96 && a.hd != 128)) return 0;
  const int S = fwd_splits(a);
  return S > 1 ? (int64_t)S * a.B * a.H * a.n * (a.hd + 2) : 0;
}

hipError_t swa_decode_blocks(const AttnArgs& a, int S, hipStream_t s) {
  if (S < 1 || S != decode_splits(a)) return hipErrorInvalidValue;
  if (a.hd == 128)
    hipLaunchKernelGGL(k_swa_decode<128>, dim3(S, a.H, a.B), dim3(256), 0, s, a, S);
  else
    hipLaunchKernelGGL(k_swa_decode<64>, dim3(S, a.H, a.B), dim3(256), 0, s, a, S);
  return hipGetLastError();
}

hipError_t swa_decode_merge(const AttnArgs& a, int S, hipStream_t s) {
  if (S <= 1) return hipSuccess;
  if (a.hd == 128)
    hipLaunchKernelGGL(k_swa_dec_combine<128>, dim3(a.B * a.H), dim3(256), 0, s, a, S);
  else
    hipLaunchKernelGGL(k_swa_dec_combine<64>, dim3(a.B * a.H), dim3(256), 0, s, a, S);
  return hipGetLastError();
}

hipError_t swa_fwd_mfma(const AttnArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  if (const int S = decode_splits(a)) return a.hd == 128 ? launch_decode<128>(a, S, s) : launch_decode<64>(a, S, s);
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

hipError_t swa_bwd_mfma(const AttnBwdArgs& a, hipStream_t s, AttnBwdParts* parts) {
  if (parts) *parts = AttnBwdParts{a.dq, 1, a.dk, a.dv, 1, (int64_t)a.B * a.n * a.H * a.hd};
  if (a.n == 0) return hipSuccess;
  if (a.window < a.n) return swa_bwd_simt<bf16>(a, s);
  switch (a.hd) {
    case 32: return launch_bwd<32>(a, s, parts);
    case 64: return launch_bwd<64>(a, s, parts);
    case 96: return launch_bwd<96>(a, s, parts);
    case 128: return launch_bwd<128>(a, s, parts);
    default: return swa_bwd_simt<bf16>(a, s);
  }
}
