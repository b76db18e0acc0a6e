// Kernel-level C entry points (include/ttt_kernels.h).
#include <atomic>

#include "kernels.h"
#include "ttt.h"
#include "ttt_kernels.h"

static int code(hipError_t e) { return e == hipSuccess ? TTT_OK : (e == hipErrorInvalidValue ? TTT_EINVAL : TTT_EDEVICE); }

extern "C" int tttk_gemm(int dtype, const void* A, int64_t lda, const void* B, int64_t ldb, float* C, int64_t ldc,
                         int32_t M, int32_t N, int32_t K, float* ws, int64_t ws_floats, void* stream) {
  if (!A || !B || !C || M < 0 || N < 0 || K < 1 || lda < K || ldb < K || ldc < N || ws_floats < 0) return TTT_EINVAL;
  GemmArgs g;
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.M = M;
  g.N = N;
  g.K = K;
  g.e.kind = EPI_F32;
  g.e.c = C;
  g.e.ldc = ldc;
  g.ws = ws;
  g.ws_floats = ws ? ws_floats : 0;
  if (dtype == TTT_F32) return code(gemm_simt_f32(g, (hipStream_t)stream));
  if (dtype == TTT_BF16) return code(gemm_mfma_bf16(g, (hipStream_t)stream));
  return TTT_EINVAL;
}

extern "C" int tttk_swa_fwd(int dtype, const void* q, const void* kr, const void* vr, const void* vtr, void* o,
                            float* lse, int32_t B, int32_t H, int32_t hd, int32_t n, int32_t R, int32_t window,
                            int64_t pos0, float* ws, int64_t ws_floats, void* stream) {
  if (!q || !kr || !vr || !vtr || !o || B < 1 || H < 1 || hd < 2 || hd % 2 || hd > 128 || n < 0 || window < 1 ||
      pos0 < 0 || R < window + n - 1)
    return TTT_EINVAL;
  AttnArgs a{q, kr, vr, vtr, o, lse, B, H, hd, n, R, window, pos0, ws, ws ? ws_floats : 0};
  if (dtype == TTT_F32) return code(swa_fwd_simt<float>(a, (hipStream_t)stream));
  if (dtype == TTT_BF16) return code(swa_fwd_mfma(a, (hipStream_t)stream));
  return TTT_EINVAL;
}

// ------------------------------------------------------------ no-allocation variant
// The split key-range parts of tttk_swa_fwd_noalloc live in this array (one copy per device,
// loaded with the code object and kept until the process ends).  Host code never uses the
// array's name as an address: the device address comes from hipGetSymbolAddress, once per
// device, and is what the kernels receive.
static __device__ __align__(256) float scratch[TTTK_NOALLOC_SCRATCH_FLOATS];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch[kMaxDevices];

// Nothing in the array needs clearing between calls: every part the merge kernels read is
// written by the same call's split kernel first.
// device address of `scratch` on the current device (looked up on the first call there)
hipError_t scratch_ptr(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!addr) return hipErrorInvalidSymbol;
    p = static_cast<float*>(addr);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}
}  // namespace

extern "C" int tttk_swa_fwd_noalloc(int dtype, const void* q, const void* kr, const void* vr, const void* vtr,
                                    void* o, float* lse, int32_t B, int32_t H, int32_t hd, int32_t n, int32_t R,
                                    int32_t window, int64_t pos0, void* stream) {
  if (!q || !kr || !vr || !vtr || !o || B < 1 || H < 1 || hd < 2 || hd % 2 || hd > 128 || n < 0 || window < 1 ||
      pos0 < 0 || R < window + n - 1)
    return TTT_EINVAL;
  if (dtype == TTT_F32) {  // the fp32 kernels take no workspace
    AttnArgs a{q, kr, vr, vtr, o, lse, B, H, hd, n, R, window, pos0, nullptr, 0};
    return code(swa_fwd_simt<float>(a, (hipStream_t)stream));
  }
  if (dtype != TTT_BF16) return TTT_EINVAL;
  float* ws = nullptr;
  if (scratch_ptr(&ws) != hipSuccess) return TTT_EDEVICE;
  AttnArgs a{q, kr, vr, vtr, o, lse, B, H, hd, n, R, window, pos0, ws, TTTK_NOALLOC_SCRATCH_FLOATS};
  // the split this call would take must fit the static array: no smaller split is substituted
  if (swa_fwd_mfma_ws_need(a) > TTTK_NOALLOC_SCRATCH_FLOATS) return TTT_EINVAL;
  return code(swa_fwd_mfma(a, (hipStream_t)stream));
}

extern "C" int tttk_swa_bwd(int dtype, const void* q, const void* qt, const void* kr, const void* vr, const void* vtr,
                            const void* ktr, const void* o, const void* dout, const float* lse, float* dvec, float* dq,
                            float* dk, float* dv, void* dot, int32_t B, int32_t H, int32_t hd, int32_t n, int32_t R,
                            int32_t window, int64_t pos0, float* ws, int64_t ws_floats, void* stream) {
  if (!q || !qt || !kr || !vr || !vtr || !o || !dout || !lse || !dvec || !dq || !dk || !dv || B < 1 || H < 1 ||
      hd < 2 || hd % 2 || hd > 128 || n < 0 || window < n || pos0 < 0 || R < window + n - 1)
    return TTT_EINVAL;
  AttnBwdArgs a{q, qt, kr, vr, vtr, ktr, o, dout, lse, dvec, dq, dk, dv, dot, B, H, hd, n, R, window, pos0, ws,
                ws ? ws_floats : 0};
  if (dtype == TTT_F32) return code(swa_bwd_simt<float>(a, (hipStream_t)stream));
  if (dtype == TTT_BF16) return code(swa_bwd_mfma(a, (hipStream_t)stream));
  return TTT_EINVAL;
}
