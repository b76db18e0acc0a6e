// Shared device/host helpers of the HIP path (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

// bf16 storage: raw 16-bit pattern, converted explicitly (round to nearest even).
struct bf16 {
  uint16_t x;
};

__host__ __device__ __forceinline__ float bf2f(bf16 v) {
  uint32_t u = (uint32_t)v.x << 16;
  float f;
  __builtin_memcpy(&f, &u, 4);
  return f;
}

__host__ __device__ __forceinline__ bf16 f2bf(float f) {
#if defined(__HIP_DEVICE_COMPILE__)
  // gfx950 converts in hardware (v_cvt_pk_bf16_f32, round to nearest even, NaN stays NaN)
  return bf16{__builtin_bit_cast(uint16_t, (__bf16)f)};
#else
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return bf16{(uint16_t)((u >> 16) | 0x40)};  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return bf16{(uint16_t)(u >> 16)};
#endif
}

// two floats -> packed bf16 pair (a in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16pair(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T>
__host__ __device__ __forceinline__ float to_f(const T& v);
template <>
__host__ __device__ __forceinline__ float to_f<float>(const float& v) {
  return v;
}
template <>
__host__ __device__ __forceinline__ float to_f<bf16>(const bf16& v) {
  return bf2f(v);
}

template <typename T>
__host__ __device__ __forceinline__ T from_f(float f);
template <>
__host__ __device__ __forceinline__ float from_f<float>(float f) {
  return f;
}
template <>
__host__ __device__ __forceinline__ bf16 from_f<bf16>(float f) {
  return f2bf(f);
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// block-wide sum for blockDim.x a multiple of 64 (<= 1024); sh holds >= 16 floats
__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = warp_sum(v);
  int w = threadIdx.x >> 6, l = threadIdx.x & 63, nw = blockDim.x >> 6;
  __syncthreads();
  if (l == 0) sh[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += sh[i];
  return t;
}

__device__ __forceinline__ float block_max(float v, float* sh) {
  v = warp_max(v);
  int w = threadIdx.x >> 6, l = threadIdx.x & 63, nw = blockDim.x >> 6;
  __syncthreads();
  if (l == 0) sh[w] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int i = 0; i < nw; ++i) t = fmaxf(t, sh[i]);
  return t;
}

static inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

// LDS pointer for global_load_lds (lane L of a wave writes 16 bytes at the wave's LDS
// address + 16 L)
#define LDSP(p) ((void __attribute__((address_space(3)))*)(p))
// raw buffer resource over `bytes` bytes from p (gfx9 data-format word): a buffer load takes
// a per-lane byte offset and a wave-uniform one, so a loop that advances along K moves only
// the scalar offset; loads past `bytes` return zero instead of touching memory
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes per lane from byte offset voff + soff of the buffer into LDS at the wave's
// address lds + 16 * lane (like global_load_lds)
__device__ __forceinline__ void buf_lds16(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDSP(lds), 16, voff, soff, 0, 0);
}
// wait until at most n vector-memory operations are outstanding and all LDS operations are
// done (gfx9 s_waitcnt: vmcnt in bits 15:14 and 3:0, expcnt 6:4, lgkmcnt 11:8)
#define WAIT_VM_LDS(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4))
// wait until at most n vector-memory operations are outstanding, LDS operations untouched
// (direct-to-LDS loads count as vector-memory operations until their data is in LDS)
#define WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
