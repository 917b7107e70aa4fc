// Device helpers shared by the verify-step kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

constexpr float kLog2e = 1.4426950408889634f;

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// The device's own base-2 exponential (v_exp_f32).
__device__ __forceinline__ float exp2_dev(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte vector loads of logits, widened to float.
template <typename T> struct Vec16;

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <> struct Vec16<uint16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void widen(const u32x4_t r, float (&f)[8]) {
    f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x);
    f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
    f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z);
    f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
  }
  __device__ __forceinline__ static void load(const uint16_t* p, float (&f)[8]) {
    widen(*reinterpret_cast<const u32x4_t*>(p), f);
  }
  // Nontemporal: data streamed once (keeps it from displacing reused lines).
  __device__ __forceinline__ static void load_nt(const uint16_t* p, float (&f)[8]) {
    widen(__builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)), f);
  }
  __device__ __forceinline__ static float one(const uint16_t* p) { return bf16_to_f32(*p); }
};

template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void load(const float* p, float (&f)[4]) {
    const float4 r = *reinterpret_cast<const float4*>(p);
    f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w;
  }
  __device__ __forceinline__ static void load_nt(const float* p, float (&f)[4]) {
    const f32x4_t r = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w;
  }
  __device__ __forceinline__ static float one(const float* p) { return *p; }
};

// (max, sum of 2^(y - max)) pairs: merge of two partial softmax statistics.
// Symmetric in its arguments bit for bit, so butterfly reductions leave every
// lane with the same value.
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  const float a = (m == mn) ? s : s * exp2_dev(m - mn);
  const float b = (m2 == mn) ? s2 : s2 * exp2_dev(m2 - mn);
  m = mn;
  s = a + b;
}

// (value, index) argmax merge with the lowest index winning ties; idx ==
// INT32_MAX marks "no element".
__device__ __forceinline__ void am_merge(float& v, int& i, float v2, int i2) {
  const bool take = (i == INT32_MAX) ||
                    (i2 != INT32_MAX && (v2 > v || (v2 == v && i2 < i)));
  if (take) { v = v2; i = i2; }
}

__device__ __forceinline__ void wave_ms_reduce(float& m, float& s) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float s2 = __shfl_xor(s, off, 64);
    ms_merge(m, s, m2, s2);
  }
}

__device__ __forceinline__ void wave_am_reduce(float& v, int& i) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float v2 = __shfl_xor(v, off, 64);
    const int i2 = __shfl_xor(i, off, 64);
    am_merge(v, i, v2, i2);
  }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// The append mode of the window attention: rows 0 .. N - 1 of k_new / v_new
// ([B, N, Hkv, D]) into cache positions kv_len[b] + j (kv_commit.hip).
hipError_t launch_window_store(void* kc, void* vc, const int32_t* bt, const int32_t* kv_len,
                               const void* kn, const void* vn, int B, int N, int Hkv, int D,
                               int num_blocks, int mbps, int dtype, hipStream_t st);

// Compute units of the current device (cached per device).
static inline int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cached[dev] = n;      // every caller stores the same value
  return n;
}

}  // namespace sv
