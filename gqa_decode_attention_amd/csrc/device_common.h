// Device helpers for the gfx950 attention-block kernels: 16-bit <-> fp32
// conversion, 16-byte vector loads, wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "asr_attn.h"

namespace asr {

constexpr int kWave = 64;

// ---------------------------------------------------------------- conversions

template <int DT>
__device__ __forceinline__ float cvt16(uint32_t u16) {
  if constexpr (DT == ASR_BF16) {
    return __uint_as_float(u16 << 16);
  } else {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u16)));
  }
}

// the two 16-bit values packed in a 32-bit word (low half first)
template <int DT>
__device__ __forceinline__ void cvt16x2(uint32_t w, float &lo, float &hi) {
  if constexpr (DT == ASR_BF16) {
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xffff0000u);
  } else {
    lo = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
    hi = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
  }
}

// 8 packed 16-bit values -> 8 floats
template <int DT>
__device__ __forceinline__ void unpack8(const uint4 v, float *f) {
  cvt16x2<DT>(v.x, f[0], f[1]);
  cvt16x2<DT>(v.y, f[2], f[3]);
  cvt16x2<DT>(v.z, f[4], f[5]);
  cvt16x2<DT>(v.w, f[6], f[7]);
}

// fp32 -> 16-bit, round to nearest even (hardware conversions, no flush of subnormals)
template <int DT>
__device__ __forceinline__ uint16_t rne16(float f) {
  if constexpr (DT == ASR_BF16) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
  } else {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
  }
}

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// loads of data read exactly once (KV rows, weights): keep them out of the caches' way
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- wave reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// sum over aligned groups of G consecutive lanes (G a power of two <= 64)
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }
__device__ __forceinline__ int lane_id() { return threadIdx.x % kWave; }

}  // namespace asr
