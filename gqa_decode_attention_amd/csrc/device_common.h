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

// sum of squares of 8 packed 16-bit values added to acc, on the packed dot
// instructions (v_dot2_f32_bf16 / v_dot2_f32_f16: each product is exact in fp32)
template <int DT>
__device__ __forceinline__ float sumsq8(const uint4 v, float acc) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == ASR_BF16)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[i]), __builtin_bit_cast(bf16x2_t, w[i]), acc,
                                            false);
    else
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w[i]), __builtin_bit_cast(f16x2_t, w[i]), acc, false);
  }
  return acc;
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

// ---------------------------------------------------------------- FP8 (E4M3) codes
//
// gfx950's conversions use the E4M3 layout of the cache format (bias 7,
// largest finite 448, one NaN code per sign), rounding to nearest even; an
// encode of a magnitude past the largest finite value gives NaN, so values are
// clamped to +-448 first (saturating conversion).
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// 8 codes (two dwords, lowest byte first) -> 8 floats
__device__ __forceinline__ void unpack8_e4m3(uint32_t lo, uint32_t hi, float *f) {
  const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false), d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
  f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
}

__device__ __forceinline__ float sat_e4m3(float v) { return v != v ? v : fminf(fmaxf(v, -448.f), 448.f); }

// 4 floats -> 4 codes in one dword (lowest byte first)
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(a), sat_e4m3(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(c), sat_e4m3(d), w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// loads of data read exactly once (KV rows, weights): keep them out of the caches' way
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- MFMA (gfx950 v_mfma_f32_16x16x32_{bf16,f16})
//
// Lane layout (checked on the device against a CPU product):
//   A (16 x 32): lane l holds row l % 16, k = (l / 16) * 8 .. + 7
//   B (32 x 16): lane l holds column l % 16, k = (l / 16) * 8 .. + 7
//   C (16 x 16): lane l holds column l % 16, rows (l / 16) * 4 + j, j = 0..3
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

template <int DT>
__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4 a, const uint4 b, f32x4_t c) {
  if constexpr (DT == ASR_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  }
}

// fp32 -> two 16-bit terms, hi = rne(v), lo = rne(v - hi): hi + lo carries about
// twice the 16-bit precision (two-term split of an fp32 operand for 16-bit MFMA)
template <int DT>
__device__ __forceinline__ void split8(const float *f, uint4 &hi, uint4 &lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t h0 = rne16<DT>(f[2 * i]), h1 = rne16<DT>(f[2 * i + 1]);
    const uint16_t l0 = rne16<DT>(f[2 * i] - cvt16<DT>(h0)), l1 = rne16<DT>(f[2 * i + 1] - cvt16<DT>(h1));
    h[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    l[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// ---------------------------------------------------------------- data shared between workgroups
//
// Inside one dispatch, values that one workgroup writes and another reads go
// through agent-scope relaxed atomic accesses: the hardware performs them at
// the device-coherent level (no stale per-XCD L2 copy is read, no dirty copy
// is left behind), so no cache-wide write-back or invalidate is needed.  A
// writer waits for its stores to be performed (wait_mem) before it signals.
__device__ __forceinline__ void st_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int *p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_dev(const int *p) {
  return __hip_atomic_load(const_cast<int *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until every memory operation this thread issued has been performed
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

// 16-byte accesses with the same device-coherent cache policy (sc1) through a
// buffer resource: a workgroup-uniform base and `bytes` of range; a lane's
// offset past the range reads zeros and writes nothing.
constexpr int kCachePolicyCoherent = 16;   // sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float4 ld_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicyCoherent));
}
__device__ __forceinline__ void st_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r,
                                         off, 0, kCachePolicyCoherent);
}

// ---------------------------------------------------------------- wave reductions
//
// DPP lane permutations run in the vector ALU (no trip through the LDS
// crossbar): quad_perm swaps within 4 lanes, row_half_mirror reverses 8 lanes,
// row_mirror reverses 16 lanes.  Sums over the four 16-lane rows finish with
// readlane into scalar registers, which also broadcasts the result.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ __forceinline__ float readlane(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// sum over each aligned group of 8 lanes, result in all 8
__device__ __forceinline__ float sum8(float v) {
  v += dpp<kQuadSwap1>(v);
  v += dpp<kQuadSwap2>(v);
  v += dpp<kRowHalfMirror>(v);
  return v;
}
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp<kQuadSwap1>(v));
  v = fmaxf(v, dpp<kQuadSwap2>(v));
  v = fmaxf(v, dpp<kRowHalfMirror>(v));
  return v;
}
// sum over each 16-lane row, result in all 16
__device__ __forceinline__ float sum16(float v) {
  v = sum8(v);
  return v + dpp<kRowMirror>(v);
}
__device__ __forceinline__ float wave_sum(float v) {
  v = sum16(v);
  return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = max8(v);
  v = fmaxf(v, dpp<kRowMirror>(v));
  return fmaxf(fmaxf(readlane(v, 0), readlane(v, 16)), fmaxf(readlane(v, 32), readlane(v, 48)));
}
// Lane swaps of gfx950 (VALU, no LDS round trip).  permlane32_swap(a, b)
// returns (a[0..31] b[0..31], a[32..63] b[32..63]); permlane16_swap(a, b)
// returns (rows a0 b0 a2 b2, rows a1 b1 a3 b3) for 16-lane rows.  With
// (a, b) = (low value, high value) of every lane, the sum of the two results
// holds, in lanes with the MASK bit clear, low + low of lane l ^ MASK, and in
// the others high + high of lane l ^ MASK.
template <int MASK>
__device__ __forceinline__ float swap_sum(float lo, float hi) {
  static_assert(MASK == 16 || MASK == 32, "lane masks 16 and 32");
  const unsigned a = __builtin_bit_cast(unsigned, lo), b = __builtin_bit_cast(unsigned, hi);
  if constexpr (MASK == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
  }
}

// v of lane l ^ MASK (MASK 16 or 32)
template <int MASK>
__device__ __forceinline__ float xpart(float v) {
  static_assert(MASK == 16 || MASK == 32, "lane masks 16 and 32");
  const unsigned a = __builtin_bit_cast(unsigned, v);
  if constexpr (MASK == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
    return __builtin_bit_cast(float, (unsigned)((threadIdx.x & 32) ? r[0] : r[1]));
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
    return __builtin_bit_cast(float, (unsigned)((threadIdx.x & 16) ? r[0] : r[1]));
  }
}
__device__ __forceinline__ float xpartner32(float v) { return xpart<32>(v); }

// v plus v of lane l ^ MASK, in every lane
template <int MASK>
__device__ __forceinline__ float xsum(float v) {
  if constexpr (MASK == 8) return v + dpp<0x128>(v);   // row_ror:8 within 16-lane rows
  else return swap_sum<MASK>(v, v);
}

// sum over the 8 lanes {l & 7, (l & 7) + 8, ..., (l & 7) + 56}; the total lands in the
// lanes 8..15 of every 16-lane row (row_shr:8 adds lane i - 8 to lane i within a row)
__device__ __forceinline__ float sum_stride8(float v) {
  v += dpp<0x118>(v);
  v = xsum<16>(v);
  v = xsum<32>(v);
  return v;
}

// wave index in the workgroup, as a uniform (scalar) value
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }
__device__ __forceinline__ int lane_id() { return threadIdx.x % kWave; }

// Order one wave's LDS accesses across its lanes: the stores (or reads) before
// this point complete before the reads (or overwrites) after it by any lane of
// the wave.  The hardware runs a wave's LDS instructions in order, so this only
// keeps the compiler from moving accesses across it (it emits no instruction).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Reduce-scatter over the lanes l ^ MASK: lanes with the MASK bit clear keep
// the low half of the values, the others the high half, each summed with its
// partner's copy.
template <int N, int MASK>
__device__ __forceinline__ void rs_half(const float (&in)[N], float (&out)[N / 2]) {
  if constexpr (MASK == 8) {
    const bool hi = (lane_id() & MASK) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float keep = hi ? in[N / 2 + i] : in[i];
      const float send = hi ? in[i] : in[N / 2 + i];
      out[i] = keep + dpp<0x128>(send);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) out[i] = swap_sum<MASK>(in[i], in[N / 2 + i]);
  }
}

}  // namespace asr
