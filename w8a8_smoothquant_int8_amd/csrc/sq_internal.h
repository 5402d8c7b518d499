// Internal helpers for the libsq HIP kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/sq.h"

namespace sq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v8u16 __attribute__((ext_vector_type(8)));
// LDS address, the destination operand of the direct global-to-LDS load
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// 16-bit storage formats. bf16 -> fp32 is exact (the bf16 bits are the top
// half of the fp32 word); fp16 -> fp32 is exact. fp32 -> bf16/fp16 round to
// nearest, ties to even.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  _Float16 h = __builtin_bit_cast(_Float16, (unsigned short)b);
  return (float)h;
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);   // finite inputs only
  return u >> 16;
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  // Without the empty register barrier the compiler folds a preceding fp32
  // multiply into one mixed-precision FMA that rounds only once, straight to
  // fp16; the path's semantics are an fp32 rounding followed by an fp16 one.
  asm volatile("" : "+v"(f));
  _Float16 h = (_Float16)f;          // v_cvt_f16_f32: round to nearest even
  return (uint32_t)__builtin_bit_cast(unsigned short, h);
}

// Load 8 consecutive elements of dtype DT starting at p (16-byte aligned for
// 16-bit types; fp32 uses two 16-byte loads) and widen them to fp32.
template <int DT>
__device__ __forceinline__ void load8_f32(const void* p, float* out) {
  if constexpr (DT == SQ_F32) {
    const float4* q = (const float4*)p;
    float4 a = q[0], b = q[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  } else {
    uint4 v = *(const uint4*)p;
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == SQ_BF16) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      } else {
        out[2 * i] = f16_bits_to_f32(w[i] & 0xFFFFu);
        out[2 * i + 1] = f16_bits_to_f32(w[i] >> 16);
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ float load1_f32(const void* p) {
  if constexpr (DT == SQ_F32) return *(const float*)p;
  else if constexpr (DT == SQ_BF16) return bf16_bits_to_f32(*(const unsigned short*)p);
  else return f16_bits_to_f32(*(const unsigned short*)p);
}

template <int DT> struct DtSize { static constexpr int v = (DT == SQ_F32) ? 4 : 2; };

// ---------------------------------------------------------------------------
// Correctly rounded fp32 quotient through an fp64 reciprocal.
//
// For fp32 x and d (d > 0) whose quotient is in the normal fp32 range, and
// rd = RN64(1/d):  RN32(RN64(x * rd)) == RN32(x / d).
// Why: write x = X 2^a and d = D 2^c with integers |X| < 2^24, D < 2^24, and
// an fp32 rounding midpoint m = A 2^b with A odd and 2^24 <= A < 2^25. The
// odd part of A*D is at least A >= 2^24 while |X| < 2^24, so x != m*d; and
// x - m*d is a multiple of 2^min(a, b+c), hence at least that large. Both
// cases put the exact quotient x/d more than 2^-49 (relative) away from every
// midpoint. The fp64 product x * rd carries two roundings, a relative error
// below 2^-52, so it lies strictly between the same two midpoints as x/d and
// rounds to the same fp32 value. Cost: three VALU ops (widen, multiply,
// narrow) per element instead of the dozen of an IEEE fp32 division.
// Below the normal range (|x / d| < 2^-126) the midpoints are coarser and the
// quotient can sit exactly on one (x = d * (2j + 1) * 2^-150 with d of small
// odd part); then the two roundings may land one subnormal ulp (2^-149) off
// the IEEE quotient. Elsewhere in that range the result is still exact. A
// smoothed value that small changes a code only in a row whose largest
// smoothed value is itself subnormal.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float div_rn(float x, double rd) {
  return (float)((double)x * rd);
}

// RN64(1/d) for an fp32 d > 0 without the fp64 division sequence (Newton-
// Raphson reciprocal refinement): the hardware approximate reciprocal
// V_RCP_F64, then two steps r <- r + r (1 - d r), each one FMA for the
// residual and one for the update. Each step squares the relative error and
// adds one rounding: about 2^-24.4 -> 2^-48.7 -> 2^-53 on gfx950, measured
// over every fp32 mantissa at exponents -149 (denormals) to 127, where the
// result equalled the correctly rounded fp64 reciprocal in every case.
// div_rn needs only a relative error below 2^-50 (see there).
__device__ __forceinline__ double rcp_rn64(float d) {
  const double dd = (double)d;
  double r = __builtin_amdgcn_rcp(dd);
  r = __builtin_fma(r, __builtin_fma(-dd, r, 1.0), r);
  r = __builtin_fma(r, __builtin_fma(-dd, r, 1.0), r);
  return r;
}

// The INT8 code of a quotient q, clamp(rint(q), -127, 127) with rint rounding
// half to even, as the low byte of a 32-bit word, in one add: clamping first
// gives the same code (127 is an integer), and the sum t + 1.5 * 2^23 lies in
// [2^23, 2^24), where the fp32 numbers are the integers, so the add rounds t
// half to even; the low mantissa byte of the sum is then rint(t) in two's
// complement (1.5 * 2^23 - 2^23 = 2^22 adds no low bits).
__device__ __forceinline__ uint32_t code_word(float q) {
  const float t = __builtin_fminf(__builtin_fmaxf(q, -127.0f), 127.0f);
  return __float_as_uint(t + 12582912.0f);
}

// The same code as an int: round half to even, clamp to [-127, 127].
__device__ __forceinline__ int quant_code(float q) {
  float r = __builtin_rintf(q);
  r = __builtin_fminf(__builtin_fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
         ((uint32_t)(d & 0xFF) << 24);
}

// Four code words (low bytes) into one packed word, first in the low byte.
__device__ __forceinline__ uint32_t pack4_codes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return (a & 0xFFu) | ((b & 0xFFu) << 8) | ((c & 0xFFu) << 16) | (d << 24);
}

// 1 if the code of q clamps: the rounded value lies beyond +-127.
__device__ __forceinline__ int clips(float q) {
  return __builtin_fabsf(__builtin_rintf(q)) > 127.0f ? 1 : 0;
}

// Max over a wave64 (all lanes get the result). Max is exact and order-free.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Sum over a wave64 (all lanes get the result).
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Atomic max for non-negative floats through their bit patterns (the order of
// non-negative IEEE floats equals the order of their bit patterns).
__device__ __forceinline__ void atomic_max_nonneg(float* p, float v) {
  atomicMax((unsigned int*)p, __float_as_uint(v));
}


// Widen one chunk of 8 elements (one 16-byte word for 16-bit types, two for
// fp32) to fp32.
template <int DT>
__device__ __forceinline__ void widen8(const uint4* w, float* out) {
  if constexpr (DT == SQ_F32) {
    out[0] = __uint_as_float(w[0].x); out[1] = __uint_as_float(w[0].y);
    out[2] = __uint_as_float(w[0].z); out[3] = __uint_as_float(w[0].w);
    out[4] = __uint_as_float(w[1].x); out[5] = __uint_as_float(w[1].y);
    out[6] = __uint_as_float(w[1].z); out[7] = __uint_as_float(w[1].w);
  } else {
    uint32_t u[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == SQ_BF16) {
        out[2 * i] = __uint_as_float(u[i] << 16);
        out[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
      } else {
        out[2 * i] = f16_bits_to_f32(u[i] & 0xFFFFu);
        out[2 * i + 1] = f16_bits_to_f32(u[i] >> 16);
      }
    }
  }
}

// Sum over a wave64, fp64 (all lanes get the result; the butterfly order is
// fixed, so the result is the same on every run).
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Resident blocks of one kernel on the current device (occupancy x CUs),
// cached per kernel instantiation and device. The cache entries are atomics:
// calls from several host threads may fill one at the same time, each with
// the same value.
template <typename Tag>
inline int64_t resident_blocks(const void* f, int T) {
  static std::atomic<int> per_cu[16];
  static std::atomic<int> cus[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
  int b = per_cu[dev].load(std::memory_order_relaxed);
  int n = cus[dev].load(std::memory_order_relaxed);
  if (b == 0 || n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, f, T, 0) != hipSuccess || b <= 0) b = 1;
    cus[dev].store(n, std::memory_order_relaxed);
    per_cu[dev].store(b, std::memory_order_relaxed);
  }
  return (int64_t)b * n;
}

}  // namespace sq

// Host-side launch helpers.
#define SQ_LAUNCH_CHECK()                               \
  do {                                                  \
    if (hipGetLastError() != hipSuccess) return SQ_ERR_HIP; \
  } while (0)
