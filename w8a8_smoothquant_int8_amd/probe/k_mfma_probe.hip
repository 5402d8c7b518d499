// INT8 matrix-core rate probe (see include/sq_probe.h): MFMAs from registers
// only, at the INT8 GEMM's occupancy, with the shader clock it runs at.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sq_probe.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;   // 8 waves: two per SIMD

template <int MODE>
__global__ void __launch_bounds__(kThreads, 2)
k_mfma_probe(const int32_t* __restrict__ rnd, int iters, uint64_t* __restrict__ clk,
             int32_t* __restrict__ sink) {
  v4i a[8], b[8];
  const int tid = blockIdx.x * kThreads + threadIdx.x;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    if constexpr (MODE == 0) {
      a[q] = v4i{0x05030201, 0x0b070503, 0x110d0b07, 0x1d17130d};
      b[q] = a[q];
    } else {
      a[q] = *(const v4i*)(rnd + ((int64_t)tid * 64 + 4 * q));
      b[q] = *(const v4i*)(rnd + ((int64_t)tid * 64 + 32 + 4 * q));
    }
  }
  v16i acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = v16i{};
  uint64_t t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
    // 8 rounds of 8 MFMAs: accumulator q takes a[q] with b[(q + u) % 8], so
    // the operand pair changes from one instruction to the next
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q)
        acc[q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b[(q + u) & 7], a[q], acc[q], 0, 0, 0);
  }
  if (threadIdx.x == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
  int32_t s = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[q][e];
  sink[tid] = s;
}

}  // namespace

extern "C" int sq_probe_mfma_i8(int mode, int blocks, int iters, const int32_t* rnd, uint64_t* clk,
                                int32_t* sink, void* stream) {
  if (blocks < 1 || iters < 1 || (mode != 0 && mode != 1) || clk == nullptr || sink == nullptr ||
      (mode == 1 && rnd == nullptr))
    return -1;
  hipStream_t st = (hipStream_t)stream;
  if (mode == 0)
    k_mfma_probe<0><<<blocks, kThreads, 0, st>>>(rnd, iters, clk, sink);
  else
    k_mfma_probe<1><<<blocks, kThreads, 0, st>>>(rnd, iters, clk, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
