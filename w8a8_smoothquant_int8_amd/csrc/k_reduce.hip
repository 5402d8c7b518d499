// Column reductions and per-channel scale math:
//  - running per-channel absmax of activations (calibration, [SQ] Step 4) and
//    of weights (w_max in [SQ] Step 3) - the same column-max kernel;
//  - the smoothing scale s ([SQ] Step 3, the sketch's smooth_layer);
//  - the static per-tensor activation scale ([SQ] Step 6, static variant).
//
// All three are HBM-bound or tiny. The column max reads every element once
// with 16-byte loads; a block covers a strip of columns and a slice of rows,
// reduces in registers and LDS, and merges into the output with an atomic max
// on the float bit pattern (exact and independent of the merge order).
#include "sq_internal.h"

namespace sq {

constexpr int kColThreads = 256;            // 4 waves
constexpr int kColWavesPerBlock = 4;

// out[k] = max(out[k], max over rows of |X[m, k]|), rows [row0, row0+rows).
// Block: 4 waves; every lane owns 8 consecutive columns (one 16-byte load for
// 16-bit types), so a wave covers 512 columns; the 4 waves walk interleaved
// rows of the same strip. Grid: (column strips, row slices).
template <int DT>
__global__ void __launch_bounds__(kColThreads)
k_colmax(const char* __restrict__ X, int64_t M, int64_t K, int64_t ldx_bytes, int rows_per_slice,
         float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t col0 = (int64_t)blockIdx.x * 512 + lane * 8;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_slice;
  const int64_t r1 = r0 + rows_per_slice < M ? r0 + rows_per_slice : M;
  float mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (col0 < K) {
#pragma unroll 4
    for (int64_t r = r0 + wave; r < r1; r += kColWavesPerBlock) {
      float v[8];
      load8_f32<DT>(X + r * ldx_bytes + col0 * DtSize<DT>::v, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) mx[i] = __builtin_fmaxf(mx[i], __builtin_fabsf(v[i]));
    }
  }
  __shared__ float red[kColWavesPerBlock][512];
#pragma unroll
  for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = mx[i];
  __syncthreads();
  for (int c = threadIdx.x; c < 512; c += kColThreads) {
    float m = red[0][c];
#pragma unroll
    for (int w = 1; w < kColWavesPerBlock; ++w) m = __builtin_fmaxf(m, red[w][c]);
    const int64_t k = (int64_t)blockIdx.x * 512 + c;
    if (k < K && r0 < r1) atomic_max_nonneg(out + k, m);
  }
}

__global__ void k_fill_f32(float* __restrict__ p, int64_t n, float v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// s[k] = fp32(max(a^alpha / w^(1 - alpha), 1e-5)) with a = max(act_max[k], 1e-5),
// w = max(w_max[k], 1e-5), all in fp64. On entry s holds w_max (in place).
// sqrt_form: alpha == 0.5, where both powers are square roots (correctly
// rounded in fp64), so the result is the correctly rounded quotient.
__global__ void k_smooth_scale(const float* __restrict__ act_max, float* __restrict__ s, int64_t K,
                               double alpha, double one_minus_alpha, int sqrt_form) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  const double lo = 1e-5;
  double a = (double)act_max[k];
  double w = (double)s[k];
  a = a > lo ? a : lo;
  w = w > lo ? w : lo;
  double v = sqrt_form ? __builtin_sqrt(a) / __builtin_sqrt(w) : pow(a, alpha) / pow(w, one_minus_alpha);
  v = v > lo ? v : lo;
  s[k] = (float)v;
}

// a_scale[0] = max_k fp32(act_max[k] / s[k]) / 127 - one block.
__global__ void __launch_bounds__(1024)
k_static_scale(const float* __restrict__ act_max, const float* __restrict__ s, int64_t K,
               float* __restrict__ a_scale) {
  float m = 0.0f;
  for (int64_t k = threadIdx.x; k < K; k += blockDim.x) {
    float v = s ? act_max[k] / s[k] : act_max[k];   // IEEE fp32 division
    m = __builtin_fmaxf(m, v);
  }
  m = wave_max(m);
  __shared__ float red[16];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = __builtin_fmaxf(r, red[w]);
    a_scale[0] = r / 127.0f;
  }
}

// ---------------------------------------------------------------------------
// Host launchers (called from sq_api.hip after validation).
// ---------------------------------------------------------------------------
int launch_colmax(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, float* out,
                  hipStream_t st) {
  if (M == 0) return SQ_OK;
  const int64_t strips = (K + 511) / 512;
  // About 1024 blocks, at least 16 rows per block (4 per wave, whose loads
  // the unrolled loop keeps in flight together), at most 65535 row slices.
  int64_t slices = (1024 + strips - 1) / strips;
  int64_t rows = (M + slices - 1) / slices;
  if (rows < 16) rows = 16;
  if ((M + rows - 1) / rows > 65535) rows = (M + 65534) / 65535;
  slices = (M + rows - 1) / rows;
  dim3 grid((unsigned)strips, (unsigned)slices);
  const int esz = xt == SQ_F32 ? 4 : 2;
  const char* x = (const char*)X;
  switch (xt) {
    case SQ_F32: k_colmax<SQ_F32><<<grid, kColThreads, 0, st>>>(x, M, K, ldx * esz, (int)rows, out); break;
    case SQ_F16: k_colmax<SQ_F16><<<grid, kColThreads, 0, st>>>(x, M, K, ldx * esz, (int)rows, out); break;
    default:     k_colmax<SQ_BF16><<<grid, kColThreads, 0, st>>>(x, M, K, ldx * esz, (int)rows, out); break;
  }
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

int launch_fill(float* p, int64_t n, float v, hipStream_t st) {
  k_fill_f32<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n, v);
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

int launch_smooth_scale(const float* act_max, float* s_inout, int64_t K, double alpha,
                        hipStream_t st) {
  const int sqrt_form = alpha == 0.5;
  k_smooth_scale<<<(unsigned)((K + 255) / 256), 256, 0, st>>>(act_max, s_inout, K, alpha,
                                                               1.0 - alpha, sqrt_form);
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

int launch_static_scale(const float* act_max, const float* s, int64_t K, float* a_scale,
                        hipStream_t st) {
  k_static_scale<<<1, 1024, 0, st>>>(act_max, s, K, a_scale);
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

}  // namespace sq
