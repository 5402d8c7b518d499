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
// One column-max job: X [M, K] (row stride ldx_bytes) into out [K], split
// into 512-column strips x row slices of rows_per_slice rows.
struct ColmaxJob {
  const char* X;
  int64_t M, K, ldx_bytes;
  int rows_per_slice, strips;
  float* out;
};

template <int DT>
__device__ __forceinline__ void colmax_block(const ColmaxJob& j, int64_t strip, int64_t slice) {
  const char* __restrict__ X = j.X;
  const int64_t M = j.M, K = j.K, ldx_bytes = j.ldx_bytes;
  const int rows_per_slice = j.rows_per_slice;
  float* __restrict__ out = j.out;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t col0 = strip * 512 + lane * 8;
  const int64_t r0 = slice * rows_per_slice;
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
    const int64_t k = strip * 512 + c;
    if (k < K && r0 < r1) atomic_max_nonneg(out + k, m);
  }
}

// One job: grid (strips, slices).
template <int DT>
__global__ void __launch_bounds__(kColThreads) k_colmax(ColmaxJob j) {
  colmax_block<DT>(j, blockIdx.x, blockIdx.y);
}

// Two jobs in one launch (same input dtype): 1-D grid, the first job's
// strips x slices blocks, then the second's.
template <int DT>
__global__ void __launch_bounds__(kColThreads) k_colmax2(ColmaxJob a, ColmaxJob b) {
  const int64_t na = (int64_t)a.strips * ((a.M + a.rows_per_slice - 1) / a.rows_per_slice);
  const int64_t id = blockIdx.x;
  if (id < na) colmax_block<DT>(a, id % a.strips, id / a.strips);
  else colmax_block<DT>(b, (id - na) % b.strips, (id - na) / b.strips);
}

// out1[0:n1] = v, out2[0:n2] = v in one launch.
__global__ void k_fill2_f32(float* __restrict__ p1, int64_t n1, float* __restrict__ p2, int64_t n2,
                            float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n1) p1[i] = v;
  else if (i - n1 < n2) p2[i - n1] = v;
}

__global__ void k_fill_f32(float* __restrict__ p, int64_t n, float v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// s[k] = fp32(max(a^alpha / w^(1 - alpha), 1e-5)) with a = max(act_max[k], 1e-5),
// w = max(w_max[k], 1e-5), all in fp64. w_max may be s itself (in place).
// sqrt_form: alpha == 0.5, where both powers are square roots (correctly
// rounded in fp64), so the result is the correctly rounded quotient.
__global__ void k_smooth_scale(const float* __restrict__ act_max, const float* w_max, float* s,
                               int64_t K, double alpha, double one_minus_alpha, int sqrt_form) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  const double lo = 1e-5;
  double a = (double)act_max[k];
  double w = (double)w_max[k];
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
// Strips of 512 columns x row slices: about 1024 blocks, at least 16 rows
// per block (4 per wave, whose loads the unrolled loop keeps in flight
// together), at most 65535 row slices.
static ColmaxJob colmax_job(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, float* out) {
  const int64_t strips = (K + 511) / 512;
  int64_t slices = (1024 + strips - 1) / strips;
  int64_t rows = (M + slices - 1) / slices;
  if (rows < 16) rows = 16;
  if ((M + rows - 1) / rows > 65535) rows = (M + 65534) / 65535;
  const int esz = xt == SQ_F32 ? 4 : 2;
  return ColmaxJob{(const char*)X, M, K, ldx * esz, (int)rows, (int)strips, out};
}

int launch_colmax(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, float* out,
                  hipStream_t st) {
  if (M == 0) return SQ_OK;
  const ColmaxJob j = colmax_job(X, xt, M, K, ldx, out);
  dim3 grid((unsigned)j.strips, (unsigned)((M + j.rows_per_slice - 1) / j.rows_per_slice));
  switch (xt) {
    case SQ_F32: k_colmax<SQ_F32><<<grid, kColThreads, 0, st>>>(j); break;
    case SQ_F16: k_colmax<SQ_F16><<<grid, kColThreads, 0, st>>>(j); break;
    default:     k_colmax<SQ_BF16><<<grid, kColThreads, 0, st>>>(j); break;
  }
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

// Two column-max jobs in one launch when their inputs share a dtype (else
// two launches).
int launch_colmax2(const void* X1, int xt1, int64_t M1, int64_t K1, int64_t ld1, float* out1,
                   const void* X2, int xt2, int64_t M2, int64_t K2, int64_t ld2, float* out2,
                   hipStream_t st) {
  if (M1 == 0 || M2 == 0 || xt1 != xt2) {
    int rc = launch_colmax(X1, xt1, M1, K1, ld1, out1, st);
    if (rc != SQ_OK) return rc;
    return launch_colmax(X2, xt2, M2, K2, ld2, out2, st);
  }
  const ColmaxJob a = colmax_job(X1, xt1, M1, K1, ld1, out1);
  const ColmaxJob b = colmax_job(X2, xt2, M2, K2, ld2, out2);
  const int64_t blocks = (int64_t)a.strips * ((M1 + a.rows_per_slice - 1) / a.rows_per_slice) +
                         (int64_t)b.strips * ((M2 + b.rows_per_slice - 1) / b.rows_per_slice);
  switch (xt1) {
    case SQ_F32: k_colmax2<SQ_F32><<<(unsigned)blocks, kColThreads, 0, st>>>(a, b); break;
    case SQ_F16: k_colmax2<SQ_F16><<<(unsigned)blocks, kColThreads, 0, st>>>(a, b); break;
    default:     k_colmax2<SQ_BF16><<<(unsigned)blocks, kColThreads, 0, st>>>(a, b); break;
  }
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

int launch_fill2(float* p1, int64_t n1, float* p2, int64_t n2, float v, hipStream_t st) {
  const int64_t n = n1 + n2;
  k_fill2_f32<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p1, n1, p2, n2, v);
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

int launch_fill(float* p, int64_t n, float v, hipStream_t st) {
  k_fill_f32<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n, v);
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

// s from act_max and w_max (w_max may equal s).
int launch_smooth_scale_from(const float* act_max, const float* w_max, float* s, int64_t K,
                             double alpha, hipStream_t st) {
  const int sqrt_form = alpha == 0.5;
  k_smooth_scale<<<(unsigned)((K + 255) / 256), 256, 0, st>>>(act_max, w_max, s, K, alpha,
                                                               1.0 - alpha, sqrt_form);
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

int launch_smooth_scale(const float* act_max, float* s_inout, int64_t K, double alpha,
                        hipStream_t st) {
  return launch_smooth_scale_from(act_max, s_inout, s_inout, K, alpha, st);
}

int launch_static_scale(const float* act_max, const float* s, int64_t K, float* a_scale,
                        hipStream_t st) {
  k_static_scale<<<1, 1024, 0, st>>>(act_max, s, K, a_scale);
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

}  // namespace sq
