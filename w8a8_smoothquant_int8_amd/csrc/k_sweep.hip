// Per-layer choice of the migration strength alpha ("SmoothQuant" explainer,
// "Calibration in practice": the best alpha differs between layers and is
// found by measuring, on calibration data, how far the quantized layer's
// output lands from the unquantized one).
//
// The sweep reuses the path's own kernels for everything that depends on
// alpha (smoothing scale, fold + weight quant, activation quant, INT8 GEMM
// with an fp32 dequant epilogue). This file adds the two pieces it needs on
// top:
//  - k_ref_gemm: the unquantized output Y_ref = X W^T in fp64 with exact
//    products, computed once per sweep on the fp64 matrix instruction.
//  - k_err_partial / k_err_final: sum (Yq - Y_ref)^2 and sum Y_ref^2 in
//    fp64, in a fixed order (block partials, then one block), so the result
//    is the same on every run.
#include "sq_internal.h"

namespace sq {

typedef double v4d __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Reference GEMM: Y_ref = X W^T with exact products and fp64 sums. Every input
// value (fp32, fp16 or bf16) widens exactly to fp64, and the product of two
// of them needs at most 48 significand bits, so V_MFMA_F64_16X16X4_F64 forms
// each product exactly and only the fp64 additions round: the result is
// within about K * 2^-53 of the exact sum, far below the quantization errors
// being measured.
// Block tile 64 x 64, K-tile 16 (K is a multiple of 16), 4 waves in 2 x 2,
// each 32 x 32 = 2 x 2 MFMA tiles. The tile sits in LDS k-major as fp64; a
// row of 80 doubles puts the four 16-lane groups of one operand read on
// distinct bank halves. The next K-tile's values are loaded into registers
// while the current one is multiplied.
// ---------------------------------------------------------------------------
constexpr int kRefBM = 64, kRefBN = 64, kRefBK = 16;
constexpr int kRefThreads = 256;
constexpr int kRefLd = 80;

template <int DT>
__device__ __forceinline__ void load4_f32(const char* p, float* v) {
  if constexpr (DT == SQ_F32) {
    const float4 q = *(const float4*)p;
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else {
    const uint2 q = *(const uint2*)p;
    const uint32_t w[2] = {q.x, q.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (DT == SQ_BF16) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      } else {
        v[2 * i] = f16_bits_to_f32(w[i] & 0xFFFFu);
        v[2 * i + 1] = f16_bits_to_f32(w[i] >> 16);
      }
    }
  }
}

template <int XT, int WT>
__global__ void __launch_bounds__(kRefThreads)
k_ref_gemm(const char* __restrict__ X, int64_t ldx, const char* __restrict__ W, int64_t ldw, int M,
           int N, int K, double* __restrict__ Y) {
  __shared__ double sA[kRefBK][kRefLd];
  __shared__ double sB[kRefBK][kRefLd];
  const int tiles_n = (N + kRefBN - 1) / kRefBN;
  const int m0 = (blockIdx.x / tiles_n) * kRefBM;
  const int n0 = (blockIdx.x % tiles_n) * kRefBN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // loader: 4 consecutive k of one row of each operand
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const int gm = m0 + lrow, gn = n0 + lrow;
  float va[4], vb[4];
  auto gload = [&](int k0) {
    if (gm < M) load4_f32<XT>(X + ((int64_t)gm * ldx + k0 + lk) * DtSize<XT>::v, va);
    else va[0] = va[1] = va[2] = va[3] = 0.0f;
    if (gn < N) load4_f32<WT>(W + ((int64_t)gn * ldw + k0 + lk) * DtSize<WT>::v, vb);
    else vb[0] = vb[1] = vb[2] = vb[3] = 0.0f;
  };
  v4d acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v4d{};

  gload(0);
  for (int k0 = 0; k0 < K; k0 += kRefBK) {
    __syncthreads();                      // the previous tile's reads are done
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sA[lk + e][lrow] = (double)va[e];
      sB[lk + e][lrow] = (double)vb[e];
    }
    __syncthreads();
    if (k0 + kRefBK < K) gload(k0 + kRefBK);
    // lane l supplies row (or column) l % 16 at k = 4 s + l / 16
#pragma unroll
    for (int s4 = 0; s4 < kRefBK / 4; ++s4) {
      const int k = 4 * s4 + (lane >> 4);
      double a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = sA[k][wm * 32 + i * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = sB[k][wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  // output element e of a 16 x 16 tile: row lane / 16 + 4 e, column lane % 16
  // (this instruction interleaves the rows, unlike the 32-bit ones)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = m0 + wm * 32 + i * 16 + (lane >> 4) + 4 * e;
        const int c = n0 + wn * 32 + j * 16 + (lane & 15);
        if (r < M && c < N) Y[(int64_t)r * N + c] = acc[i][j][e];
      }
}

// ---------------------------------------------------------------------------
// Squared error and squared norm, fp64, fixed order.
// ---------------------------------------------------------------------------
constexpr int kErrBlocks = 1024;
constexpr int kErrThreads = 256;

// Sum of two values over a 256-thread block, the same order every run;
// thread 0 gets the result.
__device__ __forceinline__ void block_sum2(double& d, double& r) {
  __shared__ double red[2][kErrThreads / 64];
  d = wave_sum_f64(d);
  r = wave_sum_f64(r);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[0][wave] = d; red[1][wave] = r; }
  __syncthreads();
  if (threadIdx.x == 0) {
    d = red[0][0]; r = red[1][0];
    for (int w = 1; w < kErrThreads / 64; ++w) { d += red[0][w]; r += red[1][w]; }
  }
}

// part[b] = this block's share of sum (q - ref)^2, part[kErrBlocks + b] of sum ref^2.
__global__ void __launch_bounds__(kErrThreads)
k_err_partial(const float4* __restrict__ q, const double2* __restrict__ ref, int64_t n4,
              double* __restrict__ part) {
  double d = 0.0, r = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * kErrThreads + threadIdx.x; i < n4;
       i += (int64_t)kErrBlocks * kErrThreads) {
    const float4 a = q[i];
    const double2 b0 = ref[2 * i], b1 = ref[2 * i + 1];
    const double e0 = (double)a.x - b0.x, e1 = (double)a.y - b0.y;
    const double e2 = (double)a.z - b1.x, e3 = (double)a.w - b1.y;
    d += e0 * e0 + e1 * e1 + e2 * e2 + e3 * e3;
    r += b0.x * b0.x + b0.y * b0.y + b1.x * b1.x + b1.y * b1.y;
  }
  block_sum2(d, r);
  if (threadIdx.x == 0) { part[blockIdx.x] = d; part[kErrBlocks + blockIdx.x] = r; }
}

// out[0] = sum of the error partials, out[1] = sum of the norm partials.
__global__ void __launch_bounds__(kErrThreads)
k_err_final(const double* __restrict__ part, double* __restrict__ out) {
  double d = 0.0, r = 0.0;
  for (int b = threadIdx.x; b < kErrBlocks; b += kErrThreads) {
    d += part[b];
    r += part[kErrBlocks + b];
  }
  block_sum2(d, r);
  if (threadIdx.x == 0) { out[0] = d; out[1] = r; }
}

// The choice among the alphas: rel[i] = err[2i] / err[2i + 1] (fp64; 0 when
// the reference norm is 0), best = the index of the smallest rel, the first
// on ties. One thread walks the (at most 1024) alphas in order.
__global__ void __launch_bounds__(64)
k_sweep_pick(const double* __restrict__ err, int n, double* __restrict__ rel,
             int32_t* __restrict__ best) {
  if (threadIdx.x != 0) return;
  int b = 0;
  double rb = 0.0;
  for (int i = 0; i < n; ++i) {
    const double ref = err[2 * i + 1];
    const double r = ref > 0.0 ? err[2 * i] / ref : 0.0;
    if (rel != nullptr) rel[i] = r;
    if (i == 0 || r < rb) {
      rb = r;
      b = i;
    }
  }
  if (best != nullptr) best[0] = b;
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
size_t err_partials_bytes() { return 2 * kErrBlocks * sizeof(double); }

int launch_sweep_pick(const double* err, int n, double* rel, int32_t* best, hipStream_t st) {
  k_sweep_pick<<<1, 64, 0, st>>>(err, n, rel, best);
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

template <int XT>
static void launch_ref_w(const void* X, int64_t ldx, const void* W, int wt, int64_t ldw, int M,
                         int N, int K, double* Y, unsigned blocks, hipStream_t st) {
  switch (wt) {
    case SQ_F32:
      k_ref_gemm<XT, SQ_F32><<<blocks, kRefThreads, 0, st>>>((const char*)X, ldx, (const char*)W,
                                                             ldw, M, N, K, Y);
      break;
    case SQ_F16:
      k_ref_gemm<XT, SQ_F16><<<blocks, kRefThreads, 0, st>>>((const char*)X, ldx, (const char*)W,
                                                             ldw, M, N, K, Y);
      break;
    default:
      k_ref_gemm<XT, SQ_BF16><<<blocks, kRefThreads, 0, st>>>((const char*)X, ldx, (const char*)W,
                                                              ldw, M, N, K, Y);
      break;
  }
}

// Y [M, N] fp64 (row stride N) = X W^T, exact products, fp64 sums. K % 16 == 0.
int launch_ref_gemm(const void* X, int xt, int64_t ldx, const void* W, int wt, int64_t ldw,
                    int64_t M, int64_t N, int64_t K, double* Y, hipStream_t st) {
  if (M == 0) return SQ_OK;
  const unsigned blocks = (unsigned)(((M + kRefBM - 1) / kRefBM) * ((N + kRefBN - 1) / kRefBN));
  switch (xt) {
    case SQ_F32: launch_ref_w<SQ_F32>(X, ldx, W, wt, ldw, (int)M, (int)N, (int)K, Y, blocks, st); break;
    case SQ_F16: launch_ref_w<SQ_F16>(X, ldx, W, wt, ldw, (int)M, (int)N, (int)K, Y, blocks, st); break;
    default:     launch_ref_w<SQ_BF16>(X, ldx, W, wt, ldw, (int)M, (int)N, (int)K, Y, blocks, st); break;
  }
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

// out[0:2] = (sum (q - ref)^2, sum ref^2) over n values, q fp32 and ref fp64
// (n a multiple of 4, both 16-byte aligned). part: err_partials_bytes() of
// device scratch.
int launch_sq_err(const float* q, const double* ref, int64_t n, double* part, double* out,
                  hipStream_t st) {
  k_err_partial<<<kErrBlocks, kErrThreads, 0, st>>>((const float4*)q, (const double2*)ref, n / 4,
                                                   part);
  k_err_final<<<1, kErrThreads, 0, st>>>(part, out);
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

}  // namespace sq
