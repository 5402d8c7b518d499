// Normalization with the smoothing division folded into its weight, fused
// with the activation quantizer ("SmoothQuant" explainer, "How it works",
// Step 5: the layer input follows a normalization, whose weight (and bias)
// can absorb 1/s, so the path needs no separate division; the sketch's
// smooth_layer divides the norm weight and bias by s).
//
// One kernel reads the residual stream h once and writes the INT8 codes of
//   RMSNorm:   x_s = fp32(fp32(h * r) * g')                 r = 1/sqrt(mean(h^2) + eps)
//   LayerNorm: x_s = fp32(fp32(fp32((h - mu) * r) * g') + b')  r = 1/sqrt(var(h) + eps)
// with g' = g / s, b' = b / s, quantized per token (or with a static scale)
// exactly as the path's quantizer does. Row sums run in fp64 (each square is
// exact in fp64), in a fixed order; the mean and r are rounded to fp32.
//
// Shape: the wave-per-row design of the quantizer. WPR = 1, 2 or 4 waves per
// row, each lane holding at most CPL = 8 chunks of 8 channels in registers
// (16-bit inputs up to K = 16384, fp32 up to 4096). A row takes one fp64
// reduction (RMS) or two (LayerNorm), then the row max; with WPR > 1 each is
// a wave reduction plus one exchange in LDS. The folded weight and bias sit
// in LDS as in the quantizer's factor table. After the last pass over the
// raw registers, they take the wave's next row.
#include "sq_internal.h"

namespace sq {

enum NormKind { N_RMS = 0, N_LAYER = 1 };

constexpr int kNormThreads = 512;

template <int DT, int NORM, bool STATIC, int CPL, int WPR>
struct NormCfg {
  static constexpr int kWords = DT == SQ_F32 ? 2 : 1;
  static constexpr int kTabParts = NORM == N_LAYER ? 4 : 2;   // 16-byte words per chunk
  static_assert(CPL <= 8 && (WPR == 1 || WPR == 2 || WPR == 4), "row share must fit registers");
};

// Row-wide fp64 sum for WPR waves: wave butterfly, then the row's waves
// exchange through LDS (buf: this stage's buffer for this iteration).
template <int WPR>
__device__ __forceinline__ double row_sum_f64(double v, double* buf, int wave, int slot) {
  v = wave_sum_f64(v);
  if constexpr (WPR > 1) {
    if ((threadIdx.x & 63) == 0) buf[wave] = v;
    __syncthreads();
    v = buf[WPR * slot];
#pragma unroll
    for (int w = 1; w < WPR; ++w) v += buf[WPR * slot + w];
  }
  return v;
}

template <int DT, int NORM, bool STATIC, int CPL, int WPR>
__global__ void __launch_bounds__(kNormThreads)
k_norm_quant(const char* __restrict__ in, int64_t rows, int K, int64_t in_ld_bytes,
             const float* __restrict__ g, const float* __restrict__ b, double eps,
             float* __restrict__ scale_io, int8_t* __restrict__ out, float* __restrict__ stats) {
  using Cfg = NormCfg<DT, NORM, STATIC, CPL, WPR>;
  constexpr int kWords = Cfg::kWords;
  constexpr int kSpan = 64 * CPL;
  constexpr int kWaves = kNormThreads / 64;
  // word p of chunk c at tab[p * kSpan * WPR + c]: g' (2 words), then b' (2 words)
  __shared__ uint4 tab[Cfg::kTabParts * kSpan * WPR];
  __shared__ double red_mu[2][kWaves], red_ss[2][kWaves];
  __shared__ float red_max[2][kWaves];
  const int nch = K / 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = wave % WPR;
  const int slot = wave / WPR;
  const int slots = kWaves / WPR;
  const int64_t row_step = (int64_t)gridDim.x * slots;
  const int64_t iters = (rows + row_step - 1) / row_step;   // the same for every wave
  int64_t m = (int64_t)blockIdx.x * slots + slot;
  const int c0 = kSpan * half + lane;
  const double dk = (double)K;

  // Chunks past the row end read chunk nch - 1 (no branch in the loads) and
  // are masked out of every sum, max and store.
  uint4 raw[CPL][kWords];
  auto chunk = [&](int j) { return c0 + 64 * j < nch ? c0 + 64 * j : nch - 1; };
  auto load = [&](int64_t row) {
    const char* p = in + row * in_ld_bytes;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
#pragma unroll
      for (int q = 0; q < kWords; ++q)
        raw[j][q] = ((const uint4*)(p + (int64_t)chunk(j) * 8 * DtSize<DT>::v))[q];
    }
  };
  if (m < rows) load(m);

  for (int c = threadIdx.x; c < nch; c += blockDim.x) {
    const float4* gp = (const float4*)(g + (int64_t)c * 8);
    const float4 g0 = gp[0], g1 = gp[1];
    tab[c] = make_uint4(__float_as_uint(g0.x), __float_as_uint(g0.y), __float_as_uint(g0.z),
                        __float_as_uint(g0.w));
    tab[kSpan * WPR + c] = make_uint4(__float_as_uint(g1.x), __float_as_uint(g1.y),
                                      __float_as_uint(g1.z), __float_as_uint(g1.w));
    if constexpr (NORM == N_LAYER) {
      float4 b0 = make_float4(0.f, 0.f, 0.f, 0.f), b1 = b0;
      if (b != nullptr) {
        const float4* bp = (const float4*)(b + (int64_t)c * 8);
        b0 = bp[0];
        b1 = bp[1];
      }
      tab[2 * kSpan * WPR + c] = make_uint4(__float_as_uint(b0.x), __float_as_uint(b0.y),
                                            __float_as_uint(b0.z), __float_as_uint(b0.w));
      tab[3 * kSpan * WPR + c] = make_uint4(__float_as_uint(b1.x), __float_as_uint(b1.y),
                                            __float_as_uint(b1.z), __float_as_uint(b1.w));
    }
  }
  __syncthreads();

  float a_static = 0.0f;
  double r_static = 0.0;
  if constexpr (STATIC) {
    a_static = scale_io[0];
    r_static = a_static != 0.0f ? rcp_rn64(a_static) : 0.0;
  }

  for (int64_t it = 0; it < iters; ++it, m += row_step) {
    const bool active = m < rows;                 // uniform over the row's waves
    const int par = (int)(it & 1);
    // pass 1 (LayerNorm): the row mean
    float mu = 0.0f;
    if constexpr (NORM == N_LAYER) {
      double sum = 0.0;
      if (active) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          float x[8];
          widen8<DT>(raw[j], x);
          const bool in_row = c0 + 64 * j < nch;
#pragma unroll
          for (int e = 0; e < 8; ++e) sum += in_row ? (double)x[e] : 0.0;
        }
      }
      mu = (float)(row_sum_f64<WPR>(sum, red_mu[par], wave, slot) / dk);   // IEEE fp64 division
    }
    // pass 2: sum of squared deviations (RMS: of the values), exact squares
    double ss = 0.0;
    if (active) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        float x[8];
        widen8<DT>(raw[j], x);
        const bool in_row = c0 + 64 * j < nch;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double d = (double)(NORM == N_LAYER ? x[e] - mu : x[e]);   // fp32 subtraction
          ss += in_row ? d * d : 0.0;
        }
      }
    }
    ss = row_sum_f64<WPR>(ss, red_ss[par], wave, slot);
    const float r = (float)(1.0 / __builtin_sqrt(ss / dk + eps));
    // pass 3: x_s and the row max
    float v[CPL][8];
    float amax = 0.0f;
    if (active) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        float x[8];
        widen8<DT>(raw[j], x);
        const int c = chunk(j);
        const uint4 f0 = tab[c], f1 = tab[kSpan * WPR + c];
        const float gf[8] = {__uint_as_float(f0.x), __uint_as_float(f0.y), __uint_as_float(f0.z),
                             __uint_as_float(f0.w), __uint_as_float(f1.x), __uint_as_float(f1.y),
                             __uint_as_float(f1.z), __uint_as_float(f1.w)};
        const bool in_row = c0 + 64 * j < nch;
        if constexpr (NORM == N_LAYER) {
          const uint4 h0 = tab[2 * kSpan * WPR + c], h1 = tab[3 * kSpan * WPR + c];
          const float bf[8] = {__uint_as_float(h0.x), __uint_as_float(h0.y), __uint_as_float(h0.z),
                               __uint_as_float(h0.w), __uint_as_float(h1.x), __uint_as_float(h1.y),
                               __uint_as_float(h1.z), __uint_as_float(h1.w)};
#pragma unroll
          for (int e = 0; e < 8; ++e) v[j][e] = ((x[e] - mu) * r) * gf[e] + bf[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[j][e] = (x[e] * r) * gf[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, in_row ? __builtin_fabsf(v[j][e]) : 0.0f);
      }
      // the raw registers are free: the wave's next row (not before pass 3 is
      // done with them: an opaque zero that depends on the row max)
      if (m + row_step < rows) {
        int zero;
        asm volatile("v_mov_b32 %0, 0" : "=v"(zero) : "v"(amax));
        load(m + row_step + zero);
      }
    }
    float scale;
    double rscale;
    if constexpr (STATIC) {
      scale = a_static;
      rscale = r_static;
    } else {
      amax = wave_max(amax);
      if constexpr (WPR > 1) {
        if (lane == 0) red_max[par][wave] = amax;
        __syncthreads();
        amax = red_max[par][WPR * slot];
#pragma unroll
        for (int w = 1; w < WPR; ++w) amax = __builtin_fmaxf(amax, red_max[par][WPR * slot + w]);
      }
      scale = amax / 127.0f;                                     // IEEE fp32 division
      rscale = scale != 0.0f ? rcp_rn64(scale) : 0.0;
      if (active && half == 0 && lane == 0) scale_io[m] = scale;
    }
    if (!active) continue;
    if (stats != nullptr && half == 0 && lane == 0) {
      stats[2 * m] = mu;
      stats[2 * m + 1] = r;
    }
    int8_t* orow = out + m * K;
    const uint32_t keep = scale != 0.0f ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = c0 + 64 * j;
      uint32_t q[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = code_word(div_rn(v[j][e], rscale));
      uint2 pk;
      pk.x = pack4_codes(q[0], q[1], q[2], q[3]) & keep;
      pk.y = pack4_codes(q[4], q[5], q[6], q[7]) & keep;
      if (c < nch) *(uint2*)(orow + c * 8) = pk;
    }
  }
}

// out[k] = fp32(widen(w[k]) / s[k]) (s == NULL: widen only), k < K.
template <int DT>
__global__ void k_fold_norm(const char* __restrict__ w, const float* __restrict__ s, int64_t K,
                            float* __restrict__ out) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  const float v = load1_f32<DT>(w + k * DtSize<DT>::v);
  out[k] = s != nullptr ? v / s[k] : v;                  // IEEE fp32 division
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
template <int DT, int NORM, bool STATIC, int CPL, int WPR>
static void launch_norm_shape(const char* p, int64_t rows, int K, int64_t ldb, const float* g,
                              const float* b, double eps, float* scale_io, int8_t* out,
                              float* stats, hipStream_t st) {
  auto f = k_norm_quant<DT, NORM, STATIC, CPL, WPR>;
  constexpr int slots = kNormThreads / 64 / WPR;
  int64_t grid = (rows + slots - 1) / slots;
  const int64_t cap =
      resident_blocks<NormCfg<DT, NORM, STATIC, CPL, WPR>>((const void*)f, kNormThreads);
  if (grid > cap) grid = cap;
  f<<<(unsigned)grid, kNormThreads, 0, st>>>(p, rows, K, ldb, g, b, eps, scale_io, out, stats);
}

// Waves per row and chunks per lane: one wave up to 512 chunks (K 4096, 2, 4
// or 8 chunks per lane), then 2 or 4 waves (16-bit inputs only) with the
// fewest chunks per lane (5 to 8) that cover the row, so no lane carries
// chunks past the row end it does not need.
template <int DT, int NORM, bool STATIC, int WPR>
static void launch_norm_w(int cpl, const char* p, int64_t rows, int K, int64_t ldb, const float* g,
                          const float* b, double eps, float* scale_io, int8_t* out, float* stats,
                          hipStream_t st) {
#define SQ_NORM_ARGS p, rows, K, ldb, g, b, eps, scale_io, out, stats, st
  switch (cpl) {
    case 5: launch_norm_shape<DT, NORM, STATIC, 5, WPR>(SQ_NORM_ARGS); break;
    case 6: launch_norm_shape<DT, NORM, STATIC, 6, WPR>(SQ_NORM_ARGS); break;
    case 7: launch_norm_shape<DT, NORM, STATIC, 7, WPR>(SQ_NORM_ARGS); break;
    default: launch_norm_shape<DT, NORM, STATIC, 8, WPR>(SQ_NORM_ARGS); break;
  }
}

template <int DT, int NORM, bool STATIC>
static int launch_norm_dt(const char* p, int64_t rows, int K, int64_t ldb, const float* g,
                          const float* b, double eps, float* scale_io, int8_t* out, float* stats,
                          hipStream_t st) {
  const int lane_chunks = (K / 8 + 63) / 64;
  if (lane_chunks <= 2) launch_norm_shape<DT, NORM, STATIC, 2, 1>(SQ_NORM_ARGS);
  else if (lane_chunks <= 4) launch_norm_shape<DT, NORM, STATIC, 4, 1>(SQ_NORM_ARGS);
  else if (lane_chunks <= 8) launch_norm_shape<DT, NORM, STATIC, 8, 1>(SQ_NORM_ARGS);
  else if constexpr (DT != SQ_F32) {
    if (lane_chunks <= 16)
      launch_norm_w<DT, NORM, STATIC, 2>((lane_chunks + 1) / 2, SQ_NORM_ARGS);
    else
      launch_norm_w<DT, NORM, STATIC, 4>((lane_chunks + 3) / 4, SQ_NORM_ARGS);
  }
#undef SQ_NORM_ARGS
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

template <int NORM, bool STATIC>
static int launch_norm_k(const void* H, int ht, int64_t M, int K, int64_t ldh, const float* g,
                         const float* b, double eps, float* a_scale, int8_t* Xq, float* stats,
                         hipStream_t st) {
  const char* p = (const char*)H;
  switch (ht) {
    case SQ_F32:
      return launch_norm_dt<SQ_F32, NORM, STATIC>(p, M, K, ldh * 4, g, b, eps, a_scale, Xq, stats, st);
    case SQ_F16:
      return launch_norm_dt<SQ_F16, NORM, STATIC>(p, M, K, ldh * 2, g, b, eps, a_scale, Xq, stats, st);
    default:
      return launch_norm_dt<SQ_BF16, NORM, STATIC>(p, M, K, ldh * 2, g, b, eps, a_scale, Xq, stats, st);
  }
}

// Largest K the fused kernel takes for an input dtype.
int64_t norm_quant_max_k(int ht) { return ht == SQ_F32 ? 4096 : 16384; }

int launch_norm_quant(const void* H, int ht, int64_t M, int64_t K, int64_t ldh, int norm,
                      const float* g, const float* b, double eps, int mode, int8_t* Xq,
                      float* a_scale, float* stats, hipStream_t st) {
  if (M == 0) return SQ_OK;
  const bool stat = mode == SQ_ACT_PER_TENSOR_STATIC;
  if (norm == N_LAYER)
    return stat ? launch_norm_k<N_LAYER, true>(H, ht, M, (int)K, ldh, g, b, eps, a_scale, Xq, stats, st)
                : launch_norm_k<N_LAYER, false>(H, ht, M, (int)K, ldh, g, b, eps, a_scale, Xq, stats, st);
  return stat ? launch_norm_k<N_RMS, true>(H, ht, M, (int)K, ldh, g, nullptr, eps, a_scale, Xq, stats, st)
              : launch_norm_k<N_RMS, false>(H, ht, M, (int)K, ldh, g, nullptr, eps, a_scale, Xq, stats, st);
}

int launch_fold_norm(const void* w, int wt, const float* s, int64_t K, float* out, hipStream_t st) {
  const unsigned blocks = (unsigned)((K + 255) / 256);
  switch (wt) {
    case SQ_F32: k_fold_norm<SQ_F32><<<blocks, 256, 0, st>>>((const char*)w, s, K, out); break;
    case SQ_F16: k_fold_norm<SQ_F16><<<blocks, 256, 0, st>>>((const char*)w, s, K, out); break;
    default:     k_fold_norm<SQ_BF16><<<blocks, 256, 0, st>>>((const char*)w, s, K, out); break;
  }
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

}  // namespace sq
