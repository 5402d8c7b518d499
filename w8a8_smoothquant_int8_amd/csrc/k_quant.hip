// Row-wise symmetric INT8 quantization ([SQ] Steps 5-6 and the sketch's
// quantize_int8), in three flavours sharing one kernel:
//   FOLD    (weights, per output channel): v = fp32(W[n,k] * s[k]);
//           scale = max_k |v| / 127; code = clamp(rne(fp32(v / scale)), +-127)
//   DYNAMIC (activations, per token):      v = fp32(X[m,k] / s[k]); same scale
//   STATIC  (activations, per tensor):     v = fp32(X[m,k] / s[k]); scale given
//
// The kernel is HBM-bound: it reads each input element once (16-byte loads)
// and writes one byte per element. A block owns one row at a time and walks
// rows with a grid stride; each thread keeps CPT chunks of 8 consecutive
// channels of the row in registers, so the row is read once, reduced (wave
// max, then LDS across waves) and quantized from registers. The per-channel
// fp64 reciprocals 1/s[k] that make the divisions exact (div_rn) are computed
// once per block and reused for every row the block visits; the next row's
// input is loaded before the current row is reduced, to keep HBM busy.
#include "sq_internal.h"

namespace sq {

enum QuantKind { Q_FOLD = 0, Q_DYNAMIC = 1, Q_STATIC = 2 };

constexpr int kQuantMaxThreads = 1024;

template <int DT, int CPT>
struct RowChunks {
  // raw 16-byte words of the row chunks (fp32 needs two per chunk)
  static constexpr int kWords = (DT == SQ_F32) ? 2 : 1;
  uint4 w[CPT][kWords];
};

template <int DT, int CPT>
__device__ __forceinline__ void load_row(RowChunks<DT, CPT>& r, const char* row, int64_t K, int tid,
                                         int T) {
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int64_t c = tid + (int64_t)j * T;   // chunk index
    if (c * 8 < K) {
      const uint4* p = (const uint4*)(row + c * 8 * DtSize<DT>::v);
#pragma unroll
      for (int q = 0; q < RowChunks<DT, CPT>::kWords; ++q) r.w[j][q] = p[q];
    }
  }
}

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

// rows: M (activations) or N (weights). in_ld_bytes: input row stride.
// s: [K] or null (no smoothing). scale_io: [rows] written (FOLD, DYNAMIC) or
// [1] read (STATIC). out: [rows, K] int8 contiguous.
template <int DT, int CPT, int KIND>
__global__ void __launch_bounds__(kQuantMaxThreads)
k_quant_rows(const char* __restrict__ in, int64_t rows, int64_t K, int64_t in_ld_bytes,
             const float* __restrict__ s, float* __restrict__ scale_io, int8_t* __restrict__ out) {
  const int tid = threadIdx.x;
  const int T = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = T >> 6;

  // Per-channel factor: fp32 s (FOLD multiplies) or fp64 1/s (divisions).
  float sm[CPT][8];
  double rs[CPT][8];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int64_t c = tid + (int64_t)j * T;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float sv = (s != nullptr && c * 8 < K) ? s[c * 8 + e] : 1.0f;
      if constexpr (KIND == Q_FOLD) sm[j][e] = sv;
      else rs[j][e] = 1.0 / (double)sv;      // RN64(1/s), IEEE fp64 division
    }
  }

  double r_static = 0.0;
  float a_static = 0.0f;
  if constexpr (KIND == Q_STATIC) {
    a_static = scale_io[0];
    r_static = a_static != 0.0f ? 1.0 / (double)a_static : 0.0;
  }

  __shared__ float red[2][kQuantMaxThreads / 64];

  // Rows of up to 2 chunks per thread also prefetch the next row; wider rows
  // would need more registers than a 1024-thread block can give a thread.
  constexpr bool kPrefetch = CPT <= 2;
  RowChunks<DT, CPT> cur, nxt;
  int64_t m = blockIdx.x;
  if (kPrefetch && m < rows) load_row<DT, CPT>(cur, in + m * in_ld_bytes, K, tid, T);
  int parity = 0;
  for (; m < rows; m += gridDim.x) {
    const int64_t mn = m + gridDim.x;
    if (kPrefetch) {
      if (mn < rows) load_row<DT, CPT>(nxt, in + mn * in_ld_bytes, K, tid, T);
    } else {
      load_row<DT, CPT>(cur, in + m * in_ld_bytes, K, tid, T);
    }

    float v[CPT][8];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t c = tid + (int64_t)j * T;
      float x[8];
      widen8<DT>(cur.w[j], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float t;
        if constexpr (KIND == Q_FOLD) t = x[e] * sm[j][e];     // fp32 multiply
        else t = div_rn(x[e], rs[j][e]);                      // fp32(x / s), exact
        v[j][e] = t;
        if (c * 8 < K) amax = __builtin_fmaxf(amax, __builtin_fabsf(t));
      }
    }

    float scale;
    double rscale;
    if constexpr (KIND == Q_STATIC) {
      scale = a_static;
      rscale = r_static;
    } else {
      amax = wave_max(amax);
      if (lane == 0) red[parity][wave] = amax;
      __syncthreads();
      amax = red[parity][0];
      for (int w = 1; w < nwaves; ++w) amax = __builtin_fmaxf(amax, red[parity][w]);
      parity ^= 1;
      scale = amax / 127.0f;                                  // IEEE fp32 division
      rscale = scale != 0.0f ? 1.0 / (double)scale : 0.0;
      if (tid == 0) scale_io[m] = scale;
    }

    int8_t* orow = out + m * K;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t c = tid + (int64_t)j * T;
      if (c * 8 < K) {
        int q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = scale != 0.0f ? quant_code(div_rn(v[j][e], rscale)) : 0;
        uint2 pk;
        pk.x = pack4_i8(q[0], q[1], q[2], q[3]);
        pk.y = pack4_i8(q[4], q[5], q[6], q[7]);
        *(uint2*)(orow + c * 8) = pk;
      }
    }
    if (kPrefetch) cur = nxt;
  }
}

// Pick threads per block T (multiple of 64, <= 1024) and chunks per thread
// CPT (<= 4) so that T * CPT * 8 >= K, preferring CPT <= 2 (prefetching).
static void pick_shape(int64_t K, int* T, int* cpt) {
  const int64_t chunks = K / 8;
  int64_t t = (chunks + 1) / 2;
  t = (t + 63) / 64 * 64;
  if (t < 64) t = 64;
  if (t > kQuantMaxThreads) t = kQuantMaxThreads;
  *T = (int)t;
  *cpt = (int)((chunks + t - 1) / t);
}

template <int DT, int KIND>
static int launch_rows_dt(const void* in, int64_t rows, int64_t K, int64_t ld, const float* s,
                          float* scale_io, int8_t* out, hipStream_t st) {
  int T, cpt;
  pick_shape(K, &T, &cpt);
  // At least 4 rows per block, so the per-block reciprocal setup is amortised,
  // and no more blocks than about 8 waves per SIMD could hold.
  int64_t grid = (rows + 3) / 4;
  const int64_t cap = 256LL * (2048 / T);
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  const char* p = (const char*)in;
  const int64_t ldb = ld * DtSize<DT>::v;
  switch (cpt) {
    case 1: k_quant_rows<DT, 1, KIND><<<(unsigned)grid, T, 0, st>>>(p, rows, K, ldb, s, scale_io, out); break;
    case 2: k_quant_rows<DT, 2, KIND><<<(unsigned)grid, T, 0, st>>>(p, rows, K, ldb, s, scale_io, out); break;
    case 3: k_quant_rows<DT, 3, KIND><<<(unsigned)grid, T, 0, st>>>(p, rows, K, ldb, s, scale_io, out); break;
    case 4: k_quant_rows<DT, 4, KIND><<<(unsigned)grid, T, 0, st>>>(p, rows, K, ldb, s, scale_io, out); break;
    default: return SQ_ERR_INVALID_ARG;   // K > 32768 is rejected by validation
  }
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

template <int KIND>
static int launch_rows(const void* in, int dt, int64_t rows, int64_t K, int64_t ld, const float* s,
                       float* scale_io, int8_t* out, hipStream_t st) {
  if (rows == 0) return SQ_OK;
  switch (dt) {
    case SQ_F32: return launch_rows_dt<SQ_F32, KIND>(in, rows, K, ld, s, scale_io, out, st);
    case SQ_F16: return launch_rows_dt<SQ_F16, KIND>(in, rows, K, ld, s, scale_io, out, st);
    default:     return launch_rows_dt<SQ_BF16, KIND>(in, rows, K, ld, s, scale_io, out, st);
  }
}

int launch_fold_quant(const void* W, int wt, int64_t N, int64_t K, int64_t ldw, const float* s,
                      int8_t* Wq, float* w_scale, hipStream_t st) {
  return launch_rows<Q_FOLD>(W, wt, N, K, ldw, s, w_scale, Wq, st);
}

int launch_quant_act(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const float* s,
                     int mode, int8_t* Xq, float* a_scale, hipStream_t st) {
  if (mode == SQ_ACT_PER_TENSOR_STATIC)
    return launch_rows<Q_STATIC>(X, xt, M, K, ldx, s, a_scale, Xq, st);
  return launch_rows<Q_DYNAMIC>(X, xt, M, K, ldx, s, a_scale, Xq, st);
}

}  // namespace sq
