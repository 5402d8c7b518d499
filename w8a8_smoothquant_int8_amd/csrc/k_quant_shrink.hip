// Per-token INT8 quant and the LoRA shrink from one read of X.
//
// The quant ([SQ] "How it works", Steps 5-6: x_s = x / s, codes against the
// row's absmax / 127, or a static scale) and the first half of the LoRA path
// ([LoRA] Pitch: T = bf16(bf16(X) A^T), fp32 sums) read the same activations.
// Here one kernel serves both: a block owns 16 rows, its W waves split K
// into interleaved 32-element steps, and every lane keeps its share of one
// row in registers for the whole kernel:
//   - the shrink: each step's 16-byte chunk (row lane % 16, k offset
//     8 (lane / 16)) is exactly the second operand of the bf16 matrix
//     instruction V_MFMA_F32_16X16X32_BF16; the adapter rows (the first
//     operand) come from L2, where the whole of A stays resident. The W
//     per-wave partial sums meet in LDS and are added in a fixed order, one
//     rank tile at a time;
//   - the quant: x_s = fp32(x / s) through the fp64 reciprocals of s held in
//     LDS, the row max (4 lanes per row in a wave, then W waves through LDS),
//     and the codes from the same registers.
// X is read from HBM once instead of twice; the cost is a block of 16 rows
// per CU, so M / 16 blocks, each reading all of A (r K bf16) from L2. At the
// Llama-3-8B shapes (M = 2048, K = 4096, r = 16..48) that makes it 1.0-1.3x
// slower than the two separate kernels, so the path keeps those by default.
#include "sq_internal.h"

namespace sq {

constexpr int kQSRows = 16;

template <int XT>
__device__ __forceinline__ uint4 chunk_as_bf16(uint4 u) {
  if constexpr (XT == SQ_BF16) {
    return u;
  } else {
    float v[8];
    widen8<XT>(&u, v);
    uint4 r;
    r.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
    r.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
    r.z = f32_to_bf16_bits(v[4]) | (f32_to_bf16_bits(v[5]) << 16);
    r.w = f32_to_bf16_bits(v[6]) | (f32_to_bf16_bits(v[7]) << 16);
    return r;
  }
}

// XT: bf16 or fp16 X. W waves, CPL steps of 32 per lane (W * CPL * 32 >= K),
// NT rank tiles of 16 (16 NT >= R). KMAX: the reciprocal table's size.
template <int XT, int W, int CPL, int NT, int KMAX>
__global__ void __launch_bounds__(W * 64)
k_quant_shrink(const char* __restrict__ X, int64_t ldx_bytes, int M, int K,
               const float* __restrict__ s, int is_static, float* __restrict__ scale_io,
               int8_t* __restrict__ Xq, const unsigned short* __restrict__ A, int R,
               unsigned short* __restrict__ T, int64_t ldt) {
  __shared__ double rtab[KMAX];                 // RN64(1 / s[k])
  __shared__ float red[W][16 * 16];             // one rank tile of per-wave partial sums
  __shared__ float rmax[W][kQSRows];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, kg = lane >> 4;
  const int m0 = blockIdx.x * kQSRows;
  const bool row_ok = m0 + lrow < M;
  const int mrow = row_ok ? m0 + lrow : M - 1;  // rows past M read row M - 1, never stored
  const char* xrow = X + (int64_t)mrow * ldx_bytes;

  // This lane's chunks: step g = wave + W j, elements k = 32 g + 8 kg .. + 7.
  auto kof = [&](int j) { return 32 * (wave + W * j) + 8 * kg; };
  uint4 xr[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j)
    xr[j] = kof(j) < K ? *(const uint4*)(xrow + (int64_t)kof(j) * 2) : make_uint4(0, 0, 0, 0);

  for (int k = tid; k < K; k += W * 64) rtab[k] = s != nullptr ? rcp_rn64(s[k]) : 1.0;

  // The shrink. Register e of rank tile t: rank 16 t + 4 kg + e, row lrow.
  v4f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = v4f{0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int k = kof(j);
    const bool kin = k < K;
    const v8bf xb = __builtin_bit_cast(v8bf, chunk_as_bf16<XT>(xr[j]));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int i = t * 16 + lrow;
      const uint4 au = (kin && i < R) ? *(const uint4*)(A + (int64_t)i * K + k) : make_uint4(0, 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, au), xb, acc[t], 0, 0, 0);
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][(4 * kg + e) * 16 + lrow] = acc[t][e];
    __syncthreads();
    if (tid < 128) {
      // thread: row tid / 8, ranks 2 (tid % 8) and + 1 of this tile; waves in order
      const int row = tid >> 3, rp = (tid & 7) * 2;
      float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        a0 += red[w][rp * 16 + row];
        a1 += red[w][(rp + 1) * 16 + row];
      }
      const int i = t * 16 + rp, m = m0 + row;
      if (m < M && i < R)                        // R % 8 == 0: i < R implies i + 1 < R
        *(uint32_t*)(T + (int64_t)m * ldt + i) = f32_to_bf16_bits(a0) | (f32_to_bf16_bits(a1) << 16);
    }
    __syncthreads();
  }

  // The quant: pass 1, x_s and its row max. While the registers allow (a
  // 16-wave block leaves 128 per lane), x_s stays in registers for pass 2: one
  // read of the reciprocal table per element; otherwise pass 2 forms it again.
  constexpr bool kStoreV = W <= 8 ? CPL <= 8 : CPL <= 4;
  float v[kStoreV ? CPL : 1][8];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int k = kof(j);
    if (k < K) {
      float x[8];
      widen8<XT>(&xr[j], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = div_rn(x[e], rtab[k + e]);
        if constexpr (kStoreV) v[j][e] = y;
        amax = __builtin_fmaxf(amax, __builtin_fabsf(y));
      }
    }
  }
  float scale;
  if (is_static) {
    scale = scale_io[0];
  } else {
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16, kWave));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32, kWave));
    if (kg == 0) rmax[wave][lrow] = amax;
    __syncthreads();
    amax = rmax[0][lrow];
#pragma unroll
    for (int w = 1; w < W; ++w) amax = __builtin_fmaxf(amax, rmax[w][lrow]);
    scale = amax / 127.0f;                                       // IEEE fp32 division
    if (wave == 0 && kg == 0 && row_ok) scale_io[m0 + lrow] = scale;
  }
  if (!row_ok) return;
  const double rscale = scale != 0.0f ? rcp_rn64(scale) : 0.0;
  const uint32_t keep = scale != 0.0f ? 0xFFFFFFFFu : 0u;
  int8_t* orow = Xq + (int64_t)(m0 + lrow) * K;
  // pass 2: the codes
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int k = kof(j);
    if (k < K) {
      float y[8];
      if constexpr (kStoreV) {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = v[j][e];
      } else {
        widen8<XT>(&xr[j], y);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = div_rn(y[e], rtab[k + e]);
      }
      uint32_t q[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = code_word(div_rn(y[e], rscale));
      uint2 pk;
      pk.x = pack4_codes(q[0], q[1], q[2], q[3]) & keep;
      pk.y = pack4_codes(q[4], q[5], q[6], q[7]) & keep;
      *(uint2*)(orow + k) = pk;
    }
  }
}

// ---------------------------------------------------------------------------
// Host launcher.
// ---------------------------------------------------------------------------
// The fused kernel covers bf16 X up to K = 8192 and fp16 X up to 4096 (the
// fp16 -> bf16 rounding of the shrink operand needs registers that 32 chunks
// per lane leave no room for), R <= 128.
int64_t quant_shrink_max_k(int xt) { return xt == SQ_BF16 ? 8192 : xt == SQ_F16 ? 4096 : 0; }

template <int XT, int W, int CPL, int KMAX>
static void launch_qs_nt(int nt, const char* x, int64_t ldb, int M, int K, const float* s,
                         int is_static, float* a, int8_t* Xq, const unsigned short* A, int R,
                         unsigned short* T, int64_t ldt, unsigned blocks, hipStream_t st) {
#define SQ_QS(NT_)                                                                            \
  k_quant_shrink<XT, W, CPL, NT_, KMAX><<<blocks, W * 64, 0, st>>>(x, ldb, M, K, s, is_static, a, \
                                                                   Xq, A, R, T, ldt)
  switch (nt) {
    case 1: SQ_QS(1); break;
    case 2: SQ_QS(2); break;
    case 3: SQ_QS(3); break;
    case 4: SQ_QS(4); break;
    default: SQ_QS(8); break;
  }
#undef SQ_QS
}

template <int XT>
static void launch_qs_dt(const char* x, int64_t ldb, int M, int K, const float* s, int is_static,
                         float* a, int8_t* Xq, const unsigned short* A, int R, unsigned short* T,
                         int64_t ldt, hipStream_t st) {
  const unsigned blocks = (unsigned)((M + kQSRows - 1) / kQSRows);
  const int nt = (R + 15) / 16;
  const int steps = (K + 31) / 32;
  // 16 waves per block up to K = 4096: a block of 16 rows is one CU's work, so
  // its waves are what hides the latency of the X and A loads.
  if (steps <= 16 * 4)
    launch_qs_nt<XT, 16, 4, 2048>(nt, x, ldb, M, K, s, is_static, a, Xq, A, R, T, ldt, blocks, st);
  else if (steps <= 16 * 8 && (XT == SQ_BF16 || nt <= 4))
    launch_qs_nt<XT, 16, 8, 4096>(nt, x, ldb, M, K, s, is_static, a, Xq, A, R, T, ldt, blocks, st);
  else if (steps <= 16 * 8)   // fp16, ranks above 64: the bf16 rounding needs 8 waves' registers
    k_quant_shrink<XT, 8, 16, 8, 4096><<<blocks, 512, 0, st>>>(x, ldb, M, K, s, is_static, a, Xq, A,
                                                                 R, T, ldt);
  else if constexpr (XT == SQ_BF16)   // 32 chunks per lane: 8 waves (2 per SIMD), up to 256 registers each
    launch_qs_nt<XT, 8, 32, 8192>(nt, x, ldb, M, K, s, is_static, a, Xq, A, R, T, ldt, blocks, st);
}

int launch_quant_shrink(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const float* s,
                        int mode, int8_t* Xq, float* a_scale, const void* A, int r, void* T,
                        int64_t ldt, hipStream_t st) {
  if (M == 0) return SQ_OK;
  const int is_static = mode == SQ_ACT_PER_TENSOR_STATIC;
  const char* x = (const char*)X;
  if (xt == SQ_BF16)
    launch_qs_dt<SQ_BF16>(x, ldx * 2, (int)M, (int)K, s, is_static, a_scale, Xq,
                          (const unsigned short*)A, r, (unsigned short*)T, ldt, st);
  else
    launch_qs_dt<SQ_F16>(x, ldx * 2, (int)M, (int)K, s, is_static, a_scale, Xq,
                         (const unsigned short*)A, r, (unsigned short*)T, ldt, st);
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

}  // namespace sq
