// INT8 x INT8 -> INT32 GEMM with the dequant epilogue ([SQ] Step 7):
//   acc[m, n] = sum_k Xq[m, k] * Wq[n, k]            (exact INT32)
//   Y[m, n]   = out((fp32(acc) * a_scale[m]) * w_scale[n])
//
// Both operands are K-contiguous ([M, K] and [N, K]), the layout the gfx950
// INT8 matrix instruction V_MFMA_I32_32X32X32_I8 wants for both of its inputs:
// each lane supplies 16 consecutive k-bytes of one row. Tiles of both
// operands are staged through LDS with 16-byte global loads, double-buffered
// so the next K-tile is in flight while the current one feeds the MFMAs.
//
// LDS layout: a tile row holds BK = 128 bytes = 8 chunks of 16 bytes; chunk c
// of row r is stored at chunk position c ^ (r & 7). The MFMA operand read has
// 32 lanes reading the same logical chunk of 32 consecutive rows; the XOR
// spreads any 8 consecutive rows over all 8 chunk positions (all 32 banks),
// so the 16-byte reads are free of bank conflicts, and the 8 lanes that fill
// one row on the store side also hit 8 distinct positions.
#include "sq_internal.h"

namespace sq {

constexpr int kBM = 128, kBN = 128, kBK = 128;   // block tile (bytes along K)
constexpr int kGemmThreads = 256;                // 4 waves, 2 x 2, 64 x 64 each

enum OutKind { OUT_I32 = 0, OUT_BF16 = 1, OUT_F16 = 2, OUT_F32 = 3 };

template <int OUT>
__device__ __forceinline__ void store_out(void* Y, int64_t ldy, int64_t m, int64_t n, int acc,
                                          float as, float ws) {
  if constexpr (OUT == OUT_I32) {
    ((int32_t*)Y)[m * ldy + n] = acc;
  } else {
    const float y = ((float)acc * as) * ws;        // two fp32 roundings, left to right
    if constexpr (OUT == OUT_F32) ((float*)Y)[m * ldy + n] = y;
    else if constexpr (OUT == OUT_BF16) ((unsigned short*)Y)[m * ldy + n] = (unsigned short)f32_to_bf16_bits(y);
    else ((unsigned short*)Y)[m * ldy + n] = (unsigned short)f32_to_f16_bits(y);
  }
}

template <int OUT, bool STATIC_A>
__global__ void __launch_bounds__(kGemmThreads)
k_w8a8_gemm(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
            const float* __restrict__ a_scale, const float* __restrict__ w_scale, int M, int N,
            int K, void* __restrict__ Y, int64_t ldy) {
  __shared__ __attribute__((aligned(16))) char sA[2][kBM * kBK];
  __shared__ __attribute__((aligned(16))) char sB[2][kBN * kBK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Tile order: consecutive blocks walk down M within a column of N tiles, so
  // blocks running at the same time share their Wq tile through L2.
  const int tiles_m = (M + kBM - 1) / kBM;
  const int bm = blockIdx.x % tiles_m;
  const int bn = blockIdx.x / tiles_m;
  const int m0 = bm * kBM, n0 = bn * kBN;

  // Global -> LDS: 1024 chunks of 16 bytes per operand tile, 4 per thread.
  // Thread t moves chunks t + 256 i: row = id / 8, chunk = id % 8.
  const int64_t ldk = K;
  const int nk = (K + kBK - 1) / kBK;
  uint4 ra[4], rb[4];

  auto gload = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + i * kGemmThreads;
      const int r = id >> 3, c = id & 7;
      const int kk = k0 + c * 16;
      int ma = m0 + r; ma = ma < M ? ma : M - 1;
      int nb = n0 + r; nb = nb < N ? nb : N - 1;
      if (kk < K) {
        ra[i] = *(const uint4*)(A + (int64_t)ma * ldk + kk);
        rb[i] = *(const uint4*)(B + (int64_t)nb * ldk + kk);
      } else {
        ra[i] = make_uint4(0, 0, 0, 0);
        rb[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + i * kGemmThreads;
      const int r = id >> 3, c = id & 7;
      const int off = r * kBK + ((c ^ (r & 7)) << 4);
      *(uint4*)(&sA[buf][off]) = ra[i];
      *(uint4*)(&sB[buf][off]) = rb[i];
    }
  };

  v16i acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16i{};

  gload(0);
  sstore(0);
  __syncthreads();

  const int lrow = lane & 31;       // row within a 32-row MFMA operand
  const int lhalf = lane >> 5;      // which 16-byte half of a 32-byte k step
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      const int c = ks * 2 + lhalf;
      v4i fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + lrow;
        fa[i] = *(const v4i*)(&sA[buf][r * kBK + ((c ^ (r & 7)) << 4)]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + j * 32 + lrow;
        fb[j] = *(const v4i*)(&sB[buf][r * kBK + ((c ^ (r & 7)) << 4)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue. Output register q of a 32x32 tile holds row 8*(q/4) + 4*(lane/32)
  // + q%4 and column lane%32.
  const float as_static = STATIC_A && OUT != OUT_I32 ? a_scale[0] : 0.0f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + lrow;
    if (n >= N) continue;
    const float ws = OUT != OUT_I32 ? w_scale[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (q >> 2) + 4 * lhalf + (q & 3);
        if (m < M) {
          const float as = OUT == OUT_I32 ? 0.0f : (STATIC_A ? as_static : a_scale[m]);
          store_out<OUT>(Y, ldy, m, n, acc[i][j][q], as, ws);
        }
      }
    }
  }
}

template <int OUT, bool STATIC_A>
static int launch_gemm_t(const int8_t* Xq, const int8_t* Wq, const float* a_scale,
                         const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y,
                         int64_t ldy, hipStream_t st) {
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  k_w8a8_gemm<OUT, STATIC_A><<<(unsigned)tiles, kGemmThreads, 0, st>>>(
      Xq, Wq, a_scale, w_scale, (int)M, (int)N, (int)K, Y, ldy);
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

int launch_gemm(const int8_t* Xq, const int8_t* Wq, const float* a_scale, int mode,
                const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y, int yt,
                int64_t ldy, hipStream_t st) {
  if (M == 0) return SQ_OK;
  const bool stat = mode == SQ_ACT_PER_TENSOR_STATIC;
  switch (yt) {
    case SQ_BF16: return stat ? launch_gemm_t<OUT_BF16, true>(Xq, Wq, a_scale, w_scale, M, N, K, Y, ldy, st)
                              : launch_gemm_t<OUT_BF16, false>(Xq, Wq, a_scale, w_scale, M, N, K, Y, ldy, st);
    case SQ_F16:  return stat ? launch_gemm_t<OUT_F16, true>(Xq, Wq, a_scale, w_scale, M, N, K, Y, ldy, st)
                              : launch_gemm_t<OUT_F16, false>(Xq, Wq, a_scale, w_scale, M, N, K, Y, ldy, st);
    default:      return stat ? launch_gemm_t<OUT_F32, true>(Xq, Wq, a_scale, w_scale, M, N, K, Y, ldy, st)
                              : launch_gemm_t<OUT_F32, false>(Xq, Wq, a_scale, w_scale, M, N, K, Y, ldy, st);
  }
}

int launch_gemm_i32(const int8_t* Xq, const int8_t* Wq, int64_t M, int64_t N, int64_t K,
                    int32_t* acc, hipStream_t st) {
  if (M == 0) return SQ_OK;
  return launch_gemm_t<OUT_I32, false>(Xq, Wq, nullptr, nullptr, M, N, K, acc, N, st);
}

}  // namespace sq
