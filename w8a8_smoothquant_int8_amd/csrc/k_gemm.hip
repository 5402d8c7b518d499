// INT8 x INT8 -> INT32 GEMM with the dequant epilogue ([SQ] Step 7):
//   acc[m, n] = sum_k Xq[m, k] * Wq[n, k]            (exact INT32)
//   Y[m, n]   = out((fp32(acc) * a_scale[m]) * w_scale[n])
//
// Both operands are K-contiguous ([M, K] and [N, K]), the layout the gfx950
// INT8 matrix instruction V_MFMA_I32_32X32X32_I8 wants for both inputs: each
// lane supplies 16 consecutive k-bytes of one row, lanes 0-31 and 32-63 the
// two 16-byte halves of a 32-byte k step.
//
// Main kernel (K a multiple of 128): block tile BM x BN, K-tile 128 bytes,
// 2-stage LDS ring filled straight from global memory by buffer loads into
// LDS (no register staging; a 32-bit per-lane offset and a scalar K-tile
// offset, so no 64-bit address arithmetic per load). One wave instruction
// moves 1 KB = 8 tile rows into consecutive LDS; each lane picks which 16-byte chunk
// of its row to fetch so that the tile lands XOR-swizzled (swz below) and the
// MFMA operand reads are free of bank conflicts. Tiles are assigned XCD by
// XCD: the hardware deals workgroups round-robin to the 8 XCDs, so block b
// runs on XCD b % 8; each XCD gets a contiguous run of the tile order, which
// walks patches of 8 tile rows column by column, so the blocks an XCD runs at
// once share operand panels in its L2.
//
// Decode kernel (M <= 64, no LoRA): 64-column blocks over all rows with a
// 4-slot LDS ring (three K-tiles in flight), K split across blocks through a
// workspace where the column blocks alone are too few.
//
// Skinny kernel (M <= 64 with the LoRA epilogue, narrow N): 32-column blocks
// over all rows, K split across the block's waves, fragments straight from
// global memory.
//
// Generic kernel (any K multiple of 16): 128 x 128 tiles staged through
// registers, zero-filling the K tail.
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "sq_internal.h"

namespace sq {

enum OutKind { OUT_I32 = 0, OUT_BF16 = 1, OUT_F16 = 2, OUT_F32 = 3 };

// LDS position of 16-byte chunk c of tile row r (rows are 128 bytes). gfx950
// LDS has 64 banks (256 bytes); a 16-byte read serves 16 lanes per cycle. The
// MFMA operand read has 16 lanes reading the same logical chunk of 16
// consecutive rows: even rows share bank half 0, odd rows half 1, and
// c ^ ((r >> 1) & 7) gives the 8 even (and the 8 odd) rows 8 distinct chunk
// positions, so the 16 lanes cover all 64 banks once.
__device__ __forceinline__ int swz(int r, int c) { return (c ^ ((r >> 1) & 7)) << 4; }

// Optional LoRA delta added in the epilogue ([LoRA] Pitch): T [M, r] bf16
// (row stride ldt) and B [N, r] bf16, Y = out(out(y) + scale * T B^T).
//
// Parts: adapters of projections that share one input are stacked along r,
// and B is block-diagonal (part p = columns [n_end[p-1], n_end[p]) uses only
// ranks [r_end[p-1], r_end[p]); B is zero elsewhere). A tile then multiplies
// only the ranks of the parts its columns touch, rounded out to whole 16-rank
// MFMA steps: the steps it leaves out hold only zero products, and the steps
// it keeps are the same 16-aligned steps in the same order, so the result is
// that of the full rank range bit for bit. parts <= 1: every column uses all
// r ranks.
constexpr int kMaxLoraParts = 4;
struct LoraEpi {
  const unsigned short* T;
  int64_t ldt;
  const unsigned short* B;
  int r;
  float scale;
  int parts;
  int n_end[kMaxLoraParts];
  int r_end[kMaxLoraParts];
};

// Rank window [klo, khi) for output columns [c0, c1) (c1 exclusive, c0 < c1).
__device__ __forceinline__ void lora_window(const LoraEpi& le, int c0, int c1, int& klo, int& khi) {
  if (le.parts <= 1) {
    klo = 0;
    khi = le.r;
    return;
  }
  int plo = 0;
  while (plo + 1 < le.parts && le.n_end[plo] <= c0) ++plo;
  int phi = plo;
  while (phi + 1 < le.parts && le.n_end[phi] < c1) ++phi;
  klo = (plo == 0 ? 0 : le.r_end[plo - 1]) & ~15;
  khi = (le.r_end[phi] + 15) & ~15;
  khi = khi < le.r ? khi : le.r;
}

// Map a block to its (tile_m, tile_n), grouping tiles by XCD. Returns false
// for padding blocks beyond the last tile.
// Within the tile order, tiles go in groups of kGroupM tile rows: a group
// walks its kGroupM x tiles_n patch column by column, so the 32 blocks an XCD
// runs at once cover about 8 x 4 tiles and share 8 A panels and 4 B panels.
constexpr int kGroupM = 8;
__device__ __forceinline__ bool xcd_tile(int tiles_m, int tiles, int& tm, int& tn) {
  const int per = (tiles + 7) / 8;
  const int t = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (t >= tiles) return false;
  const int tiles_n = tiles / tiles_m;
  const int group = t / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gsize = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  const int in = t - group * kGroupM * tiles_n;
  tm = first_m + in % gsize;
  tn = in / gsize;
  return true;
}

constexpr int kBK = 128;          // K-tile in bytes
// Word 3 of a raw buffer resource (no stride, no swizzle, 32-bit data format).
constexpr int kBufferRsrcWord3 = 0x00020000;
// s_waitcnt immediate for vmcnt(vm) lgkmcnt(0) (vmcnt in bits 3:0 and 15:14).
constexpr int wait_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | 0x0070; }

// Epilogue shared by both kernels. The MFMAs take the B rows as their first
// operand and the A rows as their second, so acc[i][j] holds the 32x32 tile
// transposed: output register q holds row m = row0 + 32 i + lane % 32 and
// column n = col0 + 32 j + 8 (q / 4) + 4 (lane / 32) + q % 4. Each lane thus
// has 4 consecutive columns of one row per register group.
//
// With LORA, the rank-r product for the same tile comes from
// V_MFMA_F32_32X32X16_BF16 with the B rows first and the T rows second, whose
// output has that same layout, so it lines up register for register with the
// INT32 accumulators. When scale is 1 the accumulators are first turned in
// place into the output-rounded GEMM values, and the bf16 MFMAs accumulate
// T B^T straight onto them. Other scales keep a separate delta per tile. The
// MFMAs run in uniform control flow; rows and columns past M and N read
// clamped (valid) addresses and are never stored.
//
// 16-bit outputs are rounded two at a time by V_CVT_PK_BF16_F32 /
// V_CVT_PK_F16_F32 (round to nearest even). One V_PERMLANE32_SWAP per packed
// register pair then gives every lane 8 consecutive columns, stored as one
// 16-byte piece: lane l < 32 holds columns 0-7 of a 16-column group, lane
// l + 32 columns 8-15.
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int OUT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (OUT == OUT_BF16) {
    const bf16x2 p = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, p);
  } else {
    // The empty register barrier keeps the compiler from folding a preceding
    // fp32 multiply into a mixed-precision FMA that rounds once, straight to
    // fp16; the path's semantics are an fp32 rounding, then an fp16 one.
    asm volatile("" : "+v"(a), "+v"(b));
    const f16x2 p = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, p);
  }
}

// Round a pair of fp32 values to the 16-bit output type and back (exact).
template <int OUT>
__device__ __forceinline__ void round2(float& a, float& b) {
  const uint32_t p = pack2<OUT>(a, b);
  if constexpr (OUT == OUT_BF16) {
    a = __uint_as_float(p << 16);
    b = __uint_as_float(p & 0xFFFF0000u);
  } else {
    a = f16_bits_to_f32(p & 0xFFFFu);
    b = f16_bits_to_f32(p >> 16);
  }
}

template <int OUT>
__device__ __forceinline__ float round_out(float y) {
  if constexpr (OUT == OUT_BF16) return bf16_bits_to_f32(f32_to_bf16_bits(y));
  else if constexpr (OUT == OUT_F16) return f16_bits_to_f32(f32_to_f16_bits(y));
  else return y;
}

// Store one transposed 32x32 tile of final fp32 values (or INT32 bits for
// OUT_I32): rows m = m_base + lane % 32, columns n_base + 0..31.
template <int OUT>
__device__ __forceinline__ void store_tile(const v16i& v, int64_t m, bool m_ok, int n_base, int N,
                                           void* __restrict__ Y, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int lhalf = lane >> 5;
  if constexpr (OUT == OUT_BF16 || OUT == OUT_F16) {
    const v16f y = __builtin_bit_cast(v16f, v);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      // groups g = 2p (columns 16p + 4 lhalf + 0..3) and 2p + 1 (16p + 8 + ...)
      uint32_t lo0 = pack2<OUT>(y[8 * p + 0], y[8 * p + 1]);
      uint32_t lo1 = pack2<OUT>(y[8 * p + 2], y[8 * p + 3]);
      uint32_t hi0 = pack2<OUT>(y[8 * p + 4], y[8 * p + 5]);
      uint32_t hi1 = pack2<OUT>(y[8 * p + 6], y[8 * p + 7]);
      const auto s0 = __builtin_amdgcn_permlane32_swap(lo0, hi0, false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(lo1, hi1, false, false);
      const int n = n_base + 16 * p + 8 * lhalf;
      if (m_ok && n < N)
        *(uint4*)((unsigned short*)Y + m * ldy + n) = make_uint4(s0[0], s1[0], s0[1], s1[1]);
    }
  } else {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = n_base + 8 * g + 4 * lhalf;
      if (m_ok && n < N)
        *(v4i*)((int32_t*)Y + m * ldy + n) = v4i{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
    }
  }
}

// Non-staged epilogue (the generic kernel, INT32 output, and LoRA with a
// scale other than 1): scales and LoRA fragments straight from global memory.
// LORA: 0 none, 1 LoRA delta with scale 1 (accumulated onto y in place),
// 2 LoRA delta with any scale (separate delta per tile).
template <int OUT, bool STATIC_A, int LORA, int TM, int TN>
__device__ __forceinline__ void epilogue(v16i (&acc)[TM][TN], int row0, int col0, int M, int N,
                                         const float* __restrict__ a_scale,
                                         const float* __restrict__ w_scale, void* __restrict__ Y,
                                         int64_t ldy, const LoraEpi& le) {
  const int lane = threadIdx.x & 63;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const float as_static = (STATIC_A && OUT != OUT_I32) ? a_scale[0] : 0.0f;
  int klo = 0, khi = 0;
  if constexpr (LORA != 0) lora_window(le, col0, col0 + 32 * TN < N ? col0 + 32 * TN : N, klo, khi);
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    float ws[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int n = col0 + j * 32 + 8 * (q >> 2) + 4 * lhalf + (q & 3);
      ws[q] = (OUT != OUT_I32 && n < N) ? w_scale[n] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = row0 + i * 32 + lrow;
      const bool m_ok = m < M;
      if constexpr (OUT != OUT_I32) {
        const float as = STATIC_A ? as_static : (m_ok ? a_scale[m] : 0.0f);
        v16f y;
#pragma unroll
        for (int q = 0; q < 16; ++q) y[q] = ((float)acc[i][j][q] * as) * ws[q];   // two roundings, left to right
        if constexpr (LORA != 0) {
          const int64_t mr = m_ok ? m : M - 1;
          const int64_t nr = col0 + j * 32 + lrow < N ? col0 + j * 32 + lrow : N - 1;
          // scale 1: accumulate onto the rounded GEMM values, as the staged epilogue does
          v16f d;
#pragma unroll
          for (int q = 0; q < 16; ++q) d[q] = LORA == 1 ? round_out<OUT>(y[q]) : 0.0f;
          for (int k0 = klo; k0 < khi; k0 += 16) {
            const int k = k0 + 8 * lhalf;
            uint4 tu = make_uint4(0, 0, 0, 0), bu = make_uint4(0, 0, 0, 0);
            if (k < khi) {
              tu = *(const uint4*)(le.T + mr * le.ldt + k);
              bu = *(const uint4*)(le.B + nr * le.r + k);
            }
            d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, bu),
                                                        __builtin_bit_cast(v8bf, tu), d, 0, 0, 0);
          }
#pragma unroll
          for (int q = 0; q < 16; ++q) y[q] = LORA == 1 ? d[q] : round_out<OUT>(y[q]) + le.scale * d[q];
        }
        store_tile<OUT>(__builtin_bit_cast(v16i, y), m, m_ok, col0 + j * 32, N, Y, ldy);
      } else {
        store_tile<OUT>(acc[i][j], m, m_ok, col0 + j * 32, N, Y, ldy);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// LDS-staged epilogue of the main kernel (16-bit or fp32 output; no LoRA, or
// LoRA with scale 1). Its operands are already in LDS when the K loop ends:
//   - the block's a_scale and w_scale slices, requested with direct
//     global->LDS loads at the start of the kernel into a region of their own;
//   - the T and B rows of the first 64 LoRA ranks, requested at the sync point
//     of the K-tile before the last, into the ring stage it releases (at the
//     start of the kernel when there is a single K-tile).
// The K loop's last wait and barrier cover both. More than 64 ranks: the next
// 64 go through the same stage, one wait and two barriers per pass.
// Values and operation order are those of the epilogue above.
// ---------------------------------------------------------------------------
constexpr int kStageRanks = 64;

// Direct global->LDS copy of `count` 4-byte words from src[idx(i)] to dst[i]
// (one 64-word load per wave instruction), shared by the block's waves.
template <int NW, typename Idx>
__device__ __forceinline__ void stage_words(const float* src, char* dst, int count, int wave,
                                            int lane, Idx idx) {
  for (int base = wave * 64; base < count; base += NW * 64) {
    const int i = base + lane;
    if (i < count)
      __builtin_amdgcn_global_load_lds((const void*)(src + idx(i)), (lds_ptr_t)(dst + 4 * base), 4,
                                       0, 0);
  }
}

// Direct copy of `rows` rows of `r16` 16-byte chunks each: row i of the LDS
// tile (packed, r16 chunks per row) from src + row_off(i) (bytes).
template <int NW, typename RowOff>
__device__ __forceinline__ void stage_rows(const char* src, char* dst, int rows, int r16, int wave,
                                           int lane, RowOff row_off) {
  const int total = rows * r16;
  for (int base = wave * 64; base < total; base += NW * 64) {
    const int g = base + lane;
    if (g < total) {
      const int row = g / r16, ch = g - row * r16;
      __builtin_amdgcn_global_load_lds((const void*)(src + row_off(row) + 16 * ch),
                                       (lds_ptr_t)(dst + 16 * base), 16, 0, 0);
    }
  }
}

// LoRA ranks [k_base, k_base + 64) of the block's T rows and B rows into LDS
// at dst: T [BM][rp] then B [BN][rp] bf16, rp = min(64, khi - k_base).
template <int NW, int BM, int BN>
__device__ __forceinline__ void stage_lora(const LoraEpi& le, char* dst, int k_base, int khi, int m0,
                                           int n0, int M, int N, int wave, int lane) {
  const int rp = khi - k_base < kStageRanks ? khi - k_base : kStageRanks;
  const int r16 = rp / 8;
  stage_rows<NW>((const char*)le.T, dst, BM, r16, wave, lane, [&](int row) -> int64_t {
    const int64_t m = m0 + row < M ? m0 + row : M - 1;
    return (m * le.ldt + k_base) * 2;
  });
  stage_rows<NW>((const char*)le.B, dst + 2 * BM * rp, BN, r16, wave, lane, [&](int row) -> int64_t {
    const int64_t n = n0 + row < N ? n0 + row : N - 1;
    return (n * le.r + k_base) * 2;
  });
}

template <int OUT, bool STATIC_A, int LORA, int BM, int BN, int WM, int WN>
__device__ __forceinline__ void epilogue_staged(v16i (&acc)[BM / WM / 32][BN / WN / 32],
                                                const char* s_sc, char* s_lora, int m0, int n0,
                                                int wm, int wn, int M, int N,
                                                const float* __restrict__ a_scale, void* __restrict__ Y,
                                                int64_t ldy, const LoraEpi& le, int klo, int khi,
                                                char* s_out /* the ring, 2 BM BN bytes free */) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int row0 = wm * (BM / WM), col0 = wn * (BN / WN);   // wave sub-tile within the block
  const char* s_as = s_sc;            // [BM] fp32
  const char* s_ws = s_sc + 4 * BM;   // [BN] fp32

  // y = out((fp32(acc) * a_scale[m]) * w_scale[n]), in place in the accumulators
  // (rounded to the output type only when the LoRA delta is added after it)
  const float as_static = STATIC_A ? a_scale[0] : 0.0f;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    float ws[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 v = *(const float4*)(s_ws + 4 * (col0 + j * 32 + 8 * g + 4 * lhalf));
      ws[4 * g] = v.x; ws[4 * g + 1] = v.y; ws[4 * g + 2] = v.z; ws[4 * g + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const float as = STATIC_A ? as_static : *(const float*)(s_as + 4 * (row0 + i * 32 + lrow));
      float t[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) t[q] = ((float)acc[i][j][q] * as) * ws[q];
      if constexpr (LORA == 1 && OUT != OUT_F32) {
#pragma unroll
        for (int q = 0; q < 16; q += 2) round2<OUT>(t[q], t[q + 1]);
      }
      v16f tv;
#pragma unroll
      for (int q = 0; q < 16; ++q) tv[q] = t[q];
      acc[i][j] = __builtin_bit_cast(v16i, tv);
    }
  }

  if constexpr (LORA == 1) {
    for (int k_base = klo; k_base < khi; k_base += kStageRanks) {
      if (k_base > klo) {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's reads of the last pass are done
        __builtin_amdgcn_s_barrier();         // every wave is done with the previous ranks
        stage_lora<NW, BM, BN>(le, s_lora, k_base, khi, m0, n0, M, N, wave, lane);
        __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
      }
      const int rp = khi - k_base < kStageRanks ? khi - k_base : kStageRanks;
      const char* s_t = s_lora;
      const char* s_b = s_lora + 2 * BM * rp;
      for (int k0 = 0; k0 < rp; k0 += 16) {
        const int k = k0 + 8 * lhalf;          // rank within this pass
        const bool kin = k < rp;
        uint4 tf[TM], bf[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
          tf[i] = kin ? *(const uint4*)(s_t + 2 * ((row0 + i * 32 + lrow) * rp + k)) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bf[j] = kin ? *(const uint4*)(s_b + 2 * ((col0 + j * 32 + lrow) * rp + k)) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_bit_cast(
                v16i, __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, bf[j]),
                                                              __builtin_bit_cast(v8bf, tf[i]),
                                                              __builtin_bit_cast(v16f, acc[i][j]),
                                                              0, 0, 0));
      }
    }
  }

  if constexpr (OUT == OUT_BF16 || OUT == OUT_F16) {
    // The output tile goes through the (now free) LDS ring, row r's 16-byte
    // slot c at (c + r) % (BN / 8), and leaves in whole rows: one store
    // instruction writes 1 KB of consecutive row bytes instead of 32 bytes of
    // each of 32 rows, and the round's output burst (every block ends its
    // tile at about the same time) takes fewer write requests: the fixed cost
    // per round of tiles fell from 13.2 to 11.4 us at 8192 x 57344.
    // Needs 2 BM BN bytes, at most the ring's two stages.
    constexpr int SPR = BN / 8;
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = row0 + i * 32 + lrow;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v16f y = __builtin_bit_cast(v16f, acc[i][j]);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          uint32_t lo0 = pack2<OUT>(y[8 * p + 0], y[8 * p + 1]);
          uint32_t lo1 = pack2<OUT>(y[8 * p + 2], y[8 * p + 3]);
          uint32_t hi0 = pack2<OUT>(y[8 * p + 4], y[8 * p + 5]);
          uint32_t hi1 = pack2<OUT>(y[8 * p + 6], y[8 * p + 7]);
          const auto s0 = __builtin_amdgcn_permlane32_swap(lo0, hi0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(lo1, hi1, false, false);
          const int c = (col0 + j * 32 + 16 * p + 8 * lhalf) / 8;
          *(uint4*)(s_out + r * (BN * 2) + (((c + r) % SPR) << 4)) = make_uint4(s0[0], s1[0], s0[1], s1[1]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    const int tid = threadIdx.x;
    constexpr int T = NW * 64;
    constexpr int RPI = T / SPR;            // rows per pass
    const int s = tid % SPR;
#pragma unroll 4
    for (int r = tid < RPI * SPR ? tid / SPR : BM; r < BM; r += RPI) {
      const int m = m0 + r, n = n0 + 8 * s;
      const v4u v = *(const v4u*)(s_out + r * (BN * 2) + (((s + r) % SPR) << 4));
      // Non-temporal: the output is not read again by this kernel, and its
      // lines would otherwise displace operand panels from L2 (gate+up
      // 8192x57344x8192 -0.5%, down 8192x8192x28672 -1.3%, alternated runs).
      if (m < M && n < N) __builtin_nontemporal_store(v, (v4u*)((unsigned short*)Y + (int64_t)m * ldy + n));
    }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + row0 + i * 32 + lrow;
#pragma unroll
      for (int j = 0; j < TN; ++j) store_tile<OUT>(acc[i][j], m, m < M, n0 + col0 + j * 32, N, Y, ldy);
    }
  }
}

// ---------------------------------------------------------------------------
// Main kernel, K % 128 == 0. WM x WN waves; each wave owns a (BM/WM) x (BN/WN)
// sub-tile of 32x32 MFMA tiles. The MFMA operand fragments are double-buffered
// in registers: the LDS reads for k-step s+1 are in flight while the MFMAs of
// k-step s run (scheduling hints put one read after each MFMA). Two K-tiles
// of direct loads are in flight, and each K-tile has one sync point, in its
// last k-step: wait, barrier, then the loads of the K-tile after next and the
// reads of the next K-tile's first fragments, interleaved with that k-step's
// MFMAs. The barrier carries no memory fence (a fence would also wait for
// direct loads still meant to be in flight): each wave waits for its own
// direct loads of the next K-tile (vmcnt) and its reads of this one (lgkmcnt),
// then all waves meet.
// ---------------------------------------------------------------------------
// Scheduling-group pattern for one k-step of NMF MFMAs: each MFMA is followed
// by one LDS read while the NR reads last, and the NV direct loads are spread
// over the MFMAs.
template <int U, int NMF, int NR, int NV>
__device__ __forceinline__ void sched_slots() {
  if constexpr (U < NMF) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      // one MFMA
    if constexpr (U < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // one LDS read
    constexpr int c = ((U + 1) * NV) / NMF - (U * NV) / NMF;
    if constexpr (c > 0) __builtin_amdgcn_sched_group_barrier(0x060, c, 0);  // direct loads
    sched_slots<U + 1, NMF, NR, NV>();
  }
}

template <int BM, int BN, int WM, int WN, int OUT, bool STATIC_A, int LORA>
__global__ void __launch_bounds__(WM * WN * 64, 2)   // 2 waves per SIMD: 8-wave blocks, or 2 blocks of 4
k_gemm_pipe(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
            const float* __restrict__ a_scale, const float* __restrict__ w_scale, int M, int N,
            int K, void* __restrict__ Y, int64_t ldy, LoraEpi le) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  constexpr int STAGE = (BM + BN) * kBK;            // bytes per LDS stage
  constexpr int IA = BM / 8 / NW, IB = BN / 8 / NW; // 1 KB direct loads per wave per stage
  constexpr int KS = kBK / 32;                      // MFMA k-steps per K-tile
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile rows must split over waves");
  constexpr bool STAGED = OUT != OUT_I32 && LORA != 2;   // epilogue operands staged in LDS
  static_assert((BM + BN) * 2 * kStageRanks <= STAGE, "64 LoRA ranks must fit one ring stage");
  static_assert(2 * BM * BN <= 2 * STAGE, "a 16-bit output tile must fit the ring");
  // ring of 2 stages, then the block's a_scale [BM] and w_scale [BN] slices
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE + (STAGED ? 4 * (BM + BN) : 0)];
  char* const s_sc = smem + 2 * STAGE;

  const int tiles_m = (M + BM - 1) / BM;
  const int tiles = tiles_m * ((N + BN - 1) / BN);
  int tm, tn;
  if (!xcd_tile(tiles_m, tiles, tm, tn)) return;
  const int m0 = tm * BM, n0 = tn * BN;
  int klo = 0, khi = 0;   // the block's LoRA rank window
  if constexpr (LORA == 1 && STAGED) lora_window(le, n0, n0 + BN < N ? n0 + BN : N, klo, khi);

  const int lane = threadIdx.x & 63;
  // wave index as a scalar: the LDS destination of a direct load must be uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane >> 3, lp = lane & 7;

  // 32-bit per-lane source offsets (operands < 4 GiB; checked by the host).
  // Load instruction q of this wave moves tile rows 8 (wave + NW q) + 0..7;
  // lane l fetches the chunk that belongs at position l & 7 of row l / 8.
  // Rows past M or N read the last valid row; their results are never stored.
  uint32_t offA[IA], offB[IB];
#pragma unroll
  for (int q = 0; q < IA; ++q) {
    const int r = 8 * (wave + NW * q) + lr;
    int g = m0 + r; g = g < M ? g : M - 1;
    offA[q] = (uint32_t)g * (uint32_t)K + (uint32_t)swz(r, lp);
  }
#pragma unroll
  for (int q = 0; q < IB; ++q) {
    const int r = 8 * (wave + NW * q) + lr;
    int g = n0 + r; g = g < N ? g : N - 1;
    offB[q] = (uint32_t)g * (uint32_t)K + (uint32_t)swz(r, lp);
  }

  // Buffer loads straight into LDS: the per-lane offset is a 32-bit VGPR and
  // the K-tile's offset a scalar, so a load costs no address arithmetic (the
  // 64-bit global form needs two VALU adds per load and was 2-3% slower).
  // The resource's size is the operand's, so no access can leave it.
  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)((uint32_t)M * (uint32_t)K), kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsB =
      __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, (int)((uint32_t)N * (uint32_t)K), kBufferRsrcWord3);
  auto issue = [&](int kt, int stage) {
    char* sa = smem + stage * STAGE;
    char* sb = sa + BM * kBK;
    const int koff = kt * kBK;
#pragma unroll
    for (int q = 0; q < IA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_ptr_t)(sa + 1024 * (wave + NW * q)), 16,
                                               (int)offA[q], koff, 0, 0);
#pragma unroll
    for (int q = 0; q < IB; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_ptr_t)(sb + 1024 * (wave + NW * q)), 16,
                                               (int)offB[q], koff, 0, 0);
  };

  const int lrow = lane & 31, lhalf = lane >> 5;
  int rowA[TM], rowB[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) rowA[i] = wm * (BM / WM) + i * 32 + lrow;
#pragma unroll
  for (int j = 0; j < TN; ++j) rowB[j] = wn * (BN / WN) + j * 32 + lrow;

  auto load_frags = [&](const char* sa, int ks, v4i* fa, v4i* fb) {
    const char* sb = sa + BM * kBK;
    const int c = ks * 2 + lhalf;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = *(const v4i*)(sa + rowA[i] * kBK + swz(rowA[i], c));
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = *(const v4i*)(sb + rowB[j] * kBK + swz(rowB[j], c));
  };

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};
  v4i fa[2][TM], fb[2][TN];   // operand fragments, double-buffered over k-steps

  const int nk = K / kBK;
  constexpr int NL = IA + IB;                       // direct loads per wave per K-tile
  static_assert(NL < 16, "vmcnt immediate below");
  auto mfmas = [&](int cur) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[cur][j], fa[cur][i], acc[i][j], 0, 0, 0);
  };
  auto stage_scales = [&]() {
    if constexpr (STAGED) {
      if constexpr (!STATIC_A)
        stage_words<NW>(a_scale, s_sc, BM, wave, lane, [&](int i) { return m0 + i < M ? m0 + i : M - 1; });
      stage_words<NW>(w_scale, s_sc + 4 * BM, BN, wave, lane,
                      [&](int i) { return n0 + i < N ? n0 + i : N - 1; });
    }
  };

  // Two K-tiles in flight. One sync point per K-tile, in its last k-step:
  // wait for this wave's loads of the next K-tile and its reads of this
  // one, barrier; then, interleaved with that k-step's MFMAs (whose
  // fragments are already in registers), the reads of the next K-tile's
  // first fragments and the loads of the K-tile after next into the stage
  // just released. Scheduling barriers keep every MFMA on its side of the
  // sync point.
  stage_scales();
  issue(0, 0);
  if (nk > 1) {
    issue(1, 1);
    __builtin_amdgcn_s_waitcnt(0x0070 | NL);   // vmcnt(NL) lgkmcnt(0): K-tile 0 and the scales
  } else {
    if constexpr (LORA == 1 && STAGED)
      stage_lora<NW, BM, BN>(le, smem + STAGE, klo, khi, m0, n0, M, N, wave, lane);
    __builtin_amdgcn_s_waitcnt(0x0070);
  }
  __builtin_amdgcn_s_barrier();
  load_frags(smem, 0, fa[0], fb[0]);

  // MODE 0: K-tiles kt + 1 and kt + 2 exist; 1: only kt + 1 (the free stage
  // takes the first LoRA ranks); 2: last K-tile.
  auto ktile = [&](int kt, auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    const int stage = kt & 1;
    const char* sa = smem + stage * STAGE;
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
      load_frags(sa, ks + 1, fa[(ks & 1) ^ 1], fb[(ks & 1) ^ 1]);
      mfmas(ks & 1);
      sched_slots<0, TM * TN, TM + TN, 0>();
    }
    constexpr int cur = (KS - 1) & 1;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0070);        // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MODE == 0) issue(kt + 2, stage);
    if constexpr (MODE == 1 && LORA == 1 && STAGED)
      stage_lora<NW, BM, BN>(le, smem + stage * STAGE, klo, khi, m0, n0, M, N, wave, lane);
    if constexpr (MODE != 2) load_frags(smem + (stage ^ 1) * STAGE, 0, fa[cur ^ 1], fb[cur ^ 1]);
    mfmas(cur);
    if constexpr (MODE == 0) sched_slots<0, TM * TN, TM + TN, NL>();
    else if constexpr (MODE == 1) sched_slots<0, TM * TN, TM + TN, 0>();
  };
  int kt = 0;
  for (; kt + 2 < nk; ++kt) ktile(kt, std::integral_constant<int, 0>{});
  if (kt + 1 < nk) ktile(kt++, std::integral_constant<int, 1>{});
  ktile(kt, std::integral_constant<int, 2>{});

  if constexpr (STAGED)
    epilogue_staged<OUT, STATIC_A, LORA, BM, BN, WM, WN>(acc, s_sc, smem + (((nk - 1) & 1) ^ 1) * STAGE,
                                                          m0, n0, wm, wn, M, N, a_scale, Y, ldy, le,
                                                          klo, khi, smem);
  else
    epilogue<OUT, STATIC_A, LORA, TM, TN>(acc, m0 + wm * (BM / WM), n0 + wn * (BN / WN), M, N,
                                          a_scale, w_scale, Y, ldy, le);
}

// ---------------------------------------------------------------------------
// Skinny kernel (M <= 64, K % 128 == 0): decode-sized GEMMs stream the
// weights once and are HBM-bound, and 128x128 tiles would leave most CUs
// idle (N = 5120 gives 40 of them). Here a block owns 32 output columns
// over all M rows (one row tile of 32 for M <= 32, two for M <= 64), and its
// 8 waves split K: wave w takes the 128-byte K-tiles w, w + 8, ... Operand
// fragments come straight from global memory into registers, double-buffered
// over the wave's K-tiles (the few A rows are shared by every block through
// L2). The waves' INT32 partial sums meet in LDS (exact in any order) and
// wave 0 runs the epilogue. Accumulators are transposed as in the other
// kernels (B rows as the first MFMA operand).
// ---------------------------------------------------------------------------
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyBN = 32;

template <int OUT, bool STATIC_A, int LORA, int TM>
__global__ void __launch_bounds__(kSkinnyWaves * 64)
k_gemm_skinny(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
              const float* __restrict__ a_scale, const float* __restrict__ w_scale, int M, int N,
              int K, void* __restrict__ Y, int64_t ldy, LoraEpi le) {
  __shared__ int32_t red[kSkinnyWaves - 1][TM][16][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * kSkinnyBN;
  const int lrow = lane & 31, lhalf = lane >> 5;
  // lane l supplies 16 bytes (k-half l / 32 of a 32-byte step) of row l % 32;
  // rows past N or M read the last valid row and are never stored
  const int nrow = n0 + lrow < N ? n0 + lrow : N - 1;
  const int8_t* bp = B + (int64_t)nrow * K + 16 * lhalf;
  const int8_t* ap[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int mrow = 32 * i + lrow < M ? 32 * i + lrow : M - 1;
    ap[i] = A + (int64_t)mrow * K + 16 * lhalf;
  }
  const int nk = K / kBK;
  const int t0 = 0, t1 = nk;

  auto load = [&](int kt, v4i (&fb)[4], v4i (&fa)[4][TM]) {
    const int64_t off = (int64_t)kt * kBK;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      fb[st] = *(const v4i*)(bp + off + 32 * st);
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[st][i] = *(const v4i*)(ap[i] + off + 32 * st);
    }
  };
  v16i acc[TM][1];
#pragma unroll
  for (int i = 0; i < TM; ++i) acc[i][0] = v16i{};
  auto mma = [&](const v4i (&fb)[4], const v4i (&fa)[4][TM]) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < TM; ++i)
        acc[i][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[st], fa[st][i], acc[i][0], 0, 0, 0);
  };

  v4i fb0[4], fa0[4][TM], fb1[4], fa1[4][TM];
  constexpr int W = kSkinnyWaves;
  if (t0 + wave < t1) load(t0 + wave, fb0, fa0);
  for (int kt = t0 + wave; kt < t1; kt += 2 * W) {
    const bool more = kt + W < t1;
    if (more) load(kt + W, fb1, fa1);
    mma(fb0, fa0);
    if (!more) break;
    if (kt + 2 * W < t1) load(kt + 2 * W, fb0, fa0);
    mma(fb1, fa1);
  }

  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) red[wave - 1][i][q][lane] = acc[i][0][q];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll 1   // one wave's partials at a time (all at once would not fit the registers)
  for (int w = 0; w < W - 1; ++w)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][0][q] += red[w][i][q][lane];
  epilogue<OUT, STATIC_A, LORA, TM, 1>(acc, 0, n0, M, N, a_scale, w_scale, Y, ldy, le);
}

// The KS slices of a split-K decode GEMM (INT32 sums, 1024 words per 32 x 32
// tile in register order: word q * 64 + lane; two row tiles per 32-column
// tile), added up, then the epilogue. INT32 addition is exact (and wraps the
// same in any order), so the result is that of the unsplit kernel bit for
// bit. One wave per (32-column tile, row tile): block (x, y) takes column
// tile x and row tile y. The slices are read in groups of four whose 64
// loads are all issued before the first add (a group past the last slice
// re-reads that slice and adds nothing), so the wave waits for memory once
// per group rather than once per slice.
template <int OUT, bool STATIC_A>
__global__ void __launch_bounds__(64)
k_gemm_skinny_finish(const int32_t* __restrict__ part, int KS, const float* __restrict__ a_scale,
                     const float* __restrict__ w_scale, int M, int N, void* __restrict__ Y,
                     int64_t ldy) {
  const int lane = threadIdx.x;
  const int64_t tile_words = (int64_t)gridDim.x * 2048;     // one slice of every column tile
  const int32_t* src = part + (int64_t)blockIdx.x * 2048 + blockIdx.y * 1024 + lane;
  v16i acc[1][1];
  acc[0][0] = v16i{};
  for (int sl = 0; sl < KS; sl += 4) {
    int32_t v[4][16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t o = (int64_t)(sl + u < KS ? sl + u : KS - 1) * tile_words;
#pragma unroll
      for (int q = 0; q < 16; ++q) v[u][q] = src[o + q * 64];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int keep = sl + u < KS ? -1 : 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[0][0][q] += v[u][q] & keep;
    }
  }
  const LoraEpi none{nullptr, 0, nullptr, 0, 0.0f, 0, {}, {}};
  epilogue<OUT, STATIC_A, 0, 1, 1>(acc, 32 * blockIdx.y, blockIdx.x * kSkinnyBN, M, N, a_scale,
                                   w_scale, Y, ldy, none);
}

// ---------------------------------------------------------------------------
// Decode kernel (M <= 64, K % 128 == 0, no LoRA). A decode GEMM streams its
// weights once; its MFMA work per byte is small, so its speed is the weight
// stream's: bytes in flight per CU over the memory latency. A block owns BN
// output columns over all (up to 64) rows and a range of K-tiles, and keeps
// NST - 1 K-tiles of both operands in flight in an LDS ring (direct buffer
// loads), where the two-stage GEMM tiles keep one K-tile. One barrier per
// K-tile guards the ring slot that the next loads overwrite.
// SPLITK: block (x, y) takes K-tiles [y kps, (y + 1) kps) and writes its
// INT32 sums to `part` in the layout k_gemm_skinny_finish adds up (32-column
// tile ct = (BN / 32) x + wave % (BN / 32), row tile wave / (BN / 32)).
// ---------------------------------------------------------------------------
// s_waitcnt vmcnt(LPW j) lgkmcnt(0) for a wave-uniform j in [0, 6].
template <int LPW>
__device__ __forceinline__ void dec_wait(int j) {
  switch (j) {
    case 0: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(LPW)); break;
    case 2: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(2 * LPW)); break;
    case 3: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(3 * LPW)); break;
    case 4: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(4 * LPW)); break;
    case 5: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(5 * LPW)); break;
    default: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(6 * LPW)); break;
  }
}

// BN output columns per block, NST LDS ring slots; 2 x BN / 32 waves, each
// owning one 32 x 32 output tile (row tile wave / (BN / 32)).
template <int OUT, bool STATIC_A, bool SPLITK, int BN, int NST>
__global__ void __launch_bounds__(2 * BN / 32 * 64)
k_gemm_decode(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
              const float* __restrict__ a_scale, const float* __restrict__ w_scale, int M, int N,
              int K, void* __restrict__ Y, int64_t ldy, int kps, int32_t* __restrict__ part) {
  constexpr int CTB = BN / 32;                   // 32-column tiles per block
  constexpr int NW = 2 * CTB;                    // waves
  constexpr int SLOT = (64 + BN) * kBK;          // one K-tile of both operands
  constexpr int LA = 8 / NW, LB = BN / 8 / NW;   // 1 KB loads per wave per K-tile
  constexpr int LPW = LA + LB;
  static_assert(8 % NW == 0 || NW > 8, "activation rows must split over the waves");
  static_assert(NST >= 2 && NST <= 8, "dec_wait covers up to 6 K-tiles issued ahead");
  __shared__ __attribute__((aligned(1024))) char smem[NST * SLOT];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * BN;
  const int nk = K / kBK;
  const int t0 = SPLITK ? (int)blockIdx.y * kps : 0;
  const int t1 = SPLITK ? (t0 + kps < nk ? t0 + kps : nk) : nk;
  const int cnt = t1 - t0;                       // >= 1: the host makes every slice non-empty

  // Load instruction q of wave w moves 8 tile rows (activations: rows
  // 8 (w + NW q); weights: rows 8 (w + NW q) of the block's columns); lane l
  // fetches the chunk that belongs at position l & 7 of row l / 8, XOR-
  // swizzled as in k_gemm_pipe. Rows past M or N read the last valid row;
  // their sums are never stored.
  const int lr = lane >> 3, lp = lane & 7;
  uint32_t offA[LA > 0 ? LA : 1], offB[LB];
#pragma unroll
  for (int q = 0; q < LA; ++q) {
    const int r = 8 * (wave + NW * q) + lr;
    const int g = r < M ? r : M - 1;
    offA[q] = (uint32_t)g * (uint32_t)K + (uint32_t)swz(r, lp);
  }
#pragma unroll
  for (int q = 0; q < LB; ++q) {
    const int r = 8 * (wave + NW * q) + lr;
    const int g = n0 + r < N ? n0 + r : N - 1;
    offB[q] = (uint32_t)g * (uint32_t)K + (uint32_t)swz(r, lp);
  }
  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)((uint32_t)M * (uint32_t)K), kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsB =
      __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, (int)((uint32_t)N * (uint32_t)K), kBufferRsrcWord3);
  auto issue = [&](int i) {                      // K-tile t0 + i into slot i % NST
    char* sl = smem + (i % NST) * SLOT;
    const int koff = (t0 + i) * kBK;
#pragma unroll
    for (int q = 0; q < LA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_ptr_t)(sl + 1024 * (wave + NW * q)), 16,
                                               (int)offA[q], koff, 0, 0);
#pragma unroll
    for (int q = 0; q < LB; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_ptr_t)(sl + 64 * kBK + 1024 * (wave + NW * q)),
                                               16, (int)offB[q], koff, 0, 0);
  };

  const int lrow = lane & 31, lhalf = lane >> 5;
  const int wm = wave / CTB, wn = wave % CTB;
  const int rowA = wm * 32 + lrow, rowB = 64 + wn * 32 + lrow;
  // one accumulator per k-step of the K-tile: the four MFMAs of a K-tile are
  // independent, and the partial sums meet once at the end (exact)
  v16i acc4[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc4[u] = v16i{};

  const int pre = cnt < NST - 1 ? cnt : NST - 1;
  for (int i = 0; i < pre; ++i) issue(i);
  for (int i = 0; i < cnt; ++i) {
    // this wave's loads of K-tile i have landed (the later ones may not) and
    // its fragment reads of K-tile i - 1 are done; then every wave's are
    const int last = i + NST - 1 < cnt ? i + NST - 1 : cnt;
    dec_wait<LPW>(last - 1 - i);
    __builtin_amdgcn_s_barrier();
    if (i + NST - 1 < cnt) issue(i + NST - 1);   // into the slot of K-tile i - 1
    const char* sl = smem + (i % NST) * SLOT;
    v4i fa[4], fb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = ks * 2 + lhalf;
      fa[ks] = *(const v4i*)(sl + rowA * kBK + swz(rowA, c));
      fb[ks] = *(const v4i*)(sl + rowB * kBK + swz(rowB, c));
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc4[ks] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[ks], fa[ks], acc4[ks], 0, 0, 0);
  }
  v16i acc[1][1];
  acc[0][0] = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);

  if constexpr (SPLITK) {
    const int ct = blockIdx.x * CTB + wn;         // 32-column tile
    const int CT = (N + 31) / 32;
    if (ct < CT) {
      int32_t* dst = part + ((int64_t)blockIdx.y * CT + ct) * 2048 + wm * 1024;
#pragma unroll
      for (int q = 0; q < 16; ++q) dst[q * 64 + lane] = acc[0][0][q];
    }
  } else {
    const LoraEpi none{nullptr, 0, nullptr, 0, 0.0f, 0, {}, {}};
    epilogue<OUT, STATIC_A, 0, 1, 1>(acc, wm * 32, n0 + wn * 32, M, N, a_scale, w_scale, Y, ldy,
                                     none);
  }
}
// 64 columns and 4 slots (64 KB of LDS, two blocks per CU) measured fastest
// on the OPT-13B decode shapes among 64 / 128 columns and 4 / 6 / 8 slots,
// weights rotated past the MALL: 64x15360x5120 20.5 us, 64x5120x5120 16.9,
// 64x20480x5120 36.4, 64x5120x20480 56.7 (30.4 split over 3 K slices),
// against 38.6 / 22.0 / 39.8 / 67.5 (61.5) for the 128x128 tiles or the
// skinny kernel used before. One accumulator per k-step instead of one per
// wave gained 1-3%.
constexpr int kDecBN = 64;
constexpr int kDecStages = 4;

// ---------------------------------------------------------------------------
// Generic kernel: any K % 16 == 0; 128 x 128 tiles staged through registers.
// ---------------------------------------------------------------------------
constexpr int kGBM = 128, kGBN = 128;
constexpr int kGemmThreads = 256;   // 4 waves, 2 x 2, 64 x 64 each

template <int OUT, bool STATIC_A, int LORA>
__global__ void __launch_bounds__(kGemmThreads)
k_gemm_generic(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
               const float* __restrict__ a_scale, const float* __restrict__ w_scale, int M, int N,
               int K, void* __restrict__ Y, int64_t ldy, LoraEpi le) {
  __shared__ __attribute__((aligned(16))) char sA[2][kGBM * kBK];
  __shared__ __attribute__((aligned(16))) char sB[2][kGBN * kBK];

  const int tiles_m = (M + kGBM - 1) / kGBM;
  const int tiles = tiles_m * ((N + kGBN - 1) / kGBN);
  int tm, tn;
  if (!xcd_tile(tiles_m, tiles, tm, tn)) return;
  const int m0 = tm * kGBM, n0 = tn * kGBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

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
      const int off = r * kBK + swz(r, c);
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

  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
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
        fa[i] = *(const v4i*)(&sA[buf][r * kBK + swz(r, c)]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + j * 32 + lrow;
        fb[j] = *(const v4i*)(&sB[buf][r * kBK + swz(r, c)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  epilogue<OUT, STATIC_A, LORA, 2, 2>(acc, m0 + wm * 64, n0 + wn * 64, M, N, a_scale, w_scale, Y,
                                      ldy, le);
}

// ---------------------------------------------------------------------------
// Host side: pick a kernel and tile for the shape.
// ---------------------------------------------------------------------------
// Tile configurations (measured on MI355X over the workload shapes):
//   CFG_256:     256x256 tiles, 8 waves of 128x64 - the fastest at full
//                occupancy (it reads the least L2 data per op);
//   CFG_256x192: 256x192 tiles, 8 waves of 64x96 - fills the chip where
//                256x256 tiles would leave CUs idle (M = 2048, N = 6144:
//                256 tiles instead of 192);
//   CFG_128:     128x128 tiles, 4 waves of 64x64, two blocks per CU - wins
//                for narrow outputs (N = 4096) and small M;
//   CFG_SKINNY:  M <= 64 and N < 12288 (decode): 32-column blocks over all
//                rows, K split over the block's waves.
//   CFG_DECODE:  M <= 64 without LoRA: 64-column blocks with a deep LDS ring,
//                K split across blocks when a workspace is given.
enum TileCfg { CFG_GENERIC = 0, CFG_256 = 1, CFG_128 = 2, CFG_256x192 = 3, CFG_SKINNY = 4, CFG_DECODE = 5 };

// Score of a tile configuration: the share of the launched tile work that is
// useful (rows and columns padded up to whole tiles, and the last round of
// tiles over the chip's resident blocks) times the configuration's measured
// relative throughput at full occupancy.
static double tile_score(int64_t M, int64_t N, int64_t bm, int64_t bn, int64_t resident, double rate) {
  const int64_t tm = (M + bm - 1) / bm, tn = (N + bn - 1) / bn, tiles = tm * tn;
  const int64_t rounds = (tiles + resident - 1) / resident;
  const double pad = (double)M / (double)(tm * bm) * (double)N / (double)(tn * bn);
  return rate * pad * (double)tiles / (double)(rounds * resident);
}

// Tuning override: SQ_GEMM_TILE=0..5 forces a configuration (read once per
// process; 4, the skinny kernel, and 5, the decode kernel, only where M <= 64).
static int forced_cfg() {
  static const int forced = [] {
    const char* e = std::getenv("SQ_GEMM_TILE");
    const int o = (e && *e) ? std::atoi(e) : -1;
    return (o >= 0 && o <= 5) ? o : -1;
  }();
  return forced;
}

// Tile configuration of the LoRA-capable kernels (the decode kernel, chosen
// before this for M <= 64 without LoRA, is not one of them).
static int pick_cfg(int64_t M, int64_t N, int64_t K) {
  if (K % kBK != 0 || M * K >= (1LL << 32) || N * K >= (1LL << 32)) return CFG_GENERIC;
  const int forced = forced_cfg();
  if (forced >= 0 && forced != CFG_DECODE && (forced != CFG_SKINNY || M <= 64)) return forced;
  // M <= 64 with fewer than 96 column tiles of 128: the skinny kernel (measured
  // 1.7-3.6x faster at N = 5120); with more, 128x128 tiles already spread the
  // weight stream over the chip and win (by 8-34% at N = 15360 ... 28672).
  if (M <= 64 && (N + 127) / 128 < 96) return CFG_SKINNY;
  // 256 CUs: one 256x256 or 256x192 block per CU, two 128x128 blocks per CU.
  // Rates relative to 256x256 at full occupancy, measured on MI355X: 256x192
  // 0.94 (2048x24576x4096, whole rounds for both), taken as 0.93 so that
  // near-ties go to 256x256, which fetches less from the memory fabric per op
  // (the chip runs these GEMMs at its power limit; on the Llama-3-8B step,
  // gate+up on 256x256 beat 256x192 by 3% with equal times alone); 128x128 0.8.
  const double s256 = tile_score(M, N, 256, 256, 256, 1.0);
  const double s192 = tile_score(M, N, 256, 192, 256, 0.93);
  const double s128 = tile_score(M, N, 128, 128, 512, 0.8);
  if (s256 >= s192 && s256 >= s128) return CFG_256;
  return s192 >= s128 ? CFG_256x192 : CFG_128;
}

template <int BM, int BN, int WM, int WN, int OUT, bool STATIC_A, int LORA>
static int launch_pipe(const int8_t* Xq, const int8_t* Wq, const float* a_scale, const float* w_scale,
                       int64_t M, int64_t N, int64_t K, void* Y, int64_t ldy, const LoraEpi& le,
                       hipStream_t st) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t blocks = (tiles + 7) / 8 * 8;
  k_gemm_pipe<BM, BN, WM, WN, OUT, STATIC_A, LORA><<<(unsigned)blocks, WM * WN * 64, 0, st>>>(
      Xq, Wq, a_scale, w_scale, (int)M, (int)N, (int)K, Y, ldy, le);
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

// The decode kernel for M <= 64 (no LoRA epilogue): K a multiple of 128 and
// operands below 4 GiB, unless SQ_GEMM_TILE forces another configuration.
static bool decode_ok(int64_t M, int64_t N, int64_t K) {
  if (M > 64 || K % kBK != 0 || M * K >= (1LL << 32) || N * K >= (1LL << 32)) return false;
  const int f = forced_cfg();
  return f < 0 || f == CFG_DECODE;
}

// K split of the decode kernel across blocks, given a workspace, where the
// column blocks alone leave most CUs idle: slices of whole K-tiles so that
// at most 256 blocks stream (one per CU), each slice at least 8 K-tiles, so
// that the INT32 partial sums (KS x 64 x N x 4 bytes) stay at most a quarter
// of the weight bytes. 1: no split.
static int decode_splits(int64_t M, int64_t N, int64_t K) {
  if (!decode_ok(M, N, K)) return 1;
  const int64_t ct = (N + kDecBN - 1) / kDecBN;
  // A CU streams about as fast with one decode block as with two, so the
  // split stops at one block per CU (64x5120x20480: 56.7 us unsplit, 30.4 us
  // in 3 slices = 240 blocks, 38.6 us in 4 = 320 blocks; 64x5120x5120: 17.1,
  // 14.3 and 16.5 us); with 128 or more column blocks it does not pay
  // (64x15360x5120: 20.4 us unsplit, 26.3 us in 2 slices).
  if (ct >= 128) return 1;
  const int64_t kmax = (K / kBK) / 8;
  int64_t ks = 256 / ct;
  if (ks > kmax) ks = kmax;
  return ks > 1 ? (int)ks : 1;
}

size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const int ks = decode_splits(M, N, K);
  if (ks <= 1) return 0;
  const int64_t ct = (N + 31) / 32;            // 32-column tiles, two row tiles each
  return (size_t)ks * (size_t)ct * 2048 * sizeof(int32_t);
}

template <int OUT, bool STATIC_A>
static int launch_decode(const int8_t* Xq, const int8_t* Wq, const float* a_scale,
                         const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y, int64_t ldy,
                         int32_t* part, hipStream_t st) {
  const unsigned bn = (unsigned)((N + kDecBN - 1) / kDecBN);
  const int ks = part != nullptr ? decode_splits(M, N, K) : 1;
  if (ks <= 1) {
    if (bn > 256) {
      // More 64-column blocks than CUs: blocks of 128 columns (8 waves, 96 KB
      // of LDS) read the activation rows half as often per weight byte
      // (64x20480x5120: 36.3 -> 32.8 us; splitting K does not help there).
      constexpr int BN2 = 2 * kDecBN;
      k_gemm_decode<OUT, STATIC_A, false, BN2, kDecStages><<<(unsigned)((N + BN2 - 1) / BN2), BN2 / 16 * 64,
                                                             0, st>>>(
          Xq, Wq, a_scale, w_scale, (int)M, (int)N, (int)K, Y, ldy, 0, nullptr);
    } else {
      k_gemm_decode<OUT, STATIC_A, false, kDecBN, kDecStages><<<bn, kDecBN / 16 * 64, 0, st>>>(
          Xq, Wq, a_scale, w_scale, (int)M, (int)N, (int)K, Y, ldy, 0, nullptr);
    }
    SQ_LAUNCH_CHECK();
    return SQ_OK;
  }
  const int nk = (int)(K / kBK);
  const int kps = (nk + ks - 1) / ks;
  const int slices = (nk + kps - 1) / kps;   // every slice non-empty
  k_gemm_decode<OUT, STATIC_A, true, kDecBN, kDecStages><<<dim3(bn, (unsigned)slices), kDecBN / 16 * 64, 0,
                                                           st>>>(
      Xq, Wq, a_scale, w_scale, (int)M, (int)N, (int)K, Y, ldy, kps, part);
  SQ_LAUNCH_CHECK();
  const unsigned ct = (unsigned)((N + 31) / 32);
  k_gemm_skinny_finish<OUT, STATIC_A><<<dim3(ct, M > 32 ? 2u : 1u), 64, 0, st>>>(
      part, slices, a_scale, w_scale, (int)M, (int)N, Y, ldy);
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

template <int OUT, bool STATIC_A, int LORA>
static int launch_gemm_t(const int8_t* Xq, const int8_t* Wq, const float* a_scale,
                         const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y,
                         int64_t ldy, const LoraEpi& le, hipStream_t st, int32_t* part = nullptr) {
  if constexpr (LORA == 0) {
    if (decode_ok(M, N, K))
      return launch_decode<OUT, STATIC_A>(Xq, Wq, a_scale, w_scale, M, N, K, Y, ldy, part, st);
  }
  switch (pick_cfg(M, N, K)) {
    case CFG_256:
      return launch_pipe<256, 256, 2, 4, OUT, STATIC_A, LORA>(Xq, Wq, a_scale, w_scale, M, N, K, Y,
                                                                 ldy, le, st);
    case CFG_256x192:
      return launch_pipe<256, 192, 4, 2, OUT, STATIC_A, LORA>(Xq, Wq, a_scale, w_scale, M, N, K, Y,
                                                                  ldy, le, st);
    case CFG_128:
      return launch_pipe<128, 128, 2, 2, OUT, STATIC_A, LORA>(Xq, Wq, a_scale, w_scale, M, N, K, Y,
                                                                 ldy, le, st);
    case CFG_SKINNY: {
      const unsigned blocks = (unsigned)((N + kSkinnyBN - 1) / kSkinnyBN);
      if (M <= 32)
        k_gemm_skinny<OUT, STATIC_A, LORA, 1><<<blocks, kSkinnyWaves * 64, 0, st>>>(
            Xq, Wq, a_scale, w_scale, (int)M, (int)N, (int)K, Y, ldy, le);
      else
        k_gemm_skinny<OUT, STATIC_A, LORA, 2><<<blocks, kSkinnyWaves * 64, 0, st>>>(
            Xq, Wq, a_scale, w_scale, (int)M, (int)N, (int)K, Y, ldy, le);
      SQ_LAUNCH_CHECK();
      return SQ_OK;
    }
    default:
      break;
  }
  const int64_t tiles = ((M + kGBM - 1) / kGBM) * ((N + kGBN - 1) / kGBN);
  const int64_t blocks = (tiles + 7) / 8 * 8;
  k_gemm_generic<OUT, STATIC_A, LORA><<<(unsigned)blocks, kGemmThreads, 0, st>>>(
      Xq, Wq, a_scale, w_scale, (int)M, (int)N, (int)K, Y, ldy, le);
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

template <int LORA>
static int launch_gemm_any(const int8_t* Xq, const int8_t* Wq, const float* a_scale, int mode,
                           const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y, int yt,
                           int64_t ldy, const LoraEpi& le, hipStream_t st,
                           int32_t* part = nullptr) {
  if (M == 0) return SQ_OK;
  const bool stat = mode == SQ_ACT_PER_TENSOR_STATIC;
#define SQ_GEMM_OUT(O)                                                                               \
  return stat ? launch_gemm_t<O, true, LORA>(Xq, Wq, a_scale, w_scale, M, N, K, Y, ldy, le, st, part)      \
              : launch_gemm_t<O, false, LORA>(Xq, Wq, a_scale, w_scale, M, N, K, Y, ldy, le, st, part);
  switch (yt) {
    case SQ_BF16: SQ_GEMM_OUT(OUT_BF16)
    case SQ_F16:  SQ_GEMM_OUT(OUT_F16)
    default:      SQ_GEMM_OUT(OUT_F32)
  }
#undef SQ_GEMM_OUT
}

int launch_gemm(const int8_t* Xq, const int8_t* Wq, const float* a_scale, int mode,
                const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y, int yt,
                int64_t ldy, hipStream_t st) {
  const LoraEpi none{nullptr, 0, nullptr, 0, 0.0f, 0, {}, {}};
  return launch_gemm_any<0>(Xq, Wq, a_scale, mode, w_scale, M, N, K, Y, yt, ldy, none, st);
}

int launch_gemm_ws(const int8_t* Xq, const int8_t* Wq, const float* a_scale, int mode,
                   const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y, int yt,
                   int64_t ldy, void* ws, hipStream_t st) {
  const LoraEpi none{nullptr, 0, nullptr, 0, 0.0f, 0, {}, {}};
  return launch_gemm_any<0>(Xq, Wq, a_scale, mode, w_scale, M, N, K, Y, yt, ldy, none, st,
                            (int32_t*)ws);
}

int launch_gemm_lora(const int8_t* Xq, const int8_t* Wq, const float* a_scale, int mode,
                     const float* w_scale, int64_t M, int64_t N, int64_t K, const void* T,
                     int64_t ldt, const void* B, int r, float scale, void* Y, int yt, int64_t ldy,
                     hipStream_t st, int parts, const int64_t* n_end, const int* r_end) {
  LoraEpi le{(const unsigned short*)T, ldt, (const unsigned short*)B, r, scale, 0, {}, {}};
  if (parts > 1) {
    le.parts = parts;
    for (int p = 0; p < parts; ++p) {
      le.n_end[p] = (int)n_end[p];
      le.r_end[p] = r_end[p];
    }
  }
  if (scale == 1.0f)
    return launch_gemm_any<1>(Xq, Wq, a_scale, mode, w_scale, M, N, K, Y, yt, ldy, le, st);
  return launch_gemm_any<2>(Xq, Wq, a_scale, mode, w_scale, M, N, K, Y, yt, ldy, le, st);
}

int launch_gemm_i32(const int8_t* Xq, const int8_t* Wq, int64_t M, int64_t N, int64_t K,
                    int32_t* acc, hipStream_t st) {
  if (M == 0) return SQ_OK;
  const LoraEpi none{nullptr, 0, nullptr, 0, 0.0f, 0, {}, {}};
  return launch_gemm_t<OUT_I32, false, 0>(Xq, Wq, nullptr, nullptr, M, N, K, acc, N, none, st);
}

}  // namespace sq
