// Row-wise symmetric INT8 quantization ([SQ] Steps 5-6 and the sketch's
// quantize_int8), in three flavours sharing one kernel:
//   FOLD    (weights, per output channel): v = fp32(W[n,k] * s[k]);
//           scale = max_k |v| / 127; code = clamp(rne(fp32(v / scale)), +-127)
//   DYNAMIC (activations, per token):      v = fp32(X[m,k] / s[k]); same scale
//   STATIC  (activations, per tensor):     v = fp32(X[m,k] / s[k]); scale given
//
// The kernel is HBM-bound: it reads each input element once (16-byte loads)
// and writes one byte per element. A block owns RPB rows at a time and walks
// rows with a grid stride; each thread covers CPT chunks of 8 consecutive
// channels. The first pass turns the raw row into the smoothed fp32 values v
// (kept in registers) and their max; the raw registers are then free, so the
// block's next rows are loaded into them while this row group is reduced
// (wave max, then LDS across waves: one barrier per group) and quantized from
// v (at 8 chunks per thread v is recomputed instead, for registers, and the
// next rows load after the group). The per-channel factors (fp32 s for FOLD,
// the fp64 reciprocals 1/s that make the divisions exact for the others, see
// div_rn and rcp_rn64) are computed once per block, after its first loads are
// issued, and reused for all its rows.
//
// Two more shapes of the same arithmetic: k_quant_wave (one to four waves per
// row, K <= 16384 for 16-bit inputs) and k_quant_long (one block per row and
// the next row in flight, 16384 < K <= 32768 for 16-bit inputs); the kernel
// above serves fp32 inputs beyond K = 4096.
#include <cstdlib>

#include "sq_internal.h"

namespace sq {

// Q_STATIC_CLIP: Q_STATIC that also counts the codes it clamps (a kind of its
// own, so the plain static kernels carry none of the counting registers).
enum QuantKind { Q_FOLD = 0, Q_DYNAMIC = 1, Q_STATIC = 2, Q_STATIC_CLIP = 3 };
template <int KIND>
constexpr bool kStaticKind = KIND == Q_STATIC || KIND == Q_STATIC_CLIP;

constexpr int kQuantMaxThreads = 512;

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


// rows: M (activations) or N (weights). in_ld_bytes: input row stride.
// s: [K] or null (no smoothing). scale_io: [rows] written (FOLD, DYNAMIC) or
// [1] read (STATIC). out: [rows, K] int8 contiguous.
template <int DT, int CPT, int KIND, int RPB>
__global__ void __launch_bounds__(kQuantMaxThreads)
k_quant_rows(const char* __restrict__ in, int64_t rows, int64_t K, int64_t in_ld_bytes,
             const float* __restrict__ s, float* __restrict__ scale_io, int8_t* __restrict__ out,
             unsigned long long* __restrict__ clip) {
  const int tid = threadIdx.x;
  const int T = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = T >> 6;
  const int64_t stride = (int64_t)gridDim.x * RPB;

  // At 8 chunks per thread the registers do not hold v next to the factors:
  // v is recomputed from the raw row in the second pass, so the next rows are
  // loaded only after it.
  constexpr bool kStoreV = CPT <= 4;
  RowChunks<DT, CPT> raw[RPB];
  auto load_group = [&](int64_t m0) {
#pragma unroll
    for (int r = 0; r < RPB; ++r)
      if (m0 + r < rows) load_row<DT, CPT>(raw[r], in + (m0 + r) * in_ld_bytes, K, tid, T);
  };
  int64_t m0 = (int64_t)blockIdx.x * RPB;
  if (m0 < rows) load_group(m0);

  // Per-channel factor: fp32 s (FOLD multiplies) or fp64 1/s (divisions).
  float sm[CPT][8];
  double rs[CPT][8];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int64_t c = tid + (int64_t)j * T;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sv = (s != nullptr && c * 8 < K) ? s[c * 8 + e] : 1.0f;
      if constexpr (KIND == Q_FOLD) sm[j][e] = sv;
      else rs[j][e] = 1.0 / (double)sv;       // RN64(1/s), IEEE fp64 division (once per block)
    }
  }

  constexpr bool counting = KIND == Q_STATIC_CLIP;   // clipped-code count into *clip
  int nclip = 0;
  float a_static = 0.0f;
  double r_static = 0.0;
  if constexpr (kStaticKind<KIND>) {
    a_static = scale_io[0];
    r_static = a_static != 0.0f ? rcp_rn64(a_static) : 0.0;
  }

  __shared__ float red[2][RPB][kQuantMaxThreads / 64];
  int parity = 0;
  for (; m0 < rows; m0 += stride) {
    if (!kStoreV && m0 != (int64_t)blockIdx.x * RPB) load_group(m0);
    auto smooth = [&](const float x, int j, int e) -> float {
      if constexpr (KIND == Q_FOLD) return x * sm[j][e];   // fp32 multiply
      else return div_rn(x, rs[j][e]);                     // fp32(x / s), exact
    };
    // pass 1: smoothed values and their row max
    float v[RPB][kStoreV ? CPT : 1][8];
    float amax[RPB];
#pragma unroll
    for (int r = 0; r < RPB; ++r) {
      amax[r] = 0.0f;
      if (m0 + r < rows) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          const int64_t c = tid + (int64_t)j * T;
          if (c * 8 < K) {
            float x[8];
            widen8<DT>(raw[r].w[j], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float y = smooth(x[e], j, e);
              if constexpr (kStoreV) v[r][j][e] = y;
              amax[r] = __builtin_fmaxf(amax[r], __builtin_fabsf(y));
            }
          }
        }
      }
    }
    // the raw registers are free: load the block's next rows into them
    if (kStoreV && m0 + stride < rows) load_group(m0 + stride);

    float scale[RPB];
    double rscale[RPB];
    if constexpr (kStaticKind<KIND>) {
#pragma unroll
      for (int r = 0; r < RPB; ++r) { scale[r] = a_static; rscale[r] = r_static; }
    } else {
#pragma unroll
      for (int r = 0; r < RPB; ++r) {
        amax[r] = wave_max(amax[r]);
        if (lane == 0) red[parity][r][wave] = amax[r];
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < RPB; ++r) {
        float a = red[parity][r][0];
        for (int w = 1; w < nwaves; ++w) a = __builtin_fmaxf(a, red[parity][r][w]);
        scale[r] = a / 127.0f;                                   // IEEE fp32 division
        rscale[r] = scale[r] != 0.0f ? rcp_rn64(scale[r]) : 0.0;
        if (tid == 0 && m0 + r < rows) scale_io[m0 + r] = scale[r];
      }
      parity ^= 1;
    }
    // Clip counting: rne(fp32(y / scale)) passes 127 exactly when the quotient
    // reaches 127.5, and the quotient grows with |y|, so a thread whose largest
    // |y| stays below that clips nothing and skips the count (nearly all do).
    bool maybe[RPB];
#pragma unroll
    for (int r = 0; r < RPB; ++r) maybe[r] = counting && div_rn(amax[r], rscale[r]) >= 127.5f;

    // pass 2: codes from v
#pragma unroll
    for (int r = 0; r < RPB; ++r) {
      if (m0 + r >= rows) break;
      int8_t* orow = out + (m0 + r) * K;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int64_t c = tid + (int64_t)j * T;
        if (c * 8 < K) {
          float y[8];
          if constexpr (kStoreV) {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = v[r][j][e];
          } else {
            widen8<DT>(raw[r].w[j], y);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = smooth(y[e], j, e);
          }
          // scale == 0 (all-zero row, or a zero static scale): every code is 0
          // (selected per element: a row mask here costs this kernel a spill)
          uint32_t q[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) q[e] = scale[r] != 0.0f ? code_word(div_rn(y[e], rscale[r])) : 0u;
          uint2 pk;
          pk.x = pack4_codes(q[0], q[1], q[2], q[3]);
          pk.y = pack4_codes(q[4], q[5], q[6], q[7]);
          *(uint2*)(orow + c * 8) = pk;
        }
      }
      // the rare count: a loop of its own, so the code loop above keeps its registers
      // (with kStoreV the raw registers already hold the next rows: v is used)
      if (maybe[r]) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          const int64_t c = tid + (int64_t)j * T;
          if (c * 8 < K) {
            float y[8];
            if constexpr (kStoreV) {
#pragma unroll
              for (int e = 0; e < 8; ++e) y[e] = v[r][j][e];
            } else {
              widen8<DT>(raw[r].w[j], y);
#pragma unroll
              for (int e = 0; e < 8; ++e) y[e] = smooth(y[e], j, e);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) nclip += clips(div_rn(y[e], rscale[r]));
          }
        }
      }
    }
  }
  if constexpr (counting) {
    // every lane reaches this point; one atomic per wave
    const int n = wave_sum(nclip);
    if ((threadIdx.x & 63) == 0 && n != 0) atomicAdd(clip, (unsigned long long)n);
  }
}

// ---------------------------------------------------------------------------
// Wave-per-row quantizer: WPR = 1, 2 or 4 waves per row (K <= 4096, 8192,
// 16384 for 16-bit inputs; fp32 inputs up to 4096), each lane covering at
// most CPL = 8 chunks of 8 channels, so that the raw row share, its smoothed
// values v and the next row's loads all fit in registers. With one wave per
// row the row max is a wave reduction and the kernel has no barrier after its
// start; with 2 or 4 the row's waves meet in LDS, one block barrier per row.
// The per-channel factors live in LDS, computed once per block: fp32 s for
// FOLD, fp64 1/s otherwise, laid out so that the 16-byte reads of consecutive
// lanes are consecutive (no bank conflict). Lane l of the row's wave h covers
// chunks c = 64 CPL h + l + 64 j (j < CPL); pass 1 forms v and the row max,
// the raw registers then take the wave's next row while this one is reduced
// and quantized from v.
// ---------------------------------------------------------------------------
constexpr int kWaveRowThreads = 512;

template <int DT, int KIND, int CPL, int WPR>
struct WaveRowCfg {
  static constexpr int kWords = DT == SQ_F32 ? 2 : 1;          // 16-byte words per chunk
  static constexpr int kTabParts = KIND == Q_FOLD ? 2 : 4;     // 16-byte factor words per chunk
  static constexpr int kGroup = 4;                             // chunks per factor-read group
  static_assert(CPL <= 8, "raw row, v and the next row must fit the registers");
  static_assert(WPR == 1 || WPR == 2 || WPR == 4, "1, 2 or 4 waves per row");
};

template <int DT, int KIND, int CPL, int WPR>
__global__ void __launch_bounds__(kWaveRowThreads)
k_quant_wave(const char* __restrict__ in, int64_t rows, int K, int64_t in_ld_bytes,
             const float* __restrict__ s, float* __restrict__ scale_io, int8_t* __restrict__ out,
             unsigned long long* __restrict__ clip) {
  using Cfg = WaveRowCfg<DT, KIND, CPL, WPR>;
  constexpr int kWords = Cfg::kWords;
  constexpr int kGroup = Cfg::kGroup;
  constexpr int kSpan = 64 * CPL;                  // chunks per wave
  // factor word p of chunk c at tab[p * kSpan * WPR + c]
  __shared__ uint4 tab[Cfg::kTabParts * kSpan * WPR];
  __shared__ float red[2][kWaveRowThreads / 64];
  const int nch = K / 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = wave % WPR;
  const int slot = wave / WPR;                     // row slot within the block
  const int slots = (blockDim.x >> 6) / WPR;
  const int64_t row_step = (int64_t)gridDim.x * slots;
  const int64_t iters = (rows + row_step - 1) / row_step;   // the same for every wave
  int64_t m = (int64_t)blockIdx.x * slots + slot;
  const int c0 = kSpan * half + lane;              // this lane's first chunk

  // Chunks past the row end (c >= nch) load chunk nch - 1 and read its factors;
  // their values are zeroed before the max and they are never stored. No
  // branch in the arithmetic, so loads and LDS reads can be issued early.
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
    float sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] = s != nullptr ? s[c * 8 + e] : 1.0f;
    if constexpr (KIND == Q_FOLD) {
      tab[c] = make_uint4(__float_as_uint(sv[0]), __float_as_uint(sv[1]), __float_as_uint(sv[2]),
                          __float_as_uint(sv[3]));
      tab[kSpan * WPR + c] = make_uint4(__float_as_uint(sv[4]), __float_as_uint(sv[5]),
                                        __float_as_uint(sv[6]), __float_as_uint(sv[7]));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double r0 = rcp_rn64(sv[2 * q]);            // RN64(1/s)
        const double r1 = rcp_rn64(sv[2 * q + 1]);
        const unsigned long long b0 = __double_as_longlong(r0), b1 = __double_as_longlong(r1);
        tab[q * kSpan * WPR + c] = make_uint4((uint32_t)b0, (uint32_t)(b0 >> 32), (uint32_t)b1,
                                              (uint32_t)(b1 >> 32));
      }
    }
  }
  __syncthreads();

  // v for chunk j of this lane from its raw 8 values. `dep` is a value the
  // factor reads must wait for (see the pass-1 loop); through it the factor
  // index is opaque to the compiler, which would otherwise hoist the reads of
  // all chunks (16 registers each) out of the row loop or to its top, and spill.
  auto smooth8 = [&](int j, float* x, float dep) {
    int c = chunk(j);
    asm volatile("" : "+v"(c) : "v"(dep));
    if constexpr (KIND == Q_FOLD) {
      const uint4 f0 = tab[c], f1 = tab[kSpan * WPR + c];
      const float f[8] = {__uint_as_float(f0.x), __uint_as_float(f0.y), __uint_as_float(f0.z),
                          __uint_as_float(f0.w), __uint_as_float(f1.x), __uint_as_float(f1.y),
                          __uint_as_float(f1.z), __uint_as_float(f1.w)};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = x[e] * f[e];          // fp32 multiply
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 f = tab[q * kSpan * WPR + c];
        const double r0 = __longlong_as_double(((unsigned long long)f.y << 32) | f.x);
        const double r1 = __longlong_as_double(((unsigned long long)f.w << 32) | f.z);
        x[2 * q] = div_rn(x[2 * q], r0);                        // fp32(x / s), exact
        x[2 * q + 1] = div_rn(x[2 * q + 1], r1);
      }
    }
  };

  constexpr bool counting = KIND == Q_STATIC_CLIP;   // clipped-code count into *clip
  int nclip = 0;
  float a_static = 0.0f;
  double r_static = 0.0;
  if constexpr (kStaticKind<KIND>) {
    a_static = scale_io[0];
    r_static = a_static != 0.0f ? rcp_rn64(a_static) : 0.0;
  }

  for (int64_t it = 0; it < iters; ++it, m += row_step) {
    const bool active = m < rows;                 // uniform over the wave pair
    float v[CPL][8];
    float amax = 0.0f;
    if (active) {
      // Chunks in groups of kGroup: a group's factor reads wait for the
      // previous group's results (registers stay bounded).
      float dep = 0.0f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        if (j % kGroup == 0 && j > 0) dep = v[j - 1][7];
        float x[8];
        widen8<DT>(raw[j], x);
        smooth8(j, x, dep);
        // the chunk's max, masked once per chunk (chunks past the row end hold a re-read)
        const bool in_row = c0 + 64 * j < nch;
        float cm = __builtin_fabsf(x[0]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[j][e] = x[e];
          cm = __builtin_fmaxf(cm, __builtin_fabsf(x[e]));
        }
        amax = __builtin_fmaxf(amax, in_row ? cm : 0.0f);
      }
      // The next row's loads reuse the raw registers: they must not be
      // issued before pass 1 is done with them (an opaque zero that depends
      // on the row max keeps the compiler from hoisting them).
      if (m + row_step < rows) {
        int zero;
        asm volatile("v_mov_b32 %0, 0" : "=v"(zero) : "v"(amax));
        load(m + row_step + zero);
      }
    }

    float scale;
    double rscale;
    if constexpr (kStaticKind<KIND>) {
      scale = a_static;
      rscale = r_static;
    } else {
      amax = wave_max(amax);
      if constexpr (WPR > 1) {
        // the row's waves meet in LDS (double-buffered: one barrier per row)
        float* r = red[it & 1];
        if (lane == 0) r[wave] = amax;
        __syncthreads();
        amax = r[WPR * slot];
#pragma unroll
        for (int w = 1; w < WPR; ++w) amax = __builtin_fmaxf(amax, r[WPR * slot + w]);
      }
      scale = amax / 127.0f;                                     // IEEE fp32 division
      rscale = scale != 0.0f ? rcp_rn64(scale) : 0.0;
      if (active && half == 0 && lane == 0) scale_io[m] = scale;
    }
    if (!active) continue;

    int8_t* orow = out + m * K;
    // scale == 0 (all-zero row, or a zero static scale): every code is 0
    const uint32_t keep = scale != 0.0f ? 0xFFFFFFFFu : 0u;
    // Clip counting: rne(fp32(v / scale)) passes 127 exactly when the quotient
    // reaches 127.5, and the quotient grows with |v|, so a lane whose largest
    // in-row |v| stays below that clips nothing and skips the count.
    const bool maybe = counting && div_rn(amax, rscale) >= 127.5f;
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
    // the rare count, in a loop of its own; chunks past the row end hold a
    // clamped re-read of the row and are not counted
    if (maybe) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        if (c0 + 64 * j < nch) {
#pragma unroll
          for (int e = 0; e < 8; ++e) nclip += clips(div_rn(v[j][e], rscale));
        }
      }
    }
  }
  if constexpr (counting) {
    // every lane reaches this point; one atomic per wave
    const int n = wave_sum(nclip);
    if ((threadIdx.x & 63) == 0 && n != 0) atomicAdd(clip, (unsigned long long)n);
  }
}


template <int DT, int KIND, int CPL, int WPR>
static void launch_wave(const char* p, int64_t rows, int64_t K, int64_t ldb, const float* s,
                        float* scale_io, int8_t* out, unsigned long long* clip, hipStream_t st) {
  auto f = k_quant_wave<DT, KIND, CPL, WPR>;
  constexpr int slots = kWaveRowThreads / 64 / WPR;
  int64_t grid = (rows + slots - 1) / slots;
  const int64_t cap =
      resident_blocks<WaveRowCfg<DT, KIND, CPL, WPR>>((const void*)f, kWaveRowThreads);
  if (grid > cap) grid = cap;
  f<<<(unsigned)grid, kWaveRowThreads, 0, st>>>(p, rows, (int)K, ldb, s, scale_io, out, clip);
}

// ---------------------------------------------------------------------------
// Long-row quantizer (16-bit inputs, 16384 < K <= 32768): one 512-thread
// block per row, lane chunks CPT = ceil(K / 4096) (5 at K = 20480, 7 at
// K = 28672), persistent over the rows. Two raw rows live in registers next
// to the per-channel factors: pass 1 turns the current row into v (kept in
// LDS, as per-thread storage) and its row max, and its registers then take
// the row after next, so two rows stay in flight through the block reduction
// and pass 2, which quantizes v from LDS. Chunks past the row end (K not a
// multiple of 4096) re-read the last chunk, are left out of the max and are
// not stored.
// ---------------------------------------------------------------------------
template <int DT, int CPT, int KIND>
__global__ void __launch_bounds__(kQuantMaxThreads)
k_quant_long(const char* __restrict__ in, int64_t rows, int K, int64_t in_ld_bytes,
             const float* __restrict__ s, float* __restrict__ scale_io, int8_t* __restrict__ out,
             unsigned long long* __restrict__ clip) {
  static_assert(DT != SQ_F32, "16-bit inputs: one 16-byte word per chunk");
  constexpr int T = kQuantMaxThreads;
  constexpr int NW = T / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nch = K / 8;
  const int64_t step = gridDim.x;
  auto chunk = [&](int j) { return tid + T * j < nch ? tid + T * j : nch - 1; };
  auto load = [&](uint4 (&r)[CPT], int64_t row) {
    const char* p = in + row * in_ld_bytes;
#pragma unroll
    for (int j = 0; j < CPT; ++j) r[j] = *(const uint4*)(p + (int64_t)chunk(j) * 16);
  };
  // Two raw rows in registers: the one being quantized and the next, in
  // flight. Pass 1 turns the row into v, so its registers are free at once and
  // take the row after next: two rows stay in flight through the row
  // reduction and pass 2.
  uint4 ra[CPT], rb[CPT];
  int64_t m = blockIdx.x;
  if (m < rows) load(ra, m);
  if (m + step < rows) load(rb, m + step);

  // per-channel factors of this thread's chunks, once per block
  float sm[KIND == Q_FOLD ? CPT : 1][8];
  double rs[KIND == Q_FOLD ? 1 : CPT][8];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = chunk(j);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sv = s != nullptr ? s[c * 8 + e] : 1.0f;
      if constexpr (KIND == Q_FOLD) sm[j][e] = sv;
      else rs[j][e] = rcp_rn64(sv);                // RN64(1/s)
    }
  }
  constexpr bool counting = KIND == Q_STATIC_CLIP;
  int nclip = 0;
  float a_static = 0.0f;
  double r_static = 0.0;
  if constexpr (kStaticKind<KIND>) {
    a_static = scale_io[0];
    r_static = a_static != 0.0f ? rcp_rn64(a_static) : 0.0;
  }
  __shared__ float red[2][NW];
  // v of this thread's chunks, kept in LDS between the passes (the registers
  // hold the factors and two raw rows): half h of chunk j at vst[h][j T + tid],
  // so consecutive lanes touch consecutive 16-byte words. Each thread reads
  // back only what it wrote itself, so no barrier guards it.
  __shared__ float4 vst[2][CPT * T];

  auto smooth = [&](const float x, int j, int e) -> float {
    if constexpr (KIND == Q_FOLD) return x * sm[j][e];   // fp32 multiply
    else return div_rn(x, rs[j][e]);                     // fp32(x / s), exact
  };
  // (the index passes through an opaque copy that depends on `dep`, a value
  // known only after pass 1 (and the row reduction): otherwise the compiler
  // hoists every read above it and holds all of v in registers, and spills)
  auto read_v = [&](int j, float* y, uint32_t dep) {
    int i = j * T + tid;
    asm volatile("" : "+v"(i) : "v"(dep));
    const float4 v0 = vst[0][i], v1 = vst[1][i];
    y[0] = v0.x; y[1] = v0.y; y[2] = v0.z; y[3] = v0.w;
    y[4] = v1.x; y[5] = v1.y; y[6] = v1.z; y[7] = v1.w;
  };
  auto process = [&](uint4 (&cur)[CPT], int64_t row, int par) {
    // pass 1: v and the row max
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      float x[8];
      widen8<DT>(&cur[j], x);
      float cm = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = smooth(x[e], j, e);
        cm = __builtin_fmaxf(cm, __builtin_fabsf(x[e]));
      }
      vst[0][j * T + tid] = make_float4(x[0], x[1], x[2], x[3]);
      vst[1][j * T + tid] = make_float4(x[4], x[5], x[6], x[7]);
      amax = __builtin_fmaxf(amax, tid + T * j < nch ? cm : 0.0f);
    }
    if (row + 2 * step < rows) {
      // an opaque zero that depends on the row max: the loads may not move
      // above pass 1, whose registers they reuse
      int zero;
      asm volatile("v_mov_b32 %0, 0" : "=v"(zero) : "v"(amax));
      load(cur, row + 2 * step + zero);
    }
    float scale;
    double rscale;
    if constexpr (kStaticKind<KIND>) {
      scale = a_static;
      rscale = r_static;
    } else {
      amax = wave_max(amax);
      if (lane == 0) red[par][wave] = amax;
      __syncthreads();
      amax = red[par][0];
#pragma unroll
      for (int w = 1; w < NW; ++w) amax = __builtin_fmaxf(amax, red[par][w]);
      scale = amax / 127.0f;                                   // IEEE fp32 division
      rscale = scale != 0.0f ? rcp_rn64(scale) : 0.0;
      if (tid == 0) scale_io[row] = scale;
    }
    // pass 2: codes from v (scale == 0: every code is 0)
    const uint32_t keep = scale != 0.0f ? 0xFFFFFFFFu : 0u;
    int8_t* orow = out + row * K;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      float y[8];
      read_v(j, y, __float_as_uint(amax));
      uint32_t q[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = code_word(div_rn(y[e], rscale));
      uint2 pk;
      pk.x = pack4_codes(q[0], q[1], q[2], q[3]) & keep;
      pk.y = pack4_codes(q[4], q[5], q[6], q[7]) & keep;
      const int c = tid + T * j;
      if (c < nch) *(uint2*)(orow + c * 8) = pk;
    }
    // the rare count (see k_quant_rows)
    if (counting && div_rn(amax, rscale) >= 127.5f) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        if (tid + T * j < nch) {
          float y[8];
          read_v(j, y, (uint32_t)nclip);
#pragma unroll
          for (int e = 0; e < 8; ++e) nclip += clips(div_rn(y[e], rscale));
        }
      }
    }
  };
  // the k-th row of the block uses LDS reduction slot k & 1
  for (; m < rows; m += 2 * step) {
    process(ra, m, 0);
    if (m + step < rows) process(rb, m + step, 1);
  }
  if constexpr (counting) {
    const int n = wave_sum(nclip);
    if (lane == 0 && n != 0) atomicAdd(clip, (unsigned long long)n);
  }
}

template <int DT, int CPT, int KIND>
struct LongTag {};

template <int DT, int CPT, int KIND>
static void launch_long(const char* p, int64_t rows, int64_t K, int64_t ldb, const float* s,
                        float* scale_io, int8_t* out, unsigned long long* clip, hipStream_t st) {
  auto f = k_quant_long<DT, CPT, KIND>;
  int64_t grid = rows;
  const int64_t cap = resident_blocks<LongTag<DT, CPT, KIND>>((const void*)f, kQuantMaxThreads);
  if (grid > cap) grid = cap;
  f<<<(unsigned)grid, kQuantMaxThreads, 0, st>>>(p, rows, (int)K, ldb, s, scale_io, out, clip);
}

// Block-per-row-group shape: chunks per thread CPT in {1, 2, 4, 8}, the
// smallest that lets at most 512 threads cover the row; T = threads, a
// multiple of 256 (the same number of waves on each of the CU's 4 SIMDs);
// rows per block iteration RPB = 2 for CPT <= 2, else 1.
static void pick_shape(int64_t K, int* T, int* cpt, int* rpb) {
  const int64_t chunks = K / 8;
  int c = 1;
  while (c < 8 && (chunks + c - 1) / c > kQuantMaxThreads) c *= 2;
  int64_t t = (chunks + c - 1) / c;
  t = (t + 255) / 256 * 256;
  *T = (int)t;
  *cpt = c;
  *rpb = c <= 2 ? 2 : 1;
}

template <int DT, int CPT, int KIND, int RPB>
struct RowsTag {};

template <int DT, int CPT, int KIND, int RPB>
static void launch_shape(const char* p, int64_t rows, int64_t K, int64_t ldb, const float* s,
                         float* scale_io, int8_t* out, unsigned long long* clip, int T,
                         hipStream_t st) {
  auto f = k_quant_rows<DT, CPT, KIND, RPB>;
  // One row group per block while the whole problem fits on the chip at once;
  // beyond that a full wave of blocks, each walking several groups.
  int64_t grid = (rows + RPB - 1) / RPB;
  const int64_t cap = resident_blocks<RowsTag<DT, CPT, KIND, RPB>>((const void*)f, T);
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  f<<<(unsigned)grid, T, 0, st>>>(p, rows, K, ldb, s, scale_io, out, clip);
}

// SQ_QUANT_LONG=0 selects the block-per-row-group kernel for long rows too
// (both kernels give the same codes and scales; the switch exists to time and
// test one against the other).
static bool long_rows_off() {
  const char* e = std::getenv("SQ_QUANT_LONG");
  return e != nullptr && e[0] == '0';
}

template <int DT, int KIND>
static int launch_rows_dt(const void* in, int64_t rows, int64_t K, int64_t ld, const float* s,
                          float* scale_io, int8_t* out, unsigned long long* clip, hipStream_t st) {
  const char* p = (const char*)in;
  const int64_t ldb = ld * DtSize<DT>::v;
  // waves per row: 1 up to K = 4096 (8 chunks per lane); for 16-bit inputs
  // 2 up to 8192 and 4 up to 16384
  const int64_t lane_chunks = (K / 8 + 63) / 64;
  if (lane_chunks <= 8) {
    if (lane_chunks <= 2) launch_wave<DT, KIND, 2, 1>(p, rows, K, ldb, s, scale_io, out, clip, st);
    else if (lane_chunks <= 4) launch_wave<DT, KIND, 4, 1>(p, rows, K, ldb, s, scale_io, out, clip, st);
    else launch_wave<DT, KIND, 8, 1>(p, rows, K, ldb, s, scale_io, out, clip, st);
    SQ_LAUNCH_CHECK();
    return SQ_OK;
  }
  if constexpr (DT != SQ_F32) {
    if (lane_chunks <= 32) {
      const int wpr = lane_chunks <= 16 ? 2 : 4;
      const int64_t cpl = (lane_chunks + wpr - 1) / wpr;    // 5 .. 8
#define SQ_WAVE_CPL(W)                                                                       \
  switch (cpl) {                                                                             \
    case 5: launch_wave<DT, KIND, 5, W>(p, rows, K, ldb, s, scale_io, out, clip, st); break;       \
    case 6: launch_wave<DT, KIND, 6, W>(p, rows, K, ldb, s, scale_io, out, clip, st); break;       \
    case 7: launch_wave<DT, KIND, 7, W>(p, rows, K, ldb, s, scale_io, out, clip, st); break;       \
    default: launch_wave<DT, KIND, 8, W>(p, rows, K, ldb, s, scale_io, out, clip, st); break;      \
  }
      if (wpr == 2) { SQ_WAVE_CPL(2) } else { SQ_WAVE_CPL(4) }
#undef SQ_WAVE_CPL
      SQ_LAUNCH_CHECK();
      return SQ_OK;
    }
    if (!long_rows_off()) {
      // 16384 < K <= 32768: one block per row, chunks per lane 5 .. 8
      switch ((K / 8 + kQuantMaxThreads - 1) / kQuantMaxThreads) {
        case 5: launch_long<DT, 5, KIND>(p, rows, K, ldb, s, scale_io, out, clip, st); break;
        case 6: launch_long<DT, 6, KIND>(p, rows, K, ldb, s, scale_io, out, clip, st); break;
        case 7: launch_long<DT, 7, KIND>(p, rows, K, ldb, s, scale_io, out, clip, st); break;
        default: launch_long<DT, 8, KIND>(p, rows, K, ldb, s, scale_io, out, clip, st); break;
      }
      SQ_LAUNCH_CHECK();
      return SQ_OK;
    }
  }
  int T, cpt, rpb;
  pick_shape(K, &T, &cpt, &rpb);
  switch (cpt) {
    case 1: launch_shape<DT, 1, KIND, 2>(p, rows, K, ldb, s, scale_io, out, clip, T, st); break;
    case 2: launch_shape<DT, 2, KIND, 2>(p, rows, K, ldb, s, scale_io, out, clip, T, st); break;
    case 4: launch_shape<DT, 4, KIND, 1>(p, rows, K, ldb, s, scale_io, out, clip, T, st); break;
    case 8: launch_shape<DT, 8, KIND, 1>(p, rows, K, ldb, s, scale_io, out, clip, T, st); break;
    default: return SQ_ERR_INVALID_ARG;   // K > 32768 is rejected by validation
  }
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

template <int KIND>
static int launch_rows(const void* in, int dt, int64_t rows, int64_t K, int64_t ld, const float* s,
                       float* scale_io, int8_t* out, unsigned long long* clip, hipStream_t st) {
  if (rows == 0) return SQ_OK;
  switch (dt) {
    case SQ_F32: return launch_rows_dt<SQ_F32, KIND>(in, rows, K, ld, s, scale_io, out, clip, st);
    case SQ_F16: return launch_rows_dt<SQ_F16, KIND>(in, rows, K, ld, s, scale_io, out, clip, st);
    default:     return launch_rows_dt<SQ_BF16, KIND>(in, rows, K, ld, s, scale_io, out, clip, st);
  }
}

int launch_fold_quant(const void* W, int wt, int64_t N, int64_t K, int64_t ldw, const float* s,
                      int8_t* Wq, float* w_scale, hipStream_t st) {
  return launch_rows<Q_FOLD>(W, wt, N, K, ldw, s, w_scale, Wq, nullptr, st);
}

// clip (static mode only, may be null): device uint64 the number of clamped
// codes is added to.
int launch_quant_act(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const float* s,
                     int mode, int8_t* Xq, float* a_scale, unsigned long long* clip,
                     hipStream_t st) {
  if (mode == SQ_ACT_PER_TENSOR_STATIC && clip != nullptr)
    return launch_rows<Q_STATIC_CLIP>(X, xt, M, K, ldx, s, a_scale, Xq, clip, st);
  if (mode == SQ_ACT_PER_TENSOR_STATIC)
    return launch_rows<Q_STATIC>(X, xt, M, K, ldx, s, a_scale, Xq, nullptr, st);
  return launch_rows<Q_DYNAMIC>(X, xt, M, K, ldx, s, a_scale, Xq, nullptr, st);
}

}  // namespace sq
