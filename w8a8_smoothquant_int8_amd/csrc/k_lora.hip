// LoRA delta in bf16, added to the dequantized INT8 GEMM output ([LoRA]
// Pitch), for one adapter or one adapter per request segment ([GRP]).
//
//   shrink:  P[s, m, i] = sum_{k in split s} bf16(X[m, k]) * A[i, k]   (fp32)
//   reduce:  T[m, i]    = bf16(sum_s P[s, m, i])        (fixed order of s)
//   expand:  Y[m, n]    = out(fp32(Y[m, n]) + scale * sum_i T[m, i] * B[n, i])
//
// Both are dense contractions and run on the gfx950 bf16 matrix instruction
// V_MFMA_F32_16X16X32_BF16. The shrink reads X once and is HBM-bound; with
// few row blocks at small M it splits K into S slices so enough blocks stream
// X, and writes fp32 partial sums to the caller's workspace. There is no
// atomic: a small reduce kernel sums the S partials in a fixed order into T
// (in the workspace, after the partials, for the separate expand; in the
// caller's T for the fused GEMM epilogue), so results are reproducible bit
// for bit. The expand's traffic is the read-modify-write of Y; its product
// goes through LDS so that Y is read and written in whole rows per
// instruction.
//
// Segments: each block finds the requests that overlap its rows by binary
// search in seg_start, and runs the MFMAs once per overlapping request with
// the rows of other requests zeroed, so each row picks up only its own
// adapter's product. Rows of requests without an adapter (-1) are not written.
#include "sq_internal.h"

namespace sq {

constexpr int kLoraThreads = 256;
constexpr int kMaxRankTiles = SQ_MAX_LORA_RANK / 16;   // rank tiles of 16 in the shrink
constexpr int kMaxRankSteps = SQ_MAX_LORA_RANK / 32;   // rank steps of 32 in the expand

__device__ __forceinline__ v8bf bits_to_v8bf(uint4 u) { return __builtin_bit_cast(v8bf, u); }

// 8 elements of X at p as bf16 bits (RNE for f32/f16 inputs).
template <int XT>
__device__ __forceinline__ uint4 load8_as_bf16(const char* p) {
  if constexpr (XT == SQ_BF16) {
    return *(const uint4*)p;
  } else {
    float v[8];
    load8_f32<XT>(p, v);
    uint4 u;
    u.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
    u.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
    u.z = f32_to_bf16_bits(v[4]) | (f32_to_bf16_bits(v[5]) << 16);
    u.w = f32_to_bf16_bits(v[6]) | (f32_to_bf16_bits(v[7]) << 16);
    return u;
  }
}

// Largest g with seg_start[g] <= m (segments are non-decreasing, seg_start[0] = 0).
__device__ __forceinline__ int find_segment(const int32_t* seg_start, int nseg, int m) {
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seg_start[mid] <= m) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One (request, 64-row tile) pair of a segmented call: rows [m0, mend) of
// one request and its adapter; ad = -1 past the last pair.
struct SegPair {
  int m0, mend, ad, pad;
};

struct LoraArgs {
  // single adapter
  const unsigned short* A;   // [r, K] bf16
  const unsigned short* B;   // [N, r] bf16
  int r;
  // segmented
  const int32_t* seg_start;
  const int32_t* seg_adapter;
  int nseg;
  const void* const* A_ptrs;
  const void* const* B_ptrs;
  const int32_t* ranks;
  const SegPair* pairs;      // the call's pair table (k_seg_pairs), in the workspace
};

// Single-adapter shrink, written as partial sums P[s] over groups of k-chunks.
//
// grid: (ceil(M / (64 * RT)), S). A block has 4 waves; wave w owns RT row
// tiles of 16 rows (rows m0 + 16 * rt + 0..15), so a block covers 64 * RT
// rows. The block visits k-chunks c = blockIdx.y, blockIdx.y + S, ... of
// KC = 32 * KS elements. For each chunk it stages A[0:R, chunk] in LDS once
// for all its waves (direct global-to-LDS loads) while each wave loads its
// rows' X for the chunk into registers, all in flight together; then every
// 16-row rank tile of A is read from LDS once per k-step and multiplied with
// each of the wave's row tiles.
//
// LDS layout of the staged chunk: row i of A at i * KC * 2 bytes, its 16-byte
// slot p holding k-chunk p ^ (i & 15). Rows are a multiple of 256 bytes long,
// so the 16 lanes of one fragment read (rows 16t + 0..15, one logical slot)
// land on 16 distinct 16-byte bank groups: all 64 banks, no conflict.
//
// The product is computed transposed (A rows as the first MFMA operand), so a
// lane's 4 output registers are 4 consecutive ranks of one row: one 16-byte
// store into P[s, m, i..i+3].
template <int XT, int KS, int RT, int NT>
__global__ void __launch_bounds__(kLoraThreads)
k_lora_shrink(const char* __restrict__ X, int64_t ldx_bytes, int M, int K,
              const unsigned short* __restrict__ A, int R, int S, float* __restrict__ P) {
  extern __shared__ __attribute__((aligned(1024))) char lds_a[];   // R x KC bf16
  constexpr int KC = 32 * KS;        // k elements per chunk
  constexpr int CPR = KC / 8;        // 16-byte slots per staged row (32 or 16)
  constexpr int RPI = 64 / CPR;      // staged rows per direct load (2 or 4)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 15, kg = lane >> 4;
  const int nI = R / RPI;            // direct loads per chunk (R % 8 == 0)
  const int nchunks = (K + KC - 1) / KC;
  const int m0 = blockIdx.x * (64 * RT) + wave * (16 * RT);

  // Rows past M read row M - 1; their sums are never stored.
  const char* xrow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int m = m0 + rt * 16 + lrow;
    m = m < M ? m : M - 1;
    xrow[rt] = X + (int64_t)m * ldx_bytes;
  }

  v4f acc[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[rt][t] = v4f{0, 0, 0, 0};

#pragma unroll 1
  for (int c = blockIdx.y; c < nchunks; c += S) {
    const int kc0 = c * KC;
    __syncthreads();   // every wave is done reading the previous chunk
    // A chunk -> LDS. Load j moves staged rows j * RPI .. + RPI - 1; lane l
    // fills slot l % CPR of row j * RPI + l / CPR with the k-chunk that
    // belongs there. Slots past K read a valid chunk and are zeroed on use.
    for (int j = wave; j < nI; j += 4) {
      const int i = j * RPI + lane / CPR;
      const int kk = kc0 + ((lane % CPR) ^ (i & 15)) * 8;
      const int ksrc = kk < K ? kk : K - 8;
      __builtin_amdgcn_global_load_lds((const void*)(A + (int64_t)i * K + ksrc),
                                       (lds_ptr_t)(lds_a + 1024 * j), 16, 0, 0);
    }
    uint4 xu[RT][KS];
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      const int kk = kc0 + u * 32 + kg * 8;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        xu[rt][u] = kk < K ? load8_as_bf16<XT>(xrow[rt] + (int64_t)kk * DtSize<XT>::v)
                           : make_uint4(0, 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): the chunk is in LDS
    __syncthreads();

    // Rank rows past R (the last tile of a rank that is not a multiple of
    // 16) and slots past K read staged row R - 1 and are replaced by zeros.
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      const int slot = u * 4 + kg;
      const bool kin = kc0 + slot * 8 < K;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int i = t * 16 + lrow;
        const int ic = i < R ? i : R - 1;
        uint4 au = *(const uint4*)(lds_a + ic * (KC * 2) + ((slot ^ (ic & 15)) << 4));
        if (!(kin && i < R)) au = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bits_to_v8bf(au),
                                                              bits_to_v8bf(xu[rt][u]),
                                                              acc[rt][t], 0, 0, 0);
      }
    }
  }

  // Register j of rank tile t: rank 16 t + 4 (lane / 16) + j, row lane % 16.
  float* Ps = P + (int64_t)blockIdx.y * M * R;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int m = m0 + rt * 16 + lrow;
    if (m >= M) continue;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int i = t * 16 + kg * 4;
      if (i < R)
        *(float4*)(Ps + (int64_t)m * R + i) =
            make_float4(acc[rt][t][0], acc[rt][t][1], acc[rt][t][2], acc[rt][t][3]);
    }
  }
}

// 8 values of a 16-bit X as bf16 bits (RNE from fp16; identity for bf16).
template <int XT>
__device__ __forceinline__ uint4 raw16_as_bf16(uint4 raw) {
  if constexpr (XT == SQ_BF16) {
    return raw;
  } else {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = f32_to_bf16_bits(f16_bits_to_f32(w[q] & 0xFFFFu)) |
             (f32_to_bf16_bits(f16_bits_to_f32(w[q] >> 16)) << 16);
    return make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Pipelined single-adapter shrink for 16-bit X: the same partial sums P[s] as
// k_lora_shrink, with one chunk of loads always in flight. Per chunk:
//   wait for this wave's loads of the chunk (vmcnt(0): they are the only
//   ones outstanding), barrier (the chunk's staged A is complete for every
//   wave, and every wave is done with the chunk before);
//   stage the next chunk's A into the other slot of a two-slot LDS ring and
//   load this wave's X for it into the other register set;
//   multiply the current chunk.
// A slot holds NT * 16 staged rows (rows past R re-read row R - 1; their
// products land in ranks that are never stored), swizzled as in
// k_lora_shrink. Every load is unconditional, with addresses past K clamped
// to valid ones and the X values zeroed on use, so each wave issues the same
// loads per chunk. grid: (ceil(M / (64 * RT)), S); block: 4 waves of RT row
// tiles of 16 rows.
template <int XT, int KS, int RT, int NT>
__global__ void __launch_bounds__(kLoraThreads)
k_lora_shrink_pipe(const char* __restrict__ X, int64_t ldx_bytes, int M, int K,
                   const unsigned short* __restrict__ A, int R, int S, float* __restrict__ P) {
  extern __shared__ __attribute__((aligned(1024))) char lds_a[];   // 2 x (NT*16) x KC bf16
  constexpr int KC = 32 * KS;        // k elements per chunk
  constexpr int CPR = KC / 8;        // 16-byte slots per staged row
  constexpr int RPI = 64 / CPR;      // staged rows per direct load
  constexpr int ROWS = NT * 16;      // staged rows per slot
  constexpr int NA = ROWS / RPI / 4; // direct loads per wave per chunk
  constexpr int SLOT = ROWS * KC * 2;
  static_assert(ROWS % (RPI * 4) == 0, "staged rows must split over the 4 waves");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 15, kg = lane >> 4;
  const int nchunks = (K + KC - 1) / KC;
  const int m0 = blockIdx.x * (64 * RT) + wave * (16 * RT);

  // Rows past M read row M - 1; their sums are never stored.
  const char* xrow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int m = m0 + rt * 16 + lrow;
    m = m < M ? m : M - 1;
    xrow[rt] = X + (int64_t)m * ldx_bytes;
  }

  auto stage = [&](int c, int slot) {
    const int kc0 = c * KC;
    char* dst = lds_a + slot * SLOT;
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      const int j = wave + 4 * q;
      const int i = j * RPI + lane / CPR;
      const int isrc = i < R ? i : R - 1;
      const int kk = kc0 + ((lane % CPR) ^ (i & 15)) * 8;
      const int ksrc = kk < K ? kk : K - 8;
      __builtin_amdgcn_global_load_lds((const void*)(A + (int64_t)isrc * K + ksrc),
                                       (lds_ptr_t)(dst + 1024 * j), 16, 0, 0);
    }
  };
  auto load_x = [&](int c, uint4 (&xu)[RT][KS]) {
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      const int kk = c * KC + u * 32 + kg * 8;
      const int ksrc = kk < K ? kk : K - 8;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) xu[rt][u] = *(const uint4*)(xrow[rt] + (int64_t)ksrc * 2);
    }
  };

  v4f acc[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[rt][t] = v4f{0, 0, 0, 0};

  auto multiply = [&](int c, int slot, const uint4 (&xu)[RT][KS]) {
    const int kc0 = c * KC;
    const char* sa = lds_a + slot * SLOT;
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      const int sl = u * 4 + kg;
      const bool kin = kc0 + sl * 8 < K;
      uint4 xv[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) xv[rt] = kin ? raw16_as_bf16<XT>(xu[rt][u]) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int i = t * 16 + lrow;
        const uint4 au = *(const uint4*)(sa + i * (KC * 2) + ((sl ^ (i & 15)) << 4));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bits_to_v8bf(au), bits_to_v8bf(xv[rt]),
                                                              acc[rt][t], 0, 0, 0);
      }
    }
  };

  // one chunk: the current loads in `cur`, slot `slot`; the next chunk's into `nxt`
  auto step = [&](int c, int slot, const uint4 (&cur)[RT][KS], uint4 (&nxt)[RT][KS]) {
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    if (c + S < nchunks) {
      stage(c + S, slot ^ 1);
      load_x(c + S, nxt);
    }
    multiply(c, slot, cur);
  };

  uint4 xa[RT][KS], xb[RT][KS];
  int c = blockIdx.y;
  if (c < nchunks) {
    stage(c, 0);
    load_x(c, xa);
  }
#pragma unroll 1
  for (; c < nchunks; c += 2 * S) {
    step(c, 0, xa, xb);
    if (c + S >= nchunks) break;
    step(c + S, 1, xb, xa);
  }

  // Register j of rank tile t: rank 16 t + 4 (lane / 16) + j, row lane % 16.
  float* Ps = P + (int64_t)blockIdx.y * M * R;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int m = m0 + rt * 16 + lrow;
    if (m >= M) continue;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int i = t * 16 + kg * 4;
      if (i < R)
        *(float4*)(Ps + (int64_t)m * R + i) =
            make_float4(acc[rt][t][0], acc[rt][t][1], acc[rt][t][2], acc[rt][t][3]);
    }
  }
}

// Segmented shrink. grid: (ceil(M / 64), S); 4 waves, each a 16-row tile of
// its K slice. A fragments come straight from global memory (L2): the
// adapter can change from one row tile to the next.
template <int XT>
__global__ void __launch_bounds__(kLoraThreads)
k_lora_shrink_seg(const char* __restrict__ X, int64_t ldx_bytes, int M, int K, LoraArgs la, int R,
                  int kchunk, float* __restrict__ P) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m0 = blockIdx.x * 64 + wave * 16;
  if (m0 >= M) return;
  const int s = blockIdx.y;
  const int ks = s * kchunk;
  const int ke = ks + kchunk < K ? ks + kchunk : K;
  const int lrow = lane & 15, kg = lane >> 4;
  const int my_m = m0 + lrow;
  const int NT = (R + 15) / 16;

  v4f acc[kMaxRankTiles];
#pragma unroll
  for (int t = 0; t < kMaxRankTiles; ++t) acc[t] = v4f{0, 0, 0, 0};

  const int g0 = find_segment(la.seg_start, la.nseg, m0);
  int g1 = g0;
  {
    const int mend = m0 + 16 < M ? m0 + 16 : M;
    while (g1 + 1 < la.nseg && la.seg_start[g1 + 1] < mend) ++g1;
  }

  // U k-steps per batch: the batch's X fragments, then per request and rank
  // tile its U adapter fragments, are all issued before their MFMAs, so
  // loads overlap instead of one load -> MFMA round trip per k-step. For each
  // row only its own request contributes (other rows' fragments are zero),
  // in increasing k, as with one k-step at a time.
  constexpr int U = 8;
  for (int k = ks; k < ke; k += 32 * U) {
    uint4 xu[U];
    bool kin[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k + 32 * u + kg * 8;
      kin[u] = kk < ke;
      xu[u] = (kin[u] && my_m < M)
                  ? load8_as_bf16<XT>(X + (int64_t)my_m * ldx_bytes + (int64_t)kk * DtSize<XT>::v)
                  : make_uint4(0, 0, 0, 0);
    }
    for (int g = g0; g <= g1; ++g) {
      const int ad = la.seg_adapter[g];
      if (ad < 0) continue;
      const int ra = la.ranks[ad];
      const unsigned short* Ag = (const unsigned short*)la.A_ptrs[ad];
      const bool mine = my_m >= la.seg_start[g] && my_m < la.seg_start[g + 1];
#pragma unroll
      for (int t = 0; t < kMaxRankTiles; ++t) {
        if (t < NT) {
          const int i = t * 16 + lrow;
          uint4 au[U];
#pragma unroll
          for (int u = 0; u < U; ++u)
            au[u] = (kin[u] && i < ra) ? *(const uint4*)(Ag + (int64_t)i * K + k + 32 * u + kg * 8)
                                       : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int u = 0; u < U; ++u)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                bits_to_v8bf(mine ? xu[u] : make_uint4(0, 0, 0, 0)), bits_to_v8bf(au[u]), acc[t], 0, 0, 0);
        }
      }
    }
  }

  // Output register j of a 16x16 tile holds row 4*(lane/16) + j, column lane%16.
  float* Ps = P + (int64_t)s * M * R;
#pragma unroll
  for (int t = 0; t < kMaxRankTiles; ++t) {
    if (t < NT) {
      const int i = t * 16 + lrow;
      if (i < R) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = m0 + kg * 4 + j;
          if (m < M) Ps[(int64_t)m * R + i] = acc[t][j];
        }
      }
    }
  }
}

// The (request, 64-row tile) pairs of a segmented call, in request order:
// ceil(len / 64) of them for every non-empty request with an adapter. One
// block scans the request table once per call, kSegScan requests per round
// (wave prefix sums with lane shifts, then the wave totals), and writes entry
// b of the table for every pair b; the entries from the pair count up to
// n_entries get ad = -1. The shrink and expand blocks then find their pair
// with one load instead of each scanning the table (they read the adapter's
// rank next to its A or B pointer). n_entries = ceil(M / 64) +
// min(requests, M) bounds the pair count of well-formed tables (rows within
// [0, M)); writes past it are dropped.
constexpr int kSegScan = 256;
__global__ void __launch_bounds__(kSegScan) k_seg_pairs(LoraArgs la, SegPair* __restrict__ tab,
                                                        int n_entries) {
  constexpr int NW = kSegScan / 64;
  __shared__ int s_wsum[NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int base = 0;
  for (int c0 = 0; c0 < la.nseg; c0 += kSegScan) {
    const int g = c0 + tid;
    int tiles = 0, s0 = 0, s1 = 0, ad = -1;
    if (g < la.nseg) {
      ad = la.seg_adapter[g];
      s0 = la.seg_start[g];
      s1 = la.seg_start[g + 1];
      if (ad >= 0 && s1 > s0) tiles = (s1 - s0 + 63) >> 6;
    }
    int incl = tiles;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int before = base, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      before += w < wave ? s_wsum[w] : 0;
      total += s_wsum[w];
    }
    const int e = before + incl - tiles;   // this request's first pair
    for (int q = 0; q < tiles && e + q < n_entries; ++q) {
      const int m0 = s0 + 64 * q;
      tab[e + q] = SegPair{m0, m0 + 64 < s1 ? m0 + 64 : s1, ad, 0};
    }
    base += total;
    __syncthreads();   // s_wsum is rewritten by the next round
  }
  for (int b = base + tid; b < n_entries; b += blockDim.x) tab[b] = SegPair{0, 0, -1, 0};
}

// Pipelined segmented shrink for 16-bit X: k_lora_shrink_pipe with one
// adapter per block. Block (b, s) takes pair b of the call's pair table, so
// every row of the block uses one adapter: its
// A[0:r, chunk] is staged in the two-slot LDS ring (r rounded up to 16; rows
// past r re-read row r - 1) and multiplied over the adapter's rank tiles
// only; ranks r .. R - 1 of the partial sums are stored as 0. Rows past the request's end read its last
// row and are not stored. The K slices, the chunk order and the arithmetic
// per row are those of k_lora_shrink_pipe for the same S, so a single
// adapter over all rows gives the same partial sums bit for bit.
// grid: (ceil(M / 64) + requests, S); blocks past the last tile exit.
template <int XT, int KS, int NT>
__global__ void __launch_bounds__(kLoraThreads)
k_lora_shrink_seg_pipe(const char* __restrict__ X, int64_t ldx_bytes, int M, int K, LoraArgs la,
                       int R, int S, float* __restrict__ P) {
  extern __shared__ __attribute__((aligned(1024))) char lds_a[];   // 2 x (NT*16) x KC bf16
  constexpr int KC = 32 * KS;
  constexpr int CPR = KC / 8;
  constexpr int RPI = 64 / CPR;
  constexpr int ROWS = NT * 16;
  constexpr int NA = ROWS / RPI / 4;
  constexpr int SLOT = ROWS * KC * 2;
  static_assert(ROWS % (RPI * 4) == 0, "staged rows must split over the 4 waves");
  const SegPair pr = la.pairs[blockIdx.x];
  if (pr.ad < 0) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 15, kg = lane >> 4;
  const int nchunks = (K + KC - 1) / KC;
  const int s_end = pr.mend;
  const int w0 = pr.m0 + wave * 16;
  const int my_m = w0 + lrow;
  const bool wave_rows = w0 < s_end;   // the wave holds rows of the request
  const char* xrow = X + (int64_t)(my_m < s_end ? my_m : s_end - 1) * ldx_bytes;
  const int ra = la.ranks[pr.ad];
  const int ntg = (ra + 15) >> 4;
  const unsigned short* Ag = (const unsigned short*)la.A_ptrs[pr.ad];

  auto stage = [&](int c, int slot) {
    const int kc0 = c * KC;
    char* dst = lds_a + slot * SLOT;
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      const int j = wave + 4 * q;
      if (j * RPI < ntg * 16) {
        const int i = j * RPI + lane / CPR;
        const int isrc = i < ra ? i : ra - 1;
        const int kk = kc0 + ((lane % CPR) ^ (i & 15)) * 8;
        const int ksrc = kk < K ? kk : K - 8;
        __builtin_amdgcn_global_load_lds((const void*)(Ag + (int64_t)isrc * K + ksrc),
                                         (lds_ptr_t)(dst + 1024 * j), 16, 0, 0);
      }
    }
  };
  auto load_x = [&](int c, uint4 (&xu)[KS]) {
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      const int kk = c * KC + u * 32 + kg * 8;
      const int ksrc = kk < K ? kk : K - 8;
      xu[u] = *(const uint4*)(xrow + (int64_t)ksrc * 2);
    }
  };

  v4f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = v4f{0, 0, 0, 0};

  auto multiply = [&](int c, int slot, const uint4 (&xu)[KS]) {
    if (!wave_rows) return;
    const int kc0 = c * KC;
    const char* sa = lds_a + slot * SLOT;
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      const int sl = u * 4 + kg;
      const uint4 xv = kc0 + sl * 8 < K ? raw16_as_bf16<XT>(xu[u]) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < ntg) {
          const int i = t * 16 + lrow;
          const uint4 au = *(const uint4*)(sa + i * (KC * 2) + ((sl ^ (i & 15)) << 4));
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bits_to_v8bf(au), bits_to_v8bf(xv), acc[t],
                                                           0, 0, 0);
        }
      }
    }
  };

  auto step = [&](int c, int slot, const uint4 (&cur)[KS], uint4 (&nxt)[KS]) {
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    if (c + S < nchunks) {
      stage(c + S, slot ^ 1);
      load_x(c + S, nxt);
    }
    multiply(c, slot, cur);
  };

  uint4 xa[KS], xb[KS];
  int c = blockIdx.y;
  if (c < nchunks) {
    load_x(c, xa);   // needs only the pair; the staging waits for the adapter pointer
    stage(c, 0);
  }
#pragma unroll 1
  for (; c < nchunks; c += 2 * S) {
    step(c, 0, xa, xb);
    if (c + S >= nchunks) break;
    step(c + S, 1, xb, xa);
  }

  // Register j of rank tile t: rank 16 t + 4 (lane / 16) + j, row lane % 16.
  // Ranks from the adapter's r up to R are stored as 0 (r is a multiple of 8,
  // so a group of 4 is wholly in or out).
  float* Ps = P + (int64_t)blockIdx.y * M * R;
  if (my_m < s_end) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int i = t * 16 + kg * 4;
      if (i < R)
        *(float4*)(Ps + (int64_t)my_m * R + i) =
            i < ra ? make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// Expand over 64 x 256 output tiles, with the product passed through LDS so
// that the read-modify-write of Y is coalesced. 4 waves.
//   1. Every thread issues its loads of the Y tile first: 16 bytes per lane,
//      consecutive lanes along a row (a row of the tile is 512 bytes of
//      16-bit Y or 1024 of fp32).
//   2. Wave w computes D = T[rows] . B[cols 64 w .. 64 w + 63]^T for all 64
//      rows (4 x 4 tiles of 16 x 16), so every B fragment it loads serves 64
//      rows. With segments, row tile x is pair x of the call's pair table:
//      all its rows use one adapter, and rows past the request's end are
//      neither read nor written.
//   3. D goes to LDS as fp32 (float4 slot c of row i stored at c ^ (i & 15):
//      the 16 rows of an MFMA tile land on all 64 banks); after a barrier each
//      thread reads the D values of its Y elements and writes
//      out(fp32(y) + scale * d). Rows without an adapter are not written.
// KSM: rank steps of 32, ceil(R / 32): T's rows hold 32 * KSM ranks, zero from R on.
// grid: (ceil(M / 64), ceil(N / 256)); with segments ceil(M / 64) + min(requests, M)
// row blocks, those past the last (request, tile) pair exiting at once.
template <int YT, bool SEG, int KSM>
__global__ void __launch_bounds__(kLoraThreads, 2)
k_lora_expand(const unsigned short* __restrict__ T, int M, int N, LoraArgs la, float scale,
              void* __restrict__ Y, int64_t ldy, int row_tiles, int col_tiles) {
  constexpr int BM = 64, BN = 256;
  __shared__ __attribute__((aligned(16))) float dl[BM * BN];   // 64 KB
  constexpr int VPT = YT == SQ_F32 ? 4 : 8;   // Y values per 16-byte access
  constexpr int TPR = BN / VPT;               // threads per tile row
  constexpr int RPP = 256 / TPR;              // tile rows per pass
  constexpr int NP = BM / RPP;                // passes
  // The next tile's Y loads are issued before this tile's product where the
  // registers allow a second Y tile next to the B and T fragments: 16-bit Y
  // (8 words a thread) and ranks up to 64.
  constexpr bool PF = KSM <= 2 && YT != SQ_F32;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 15, kg = lane >> 4;
  const int pr = tid / TPR, pc = (tid % TPR) * VPT;

  // Tile `it` (column tiles fastest): rows [m0, mend), their adapter, and
  // columns from n0. False when it holds no rows (past the last (request,
  // tile) pair; every later tile is then empty too). Block-uniform.
  struct Tile {
    int m0, mend, r, n0;
    const unsigned short* Bm;
  };
  auto tile_of = [&](int it, Tile& t) -> bool {
    if (it >= row_tiles * col_tiles) return false;
    const int tm = it / col_tiles;
    t.n0 = (it % col_tiles) * BN;
    if constexpr (SEG) {
      const SegPair pr = la.pairs[tm];
      if (pr.ad < 0) return false;
      t.m0 = pr.m0;
      t.mend = pr.mend;
      t.Bm = (const unsigned short*)la.B_ptrs[pr.ad];
      t.r = la.ranks[pr.ad];
    } else {
      t.m0 = tm * BM;
      t.mend = t.m0 + BM < M ? t.m0 + BM : M;
      t.Bm = la.B;
      t.r = la.r;
    }
    return true;
  };
  // The Y tile, coalesced (rows past mend and columns past N read the tile's
  // first row and column, and are not stored).
  auto load_y = [&](const Tile& t, uint4 (&yv)[NP]) {
    const bool col_ok = t.n0 + pc < N;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int m = t.m0 + p * RPP + pr;
      const int64_t off = (int64_t)(m < t.mend ? m : t.m0) * ldy + (col_ok ? t.n0 + pc : t.n0);
      yv[p] = YT == SQ_F32 ? *(const uint4*)((const float*)Y + off)
                           : *(const uint4*)((const unsigned short*)Y + off);
    }
  };

  // One tile: Y (its values in yc, loaded earlier with PF) += scale * T B^T.
  // Every load is unconditional, with out-of-range addresses clamped to
  // valid ones, and no value needs masking: T rows are zero from the
  // adapter's rank up to Rp (its B columns past r, clamped, meet zeros),
  // clamped T rows stay inside the block's request (finite values whose D
  // rows are not stored), and D columns past N are not stored either.
  // (A select between a loaded value and 0, or a load skipped by a branch,
  // would end in a wait for all loads in flight, the Y tiles' included.)
  auto process = [&](const Tile& t, uint4 (&yc)[NP], const Tile* nxt, uint4 (&yn)[NP]) {
    const int nw = t.n0 + 64 * wave;   // this wave's 64 columns of the tile
    constexpr int Rp = 32 * KSM;       // T's row stride (R rounded up to 32)
    const int r = t.r, m0 = t.m0, mend = t.mend;
    const unsigned short* Bm = t.Bm;
    // The B and T fragments of rank step ks: B rows nw + 16 u + lane % 16,
    // T rows m0 + 16 rt + lane % 16, ranks 32 ks + 8 (lane / 16) .. + 7.
    auto load_bt = [&](int ks, uint4 (&bu)[4], uint4 (&tu)[4]) {
      const int k = ks * 32 + kg * 8;
      const int kb = k < r ? k : r - 8;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int n = nw + u * 16 + lrow;
        bu[u] = *(const uint4*)(Bm + (int64_t)(n < N ? n : N - 1) * r + kb);
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int m = m0 + rt * 16 + lrow;
        tu[rt] = *(const uint4*)(T + (int64_t)(m < mend ? m : mend - 1) * Rp + k);
      }
    };
    // The fragments of the first PRE rank steps load first (the scheduling
    // barriers keep the order), so the MFMAs wait only for them while the Y
    // loads stay in flight through the product.
    constexpr int PRE = YT == SQ_F32 && KSM > 2 ? 2 : KSM;
    uint4 bf[KSM][4], tf[KSM][4];
#pragma unroll
    for (int ks = 0; ks < PRE; ++ks) load_bt(ks, bf[ks], tf[ks]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (PF) {
      if (nxt != nullptr) load_y(*nxt, yn);
    } else {
      load_y(t, yc);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = PRE; ks < KSM; ++ks) load_bt(ks, bf[ks], tf[ks]);

    // D for rows m0 .. m0 + 63, columns nw .. nw + 63: per rank step 16
    // MFMAs (4 row tiles x 4 column tiles of 16 x 16).
    v4f acc[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[rt][u] = v4f{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < KSM; ++ks)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc[rt][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bits_to_v8bf(bf[ks][u]), bits_to_v8bf(tf[ks][rt]),
                                                               acc[rt][u], 0, 0, 0);

    // D through LDS (float4 slot c of row i stored at c ^ (i & 15)): register
    // j of tile (rt, u) is row 16 rt + lane % 16, column 64 w + 16 u + 4 kg + j.
    __syncthreads();   // every thread is done reading the previous tile's D
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int i = rt * 16 + lrow;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c4 = 16 * wave + 4 * u + kg;
        *(float4*)(dl + i * BN + ((c4 ^ (i & 15)) << 2)) =
            make_float4(acc[rt][u][0], acc[rt][u][1], acc[rt][u][2], acc[rt][u][3]);
      }
    }
    __syncthreads();

    const bool col_ok = t.n0 + pc < N;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int i = p * RPP + pr;
      const int m = m0 + i;
      if (m >= mend || !col_ok) continue;
      const int64_t off = (int64_t)m * ldy + t.n0 + pc;
      const int c4 = pc >> 2;
      const float4 d0 = *(const float4*)(dl + i * BN + ((c4 ^ (i & 15)) << 2));
      if constexpr (YT == SQ_F32) {
        float4 y = make_float4(__uint_as_float(yc[p].x), __uint_as_float(yc[p].y),
                               __uint_as_float(yc[p].z), __uint_as_float(yc[p].w));
        y.x = y.x + scale * d0.x; y.y = y.y + scale * d0.y;
        y.z = y.z + scale * d0.z; y.w = y.w + scale * d0.w;
        *(float4*)((float*)Y + off) = y;
      } else {
        const float4 d1 = *(const float4*)(dl + i * BN + (((c4 + 1) ^ (i & 15)) << 2));
        const float d[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
        const uint32_t w[4] = {yc[p].x, yc[p].y, yc[p].z, yc[p].w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t h[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t bb = e ? w[q] >> 16 : w[q] & 0xFFFFu;
            float y = YT == SQ_BF16 ? bf16_bits_to_f32(bb) : f16_bits_to_f32(bb);
            y = y + scale * d[2 * q + e];
            h[e] = YT == SQ_BF16 ? f32_to_bf16_bits(y) : f32_to_f16_bits(y);
          }
          o[q] = h[0] | (h[1] << 16);
        }
        *(uint4*)((unsigned short*)Y + off) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  };

  // Persistent over the tiles (blockIdx.x, + gridDim.x, ...), two Y register
  // sets taking turns. A tile's Y rows are read and written only by its own
  // block, so the prefetch of the next tile never meets a store of another.
  Tile ta, tb;
  uint4 ya[NP], yb[NP];
  int it = blockIdx.x;
  if (!tile_of(it, ta)) return;
  if constexpr (PF) load_y(ta, ya);
  for (;;) {
    const bool hb = tile_of(it + (int)gridDim.x, tb);
    process(ta, ya, hb ? &tb : nullptr, yb);
    if (!hb) break;
    it += gridDim.x;
    const bool ha = tile_of(it + (int)gridDim.x, ta);
    process(tb, yb, ha ? &ta : nullptr, ya);
    if (!ha) break;
    it += gridDim.x;
  }
}

// T[m, i] = bf16(sum_s P[s, m, i]) (fixed order of s) for i < R, and 0 for
// R <= i < RT (zero padding of T's rows up to a whole rank step of the
// expand). One thread per 4 consecutive ranks of one row, 64-thread blocks
// (enough blocks at small M). The loads of 8 slices are issued together; the
// sums stay in slice order.
__global__ void __launch_bounds__(64)
k_lora_reduce(const float* __restrict__ P, int S, int R, int RT, int M, unsigned short* __restrict__ T,
              int64_t ldt) {
  const int64_t id = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const int per_row = RT / 4;
  if (id >= (int64_t)M * per_row) return;
  const int m = (int)(id / per_row), i = (int)(id % per_row) * 4;
  float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
  if (i < R) {
    const int64_t slice = (int64_t)M * R;
    const float* p = P + (int64_t)m * R + i;
    int s = 0;
    for (; s + 8 <= S; s += 8) {
      float4 a[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] = *(const float4*)(p + (s + u) * slice);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        t.x += a[u].x; t.y += a[u].y; t.z += a[u].z; t.w += a[u].w;
      }
    }
    for (; s < S; ++s) {
      const float4 a = *(const float4*)(p + s * slice);
      t.x += a.x; t.y += a.y; t.z += a.z; t.w += a.w;
    }
  }
  uint2 u;
  u.x = f32_to_bf16_bits(t.x) | (f32_to_bf16_bits(t.y) << 16);
  u.y = f32_to_bf16_bits(t.z) | (f32_to_bf16_bits(t.w) << 16);
  *(uint2*)(T + (int64_t)m * ldt + i) = u;
}

// Launch plan of the single-adapter shrink. KC = 256 (8 k-steps) when the
// staged A chunk (R x KC bf16) fits in 32 KB, else 128. Two row tiles per
// wave (A fragments read from LDS serve 32 rows) unless that leaves fewer
// than ~512 (row block, chunk) pairs. S slices, each a strided set of J
// chunks: S <= 32 bounds the partial sums at 32 * M * R fp32.
struct ShrinkPlan {
  int ks, rt, nt, S;   // nt: rank tiles of 16, rounded up to 1, 2, 4 or 8
  int64_t blocks_m;
};

static ShrinkPlan plan_shrink(int64_t M, int64_t K, int R) {
  ShrinkPlan p;
  p.ks = R <= 64 ? 8 : 4;
  p.nt = R <= 16 ? 1 : R <= 32 ? 2 : R <= 64 ? 4 : 8;
  const int64_t kc = 32 * p.ks;
  const int64_t nch = (K + kc - 1) / kc;
  p.rt = 2;
  p.blocks_m = (M + 127) / 128;
  if (p.blocks_m * nch < 512 && M > 64) {
    p.rt = 1;
    p.blocks_m = (M + 63) / 64;
  }
  int64_t s = (512 + p.blocks_m - 1) / p.blocks_m;
  if (s > 32) s = 32;
  if (s > nch) s = nch;
  const int64_t j = (nch + s - 1) / s;   // chunks per slice
  p.S = (int)((nch + j - 1) / j);
  return p;
}

// Plan of the pipelined shrink (16-bit X): one row tile per wave (64 rows per
// block), about 512 blocks (two per CU, the LDS ring allowing), and as few
// K slices as that takes, so that blocks keep several chunks for the
// pipeline and the partial sums stay small.
static ShrinkPlan plan_shrink_pipe(int64_t M, int64_t K, int R) {
  ShrinkPlan p;
  p.ks = R <= 64 ? 8 : 4;
  p.nt = R <= 16 ? 1 : R <= 32 ? 2 : R <= 64 ? 4 : 8;
  const int64_t kc = 32 * p.ks;
  const int64_t nch = (K + kc - 1) / kc;
  p.rt = 1;
  p.blocks_m = (M + 63) / 64;
  int64_t s = (512 + p.blocks_m - 1) / p.blocks_m;
  if (s > 32) s = 32;
  if (s > nch) s = nch;
  if (s < 1) s = 1;
  const int64_t j = (nch + s - 1) / s;
  p.S = (int)((nch + j - 1) / j);
  return p;
}

// Split of K for the segmented shrink: about 2048 (16-row tile, slice) waves,
// slices of at least 256 and a multiple of 32 elements, at most 16 slices.
static void seg_split(int64_t M, int64_t K, int* S, int* kchunk) {
  const int64_t m_tiles = (M + 15) / 16;
  int64_t s = (2048 + m_tiles - 1) / (m_tiles > 0 ? m_tiles : 1);
  int64_t smax = K / 256;
  if (smax < 1) smax = 1;
  if (s > smax) s = smax;
  if (s > 16) s = 16;
  if (s < 1) s = 1;
  int64_t kc = (K + s - 1) / s;
  kc = (kc + 31) / 32 * 32;
  *kchunk = (int)kc;
  *S = (int)((K + kc - 1) / kc);
}

// Partial sums and T for any rank up to R, single-adapter or segmented: the
// offset of the segmented pair table in the workspace.
static size_t lora_ws_base(int64_t M, int64_t K, int R) {
  int S, kc;
  seg_split(M, K, &S, &kc);
  int64_t smax = S;
  const int probe[2] = {R < 64 ? R : 64, R};   // both chunk widths the rank range can use
  for (int q = 0; q < 2; ++q) {
    const ShrinkPlan p = plan_shrink(M, K, probe[q]);
    if (p.S > smax) smax = p.S;
    const ShrinkPlan pp = plan_shrink_pipe(M, K, probe[q]);
    if (pp.S > smax) smax = pp.S;
  }
  // fp32 partial sums of up to smax slices, then the reduced T [M, Rp] bf16
  // (rows zero-padded to Rp = 32 * ceil(R / 32) ranks)
  const int64_t Rp = (R + 31) / 32 * 32;
  return (size_t)smax * (size_t)M * (size_t)R * sizeof(float) + (size_t)M * (size_t)Rp * 2;
}

// Entries of a segmented call's pair table: ceil(M / 64) + min(requests, M).
static int64_t seg_pair_entries(int64_t M, int nseg) {
  return (M + 63) / 64 + (nseg < M ? nseg : M);
}

// The whole workspace: partial sums, T, then room for the pair table of a
// segmented call with any number of requests.
size_t lora_ws_bytes(int64_t M, int64_t K, int R) {
  return lora_ws_base(M, K, R) + (size_t)seg_pair_entries(M, (int)(M < INT32_MAX ? M : INT32_MAX)) *
                                     sizeof(SegPair);
}

// Single-adapter shrink into P; returns the number of slices written.
template <int XT>
static int launch_shrink_p(const void* X, int64_t M, int64_t K, int64_t ldx, const unsigned short* A,
                           int R, float* P, hipStream_t st) {
  if constexpr (XT != SQ_F32) {
    const ShrinkPlan p = plan_shrink_pipe(M, K, R);
    const dim3 grid((unsigned)p.blocks_m, (unsigned)p.S);
    const size_t lds = 2 * (size_t)p.nt * 16 * 32 * p.ks * 2;
    const char* x = (const char*)X;
    const int64_t ldb = ldx * DtSize<XT>::v;
    switch (p.nt) {
      case 1: k_lora_shrink_pipe<XT, 8, 1, 1><<<grid, kLoraThreads, lds, st>>>(x, ldb, (int)M, (int)K, A, R, p.S, P); break;
      case 2: k_lora_shrink_pipe<XT, 8, 1, 2><<<grid, kLoraThreads, lds, st>>>(x, ldb, (int)M, (int)K, A, R, p.S, P); break;
      case 4: k_lora_shrink_pipe<XT, 8, 1, 4><<<grid, kLoraThreads, lds, st>>>(x, ldb, (int)M, (int)K, A, R, p.S, P); break;
      default: k_lora_shrink_pipe<XT, 4, 1, 8><<<grid, kLoraThreads, lds, st>>>(x, ldb, (int)M, (int)K, A, R, p.S, P); break;
    }
    return p.S;
  }
  const ShrinkPlan p = plan_shrink(M, K, R);
  const dim3 grid((unsigned)p.blocks_m, (unsigned)p.S);
  const size_t lds = (size_t)R * 32 * p.ks * 2;
  const char* x = (const char*)X;
  const int64_t ldb = ldx * DtSize<XT>::v;
#define SQ_SHRINK(KS_, NT_)                                                                  \
  (p.rt == 2 ? k_lora_shrink<XT, KS_, 2, NT_><<<grid, kLoraThreads, lds, st>>>(x, ldb, (int)M, \
                                                   (int)K, A, R, p.S, P)                      \
             : k_lora_shrink<XT, KS_, 1, NT_><<<grid, kLoraThreads, lds, st>>>(x, ldb, (int)M, \
                                                   (int)K, A, R, p.S, P))
  switch (p.nt) {
    case 1: SQ_SHRINK(8, 1); break;
    case 2: SQ_SHRINK(8, 2); break;
    case 4: SQ_SHRINK(8, 4); break;
    default: SQ_SHRINK(4, 8); break;
  }
#undef SQ_SHRINK
  return p.S;
}

template <int XT>
static int launch_shrink_seg_p(const void* X, int64_t M, int64_t K, int64_t ldx, const LoraArgs& la,
                               int R, float* P, hipStream_t st) {
  if constexpr (XT != SQ_F32) {
    // one block per (request, 64-row tile) pair; the slices are those of the
    // single-adapter rule for as many 64-row blocks as the grid has (the
    // pairs outnumber the 64-row tiles: 8192 x 4096 in 64 requests, r 64:
    // 3 slices, whole call 68.6 -> 63.4 us, where M / 64 rows would give 4)
    const int64_t tiles_max = seg_pair_entries(M, la.nseg);
    const ShrinkPlan p = plan_shrink_pipe(tiles_max * 64, K, R);
    const dim3 grid((unsigned)tiles_max, (unsigned)p.S);
    const size_t lds = 2 * (size_t)p.nt * 16 * 32 * p.ks * 2;
    const char* x = (const char*)X;
    const int64_t ldb = ldx * DtSize<XT>::v;
    switch (p.nt) {
      case 1: k_lora_shrink_seg_pipe<XT, 8, 1><<<grid, kLoraThreads, lds, st>>>(x, ldb, (int)M, (int)K, la, R, p.S, P); break;
      case 2: k_lora_shrink_seg_pipe<XT, 8, 2><<<grid, kLoraThreads, lds, st>>>(x, ldb, (int)M, (int)K, la, R, p.S, P); break;
      case 4: k_lora_shrink_seg_pipe<XT, 8, 4><<<grid, kLoraThreads, lds, st>>>(x, ldb, (int)M, (int)K, la, R, p.S, P); break;
      default: k_lora_shrink_seg_pipe<XT, 4, 8><<<grid, kLoraThreads, lds, st>>>(x, ldb, (int)M, (int)K, la, R, p.S, P); break;
    }
    return p.S;
  }
  int S, kc;
  seg_split(M, K, &S, &kc);
  dim3 g1((unsigned)((M + 63) / 64), (unsigned)S);
  k_lora_shrink_seg<XT><<<g1, kLoraThreads, 0, st>>>((const char*)X, ldx * DtSize<XT>::v, (int)M,
                                                     (int)K, la, R, kc, P);
  return S;
}

template <int YT, bool SEG>
struct ExpandTag {};

template <int XT, int YT, bool SEG>
static int launch_lora_t(const void* X, int64_t M, int64_t K, int64_t ldx, const LoraArgs& la, int R,
                         float scale, void* Y, int64_t N, int64_t ldy, void* ws, hipStream_t st) {
  float* P = (float*)ws;
  LoraArgs lp = la;
  if constexpr (SEG) {
    // the pair table after the partial sums and T
    SegPair* tab = (SegPair*)((char*)ws + lora_ws_base(M, K, R));
    k_seg_pairs<<<1, kSegScan, 0, st>>>(la, tab, (int)seg_pair_entries(M, la.nseg));
    SQ_LAUNCH_CHECK();
    lp.pairs = tab;
  }
  const int S = SEG ? launch_shrink_seg_p<XT>(X, M, K, ldx, lp, R, P, st)
                    : launch_shrink_p<XT>(X, M, K, ldx, la.A, R, P, st);
  SQ_LAUNCH_CHECK();
  // T = bf16(sum of the S partials) once, after the partials in the workspace;
  // the expand's waves then read it instead of each summing the partials again
  // (rows padded with zeros to Rp = 32 * ceil(R / 32) ranks)
  unsigned short* Tw = (unsigned short*)((char*)ws + (size_t)S * (size_t)M * (size_t)R * sizeof(float));
  const int Rp = (R + 31) / 32 * 32;
  const int64_t rthreads = M * (Rp / 4);
  k_lora_reduce<<<(unsigned)((rthreads + 63) / 64), 64, 0, st>>>(P, S, R, Rp, (int)M, Tw, Rp);
  SQ_LAUNCH_CHECK();
  // Row tiles of 64 (with segments: at most one more per request, tiles
  // past the last (request, tile) pair are empty) times column tiles of 256;
  // a persistent grid of two blocks per CU walks them.
  const int64_t row_tiles = SEG ? seg_pair_entries(M, la.nseg) : (M + 63) / 64;
  const int64_t col_tiles = (N + 255) / 256;
  int64_t grid = row_tiles * col_tiles;
  const int64_t cap = resident_blocks<ExpandTag<YT, SEG>>((const void*)k_lora_expand<YT, SEG, 1>, kLoraThreads);
  if (grid > cap) grid = cap;
#define SQ_EXPAND(KSM_)                                                                      \
  k_lora_expand<YT, SEG, KSM_><<<(unsigned)grid, kLoraThreads, 0, st>>>(                     \
      Tw, (int)M, (int)N, lp, scale, Y, ldy, (int)row_tiles, (int)col_tiles)
  switch (Rp / 32) {
    case 1: SQ_EXPAND(1); break;
    case 2: SQ_EXPAND(2); break;
    case 3: SQ_EXPAND(3); break;
    default: SQ_EXPAND(4); break;
  }
#undef SQ_EXPAND
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

template <bool SEG>
static int launch_lora_any(const void* X, int xt, int64_t M, int64_t K, int64_t ldx,
                           const LoraArgs& la, int R, float scale, void* Y, int yt, int64_t N,
                           int64_t ldy, void* ws, hipStream_t st) {
#define SQ_LORA_Y(XT)                                                                              \
  switch (yt) {                                                                                    \
    case SQ_F32: return launch_lora_t<XT, SQ_F32, SEG>(X, M, K, ldx, la, R, scale, Y, N, ldy, ws, st); \
    case SQ_F16: return launch_lora_t<XT, SQ_F16, SEG>(X, M, K, ldx, la, R, scale, Y, N, ldy, ws, st); \
    default:     return launch_lora_t<XT, SQ_BF16, SEG>(X, M, K, ldx, la, R, scale, Y, N, ldy, ws, st); \
  }
  switch (xt) {
    case SQ_F32: SQ_LORA_Y(SQ_F32)
    case SQ_F16: SQ_LORA_Y(SQ_F16)
    default:     SQ_LORA_Y(SQ_BF16)
  }
#undef SQ_LORA_Y
}

template <int XT>
static int launch_shrink_t(const void* X, int64_t M, int64_t K, int64_t ldx, const LoraArgs& la, int R,
                           unsigned short* T, int64_t ldt, void* ws, hipStream_t st) {
  float* P = (float*)ws;
  const int S = launch_shrink_p<XT>(X, M, K, ldx, la.A, R, P, st);
  SQ_LAUNCH_CHECK();
  const int64_t threads = M * (R / 4);
  k_lora_reduce<<<(unsigned)((threads + 63) / 64), 64, 0, st>>>(P, S, R, R, (int)M, T, ldt);
  SQ_LAUNCH_CHECK();
  return SQ_OK;
}

int launch_lora_shrink(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const void* A,
                       int r, void* T, int64_t ldt, void* ws, hipStream_t st) {
  if (M == 0) return SQ_OK;
  LoraArgs la{};
  la.A = (const unsigned short*)A;
  la.r = r;
  unsigned short* t = (unsigned short*)T;
  switch (xt) {
    case SQ_F32: return launch_shrink_t<SQ_F32>(X, M, K, ldx, la, r, t, ldt, ws, st);
    case SQ_F16: return launch_shrink_t<SQ_F16>(X, M, K, ldx, la, r, t, ldt, ws, st);
    default:     return launch_shrink_t<SQ_BF16>(X, M, K, ldx, la, r, t, ldt, ws, st);
  }
}

int launch_lora(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const void* A,
                const void* B, int r, float scale, void* Y, int yt, int64_t N, int64_t ldy,
                void* ws, hipStream_t st) {
  if (M == 0) return SQ_OK;
  LoraArgs la{};
  la.A = (const unsigned short*)A;
  la.B = (const unsigned short*)B;
  la.r = r;
  return launch_lora_any<false>(X, xt, M, K, ldx, la, r, scale, Y, yt, N, ldy, ws, st);
}

int launch_lora_segmented(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, int nseg,
                          const int32_t* seg_start, const int32_t* seg_adapter,
                          const void* const* A_ptrs, const void* const* B_ptrs,
                          const int32_t* ranks, int max_rank, float scale, void* Y, int yt,
                          int64_t N, int64_t ldy, void* ws, hipStream_t st) {
  if (M == 0 || nseg == 0) return SQ_OK;
  LoraArgs la{};
  la.seg_start = seg_start;
  la.seg_adapter = seg_adapter;
  la.nseg = nseg;
  la.A_ptrs = A_ptrs;
  la.B_ptrs = B_ptrs;
  la.ranks = ranks;
  return launch_lora_any<true>(X, xt, M, K, ldx, la, max_rank, scale, Y, yt, N, ldy, ws, st);
}

}  // namespace sq
