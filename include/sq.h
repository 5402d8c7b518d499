/*
 * sq.h - C ABI of libsq, the SmoothQuant W8A8 linear-layer hot path for
 * AMD Instinct MI355X (gfx950), with a bf16 LoRA delta.
 *
 * What the calls compute (sources are cited per call):
 *   [SQ]   "SmoothQuant" explainer (ozercemkelahmet.com/tools/smoothquant),
 *          "How it works" Steps 2-7, "A short Python sketch",
 *          "Calibration in practice".
 *   [LoRA] TensorRT-LLM issue #12703, "LoRA support for W8A8 SmoothQuant
 *          (SmoothQuantAttention / SmoothQuantLinear)", section "Pitch".
 *   [GRP]  TensorRT-LLM PR #17521, "Add FP8 LoRA support for B200",
 *          "Description" (per-request adapters, eager and graph replay).
 *
 * Conventions shared by every call.
 *  - Layouts are row-major. X is [M, K] (tokens x input channels) with a row
 *    stride ldx in elements; W is [N, K] (output x input channels, the
 *    nn.Linear convention); Y is [M, N] with row stride ldy.
 *  - Every pointer except `act_max`, `s`, `a_scale`, `w_scale` and the segment
 *    tables must be 16-byte aligned; K, N and every ld must be multiples of
 *    16 elements; K <= 32768. M may be any value >= 0; M == 0 returns SQ_OK
 *    and launches nothing.
 *  - Ownership: the caller owns every buffer. The library never allocates,
 *    frees or keeps a pointer after a call returns.
 *  - Execution: each call validates its arguments on the host, then enqueues
 *    kernels on `stream` (a hipStream_t passed as void*; NULL means the null
 *    stream) and returns without synchronising. No call reads device memory
 *    on the host, so every call may be captured into a HIP graph. Faults that
 *    only the device can detect surface at the caller's next synchronisation.
 *  - Errors: argument errors are detected before any HIP call and returned as
 *    a negative sq_status; nothing is enqueued in that case. A device that is
 *    not gfx950 gives SQ_ERR_UNSUPPORTED_ARCH (with one warning on stderr per
 *    process). Results are deterministic: two runs on the same inputs give
 *    bitwise identical outputs.
 *  - NaN and Inf inputs are outside the contract. Smoothed activations x / s
 *    below the normal fp32 range (|x / s| < 2^-126) are computed exactly
 *    except when the quotient lies exactly on a rounding midpoint of the
 *    subnormal grid; there the result may be one subnormal ulp (2^-149) off
 *    the IEEE quotient. This can change codes only in a row whose largest
 *    smoothed value is itself that small.
 */
#ifndef SQ_H
#define SQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SQ_OK = 0,
  SQ_ERR_INVALID_ARG = -1,       /* null pointer, negative or zero size, bad enum, alpha out of [0,1] */
  SQ_ERR_UNSUPPORTED_DTYPE = -2, /* dtype not allowed for this argument */
  SQ_ERR_MISALIGNED = -3,        /* pointer not 16-byte aligned, or K/N/ld not a multiple of 16 */
  SQ_ERR_UNSUPPORTED_ARCH = -4,  /* current device is not gfx950 (or no device) */
  SQ_ERR_WORKSPACE = -5,         /* workspace missing or smaller than required */
  SQ_ERR_HIP = -6                /* a HIP runtime call failed (launch error) */
} sq_status;

typedef enum { SQ_F32 = 0, SQ_F16 = 1, SQ_BF16 = 2 } sq_dtype;

typedef enum {
  SQ_ACT_PER_TOKEN_DYNAMIC = 0,  /* one scale per row, computed from the row ([SQ] Step 6) */
  SQ_ACT_PER_TENSOR_STATIC = 1   /* one scale for the tensor, fixed by calibration ([SQ] Step 6) */
} sq_act_mode;

/* Largest LoRA rank the LoRA calls accept. */
#define SQ_MAX_LORA_RANK 128
/* Most projections one group call stacks adapters for (Q/K/V is three). */
#define SQ_MAX_LORA_PARTS 4

/* Capability query ([GRP]: gate on what the library was compiled for).
 * Sets *supported to 1 if `device` is a gfx950 device this library has code
 * for, else 0. Returns SQ_OK, SQ_ERR_INVALID_ARG (null pointer) or SQ_ERR_HIP
 * (device query failed; *supported is set to 0). */
int sq_query_support(int device, int* supported);

/* Static string naming a status code. Never NULL. */
const char* sq_status_string(int status);

/* [SQ] Step 4 / "Calibration in practice": running per-channel absmax.
 * act_max[k] = max(act_max[k], max_m |X[m, k]|) for m < M.
 * X: [M, K] of dtype xt (f32, f16 or bf16), row stride ldx.
 * act_max: [K] fp32, device, in/out. The caller zero-fills it before the first
 * batch; later batches keep raising it. The maximum is exact and independent
 * of the order rows are visited. */
int sq_calibrate_absmax(const void* X, int xt, int64_t M, int64_t K, int64_t ldx,
                        float* act_max, void* stream);

/* [SQ] Step 3 and the sketch's smooth_layer: smoothing scale.
 * w_max[k] = max_n |W[n, k]|; with a = max(act_max[k], 1e-5) and
 * w = max(w_max[k], 1e-5) (fp64 constants), s[k] = fp32(max(a^alpha /
 * w^(1-alpha), 1e-5)) evaluated in fp64 (square roots when alpha == 0.5).
 * W: [N, K] dtype wt, row stride ldw. alpha in [0, 1].
 * s_out: [K] fp32, device, written. */
int sq_smooth_scale(const float* act_max, const void* W, int wt, int64_t N, int64_t K,
                    int64_t ldw, double alpha, float* s_out, void* stream);

/* [SQ] Step 5 (multiply weight columns by s) and Step 6 (per-output-channel
 * INT8): W_s[n, k] = fp32(W[n, k] * s[k]); w_scale[n] = max_k |W_s[n, k]| / 127
 * (fp32); Wq[n, k] = clamp(rne(fp32(W_s[n, k] / w_scale[n])), -127, 127). A row
 * whose absmax is 0 gets w_scale 0 and codes 0. s == NULL means s = 1.
 * Wq: [N, K] int8, contiguous (row stride K). w_scale: [N] fp32. */
int sq_fold_quant_weights(const void* W, int wt, int64_t N, int64_t K, int64_t ldw,
                          const float* s, int8_t* Wq, float* w_scale, void* stream);

/* sq_smooth_scale followed by sq_fold_quant_weights on the same stream.
 * Projections that read the same input (Q/K/V, or gate/up) share one s: pass
 * their weights stacked as one [N_total, K] matrix. */
int sq_smooth_fold(const float* act_max, const void* W, int wt, int64_t N, int64_t K,
                   int64_t ldw, double alpha, float* s_out, int8_t* Wq, float* w_scale,
                   void* stream);

/* [SQ] Step 6, static variant: one per-tensor activation scale from
 * calibration maxima: a_scale[0] = max_k fp32(act_max[k] / s[k]) / 127 (fp32),
 * the per-tensor absmax of the smoothed calibration batch over 127.
 * s == NULL means s = 1. a_scale: [1] fp32, device, written. */
int sq_static_act_scale(const float* act_max, const float* s, int64_t K, float* a_scale,
                        void* stream);

/* [SQ] Step 5 (divide the layer input by s) and Step 6 (INT8 activations).
 * x_s[m, k] = fp32(X[m, k] / s[k]) (IEEE division result; s == NULL: x_s = X).
 * Dynamic: a_scale[m] = max_k |x_s[m, k]| / 127 (fp32), written ([M]).
 * Static:  a_scale[0] is read ([1]); values beyond it clip.
 * Xq[m, k] = clamp(rne(fp32(x_s[m, k] / a_scale)), -127, 127); a zero scale
 * gives codes 0. Xq: [M, K] int8, contiguous (row stride K). */
int sq_quant_per_token(const void* X, int xt, int64_t M, int64_t K, int64_t ldx,
                       const float* s, int mode, int8_t* Xq, float* a_scale, void* stream);

/* Normalization kinds for sq_norm_quant. */
typedef enum {
  SQ_NORM_RMS = 0,    /* x = h / sqrt(mean_k h^2 + eps) * g */
  SQ_NORM_LAYER = 1   /* x = (h - mean_k h) / sqrt(var_k h + eps) * g + b (biased variance) */
} sq_norm_kind;

/* [SQ] "How it works", Step 5 and the sketch's smooth_layer: the division by
 * s rides on the normalization before the projection, whose weight and bias
 * are divided by s once, offline.
 * gamma_out[k] = fp32(gamma[k] / s[k]), beta_out[k] = fp32(beta[k] / s[k])
 * (IEEE fp32 divisions; s == NULL: the values widened to fp32). gamma, beta:
 * [K] of dtype gt (beta may be NULL, then beta_out must be NULL too);
 * gamma_out, beta_out: [K] fp32, device, written. */
int sq_fold_norm_weight(const void* gamma, const void* beta, int gt, int64_t K, const float* s,
                        float* gamma_out, float* beta_out, void* stream);

/* [SQ] Steps 5-6 fused with the normalization that precedes the projection:
 * one pass over the residual stream H [M, K] (dtype ht, row stride ldh)
 * writes the INT8 codes of x_s = norm(H) with the folded weight:
 *   RMS:   x_s = fp32(fp32(h * r) * gamma)             r = fp32(1 / sqrt(ss / K + eps))
 *   LAYER: x_s = fp32(fp32(fp32(fp32(h - mu) * r) * gamma) + beta)
 *          mu = fp32(sum_k h / K), ss = sum_k fp32(h - mu)^2   (RMS: ss = sum_k h^2)
 * Row sums in fp64 (squares exact), fixed order; sqrt and 1/x in fp64.
 * gamma, beta: the folded [K] fp32 weight and bias (sq_fold_norm_weight),
 * 16-byte aligned; beta NULL means 0 and must be NULL for RMS. eps >= 0.
 * Then exactly sq_quant_per_token on x_s (no further division by s):
 * dynamic writes a_scale [M]; static reads a_scale[0]. stats: NULL or
 * [M, 2] fp32, written with (mu, r) per row (mu = 0 for RMS).
 * K <= 16384 for 16-bit H and <= 4096 for fp32 H (SQ_ERR_INVALID_ARG
 * beyond): a row lives in the registers of at most 4 waves. */
int sq_norm_quant(const void* H, int ht, int64_t M, int64_t K, int64_t ldh, int norm,
                  const float* gamma, const float* beta, float eps, int mode, int8_t* Xq,
                  float* a_scale, float* stats, void* stream);

/* [SQ] Steps 5-6 and the first half of [LoRA] Pitch from one read of X:
 * Xq and a_scale exactly as sq_quant_per_token(X, s, mode), and
 * T[m, i] = bf16(sum_k bf16(X[m, k]) * A[i, k]) (fp32 sums) as sq_lora_shrink
 * computes it (the fp32 summation order differs, so T can differ from that
 * call's in the last bf16 bit). X: bf16 with K <= 8192, or fp16 with
 * K <= 4096 (SQ_ERR_UNSUPPORTED_DTYPE / SQ_ERR_INVALID_ARG otherwise); A: [r, K] bf16,
 * 8 <= r <= SQ_MAX_LORA_RANK, r % 8 == 0; T: [M, r] bf16, row stride ldt
 * (>= r, a multiple of 8). No workspace. */
int sq_quant_shrink(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const float* s,
                    int mode, int8_t* Xq, float* a_scale, const void* A, int r, void* T,
                    int64_t ldt, void* stream);

/* [SQ] Step 6, static variant, with the clip count that "Calibration in
 * practice" and the page's closing advice ask to watch: a fixed per-tensor
 * scale lets values beyond the calibrated range clip, and the share of
 * clipped codes is the signal that the static scale no longer fits.
 * Xq exactly as sq_quant_per_token in static mode (a_scale[0] read, [1]).
 * *clipped += the number of elements whose rounded code rne(x_s / a_scale)
 * had magnitude above 127 and was clamped (a zero scale clips nothing).
 * clipped: one device uint64, 8-byte aligned, accumulated (never reset by
 * this call), so several batches or layers can share one counter; the
 * caller zeroes it. Count is exact and independent of launch order. */
int sq_quant_static_clipped(const void* X, int xt, int64_t M, int64_t K, int64_t ldx,
                            const float* s, const float* a_scale, int8_t* Xq,
                            unsigned long long* clipped, void* stream);

/* [SQ] Step 7: INT8 x INT8 -> INT32 GEMM with the dequant epilogue.
 * acc[m, n] = sum_k Xq[m, k] * Wq[n, k] (exact INT32: |acc| <= K * 127^2);
 * Y[m, n] = yt((fp32(acc) * a_scale[m]) * w_scale[n]), one RNE rounding to yt.
 * Xq: [M, K], Wq: [N, K], both int8 contiguous. a_scale: [M] (dynamic) or [1]
 * (static, mode = SQ_ACT_PER_TENSOR_STATIC). w_scale: [N]. Y: [M, N] of
 * dtype yt (bf16, f16 or f32), row stride ldy. */
int sq_w8a8_gemm(const int8_t* Xq, const int8_t* Wq, const float* a_scale, int mode,
                 const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y, int yt,
                 int64_t ldy, void* stream);

/* Bytes of device workspace sq_w8a8_gemm_ws uses for this shape: 0 where it
 * runs as sq_w8a8_gemm. Nonzero for decode-sized GEMMs (M <= 64, few
 * 32-column tiles), whose K is then split across blocks: INT32 partial sums
 * per K slice, KS x ceil(N / 32) x (1 or 2) x 4 KB. 0 for invalid shapes. */
size_t sq_w8a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* [SQ] Step 7, as sq_w8a8_gemm, with a caller's device workspace (ws, ws_bytes >=
 * sq_w8a8_gemm_workspace_bytes(M, N, K), 16-byte aligned; ignored, and may
 * be NULL, when that is 0). Same arguments, errors and results bit for bit:
 * the split partial sums are INT32, added in a fixed order before the same
 * epilogue. The workspace is overwritten; calls that share one must not
 * overlap. SQ_ERR_WORKSPACE if it is missing or too small. */
int sq_w8a8_gemm_ws(const int8_t* Xq, const int8_t* Wq, const float* a_scale, int mode,
                    const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y, int yt,
                    int64_t ldy, void* ws, size_t ws_bytes, void* stream);

/* The same GEMM with the raw INT32 accumulators as output ([M, N] contiguous),
 * for checking the integer products on their own. */
int sq_w8a8_gemm_i32(const int8_t* Xq, const int8_t* Wq, int64_t M, int64_t N, int64_t K,
                     int32_t* acc, void* stream);

/* Bytes of device workspace the LoRA calls need for M rows of K channels and
 * ranks up to max_rank (fp32 partial sums of the rank-r intermediate, and the
 * intermediate itself in bf16 for the expand, its rows zero-padded to a
 * multiple of 32 ranks), plus 16 * (ceil(M / 64) + M) bytes for the table of
 * (request, 64-row tile) pairs a segmented call writes once per call. */
size_t sq_lora_workspace_bytes(int64_t M, int64_t K, int max_rank);

/* [LoRA] Pitch, first half: the rank-r intermediate of the LoRA path,
 *   T[m, i] = bf16(sum_k bf16(X[m, k]) * A[i, k])      (fp32 accumulation)
 * X: [M, K] dtype xt, the layer's original (unsmoothed) input; A: [r, K] bf16
 * contiguous; 8 <= r <= SQ_MAX_LORA_RANK, r a multiple of 8. Several adapters
 * that read the same X can be stacked along r. T: [M, r] bf16, row stride ldt
 * (>= r, a multiple of 8), written. ws: device workspace of at least
 * sq_lora_workspace_bytes(M, K, r) bytes. */
int sq_lora_shrink(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const void* A, int r,
                   void* T, int64_t ldt, void* ws, size_t ws_bytes, void* stream);

/* [SQ] Step 7 with the [LoRA] delta fused into the GEMM epilogue:
 *   y[m, n] = yt((fp32(acc) * a_scale[m]) * w_scale[n])      (as sq_w8a8_gemm)
 *   Y[m, n] = yt(fp32(y[m, n]) + scale * sum_i T[m, i] * B[n, i])
 * i.e. the same result as sq_w8a8_gemm followed by the expand half of
 * sq_lora_apply, without a second pass over Y. T: [M, r] bf16 (row stride
 * ldt >= r, a multiple of 8), e.g. from sq_lora_shrink; B: [N, r] bf16
 * contiguous; r as for sq_lora_shrink. Other arguments as sq_w8a8_gemm. */
int sq_w8a8_gemm_lora(const int8_t* Xq, const int8_t* Wq, const float* a_scale, int mode,
                      const float* w_scale, int64_t M, int64_t N, int64_t K, const void* T,
                      int64_t ldt, const void* B, int r, float scale, void* Y, int yt,
                      int64_t ldy, void* stream);

/* [LoRA] Pitch: the low-rank path runs after the INT8 GEMM in bf16 and is
 * added to the dequantized output:
 *   T[m, i] = bf16(sum_k bf16(X[m, k]) * A[i, k])      (fp32 accumulation)
 *   Y[m, n] = yt(fp32(Y[m, n]) + scale * sum_i T[m, i] * B[n, i])
 * X is the layer's original (unsmoothed) input, dtype xt. A: [r, K] bf16
 * contiguous; B: [N, r] bf16 contiguous; 8 <= r <= SQ_MAX_LORA_RANK, r a
 * multiple of 8. Y: [M, N] dtype yt, row stride ldy, updated in place.
 * ws: device workspace of at least sq_lora_workspace_bytes(M, K, r) bytes. */
int sq_lora_apply(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const void* A,
                  const void* B, int r, float scale, void* Y, int yt, int64_t N, int64_t ldy,
                  void* ws, size_t ws_bytes, void* stream);

/* [LoRA] + [GRP]: one adapter per request. Rows [seg_start[g], seg_start[g+1])
 * of X and Y form request g (0 <= g < num_segments) and use adapter
 * seg_adapter[g]; -1 means no adapter (those rows of Y are not touched).
 * Device tables: seg_start [num_segments+1] int32, non-decreasing, from 0 to
 * M; seg_adapter [num_segments] int32; A_ptrs / B_ptrs [num_adapters] device
 * pointers to each adapter's A [r_a, K] and B [N, r_a] (bf16, contiguous,
 * 16-byte aligned); ranks [num_adapters] int32, each a multiple of 8 in
 * [8, max_rank]. The host never reads these tables; an out-of-contract table
 * is undefined behaviour. max_rank <= SQ_MAX_LORA_RANK bounds every rank and
 * sizes the workspace: sq_lora_workspace_bytes(M, K, max_rank). */
int sq_lora_apply_segmented(const void* X, int xt, int64_t M, int64_t K, int64_t ldx,
                            int num_segments, const int32_t* seg_start,
                            const int32_t* seg_adapter, int num_adapters,
                            const void* const* A_ptrs, const void* const* B_ptrs,
                            const int32_t* ranks, int max_rank, float scale, void* Y, int yt,
                            int64_t N, int64_t ldy, void* ws, size_t ws_bytes, void* stream);

/* sq_lora_apply_segmented for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without ws / ws_bytes, the same kernels and
 * the same results bit for bit. Its scratch memory is a 32 MiB device array
 * inside the library, one per device, kept until the process ends; the call
 * allocates and frees nothing. Shapes whose workspace
 * sq_lora_workspace_bytes(M, K, max_rank) exceeds 32 MiB return
 * SQ_ERR_WORKSPACE (then use sq_lora_apply_segmented). Every call on one
 * device shares that device's array and nothing in it needs clearing (each
 * call writes what it reads); calls that overlap on one device (other
 * streams, other host threads) race and must not be issued. */
int sq_lora_apply_segmented_noalloc(const void* X, int xt, int64_t M, int64_t K, int64_t ldx,
                                    int num_segments, const int32_t* seg_start,
                                    const int32_t* seg_adapter, int num_adapters,
                                    const void* const* A_ptrs, const void* const* B_ptrs,
                                    const int32_t* ranks, int max_rank, float scale, void* Y,
                                    int yt, int64_t N, int64_t ldy, void* stream);

/* The whole path for one input group ([SQ] "How it works", Steps 4-7, in
 * order; [LoRA] Pitch): the projections that read the same activations, with
 * their weights stacked along N and their adapters stacked along r, run as
 * one call, so a step costs one host call per group instead of one per
 * kernel. Every pointer and size below has the meaning and the rules it has
 * in the single-purpose call named beside it. */
#define SQ_GROUP_CALIBRATE 1  /* act_max := 0, then sq_calibrate_absmax over X_cal */
#define SQ_GROUP_FOLD 2       /* sq_smooth_fold; static mode: then sq_static_act_scale */
#define SQ_GROUP_FORWARD 4    /* sq_quant_per_token, sq_lora_shrink (r > 0), then
                                 sq_w8a8_gemm_lora (r > 0) or sq_w8a8_gemm */

typedef struct {
  const void* X;          /* [M, K] activations, dtype xt, row stride ldx */
  int xt;
  int64_t M, ldx;
  const void* X_cal;      /* [M_cal, K] calibration batch, dtype xt, stride ld_cal */
  int64_t M_cal, ld_cal;
  const void* W;          /* [N, K] stacked weights, dtype wt, row stride ldw */
  int wt;
  int64_t N, K, ldw;
  double alpha;           /* migration strength, 0 <= alpha <= 1 */
  int mode;               /* sq_act_mode */
  float* act_max;         /* [K] */
  float* s;               /* [K] smoothing vector, written by FOLD */
  int8_t* Wq;             /* [N, K], written by FOLD */
  float* w_scale;         /* [N], written by FOLD */
  int8_t* Xq;             /* [M, K], written by FORWARD */
  float* a_scale;         /* [M] (dynamic: written by FORWARD) or [1] (static: written by FOLD) */
  const void* A;          /* [r, K] bf16 stacked adapters; r == 0: no LoRA */
  const void* B;          /* [N, r] bf16 */
  int r;
  float lora_scale;
  void* T;                /* [M, r] bf16, row stride ldt */
  int64_t ldt;
  void* workspace;        /* r > 0: >= sq_lora_workspace_bytes(M, K, r) bytes. r == 0:
                             optional; with at least sq_w8a8_gemm_workspace_bytes(M, N, K)
                             bytes (16-byte aligned) the GEMM runs as sq_w8a8_gemm_ws */
  size_t workspace_bytes;
  void* Y;                /* [M, N] dtype yt, row stride ldy */
  int yt;
  int64_t ldy;
  /* Stacked adapters ([LoRA] Pitch, one adapter per projection of the group):
   * lora_parts = P in 2..SQ_MAX_LORA_PARTS splits the N output columns into
   * P projections, projection p owning columns [n_end[p-1], n_end[p]) and
   * ranks [r_end[p-1], r_end[p]) (n_end[-1] = r_end[-1] = 0), with
   * lora_n_end[P-1] == N and lora_r_end[P-1] == r, both strictly increasing;
   * column bounds multiples of 16, rank bounds multiples of 8. B must then be
   * zero outside each projection's ranks (block-diagonal), which is what
   * stacking separate adapters gives; the GEMM epilogue skips the all-zero
   * rank steps, and Y is bit for bit what the full rank range gives.
   * lora_parts 0 or 1: every column uses all r ranks (no further rule). */
  int lora_parts;
  int64_t lora_n_end[SQ_MAX_LORA_PARTS];
  int lora_r_end[SQ_MAX_LORA_PARTS];
} sq_linear_group;

/* Optional HIP events (hipEvent_t as void*, or NULL) that sq_linear_group_run
 * records on its stream between its launches, so a caller can time each stage
 * of the group without issuing the stages one by one:
 *   begin        - before the first launch of the call;
 *   quant_begin  - before the activation quant (FORWARD);
 *   shrink_begin - before the LoRA shrink (FORWARD with r > 0);
 *   gemm_begin   - before the GEMM (FORWARD);
 *   gemm_end     - after the GEMM (FORWARD).
 * FORWARD events are recorded only when M > 0. A failed record returns
 * SQ_ERR_HIP. */
typedef struct {
  void* begin;
  void* quant_begin;
  void* shrink_begin;
  void* gemm_begin;
  void* gemm_end;
} sq_group_events;

/* Runs the phases selected by `flags` (a nonzero OR of SQ_GROUP_*) for group
 * `g`, in the order calibrate, fold, forward, all on `stream`. Every phase's
 * arguments are validated before anything is enqueued; on an argument error
 * nothing runs. events: NULL, or the events to record between the launches
 * (sq_group_events). The call allocates nothing and may be captured into a
 * HIP graph. */
int sq_linear_group_run(const sq_linear_group* g, int flags, void* stream,
                        const sq_group_events* events);

/* Bytes of device workspace sq_alpha_sweep needs for an [M, K] calibration
 * batch and [N, K] weights (0 if any size is <= 0). About
 * 12*M*N + N*K + M*K + 12*K + 4*N + 4*M bytes plus 16 KB. */
size_t sq_alpha_sweep_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* [SQ] "Calibration in practice": the migration strength alpha is a per-layer
 * choice, made by how well the quantized layer reproduces its unquantized
 * output on calibration data. For every alphas[i] this runs the whole path
 * on X (which also supplies the activation maxima) with the same kernels as
 * the calls above:
 *   s = sq_smooth_scale(max_m |X|, W, alphas[i]); Wq, w_scale = fold + quant;
 *   Xq, a_scale = quant of X (mode: per-token dynamic, or per-tensor static
 *   from the same maxima); y = fp32 dequant of Xq Wq^T (yt = f32)
 * and compares y with the unquantized output y_ref = X W^T (exact
 * products, fp64 sums: within about K * 2^-53 of the exact value):
 *   err[2 i]     = sum_{m,n} (y[m, n] - y_ref[m, n])^2
 *   err[2 i + 1] = sum_{m,n} y_ref[m, n]^2
 * both summed in fp64 in a fixed order (deterministic). Then the choice:
 *   rel[i] = err[2 i] / err[2 i + 1]   (fp64; 0 when err[2 i + 1] == 0)
 *   best[0] = the i of the smallest rel[i], the first one on ties.
 * X: [M, K] dtype xt, row stride ldx; W: [N, K] dtype wt, row stride ldw
 * (N a multiple of 16). alphas: host array of n_alpha values in [0, 1]
 * (1 <= n_alpha <= 1024). err: device, [n_alpha, 2] fp64, written. rel:
 * device [n_alpha] fp64, or NULL; best: device [1] int32, or NULL.
 * ws: device workspace, 256-byte aligned, at least
 * sq_alpha_sweep_workspace_bytes(M, N, K) bytes (SQ_ERR_WORKSPACE if not).
 * M == 0 writes nothing. */
int sq_alpha_sweep(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const void* W,
                   int wt, int64_t N, int64_t ldw, const double* alphas, int n_alpha, int mode,
                   double* err, double* rel, int32_t* best, void* ws, size_t ws_bytes,
                   void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SQ_H */
