// C ABI of libsq: argument validation, the architecture gate, dispatch.
//
// Validation runs on the host before any HIP call, so an invalid call never
// enqueues work and can be tested without a GPU. The architecture gate
// follows the capability-query pattern of TensorRT-LLM PR #17521
// ("Description": gate on what the binary was compiled for, reject other
// devices, warn once instead of failing deep inside a kernel).
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "sq_internal.h"

namespace sq {
int launch_colmax(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, float* out, hipStream_t st);
int launch_fill(float* p, int64_t n, float v, hipStream_t st);
int launch_fill2(float* p1, int64_t n1, float* p2, int64_t n2, float v, hipStream_t st);
int launch_colmax2(const void* X1, int xt1, int64_t M1, int64_t K1, int64_t ld1, float* out1,
                   const void* X2, int xt2, int64_t M2, int64_t K2, int64_t ld2, float* out2,
                   hipStream_t st);
int launch_smooth_scale(const float* act_max, float* s_inout, int64_t K, double alpha, hipStream_t st);
int launch_smooth_scale_from(const float* act_max, const float* w_max, float* s, int64_t K,
                             double alpha, hipStream_t st);
int launch_ref_gemm(const void* X, int xt, int64_t ldx, const void* W, int wt, int64_t ldw,
                    int64_t M, int64_t N, int64_t K, double* Y, hipStream_t st);
int launch_sq_err(const float* q, const double* ref, int64_t n, double* part, double* out,
                  hipStream_t st);
size_t err_partials_bytes();
int launch_sweep_pick(const double* err, int n, double* rel, int32_t* best, hipStream_t st);
int64_t norm_quant_max_k(int ht);
int launch_norm_quant(const void* H, int ht, int64_t M, int64_t K, int64_t ldh, int norm,
                      const float* g, const float* b, double eps, int mode, int8_t* Xq,
                      float* a_scale, float* stats, hipStream_t st);
int launch_fold_norm(const void* w, int wt, const float* s, int64_t K, float* out, hipStream_t st);
int64_t quant_shrink_max_k(int xt);
int launch_quant_shrink(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const float* s,
                        int mode, int8_t* Xq, float* a_scale, const void* A, int r, void* T,
                        int64_t ldt, hipStream_t st);
int launch_static_scale(const float* act_max, const float* s, int64_t K, float* a_scale, hipStream_t st);
int launch_fold_quant(const void* W, int wt, int64_t N, int64_t K, int64_t ldw, const float* s,
                      int8_t* Wq, float* w_scale, hipStream_t st);
int launch_quant_act(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const float* s,
                     int mode, int8_t* Xq, float* a_scale, unsigned long long* clip, hipStream_t st);
int launch_gemm(const int8_t* Xq, const int8_t* Wq, const float* a_scale, int mode,
                const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y, int yt,
                int64_t ldy, hipStream_t st);
int launch_gemm_ws(const int8_t* Xq, const int8_t* Wq, const float* a_scale, int mode,
                   const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y, int yt,
                   int64_t ldy, void* ws, hipStream_t st);
size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K);
int launch_gemm_i32(const int8_t* Xq, const int8_t* Wq, int64_t M, int64_t N, int64_t K,
                    int32_t* acc, hipStream_t st);
int launch_gemm_lora(const int8_t* Xq, const int8_t* Wq, const float* a_scale, int mode,
                     const float* w_scale, int64_t M, int64_t N, int64_t K, const void* T,
                     int64_t ldt, const void* B, int r, float scale, void* Y, int yt, int64_t ldy,
                     hipStream_t st, int parts, const int64_t* n_end, const int* r_end);
int launch_lora_shrink(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const void* A,
                       int r, void* T, int64_t ldt, void* ws, hipStream_t st);
size_t lora_ws_bytes(int64_t M, int64_t K, int R);
int launch_lora(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const void* A,
                const void* B, int r, float scale, void* Y, int yt, int64_t N, int64_t ldy,
                void* ws, hipStream_t st);
int launch_lora_segmented(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, int nseg,
                          const int32_t* seg_start, const int32_t* seg_adapter,
                          const void* const* A_ptrs, const void* const* B_ptrs,
                          const int32_t* ranks, int max_rank, float scale, void* Y, int yt,
                          int64_t N, int64_t ldy, void* ws, hipStream_t st);
}  // namespace sq

namespace {

constexpr int64_t kMaxK = 32768;     // row kernels hold a whole row in registers
constexpr int64_t kMaxDim = (1LL << 31) - 1;
constexpr int kMaxSweepAlphas = 1024;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
bool valid_dtype(int t) { return t == SQ_F32 || t == SQ_F16 || t == SQ_BF16; }
bool valid_mode(int m) { return m == SQ_ACT_PER_TOKEN_DYNAMIC || m == SQ_ACT_PER_TENSOR_STATIC; }

#define SQ_REQUIRE(cond, err) \
  do {                        \
    if (!(cond)) return (err); \
  } while (0)

// Shape rules shared by calls that read an [rows, K] matrix with stride ld.
int check_matrix(const void* p, int dt, int64_t rows, int64_t K, int64_t ld) {
  SQ_REQUIRE(p != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(valid_dtype(dt), SQ_ERR_UNSUPPORTED_DTYPE);
  SQ_REQUIRE(rows >= 0 && rows <= kMaxDim, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(K >= 1 && K <= kMaxK, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(ld >= K, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(K % 16 == 0 && ld % 16 == 0 && aligned16(p), SQ_ERR_MISALIGNED);
  return SQ_OK;
}

// Architecture gate: the library carries gfx950 code only.
std::atomic<int> g_arch_cache[64];   // 0 unknown, 1 supported, 2 unsupported
std::atomic<bool> g_warned{false};

int arch_of_device(int device, int* supported) {
  *supported = 0;
  const char* forced = std::getenv("SQ_FORCE_ARCH");
  if (forced != nullptr && forced[0] != '\0') {
    *supported = std::strncmp(forced, "gfx950", 6) == 0;
    return SQ_OK;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return SQ_ERR_HIP;
  *supported = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  return SQ_OK;
}

int gate() {
  int dev = 0;
  int supported = 0;
  bool known = false;
  const char* forced = std::getenv("SQ_FORCE_ARCH");
  if (forced != nullptr && forced[0] != '\0') {
    arch_of_device(0, &supported);
    known = true;
  } else if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    int c = g_arch_cache[dev].load(std::memory_order_relaxed);
    if (c == 0) {
      if (arch_of_device(dev, &supported) == SQ_OK) {
        g_arch_cache[dev].store(supported ? 1 : 2, std::memory_order_relaxed);
        known = true;
      }
    } else {
      supported = c == 1;
      known = true;
    }
  } else {
    (void)hipGetLastError();   // clear the sticky error of a failed device query
  }
  if (known && supported) return SQ_OK;
  if (!g_warned.exchange(true)) {
    std::fprintf(stderr,
                 "libsq: the current device is not gfx950 (or no HIP device is present); "
                 "SmoothQuant kernels are unavailable and calls return SQ_ERR_UNSUPPORTED_ARCH\n");
  }
  return SQ_ERR_UNSUPPORTED_ARCH;
}

hipStream_t as_stream(void* s) { return (hipStream_t)s; }

}  // namespace

extern "C" {

const char* sq_status_string(int st) {
  switch (st) {
    case SQ_OK: return "SQ_OK";
    case SQ_ERR_INVALID_ARG: return "SQ_ERR_INVALID_ARG: null pointer, bad size or bad argument";
    case SQ_ERR_UNSUPPORTED_DTYPE: return "SQ_ERR_UNSUPPORTED_DTYPE: dtype not allowed here";
    case SQ_ERR_MISALIGNED: return "SQ_ERR_MISALIGNED: pointer not 16-byte aligned or K/N/ld not a multiple of 16";
    case SQ_ERR_UNSUPPORTED_ARCH: return "SQ_ERR_UNSUPPORTED_ARCH: current device is not gfx950";
    case SQ_ERR_WORKSPACE: return "SQ_ERR_WORKSPACE: workspace missing or too small";
    case SQ_ERR_HIP: return "SQ_ERR_HIP: a HIP runtime call failed";
    default: return "unknown sq_status";
  }
}

int sq_query_support(int device, int* supported) {
  SQ_REQUIRE(supported != nullptr, SQ_ERR_INVALID_ARG);
  *supported = 0;
  SQ_REQUIRE(device >= 0, SQ_ERR_INVALID_ARG);
  const int rc = arch_of_device(device, supported);
  if (rc != SQ_OK) (void)hipGetLastError();
  return rc;
}

int sq_calibrate_absmax(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, float* act_max,
                        void* stream) {
  int rc = check_matrix(X, xt, M, K, ldx);
  if (rc != SQ_OK) return rc;
  SQ_REQUIRE(act_max != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(aligned4(act_max), SQ_ERR_MISALIGNED);
  if (M == 0) return SQ_OK;
  if ((rc = gate()) != SQ_OK) return rc;
  return sq::launch_colmax(X, xt, M, K, ldx, act_max, as_stream(stream));
}

int sq_smooth_scale(const float* act_max, const void* W, int wt, int64_t N, int64_t K, int64_t ldw,
                    double alpha, float* s_out, void* stream) {
  int rc = check_matrix(W, wt, N, K, ldw);
  if (rc != SQ_OK) return rc;
  SQ_REQUIRE(N >= 1, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(act_max != nullptr && s_out != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(aligned4(act_max) && aligned4(s_out), SQ_ERR_MISALIGNED);
  SQ_REQUIRE(std::isfinite(alpha) && alpha >= 0.0 && alpha <= 1.0, SQ_ERR_INVALID_ARG);
  if ((rc = gate()) != SQ_OK) return rc;
  hipStream_t st = as_stream(stream);
  // w_max accumulates in s_out, which the scale kernel then turns into s.
  if ((rc = sq::launch_fill(s_out, K, 0.0f, st)) != SQ_OK) return rc;
  if ((rc = sq::launch_colmax(W, wt, N, K, ldw, s_out, st)) != SQ_OK) return rc;
  return sq::launch_smooth_scale(act_max, s_out, K, alpha, st);
}

int sq_fold_quant_weights(const void* W, int wt, int64_t N, int64_t K, int64_t ldw, const float* s,
                          int8_t* Wq, float* w_scale, void* stream) {
  int rc = check_matrix(W, wt, N, K, ldw);
  if (rc != SQ_OK) return rc;
  SQ_REQUIRE(N >= 1, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(Wq != nullptr && w_scale != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(aligned16(Wq) && aligned4(w_scale) && (s == nullptr || aligned4(s)), SQ_ERR_MISALIGNED);
  if ((rc = gate()) != SQ_OK) return rc;
  return sq::launch_fold_quant(W, wt, N, K, ldw, s, Wq, w_scale, as_stream(stream));
}

int sq_smooth_fold(const float* act_max, const void* W, int wt, int64_t N, int64_t K, int64_t ldw,
                   double alpha, float* s_out, int8_t* Wq, float* w_scale, void* stream) {
  int rc = check_matrix(W, wt, N, K, ldw);
  if (rc != SQ_OK) return rc;
  SQ_REQUIRE(Wq != nullptr && w_scale != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(aligned16(Wq) && aligned4(w_scale), SQ_ERR_MISALIGNED);
  if ((rc = sq_smooth_scale(act_max, W, wt, N, K, ldw, alpha, s_out, stream)) != SQ_OK) return rc;
  return sq::launch_fold_quant(W, wt, N, K, ldw, s_out, Wq, w_scale, as_stream(stream));
}

int sq_static_act_scale(const float* act_max, const float* s, int64_t K, float* a_scale, void* stream) {
  SQ_REQUIRE(act_max != nullptr && a_scale != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(K >= 1 && K <= kMaxDim, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(aligned4(act_max) && aligned4(a_scale) && (s == nullptr || aligned4(s)), SQ_ERR_MISALIGNED);
  int rc = gate();
  if (rc != SQ_OK) return rc;
  return sq::launch_static_scale(act_max, s, K, a_scale, as_stream(stream));
}

int sq_quant_per_token(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const float* s,
                       int mode, int8_t* Xq, float* a_scale, void* stream) {
  int rc = check_matrix(X, xt, M, K, ldx);
  if (rc != SQ_OK) return rc;
  SQ_REQUIRE(valid_mode(mode), SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(Xq != nullptr && a_scale != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(aligned16(Xq) && aligned4(a_scale) && (s == nullptr || aligned4(s)), SQ_ERR_MISALIGNED);
  if (M == 0) return SQ_OK;
  if ((rc = gate()) != SQ_OK) return rc;
  return sq::launch_quant_act(X, xt, M, K, ldx, s, mode, Xq, a_scale, nullptr, as_stream(stream));
}

int sq_fold_norm_weight(const void* gamma, const void* beta, int gt, int64_t K, const float* s,
                        float* gamma_out, float* beta_out, void* stream) {
  SQ_REQUIRE(gamma != nullptr && gamma_out != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE((beta == nullptr) == (beta_out == nullptr), SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(valid_dtype(gt), SQ_ERR_UNSUPPORTED_DTYPE);
  SQ_REQUIRE(K >= 1 && K <= kMaxK, SQ_ERR_INVALID_ARG);
  const int esz = gt == SQ_F32 ? 4 : 2;
  SQ_REQUIRE(((uintptr_t)gamma % esz) == 0 && (beta == nullptr || ((uintptr_t)beta % esz) == 0) &&
                 aligned4(gamma_out) && (beta_out == nullptr || aligned4(beta_out)) &&
                 (s == nullptr || aligned4(s)),
             SQ_ERR_MISALIGNED);
  int rc = gate();
  if (rc != SQ_OK) return rc;
  hipStream_t st = as_stream(stream);
  if ((rc = sq::launch_fold_norm(gamma, gt, s, K, gamma_out, st)) != SQ_OK) return rc;
  if (beta != nullptr) rc = sq::launch_fold_norm(beta, gt, s, K, beta_out, st);
  return rc;
}

int sq_norm_quant(const void* H, int ht, int64_t M, int64_t K, int64_t ldh, int norm,
                  const float* gamma, const float* beta, float eps, int mode, int8_t* Xq,
                  float* a_scale, float* stats, void* stream) {
  int rc = check_matrix(H, ht, M, K, ldh);
  if (rc != SQ_OK) return rc;
  SQ_REQUIRE(norm == SQ_NORM_RMS || norm == SQ_NORM_LAYER, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(norm == SQ_NORM_LAYER || beta == nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(K <= sq::norm_quant_max_k(ht), SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(valid_mode(mode), SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(std::isfinite(eps) && eps >= 0.0f, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(gamma != nullptr && Xq != nullptr && a_scale != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(aligned16(gamma) && (beta == nullptr || aligned16(beta)) && aligned16(Xq) &&
                 aligned4(a_scale) && (stats == nullptr || aligned4(stats)),
             SQ_ERR_MISALIGNED);
  if (M == 0) return SQ_OK;
  if ((rc = gate()) != SQ_OK) return rc;
  return sq::launch_norm_quant(H, ht, M, K, ldh, norm, gamma, beta, (double)eps, mode, Xq, a_scale,
                               stats, as_stream(stream));
}

static int check_rank(int r);

int sq_quant_shrink(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const float* s,
                    int mode, int8_t* Xq, float* a_scale, const void* A, int r, void* T,
                    int64_t ldt, void* stream) {
  int rc = check_matrix(X, xt, M, K, ldx);
  if (rc != SQ_OK) return rc;
  SQ_REQUIRE(xt == SQ_BF16 || xt == SQ_F16, SQ_ERR_UNSUPPORTED_DTYPE);
  SQ_REQUIRE(K <= sq::quant_shrink_max_k(xt), SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(valid_mode(mode), SQ_ERR_INVALID_ARG);
  if ((rc = check_rank(r)) != SQ_OK) return rc;
  SQ_REQUIRE(Xq != nullptr && a_scale != nullptr && A != nullptr && T != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(ldt >= r, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(ldt % 8 == 0 && aligned16(Xq) && aligned16(A) && aligned16(T) && aligned4(a_scale) &&
                 (s == nullptr || aligned4(s)),
             SQ_ERR_MISALIGNED);
  if (M == 0) return SQ_OK;
  if ((rc = gate()) != SQ_OK) return rc;
  return sq::launch_quant_shrink(X, xt, M, K, ldx, s, mode, Xq, a_scale, A, r, T, ldt,
                                 as_stream(stream));
}

int sq_quant_static_clipped(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const float* s,
                            const float* a_scale, int8_t* Xq, unsigned long long* clipped,
                            void* stream) {
  int rc = check_matrix(X, xt, M, K, ldx);
  if (rc != SQ_OK) return rc;
  SQ_REQUIRE(Xq != nullptr && a_scale != nullptr && clipped != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(aligned16(Xq) && aligned4(a_scale) && (s == nullptr || aligned4(s)) &&
                 ((uintptr_t)clipped & 7u) == 0,
             SQ_ERR_MISALIGNED);
  if (M == 0) return SQ_OK;
  if ((rc = gate()) != SQ_OK) return rc;
  // static mode only reads the scale
  return sq::launch_quant_act(X, xt, M, K, ldx, s, SQ_ACT_PER_TENSOR_STATIC, Xq,
                              const_cast<float*>(a_scale), clipped, as_stream(stream));
}

static int check_gemm(const int8_t* Xq, const int8_t* Wq, int64_t M, int64_t N, int64_t K) {
  SQ_REQUIRE(Xq != nullptr && Wq != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(M >= 0 && M <= kMaxDim && N >= 1 && N <= kMaxDim, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(K >= 1 && K <= kMaxK, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(K % 16 == 0 && N % 16 == 0 && aligned16(Xq) && aligned16(Wq), SQ_ERR_MISALIGNED);
  return SQ_OK;
}

int sq_w8a8_gemm(const int8_t* Xq, const int8_t* Wq, const float* a_scale, int mode,
                 const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y, int yt, int64_t ldy,
                 void* stream) {
  int rc = check_gemm(Xq, Wq, M, N, K);
  if (rc != SQ_OK) return rc;
  SQ_REQUIRE(valid_mode(mode), SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(a_scale != nullptr && w_scale != nullptr && Y != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(valid_dtype(yt), SQ_ERR_UNSUPPORTED_DTYPE);
  SQ_REQUIRE(ldy >= N, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(ldy % 16 == 0 && aligned16(Y) && aligned4(a_scale) && aligned4(w_scale), SQ_ERR_MISALIGNED);
  if (M == 0) return SQ_OK;
  if ((rc = gate()) != SQ_OK) return rc;
  return sq::launch_gemm(Xq, Wq, a_scale, mode, w_scale, M, N, K, Y, yt, ldy, as_stream(stream));
}

size_t sq_w8a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxK) return 0;
  return sq::gemm_ws_bytes(M, N, K);
}

int sq_w8a8_gemm_ws(const int8_t* Xq, const int8_t* Wq, const float* a_scale, int mode,
                    const float* w_scale, int64_t M, int64_t N, int64_t K, void* Y, int yt,
                    int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_gemm(Xq, Wq, M, N, K);
  if (rc != SQ_OK) return rc;
  SQ_REQUIRE(valid_mode(mode), SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(a_scale != nullptr && w_scale != nullptr && Y != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(valid_dtype(yt), SQ_ERR_UNSUPPORTED_DTYPE);
  SQ_REQUIRE(ldy >= N, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(ldy % 16 == 0 && aligned16(Y) && aligned4(a_scale) && aligned4(w_scale), SQ_ERR_MISALIGNED);
  if (M == 0) return SQ_OK;
  const size_t need = sq::gemm_ws_bytes(M, N, K);
  if (need > 0) {
    SQ_REQUIRE(ws != nullptr && ws_bytes >= need, SQ_ERR_WORKSPACE);
    SQ_REQUIRE(aligned16(ws), SQ_ERR_MISALIGNED);
  }
  if ((rc = gate()) != SQ_OK) return rc;
  return sq::launch_gemm_ws(Xq, Wq, a_scale, mode, w_scale, M, N, K, Y, yt, ldy,
                            need > 0 ? ws : nullptr, as_stream(stream));
}

static int check_rank(int r) {
  SQ_REQUIRE(r >= 1 && r <= SQ_MAX_LORA_RANK, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(r % 8 == 0, SQ_ERR_MISALIGNED);
  return SQ_OK;
}

int sq_w8a8_gemm_lora(const int8_t* Xq, const int8_t* Wq, const float* a_scale, int mode,
                      const float* w_scale, int64_t M, int64_t N, int64_t K, const void* T,
                      int64_t ldt, const void* B, int r, float scale, void* Y, int yt, int64_t ldy,
                      void* stream) {
  int rc = check_gemm(Xq, Wq, M, N, K);
  if (rc != SQ_OK) return rc;
  SQ_REQUIRE(valid_mode(mode), SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(a_scale != nullptr && w_scale != nullptr && Y != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(T != nullptr && B != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(valid_dtype(yt), SQ_ERR_UNSUPPORTED_DTYPE);
  SQ_REQUIRE(ldy >= N, SQ_ERR_INVALID_ARG);
  if ((rc = check_rank(r)) != SQ_OK) return rc;
  SQ_REQUIRE(std::isfinite(scale), SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(ldt >= r, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(ldt % 8 == 0 && aligned16(T) && aligned16(B), SQ_ERR_MISALIGNED);
  SQ_REQUIRE(ldy % 16 == 0 && aligned16(Y) && aligned4(a_scale) && aligned4(w_scale), SQ_ERR_MISALIGNED);
  if (M == 0) return SQ_OK;
  if ((rc = gate()) != SQ_OK) return rc;
  return sq::launch_gemm_lora(Xq, Wq, a_scale, mode, w_scale, M, N, K, T, ldt, B, r, scale, Y, yt,
                              ldy, as_stream(stream), 0, nullptr, nullptr);
}

int sq_w8a8_gemm_i32(const int8_t* Xq, const int8_t* Wq, int64_t M, int64_t N, int64_t K,
                     int32_t* acc, void* stream) {
  int rc = check_gemm(Xq, Wq, M, N, K);
  if (rc != SQ_OK) return rc;
  SQ_REQUIRE(acc != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(aligned16(acc), SQ_ERR_MISALIGNED);
  if (M == 0) return SQ_OK;
  if ((rc = gate()) != SQ_OK) return rc;
  return sq::launch_gemm_i32(Xq, Wq, M, N, K, acc, as_stream(stream));
}

size_t sq_lora_workspace_bytes(int64_t M, int64_t K, int max_rank) {
  if (M <= 0 || K <= 0 || max_rank <= 0) return 0;
  return sq::lora_ws_bytes(M, K, max_rank);
}

static int check_lora_common(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, void* Y,
                             int yt, int64_t N, int64_t ldy, int rank, float scale) {
  int rc = check_matrix(X, xt, M, K, ldx);
  if (rc != SQ_OK) return rc;
  SQ_REQUIRE(Y != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(valid_dtype(yt), SQ_ERR_UNSUPPORTED_DTYPE);
  SQ_REQUIRE(N >= 1 && N <= kMaxDim && ldy >= N, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(N % 16 == 0 && ldy % 16 == 0 && aligned16(Y), SQ_ERR_MISALIGNED);
  SQ_REQUIRE(rank >= 1 && rank <= SQ_MAX_LORA_RANK, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(rank % 8 == 0, SQ_ERR_MISALIGNED);
  SQ_REQUIRE(std::isfinite(scale), SQ_ERR_INVALID_ARG);
  return SQ_OK;
}

int sq_lora_shrink(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const void* A, int r,
                   void* T, int64_t ldt, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_matrix(X, xt, M, K, ldx);
  if (rc != SQ_OK) return rc;
  if ((rc = check_rank(r)) != SQ_OK) return rc;
  SQ_REQUIRE(A != nullptr && T != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(ldt >= r, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(ldt % 8 == 0 && aligned16(A) && aligned16(T), SQ_ERR_MISALIGNED);
  if (M == 0) return SQ_OK;
  const size_t need = sq_lora_workspace_bytes(M, K, r);
  SQ_REQUIRE(ws != nullptr && ws_bytes >= need, SQ_ERR_WORKSPACE);
  SQ_REQUIRE(aligned16(ws), SQ_ERR_MISALIGNED);
  if ((rc = gate()) != SQ_OK) return rc;
  return sq::launch_lora_shrink(X, xt, M, K, ldx, A, r, T, ldt, ws, as_stream(stream));
}

int sq_lora_apply(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const void* A,
                  const void* B, int r, float scale, void* Y, int yt, int64_t N, int64_t ldy,
                  void* ws, size_t ws_bytes, void* stream) {
  int rc = check_lora_common(X, xt, M, K, ldx, Y, yt, N, ldy, r, scale);
  if (rc != SQ_OK) return rc;
  SQ_REQUIRE(A != nullptr && B != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(aligned16(A) && aligned16(B), SQ_ERR_MISALIGNED);
  if (M == 0) return SQ_OK;
  const size_t need = sq_lora_workspace_bytes(M, K, r);
  SQ_REQUIRE(ws != nullptr && ws_bytes >= need, SQ_ERR_WORKSPACE);
  SQ_REQUIRE(aligned16(ws), SQ_ERR_MISALIGNED);
  if ((rc = gate()) != SQ_OK) return rc;
  return sq::launch_lora(X, xt, M, K, ldx, A, B, r, scale, Y, yt, N, ldy, ws, as_stream(stream));
}

// Arguments of the segmented LoRA call other than the workspace.
static int check_segmented(const void* X, int xt, int64_t M, int64_t K, int64_t ldx,
                           int num_segments, const int32_t* seg_start, const int32_t* seg_adapter,
                           int num_adapters, const void* const* A_ptrs, const void* const* B_ptrs,
                           const int32_t* ranks, int max_rank, float scale, void* Y, int yt,
                           int64_t N, int64_t ldy) {
  int rc = check_lora_common(X, xt, M, K, ldx, Y, yt, N, ldy, max_rank, scale);
  if (rc != SQ_OK) return rc;
  SQ_REQUIRE(num_segments >= 0 && num_adapters >= 1, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(seg_start != nullptr && seg_adapter != nullptr && A_ptrs != nullptr &&
                 B_ptrs != nullptr && ranks != nullptr,
             SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(aligned4(seg_start) && aligned4(seg_adapter) && aligned4(ranks) &&
                 ((uintptr_t)A_ptrs & 7u) == 0 && ((uintptr_t)B_ptrs & 7u) == 0,
             SQ_ERR_MISALIGNED);
  return SQ_OK;
}

int sq_lora_apply_segmented(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, int num_segments,
                            const int32_t* seg_start, const int32_t* seg_adapter, int num_adapters,
                            const void* const* A_ptrs, const void* const* B_ptrs,
                            const int32_t* ranks, int max_rank, float scale, void* Y, int yt,
                            int64_t N, int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_segmented(X, xt, M, K, ldx, num_segments, seg_start, seg_adapter, num_adapters,
                           A_ptrs, B_ptrs, ranks, max_rank, scale, Y, yt, N, ldy);
  if (rc != SQ_OK) return rc;
  if (M == 0 || num_segments == 0) return SQ_OK;
  const size_t need = sq_lora_workspace_bytes(M, K, max_rank);
  SQ_REQUIRE(ws != nullptr && ws_bytes >= need, SQ_ERR_WORKSPACE);
  SQ_REQUIRE(aligned16(ws), SQ_ERR_MISALIGNED);
  if ((rc = gate()) != SQ_OK) return rc;
  return sq::launch_lora_segmented(X, xt, M, K, ldx, num_segments, seg_start, seg_adapter, A_ptrs,
                                   B_ptrs, ranks, max_rank, scale, Y, yt, N, ldy, ws,
                                   as_stream(stream));
}

// Projection table of a group's stacked adapters (sq_linear_group.lora_parts).
static int check_lora_parts(const sq_linear_group* g) {
  if (g->lora_parts <= 1) {
    SQ_REQUIRE(g->lora_parts >= 0, SQ_ERR_INVALID_ARG);
    return SQ_OK;
  }
  SQ_REQUIRE(g->lora_parts <= SQ_MAX_LORA_PARTS, SQ_ERR_INVALID_ARG);
  int64_t n_prev = 0;
  int r_prev = 0;
  for (int p = 0; p < g->lora_parts; ++p) {
    SQ_REQUIRE(g->lora_n_end[p] > n_prev && g->lora_r_end[p] > r_prev, SQ_ERR_INVALID_ARG);
    SQ_REQUIRE(g->lora_n_end[p] % 16 == 0 && g->lora_r_end[p] % 8 == 0, SQ_ERR_MISALIGNED);
    n_prev = g->lora_n_end[p];
    r_prev = g->lora_r_end[p];
  }
  SQ_REQUIRE(n_prev == g->N && r_prev == g->r, SQ_ERR_INVALID_ARG);
  return SQ_OK;
}

static int record(void* ev, hipStream_t st) {
  if (ev != nullptr && hipEventRecord((hipEvent_t)ev, st) != hipSuccess) return SQ_ERR_HIP;
  return SQ_OK;
}

// ---------------------------------------------------------------------------
// The segmented LoRA call without a caller workspace, for callers that cannot
// allocate. Its scratch memory is this file-scope device array, one copy per
// device, held until the process ends. In host code the name `scratch` stands
// for a host-side shadow, not a device address, so host code never passes it
// to a kernel or a copy: it uses the address hipGetSymbolAddress returns for
// the current device, looked up once per device and kept in g_scratch_ptr.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

static int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return SQ_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return SQ_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SQ_OK;
}

int sq_lora_apply_segmented_noalloc(const void* X, int xt, int64_t M, int64_t K, int64_t ldx,
                                    int num_segments, const int32_t* seg_start,
                                    const int32_t* seg_adapter, int num_adapters,
                                    const void* const* A_ptrs, const void* const* B_ptrs,
                                    const int32_t* ranks, int max_rank, float scale, void* Y,
                                    int yt, int64_t N, int64_t ldy, void* stream) {
  int rc = check_segmented(X, xt, M, K, ldx, num_segments, seg_start, seg_adapter, num_adapters,
                           A_ptrs, B_ptrs, ranks, max_rank, scale, Y, yt, N, ldy);
  if (rc != SQ_OK) return rc;
  if (M == 0 || num_segments == 0) return SQ_OK;
  SQ_REQUIRE(sq_lora_workspace_bytes(M, K, max_rank) <= kNoAllocScratchBytes, SQ_ERR_WORKSPACE);
  if ((rc = gate()) != SQ_OK) return rc;
  void* ws = nullptr;
  if ((rc = scratch_ptr(&ws)) != SQ_OK) return rc;
  return sq::launch_lora_segmented(X, xt, M, K, ldx, num_segments, seg_start, seg_adapter, A_ptrs,
                                   B_ptrs, ranks, max_rank, scale, Y, yt, N, ldy, ws,
                                   as_stream(stream));
}

int sq_linear_group_run(const sq_linear_group* g, int flags, void* stream,
                        const sq_group_events* events) {
  SQ_REQUIRE(g != nullptr, SQ_ERR_INVALID_ARG);
  constexpr int kAll = SQ_GROUP_CALIBRATE | SQ_GROUP_FOLD | SQ_GROUP_FORWARD;
  SQ_REQUIRE(flags != 0 && (flags & ~kAll) == 0, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(valid_mode(g->mode), SQ_ERR_INVALID_ARG);
  const bool lora = g->r != 0;
  const bool is_static = g->mode == SQ_ACT_PER_TENSOR_STATIC;
  int rc;
  // 1. validate every selected phase
  if (flags & SQ_GROUP_CALIBRATE) {
    if ((rc = check_matrix(g->X_cal, g->xt, g->M_cal, g->K, g->ld_cal)) != SQ_OK) return rc;
    SQ_REQUIRE(g->act_max != nullptr, SQ_ERR_INVALID_ARG);
    SQ_REQUIRE(aligned4(g->act_max), SQ_ERR_MISALIGNED);
  }
  if (flags & SQ_GROUP_FOLD) {
    if ((rc = check_matrix(g->W, g->wt, g->N, g->K, g->ldw)) != SQ_OK) return rc;
    SQ_REQUIRE(g->N >= 1, SQ_ERR_INVALID_ARG);
    SQ_REQUIRE(g->act_max != nullptr && g->s != nullptr && g->Wq != nullptr && g->w_scale != nullptr,
               SQ_ERR_INVALID_ARG);
    SQ_REQUIRE(aligned4(g->act_max) && aligned4(g->s) && aligned16(g->Wq) && aligned4(g->w_scale),
               SQ_ERR_MISALIGNED);
    SQ_REQUIRE(std::isfinite(g->alpha) && g->alpha >= 0.0 && g->alpha <= 1.0, SQ_ERR_INVALID_ARG);
    if (is_static) {
      SQ_REQUIRE(g->a_scale != nullptr, SQ_ERR_INVALID_ARG);
      SQ_REQUIRE(aligned4(g->a_scale), SQ_ERR_MISALIGNED);
    }
  }
  if (flags & SQ_GROUP_FORWARD) {
    if ((rc = check_matrix(g->X, g->xt, g->M, g->K, g->ldx)) != SQ_OK) return rc;
    SQ_REQUIRE(g->s != nullptr && g->Xq != nullptr && g->a_scale != nullptr, SQ_ERR_INVALID_ARG);
    SQ_REQUIRE(aligned4(g->s) && aligned16(g->Xq) && aligned4(g->a_scale), SQ_ERR_MISALIGNED);
    if ((rc = check_gemm(g->Xq, g->Wq, g->M, g->N, g->K)) != SQ_OK) return rc;
    SQ_REQUIRE(g->w_scale != nullptr && g->Y != nullptr, SQ_ERR_INVALID_ARG);
    SQ_REQUIRE(valid_dtype(g->yt), SQ_ERR_UNSUPPORTED_DTYPE);
    SQ_REQUIRE(g->ldy >= g->N, SQ_ERR_INVALID_ARG);
    SQ_REQUIRE(g->ldy % 16 == 0 && aligned16(g->Y) && aligned4(g->w_scale), SQ_ERR_MISALIGNED);
    if (lora) {
      if ((rc = check_rank(g->r)) != SQ_OK) return rc;
      SQ_REQUIRE(g->A != nullptr && g->B != nullptr && g->T != nullptr, SQ_ERR_INVALID_ARG);
      SQ_REQUIRE(std::isfinite(g->lora_scale), SQ_ERR_INVALID_ARG);
      SQ_REQUIRE(g->ldt >= g->r, SQ_ERR_INVALID_ARG);
      SQ_REQUIRE(g->ldt % 8 == 0 && aligned16(g->A) && aligned16(g->B) && aligned16(g->T),
                 SQ_ERR_MISALIGNED);
      if ((rc = check_lora_parts(g)) != SQ_OK) return rc;
      if (g->M > 0) {
        SQ_REQUIRE(g->workspace != nullptr &&
                       g->workspace_bytes >= sq_lora_workspace_bytes(g->M, g->K, g->r),
                   SQ_ERR_WORKSPACE);
        SQ_REQUIRE(aligned16(g->workspace), SQ_ERR_MISALIGNED);
      }
    }
  }
  if ((rc = gate()) != SQ_OK) return rc;
  hipStream_t st = as_stream(stream);
  const sq_group_events ev = events != nullptr ? *events : sq_group_events{};
  // 2. launch
  if ((rc = record(ev.begin, st)) != SQ_OK) return rc;
  const bool cal = flags & SQ_GROUP_CALIBRATE, fold = flags & SQ_GROUP_FOLD;
  if (cal && fold) {
    // both column maxima (act_max over X_cal, w_max over W, accumulated in s)
    // from one zero-fill and one two-job column-max launch
    if ((rc = sq::launch_fill2(g->act_max, g->K, g->s, g->K, 0.0f, st)) != SQ_OK) return rc;
    if ((rc = sq::launch_colmax2(g->X_cal, g->xt, g->M_cal, g->K, g->ld_cal, g->act_max, g->W,
                                 g->wt, g->N, g->K, g->ldw, g->s, st)) != SQ_OK)
      return rc;
  } else if (cal) {
    if ((rc = sq::launch_fill(g->act_max, g->K, 0.0f, st)) != SQ_OK) return rc;
    if ((rc = sq::launch_colmax(g->X_cal, g->xt, g->M_cal, g->K, g->ld_cal, g->act_max, st)) != SQ_OK)
      return rc;
  } else if (fold) {
    if ((rc = sq::launch_fill(g->s, g->K, 0.0f, st)) != SQ_OK) return rc;
    if ((rc = sq::launch_colmax(g->W, g->wt, g->N, g->K, g->ldw, g->s, st)) != SQ_OK) return rc;
  }
  if (fold) {
    if ((rc = sq::launch_smooth_scale(g->act_max, g->s, g->K, g->alpha, st)) != SQ_OK) return rc;
    if ((rc = sq::launch_fold_quant(g->W, g->wt, g->N, g->K, g->ldw, g->s, g->Wq, g->w_scale, st)) !=
        SQ_OK)
      return rc;
    if (is_static && (rc = sq::launch_static_scale(g->act_max, g->s, g->K, g->a_scale, st)) != SQ_OK)
      return rc;
  }
  if ((flags & SQ_GROUP_FORWARD) && g->M > 0) {
    // The quant and the shrink as two kernels: at the workload's shapes they
    // are faster alone than the one-read sq_quant_shrink (and equal inside the
    // overlapped step), which needs a 16-row block per CU and reads all of A
    // per block.
    if ((rc = record(ev.quant_begin, st)) != SQ_OK) return rc;
    if ((rc = sq::launch_quant_act(g->X, g->xt, g->M, g->K, g->ldx, g->s, g->mode, g->Xq, g->a_scale,
                                   nullptr, st)) != SQ_OK)
      return rc;
    if (lora) {
      if ((rc = record(ev.shrink_begin, st)) != SQ_OK) return rc;
      if ((rc = sq::launch_lora_shrink(g->X, g->xt, g->M, g->K, g->ldx, g->A, g->r, g->T, g->ldt,
                                       g->workspace, st)) != SQ_OK)
        return rc;
    }
    if ((rc = record(ev.gemm_begin, st)) != SQ_OK) return rc;
    // Without LoRA, a workspace large enough for the split-K GEMM of decode
    // shapes lets the GEMM use it (sq_w8a8_gemm_ws); the result is the same.
    const size_t gws = lora ? 0 : sq::gemm_ws_bytes(g->M, g->N, g->K);
    const bool split = gws > 0 && g->workspace != nullptr && g->workspace_bytes >= gws &&
                       aligned16(g->workspace);
    if (lora)
      rc = sq::launch_gemm_lora(g->Xq, g->Wq, g->a_scale, g->mode, g->w_scale, g->M, g->N, g->K, g->T,
                                g->ldt, g->B, g->r, g->lora_scale, g->Y, g->yt, g->ldy, st,
                                g->lora_parts, g->lora_n_end, g->lora_r_end);
    else if (split)
      rc = sq::launch_gemm_ws(g->Xq, g->Wq, g->a_scale, g->mode, g->w_scale, g->M, g->N, g->K, g->Y,
                              g->yt, g->ldy, g->workspace, st);
    else
      rc = sq::launch_gemm(g->Xq, g->Wq, g->a_scale, g->mode, g->w_scale, g->M, g->N, g->K, g->Y,
                           g->yt, g->ldy, st);
    if (rc != SQ_OK) return rc;
    if ((rc = record(ev.gemm_end, st)) != SQ_OK) return rc;
  }
  return SQ_OK;
}

// ---------------------------------------------------------------------------
// Per-layer alpha sweep.
// ---------------------------------------------------------------------------
namespace {
// Workspace regions, each 256-byte aligned, in this order.
struct SweepWs {
  float *act_max, *w_max, *s, *w_scale, *a_scale, *y_q;
  double* y_ref;
  int8_t *Wq, *Xq;
  double* part;
  size_t bytes;
};
SweepWs sweep_layout(char* base, int64_t M, int64_t N, int64_t K) {
  SweepWs w{};
  size_t off = 0;
  auto take = [&](size_t n) {
    char* p = base ? base + off : nullptr;
    off += (n + 255) & ~(size_t)255;
    return p;
  };
  w.act_max = (float*)take(4 * K);
  w.w_max = (float*)take(4 * K);
  w.s = (float*)take(4 * K);
  w.w_scale = (float*)take(4 * N);
  w.a_scale = (float*)take(4 * (M > 0 ? M : 1));
  w.y_ref = (double*)take(8 * (size_t)M * N);
  w.y_q = (float*)take(4 * (size_t)M * N);
  w.Wq = (int8_t*)take((size_t)N * K);
  w.Xq = (int8_t*)take((size_t)M * K);
  w.part = (double*)take(sq::err_partials_bytes());
  w.bytes = off;
  return w;
}
}  // namespace

size_t sq_alpha_sweep_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return sweep_layout(nullptr, M, N, K).bytes;
}

int sq_alpha_sweep(const void* X, int xt, int64_t M, int64_t K, int64_t ldx, const void* W, int wt,
                   int64_t N, int64_t ldw, const double* alphas, int n_alpha, int mode, double* err,
                   double* rel, int32_t* best, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_matrix(X, xt, M, K, ldx);
  if (rc != SQ_OK) return rc;
  if ((rc = check_matrix(W, wt, N, K, ldw)) != SQ_OK) return rc;
  SQ_REQUIRE(N >= 1, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(N % 16 == 0, SQ_ERR_MISALIGNED);
  SQ_REQUIRE(valid_mode(mode), SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(alphas != nullptr && err != nullptr, SQ_ERR_INVALID_ARG);
  SQ_REQUIRE(n_alpha >= 1 && n_alpha <= kMaxSweepAlphas, SQ_ERR_INVALID_ARG);
  for (int i = 0; i < n_alpha; ++i)
    SQ_REQUIRE(alphas[i] >= 0.0 && alphas[i] <= 1.0, SQ_ERR_INVALID_ARG);   // NaN fails too
  SQ_REQUIRE(((uintptr_t)err & 7u) == 0 && ((uintptr_t)rel & 7u) == 0 && ((uintptr_t)best & 3u) == 0,
             SQ_ERR_MISALIGNED);
  if (M == 0) return SQ_OK;
  const size_t need = sq_alpha_sweep_workspace_bytes(M, N, K);
  SQ_REQUIRE(ws != nullptr && ws_bytes >= need, SQ_ERR_WORKSPACE);
  SQ_REQUIRE(((uintptr_t)ws & 255u) == 0, SQ_ERR_MISALIGNED);
  if ((rc = gate()) != SQ_OK) return rc;
  hipStream_t st = as_stream(stream);
  const SweepWs w = sweep_layout((char*)ws, M, N, K);
  const bool is_static = mode == SQ_ACT_PER_TENSOR_STATIC;
  // alpha-independent: activation and weight column maxima, the unquantized output
  if ((rc = sq::launch_fill2(w.act_max, K, w.w_max, K, 0.0f, st)) != SQ_OK) return rc;
  if ((rc = sq::launch_colmax2(X, xt, M, K, ldx, w.act_max, W, wt, N, K, ldw, w.w_max, st)) != SQ_OK)
    return rc;
  if ((rc = sq::launch_ref_gemm(X, xt, ldx, W, wt, ldw, M, N, K, w.y_ref, st)) != SQ_OK) return rc;
  for (int i = 0; i < n_alpha; ++i) {
    if ((rc = sq::launch_smooth_scale_from(w.act_max, w.w_max, w.s, K, alphas[i], st)) != SQ_OK)
      return rc;
    if ((rc = sq::launch_fold_quant(W, wt, N, K, ldw, w.s, w.Wq, w.w_scale, st)) != SQ_OK) return rc;
    if (is_static && (rc = sq::launch_static_scale(w.act_max, w.s, K, w.a_scale, st)) != SQ_OK)
      return rc;
    if ((rc = sq::launch_quant_act(X, xt, M, K, ldx, w.s, mode, w.Xq, w.a_scale, nullptr, st)) !=
        SQ_OK)
      return rc;
    if ((rc = sq::launch_gemm(w.Xq, w.Wq, w.a_scale, mode, w.w_scale, M, N, K, w.y_q, SQ_F32, N,
                              st)) != SQ_OK)
      return rc;
    if ((rc = sq::launch_sq_err(w.y_q, w.y_ref, M * N, w.part, err + 2 * i, st)) != SQ_OK) return rc;
  }
  if (rel != nullptr || best != nullptr) return sq::launch_sweep_pick(err, n_alpha, rel, best, st);
  return SQ_OK;
}

}  // extern "C"
