// Internal helpers shared by the library's translation units (not part of
// the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/mlip.h"

namespace mlip {

// ---------------------------------------------------------------- errors ---
void set_error(const char *fmt, ...);

struct Status {
  int code = MLIP_OK;
  bool ok() const { return code == MLIP_OK; }
};

#define MLIP_CHECK_ARG(cond, ...)          \
  do {                                     \
    if (!(cond)) {                         \
      ::mlip::set_error(__VA_ARGS__);      \
      return MLIP_ERR_INVALID;             \
    }                                      \
  } while (0)

#define MLIP_HIP(call)                                                        \
  do {                                                                        \
    hipError_t err_ = (call);                                                 \
    if (err_ != hipSuccess) {                                                 \
      ::mlip::set_error("%s failed: %s (%s:%d)", #call, hipGetErrorString(err_), \
                        __FILE__, __LINE__);                                  \
      return MLIP_ERR_HIP;                                                    \
    }                                                                         \
  } while (0)

// Launch check: catches bad launch configurations right away.
#define MLIP_LAUNCHED() MLIP_HIP(hipGetLastError())

// ------------------------------------------------------------- profiling ---
// Kernel classes timed by mlip_profile_*.
enum KClass {
  K_GRAPH = 0,
  K_EMBED_AGG,
  K_GEMM_DENSE,
  K_ROUTE_DISPATCH,
  K_GEMM_EXPERT_UP,      // P = u[tok] @ W1, silu
  K_GEMM_EXPERT_DOWN,    // Y = silu(P) @ W2
  K_COMBINE,
  K_READOUT,
  K_GEMM_EXPERT_VJP_DOWN,  // Q = (g[tok] @ W2^T) * silu'(P)
  K_GEMM_EXPERT_VJP_UP,    // U = Q @ W1^T
  K_EDGE_VJP,
  K_NUM_CLASSES
};

struct ProfScope {
  ProfScope(KClass k, hipStream_t s);
  ~ProfScope();
  KClass k;
  hipStream_t s;
  int slot = -1;
};

// --------------------------------------------------------------- workspace -
// Carves 256-byte aligned sub-buffers out of the caller's workspace.
struct Carver {
  char *base;
  size_t used = 0;
  explicit Carver(void *p) : base(static_cast<char *>(p)) {}
  template <typename T>
  T *take(size_t count) {
    size_t off = (used + 255) & ~size_t(255);
    used = off + count * sizeof(T);
    return base ? reinterpret_cast<T *>(base + off) : nullptr;
  }
  size_t bytes() const { return (used + 255) & ~size_t(255); }
};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroups are dealt round-robin to the 8 XCDs of the chip.  For a grid of
// padded_grid(n) workgroups, xcd_block(n) gives each XCD a contiguous range
// of the logical indices 0..n-1 (so neighbouring rows share one L2), or -1
// for a padding workgroup.
constexpr int kNumXcd = 8;
inline int64_t padded_grid(int64_t n) { return cdiv(n, kNumXcd) * kNumXcd; }
__device__ inline int64_t xcd_block(int64_t n) {
  const int64_t per = (n + kNumXcd - 1) / kNumXcd;
  const int64_t b = blockIdx.x;
  const int64_t logical = (b % kNumXcd) * per + b / kNumXcd;
  return logical < n ? logical : -1;
}

// ----------------------------------------------------------- scan / gemm ---
// Exclusive prefix sum of n int32 values (out may alias in); out[n] gets the
// total when write_total.  tmp needs scan_tmp_elems(n) int32 entries.
size_t scan_tmp_elems(int64_t n);
int exclusive_scan(const int32_t *in, int32_t *out, int64_t n, bool write_total,
                   int32_t *tmp, hipStream_t stream);

enum Epilogue {
  EPI_STORE = 0,   // C = A B
  EPI_RESID = 1,   // C = R + A B
  EPI_SILU = 2,    // C = A B, C2 = silu(A B)
  EPI_DSILU = 3,   // C = (A B) * silu'(R)
};

struct GemmArgs {
  const float *A = nullptr;   // rows of length K (row stride lda)
  int64_t lda = 0;
  const int32_t *a_rows = nullptr;  // optional row gather: A row of output row p
  const float *B = nullptr;   // per group: NN -> [K][N] (ldb = N), NT -> [N][K] (ldb = K)
  int64_t ldb = 0;
  int64_t b_group_stride = 0;
  float *C = nullptr;         // output rows p, stride ldc
  int64_t ldc = 0;
  float *C2 = nullptr;        // EPI_SILU second output (same layout as C)
  const float *R = nullptr;   // EPI_RESID residual / EPI_DSILU pre-activation
  int64_t ldr = 0;
  const int32_t *group_off = nullptr;  // [G+1] row ranges; nullptr -> one group [0, M)
  int n_groups = 1;
  int M = 0, N = 0, K = 0;
};

int launch_gemm(const GemmArgs &a, bool b_transposed, Epilogue epi, KClass cls,
                hipStream_t stream);

}  // namespace mlip
