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

// ------------------------------------------------------ debug bounds checks -
// Built with -DMLIP_DEBUG_BOUNDS (python -m element_routed_moe_amd.build
// --debug-bounds, which writes libmlip_debug.so), every index the kernels read
// from the data and then dereference (senders, reverse edges, gathered token
// rows, dispatch slots) is checked against its range.  A violation prints the
// index, its range and the source line, and the access goes to the nearest
// valid index instead, so the kernel finishes; the results are then wrong and
// the printed line names the first bad input.  Release builds compile the
// macro to the bare index.
#ifdef MLIP_DEBUG_BOUNDS
__device__ inline int64_t debug_check_index(int64_t i, int64_t n, const char *what, const char *file,
                                            int line) {
  if (n > 0 && (i < 0 || i >= n)) {
    printf("mlip bounds: %s index %lld outside [0, %lld) at %s:%d\n", what, (long long)i,
           (long long)n, file, line);
    return i < 0 ? 0 : n - 1;
  }
  return i;
}
#define MLIP_IDX(i, n, what) (::mlip::debug_check_index(int64_t(i), int64_t(n), what, __FILE__, __LINE__))
#else
#define MLIP_IDX(i, n, what) int64_t(i)
#endif

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
  K_ATTN_FWD,              // neighbour attention, edge part
  K_ATTN_VJP_RECV,         // attention VJP, receiver rows
  K_ATTN_VJP_SEND,         // attention VJP, sender rows (via the reverse edge)
  K_TRI_FWD,               // three-body update, edge part
  K_TRI_VJP_RECV,          // three-body VJP, receiver rows
  K_TRI_VJP_SEND,          // three-body VJP, sender rows
  K_GEMM_EXPERT_TAN,       // expert GEMMs of the tangent passes (training gradient)
  K_GEMM_WGRAD,            // weight-gradient GEMMs (sums over tokens / atoms)
  K_EDGE_TAN,              // edge passes of the tangents (and the W_e gradient)
  K_MOE_TAN,               // token-wise MoE tangents, gate and readout gradients
  K_ATTN_TAN,              // attention tangents (training gradient)
  K_GEMM_EXPERT_PAIR,      // Y = silu(P) W2 with Q = (g W2^T) silu'(P), one launch
  K_NUM_CLASSES
};

struct ProfScope {
  ProfScope(KClass k, hipStream_t s);
  ~ProfScope();
  ProfScope(const ProfScope &) = delete;
  ProfScope &operator=(const ProfScope &) = delete;
  KClass k;
  hipStream_t s;
  int slot = -1;               // >= 0 while this scope holds a recorded start event
  hipEvent_t a = nullptr, b = nullptr;
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

// ------------------------------------------- global -> LDS copies (gfx950) --
// global_load_lds_dwordx4 / _dword: each lane of a wave copies 16 (or 4)
// bytes from its own global address to a wave-uniform LDS base + 16 (4) x
// lane, without passing through registers.  The copies count on vmcnt.
#define MLIP_GLOBAL_PTR(p) ((const __attribute__((address_space(1))) void *)(p))
#define MLIP_LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

// s_waitcnt vmcnt(N), the other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier for pipelined k loops: this wave's LDS accesses are
// complete (lgkmcnt 0) and the compiler moves no memory access across it.
// Unlike __syncthreads() it does not wait for outstanding global loads, so
// the LDS copies of later stages stay in flight; each wave waits for its own
// copies of a stage (wait_vmcnt) before the barrier that publishes it.
// The wait is the builtin rather than asm text so that the compiler's own
// wait placement knows the LDS and scalar-load counter is clear after it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt left at their maxima
  asm volatile("s_barrier" ::: "memory");
}

// ------------------------------------------- cross-lane sums (DPP moves) --
// Moves inside 16-lane rows, with no LDS round trip: lane i ^ 1 and i ^ 2 of
// each quad, lane 7 - i of each 8-lane half row, lane 15 - i of each row.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_MIRROR = 0x140, DPP_HALF_MIRROR = 0x141;

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G a power of two).  Each step adds the
// partial of a lane in the other half of the current subgroup, whose own
// partial covers that half; a + b == b + a, so all lanes of a group end with
// the same bits.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp_mov<DPP_XOR1>(v);
  if constexpr (G >= 4) v += dpp_mov<DPP_XOR2>(v);
  if constexpr (G >= 8) v += dpp_mov<DPP_HALF_MIRROR>(v);
  if constexpr (G >= 16) v += dpp_mov<DPP_MIRROR>(v);
  if constexpr (G >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (G >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// ------------------------------------------------------- radial basis -----
// Constants of the pair-distance basis: K Gaussians exp(-gamma (r - k mu_step)^2),
// k = 0..K-1, mu_step = r_c/(K-1), gamma = (K-1)^2 / (2 r_c^2), and the cosine
// envelope f_c(r) = (cos(pi r / r_c) + 1)/2 for r < r_c.
struct Radial {
  float mu_step, gamma, pi_over_rc, rc;
};

__device__ inline Radial make_radial(float rc) {
  Radial p;
  p.rc = rc;
  p.mu_step = rc / float(MLIP_N_RBF - 1);
  p.gamma = float((MLIP_N_RBF - 1) * (MLIP_N_RBF - 1)) / (2.f * rc * rc);
  p.pi_over_rc = 3.14159265358979323846f / rc;
  return p;
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
  EPI_DSILU_Q = 4, // C = (A B) * silu'(R), C2 = A B
  EPI_TAN = 5,     // C = A B, C2 = (A B) * silu'(R)
};

struct GemmArgs {
  const float *A = nullptr;   // rows of length K (row stride lda)
  int64_t lda = 0;
  const int32_t *a_rows = nullptr;  // optional row gather: A row of output row p
  int64_t a_row_limit = 0;          // rows of A behind a_rows (debug bounds checks; 0: unknown)
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
  // Dense GEMMs only: split K into k_split parts whose products go to
  // split_ws ([k_split][M][N]) and are then summed in part order (with the
  // epilogue), when the output has too few tiles to fill the GPU.
  float *split_ws = nullptr;
  int k_split = 1;
};

int launch_gemm(const GemmArgs &a, bool b_transposed, Epilogue epi, KClass cls,
                hipStream_t stream);
// Two independent expert GEMMs over the same group_off in one launch (one
// tail instead of two); timed as class cls.
int launch_expert_pair(const GemmArgs &a, bool bt_a, Epilogue epi_a, const GemmArgs &b, bool bt_b,
                       Epilogue epi_b, KClass cls, hipStream_t stream);
// K parts a dense M x N x K GEMM is split into (1: none), and the floats of
// split_ws it then needs.
int dense_k_split(int64_t M, int64_t N, int64_t K);
int64_t dense_split_floats(int64_t M, int64_t N, int64_t K);
// The most split_ws an M x N output can need, for any K.
int64_t dense_split_floats_max(int64_t M, int64_t N);

// ------------------------------------------------------ training gradient -
// Weight-gradient sums on the matrix cores:
//   C_g = sum over rows p of group g of scale[p] * (A0[ar(p)]^T B0[br(p)] + A1[ar(p)]^T B1[br(p)])
// with ar / br optional row gathers; C is [G][Mo][No] (row-major, dense).
struct WgradArgs {
  const float *A0 = nullptr, *A1 = nullptr;   // rows of Mo floats, stride lda (A1/B1: optional term)
  const float *B0 = nullptr, *B1 = nullptr;   // rows of No floats, stride ldb
  int64_t lda = 0, ldb = 0;
  const int32_t *a_rows = nullptr, *b_rows = nullptr;
  int64_t row_limit = 0;                      // rows behind a_rows / b_rows (debug checks; 0: unknown)
  const float *scale = nullptr;               // per-row factor on the A operand
  const int32_t *group_off = nullptr;         // [G+1]; nullptr -> one group [0, P)
  int n_groups = 1, P = 0, Mo = 0, No = 0;
  float *C = nullptr;
};
// Floats of split-K scratch an ungrouped weight gradient needs (0: none).
int64_t wgrad_split_floats(const WgradArgs &a);
int launch_wgrad(const WgradArgs &a, float *split_ws, hipStream_t stream);

// One sweep over the CSR rows (see second.hip): out1 = W_e . T, out2 = W_e . U
// and, with R1, the W_e gradient sum_i R1_i T + R2_i U.
struct EdgeTanArgs {
  const int32_t *row_ptr = nullptr, *src = nullptr;
  const float *geom = nullptr;
  int n_atoms = 0;
  const float *x_dot = nullptr;               // [N][3]; the direction is x_sign * x_dot
  float x_sign = 1.f;
  const float *W_e = nullptr;                 // [K][De]
  const float *X = nullptr, *Y = nullptr;     // [N][De] sender rows (Y optional)
  float *out1 = nullptr, *out2 = nullptr;     // [N][De] (out2 optional)
  const float *R1 = nullptr, *R2 = nullptr;   // [N][De] (R1 null: no W_e gradient; R2 optional)
  float *dwe = nullptr;                       // [K][De]
  float *dwe_part = nullptr;                  // edge_tan_part_floats(N, De) scratch
  int De = 0;
  float rc = 0.f;
};
int edge_tan_groups(int n_atoms);
int64_t edge_tan_part_floats(int n_atoms, int De);   // size of dwe_part
int launch_edge_tan(const EdgeTanArgs &a, hipStream_t stream);
int launch_moe_tan(const float *P, const float *P_dot, const float *Q, const float *Q_dot, int M, int H,
                   float *act, float *act_dot, float *D, float *D_dot, float *dg, hipStream_t stream);
int launch_token_gate(const int32_t *z, const float *gate, const int32_t *slot, int N, int T, int k,
                      float *gt, hipStream_t stream);
int launch_gate_grad(const float *dg, const int32_t *z, const int32_t *topk, const float *gate,
                     const int32_t *exp_off, const int32_t *tok_atom, int T, int X, int k, double *G,
                     float *d_gate, float *d_logits, hipStream_t stream);
int64_t readout_grad_part_floats(int N, int D);
int launch_readout_grad(const float *h, const float *h_dot, const double *Ebar, const int32_t *struct_ptr,
                        int N, int B, int D, float *part, float *d_w_r, hipStream_t stream);

// ------------------------------------------------------------- attention ---
struct AttnArgs {
  const int32_t *row_ptr = nullptr, *src = nullptr, *rev = nullptr;
  const float *geom = nullptr;
  int n_atoms = 0;
  const float *Wa_e = nullptr;   // [K][Da]
  const float *qkv = nullptr;    // [N][3 Da]: q | k | v
  float *o = nullptr;            // [N][Da]
  float *stats = nullptr;        // [N][nh] (running max, weight sum)
  const float *obar = nullptr;   // [N][Da]
  float *qkv_bar = nullptr;      // [N][3 Da]
  float *edge_g = nullptr, *edge_a = nullptr;  // [E][nh]
  float *edge_c = nullptr;       // [E]
  float *grad_pos = nullptr;     // [N][3]
  float *atom_virial = nullptr;  // [N][6]
  int accumulate = 0;            // add to grad_pos / atom_virial instead of writing
  int Da = 0, nh = 0, cpl = 0, lph = 0;
  float rc = 0.f;
};

// Channels per lane (cpl) and lanes per head (lph) for Da channels in nh heads,
// one wavefront per row; MLIP_ERR_UNSUPPORTED when no layout fits.
int attn_lane_layout(int Da, int nh, int *cpl, int *lph);
int launch_attn_fwd(const AttnArgs &a, hipStream_t stream);
int launch_attn_vjp(const AttnArgs &a, hipStream_t stream);

// Tangents of the attention for the training gradient (attn.hip).
struct AttnTanArgs {
  const int32_t *row_ptr = nullptr, *src = nullptr, *rev = nullptr;
  const float *geom = nullptr;
  int n_atoms = 0;
  const float *x_dot = nullptr;   // [N][3]; position direction x_sign * x_dot
  float x_sign = 1.f;
  const float *Wa_e = nullptr;
  const float *qkv = nullptr, *qkv_dot = nullptr;   // [N][3 Da]
  const float *o = nullptr;                         // [N][Da]
  float *o_dot = nullptr;                           // [N][Da] (JVP output, VJP-tangent input)
  const float *stats = nullptr;                     // [N][nh] (max, weight sum)
  float *tstat = nullptr;                           // [N][nh] T = sum a s_dot + f_dot w / Z
  const float *obar = nullptr, *obar_dot = nullptr; // [N][Da]
  float *qkv_bar_dot = nullptr;                     // [N][3 Da]
  float *edge_g = nullptr, *edge_gd = nullptr, *edge_a = nullptr, *edge_ad = nullptr;  // [E][nh]
  float *ebar = nullptr, *ebar_dot = nullptr;       // [E][Da]
  int Da = 0, nh = 0, cpl = 0, lph = 0;
  float rc = 0.f;
};
int launch_attn_jvp(const AttnTanArgs &a, hipStream_t stream);
int launch_attn_tvjp(const AttnTanArgs &a, hipStream_t stream);
// sum_e beta_e (x) X_e + alpha_e (x) Y_e over all edges (rows of X, Y indexed
// by edge), alpha = f_c phi, beta = r_dot d(f_c phi)/dr: the gradient of a
// K x D basis map e = f_c (phi W) given per-edge dL/de (X) and its tangent (Y).
int launch_edge_basis_grad(const int32_t *row_ptr, const int32_t *src, const float *geom, int n_atoms,
                           const float *x_dot, float x_sign, const float *X, const float *Y, int D,
                           float rc, float *part, float *dW, hipStream_t stream);

// ------------------------------------------------------- three-body update -
struct TriArgs {
  const int32_t *row_ptr = nullptr, *src = nullptr, *rev = nullptr;
  const float *geom = nullptr;
  int n_atoms = 0;
  const float *s = nullptr;       // [N][Dt] = h W_s
  const float *W_ang = nullptr;   // [4][Dt]
  float *tau = nullptr;           // [N][Dt]
  const float *taubar = nullptr;  // [N][Dt]
  float *sigma = nullptr;         // [E][Dt]
  float *gvec = nullptr;          // [E][4]
  float *sbar = nullptr;          // [N][Dt]
  float *grad_pos = nullptr;      // [N][3]
  float *atom_virial = nullptr;   // [N][6]
  int accumulate = 0;
  int Dt = 0, cpl = 0;
  float rc = 0.f;
};

int tri_lane_layout(int Dt, int *cpl);
int launch_tri_fwd(const TriArgs &a, hipStream_t stream);
int launch_tri_vjp(const TriArgs &a, hipStream_t stream);
// Training tangents of the three-body update (tri.hip): tau_dot; and the
// tangent of the gradient: sigma_dot [E][Dt] (scratch), per-row W_ang
// gradient shares wang_part [N][4][Dt], sbar_dot [N][Dt].
int launch_tri_jvp(const int32_t *row_ptr, const int32_t *src, const float *geom, int n_atoms,
                   const float *x_dot, float x_sign, const float *s, const float *s_dot, const float *W_ang,
                   int Dt, float rc, float *tau_dot, hipStream_t stream);
int launch_tri_tvjp(const int32_t *row_ptr, const int32_t *src, const int32_t *rev, const float *geom,
                    int n_atoms, const float *x_dot, float x_sign, const float *s, const float *s_dot,
                    const float *W_ang, const float *taubar, const float *taubar_dot, int Dt, float rc,
                    float *sigma_dot, float *wang_part, float *sbar_dot, hipStream_t stream);
// sum over n rows of [n][KD] (fixed order, two stages; part2 holds cdiv(n, 32) x KD)
int launch_row_sum(const float *rows, int n, int KD, float *part2, float *out, hipStream_t stream);

}  // namespace mlip
