// Kernels of the training gradient: the parameter gradient of a loss on
// energies and forces through one interaction block.
//
// Paper review of "Breaking the Training Barrier of Billion-Parameter
// Universal MLIPs", section 3.3: the forces are the negative gradient of the
// energy and the potential is fitted to energies and forces, so training
// differentiates the force once more.  For L(E, F) with Ebar = dL/dE and
// Fbar = dL/dF, the parameter gradient equals the derivative of the
// reverse-mode gradient dE/dtheta along the position direction
// x_dot = -Fbar, plus the first-order gradient for the upstream Ebar w_r
// (forward over reverse).  The kernels here are the pieces of that
// derivative that the forward and input-gradient kernels do not already
// provide:
//
//   * wgrad: weight-gradient sums  C_g = sum_{p in group g} s_p (A0_p^T B0_p
//     + A1_p^T B1_p)  on the matrix cores (the two terms are the product
//     rule of a tangent, each a sum over tokens or atoms);
//   * edge_tan: one pass over the receiver-sorted edges that forms, per row
//     and column, the basis-weighted sums of the sender rows; it gives the
//     tangent of the aggregation, the primal and tangent of the sender-side
//     gradient, and the W_e gradient in the same sweep;
//   * moe_tan: token-wise SiLU tangents of the expert MLPs and the per-token
//     gate-gradient dot products;
//   * gate / readout gradients.
//
// Every sum over tokens, atoms or edges runs in a fixed order (no floating-
// point atomics), so the results do not depend on scheduling.
#include <algorithm>

#include <type_traits>

#include "common.h"

namespace mlip {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float f2v __attribute__((ext_vector_type(2)));

constexpr int K = MLIP_N_RBF;

// ----------------------------------------------------------------- wgrad --
// 128 x 128 output tile per 256-thread workgroup (2 x 2 wavefronts of
// 64 x 64, each 2 x 2 blocks of v_mfma_f32_32x32x2_f32).  K runs over the
// rows p (tokens or atoms) WK at a time.  Both operands arrive as rows of
// the output's M or N extent, so a step's tiles are [k][m] / [k][n]: 16 rows
// of 512 bytes, copied from global memory straight into LDS
// (global_load_lds_dwordx4, no register staging) through a WS-stage ring,
// WS - 1 steps ahead of the step being multiplied, one barrier per step.
// In LDS the 4-column chunk c of k-row k sits at c ^ (8 * ((k/4) & 1)), so
// the two half-waves of an MFMA read (k-rows 4 apart) hit different banks;
// each lane reads its MFMA values one float at a time.
// The rows are gathered (token -> atom) along K: the gather indices of a
// step are loaded one step before its copies are issued.  A per-row factor
// on A (the gate) is copied into LDS with the step (4 bytes per lane) and
// applied as the A values are read.  Rows past the group's end are copied
// from a valid row and zeroed in LDS before the stage is published.
//
// Tile order: a tile's cost is its group's row count, which varies widely
// between experts, so tiles are not given to the XCDs in contiguous ranges
// (whole experts per XCD): workgroup b takes tile b, and the hardware deals
// consecutive workgroups to the 8 XCDs in turn, so every XCD gets an equal
// share of every expert.
constexpr int WB = 128;
constexpr int WK = 16;   // rows per K step (32 measured 11% slower at S)
constexpr int WS = 3;    // LDS stages: 3 x 17 KB, three workgroups per CU
constexpr int W_THREADS = 256;
constexpr int W_SLOTS = WK * WB / 4 / W_THREADS;   // 16-byte copies per lane per operand and step

template <bool GA, bool GB, bool SC>
__global__ void __launch_bounds__(W_THREADS, 2) wgrad_kernel(WgradArgs g, int k_split, int64_t rows_per_split,
                                                             float *__restrict__ part) {
  // One array per stage for the A tile, the B tile and the row factors, and
  // one per stage for the gather indices, so the compiler can tell the stage
  // being read from the stages whose copies are still in flight.  Only LDS
  // copies are in flight in the k loop (the indices too travel through LDS):
  // mixed with ordinary loads, the waitcnt insertion can no longer count
  // them in order and drains the counter before LDS reads.
  // The row factors and the gather indices of a step are the same for every
  // wave: all four copy them to one shared 64-entry region (concurrent copies
  // of identical values), which keeps the LDS within three workgroups per CU.
  constexpr int STG = 2 * WK * WB + (SC ? 64 : 0);
  constexpr int NG = (GA ? 1 : 0) + (GB ? 1 : 0);   // gathered operands
  constexpr int XST = NG ? NG * 64 : 4;
  __shared__ __attribute__((aligned(16))) float L0[STG], L1[STG], L2[STG];
  __shared__ __attribute__((aligned(16))) int X0[XST], X1[XST], X2[XST];
  float *const As[WS] = {L0, L1, L2};
  float *const Bs[WS] = {L0 + WK * WB, L1 + WK * WB, L2 + WK * WB};
  float *const Ss[WS] = {L0 + 2 * WK * WB, L1 + 2 * WK * WB, L2 + 2 * WK * WB};
  int *const Xs[WS] = {X0, X1, X2};
  static_assert(WS == 3, "the k loop is written for three stages");

  const int mt = (g.Mo + WB - 1) / WB, nt = (g.No + WB - 1) / WB;
  const int G = g.group_off ? g.n_groups : 1;
  const int64_t per_group = int64_t(mt) * nt;
  const int64_t t = blockIdx.x;
  if (t >= int64_t(G) * per_group * k_split) return;
  // order: split, then group, then n-tile, then m-tile (m fastest)
  const int64_t tiles = int64_t(G) * per_group;
  const int split = int(t / tiles);
  const int64_t tg = t - int64_t(split) * tiles;
  const int grp = int(tg / per_group);
  const int rem = int(tg - int64_t(grp) * per_group);
  const int m0 = (rem % mt) * WB, n0 = (rem / mt) * WB;
  int p0 = g.group_off ? g.group_off[grp] : 0;
  int p1 = g.group_off ? g.group_off[grp + 1] : g.P;
  if (k_split > 1) {
    const int64_t a = int64_t(p0) + int64_t(split) * rows_per_split;
    const int64_t b = a + rows_per_split;
    p0 = int(a < p1 ? a : p1);
    p1 = int(b < p1 ? b : p1);
  }
  const int steps_term = p1 > p0 ? (p1 - p0 + WK - 1) / WK : 0;
  const int n_terms = (g.A1 && g.B1) ? 2 : 1;
  const int nsteps = steps_term * n_terms;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, half = lane >> 5, kh = half * 4;

  floatx16 acc[2][2];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.f;

  if (nsteps > 0) {
    // copy slot q of this lane: chunk c = (q*4 + wave)*64 + lane of the
    // [WK][WB] tile, k-row kr = c / 32, stored chunk c % 32
    int kr[W_SLOTS], ca[W_SLOTS], cb[W_SLOTS], lofs[W_SLOTS];
#pragma unroll
    for (int q = 0; q < W_SLOTS; ++q) {
      const int c = (q * 4 + wave) * 64 + lane;
      kr[q] = c >> 5;
      const int col = 4 * ((c & 31) ^ (8 * ((kr[q] >> 2) & 1)));
      ca[q] = m0 + col < g.Mo ? m0 + col : m0;   // columns past the edge copy a valid one; never stored
      cb[q] = n0 + col < g.No ? n0 + col : n0;
      lofs[q] = c * 4;
    }
    // step s -> (term, first row); steps past the last one are clamped to it
    auto step_rows = [&](int s, int &term, int &k0) {
      s = s < nsteps ? s : nsteps - 1;
      term = s >= steps_term ? 1 : 0;
      k0 = p0 + (s - term * steps_term) * WK;
    };
    // this lane's row of the step (lanes past WK repeat row 0); rows past p1 take p0
    auto lane_row = [&](int k0) {
      const int p = k0 + (lane < WK ? lane : 0);
      return p < p1 ? p : p0;
    };
    // every wave copies the step's WK gather indices to the shared X[set]
    auto issue_idx = [&](int set, int s) {
      int term, k0;
      step_rows(s, term, k0);
      const int p = lane_row(k0);
      if (GA) __builtin_amdgcn_global_load_lds(MLIP_GLOBAL_PTR(g.a_rows + p), MLIP_LDS_PTR(Xs[set]), 4, 0, 0);
      if (GB) __builtin_amdgcn_global_load_lds(MLIP_GLOBAL_PTR(g.b_rows + p), MLIP_LDS_PTR(Xs[set] + (GA ? 64 : 0)), 4, 0, 0);
    };
    auto issue = [&](int st, int set, int s) {
      int term, k0;
      step_rows(s, term, k0);
      const float *A = term ? g.A1 : g.A0;
      const float *B = term ? g.B1 : g.B0;
      int64_t ra[W_SLOTS], rb[W_SLOTS];
#pragma unroll
      for (int q = 0; q < W_SLOTS; ++q) {
        int p = k0 + kr[q];
        p = p < p1 ? p : p0;
        ra[q] = GA ? MLIP_IDX(Xs[set][kr[q]], g.row_limit, "token row") : int64_t(p);
        rb[q] = GB ? MLIP_IDX(Xs[set][(GA ? 64 : 0) + kr[q]], g.row_limit, "token row") : int64_t(p);
      }
#pragma unroll
      for (int q = 0; q < W_SLOTS; ++q)
        __builtin_amdgcn_global_load_lds(MLIP_GLOBAL_PTR(A + ra[q] * g.lda + ca[q]), MLIP_LDS_PTR(As[st] + (q * 4 + wave) * 256), 16,
                                         0, 0);
#pragma unroll
      for (int q = 0; q < W_SLOTS; ++q)
        __builtin_amdgcn_global_load_lds(MLIP_GLOBAL_PTR(B + rb[q] * g.ldb + cb[q]), MLIP_LDS_PTR(Bs[st] + (q * 4 + wave) * 256), 16,
                                         0, 0);
      if (SC) __builtin_amdgcn_global_load_lds(MLIP_GLOBAL_PTR(g.scale + lane_row(k0)), MLIP_LDS_PTR(Ss[st]), 4, 0, 0);
    };
    constexpr int NIDX = NG;
    constexpr int NL = 2 * W_SLOTS + (SC ? 1 : 0);
    // Rows past p1 (the last step of a term): each lane zeroes the chunks it
    // copied, after they have landed and before the barrier.
    auto zero_tail = [&](int st, int s) {
      int term, k0;
      step_rows(s, term, k0);
      if (k0 + WK <= p1) return;
      const floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < W_SLOTS; ++q) {
        if (k0 + kr[q] >= p1) {
          *reinterpret_cast<floatx4 *>(As[st] + lofs[q]) = z;
          *reinterpret_cast<floatx4 *>(Bs[st] + lofs[q]) = z;
        }
      }
    };
    auto compute = [&](int st) {
      const float *Ab = As[st];
      const float *Bb = Bs[st];
#pragma unroll
      for (int kg = 0; kg < WK; kg += 8) {
        floatx4 sc = {1.f, 1.f, 1.f, 1.f};
        if (SC) sc = *reinterpret_cast<const floatx4 *>(Ss[st] + kg + kh);
        float a[2][4], b[2][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = (kg + kh + q) * WB;
#pragma unroll
          for (int bi = 0; bi < 2; ++bi) a[bi][q] = Ab[row + ((wm * 64 + bi * 32 + l32) ^ (32 * half))] * sc[q];
#pragma unroll
          for (int bj = 0; bj < 2; ++bj) b[bj][q] = Bb[row + ((wn * 64 + bj * 32 + l32) ^ (32 * half))];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 2; ++bj)
              acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[bi][q], b[bj][q], acc[bi][bj], 0, 0, 0);
      }
    };
    // Issue order, one pair per step: the gather indices of step j + 1, then
    // the tiles of step j.  At the top of step kt one pair (indices of kt + 2,
    // tiles of kt + 1) is younger than step kt's tiles; after the barrier the
    // indices of kt + 2 are awaited (only the tiles of kt + 1 stay in flight),
    // read back, and the pair (indices of kt + 3, tiles of kt + 2) is issued.
    auto step = [&](auto sc_, int kt) {
      constexpr int s = decltype(sc_)::value;
      wait_vmcnt<NIDX + NL>();
      zero_tail(s, kt);
      lds_barrier();
      if (NIDX) {
        wait_vmcnt<NL>();
        issue_idx(s, kt + WS);
      }
      issue((s + WS - 1) % WS, (s + WS - 1) % WS, kt + WS - 1);
      compute(s);
    };
    if (NIDX) {
      issue_idx(0, 0);
      wait_vmcnt<0>();
      issue_idx(1, 1);
    }
    issue(0, 0, 0);
    if (NIDX) {
      wait_vmcnt<NL>();
      issue_idx(2, 2);
    }
    issue(1, 1, 1);
    int kt = 0;
    for (; kt + WS <= nsteps; kt += WS) {
      step(std::integral_constant<int, 0>{}, kt);
      step(std::integral_constant<int, 1>{}, kt + 1);
      step(std::integral_constant<int, 2>{}, kt + 2);
    }
    if (kt < nsteps) {
      step(std::integral_constant<int, 0>{}, kt);
      if (kt + 1 < nsteps) step(std::integral_constant<int, 1>{}, kt + 1);
    }
    wait_vmcnt<0>();   // no copy may land in LDS after the workgroup ends
  }

  // output element (m, n): m = 8*(r/4) + 4*(lane/32) + r%4 of the block, n = lane%32
  float *out = k_split > 1 ? part + int64_t(split) * g.Mo * g.No
                           : g.C + int64_t(grp) * g.Mo * g.No;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const int n = n0 + wn * 64 + bj * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + bi * 32 + 8 * (r >> 2) + kh + (r & 3);
        if (m < g.Mo && n < g.No) out[int64_t(m) * g.No + n] = acc[bi][bj][r];
      }
    }
}

// C = sum over the k_split partial products, in split order.
__global__ void __launch_bounds__(256) split_sum_kernel(const float4 *__restrict__ part, int k_split,
                                                        int64_t n4, float4 *__restrict__ C) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n4) return;
  float4 s = part[i];
  for (int q = 1; q < k_split; ++q) {
    const float4 v = part[int64_t(q) * n4 + i];
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  C[i] = s;
}

// -------------------------------------------------------------- edge_tan --
// Per row i and column c (rows of the receiver-sorted CSR, senders j):
//   alpha_e,k = f_c(r) phi_k(r)                         (the edge basis)
//   beta_e,k  = rdot_e d(f_c phi_k)/dr,  rdot_e = dhat_e . (xdot_j - xdot_i)
//   T_k = sum_e beta_e,k X_j + alpha_e,k Y_j,   U_k = sum_e alpha_e,k X_j
//   out1_i = sum_k W_e[k] T_k,  out2_i = sum_k W_e[k] U_k,
//   dW_e[k] += R1_i T_k + R2_i U_k.
// The edge basis and its derivative are symmetric in the two ends of an edge
// (r and rdot are the same for the reverse edge), so a pass over the rows of
// the same CSR serves both the receiver-side sums of the forward and the
// sender-side sums of the gradient.  One 64-lane workgroup owns 128 columns
// (two per lane) of a contiguous group of rows; it keeps its W_e-gradient
// partial sums in registers and writes them once.
constexpr int ET_CHUNK = 64;
constexpr int ET_COLS = 128;
constexpr int ET_MAX_GROUPS = 1024;
constexpr int ET_UNROLL = 4;

__device__ inline f2v ld2(const float *p) { return *reinterpret_cast<const f2v *>(p); }
__device__ inline void st2(float *p, f2v v) { *reinterpret_cast<f2v *>(p) = v; }

template <bool HAS_Y, bool HAS_DW>
__global__ void __launch_bounds__(64) edge_tan_kernel(EdgeTanArgs g, int n_groups, int rows_per,
                                                      int n_slices, float *__restrict__ dwe_part) {
  // per edge of the chunk: alpha (0..K-1), beta (K..2K-1)
  __shared__ __attribute__((aligned(16))) float bas[ET_CHUNK][2 * K];
  __shared__ int jj[ET_CHUNK];
  const int lane = threadIdx.x;
  const int64_t blk = xcd_block(int64_t(n_groups) * n_slices);
  if (blk < 0) return;
  const int rg = int(blk / n_slices);
  const int slice = int(blk - int64_t(rg) * n_slices);
  const int De = g.De;
  const int c = slice * ET_COLS + 2 * lane;
  const bool active = c < De;
  const int cc = active ? c : 0;
  const Radial R = make_radial(g.rc);
  const float rc = g.rc;
  const float4 *geom = reinterpret_cast<const float4 *>(g.geom);

  f2v w[K], dw[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    w[k] = ld2(g.W_e + k * De + cc);
    dw[k] = f2v{0.f, 0.f};
  }
  const int i0 = rg * rows_per;
  const int i1 = min(g.n_atoms, i0 + rows_per);
  for (int i = i0; i < i1; ++i) {
    f2v T[K], U[K];
#pragma unroll
    for (int k = 0; k < K; ++k) T[k] = U[k] = f2v{0.f, 0.f};
    const float xi0 = g.x_dot[3 * i], xi1 = g.x_dot[3 * i + 1], xi2 = g.x_dot[3 * i + 2];
    const int r0 = g.row_ptr[i], r1 = g.row_ptr[i + 1];
    for (int e0 = r0; e0 < r1; e0 += ET_CHUNK) {
      const int n = min(ET_CHUNK, r1 - e0);
      __syncthreads();   // the previous chunk's LDS rows have been read
      if (lane < n) {
        const int e = e0 + lane;
        const float4 gm = geom[e];
        const int j = int(MLIP_IDX(g.src[e], g.n_atoms, "sender"));
        const float r = gm.w;
        float rdot = 0.f;
        if (r > 0.f) {
          rdot = g.x_sign * (gm.x * (g.x_dot[3 * j] - xi0) + gm.y * (g.x_dot[3 * j + 1] - xi1) +
                             gm.z * (g.x_dot[3 * j + 2] - xi2)) / r;
        }
        float fc = 0.f, dfc = 0.f;
        if (r < rc) {
          float sn, cs;
          __sincosf(r * R.pi_over_rc, &sn, &cs);
          fc = 0.5f * (cs + 1.f);
          dfc = -0.5f * R.pi_over_rc * sn;
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float x = r - float(k) * R.mu_step;
          const float ph = __expf(-R.gamma * x * x);
          bas[lane][k] = fc * ph;
          bas[lane][K + k] = rdot * (dfc * ph + fc * (-2.f * R.gamma * x * ph));
        }
        jj[lane] = j;
      }
      __syncthreads();
      int q = 0;
      for (; q + ET_UNROLL <= n; q += ET_UNROLL) {
        f2v xv[ET_UNROLL], yv[ET_UNROLL];
#pragma unroll
        for (int u = 0; u < ET_UNROLL; ++u) {
          const int64_t j = jj[q + u];
          xv[u] = ld2(g.X + j * De + cc);
          if (HAS_Y) yv[u] = ld2(g.Y + j * De + cc);
        }
#pragma unroll
        for (int u = 0; u < ET_UNROLL; ++u) {
          const float4 *b4 = reinterpret_cast<const float4 *>(bas[q + u]);
#pragma unroll
          for (int k4 = 0; k4 < K / 4; ++k4) {
            const float4 al = b4[k4], be = b4[K / 4 + k4];
            const float av[4] = {al.x, al.y, al.z, al.w}, bv[4] = {be.x, be.y, be.z, be.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int k = 4 * k4 + t;
              T[k] += bv[t] * xv[u];
              if (HAS_Y) T[k] += av[t] * yv[u];
              U[k] += av[t] * xv[u];
            }
          }
        }
      }
      for (; q < n; ++q) {
        const int64_t j = jj[q];
        const f2v xv = ld2(g.X + j * De + cc);
        f2v yv = f2v{0.f, 0.f};
        if (HAS_Y) yv = ld2(g.Y + j * De + cc);
#pragma unroll
        for (int k = 0; k < K; ++k) {
          T[k] += bas[q][K + k] * xv;
          if (HAS_Y) T[k] += bas[q][k] * yv;
          U[k] += bas[q][k] * xv;
        }
      }
    }
    f2v o1 = f2v{0.f, 0.f}, o2 = f2v{0.f, 0.f};
#pragma unroll
    for (int k = 0; k < K; ++k) {
      o1 += w[k] * T[k];
      o2 += w[k] * U[k];
    }
    if (active) {
      st2(g.out1 + int64_t(i) * De + c, o1);
      if (g.out2) st2(g.out2 + int64_t(i) * De + c, o2);
    }
    if (HAS_DW) {
      const f2v f1 = ld2(g.R1 + int64_t(i) * De + cc);
      const f2v f2 = g.R2 ? ld2(g.R2 + int64_t(i) * De + cc) : f2v{0.f, 0.f};
#pragma unroll
      for (int k = 0; k < K; ++k) dw[k] += f1 * T[k] + f2 * U[k];
    }
  }
  if (HAS_DW && active) {
#pragma unroll
    for (int k = 0; k < K; ++k) st2(dwe_part + (int64_t(rg) * K + k) * De + c, dw[k]);
  }
}

// sum over edges of beta_e,k X_e,c + alpha_e,k Y_e,c with per-edge rows X, Y
// (not gathered): the W gradient of a basis map e = f_c (phi W) from dL/de
// (X) and its tangent (Y) when the basis moves with r_dot.  Same row groups,
// slices and partial sums as edge_tan.
__global__ void __launch_bounds__(64) edge_basis_grad_kernel(
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ src, const float4 *__restrict__ geom,
    int n_atoms, const float *__restrict__ x_dot, float x_sign, const float *__restrict__ X,
    const float *__restrict__ Y, int D, float rc, int n_groups, int rows_per, int n_slices,
    float *__restrict__ part) {
  __shared__ __attribute__((aligned(16))) float bas[ET_CHUNK][2 * K];
  const int lane = threadIdx.x;
  const int64_t blk = xcd_block(int64_t(n_groups) * n_slices);
  if (blk < 0) return;
  const int rg = int(blk / n_slices);
  const int slice = int(blk - int64_t(rg) * n_slices);
  const int c = slice * ET_COLS + 2 * lane;
  const bool active = c < D;
  const int cc = active ? c : 0;
  const Radial R = make_radial(rc);
  f2v dw[K];
#pragma unroll
  for (int k = 0; k < K; ++k) dw[k] = f2v{0.f, 0.f};
  const int i0 = rg * rows_per;
  const int i1 = min(n_atoms, i0 + rows_per);
  for (int i = i0; i < i1; ++i) {
    const float xi0 = x_dot[3 * i], xi1 = x_dot[3 * i + 1], xi2 = x_dot[3 * i + 2];
    const int r0 = row_ptr[i], r1 = row_ptr[i + 1];
    for (int e0 = r0; e0 < r1; e0 += ET_CHUNK) {
      const int n = min(ET_CHUNK, r1 - e0);
      __syncthreads();
      if (lane < n) {
        const int e = e0 + lane;
        const float4 gm = geom[e];
        const int j = int(MLIP_IDX(src[e], n_atoms, "sender"));
        const float r = gm.w;
        float rdot = 0.f;
        if (r > 0.f)
          rdot = x_sign * (gm.x * (x_dot[3 * j] - xi0) + gm.y * (x_dot[3 * j + 1] - xi1) +
                           gm.z * (x_dot[3 * j + 2] - xi2)) / r;
        float fc = 0.f, dfc = 0.f;
        if (r < rc) {
          float sn, cs;
          __sincosf(r * R.pi_over_rc, &sn, &cs);
          fc = 0.5f * (cs + 1.f);
          dfc = -0.5f * R.pi_over_rc * sn;
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float x = r - float(k) * R.mu_step;
          const float ph = __expf(-R.gamma * x * x);
          bas[lane][k] = fc * ph;
          bas[lane][K + k] = rdot * (dfc * ph + fc * (-2.f * R.gamma * x * ph));
        }
      }
      __syncthreads();
      for (int q = 0; q < n; ++q) {
        const int64_t e = e0 + q;
        const f2v xv = ld2(X + e * D + cc), yv = ld2(Y + e * D + cc);
        const float4 *b4 = reinterpret_cast<const float4 *>(bas[q]);
#pragma unroll
        for (int k4 = 0; k4 < K / 4; ++k4) {
          const float4 al = b4[k4], be = b4[K / 4 + k4];
          // two fused multiply-adds per term into the running sums
          dw[4 * k4] = be.x * xv + dw[4 * k4];
          dw[4 * k4] = al.x * yv + dw[4 * k4];
          dw[4 * k4 + 1] = be.y * xv + dw[4 * k4 + 1];
          dw[4 * k4 + 1] = al.y * yv + dw[4 * k4 + 1];
          dw[4 * k4 + 2] = be.z * xv + dw[4 * k4 + 2];
          dw[4 * k4 + 2] = al.z * yv + dw[4 * k4 + 2];
          dw[4 * k4 + 3] = be.w * xv + dw[4 * k4 + 3];
          dw[4 * k4 + 3] = al.w * yv + dw[4 * k4 + 3];
        }
      }
    }
  }
  if (active) {
#pragma unroll
    for (int k = 0; k < K; ++k) st2(part + (int64_t(rg) * K + k) * D + c, dw[k]);
  }
}

// dW_e[k][c] = sum over row groups of the partials, in two fixed-order
// stages: blocks of DWE_SPAN consecutive groups (coalesced rows of KD floats),
// then the block sums.
constexpr int DWE_SPAN = 32;
__global__ void __launch_bounds__(256) dwe_stage1_kernel(const float *__restrict__ part, int n_groups,
                                                         int KD, float *__restrict__ part2) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= KD) return;
  const int q0 = blockIdx.y * DWE_SPAN, q1 = min(n_groups, q0 + DWE_SPAN);
  float s = 0.f;
  for (int q = q0; q < q1; ++q) s += part[int64_t(q) * KD + idx];
  part2[int64_t(blockIdx.y) * KD + idx] = s;
}

__global__ void __launch_bounds__(256) dwe_sum_kernel(const float *__restrict__ part, int n_groups,
                                                      int KD, float *__restrict__ dwe) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= KD) return;
  float s = 0.f;
  for (int q = 0; q < n_groups; ++q) s += part[int64_t(q) * KD + idx];
  dwe[idx] = s;
}

// --------------------------------------------------------------- moe_tan --
// Token-wise (one wavefront per token row, H columns) with the saved
// pre-activation P, its tangent P_dot, the upstream product Q = g W2^T and
// its tangent Q_dot (optional):
//   sg = sigmoid(P), s1 = silu'(P) = sg (1 + P (1 - sg)),
//   s2 = silu''(P) = sg (1 - sg) (2 + P (1 - 2 sg));
//   act = silu(P), act_dot = s1 P_dot, D = s1 Q, D_dot = s2 P_dot Q + s1 Q_dot,
//   dg = sum over the row of (act Q_dot + act_dot Q)   (d<g, y>/dgate, tangent).
__global__ void __launch_bounds__(256) moe_tan_kernel(
    const float4 *__restrict__ P, const float4 *__restrict__ Pd, const float4 *__restrict__ Q,
    const float4 *Qd, int M, int H4, float4 *__restrict__ act, float4 *__restrict__ actd,
    float4 *__restrict__ D, float4 *Dd, float *__restrict__ dg) {
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= M) return;
  const int lane = threadIdx.x & 63;
  float acc = 0.f;
  for (int c = lane; c < H4; c += 64) {
    const int64_t o = int64_t(p) * H4 + c;
    const float4 x4 = P[o], pd4 = Pd[o], q4 = Q[o];
    const float4 qd4 = Qd ? Qd[o] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float xs[4] = {x4.x, x4.y, x4.z, x4.w}, pds[4] = {pd4.x, pd4.y, pd4.z, pd4.w};
    const float qs[4] = {q4.x, q4.y, q4.z, q4.w}, qds[4] = {qd4.x, qd4.y, qd4.z, qd4.w};
    float a[4], ad[4], d[4], dd[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float x = xs[t];
      const float sg = 1.f / (1.f + __expf(-x));
      const float s1 = sg * (1.f + x * (1.f - sg));
      const float s2 = sg * (1.f - sg) * (2.f + x * (1.f - 2.f * sg));
      a[t] = x * sg;
      ad[t] = s1 * pds[t];
      d[t] = s1 * qs[t];
      dd[t] = s2 * pds[t] * qs[t] + s1 * qds[t];
      acc += a[t] * qds[t] + ad[t] * qs[t];
    }
    act[o] = make_float4(a[0], a[1], a[2], a[3]);
    actd[o] = make_float4(ad[0], ad[1], ad[2], ad[3]);
    D[o] = make_float4(d[0], d[1], d[2], d[3]);
    Dd[o] = make_float4(dd[0], dd[1], dd[2], dd[3]);
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (lane == 0) dg[p] = acc;
}

// gt[slot(i, r)] = gate[z_i, r]: the gate of every token in dispatch order.
__global__ void __launch_bounds__(256) token_gate_kernel(const int32_t *__restrict__ z,
                                                         const float *__restrict__ gate,
                                                         const int32_t *__restrict__ slot, int N, int T,
                                                         int k, float *__restrict__ gt) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= int64_t(N) * k) return;
  const int i = int(idx / k), r = int(idx - int64_t(i) * k);
  const int t = z[i];
  if (t < 0 || t >= T) return;
  gt[MLIP_IDX(slot[idx], int64_t(N) * k, "dispatch slot")] = gate[t * k + r];
}

// G[t, r] = sum of dg over the tokens of element t routed at rank r.  Those
// tokens are contiguous: expert x = topk[t, r]'s range, ordered by element.
// One wavefront per (t, r), float64 partial sums in a fixed tree.
__global__ void __launch_bounds__(256) gate_sum_kernel(const float *__restrict__ dg,
                                                       const int32_t *__restrict__ z,
                                                       const int32_t *__restrict__ topk,
                                                       const int32_t *__restrict__ exp_off,
                                                       const int32_t *__restrict__ tok_atom, int T,
                                                       int k, double *__restrict__ G) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= T * k) return;
  const int lane = threadIdx.x & 63;
  const int t = w / k;
  const int x = topk[w];
  // first token of the expert's range with element >= t, then > t
  int lo = exp_off[x], hi = exp_off[x + 1];
  int a = lo, b = hi;
  while (a < b) {
    const int m = (a + b) >> 1;
    if (z[tok_atom[m]] < t) a = m + 1;
    else b = m;
  }
  int c = a, d = hi;
  while (c < d) {
    const int m = (c + d) >> 1;
    if (z[tok_atom[m]] <= t) c = m + 1;
    else d = m;
  }
  double acc = 0.0;
  for (int p = a + lane; p < c; p += 64) acc += double(dg[p]);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (lane == 0) G[w] = acc;
}

// d logits[t, x]: the gates are the softmax of the chosen logits, so
// dL/dlogit[t, topk[t, r]] = gate_r (G_r - sum_s gate_s G_s); the others are 0.
__global__ void __launch_bounds__(256) logits_grad_kernel(const double *__restrict__ G,
                                                          const float *__restrict__ gate,
                                                          const int32_t *__restrict__ topk, int T, int X,
                                                          int k, float *__restrict__ d_gate,
                                                          float *__restrict__ d_logits) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  double s = 0.0;
  for (int r = 0; r < k; ++r) s += double(gate[t * k + r]) * G[t * k + r];
  if (d_logits) {
    for (int x = 0; x < X; ++x) d_logits[int64_t(t) * X + x] = 0.f;
    for (int r = 0; r < k; ++r)
      d_logits[int64_t(t) * X + topk[t * k + r]] = float(double(gate[t * k + r]) * (G[t * k + r] - s));
  }
  if (d_gate)
    for (int r = 0; r < k; ++r) d_gate[t * k + r] = float(G[t * k + r]);
}

// ---------------------------------------------------------- readout grad --
// part[chunk][c] = sum over the chunk's atoms of Ebar_b(i) h_i,c + hdot_i,c.
constexpr int RG_ROWS = 64;
__global__ void __launch_bounds__(64) readout_grad_part_kernel(
    const float4 *__restrict__ h, const float4 *hd, const double *Ebar,
    const int32_t *__restrict__ struct_ptr, int B, int N, int D4, float4 *__restrict__ part) {
  const int c = blockIdx.x * 64 + threadIdx.x;
  if (c >= D4) return;
  const int ch = blockIdx.y;
  const int i0 = ch * RG_ROWS, i1 = min(N, i0 + RG_ROWS);
  // structure of atom i0: last b with struct_ptr[b] <= i0
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int m = (lo + hi) >> 1;
    if (struct_ptr[m] <= i0) lo = m;
    else hi = m;
  }
  int b = lo;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i = i0; i < i1; ++i) {
    while (b + 1 < B && struct_ptr[b + 1] <= i) ++b;
    const float lam = Ebar ? float(Ebar[b]) : 0.f;
    const float4 v = h[int64_t(i) * D4 + c];
    acc.x += lam * v.x;
    acc.y += lam * v.y;
    acc.z += lam * v.z;
    acc.w += lam * v.w;
    if (hd) {
      const float4 u = hd[int64_t(i) * D4 + c];
      acc.x += u.x;
      acc.y += u.y;
      acc.z += u.z;
      acc.w += u.w;
    }
  }
  part[int64_t(ch) * D4 + c] = acc;
}

__global__ void __launch_bounds__(256) readout_grad_sum_kernel(const float *__restrict__ part, int n_chunks,
                                                               int D, float *__restrict__ out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= D) return;
  double s = 0.0;
  for (int q = 0; q < n_chunks; ++q) s += double(part[int64_t(q) * D + c]);
  out[c] = float(s);
}

// g_i = Ebar_b(i) w_r (Ebar null: 1), the upstream of the readout for dL/dE = Ebar.
__global__ void __launch_bounds__(256) readout_seed_kernel(const float4 *__restrict__ w,
                                                           const double *Ebar,
                                                           const int32_t *__restrict__ struct_ptr, int B,
                                                           int N, int D4, float4 *__restrict__ g) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= int64_t(N) * D4) return;
  const int i = int(idx / D4), c = int(idx - int64_t(i) * D4);
  float lam = 1.f;
  if (Ebar) {
    int lo = 0, hi = B;   // last b with struct_ptr[b] <= i
    while (hi - lo > 1) {
      const int m = (lo + hi) >> 1;
      if (struct_ptr[m] <= i) lo = m;
      else hi = m;
    }
    lam = float(Ebar[lo]);
  }
  const float4 v = w[c];
  g[idx] = make_float4(lam * v.x, lam * v.y, lam * v.z, lam * v.w);
}

}  // namespace

// ------------------------------------------------------------ launchers ---
int launch_readout_seed(const float *w_r, const double *Ebar, const int32_t *struct_ptr, int N, int B,
                        int D, float *g, hipStream_t stream) {
  ProfScope ps(K_MOE_TAN, stream);
  const int D4 = D / 4;
  readout_seed_kernel<<<dim3(unsigned(cdiv(int64_t(N) * D4, 256))), dim3(256), 0, stream>>>(
      reinterpret_cast<const float4 *>(w_r), Ebar, struct_ptr, B, N, D4, reinterpret_cast<float4 *>(g));
  MLIP_LAUNCHED();
  return MLIP_OK;
}

int64_t wgrad_split_floats(const WgradArgs &a) {
  if (a.group_off) return 0;
  const int64_t tiles = cdiv(a.Mo, WB) * cdiv(a.No, WB);
  const int64_t steps = cdiv(std::max(a.P, 0), WK);
  int64_t ks = std::min<int64_t>(cdiv(1024, tiles), cdiv(steps, 16));
  ks = std::max<int64_t>(ks, 1);
  return ks > 1 ? ks * int64_t(a.Mo) * a.No : 0;
}

int launch_wgrad(const WgradArgs &a, float *split_ws, hipStream_t stream) {
  if (a.Mo <= 0 || a.No <= 0) return MLIP_OK;
  if ((a.Mo & 3) || (a.No & 3) || (a.lda & 3) || (a.ldb & 3)) {
    set_error("weight-gradient dims must be multiples of 4 (Mo=%d No=%d)", a.Mo, a.No);
    return MLIP_ERR_UNSUPPORTED;
  }
  if (a.P > 0 && (a.A1 == nullptr) != (a.B1 == nullptr)) {
    set_error("weight-gradient second term needs both operands");
    return MLIP_ERR_INVALID;
  }
  ProfScope ps(K_GEMM_WGRAD, stream);
  const int64_t tiles = cdiv(a.Mo, WB) * cdiv(a.No, WB);
  const int G = a.group_off ? a.n_groups : 1;
  int ks = 1;
  int64_t rows_per_split = 0;
  if (!a.group_off) {
    const int64_t steps = cdiv(std::max(a.P, 0), WK);
    int64_t k = std::min<int64_t>(cdiv(1024, tiles), cdiv(steps, 16));
    ks = int(std::max<int64_t>(k, 1));
    rows_per_split = cdiv(cdiv(std::max(a.P, 1), ks), WK) * WK;
  }
  if (ks > 1 && !split_ws) {
    set_error("weight-gradient split workspace missing");
    return MLIP_ERR_INVALID;
  }
  const int64_t grid = tiles * G * ks;
  if (grid > int64_t(0x7fffffff)) {
    set_error("weight-gradient GEMM too large for one launch");
    return MLIP_ERR_UNSUPPORTED;
  }
  const int variant = (a.a_rows ? 4 : 0) | (a.b_rows ? 2 : 0) | (a.scale ? 1 : 0);
  const dim3 gd = dim3(unsigned(grid)), bd = dim3(W_THREADS);
  switch (variant) {
    case 0: wgrad_kernel<false, false, false><<<gd, bd, 0, stream>>>(a, ks, rows_per_split, split_ws); break;
    case 1: wgrad_kernel<false, false, true><<<gd, bd, 0, stream>>>(a, ks, rows_per_split, split_ws); break;
    case 2: wgrad_kernel<false, true, false><<<gd, bd, 0, stream>>>(a, ks, rows_per_split, split_ws); break;
    case 3: wgrad_kernel<false, true, true><<<gd, bd, 0, stream>>>(a, ks, rows_per_split, split_ws); break;
    case 4: wgrad_kernel<true, false, false><<<gd, bd, 0, stream>>>(a, ks, rows_per_split, split_ws); break;
    case 5: wgrad_kernel<true, false, true><<<gd, bd, 0, stream>>>(a, ks, rows_per_split, split_ws); break;
    case 6: wgrad_kernel<true, true, false><<<gd, bd, 0, stream>>>(a, ks, rows_per_split, split_ws); break;
    default: wgrad_kernel<true, true, true><<<gd, bd, 0, stream>>>(a, ks, rows_per_split, split_ws); break;
  }
  MLIP_LAUNCHED();
  if (ks > 1) {
    const int64_t n4 = int64_t(a.Mo) * a.No / 4;
    split_sum_kernel<<<dim3(unsigned(cdiv(n4, 256))), dim3(256), 0, stream>>>(
        reinterpret_cast<const float4 *>(split_ws), ks, n4, reinterpret_cast<float4 *>(a.C));
    MLIP_LAUNCHED();
  }
  return MLIP_OK;
}

int edge_tan_groups(int n_atoms) { return std::max(1, std::min(n_atoms, ET_MAX_GROUPS)); }
int64_t edge_tan_part_floats(int n_atoms, int De) {
  const int n = edge_tan_groups(n_atoms);
  return (int64_t(n) + cdiv(n, DWE_SPAN)) * K * De;
}

int launch_edge_tan(const EdgeTanArgs &a, hipStream_t stream) {
  ProfScope ps(K_EDGE_TAN, stream);
  if (a.n_atoms <= 0) {
    if (a.dwe) {   // no rows: a zero W_e gradient
      const int KD = K * a.De;
      dwe_sum_kernel<<<dim3(unsigned(cdiv(KD, 256))), dim3(256), 0, stream>>>(a.dwe_part, 0, KD, a.dwe);
      MLIP_LAUNCHED();
    }
    return MLIP_OK;
  }
  const int n_groups = edge_tan_groups(a.n_atoms);
  const int rows_per = int(cdiv(a.n_atoms, n_groups));
  const int n_slices = int(cdiv(a.De, ET_COLS));
  const int64_t grid = padded_grid(int64_t(n_groups) * n_slices);
  const bool dw = a.R1 != nullptr;
  if (dw && !(a.dwe && a.dwe_part)) {
    set_error("W_e gradient needs its output and partial-sum buffers");
    return MLIP_ERR_INVALID;
  }
  if (a.Y && dw)
    edge_tan_kernel<true, true><<<dim3(unsigned(grid)), dim3(64), 0, stream>>>(a, n_groups, rows_per, n_slices, a.dwe_part);
  else if (a.Y)
    edge_tan_kernel<true, false><<<dim3(unsigned(grid)), dim3(64), 0, stream>>>(a, n_groups, rows_per, n_slices, nullptr);
  else if (dw)
    edge_tan_kernel<false, true><<<dim3(unsigned(grid)), dim3(64), 0, stream>>>(a, n_groups, rows_per, n_slices, a.dwe_part);
  else
    edge_tan_kernel<false, false><<<dim3(unsigned(grid)), dim3(64), 0, stream>>>(a, n_groups, rows_per, n_slices, nullptr);
  MLIP_LAUNCHED();
  if (dw) {
    const int KD = K * a.De;
    const int n2 = int(cdiv(n_groups, DWE_SPAN));
    float *part2 = a.dwe_part + int64_t(n_groups) * KD;
    dwe_stage1_kernel<<<dim3(unsigned(cdiv(KD, 256)), unsigned(n2)), dim3(256), 0, stream>>>(
        a.dwe_part, n_groups, KD, part2);
    MLIP_LAUNCHED();
    dwe_sum_kernel<<<dim3(unsigned(cdiv(KD, 256))), dim3(256), 0, stream>>>(part2, n2, KD, a.dwe);
    MLIP_LAUNCHED();
  }
  return MLIP_OK;
}

int launch_edge_basis_grad(const int32_t *row_ptr, const int32_t *src, const float *geom, int n_atoms,
                           const float *x_dot, float x_sign, const float *X, const float *Y, int D,
                           float rc, float *part, float *dW, hipStream_t stream) {
  ProfScope ps(K_EDGE_TAN, stream);
  const int KD = K * D;
  if (n_atoms <= 0) {
    dwe_sum_kernel<<<dim3(unsigned(cdiv(KD, 256))), dim3(256), 0, stream>>>(part, 0, KD, dW);
    MLIP_LAUNCHED();
    return MLIP_OK;
  }
  const int n_groups = edge_tan_groups(n_atoms);
  const int rows_per = int(cdiv(n_atoms, n_groups));
  const int n_slices = int(cdiv(D, ET_COLS));
  const int64_t grid = padded_grid(int64_t(n_groups) * n_slices);
  edge_basis_grad_kernel<<<dim3(unsigned(grid)), dim3(64), 0, stream>>>(
      row_ptr, src, reinterpret_cast<const float4 *>(geom), n_atoms, x_dot, x_sign, X, Y, D, rc, n_groups,
      rows_per, n_slices, part);
  MLIP_LAUNCHED();
  const int n2 = int(cdiv(n_groups, DWE_SPAN));
  float *part2 = part + int64_t(n_groups) * KD;
  dwe_stage1_kernel<<<dim3(unsigned(cdiv(KD, 256)), unsigned(n2)), dim3(256), 0, stream>>>(part, n_groups, KD,
                                                                                           part2);
  MLIP_LAUNCHED();
  dwe_sum_kernel<<<dim3(unsigned(cdiv(KD, 256))), dim3(256), 0, stream>>>(part2, n2, KD, dW);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

int launch_row_sum(const float *rows, int n, int KD, float *part2, float *out, hipStream_t stream) {
  ProfScope ps(K_EDGE_TAN, stream);
  const int n2 = int(cdiv(std::max(n, 0), DWE_SPAN));
  if (n2 > 0) {
    dwe_stage1_kernel<<<dim3(unsigned(cdiv(KD, 256)), unsigned(n2)), dim3(256), 0, stream>>>(rows, n, KD,
                                                                                             part2);
    MLIP_LAUNCHED();
  }
  dwe_sum_kernel<<<dim3(unsigned(cdiv(KD, 256))), dim3(256), 0, stream>>>(part2, n2, KD, out);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

int launch_moe_tan(const float *P, const float *P_dot, const float *Q, const float *Q_dot, int M, int H,
                   float *act, float *act_dot, float *D, float *D_dot, float *dg, hipStream_t stream) {
  if (M <= 0) return MLIP_OK;
  ProfScope ps(K_MOE_TAN, stream);
  moe_tan_kernel<<<dim3(unsigned(cdiv(M, 4))), dim3(256), 0, stream>>>(
      reinterpret_cast<const float4 *>(P), reinterpret_cast<const float4 *>(P_dot),
      reinterpret_cast<const float4 *>(Q), reinterpret_cast<const float4 *>(Q_dot), M, H / 4,
      reinterpret_cast<float4 *>(act), reinterpret_cast<float4 *>(act_dot), reinterpret_cast<float4 *>(D),
      reinterpret_cast<float4 *>(D_dot), dg);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

int launch_token_gate(const int32_t *z, const float *gate, const int32_t *slot, int N, int T, int k,
                      float *gt, hipStream_t stream) {
  if (N <= 0) return MLIP_OK;
  ProfScope ps(K_MOE_TAN, stream);
  token_gate_kernel<<<dim3(unsigned(cdiv(int64_t(N) * k, 256))), dim3(256), 0, stream>>>(z, gate, slot, N, T,
                                                                                         k, gt);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

int launch_gate_grad(const float *dg, const int32_t *z, const int32_t *topk, const float *gate,
                     const int32_t *exp_off, const int32_t *tok_atom, int T, int X, int k, double *G,
                     float *d_gate, float *d_logits, hipStream_t stream) {
  ProfScope ps(K_MOE_TAN, stream);
  gate_sum_kernel<<<dim3(unsigned(cdiv(int64_t(T) * k, 4))), dim3(256), 0, stream>>>(dg, z, topk, exp_off,
                                                                                     tok_atom, T, k, G);
  MLIP_LAUNCHED();
  logits_grad_kernel<<<dim3(unsigned(cdiv(T, 256))), dim3(256), 0, stream>>>(G, gate, topk, T, X, k, d_gate,
                                                                             d_logits);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

int64_t readout_grad_part_floats(int N, int D) { return cdiv(std::max(N, 1), RG_ROWS) * int64_t(D); }

int launch_readout_grad(const float *h, const float *h_dot, const double *Ebar, const int32_t *struct_ptr,
                        int N, int B, int D, float *part, float *d_w_r, hipStream_t stream) {
  ProfScope ps(K_MOE_TAN, stream);
  const int n_chunks = int(cdiv(std::max(N, 1), RG_ROWS));
  const int D4 = D / 4;
  if (N > 0) {
    readout_grad_part_kernel<<<dim3(unsigned(cdiv(D4, 64)), unsigned(n_chunks)), dim3(64), 0, stream>>>(
        reinterpret_cast<const float4 *>(h), reinterpret_cast<const float4 *>(h_dot), Ebar, struct_ptr, B, N,
        D4, reinterpret_cast<float4 *>(part));
    MLIP_LAUNCHED();
  }
  readout_grad_sum_kernel<<<dim3(unsigned(cdiv(D, 256))), dim3(256), 0, stream>>>(part, N > 0 ? n_chunks : 0,
                                                                                 D, d_w_r);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

}  // namespace mlip
