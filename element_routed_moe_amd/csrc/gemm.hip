// FP32 matrix-core (MFMA) GEMM for gfx950, used for the dense projections
// and, grouped over experts, for the expert MLPs of the mixture of experts
// (paper review of "Breaking the Training Barrier of Billion-Parameter
// Universal MLIPs", section 3.2: sparse MoE layers; Table II widths).
//
//   C[p, :] = epilogue( A[row(p), :] @ B_g )   for p in group g
//
// Groups are contiguous row ranges given by group_off (the expert offsets of
// the dispatch); B_g is the weight matrix of group g, either [K][N] ("NN")
// or [N][K] ("NT", i.e. the transpose is used).  An optional row index
// gathers the A rows (the tokens of each expert) straight from the node
// features, so no dispatched copy of the activations is ever written.
//
// Tiling: BM x BN output tile per 256-thread workgroup of 4 wavefronts in a
// WM x WN grid; each wavefront owns (BM/WM) x (BN/WN) as 32x32 blocks of
// v_mfma_f32_32x32x2_f32.  K advances BK at a time through an S-stage LDS
// ring: each step's A and B tiles are copied from global memory straight into
// LDS (global_load_lds_dwordx4, no register staging), S - 1 steps ahead of
// the step being multiplied, with one barrier per step.  Tiles sit in LDS
// unpadded with XOR-swizzled 16-byte chunks (A and NT-B as [row][k], NN-B as
// [k][n]), so the MFMA fragment reads are free of bank conflicts.  Each MFMA
// lane supplies the k-values k0 + 4*(lane/32) + q, q = 0..3, for four
// consecutive MFMAs, so one 16-byte LDS read feeds four instructions.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs, so each XCD is
// given a contiguous range of tile indices; within it tiles run in groups of
// 8 m-tiles (2 for the expert GEMMs) x all n-tiles, m fastest.  The tiles
// resident on an XCD at one time then share a few A row-blocks and a few
// expert weight tiles in its L2.  Expert row ranges are turned into tile
// ranges once per workgroup.
//
// Expert remainders: an expert's rows past its last whole 128-row block get
// a 32- or 64-row short tile, or, in the paired launch on 128 x 256 tiles,
// join the expert's last full tiles as "tall" 160-row tiles (short tiles
// would stream the expert's weights a second time, cold, at the end).
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace mlip {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int THREADS = 256;
constexpr int N_XCD = 8;
constexpr int RASTER_M = 8;          // dense GEMMs
constexpr int EXPERT_RASTER_M = 2;   // grouped expert GEMMs
constexpr int EXPERT_BK = 16;   // k per pipeline step of the expert GEMMs
constexpr int EXPERT_S = 3;     // LDS stages: 3 x 16 KB, three workgroups per CU
constexpr int MAX_GROUPS = 1024;

// Exclusive scan over the 256 threads of the block (one value each).
__device__ inline int block_scan_excl(int v, int *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wave; ++w) off += red[w];
  return off + x - v;
}

// One BM x BN output tile.  Each k-step's A and B tiles are copied from
// global memory straight into LDS (global_load_lds_dwordx4: every lane moves
// one 16-byte chunk to base + 16*lane), S stages deep, one barrier per step.
// LDS layouts (no padding, XOR-swizzled 16-byte chunks so that MFMA fragment
// reads are free of bank conflicts):
//   A, NT-B: [row][BK], chunk kq of row r stored at kq ^ ((r / (64/BK)) % (BK/4))
//   NN-B:    [k][BN],   4-column chunk c of row k stored at c ^ (8 * ((k/4) & 1))
//
// XR = 32 adds one more block row (rows BM .. BM + 31, "tall" tiles): it is
// split over the four wavefronts by columns, each wave taking the 32-column
// blocks 2*wm and 2*wm + 1 of its own columns, so it reuses the B fragments
// the wave has already read and costs one more A fragment per k group.
template <int BM, int BN, int BK, int WM, int WN, bool BT, int EPI, int S, int AST, int BST, int XR = 0>
__device__ __forceinline__ void gemm_tile(const GemmArgs &g, float *const *As, float *const *Bs,
                                          const float *Bg, int row0, int rows, int n0) {
  static_assert(WM * WN == 4, "four wavefronts");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(XR == 0 || (XR == 32 && WM == 2 && FN % WM == 0), "extra block row layout");
  constexpr int XFN = FN / WM;                      // extra-row blocks per wave
  constexpr int BMA = BM + XR;                      // rows staged in LDS
  constexpr int KQ = BK / 4;                        // 16-byte chunks per row of a k-slice
  constexpr int RPB = 64 / BK;                      // rows per 64-bank line
  // copy instructions per step: one 1 KB chunk-row (64 lanes x 16 bytes) each
  constexpr int NIA = BMA * KQ / 64;
  constexpr int A_LOADS = (NIA + 3) / 4;            // per wave; spare slots copy into a sink
  constexpr int B_LOADS = BN * KQ / THREADS;
  constexpr int NL = A_LOADS + B_LOADS;             // the same on every wave
  static_assert(NIA * 64 == BMA * KQ && B_LOADS >= 1 && BN * KQ % THREADS == 0, "load split");
  static_assert(BMA * BK <= AST && BN * BK <= BST, "LDS stage size");
  static_assert(NIA % 4 == 0 || XR > 0 || (NIA + 1) * 256 <= AST, "room for the A sink");
  static_assert(S >= 2 && S <= 4, "stages");
  static_assert(BT || BN % 64 == 0, "NN-B swizzle needs 64-column multiples");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS copy targets stay scalar
  const int wm = wave / WN, wn = wave % WN;

  // ---- per-lane DMA sources (k offset 0); LDS chunk c = (q*4 + wave)*64 + lane ----
  // When the staged rows do not make a multiple of four chunk-rows, the waves
  // without a chunk-row of their own in the last slot still issue a copy, so
  // that every wave issues the same number and one vmcnt value fits them all:
  // for BM = 32 a copy of chunk-row 0 into the unused LDS just past the tile;
  // for tall tiles a second copy of one of the slot's real chunk-rows onto
  // itself (the same bytes, so the two copies agree whichever lands last).
  const float *a_src[A_LOADS];
  int a_kc[A_LOADS];     // k offset (floats) of this lane's chunk within a step
  int a_dof[A_LOADS];    // LDS offset (floats) of the slot's chunk-row
#pragma unroll
  for (int q = 0; q < A_LOADS; ++q) {
    const int ci = q * 4 + wave;
    const bool real = ci < NIA;
    const int cs = real ? ci : (XR > 0 ? ci - (4 * A_LOADS - NIA) : 0);   // chunk-row copied
    a_dof[q] = (real || XR > 0 ? cs : NIA) * 256;
    const int c = cs * 64 + lane;
    const int r = c / KQ, s = c % KQ;
    a_kc[q] = 4 * (s ^ ((r / RPB) % KQ));
    int p = row0 + r;
    p = p < rows ? p : row0;             // padding rows read a valid row; never stored
    const int64_t arow = g.a_rows ? MLIP_IDX(g.a_rows[p], g.a_row_limit, "gathered row") : int64_t(p);
    a_src[q] = g.A + arow * g.lda;
  }
  const float *b_src[B_LOADS];
  int b_kc[B_LOADS];     // NT: k offset of the chunk; NN: k row of the chunk
#pragma unroll
  for (int q = 0; q < B_LOADS; ++q) {
    const int c = (q * 4 + wave) * 64 + lane;
    if (BT) {
      const int r = c / KQ, s = c % KQ;
      b_kc[q] = 4 * (s ^ ((r / RPB) % KQ));
      int n = n0 + r;
      n = n < g.N ? n : n0;
      b_src[q] = Bg + int64_t(n) * g.ldb;
    } else {
      const int k = c / (BN / 4), s = c % (BN / 4);
      b_kc[q] = k;
      int n = n0 + 4 * (s ^ (8 * ((k >> 2) & 1)));
      n = n < g.N ? n : n0;
      b_src[q] = Bg + n;
    }
  }
  const int nk = (g.K + BK - 1) / BK;
  const bool k_tail = (g.K % BK) != 0;

  auto issue = [&](float *a_dst, float *b_dst, int kt) {
    const int k0 = kt * BK;
    // chunks past K re-read k = 0 (always in range) and are zeroed below
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q) {
      const int k = k0 + a_kc[q];
      __builtin_amdgcn_global_load_lds(MLIP_GLOBAL_PTR(a_src[q] + (k < g.K ? k : 0)), MLIP_LDS_PTR(a_dst + a_dof[q]), 16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q) {
      const int k = k0 + b_kc[q];
      const int64_t off = BT ? int64_t(k < g.K ? k : 0) : int64_t(k < g.K ? k : 0) * g.ldb;
      __builtin_amdgcn_global_load_lds(MLIP_GLOBAL_PTR(b_src[q] + off), MLIP_LDS_PTR(b_dst + (q * 4 + wave) * 256), 16, 0, 0);
    }
  };
  // K tail: after its loads have landed, each lane zeroes the chunks it
  // loaded that lie past K (before the barrier that publishes the stage)
  auto zero_tail = [&](float *a_dst, float *b_dst, int kt) {
    const int k0 = kt * BK;
    const floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q)
      if (k0 + a_kc[q] >= g.K) *reinterpret_cast<floatx4 *>(a_dst + a_dof[q] + lane * 4) = z;
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q)
      if (k0 + b_kc[q] >= g.K) *reinterpret_cast<floatx4 *>(b_dst + ((q * 4 + wave) * 64 + lane) * 4) = z;
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int bi = 0; bi < FM; ++bi)
#pragma unroll
    for (int bj = 0; bj < FN; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.f;
  floatx16 acc_x[XR > 0 ? XFN : 1];   // the extra block row (tall tiles)
#pragma unroll
  for (int e = 0; e < (XR > 0 ? XFN : 1); ++e)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_x[e][r] = 0.f;

  const int l32 = lane & 31;
  const int half = lane >> 5;
  // Per-lane LDS fragment offsets (floats): A row r, logical chunk 2j + half.
  // Every 32-row block starts at a multiple of 32 rows = 8 swizzle periods of
  // RPB rows, so the chunk swizzle depends on the lane alone and the blocks
  // of a wave differ by constant offsets.
  const int xs = half ^ ((l32 / RPB) % KQ);
  const int a_off = (wm * WTM + l32) * BK;
  const int b_off = BT ? (wn * WTN + l32) * BK : (4 * half) * BN + ((wn * WTN + l32) ^ (32 * half));
  struct Frag {
    floatx4 a[FM], b[FN], ax;
  };
  auto read_frag = [&](const float *Ab, const float *Bb, int j, Frag &f) {   // k group 8j .. 8j+7
    const int kx = 4 * ((2 * j) ^ xs);
#pragma unroll
    for (int bi = 0; bi < FM; ++bi)
      f.a[bi] = *reinterpret_cast<const floatx4 *>(&Ab[a_off + bi * 32 * BK + kx]);
    if constexpr (XR > 0) f.ax = *reinterpret_cast<const floatx4 *>(&Ab[(BM + l32) * BK + kx]);
#pragma unroll
    for (int bj = 0; bj < FN; ++bj) {
      if (BT) {
        f.b[bj] = *reinterpret_cast<const floatx4 *>(&Bb[b_off + bj * 32 * BK + kx]);
      } else {
        // column n = wn*WTN + 32*bj + l32 sits at n ^ (32*half) (WTN is a multiple of 64)
        const int col = b_off + 64 * (bj >> 1) + ((bj & 1) ? (half ? -32 : 32) : 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) f.b[bj][q] = Bb[col + (8 * j + q) * BN];
      }
    }
  };
  auto compute = [&](const float *Ab, const float *Bb) {
    Frag f[2];
    read_frag(Ab, Bb, 0, f[0]);
#pragma unroll
    for (int j = 0; j < BK / 8; ++j) {
      // Two fragment buffers let the next k group's reads precede this
      // group's MFMAs; the compiler schedules them (pinning the order with
      // scheduling barriers measured slower).
      if (j + 1 < BK / 8) read_frag(Ab, Bb, j + 1, f[(j + 1) & 1]);
      const Frag &c = f[j & 1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int bi = 0; bi < FM; ++bi)
#pragma unroll
          for (int bj = 0; bj < FN; ++bj)
            acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(c.a[bi][q], c.b[bj][q], acc[bi][bj], 0, 0, 0);
        if constexpr (XR > 0) {
#pragma unroll
          for (int e = 0; e < XFN; ++e) {
            const float bx = wm ? c.b[XFN + e][q] : c.b[e][q];   // block 2*wm + e (WM = 2)
            acc_x[e] = __builtin_amdgcn_mfma_f32_32x32x2f32(c.ax[q], bx, acc_x[e], 0, 0, 0);
          }
        }
      }
    }
  };
  // Step kt reads stage kt % S.  Every step issues the copy of step
  // kt + S - 1 (clamped to the last step: past the end the copy is a dummy
  // into a stage no later step reads), so exactly (S - 2) * NL copies are
  // younger than step kt's at its top, on every path through the loop.
  // The K tail can only be the last step, which the main loop never runs, so
  // the loop carries no tail code (nor the registers of its LDS addresses).
  auto step = [&](auto sc, auto tail, int kt) {
    constexpr int s = decltype(sc)::value;
    wait_vmcnt<(S - 2) * NL>();
    if constexpr (decltype(tail)::value) {
      if (k_tail && kt == nk - 1) zero_tail(As[s], Bs[s], kt);
    }
    lds_barrier();
    issue(As[(s + S - 1) % S], Bs[(s + S - 1) % S], min(kt + S - 1, nk - 1));
    compute(As[s], Bs[s]);
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2 % S>;
  using C3 = std::integral_constant<int, 3 % S>;
  using NoTail = std::false_type;
  using Tail = std::true_type;

  if (nk > 0) {   // K = 0: the product is zero
#pragma unroll
    for (int s = 0; s < S - 1; ++s) issue(As[s], Bs[s], min(s, nk - 1));
    // whole groups of S steps that stop short of the last step (the loop's
    // back edge only follows step S - 1), then the remaining 1 .. S steps,
    // which continue at stage 0
    int kt = 0;
    for (; kt + S < nk; kt += S) {
      step(C0{}, NoTail{}, kt);
      step(C1{}, NoTail{}, kt + 1);
      if constexpr (S >= 3) step(C2{}, NoTail{}, kt + 2);
      if constexpr (S >= 4) step(C3{}, NoTail{}, kt + 3);
    }
    step(C0{}, Tail{}, kt);
    if (kt + 1 < nk) {
      step(C1{}, Tail{}, kt + 1);
      if constexpr (S >= 3) {
        if (kt + 2 < nk) {
          step(C2{}, Tail{}, kt + 2);
          if constexpr (S >= 4) {
            if (kt + 3 < nk) step(C3{}, Tail{}, kt + 3);
          }
        }
      }
    }
    wait_vmcnt<0>();   // no copy may land in LDS after the workgroup ends
  }

  // ---- epilogue: D[row][col], row = 8*(r/4) + 4*(lane/32) + r%4, col = lane%32 ----
  const int kh = half * 4;
  // One 32 x 32 block whose first row is prow.  Residual / pre-activation
  // values are fetched for the whole block first (clamped, always-valid
  // addresses), then combined and stored.
  auto store_block = [&](const floatx16 &v, int prow, int col) {
    const bool col_ok = col < g.N;
    const int colc = col_ok ? col : n0;
    float rv[16];
    if (EPI == EPI_RESID || EPI == EPI_DSILU || EPI == EPI_DSILU_Q || EPI == EPI_TAN) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = prow + 8 * (r >> 2) + kh + (r & 3);
        const int pc = p < rows ? p : row0;
        rv[r] = g.R[int64_t(pc) * g.ldr + colc];
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int p = prow + 8 * (r >> 2) + kh + (r & 3);
      float out, out2 = 0.f;
      if (EPI == EPI_STORE) {
        out = v[r];
      } else if (EPI == EPI_RESID) {
        out = rv[r] + v[r];
      } else if (EPI == EPI_SILU) {
        out = v[r];
        out2 = v[r] * __builtin_amdgcn_rcpf(1.f + __expf(-v[r]));
      } else {
        // silu'(x) = sigmoid(x) (1 + x (1 - sigmoid(x))) at the saved pre-activation
        const float x = rv[r];
        const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-x));
        const float d1 = sg * (1.f + x * (1.f - sg));
        if (EPI == EPI_TAN) {
          out = v[r];
          out2 = v[r] * d1;
        } else {
          out = v[r] * d1;
          out2 = v[r];
        }
      }
      if (col_ok && p < rows) {
        const int64_t o = int64_t(p) * g.ldc + col;
        g.C[o] = out;
        if (EPI == EPI_SILU || EPI == EPI_DSILU_Q || EPI == EPI_TAN) g.C2[o] = out2;
      }
    }
  };
#pragma unroll
  for (int bi = 0; bi < FM; ++bi)
#pragma unroll
    for (int bj = 0; bj < FN; ++bj) store_block(acc[bi][bj], row0 + wm * WTM + bi * 32, n0 + wn * WTN + bj * 32 + l32);
  if constexpr (XR > 0) {
#pragma unroll
    for (int e = 0; e < XFN; ++e) store_block(acc_x[e], row0 + BM, n0 + wn * WTN + (wm * XFN + e) * 32 + l32);
  }
}

// Expert GEMMs (group_off set, SPLIT, BM = 128): each group's rows are
// covered by 128-row tiles, except that a remainder of at most 64 rows gets
// one short tile of 32 or 64 rows (the fewer that cover it), which keeps the
// padded MFMA work of small experts low.  Full and short tiles are dealt to
// the XCDs separately, full tiles first, so every XCD receives its share of
// each and the short tiles run last.
template <int BM, int BN, int BK, int WM, int WN, bool BT, int EPI, int TAG, bool SPLIT, int S>
__global__ void __launch_bounds__(THREADS, 2) gemm_kernel(GemmArgs g) {
  constexpr int AST = BM * BK;
  constexpr int BST = BN * BK;
  constexpr int REM_MAX = BM / 2;   // longest remainder given a short tile
  static_assert(!SPLIT || BM == 128, "short tiles are 32 and 64 rows");
  // one array per stage, so the compiler can tell a stage being read from the
  // stages whose copies are still in flight
  __shared__ __attribute__((aligned(16))) float A0[AST], A1[AST], A2[S >= 3 ? AST : 4], A3[S >= 4 ? AST : 4];
  __shared__ __attribute__((aligned(16))) float B0[BST], B1[BST], B2[S >= 3 ? BST : 4], B3[S >= 4 ? BST : 4];
  float *const As[4] = {A0, A1, A2, A3};
  float *const Bs[4] = {B0, B1, B2, B3};
  // the expert tile map (dense GEMMs have none: their 128 x 64 tiles then
  // fit four workgroups per CU)
  __shared__ int s_tiles[SPLIT ? MAX_GROUPS + 1 : 1];
  __shared__ int s_red[10];   // two scans' wave sums, then the two totals

  const int tid = threadIdx.x;
  const int G = g.group_off ? g.n_groups : 1;
  const int Nt = (g.N + BN - 1) / BN;
  const int L = blockIdx.x;
  const int jx = L / N_XCD, xcd = L - jx * N_XCD;

  // ---- m-tiles per group (full and, with SPLIT, short) -> prefix in LDS ----
  int Mt, t_local, part = 0;
  bool short_tile = false;
  const int ks = (!SPLIT && g.split_ws && g.k_split > 1) ? g.k_split : 1;
  if (SPLIT && g.group_off) {
    constexpr int PER = (MAX_GROUPS + THREADS) / THREADS;   // covers entries 0..MAX_GROUPS
    int cf[PER], ch[PER], sf = 0, sh = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int gi = tid * PER + q;
      const int c = gi < G ? g.group_off[gi + 1] - g.group_off[gi] : 0;
      const int rem = c % BM;
      cf[q] = c / BM + (rem > REM_MAX ? 1 : 0);
      ch[q] = (rem > 0 && rem <= REM_MAX) ? 1 : 0;
      sf += cf[q];
      sh += ch[q];
    }
    int run_f = block_scan_excl(sf, s_red);
    int run_h = block_scan_excl(sh, s_red + 4);
    if (tid == THREADS - 1) {
      s_red[8] = run_f + sf;
      s_red[9] = run_h + sh;
    }
    __syncthreads();
    const int Mf = s_red[8], Mh = s_red[9];
    const int per_f = (Mf * Nt + N_XCD - 1) / N_XCD;
    const int per_h = (Mh * Nt + N_XCD - 1) / N_XCD;
    if (jx < per_f) {
      t_local = xcd * per_f + jx;
      Mt = Mf;
    } else {
      if (jx - per_f >= per_h) return;
      t_local = xcd * per_h + (jx - per_f);
      Mt = Mh;
      short_tile = true;
    }
    if (t_local >= Mt * Nt) return;
    // prefix of this block's class only
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int gi = tid * PER + q;
      if (gi <= G) s_tiles[gi] = short_tile ? run_h : run_f;
      run_f += cf[q];
      run_h += ch[q];
    }
    __syncthreads();
  } else {
    Mt = (g.M + BM - 1) / BM;
    const int per = (Mt * Nt * ks + N_XCD - 1) / N_XCD;
    if (jx >= per) return;
    t_local = xcd * per + jx;
    if (t_local >= Mt * Nt * ks) return;
    part = t_local / (Mt * Nt);
    t_local -= part * (Mt * Nt);
  }
  constexpr int RM = SPLIT ? EXPERT_RASTER_M : RASTER_M;
  const int group_size = RM * Nt;
  const int first_m = (t_local / group_size) * RM;
  const int gm = min(Mt - first_m, RM);
  const int rr = t_local % group_size;
  const int mt_glob = first_m + rr % gm;
  const int nt = rr / gm;

  int grp = 0, row0, rows;
  if (SPLIT && g.group_off) {
    int lo = 0, hi = G;  // last group with s_tiles[grp] <= mt_glob
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_tiles[mid] <= mt_glob) lo = mid;
      else hi = mid;
    }
    grp = lo;
    const int gbeg = g.group_off[grp];
    rows = g.group_off[grp + 1];
    if (short_tile) row0 = gbeg + ((rows - gbeg) / BM) * BM;
    else row0 = gbeg + (mt_glob - s_tiles[grp]) * BM;
  } else {
    row0 = mt_glob * BM;
    rows = g.M;
  }
  const int n0 = nt * BN;
  const float *Bg = g.B + int64_t(grp) * g.b_group_stride;
  if constexpr (SPLIT) {
    if (short_tile) {
      const int rem = rows - row0;
      if (rem <= 32) gemm_tile<32, BN, BK, 1, 4, BT, EPI, S, AST, BST>(g, As, Bs, Bg, row0, rows, n0);
      else gemm_tile<64, BN, BK, 2, 2, BT, EPI, S, AST, BST>(g, As, Bs, Bg, row0, rows, n0);
      return;
    }
  }
  if (!SPLIT && ks > 1) {
    // K part `part`: its raw product goes to split_ws[part]; the parts are
    // summed (with the epilogue) by split_epilogue_kernel
    const int Ks = ((g.K + ks - 1) / ks + BK - 1) / BK * BK;
    const int kb = min(part * Ks, g.K);
    GemmArgs gp = g;
    gp.A = g.A + kb;
    gp.B = BT ? g.B + kb : g.B + int64_t(kb) * g.ldb;
    gp.K = min(g.K - kb, Ks);
    gp.C = g.split_ws + int64_t(part) * g.M * g.N;
    gp.ldc = g.N;
    gemm_tile<BM, BN, BK, WM, WN, BT, EPI_STORE, S, AST, BST>(gp, As, Bs, gp.B, row0, rows, n0);
    return;
  }
  gemm_tile<BM, BN, BK, WM, WN, BT, EPI, S, AST, BST>(g, As, Bs, Bg, row0, rows, n0);
}

// Two independent grouped expert GEMMs over the same expert row ranges (one
// group_off, hence the same m-tiles) in one launch.  Each XCD is dealt the
// full tiles of the first, then those of the second, then the short tiles of
// each, so the second GEMM's tiles fill the slots the first one's last round
// leaves idle and the launch has one tail instead of two.
template <int BN, bool BT1, int EPI1, bool BT2, int EPI2>
__global__ void __launch_bounds__(THREADS, 2) gemm_pair_kernel(GemmArgs g1, GemmArgs g2) {
  constexpr int BM = 128, BK = EXPERT_BK, S = EXPERT_S;
  constexpr int AST = BM * BK;
  constexpr int BST = BN * BK;
  constexpr int REM_MAX = BM / 2;
  __shared__ __attribute__((aligned(16))) float A0[AST], A1[AST], A2[S >= 3 ? AST : 4], A3[S >= 4 ? AST : 4];
  __shared__ __attribute__((aligned(16))) float B0[BST], B1[BST], B2[S >= 3 ? BST : 4], B3[S >= 4 ? BST : 4];
  float *const As[4] = {A0, A1, A2, A3};
  float *const Bs[4] = {B0, B1, B2, B3};
  __shared__ int s_tiles[MAX_GROUPS + 1];
  __shared__ int s_red[10];

  const int tid = threadIdx.x;
  const int G = g1.n_groups;
  const int Nt1 = (g1.N + BN - 1) / BN, Nt2 = (g2.N + BN - 1) / BN;
  const int L = blockIdx.x;
  const int jx = L / N_XCD, xcd = L - jx * N_XCD;

  constexpr int PER = (MAX_GROUPS + THREADS) / THREADS;
  int cf[PER], ch[PER], sf = 0, sh = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int gi = tid * PER + q;
    const int c = gi < G ? g1.group_off[gi + 1] - g1.group_off[gi] : 0;
    const int rem = c % BM;
    cf[q] = c / BM + (rem > REM_MAX ? 1 : 0);
    ch[q] = (rem > 0 && rem <= REM_MAX) ? 1 : 0;
    sf += cf[q];
    sh += ch[q];
  }
  int run_f = block_scan_excl(sf, s_red);
  int run_h = block_scan_excl(sh, s_red + 4);
  if (tid == THREADS - 1) {
    s_red[8] = run_f + sf;
    s_red[9] = run_h + sh;
  }
  __syncthreads();
  const int Mf = s_red[8], Mh = s_red[9];
  const int per_f1 = (Mf * Nt1 + N_XCD - 1) / N_XCD, per_f2 = (Mf * Nt2 + N_XCD - 1) / N_XCD;
  const int per_h1 = (Mh * Nt1 + N_XCD - 1) / N_XCD, per_h2 = (Mh * Nt2 + N_XCD - 1) / N_XCD;
  int second, t_local, Mt, Nt;
  bool short_tile;
  if (jx < per_f1) {
    second = 0; short_tile = false; t_local = xcd * per_f1 + jx;
  } else if (jx < per_f1 + per_f2) {
    second = 1; short_tile = false; t_local = xcd * per_f2 + (jx - per_f1);
  } else if (jx < per_f1 + per_f2 + per_h1) {
    second = 0; short_tile = true; t_local = xcd * per_h1 + (jx - per_f1 - per_f2);
  } else {
    second = 1; short_tile = true; t_local = xcd * per_h2 + (jx - per_f1 - per_f2 - per_h1);
    if (jx - per_f1 - per_f2 - per_h1 >= per_h2) return;
  }
  Mt = short_tile ? Mh : Mf;
  Nt = second ? Nt2 : Nt1;
  if (t_local >= Mt * Nt) return;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int gi = tid * PER + q;
    if (gi <= G) s_tiles[gi] = short_tile ? run_h : run_f;
    run_f += cf[q];
    run_h += ch[q];
  }
  __syncthreads();
  constexpr int RM = EXPERT_RASTER_M;
  const int group_size = RM * Nt;
  const int first_m = (t_local / group_size) * RM;
  const int gm = min(Mt - first_m, RM);
  const int rr = t_local % group_size;
  const int mt_glob = first_m + rr % gm;
  const int nt = rr / gm;
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_tiles[mid] <= mt_glob) lo = mid;
    else hi = mid;
  }
  const int grp = lo;
  const int gbeg = g1.group_off[grp];
  const int rows = g1.group_off[grp + 1];
  const int row0 = short_tile ? gbeg + ((rows - gbeg) / BM) * BM : gbeg + (mt_glob - s_tiles[grp]) * BM;
  const int n0 = nt * BN;
  if (second) {
    const float *Bg = g2.B + int64_t(grp) * g2.b_group_stride;
    if (!short_tile) gemm_tile<BM, BN, BK, 2, 2, BT2, EPI2, S, AST, BST>(g2, As, Bs, Bg, row0, rows, n0);
    else if (rows - row0 <= 32) gemm_tile<32, BN, BK, 1, 4, BT2, EPI2, S, AST, BST>(g2, As, Bs, Bg, row0, rows, n0);
    else gemm_tile<64, BN, BK, 2, 2, BT2, EPI2, S, AST, BST>(g2, As, Bs, Bg, row0, rows, n0);
  } else {
    const float *Bg = g1.B + int64_t(grp) * g1.b_group_stride;
    if (!short_tile) gemm_tile<BM, BN, BK, 2, 2, BT1, EPI1, S, AST, BST>(g1, As, Bs, Bg, row0, rows, n0);
    else if (rows - row0 <= 32) gemm_tile<32, BN, BK, 1, 4, BT1, EPI1, S, AST, BST>(g1, As, Bs, Bg, row0, rows, n0);
    else gemm_tile<64, BN, BK, 2, 2, BT1, EPI1, S, AST, BST>(g1, As, Bs, Bg, row0, rows, n0);
  }
}

// Tile classes of one expert of c rows for the tall paired launch: f full
// 128-row tiles, then t tall tiles (128 rows plus up to 32 more), or h short
// tiles (32 or 64 rows) when the remainder cannot join a full tile.  A
// remainder of at most 32 rows joins the last full tile, one of 33 to 64
// rows is split over the last two (the first takes the larger half), and
// one of more than 64 rows gets a padded full tile.
__device__ inline void tall_classes(int c, int &f, int &t, int &h) {
  const int m = c / 128, rem = c % 128;
  f = m;
  t = 0;
  h = 0;
  if (rem == 0) return;
  if (rem > 64) {
    f = m + 1;
  } else if (rem <= 32 && m >= 1) {
    f = m - 1;
    t = 1;
  } else if (rem > 32 && m >= 2) {
    f = m - 2;
    t = 2;
  } else {
    h = 1;
  }
}

// Two independent grouped expert GEMMs over the same expert row ranges on
// 128 x 256 tiles, with each expert's short remainder folded into tall
// tiles, which read the weight columns their full rows read anyway.  Each
// XCD is dealt, in turn, its share of the full tiles of the first GEMM and
// of the second, then of the tall tiles of each, then of the short tiles of
// each (experts of at most 64 rows, or of 161 to 192).  The expert of a
// tile is found by the thread whose groups hold it (no tile map in LDS, so
// two workgroups fit per CU with 160-row A stages).
template <bool BT1, int EPI1, bool BT2, int EPI2>
__global__ void __launch_bounds__(THREADS, 2) gemm_pair_tall_kernel(GemmArgs g1, GemmArgs g2) {
  constexpr int BM = 128, BN = 256, BK = EXPERT_BK, S = EXPERT_S, XR = 32;
  constexpr int AST = (BM + XR) * BK;
  constexpr int BST = BN * BK;
  __shared__ __attribute__((aligned(16))) float A0[AST], A1[AST], A2[S >= 3 ? AST : 4], A3[S >= 4 ? AST : 4];
  __shared__ __attribute__((aligned(16))) float B0[BST], B1[BST], B2[S >= 3 ? BST : 4], B3[S >= 4 ? BST : 4];
  float *const As[4] = {A0, A1, A2, A3};
  float *const Bs[4] = {B0, B1, B2, B3};
  __shared__ int s_red[16];   // three scans' wave sums, then the three totals
  __shared__ int s_hit[2];    // the tile's expert and its index among the expert's tiles of its class

  const int tid = threadIdx.x;
  const int G = g1.n_groups;
  const int Nt1 = (g1.N + BN - 1) / BN, Nt2 = (g2.N + BN - 1) / BN;
  const int L = blockIdx.x;
  const int jx = L / N_XCD, xcd = L - jx * N_XCD;

  constexpr int PER = MAX_GROUPS / THREADS;   // groups tid*PER .. tid*PER + PER - 1
  int cn[3][PER], sum[3] = {0, 0, 0};
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int gi = tid * PER + q;
    const int c = gi < G ? g1.group_off[gi + 1] - g1.group_off[gi] : 0;
    tall_classes(c, cn[0][q], cn[1][q], cn[2][q]);
#pragma unroll
    for (int k = 0; k < 3; ++k) sum[k] += cn[k][q];
  }
  int run[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) run[k] = block_scan_excl(sum[k], s_red + 4 * k);
  if (tid == THREADS - 1) {
#pragma unroll
    for (int k = 0; k < 3; ++k) s_red[12 + k] = run[k] + sum[k];
  }
  __syncthreads();
  const int Mc[3] = {s_red[12], s_red[13], s_red[14]};   // full, tall and short m-tiles
  // the six classes in dealing order: (tile class, which GEMM)
  int cls = -1, second = 0, t_local = 0, Nt = Nt1, base = 0;
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const int kc = k >> 1, kg = k & 1;
    const int nt_k = kg ? Nt2 : Nt1;
    const int per = (Mc[kc] * nt_k + N_XCD - 1) / N_XCD;
    if (cls < 0 && jx < base + per) {
      cls = kc;
      second = kg;
      Nt = nt_k;
      t_local = xcd * per + (jx - base);
    }
    base += per;
  }
  if (cls < 0 || t_local >= (cls == 0 ? Mc[0] : cls == 1 ? Mc[1] : Mc[2]) * Nt) return;
  constexpr int RM = EXPERT_RASTER_M;
  const int Mt = cls == 0 ? Mc[0] : cls == 1 ? Mc[1] : Mc[2];
  const int group_size = RM * Nt;
  const int first_m = (t_local / group_size) * RM;
  const int gm = min(Mt - first_m, RM);
  const int rr = t_local % group_size;
  const int mt_glob = first_m + rr % gm;
  const int nt = rr / gm;
  // the one group whose class range holds mt_glob
  {
    int pre = cls == 0 ? run[0] : cls == 1 ? run[1] : run[2];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int cq = cls == 0 ? cn[0][q] : cls == 1 ? cn[1][q] : cn[2][q];
      if (mt_glob >= pre && mt_glob < pre + cq) {
        s_hit[0] = tid * PER + q;
        s_hit[1] = mt_glob - pre;
      }
      pre += cq;
    }
  }
  __syncthreads();
  const int grp = s_hit[0], sub = s_hit[1];
  const int gbeg = g1.group_off[grp], gend = g1.group_off[grp + 1];
  int f, t, h;
  tall_classes(gend - gbeg, f, t, h);
  const int rem = (gend - gbeg) % BM;
  int row0, rows = gend;
  if (cls == 0) {
    row0 = gbeg + sub * BM;
  } else if (cls == 1) {
    row0 = gbeg + f * BM;
    if (t == 2) {
      const int r1 = (rem + 1) / 2;
      if (sub == 0) rows = row0 + BM + r1;
      else row0 += BM + r1;
    }
  } else {
    row0 = gbeg + f * BM;
  }
  const int n0 = nt * BN;
  if (second) {
    const float *Bg = g2.B + int64_t(grp) * g2.b_group_stride;
    if (cls == 0) gemm_tile<BM, BN, BK, 2, 2, BT2, EPI2, S, AST, BST>(g2, As, Bs, Bg, row0, rows, n0);
    else if (cls == 1) gemm_tile<BM, BN, BK, 2, 2, BT2, EPI2, S, AST, BST, XR>(g2, As, Bs, Bg, row0, rows, n0);
    else if (rows - row0 <= 32) gemm_tile<32, BN, BK, 1, 4, BT2, EPI2, S, AST, BST>(g2, As, Bs, Bg, row0, rows, n0);
    else gemm_tile<64, BN, BK, 2, 2, BT2, EPI2, S, AST, BST>(g2, As, Bs, Bg, row0, rows, n0);
  } else {
    const float *Bg = g1.B + int64_t(grp) * g1.b_group_stride;
    if (cls == 0) gemm_tile<BM, BN, BK, 2, 2, BT1, EPI1, S, AST, BST>(g1, As, Bs, Bg, row0, rows, n0);
    else if (cls == 1) gemm_tile<BM, BN, BK, 2, 2, BT1, EPI1, S, AST, BST, XR>(g1, As, Bs, Bg, row0, rows, n0);
    else if (rows - row0 <= 32) gemm_tile<32, BN, BK, 1, 4, BT1, EPI1, S, AST, BST>(g1, As, Bs, Bg, row0, rows, n0);
    else gemm_tile<64, BN, BK, 2, 2, BT1, EPI1, S, AST, BST>(g1, As, Bs, Bg, row0, rows, n0);
  }
}

// C = (R +) the sum of the k_split parts in split_ws, in part order.
template <bool RESID>
__global__ void __launch_bounds__(256) split_epilogue_kernel(const float4 *__restrict__ part, int ks, int64_t mn4,
                                                             int n4, const float *__restrict__ R, int64_t ldr,
                                                             float *__restrict__ C, int64_t ldc) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= mn4) return;
  const int64_t m = i / n4;
  const int c = int(i - m * n4) * 4;
  float4 v = part[i];
  for (int q = 1; q < ks; ++q) {
    const float4 t = part[int64_t(q) * mn4 + i];
    v.x += t.x;
    v.y += t.y;
    v.z += t.z;
    v.w += t.w;
  }
  if (RESID) {
    const float4 r = *reinterpret_cast<const float4 *>(R + m * ldr + c);
    v.x += r.x;
    v.y += r.y;
    v.z += r.z;
    v.w += r.w;
  }
  *reinterpret_cast<float4 *>(C + m * ldc + c) = v;
}

template <int BM, int BN, int BK, int WM, int WN, bool BT, int EPI, int TAG, bool SPLIT, int S>
int launch_t(const GemmArgs &a, hipStream_t stream) {
  // Upper bounds of the per-XCD tile counts the kernel derives on the device:
  // full tiles <= (M + G*(BM/2 - 1)) / BM and short tiles <= G for grouped
  // (expert) GEMMs; surplus workgroups return at once.
  const int64_t nt = cdiv(a.N, BN);
  int64_t per;
  if (!SPLIT && a.group_off) {
    set_error("grouped GEMMs take the expert tiles");
    return MLIP_ERR_UNSUPPORTED;
  }
  if (!a.group_off) {
    const int64_t ks = (!SPLIT && a.split_ws && a.k_split > 1) ? a.k_split : 1;
    per = cdiv(cdiv(a.M, BM) * nt * ks, N_XCD);
  } else {
    const int64_t mf = (int64_t(a.M) + int64_t(a.n_groups) * (BM / 2 - 1)) / BM;
    per = cdiv(mf * nt, N_XCD) + cdiv(int64_t(a.n_groups) * nt, N_XCD);
  }
  const int64_t grid = per * N_XCD;
  if (grid <= 0) return MLIP_OK;
  if (grid > int64_t(0x7fffffff)) {
    set_error("GEMM too large for one launch");
    return MLIP_ERR_UNSUPPORTED;
  }
  gemm_kernel<BM, BN, BK, WM, WN, BT, EPI, TAG, SPLIT, S><<<dim3(unsigned(grid)), dim3(THREADS), 0, stream>>>(a);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

// Expert GEMMs: 128 x 128 tiles, 64 x 128 for short group remainders.
template <bool BT, int EPI, int TAG>
int launch_expert(const GemmArgs &a, hipStream_t s) {
  return launch_t<128, 128, EXPERT_BK, 2, 2, BT, EPI, TAG, true, EXPERT_S>(a, s);
}
// Dense projections: 128 x 64 tiles (two 32 x 32 blocks per wave) with the
// expert GEMMs' 16-deep, 3-stage ring; narrow outputs split their K loop.
template <bool BT, int EPI, int TAG>
int launch_dense(const GemmArgs &a, hipStream_t s) {
  static_assert(EPI == EPI_STORE || EPI == EPI_RESID, "dense epilogues");
  const bool split = a.split_ws && a.k_split > 1;
  int rc = launch_t<128, 64, EXPERT_BK, 2, 2, BT, EPI, TAG, false, EXPERT_S>(a, s);
  if (rc || !split) return rc;
  if ((a.ldc & 3) || (EPI == EPI_RESID && (a.ldr & 3))) {
    set_error("split-K GEMM needs ldc and ldr multiples of 4");
    return MLIP_ERR_UNSUPPORTED;
  }
  const int64_t mn4 = int64_t(a.M) * a.N / 4;
  const dim3 grid(unsigned(cdiv(mn4, 256)));
  split_epilogue_kernel<EPI == EPI_RESID><<<grid, dim3(256), 0, s>>>(
      reinterpret_cast<const float4 *>(a.split_ws), a.k_split, mn4, a.N / 4, a.R, a.ldr, a.C, a.ldc);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

template <int BN, bool BT1, int EPI1, bool BT2, int EPI2>
int launch_pair_t(const GemmArgs &a, const GemmArgs &b, hipStream_t stream) {
  // upper bounds of the per-XCD tile counts the kernel derives on the device
  const int64_t mf = (int64_t(a.M) + int64_t(a.n_groups) * 63) / 128;
  const int64_t nt1 = cdiv(a.N, BN), nt2 = cdiv(b.N, BN);
  const int64_t per = cdiv(mf * nt1, N_XCD) + cdiv(mf * nt2, N_XCD) + cdiv(int64_t(a.n_groups) * nt1, N_XCD) +
                      cdiv(int64_t(a.n_groups) * nt2, N_XCD);
  const int64_t grid = per * N_XCD;
  if (grid <= 0) return MLIP_OK;
  if (grid > int64_t(0x7fffffff)) {
    set_error("GEMM pair too large for one launch");
    return MLIP_ERR_UNSUPPORTED;
  }
  gemm_pair_kernel<BN, BT1, EPI1, BT2, EPI2><<<dim3(unsigned(grid)), dim3(THREADS), 0, stream>>>(a, b);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

template <bool BT1, int EPI1, bool BT2, int EPI2>
int launch_pair_tall_t(const GemmArgs &a, const GemmArgs &b, hipStream_t stream) {
  // upper bounds of the per-XCD tile counts the kernel derives on the device:
  // full tiles <= (M + G*63) / 128, tall tiles <= 2G, short tiles <= G
  const int64_t G = a.n_groups;
  const int64_t mc[3] = {(int64_t(a.M) + G * 63) / 128, 2 * G, G};
  const int64_t nt1 = cdiv(a.N, 256), nt2 = cdiv(b.N, 256);
  int64_t per = 0;
  for (int k = 0; k < 3; ++k) per += cdiv(mc[k] * nt1, N_XCD) + cdiv(mc[k] * nt2, N_XCD);
  const int64_t grid = per * N_XCD;
  if (grid <= 0) return MLIP_OK;
  if (grid > int64_t(0x7fffffff)) {
    set_error("GEMM pair too large for one launch");
    return MLIP_ERR_UNSUPPORTED;
  }
  gemm_pair_tall_kernel<BT1, EPI1, BT2, EPI2><<<dim3(unsigned(grid)), dim3(THREADS), 0, stream>>>(a, b);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

}  // namespace

// A dense output with few tiles leaves CUs idle (or a partly filled last
// round of workgroups) for the whole K loop.  Splitting K into ks parts turns
// one tile into ks shorter ones; the count is the one (up to 4, parts of at
// least 256) that minimises rounds(ks) / ks, the K loops' duration in units of
// the unsplit loop, plus a tenth for the summing pass, where rounds(ks) is
// the number of rounds of resident workgroups (four 128 x 64 tiles per CU)
// the tiles take.  Outputs of two rounds or more are not split.
int dense_k_split(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K < 512) return 1;
  const int64_t tiles = cdiv(M, 128) * cdiv(N, 64);
  const int64_t slots = 256 * 4;
  if (tiles >= 2 * slots) return 1;
  int best = 1;
  double best_cost = double(cdiv(tiles, slots));
  for (int ks = 2; ks <= 4 && K / ks >= 256; ++ks) {
    const double cost = double(cdiv(tiles * ks, slots)) / ks + 0.1;
    if (cost < best_cost - 1e-9) {
      best = ks;
      best_cost = cost;
    }
  }
  return best;
}
int64_t dense_split_floats(int64_t M, int64_t N, int64_t K) {
  const int ks = dense_k_split(M, N, K);
  return ks > 1 ? int64_t(ks) * M * N : 0;
}
int64_t dense_split_floats_max(int64_t M, int64_t N) { return dense_split_floats(M, N, int64_t(1) << 30); }

int launch_expert_pair(const GemmArgs &a, bool bt_a, Epilogue epi_a, const GemmArgs &b, bool bt_b,
                       Epilogue epi_b, KClass cls, hipStream_t stream) {
  if (a.M <= 0) return MLIP_OK;
  if (!a.group_off || a.group_off != b.group_off || a.n_groups != b.n_groups || a.M != b.M) {
    set_error("a GEMM pair must share its expert row ranges");
    return MLIP_ERR_INVALID;
  }
  for (const GemmArgs *g : {&a, &b}) {
    if ((g->K & 3) || (g->N & 3) || (g->lda & 3) || (g->ldb & 3) || g->N <= 0) {
      set_error("GEMM dims must be multiples of 4 (K=%d N=%d)", g->K, g->N);
      return MLIP_ERR_UNSUPPORTED;
    }
  }
  if (a.n_groups > MAX_GROUPS) {
    set_error("at most %d expert groups", MAX_GROUPS);
    return MLIP_ERR_UNSUPPORTED;
  }
  ProfScope ps(cls, stream);
  // Y = silu(P) W2 (forward) with Q = (g W2^T) silu'(P) (gradient), with or without saving g W2^T.
  // Widths that are multiples of 256 take 128 x 256 tiles, two workgroups per CU (the S, M and
  // share widths: at S the pair's 2560 full tiles are then exactly 5 rounds); others 128 x 128.
  const bool wide = a.N % 256 == 0 && b.N % 256 == 0;
  if (!bt_a && epi_a == EPI_STORE && bt_b && epi_b == EPI_DSILU)
    return wide ? launch_pair_tall_t<false, EPI_STORE, true, EPI_DSILU>(a, b, stream)
                : launch_pair_t<128, false, EPI_STORE, true, EPI_DSILU>(a, b, stream);
  if (!bt_a && epi_a == EPI_STORE && bt_b && epi_b == EPI_DSILU_Q)
    return wide ? launch_pair_tall_t<false, EPI_STORE, true, EPI_DSILU_Q>(a, b, stream)
                : launch_pair_t<128, false, EPI_STORE, true, EPI_DSILU_Q>(a, b, stream);
  set_error("unsupported GEMM pair");
  return MLIP_ERR_INVALID;
}

int launch_gemm(const GemmArgs &a, bool bt, Epilogue epi, KClass cls, hipStream_t stream) {
  if (a.M <= 0 || a.N <= 0) return MLIP_OK;
  if ((a.K & 3) || (a.N & 3) || (a.lda & 3) || (a.ldb & 3)) {
    set_error("GEMM dims must be multiples of 4 (K=%d N=%d)", a.K, a.N);
    return MLIP_ERR_UNSUPPORTED;
  }
  if (a.group_off && a.n_groups > MAX_GROUPS) {
    set_error("at most %d expert groups", MAX_GROUPS);
    return MLIP_ERR_UNSUPPORTED;
  }
  ProfScope ps(cls, stream);
  switch (cls) {
    case K_GEMM_EXPERT_UP:
      if (!bt && epi == EPI_SILU) return launch_expert<false, EPI_SILU, K_GEMM_EXPERT_UP>(a, stream);
      break;
    case K_GEMM_EXPERT_DOWN:
      if (!bt && epi == EPI_STORE) return launch_expert<false, EPI_STORE, K_GEMM_EXPERT_DOWN>(a, stream);
      break;
    case K_GEMM_EXPERT_VJP_DOWN:
      if (bt && epi == EPI_DSILU) return launch_expert<true, EPI_DSILU, K_GEMM_EXPERT_VJP_DOWN>(a, stream);
      if (bt && epi == EPI_DSILU_Q) return launch_expert<true, EPI_DSILU_Q, K_GEMM_EXPERT_VJP_DOWN>(a, stream);
      break;
    case K_GEMM_EXPERT_TAN:
      if (!bt && epi == EPI_TAN) return launch_expert<false, EPI_TAN, K_GEMM_EXPERT_TAN>(a, stream);
      if (!bt && epi == EPI_STORE) return launch_expert<false, EPI_STORE, K_GEMM_EXPERT_TAN>(a, stream);
      if (bt && epi == EPI_STORE) return launch_expert<true, EPI_STORE, K_GEMM_EXPERT_TAN>(a, stream);
      break;
    case K_GEMM_EXPERT_VJP_UP:
      if (bt && epi == EPI_STORE) return launch_expert<true, EPI_STORE, K_GEMM_EXPERT_VJP_UP>(a, stream);
      break;
    case K_GEMM_DENSE:
      if (!bt && epi == EPI_STORE) return launch_dense<false, EPI_STORE, K_GEMM_DENSE>(a, stream);
      if (!bt && epi == EPI_RESID) return launch_dense<false, EPI_RESID, K_GEMM_DENSE>(a, stream);
      if (bt && epi == EPI_STORE) return launch_dense<true, EPI_STORE, K_GEMM_DENSE>(a, stream);
      if (bt && epi == EPI_RESID) return launch_dense<true, EPI_RESID, K_GEMM_DENSE>(a, stream);
      break;
    default:
      break;
  }
  set_error("unsupported GEMM variant (class %d, transposed %d, epilogue %d)", int(cls), int(bt),
            int(epi));
  return MLIP_ERR_INVALID;
}

}  // namespace mlip
