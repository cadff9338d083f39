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
// v_mfma_f32_32x32x2_f32.  K advances BK at a time through double-buffered
// LDS with one barrier per step; the next step's global loads are in flight
// while the current one is multiplied, and are written to the other LDS
// buffer halfway through the step's multiplies.  A and NT-B tiles sit in LDS as
// [row][k] (k contiguous, row stride BK+4 floats: 16-byte reads without bank
// conflicts); NN-B tiles as [k][n].  Each MFMA lane supplies the k-values
// k0 + 4*(lane/32) + q, q = 0..3, for four consecutive MFMAs, so one 16-byte
// LDS read feeds four instructions.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs, so each XCD is
// given a contiguous range of tile indices; within it tiles run in groups of
// 8 m-tiles x all n-tiles, m fastest.  The tiles resident on an XCD at one
// time then share a few A row-blocks and a few expert weight tiles in its L2.
// Expert row ranges are turned into tile ranges once per workgroup in LDS.
#include <algorithm>

#include "common.h"

namespace mlip {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int THREADS = 256;
constexpr int N_XCD = 8;
constexpr int RASTER_M = 8;
constexpr int EXPERT_BK_NN = 16;   // [K][N] weights: 41 KB of LDS, three workgroups per CU
constexpr int EXPERT_BK_NT = 32;   // [N][K] weights: 75-78 KB of LDS, two per CU (measured faster)
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

// One BM x BN output tile: rows [row0, min(row0 + BM, rows)) of the A row
// space, columns [n0, n0 + BN).  As / Bs are the two LDS stages, AST / BST
// floats apart.
template <int BM, int BN, int BK, int WM, int WN, bool BT, int EPI, int AST, int BST>
__device__ __forceinline__ void gemm_tile(const GemmArgs &g, float *As_, float *Bs_, const float *Bg,
                                          int row0, int rows, int n0) {
  static_assert(WM * WN == 4, "four wavefronts");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  constexpr int LDK = BK + 4;
  constexpr int LDN = BN + 4;
  constexpr int KQ = BK / 4;                       // float4 per row of a k-slice
  constexpr int A_LOADS = BM * KQ / THREADS;
  constexpr int B_LOADS = BN * KQ / THREADS;
  static_assert(A_LOADS >= 1 && B_LOADS >= 1 && BM * KQ % THREADS == 0 && BN * KQ % THREADS == 0,
                "load split");
  static_assert(BM * LDK <= AST && (BT ? BN * LDK : BK * LDN) <= BST, "LDS stage size");
  typedef float AStage[AST];
  typedef float BStage[BST];
  AStage *As = reinterpret_cast<AStage *>(As_);
  BStage *Bs = reinterpret_cast<BStage *>(Bs_);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- per-thread global load assignments ----
  const float *a_src[A_LOADS];
  bool a_ok[A_LOADS];
  int a_row[A_LOADS], a_kq[A_LOADS];
#pragma unroll
  for (int q = 0; q < A_LOADS; ++q) {
    const int idx = tid + THREADS * q;
    a_row[q] = idx / KQ;
    a_kq[q] = (idx % KQ) * 4;
    const int p = row0 + a_row[q];
    a_ok[q] = p < rows;
    int64_t arow = p;
    if (a_ok[q] && g.a_rows) arow = g.a_rows[p];
    a_src[q] = g.A + (a_ok[q] ? arow * g.lda : 0);
  }
  const float *b_src[B_LOADS];
  bool b_ok[B_LOADS];
  int b_r[B_LOADS], b_c[B_LOADS];
#pragma unroll
  for (int q = 0; q < B_LOADS; ++q) {
    const int idx = tid + THREADS * q;
    if (BT) {   // [N][K]: row n, float4 along k
      b_r[q] = idx / KQ;
      b_c[q] = (idx % KQ) * 4;
      const int n = n0 + b_r[q];
      b_ok[q] = n < g.N;
      b_src[q] = Bg + (b_ok[q] ? int64_t(n) * g.ldb : 0);
    } else {    // [K][N]: row k, float4 along n
      b_r[q] = idx / (BN / 4);
      b_c[q] = (idx % (BN / 4)) * 4;
      const int n = n0 + b_c[q];
      b_ok[q] = n < g.N;
      b_src[q] = Bg + (b_ok[q] ? n : 0);
    }
  }

  // Loads are unconditional from always-valid addresses (row 0 / k 0 stand in
  // for out-of-range elements); the zero mask is applied when the values are
  // written to LDS, so nothing waits on a load before the multiply.
  floatx4 ra[A_LOADS], rb[B_LOADS];
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  auto a_ok_k = [&](int q, int k0) { return a_ok[q] && k0 + a_kq[q] < g.K; };
  auto b_ok_k = [&](int q, int k0) { return b_ok[q] && k0 + (BT ? b_c[q] : b_r[q]) < g.K; };
  auto load_global = [&](int k0) {
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q) {
      const int k = k0 + a_kq[q];
      ra[q] = *reinterpret_cast<const floatx4 *>(a_src[q] + (a_ok_k(q, k0) ? k : 0));
    }
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q) {
      if (BT) {
        const int k = k0 + b_c[q];
        rb[q] = *reinterpret_cast<const floatx4 *>(b_src[q] + (b_ok_k(q, k0) ? k : 0));
      } else {
        const int kb = k0 + b_r[q];
        rb[q] = *reinterpret_cast<const floatx4 *>(b_src[q] + (b_ok_k(q, k0) ? int64_t(kb) * g.ldb : 0));
      }
    }
  };
  auto store_lds = [&](int buf, int k0) {
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q)
      *reinterpret_cast<floatx4 *>(&As[buf][a_row[q] * LDK + a_kq[q]]) = a_ok_k(q, k0) ? ra[q] : zero4;
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q) {
      const floatx4 v = b_ok_k(q, k0) ? rb[q] : zero4;
      if (BT) *reinterpret_cast<floatx4 *>(&Bs[buf][b_r[q] * LDK + b_c[q]]) = v;
      else *reinterpret_cast<floatx4 *>(&Bs[buf][b_r[q] * LDN + b_c[q]]) = v;
    }
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int bi = 0; bi < FM; ++bi)
#pragma unroll
    for (int bj = 0; bj < FN; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.f;

  const int nk = (g.K + BK - 1) / BK;
  load_global(0);
  store_lds(0, 0);
  __syncthreads();

  const int l32 = lane & 31;
  const int kh = (lane >> 5) * 4;
  // fragments of one 8-wide k group: FM A-values and FN B-values per k
  struct Frag {
    floatx4 a[FM], b[FN];
  };
  auto read_frag = [&](const float *Ab, const float *Bb, int kg, Frag &f) {
#pragma unroll
    for (int bi = 0; bi < FM; ++bi)
      f.a[bi] = *reinterpret_cast<const floatx4 *>(&Ab[(wm * WTM + bi * 32 + l32) * LDK + kg + kh]);
#pragma unroll
    for (int bj = 0; bj < FN; ++bj) {
      if (BT) {
        f.b[bj] = *reinterpret_cast<const floatx4 *>(&Bb[(wn * WTN + bj * 32 + l32) * LDK + kg + kh]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) f.b[bj][q] = Bb[(kg + kh + q) * LDN + wn * WTN + bj * 32 + l32];
      }
    }
  };
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_global((kt + 1) * BK);
    const float *Ab = As[cur];
    const float *Bb = Bs[cur];
    Frag f[2];
    read_frag(Ab, Bb, 0, f[0]);
    // [N][K] weights: the multiplying wave takes issue priority over the
    // other wave of its SIMD while that one loads and stores (measured faster
    // there; the [K][N] variant is not helped)
    if constexpr (BT) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kg = 0; kg < BK / 8; ++kg) {
      // the next group's LDS reads are in flight while this group multiplies
      if (kg + 1 < BK / 8) read_frag(Ab, Bb, (kg + 1) * 8, f[(kg + 1) & 1]);
      const Frag &c = f[kg & 1];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int bi = 0; bi < FM; ++bi)
#pragma unroll
          for (int bj = 0; bj < FN; ++bj)
            acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(c.a[bi][q], c.b[bj][q], acc[bi][bj], 0, 0, 0);
      // halfway through the step the next tile goes to the other LDS buffer
      // (last read before the previous barrier), so the stores overlap the
      // remaining multiplies
      if (kg == BK / 16 - 1 && kt + 1 < nk) store_lds(cur ^ 1, (kt + 1) * BK);
    }
    if constexpr (BT) __builtin_amdgcn_s_setprio(0);
    __syncthreads();
  }

  // ---- epilogue: D[row][col], row = 8*(r/4) + 4*(lane/32) + r%4, col = lane%32 ----
  // Residual / pre-activation values are fetched for the whole wave tile
  // first (clamped, always-valid addresses), then combined and stored.
#pragma unroll
  for (int bi = 0; bi < FM; ++bi) {
#pragma unroll
    for (int bj = 0; bj < FN; ++bj) {
      const int col = n0 + wn * WTN + bj * 32 + l32;
      const bool col_ok = col < g.N;
      const int colc = col_ok ? col : n0;
      float rv[16];
      if (EPI == EPI_RESID || EPI == EPI_DSILU || EPI == EPI_DSILU_Q || EPI == EPI_TAN) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int p = row0 + wm * WTM + bi * 32 + 8 * (r >> 2) + kh + (r & 3);
          const int pc = p < rows ? p : row0;
          rv[r] = g.R[int64_t(pc) * g.ldr + colc];
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = row0 + wm * WTM + bi * 32 + 8 * (r >> 2) + kh + (r & 3);
        const float v = acc[bi][bj][r];
        float out, out2 = 0.f;
        if (EPI == EPI_STORE) {
          out = v;
        } else if (EPI == EPI_RESID) {
          out = rv[r] + v;
        } else if (EPI == EPI_SILU) {
          out = v;
          out2 = v * __builtin_amdgcn_rcpf(1.f + __expf(-v));
        } else {
          // silu'(x) = sigmoid(x) (1 + x (1 - sigmoid(x))) at the saved pre-activation
          const float x = rv[r];
          const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-x));
          const float d1 = sg * (1.f + x * (1.f - sg));
          if (EPI == EPI_TAN) {
            out = v;
            out2 = v * d1;
          } else {
            out = v * d1;
            out2 = v;
          }
        }
        if (col_ok && p < rows) {
          const int64_t o = int64_t(p) * g.ldc + col;
          g.C[o] = out;
          if (EPI == EPI_SILU || EPI == EPI_DSILU_Q || EPI == EPI_TAN) g.C2[o] = out2;
        }
      }
    }
  }
}

// Expert GEMMs (group_off set, SPLIT): each group's rows are covered by
// BM-row tiles, except that a remainder of at most BM/2 rows gets a BM/2-row
// tile.  The two classes are dealt to the XCDs separately, full tiles first,
// so every XCD receives its share of each and the short tiles run last.
template <int BM, int BN, int BK, int WM, int WN, bool BT, int EPI, int TAG, bool SPLIT>
__global__ void __launch_bounds__(THREADS) gemm_kernel(GemmArgs g) {
  constexpr int LDK = BK + 4;
  constexpr int LDN = BN + 4;
  constexpr int AST = BM * LDK;
  constexpr int BST = BT ? (BN * LDK) : (BK * LDN);
  constexpr int HALF = BM / 2;
  __shared__ __attribute__((aligned(16))) float As[2 * AST];
  __shared__ __attribute__((aligned(16))) float Bs[2 * BST];
  __shared__ int s_tiles[MAX_GROUPS + 1];
  __shared__ int s_red[10];   // two scans' wave sums, then the two totals

  const int tid = threadIdx.x;
  const int G = g.group_off ? g.n_groups : 1;
  const int Nt = (g.N + BN - 1) / BN;
  const int L = blockIdx.x;
  const int jx = L / N_XCD, xcd = L - jx * N_XCD;

  // ---- m-tiles per group (full and, with SPLIT, half) -> prefix in LDS ----
  int Mt, t_local;
  bool half = false;
  if (g.group_off) {
    constexpr int PER = (MAX_GROUPS + THREADS) / THREADS;   // covers entries 0..MAX_GROUPS
    int cf[PER], ch[PER], sf = 0, sh = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int gi = tid * PER + q;
      const int c = gi < G ? g.group_off[gi + 1] - g.group_off[gi] : 0;
      if (SPLIT) {
        const int rem = c % BM;
        cf[q] = c / BM + (rem > HALF ? 1 : 0);
        ch[q] = (rem > 0 && rem <= HALF) ? 1 : 0;
      } else {
        cf[q] = (c + BM - 1) / BM;
        ch[q] = 0;
      }
      sf += cf[q];
      sh += ch[q];
    }
    int run_f = block_scan_excl(sf, s_red);
    int run_h = SPLIT ? block_scan_excl(sh, s_red + 4) : 0;
    int Mf = 0, Mh = 0;
    if (tid == THREADS - 1) {
      s_red[8] = run_f + sf;
      s_red[9] = run_h + sh;
    }
    __syncthreads();
    Mf = s_red[8];
    Mh = SPLIT ? s_red[9] : 0;
    const int per_f = (Mf * Nt + N_XCD - 1) / N_XCD;
    const int per_h = (Mh * Nt + N_XCD - 1) / N_XCD;
    if (jx < per_f) {
      t_local = xcd * per_f + jx;
      Mt = Mf;
    } else {
      if (!SPLIT || jx - per_f >= per_h) return;
      t_local = xcd * per_h + (jx - per_f);
      Mt = Mh;
      half = true;
    }
    if (t_local >= Mt * Nt) return;
    // prefix of this block's class only
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int gi = tid * PER + q;
      if (gi <= G) s_tiles[gi] = half ? run_h : run_f;
      run_f += cf[q];
      run_h += ch[q];
    }
    __syncthreads();
  } else {
    Mt = (g.M + BM - 1) / BM;
    const int per = (Mt * Nt + N_XCD - 1) / N_XCD;
    if (jx >= per) return;
    t_local = xcd * per + jx;
    if (t_local >= Mt * Nt) return;
  }
  const int group_size = RASTER_M * Nt;
  const int first_m = (t_local / group_size) * RASTER_M;
  const int gm = min(Mt - first_m, RASTER_M);
  const int rr = t_local % group_size;
  const int mt_glob = first_m + rr % gm;
  const int nt = rr / gm;

  int grp = 0, row0, rows;
  if (g.group_off) {
    int lo = 0, hi = G;  // last group with s_tiles[grp] <= mt_glob
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_tiles[mid] <= mt_glob) lo = mid;
      else hi = mid;
    }
    grp = lo;
    const int gbeg = g.group_off[grp];
    rows = g.group_off[grp + 1];
    if (half) row0 = gbeg + ((rows - gbeg) / BM) * BM;
    else row0 = gbeg + (mt_glob - s_tiles[grp]) * BM;
  } else {
    row0 = mt_glob * BM;
    rows = g.M;
  }
  const int n0 = nt * BN;
  const float *Bg = g.B + int64_t(grp) * g.b_group_stride;
  if constexpr (SPLIT) {
    if (half) {
      gemm_tile<HALF, BN, BK, WM, WN, BT, EPI, AST, BST>(g, As, Bs, Bg, row0, rows, n0);
      return;
    }
  }
  gemm_tile<BM, BN, BK, WM, WN, BT, EPI, AST, BST>(g, As, Bs, Bg, row0, rows, n0);
}

template <int BM, int BN, int BK, int WM, int WN, bool BT, int EPI, int TAG, bool SPLIT>
int launch_t(const GemmArgs &a, hipStream_t stream) {
  // Upper bounds of the per-XCD tile counts the kernel derives on the device:
  // full tiles <= (M + G*BM/2) / BM and half tiles <= G with SPLIT,
  // ceil(M/BM) + G tiles without it; surplus workgroups return at once.
  const int64_t nt = cdiv(a.N, BN);
  int64_t per;
  if (!a.group_off) {
    per = cdiv(cdiv(a.M, BM) * nt, N_XCD);
  } else if (SPLIT) {
    const int64_t mf = (int64_t(a.M) + int64_t(a.n_groups) * (BM / 2)) / BM;
    per = cdiv(mf * nt, N_XCD) + cdiv(int64_t(a.n_groups) * nt, N_XCD);
  } else {
    per = cdiv((cdiv(a.M, BM) + a.n_groups) * nt, N_XCD);
  }
  const int64_t grid = per * N_XCD;
  if (grid <= 0) return MLIP_OK;
  if (grid > int64_t(0x7fffffff)) {
    set_error("GEMM too large for one launch");
    return MLIP_ERR_UNSUPPORTED;
  }
  gemm_kernel<BM, BN, BK, WM, WN, BT, EPI, TAG, SPLIT><<<dim3(unsigned(grid)), dim3(THREADS), 0, stream>>>(a);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

// Expert GEMMs: 128 x 128 tiles, 64 x 128 for short group remainders.
template <bool BT, int EPI, int TAG>
int launch_expert(const GemmArgs &a, hipStream_t s) {
  return launch_t<128, 128, BT ? EXPERT_BK_NT : EXPERT_BK_NN, 2, 2, BT, EPI, TAG, true>(a, s);
}
// Dense projections: 64 x 64 tiles when the output is narrow (enough
// workgroups for 256 CUs), else 64 x 128.
template <bool BT, int EPI, int TAG>
int launch_dense(const GemmArgs &a, hipStream_t s) {
  if (a.N <= 512) return launch_t<64, 64, 32, 2, 2, BT, EPI, TAG, false>(a, s);
  return launch_t<64, 128, 32, 2, 2, BT, EPI, TAG, false>(a, s);
}

}  // namespace

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
