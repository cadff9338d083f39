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
// Tiling: 128x128 output tile per 256-thread workgroup, 2x2 wavefronts of
// 64x64, each as 2x2 blocks of v_mfma_f32_32x32x2_f32.  K advances 32 at a
// time through double-buffered LDS with one barrier per step; the next
// step's global loads are in flight while the current one is multiplied.
// A and NT-B tiles sit in LDS as [row][k] (k contiguous, row stride 36
// floats: 16-byte reads without bank conflicts); NN-B tiles as [k][n].
// Each MFMA lane supplies the k-values k0 + 4*(lane/32) + q, q = 0..3, for
// four consecutive MFMAs, so one 16-byte LDS read feeds four instructions.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs; each XCD is
// given a contiguous range of tiles (m fastest), so the m-tiles that share a
// weight tile (same expert, same n-tile) run on one XCD and share its L2.
#include "common.h"

namespace mlip {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int THREADS = 256;
constexpr int LDK = BK + 4;    // [row][k] tiles
constexpr int LDN = BN + 4;    // [k][n] tiles
constexpr int N_XCD = 8;

__device__ inline float silu_f(float x) { return x / (1.f + __expf(-x)); }
__device__ inline float dsilu_f(float x) {
  const float sg = 1.f / (1.f + __expf(-x));
  return sg * (1.f + x * (1.f - sg));
}

template <bool BT, int EPI>
__global__ void __launch_bounds__(THREADS) gemm_kernel(GemmArgs g) {
  __shared__ float As[2][BM * LDK];
  __shared__ float Bs[2][BT ? (BN * LDK) : (BK * LDN)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile scheduling over (group, m-tile) x n-tile, XCD-contiguous ----
  int Mt = 0;
  if (g.group_off) {
    for (int q = 0; q < g.n_groups; ++q) Mt += (g.group_off[q + 1] - g.group_off[q] + BM - 1) / BM;
  } else {
    Mt = (g.M + BM - 1) / BM;
  }
  const int Nt = (g.N + BN - 1) / BN;
  const int total = Mt * Nt;
  const int per = (total + N_XCD - 1) / N_XCD;
  const int L = blockIdx.x;
  const int j = L / N_XCD, xcd = L - j * N_XCD;
  if (j >= per) return;
  const int T = xcd * per + j;
  if (T >= total) return;
  const int nt = T / Mt;
  int mt = T - nt * Mt;
  int grp = 0, row0 = 0, rows = g.M;
  if (g.group_off) {
    for (grp = 0; grp < g.n_groups; ++grp) {
      const int lo = g.group_off[grp], cnt = g.group_off[grp + 1] - lo;
      const int tiles = (cnt + BM - 1) / BM;
      if (mt < tiles) {
        row0 = lo + mt * BM;
        rows = lo + cnt;
        break;
      }
      mt -= tiles;
    }
  } else {
    row0 = mt * BM;
  }
  const int n0 = nt * BN;
  const float *Bg = g.B + int64_t(grp) * g.b_group_stride;

  // ---- per-thread global load assignments ----
  const int lr = tid >> 3;          // 0..31 row within a 32-row pass
  const int lk = (tid & 7) * 4;     // k offset of the float4
  const float *a_src[4];
  bool a_ok[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int p = row0 + lr + 32 * q;
    a_ok[q] = p < rows;
    int64_t arow = p;
    if (a_ok[q] && g.a_rows) arow = g.a_rows[p];
    a_src[q] = g.A + (a_ok[q] ? arow * g.lda : 0);
  }
  const float *b_src[4];
  bool b_ok[4];
  int b_k[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (BT) {   // [N][K]: row n, float4 along k
      const int n = n0 + lr + 32 * q;
      b_ok[q] = n < g.N;
      b_src[q] = Bg + (b_ok[q] ? int64_t(n) * g.ldb : 0);
      b_k[q] = 0;
    } else {    // [K][N]: row k, float4 along n
      const int n = n0 + (tid & 31) * 4;
      b_ok[q] = n < g.N;
      b_k[q] = (tid >> 5) + 8 * q;
      b_src[q] = Bg + (b_ok[q] ? n : 0);
    }
  }

  floatx4 ra[4], rb[4];
  auto load_global = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = k0 + lk;
      ra[q] = (a_ok[q] && k < g.K) ? *reinterpret_cast<const floatx4 *>(a_src[q] + k)
                                   : floatx4{0.f, 0.f, 0.f, 0.f};
      if (BT) {
        rb[q] = (b_ok[q] && k < g.K) ? *reinterpret_cast<const floatx4 *>(b_src[q] + k)
                                     : floatx4{0.f, 0.f, 0.f, 0.f};
      } else {
        const int kb = k0 + b_k[q];
        rb[q] = (b_ok[q] && kb < g.K)
                    ? *reinterpret_cast<const floatx4 *>(b_src[q] + int64_t(kb) * g.ldb)
                    : floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<floatx4 *>(&As[buf][(lr + 32 * q) * LDK + lk]) = ra[q];
      if (BT) {
        *reinterpret_cast<floatx4 *>(&Bs[buf][(lr + 32 * q) * LDK + lk]) = rb[q];
      } else {
        *reinterpret_cast<floatx4 *>(&Bs[buf][b_k[q] * LDN + (tid & 31) * 4]) = rb[q];
      }
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.f;

  const int nk = (g.K + BK - 1) / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();

  const int l32 = lane & 31;
  const int kh = (lane >> 5) * 4;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_global((kt + 1) * BK);
    const float *Ab = As[cur];
    const float *Bb = Bs[cur];
#pragma unroll
    for (int kg = 0; kg < BK; kg += 8) {
      floatx4 af[2], bf[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
        af[bi] = *reinterpret_cast<const floatx4 *>(&Ab[(wm * 64 + bi * 32 + l32) * LDK + kg + kh]);
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) {
        if (BT) {
          bf[bj] = *reinterpret_cast<const floatx4 *>(&Bb[(wn * 64 + bj * 32 + l32) * LDK + kg + kh]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) bf[bj][q] = Bb[(kg + kh + q) * LDN + wn * 64 + bj * 32 + l32];
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
          for (int bj = 0; bj < 2; ++bj)
            acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[bi][q], bf[bj][q], acc[bi][bj], 0, 0, 0);
    }
    if (kt + 1 < nk) store_lds(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: D[row][col], row = 8*(r/4) + 4*(lane/32) + r%4, col = lane%32 ----
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const int col = n0 + wn * 64 + bj * 32 + l32;
      if (col >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = row0 + wm * 64 + bi * 32 + 8 * (r >> 2) + kh + (r & 3);
        if (p >= rows) continue;
        float v = acc[bi][bj][r];
        const int64_t o = int64_t(p) * g.ldc + col;
        if (EPI == EPI_STORE) {
          g.C[o] = v;
        } else if (EPI == EPI_RESID) {
          g.C[o] = g.R[int64_t(p) * g.ldr + col] + v;
        } else if (EPI == EPI_SILU) {
          g.C[o] = v;
          g.C2[o] = silu_f(v);
        } else {
          g.C[o] = v * dsilu_f(g.R[int64_t(p) * g.ldr + col]);
        }
      }
    }
  }
}

template <bool BT, int EPI>
int launch_t(const GemmArgs &a, hipStream_t stream) {
  const int64_t mt_upper = cdiv(a.M, BM) + (a.group_off ? a.n_groups : 0);
  const int64_t total_upper = mt_upper * cdiv(a.N, BN);
  const int64_t grid = cdiv(total_upper, N_XCD) * N_XCD;
  if (grid <= 0) return MLIP_OK;
  if (grid > int64_t(0x7fffffff)) {
    set_error("GEMM too large for one launch");
    return MLIP_ERR_UNSUPPORTED;
  }
  gemm_kernel<BT, EPI><<<dim3(unsigned(grid)), dim3(THREADS), 0, stream>>>(a);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

}  // namespace

int launch_gemm(const GemmArgs &a, bool bt, Epilogue epi, KClass cls, hipStream_t stream) {
  if (a.M <= 0 || a.N <= 0) return MLIP_OK;
  if ((a.K & 3) || (a.N & 3) || (a.lda & 3) || (a.ldb & 3)) {
    set_error("GEMM dims must be multiples of 4 (K=%d N=%d)", a.K, a.N);
    return MLIP_ERR_UNSUPPORTED;
  }
  ProfScope ps(cls, stream);
  switch (epi) {
    case EPI_STORE: return bt ? launch_t<true, EPI_STORE>(a, stream) : launch_t<false, EPI_STORE>(a, stream);
    case EPI_RESID: return bt ? launch_t<true, EPI_RESID>(a, stream) : launch_t<false, EPI_RESID>(a, stream);
    case EPI_SILU: return bt ? launch_t<true, EPI_SILU>(a, stream) : launch_t<false, EPI_SILU>(a, stream);
    case EPI_DSILU: return bt ? launch_t<true, EPI_DSILU>(a, stream) : launch_t<false, EPI_DSILU>(a, stream);
  }
  set_error("unknown epilogue");
  return MLIP_ERR_INVALID;
}

}  // namespace mlip
