// Edge kernels: the fused edge embedding + neighbour aggregation of the
// forward pass, and the fused edge part of the input gradient (sbar and the
// per-edge distance derivative that gives the forces).
//
// Both walk the receiver-sorted CSR one row per wavefront, so every sum over
// a row is a private accumulation: no atomics, and the result does not depend
// on scheduling.  The forward follows the ScienceAI article (pair distances
// are embedded) and the paper review of "Breaking the Training Barrier of
// Billion-Parameter Universal MLIPs", section 3.5 (neighbour features are
// gathered, modulated and reduced onto the receiver); the gradient follows
// section 3.3 of that review (forces from differentiating the energy).
//
// Layout: one 64-lane workgroup per (row, 128-column slice) in the forward,
// one per row in the gradient.  Each lane owns two adjacent columns; the
// per-edge radial scalars (16 basis values) are computed once per edge by
// one lane and broadcast through LDS.
#include "common.h"

namespace mlip {

namespace {

constexpr int K = MLIP_N_RBF;
constexpr int EDGE_CHUNK = 64;
constexpr int COLS = 128;  // columns per slice: 64 lanes x float2

struct Radial {
  float mu_step, gamma, pi_over_rc, rc;
};

__device__ inline Radial make_radial(float rc) {
  Radial p;
  p.rc = rc;
  p.mu_step = rc / float(K - 1);
  p.gamma = float((K - 1) * (K - 1)) / (2.f * rc * rc);
  p.pi_over_rc = 3.14159265358979323846f / rc;
  return p;
}

// Forward: e_e = f_c(r) * (phi(r) @ W_e), fused with a_i = sum_e e_e * s_src(e).
__global__ void __launch_bounds__(64) embed_aggregate_kernel(
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ src,
    const float4 *__restrict__ geom, int n_atoms, int n_slices, const float *__restrict__ W_e,
    const float *__restrict__ s, int De, float rc, float *__restrict__ e_out,
    float *__restrict__ a_out) {
  __shared__ float phi[EDGE_CHUNK][K + 1];
  __shared__ int jj[EDGE_CHUNK];
  const int lane = threadIdx.x;
  const int i = blockIdx.x / n_slices;
  const int slice = blockIdx.x - i * n_slices;
  if (i >= n_atoms) return;
  const int c = slice * COLS + 2 * lane;
  const bool active = c < De;
  const Radial R = make_radial(rc);

  float2 w[K];
#pragma unroll
  for (int k = 0; k < K; ++k)
    w[k] = active ? *reinterpret_cast<const float2 *>(W_e + k * De + c) : make_float2(0.f, 0.f);

  float2 acc = make_float2(0.f, 0.f);
  const int r0 = row_ptr[i], r1 = row_ptr[i + 1];
  for (int e0 = r0; e0 < r1; e0 += EDGE_CHUNK) {
    const int n = min(EDGE_CHUNK, r1 - e0);
    if (lane < n) {
      const float r = geom[e0 + lane].w;
      const float fc = r < rc ? 0.5f * (__cosf(r * R.pi_over_rc) + 1.f) : 0.f;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float x = r - float(k) * R.mu_step;
        phi[lane][k] = fc * __expf(-R.gamma * x * x);
      }
      jj[lane] = src[e0 + lane];
    }
    __syncthreads();
    if (active) {
      int m = 0;
      for (; m + 2 <= n; m += 2) {
        const int j0 = jj[m], j1 = jj[m + 1];
        const float2 s0 = *reinterpret_cast<const float2 *>(s + int64_t(j0) * De + c);
        const float2 s1 = *reinterpret_cast<const float2 *>(s + int64_t(j1) * De + c);
        float2 v0 = make_float2(0.f, 0.f), v1 = make_float2(0.f, 0.f);
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float p0 = phi[m][k], p1 = phi[m + 1][k];
          v0.x += p0 * w[k].x;
          v0.y += p0 * w[k].y;
          v1.x += p1 * w[k].x;
          v1.y += p1 * w[k].y;
        }
        __builtin_nontemporal_store(v0.x, e_out + int64_t(e0 + m) * De + c);
        __builtin_nontemporal_store(v0.y, e_out + int64_t(e0 + m) * De + c + 1);
        __builtin_nontemporal_store(v1.x, e_out + int64_t(e0 + m + 1) * De + c);
        __builtin_nontemporal_store(v1.y, e_out + int64_t(e0 + m + 1) * De + c + 1);
        acc.x += v0.x * s0.x;
        acc.y += v0.y * s0.y;
        acc.x += v1.x * s1.x;
        acc.y += v1.y * s1.y;
      }
      if (m < n) {
        const int j0 = jj[m];
        const float2 s0 = *reinterpret_cast<const float2 *>(s + int64_t(j0) * De + c);
        float2 v0 = make_float2(0.f, 0.f);
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float p0 = phi[m][k];
          v0.x += p0 * w[k].x;
          v0.y += p0 * w[k].y;
        }
        __builtin_nontemporal_store(v0.x, e_out + int64_t(e0 + m) * De + c);
        __builtin_nontemporal_store(v0.y, e_out + int64_t(e0 + m) * De + c + 1);
        acc.x += v0.x * s0.x;
        acc.y += v0.y * s0.y;
      }
    }
    __syncthreads();
  }
  if (active) *reinterpret_cast<float2 *>(a_out + int64_t(i) * De + c) = acc;
}

// Gradient: for row i with senders j,
//   sbar_i = sum_e e_e * abar_j                (e is symmetric: e_rev(e) = e_e)
//   c_e + c_rev(e) = sum_c (abar_i s_j + abar_j s_i)_c * de_c/dr
//   grad_pos_i = -sum_e (c_e + c_rev(e)) d_e / r_e
// de_c/dr = sum_k W_e[k,c] g_k(r), g_k = f_c' phi_k + f_c phi_k'.
__global__ void __launch_bounds__(64) edge_vjp_kernel(
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ src,
    const float4 *__restrict__ geom, int n_atoms, const float *__restrict__ W_e,
    const float *__restrict__ e, const float *__restrict__ s, const float *__restrict__ abar,
    int De, float rc, float *__restrict__ sbar, float *__restrict__ grad_pos) {
  __shared__ float gk[EDGE_CHUNK][K + 1];
  __shared__ float4 dir[EDGE_CHUNK];  // (dhat, unused)
  __shared__ int jj[EDGE_CHUNK];
  const int lane = threadIdx.x;
  const int i = blockIdx.x;
  if (i >= n_atoms) return;
  const Radial R = make_radial(rc);
  const int r0 = row_ptr[i], r1 = row_ptr[i + 1];
  float f0 = 0.f, f1 = 0.f, f2 = 0.f;

  for (int c0 = 0; c0 < De; c0 += COLS) {
    const int c = c0 + 2 * lane;
    const bool active = c < De;
    float2 w[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
      w[k] = active ? *reinterpret_cast<const float2 *>(W_e + k * De + c) : make_float2(0.f, 0.f);
    const float2 ai = active ? *reinterpret_cast<const float2 *>(abar + int64_t(i) * De + c)
                             : make_float2(0.f, 0.f);
    const float2 si = active ? *reinterpret_cast<const float2 *>(s + int64_t(i) * De + c)
                             : make_float2(0.f, 0.f);
    float2 sb = make_float2(0.f, 0.f);
    for (int e0 = r0; e0 < r1; e0 += EDGE_CHUNK) {
      const int n = min(EDGE_CHUNK, r1 - e0);
      if (lane < n) {
        const float4 g = geom[e0 + lane];
        const float r = g.w;
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
          gk[lane][k] = dfc * ph + fc * (-2.f * R.gamma * x * ph);
        }
        const float inv = r > 0.f ? 1.f / r : 0.f;
        dir[lane] = make_float4(g.x * inv, g.y * inv, g.z * inv, 0.f);
        jj[lane] = src[e0 + lane];
      }
      __syncthreads();
      if (active) {
        for (int m = 0; m < n; ++m) {
          const int j = jj[m];
          const int64_t eo = int64_t(e0 + m) * De + c;
          const float2 ev = make_float2(__builtin_nontemporal_load(e + eo),
                                        __builtin_nontemporal_load(e + eo + 1));
          const float2 aj = *reinterpret_cast<const float2 *>(abar + int64_t(j) * De + c);
          const float2 sj = *reinterpret_cast<const float2 *>(s + int64_t(j) * De + c);
          sb.x += ev.x * aj.x;
          sb.y += ev.y * aj.y;
          float wx = 0.f, wy = 0.f;
#pragma unroll
          for (int k = 0; k < K; ++k) {
            const float g = gk[m][k];
            wx += g * w[k].x;
            wy += g * w[k].y;
          }
          const float zx = ai.x * sj.x + aj.x * si.x;
          const float zy = ai.y * sj.y + aj.y * si.y;
          const float p = zx * wx + zy * wy;
          const float4 dv = dir[m];
          f0 += p * dv.x;
          f1 += p * dv.y;
          f2 += p * dv.z;
        }
      }
      __syncthreads();
    }
    if (active) *reinterpret_cast<float2 *>(sbar + int64_t(i) * De + c) = sb;
  }
  // reduce the per-lane partial forces over the wavefront
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    f0 += __shfl_xor(f0, d, 64);
    f1 += __shfl_xor(f1, d, 64);
    f2 += __shfl_xor(f2, d, 64);
  }
  if (lane == 0) {
    grad_pos[i * 3 + 0] = -f0;
    grad_pos[i * 3 + 1] = -f1;
    grad_pos[i * 3 + 2] = -f2;
  }
}

}  // namespace

int launch_embed_aggregate(const int32_t *row_ptr, const int32_t *src, const float *geom,
                           int n_atoms, const float *W_e, const float *s, int De, float rc,
                           float *e, float *a, hipStream_t stream) {
  if (n_atoms <= 0) return MLIP_OK;
  const int n_slices = int(cdiv(De, COLS));
  ProfScope ps(K_EMBED_AGG, stream);
  embed_aggregate_kernel<<<dim3(unsigned(int64_t(n_atoms) * n_slices)), dim3(64), 0, stream>>>(
      row_ptr, src, reinterpret_cast<const float4 *>(geom), n_atoms, n_slices, W_e, s, De, rc, e, a);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

int launch_edge_vjp(const int32_t *row_ptr, const int32_t *src, const float *geom, int n_atoms,
                    const float *W_e, const float *e, const float *s, const float *abar, int De,
                    float rc, float *sbar, float *grad_pos, hipStream_t stream) {
  if (n_atoms <= 0) return MLIP_OK;
  ProfScope ps(K_EDGE_VJP, stream);
  edge_vjp_kernel<<<dim3(unsigned(n_atoms)), dim3(64), 0, stream>>>(
      row_ptr, src, reinterpret_cast<const float4 *>(geom), n_atoms, W_e, e, s, abar, De, rc, sbar,
      grad_pos);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

}  // namespace mlip
