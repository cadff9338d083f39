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
// Layout: one 64-lane workgroup per (row, 128-column slice) in the forward;
// in the gradient one workgroup per row whose wavefronts share the column
// slices.  Each lane owns two adjacent columns; the per-edge radial scalars
// (16 basis values) are computed once per edge and broadcast through LDS.
#include "common.h"

namespace mlip {

namespace {

constexpr int K = MLIP_N_RBF;
constexpr int EDGE_CHUNK = 64;
constexpr int COLS = 128;  // columns per slice: 64 lanes x float2

typedef float f2v __attribute__((ext_vector_type(2)));
constexpr int UNROLL = 4;

__device__ inline f2v ld2(const float *p) { return *reinterpret_cast<const f2v *>(p); }

// sum_k b[k] w[k] for a 16-aligned LDS row b of K floats (four 16-byte reads),
// as one chain of fused multiply-adds in k order (K instructions per column)
__device__ inline f2v basis_dot(const float *b, const f2v (&w)[K]) {
  const float4 t0 = reinterpret_cast<const float4 *>(b)[0];
  f2v v = t0.x * w[0];
  v = t0.y * w[1] + v;
  v = t0.z * w[2] + v;
  v = t0.w * w[3] + v;
#pragma unroll
  for (int q = 1; q < K / 4; ++q) {
    const float4 t = reinterpret_cast<const float4 *>(b)[q];
    v = t.x * w[4 * q] + v;
    v = t.y * w[4 * q + 1] + v;
    v = t.z * w[4 * q + 2] + v;
    v = t.w * w[4 * q + 3] + v;
  }
  return v;
}

// Forward: e_e = f_c(r) * (phi(r) @ W_e), fused with a_i = sum_e e_e * s_src(e).
// One wavefront per (row, 128-column slice).  Edges are taken UNROLL at a
// time with all their gathers issued before any arithmetic.  e is written to
// HBM only when the caller asks for it (STORE_E); the gradient can rebuild it
// from the 16 basis values at 16 FMAs per element instead of reading it back.
template <bool STORE_E>
__global__ void __launch_bounds__(64) embed_aggregate_kernel(
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ src,
    const float4 *__restrict__ geom, int n_atoms, int n_slices, const float *__restrict__ W_e,
    const float *__restrict__ s, int De, float rc, float *__restrict__ e_out,
    float *__restrict__ a_out) {
  // rows of 16 floats: every lane reads the same row (broadcast), 4 x 16 bytes
  __shared__ __attribute__((aligned(16))) float phi[EDGE_CHUNK][K];
  __shared__ int jj[EDGE_CHUNK];
  const int lane = threadIdx.x;
  const int64_t blk = xcd_block(int64_t(n_atoms) * n_slices);
  if (blk < 0) return;
  const int i = int(blk / n_slices);
  const int slice = int(blk - int64_t(i) * n_slices);
  const int c = slice * COLS + 2 * lane;
  const bool active = c < De;
  const int cc = active ? c : 0;   // clamped column for always-valid addresses
  const Radial R = make_radial(rc);

  f2v w[K];
#pragma unroll
  for (int k = 0; k < K; ++k) w[k] = ld2(W_e + k * De + cc);

  f2v acc = {0.f, 0.f};
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
      jj[lane] = int(MLIP_IDX(src[e0 + lane], n_atoms, "sender"));
    }
    __syncthreads();
    for (int m = 0; m < n; m += UNROLL) {
      f2v sv[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int mm = min(m + u, n - 1);
        sv[u] = ld2(s + int64_t(jj[mm]) * De + cc);
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (m + u < n) {
          const f2v v = basis_dot(phi[m + u], w);
          if (STORE_E && active)
            __builtin_nontemporal_store(v, reinterpret_cast<f2v *>(e_out + int64_t(e0 + m + u) * De + c));
          acc += v * sv[u];
        }
      }
    }
    __syncthreads();
  }
  if (active) *reinterpret_cast<f2v *>(a_out + int64_t(i) * De + c) = acc;
}

// Gradient: for row i with senders j,
//   sbar_i = sum_e e_e * abar_j                (e is symmetric: e_rev(e) = e_e)
//   c_e + c_rev(e) = sum_c (abar_i s_j + abar_j s_i)_c * de_c/dr
//   grad_pos_i = -sum_e (c_e + c_rev(e)) d_e / r_e
//   atom_virial_i = 1/2 sum_e (c_e + c_rev(e)) dhat_e (x) d_e    (strain gradient
//                   dL/d(eps) = sum_e c_e dhat_e (x) d_e, shared by the two atoms)
// de_c/dr = sum_k W_e[k,c] g_k(r), g_k = f_c' phi_k + f_c phi_k'.
// One workgroup of NW wavefronts per row; wavefront w takes column slices
// w, w+NW, ...; the per-edge radial terms are computed once per workgroup.
// Without a stored e (HAVE_E false) e_e = sum_k W_e[k,c] f_c phi_k is rebuilt
// from the same radial terms.
template <int NW, bool HAVE_E>
__global__ void __launch_bounds__(64 * NW) edge_vjp_kernel(
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ src,
    const float4 *__restrict__ geom, int n_atoms, const float *__restrict__ W_e,
    const float *__restrict__ e, const float *__restrict__ s, const float *__restrict__ abar,
    int De, float rc, float *__restrict__ sbar, float *__restrict__ grad_pos,
    float *__restrict__ atom_virial) {
  // rows of 16 / 8 floats: broadcast reads of 16 bytes
  __shared__ __attribute__((aligned(16))) float gk[EDGE_CHUNK][K];
  __shared__ __attribute__((aligned(16))) float pk[HAVE_E ? 1 : EDGE_CHUNK][K];   // f_c phi_k when e is rebuilt
  __shared__ float4 dir[EDGE_CHUNK];  // (dhat, unused)
  __shared__ __attribute__((aligned(16))) float vq[EDGE_CHUNK][8]; // dhat_a d_b: xx yy zz yz xz xy, 2 pad
  __shared__ int jj[EDGE_CHUNK];
  __shared__ float fred[NW][9];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t blk = xcd_block(n_atoms);
  if (blk < 0) return;
  const int i = int(blk);
  const Radial R = make_radial(rc);
  const int r0 = row_ptr[i], r1 = row_ptr[i + 1];
  const int n_slices = (De + COLS - 1) / COLS;
  f2v fxy = {0.f, 0.f};
  float fz = 0.f;
  float vir[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  for (int sl0 = 0; sl0 < n_slices; sl0 += NW) {
    const int sl = sl0 + wave;
    const int c = sl * COLS + 2 * lane;
    const bool active = sl < n_slices && c < De;
    const int cc = active ? c : 0;
    f2v w[K];
#pragma unroll
    for (int k = 0; k < K; ++k) w[k] = ld2(W_e + k * De + cc);
    const f2v ai = ld2(abar + int64_t(i) * De + cc);
    const f2v si = ld2(s + int64_t(i) * De + cc);
    f2v sb = {0.f, 0.f};
    for (int e0 = r0; e0 < r1; e0 += EDGE_CHUNK) {
      const int n = min(EDGE_CHUNK, r1 - e0);
      // radial terms: thread (wave w, lane l) computes basis functions
      // k = w, w + NW, ... of edge l
      {
        const int ed = lane, part = wave;
        if (ed < n) {
        const float4 g = geom[e0 + ed];
        const float r = g.w;
        float fc = 0.f, dfc = 0.f;
        if (r < rc) {
          float sn, cs;
          __sincosf(r * R.pi_over_rc, &sn, &cs);
          fc = 0.5f * (cs + 1.f);
          dfc = -0.5f * R.pi_over_rc * sn;
        }
        for (int k = part; k < K; k += NW) {
          const float x = r - float(k) * R.mu_step;
          const float ph = __expf(-R.gamma * x * x);
          gk[ed][k] = dfc * ph + fc * (-2.f * R.gamma * x * ph);
          if (!HAVE_E) pk[ed][k] = fc * ph;
        }
        if (part == 0) {
          const float inv = r > 0.f ? 1.f / r : 0.f;
          dir[ed] = make_float4(g.x * inv, g.y * inv, g.z * inv, 0.f);
          vq[ed][0] = g.x * g.x * inv;
          vq[ed][1] = g.y * g.y * inv;
          vq[ed][2] = g.z * g.z * inv;
          vq[ed][3] = g.y * g.z * inv;
          vq[ed][4] = g.x * g.z * inv;
          vq[ed][5] = g.x * g.y * inv;
          jj[ed] = int(MLIP_IDX(src[e0 + ed], n_atoms, "sender"));
        }
        }
      }
      __syncthreads();
      if (active) {
        for (int m = 0; m < n; m += UNROLL) {
          f2v ev[UNROLL], aj[UNROLL], sj[UNROLL];
#pragma unroll
          for (int u = 0; u < UNROLL; ++u) {
            const int mm = min(m + u, n - 1);
            const int j = jj[mm];
            if (HAVE_E)
              ev[u] = __builtin_nontemporal_load(reinterpret_cast<const f2v *>(e + int64_t(e0 + mm) * De + c));
            aj[u] = ld2(abar + int64_t(j) * De + c);
            sj[u] = ld2(s + int64_t(j) * De + c);
          }
#pragma unroll
          for (int u = 0; u < UNROLL; ++u) {
            if (m + u < n) {
              if (!HAVE_E) ev[u] = basis_dot(pk[m + u], w);
              sb += ev[u] * aj[u];
              const f2v wv = basis_dot(gk[m + u], w);
              const f2v z = ai * sj[u] + aj[u] * si;
              const f2v pz = z * wv;
              const float p = pz.x + pz.y;
              const float4 dv = dir[m + u];
              fxy += p * f2v{dv.x, dv.y};
              fz += p * dv.z;
              const float4 v0 = reinterpret_cast<const float4 *>(vq[m + u])[0];
              const float4 v1 = reinterpret_cast<const float4 *>(vq[m + u])[1];
              vir[0] += p * v0.x;
              vir[1] += p * v0.y;
              vir[2] += p * v0.z;
              vir[3] += p * v0.w;
              vir[4] += p * v1.x;
              vir[5] += p * v1.y;
            }
          }
        }
      }
      __syncthreads();
    }
    if (active) *reinterpret_cast<f2v *>(sbar + int64_t(i) * De + c) = sb;
  }
  // reduce the partial forces and virials over the lanes, then over the
  // wavefronts; each edge term is shared half and half by its two atoms
  float acc[9] = {fxy.x, fxy.y, fz, vir[0], vir[1], vir[2], vir[3], vir[4], vir[5]};
#pragma unroll
  for (int q = 0; q < 9; ++q)
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc[q] += __shfl_xor(acc[q], d, 64);
  if (lane == 0)
#pragma unroll
    for (int q = 0; q < 9; ++q) fred[wave][q] = acc[q];
  __syncthreads();
  if (tid < 9) {
    float t = 0.f;
    for (int w2 = 0; w2 < NW; ++w2) t += fred[w2][tid];
    if (tid < 3) grad_pos[i * 3 + tid] = -t;
    else atom_virial[int64_t(i) * 6 + (tid - 3)] = 0.5f * t;
  }
}

}  // namespace

int launch_embed_aggregate(const int32_t *row_ptr, const int32_t *src, const float *geom,
                           int n_atoms, const float *W_e, const float *s, int De, float rc,
                           float *e, float *a, hipStream_t stream) {
  if (n_atoms <= 0) return MLIP_OK;
  const int n_slices = int(cdiv(De, COLS));
  ProfScope ps(K_EMBED_AGG, stream);
  const dim3 grid(unsigned(padded_grid(int64_t(n_atoms) * n_slices)));
  if (e)
    embed_aggregate_kernel<true><<<grid, dim3(64), 0, stream>>>(
        row_ptr, src, reinterpret_cast<const float4 *>(geom), n_atoms, n_slices, W_e, s, De, rc, e, a);
  else
    embed_aggregate_kernel<false><<<grid, dim3(64), 0, stream>>>(
        row_ptr, src, reinterpret_cast<const float4 *>(geom), n_atoms, n_slices, W_e, s, De, rc, e, a);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

// grad_strain_b = sum over the atoms of structure b of atom_virial (float64,
// fixed reduction tree).
__global__ void __launch_bounds__(256) strain_sum_kernel(const float *__restrict__ atom_virial,
                                                         const int32_t *__restrict__ struct_ptr,
                                                         int n_atoms, double *__restrict__ grad_strain) {
  __shared__ double part[6][256];
  const int b = blockIdx.x;
  // the atom range is clamped into [0, n_atoms): a malformed struct_ptr
  // cannot make the sum read past the per-atom array
  const int lo = min(max(struct_ptr[b], 0), n_atoms);
  const int hi = min(max(struct_ptr[b + 1], lo), n_atoms);
  double acc[6] = {0, 0, 0, 0, 0, 0};
  for (int i = lo + threadIdx.x; i < hi; i += 256)
    for (int q = 0; q < 6; ++q) acc[q] += double(atom_virial[int64_t(i) * 6 + q]);
  for (int q = 0; q < 6; ++q) part[q][threadIdx.x] = acc[q];
  __syncthreads();
  for (int st = 128; st >= 1; st >>= 1) {
    if (int(threadIdx.x) < st)
      for (int q = 0; q < 6; ++q) part[q][threadIdx.x] += part[q][threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x < 6) grad_strain[b * 6 + threadIdx.x] = part[threadIdx.x][0];
}

int launch_strain_sum(const float *atom_virial, const int32_t *struct_ptr, int n_structs, int n_atoms,
                      double *grad_strain, hipStream_t stream) {
  strain_sum_kernel<<<dim3(unsigned(n_structs)), dim3(256), 0, stream>>>(atom_virial, struct_ptr,
                                                                        n_atoms, grad_strain);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

int launch_edge_vjp(const int32_t *row_ptr, const int32_t *src, const float *geom, int n_atoms,
                    const float *W_e, const float *e, const float *s, const float *abar, int De,
                    float rc, float *sbar, float *grad_pos, float *atom_virial, hipStream_t stream) {
  if (n_atoms <= 0) return MLIP_OK;
  ProfScope ps(K_EDGE_VJP, stream);
  const int n_slices = int(cdiv(De, COLS));
  const float4 *g4 = reinterpret_cast<const float4 *>(geom);
  const dim3 grid(unsigned(padded_grid(n_atoms)));
  const int nw = n_slices >= 4 ? 4 : n_slices;
#define MLIP_EDGE_VJP(NWV, HE)                                                                   \
  edge_vjp_kernel<NWV, HE><<<grid, dim3(64 * NWV), 0, stream>>>(row_ptr, src, g4, n_atoms, W_e, e, \
                                                                 s, abar, De, rc, sbar, grad_pos,  \
                                                                 atom_virial)
  if (e) {
    if (nw == 4) MLIP_EDGE_VJP(4, true);
    else if (nw == 3) MLIP_EDGE_VJP(3, true);
    else if (nw == 2) MLIP_EDGE_VJP(2, true);
    else MLIP_EDGE_VJP(1, true);
  } else {
    if (nw == 4) MLIP_EDGE_VJP(4, false);
    else if (nw == 3) MLIP_EDGE_VJP(3, false);
    else if (nw == 2) MLIP_EDGE_VJP(2, false);
    else MLIP_EDGE_VJP(1, false);
  }
#undef MLIP_EDGE_VJP
  MLIP_LAUNCHED();
  return MLIP_OK;
}

}  // namespace mlip
