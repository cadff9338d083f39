// Three-body angular update ("Tri") of the complete interaction block and
// its input gradient.
//
// The ScienceAI article (architecture section) says three-body angles are
// embedded; the paper review (section 3.4, Fig. 3) puts Tri first in every
// interaction block.  The update implemented, for receiver i with edges e
// (unit vectors dhat_e, envelopes f_e = f_c(r_e), senders j(e)):
//   tau_ic = sum over ordered pairs e != e' of f_e f_e' (sum_l P_l(dhat_e.dhat_e') W_ang[l,c])
//            s_j(e),c s_j(e'),c,              s = h W_s,  h_T = h + tau W_T.
// The O(deg^2) pair sum is evaluated in O(deg) with the addition theorem of
// the Legendre polynomials, P_l(u.v) = sum_m S_lm(u) S_lm(v) for unit u, v,
// with S_lm the Schmidt semi-normalised real spherical harmonics (l <= 3,
// 16 functions):
//   A_lm,c = sum_e f_e S_lm(dhat_e) s_j(e),c,   B_c = sum_e f_e^2 s_j(e),c^2,
//   tau_c  = sum_l W_ang[l,c] (sum_m A_lm,c^2 - B_c)          (P_l(1) = 1).
//
// Layout: one 64-lane workgroup per receiver row; lane l owns CPL
// consecutive channels; the 16 harmonics of each edge (times f_e) are
// computed once per edge and broadcast from LDS.  Gradient (taubar = dL/dtau):
//   Abar_lm,c = 2 taubar_c W_ang[l,c] A_lm,c,   Bbar_c = -taubar_c sum_l W_ang[l,c];
//   receiver pass (row i): sigma_e,c = sum_lm Abar_lm,c f_e S_lm(dhat_e) + 2 Bbar_c f_e^2 s_j,c
//     is stored per edge (it is dL/ds_j(e) from this row); in the same
//     channel loop P_lm = sum_c Abar_lm,c s_j,c and Q = sum_c Bbar_c s_j,c^2
//     are summed over the lanes, and then, one lane per edge,
//     dL/dS_lm = f_e P_lm and dL/df_e = sum_lm S_lm P_lm + 2 f_e Q give the
//     edge vector dL/dd_e = dL/df_e f_c'(r) dhat + (I - dhat dhat^T) sum_lm dL/dS_lm grad S_lm / r.
//   sender pass (row j, edges j <- i): sbar_j = sum of sigma over the reverse
//     edges; forces and virial from dL/dd_e - dL/dd_rev(e).
// No atomics anywhere.
#include "common.h"

namespace mlip {

int tri_lane_layout(int Dt, int *cpl);

namespace {

constexpr int NSH = 16;      // (l, m) for l = 0..3
constexpr int NANG = 4;      // Legendre orders l = 0..3
constexpr int CHUNK = 64;
constexpr int UNROLL = 2;

__device__ inline int l_of(int lm) { return lm == 0 ? 0 : (lm < 4 ? 1 : (lm < 9 ? 2 : 3)); }

// Schmidt semi-normalised real harmonics at the unit vector (x, y, z)
__device__ inline void harmonics(float x, float y, float z, float *S) {
  const float r3 = 1.7320508075688772f, r15 = 3.872983346207417f;
  const float a58 = 0.7905694150420949f, a38 = 0.6123724356957945f;
  const float xx = x * x, yy = y * y, zz = z * z;
  S[0] = 1.f;
  S[1] = x; S[2] = y; S[3] = z;
  S[4] = r3 * x * y;
  S[5] = r3 * y * z;
  S[6] = 0.5f * (3.f * zz - 1.f);
  S[7] = r3 * x * z;
  S[8] = 0.5f * r3 * (xx - yy);
  S[9] = a58 * y * (3.f * xx - yy);
  S[10] = r15 * x * y * z;
  S[11] = a38 * y * (5.f * zz - 1.f);
  S[12] = 0.5f * z * (5.f * zz - 3.f);
  S[13] = a38 * x * (5.f * zz - 1.f);
  S[14] = 0.5f * r15 * z * (xx - yy);
  S[15] = a58 * x * (xx - 3.f * yy);
}

// sum_lm w[lm] grad S_lm at (x, y, z) (gradient of the polynomial forms above)
__device__ inline float3 harmonics_grad(float x, float y, float z, const float *w) {
  const float r3 = 1.7320508075688772f, r15 = 3.872983346207417f;
  const float a58 = 0.7905694150420949f, a38 = 0.6123724356957945f;
  const float xx = x * x, yy = y * y, zz = z * z;
  float gx = w[1], gy = w[2], gz = w[3];
  gx += r3 * (w[4] * y + w[7] * z + w[8] * x);
  gy += r3 * (w[4] * x + w[5] * z - w[8] * y);
  gz += r3 * (w[5] * y + w[7] * x) + 3.f * z * w[6];
  gx += a58 * 6.f * x * y * w[9] + r15 * y * z * w[10] + a38 * (5.f * zz - 1.f) * w[13] +
        r15 * x * z * w[14] + a58 * 3.f * (xx - yy) * w[15];
  gy += a58 * 3.f * (xx - yy) * w[9] + r15 * x * z * w[10] + a38 * (5.f * zz - 1.f) * w[11] -
        r15 * y * z * w[14] - a58 * 6.f * x * y * w[15];
  gz += r15 * x * y * w[10] + a38 * 10.f * y * z * w[11] + 0.5f * (15.f * zz - 3.f) * w[12] +
        a38 * 10.f * x * z * w[13] + 0.5f * r15 * (xx - yy) * w[14];
  return make_float3(gx, gy, gz);
}

template <int CPL>
__device__ inline void ldc(const float *p, float (&x)[CPL]) {
  if constexpr (CPL % 4 == 0) {
#pragma unroll
    for (int q = 0; q < CPL / 4; ++q) {
      const float4 v = reinterpret_cast<const float4 *>(p)[q];
      x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
    }
  } else if constexpr (CPL % 2 == 0) {
#pragma unroll
    for (int q = 0; q < CPL / 2; ++q) {
      const float2 v = reinterpret_cast<const float2 *>(p)[q];
      x[2 * q] = v.x; x[2 * q + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int q = 0; q < CPL; ++q) x[q] = p[q];
  }
}

template <int CPL>
__device__ inline void stc(float *p, const float (&x)[CPL]) {
  if constexpr (CPL % 4 == 0) {
#pragma unroll
    for (int q = 0; q < CPL / 4; ++q)
      reinterpret_cast<float4 *>(p)[q] = make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
  } else if constexpr (CPL % 2 == 0) {
#pragma unroll
    for (int q = 0; q < CPL / 2; ++q) reinterpret_cast<float2 *>(p)[q] = make_float2(x[2 * q], x[2 * q + 1]);
  } else {
#pragma unroll
    for (int q = 0; q < CPL; ++q) p[q] = x[q];
  }
}

// Per-edge prologue shared by the kernels: f_e S_lm(dhat_e) into LDS.
struct EdgeGeo {
  float fc, dfc, inv_r;
  float3 u;
};

__device__ inline EdgeGeo edge_geo(float4 g, const Radial &R) {
  EdgeGeo o;
  const float r = g.w;
  o.fc = 0.f;
  o.dfc = 0.f;
  if (r < R.rc) {
    float sn, cs;
    __sincosf(r * R.pi_over_rc, &sn, &cs);
    o.fc = 0.5f * (cs + 1.f);
    o.dfc = -0.5f * R.pi_over_rc * sn;
  }
  o.inv_r = r > 0.f ? 1.f / r : 0.f;
  o.u = make_float3(g.x * o.inv_r, g.y * o.inv_r, g.z * o.inv_r);
  return o;
}

// Accumulates A_lm,c and B_c of row i over its edges (channel layout).
template <int CPL>
__device__ inline void accumulate_row(const int32_t *__restrict__ src, const float4 *__restrict__ geom,
                                      const float *__restrict__ s, int n_atoms, int Dt, int c0, int r0, int r1,
                                      const Radial &R, float (*ysh)[NSH], float *fsq, int *jj,
                                      float (&A)[NSH][CPL], float (&Bs)[CPL]) {
  const int lane = threadIdx.x;
#pragma unroll
  for (int lm = 0; lm < NSH; ++lm)
#pragma unroll
    for (int c = 0; c < CPL; ++c) A[lm][c] = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) Bs[c] = 0.f;
  for (int e0 = r0; e0 < r1; e0 += CHUNK) {
    const int n = min(CHUNK, r1 - e0);
    if (lane < n) {
      const EdgeGeo G = edge_geo(geom[e0 + lane], R);
      float S[NSH];
      harmonics(G.u.x, G.u.y, G.u.z, S);
#pragma unroll
      for (int lm = 0; lm < NSH; ++lm) ysh[lane][lm] = G.fc * S[lm];
      fsq[lane] = G.fc * G.fc;
      jj[lane] = int(MLIP_IDX(src[e0 + lane], n_atoms, "sender"));
    }
    __syncthreads();
    for (int mm = 0; mm < n; mm += UNROLL) {
      float sj[UNROLL][CPL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) ldc<CPL>(s + int64_t(jj[min(mm + u, n - 1)]) * Dt + c0, sj[u]);
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (mm + u < n) {
          const int me = mm + u;
          const float fq = fsq[me];
#pragma unroll
          for (int lm = 0; lm < NSH; ++lm) {
            const float y = ysh[me][lm];
#pragma unroll
            for (int c = 0; c < CPL; ++c) A[lm][c] += y * sj[u][c];
          }
#pragma unroll
          for (int c = 0; c < CPL; ++c) Bs[c] += fq * sj[u][c] * sj[u][c];
        }
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------- forward ---
template <int CPL>
__global__ void __launch_bounds__(64) tri_fwd_kernel(
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ src,
    const float4 *__restrict__ geom, int n_atoms, const float *__restrict__ s,
    const float *__restrict__ W_ang, int Dt, float rc, float *__restrict__ tau) {
  __shared__ float ysh[CHUNK][NSH];
  __shared__ float fsq[CHUNK];
  __shared__ int jj[CHUNK];
  const int lane = threadIdx.x;
  const int64_t blk = xcd_block(n_atoms);
  if (blk < 0) return;
  const int i = int(blk);
  const bool active = lane * CPL < Dt;
  const int c0 = active ? lane * CPL : 0;
  const Radial R = make_radial(rc);
  float A[NSH][CPL], Bs[CPL];
  accumulate_row<CPL>(src, geom, s, n_atoms, Dt, c0, row_ptr[i], row_ptr[i + 1], R, ysh, fsq, jj, A, Bs);
  if (!active) return;
  float w[NANG][CPL];
#pragma unroll
  for (int l = 0; l < NANG; ++l) ldc<CPL>(W_ang + int64_t(l) * Dt + c0, w[l]);
  float t[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float q[NANG] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int lm = 0; lm < NSH; ++lm) q[l_of(lm)] += A[lm][c] * A[lm][c];
    float acc = 0.f;
#pragma unroll
    for (int l = 0; l < NANG; ++l) acc += w[l][c] * (q[l] - Bs[c]);
    t[c] = acc;
  }
  stc<CPL>(tau + int64_t(i) * Dt + c0, t);
}

// Sums 16 per-lane values over the wavefront.  Inside each 16-lane row, four
// halving steps (DPP moves) leave lane l with value l & 15 summed over its row:
// at each step a lane keeps one half of its values and adds the partner's copy
// of that half, the partner keeping the other half (partners: lane 15 - i,
// 7 - i, i ^ 2, i ^ 1 within the row).  Two shuffles then add the four rows.
// Afterwards lane l holds the total of value l & 15.
__device__ inline float reduce16(const float (&v)[NSH]) {
  const int lane = threadIdx.x & 63;
  const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2, b0 = lane & 1;
  float a8[8], a4[4], a2[2];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    a8[q] = (b3 ? v[q + 8] : v[q]) + dpp_mov<DPP_MIRROR>(b3 ? v[q] : v[q + 8]);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    a4[q] = (b2 ? a8[q + 4] : a8[q]) + dpp_mov<DPP_HALF_MIRROR>(b2 ? a8[q] : a8[q + 4]);
#pragma unroll
  for (int q = 0; q < 2; ++q)
    a2[q] = (b1 ? a4[q + 2] : a4[q]) + dpp_mov<DPP_XOR2>(b1 ? a4[q] : a4[q + 2]);
  float a1 = (b0 ? a2[1] : a2[0]) + dpp_mov<DPP_XOR1>(b0 ? a2[0] : a2[1]);
  a1 += __shfl_xor(a1, 16, 64);
  a1 += __shfl_xor(a1, 32, 64);
  return a1;
}

// ------------------------------------------------ gradient: receiver rows --
template <int CPL>
__global__ void __launch_bounds__(64) tri_vjp_recv_kernel(
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ src,
    const float4 *__restrict__ geom, int n_atoms, const float *__restrict__ s,
    const float *__restrict__ W_ang, const float *__restrict__ taubar, int Dt, float rc,
    float *__restrict__ sigma, float4 *__restrict__ gvec) {
  __shared__ float ysh[CHUNK][NSH];     // f_e S_lm(dhat_e)
  __shared__ float pq[CHUNK][NSH + 1];  // sum_c Abar_lm,c s_j,c and sum_c Bbar_c s_j,c^2
  __shared__ float4 geo[CHUNK];         // (dhat, 1/r)
  __shared__ float fcs[CHUNK], dfcs[CHUNK], fsq[CHUNK];
  __shared__ int jj[CHUNK];
  const int lane = threadIdx.x;
  const int64_t blk = xcd_block(n_atoms);
  if (blk < 0) return;
  const int i = int(blk);
  const bool active = lane * CPL < Dt;
  const int c0 = active ? lane * CPL : 0;
  const Radial R = make_radial(rc);
  const int r0 = row_ptr[i], r1 = row_ptr[i + 1];
  float A[NSH][CPL], Bs[CPL];
  accumulate_row<CPL>(src, geom, s, n_atoms, Dt, c0, r0, r1, R, ysh, fsq, jj, A, Bs);

  // Abar and Bbar of this row, in place of A and B (zero on idle lanes)
  {
    float w[NANG][CPL], tb[CPL];
#pragma unroll
    for (int l = 0; l < NANG; ++l) ldc<CPL>(W_ang + int64_t(l) * Dt + c0, w[l]);
    ldc<CPL>(taubar + int64_t(i) * Dt + c0, tb);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float wsum = 0.f;
#pragma unroll
      for (int l = 0; l < NANG; ++l) wsum += w[l][c];
      Bs[c] = active ? -tb[c] * wsum : 0.f;
#pragma unroll
      for (int lm = 0; lm < NSH; ++lm) A[lm][c] = active ? 2.f * tb[c] * w[l_of(lm)][c] * A[lm][c] : 0.f;
    }
  }

  for (int e0 = r0; e0 < r1; e0 += CHUNK) {
    const int n = min(CHUNK, r1 - e0);
    if (lane < n) {
      const EdgeGeo G = edge_geo(geom[e0 + lane], R);
      float S[NSH];
      harmonics(G.u.x, G.u.y, G.u.z, S);
#pragma unroll
      for (int lm = 0; lm < NSH; ++lm) ysh[lane][lm] = G.fc * S[lm];
      geo[lane] = make_float4(G.u.x, G.u.y, G.u.z, G.inv_r);
      fcs[lane] = G.fc;
      dfcs[lane] = G.dfc;
      fsq[lane] = G.fc * G.fc;
      jj[lane] = int(MLIP_IDX(src[e0 + lane], n_atoms, "sender"));
    }
    __syncthreads();
    // channel pass: sigma_e rows, and the channel sums P_lm, Q of every edge
    for (int mm = 0; mm < n; mm += UNROLL) {
      float sj[UNROLL][CPL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) ldc<CPL>(s + int64_t(jj[min(mm + u, n - 1)]) * Dt + c0, sj[u]);
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (mm + u < n) {
          const int me = mm + u;
          float out[CPL], P[NSH], Q = 0.f;
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            out[c] = 2.f * Bs[c] * fsq[me] * sj[u][c];
            Q += Bs[c] * sj[u][c] * sj[u][c];
          }
#pragma unroll
          for (int lm = 0; lm < NSH; ++lm) {
            const float y = ysh[me][lm];
            float p = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              out[c] += A[lm][c] * y;
              p += A[lm][c] * sj[u][c];
            }
            P[lm] = p;
          }
          if (active) stc<CPL>(sigma + int64_t(e0 + me) * Dt + c0, out);
          const float ptot = reduce16(P);
          float qtot = group_sum<16>(Q);
          qtot += __shfl_xor(qtot, 16, 64);
          qtot += __shfl_xor(qtot, 32, 64);
          // lanes 0..15 hold P_lm (lm = lane), lane 16 stores Q
          if (lane <= NSH) pq[me][lane] = lane < NSH ? ptot : qtot;
        }
      }
    }
    __syncthreads();
    // edge pass: dL/dS_lm = f P_lm, dL/df = sum_lm S_lm P_lm + 2 f Q, then the edge vector
    if (lane < n) {
      const float fc = fcs[lane];
      const float4 g = geo[lane];
      float S[NSH];
      harmonics(g.x, g.y, g.z, S);
      float fbar = 2.f * fc * pq[lane][NSH];
      float sbar_lm[NSH];
#pragma unroll
      for (int lm = 0; lm < NSH; ++lm) {
        const float p = pq[lane][lm];
        fbar += S[lm] * p;
        sbar_lm[lm] = fc * p;
      }
      const float3 gu = harmonics_grad(g.x, g.y, g.z, sbar_lm);
      const float rad = gu.x * g.x + gu.y * g.y + gu.z * g.z;
      const float a = fbar * dfcs[lane];
      gvec[e0 + lane] = make_float4(a * g.x + (gu.x - rad * g.x) * g.w,
                                    a * g.y + (gu.y - rad * g.y) * g.w,
                                    a * g.z + (gu.z - rad * g.z) * g.w, 0.f);
    }
    __syncthreads();
  }
}

// -------------------------------------------------- gradient: sender rows --
template <int CPL>
__global__ void __launch_bounds__(64) tri_vjp_send_kernel(
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ rev,
    const float4 *__restrict__ geom, int n_atoms, const float *__restrict__ sigma,
    const float4 *__restrict__ gvec, int Dt, int accumulate, float *__restrict__ sbar,
    float *__restrict__ grad_pos, float *__restrict__ atom_virial) {
  __shared__ int rr[CHUNK];
  const int lane = threadIdx.x;
  const int64_t blk = xcd_block(n_atoms);
  if (blk < 0) return;
  const int j = int(blk);
  const bool active = lane * CPL < Dt;
  const int c0 = active ? lane * CPL : 0;
  float sb[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) sb[c] = 0.f;
  float fx = 0.f, fy = 0.f, fz = 0.f;
  float vir[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int r0 = row_ptr[j], r1 = row_ptr[j + 1];
  for (int e0 = r0; e0 < r1; e0 += CHUNK) {
    const int n = min(CHUNK, r1 - e0);
    if (lane < n) {
      const int e = e0 + lane;
      const int re = int(MLIP_IDX(rev[e], row_ptr[n_atoms], "reverse edge"));
      rr[lane] = re;
      const float4 ge = gvec[e], gr = gvec[re], d = geom[e];
      const float gx = ge.x - gr.x, gy = ge.y - gr.y, gz = ge.z - gr.z;   // d_rev = -d
      fx += gx;
      fy += gy;
      fz += gz;
      vir[0] += 0.5f * gx * d.x;
      vir[1] += 0.5f * gy * d.y;
      vir[2] += 0.5f * gz * d.z;
      vir[3] += 0.25f * (gy * d.z + gz * d.y);
      vir[4] += 0.25f * (gx * d.z + gz * d.x);
      vir[5] += 0.25f * (gx * d.y + gy * d.x);
    }
    __syncthreads();
    for (int mm = 0; mm < n; mm += UNROLL) {
      float sg[UNROLL][CPL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u)
        ldc<CPL>(sigma + int64_t(rr[min(mm + u, n - 1)]) * Dt + c0, sg[u]);
#pragma unroll
      for (int u = 0; u < UNROLL; ++u)
        if (mm + u < n)
#pragma unroll
          for (int c = 0; c < CPL; ++c) sb[c] += sg[u][c];
    }
    __syncthreads();
  }
  if (active) stc<CPL>(sbar + int64_t(j) * Dt + c0, sb);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    fx += __shfl_xor(fx, d, 64);
    fy += __shfl_xor(fy, d, 64);
    fz += __shfl_xor(fz, d, 64);
#pragma unroll
    for (int q = 0; q < 6; ++q) vir[q] += __shfl_xor(vir[q], d, 64);
  }
  if (lane == 0) {
    float *gp = grad_pos + int64_t(j) * 3;
    float *av = atom_virial + int64_t(j) * 6;
    const float g3[3] = {-fx, -fy, -fz};
#pragma unroll
    for (int q = 0; q < 3; ++q) gp[q] = accumulate ? gp[q] + g3[q] : g3[q];
#pragma unroll
    for (int q = 0; q < 6; ++q) av[q] = accumulate ? av[q] + vir[q] : vir[q];
  }
}

template <int CPL>
int launch_cpl(int which, const TriArgs &a, hipStream_t stream) {
  const dim3 grid(unsigned(padded_grid(a.n_atoms))), block(64);
  const float4 *g4 = reinterpret_cast<const float4 *>(a.geom);
  if (which == 0) {
    tri_fwd_kernel<CPL><<<grid, block, 0, stream>>>(a.row_ptr, a.src, g4, a.n_atoms, a.s, a.W_ang,
                                                    a.Dt, a.rc, a.tau);
  } else if (which == 1) {
    tri_vjp_recv_kernel<CPL><<<grid, block, 0, stream>>>(
        a.row_ptr, a.src, g4, a.n_atoms, a.s, a.W_ang, a.taubar, a.Dt, a.rc, a.sigma,
        reinterpret_cast<float4 *>(a.gvec));
  } else {
    tri_vjp_send_kernel<CPL><<<grid, block, 0, stream>>>(
        a.row_ptr, a.rev, g4, a.n_atoms, a.sigma, reinterpret_cast<const float4 *>(a.gvec), a.Dt,
        a.accumulate, a.sbar, a.grad_pos, a.atom_virial);
  }
  MLIP_LAUNCHED();
  return MLIP_OK;
}

int dispatch(int which, const TriArgs &a, hipStream_t stream) {
  switch (a.cpl) {
    case 1: return launch_cpl<1>(which, a, stream);
    case 2: return launch_cpl<2>(which, a, stream);
    case 3: return launch_cpl<3>(which, a, stream);
    case 4: return launch_cpl<4>(which, a, stream);
    case 6: return launch_cpl<6>(which, a, stream);
    case 8: return launch_cpl<8>(which, a, stream);
    default: break;
  }
  set_error("no three-body lane layout for %d channels per lane", a.cpl);
  return MLIP_ERR_UNSUPPORTED;
}

// ------------------------------------------------------------ tangents ---
// Training gradient: derivatives along the position direction x_dot (d_dot =
// x_dot_j - x_dot_i, r_dot = dhat . d_dot, dhat_dot = (d_dot - dhat r_dot) / r,
// f_dot = f_c' r_dot) and the feature tangent s_dot = h_dot W_s:
//   y_e = f S(dhat),  y_dot = f_dot S + f (grad S . dhat_dot)
//   A_dot = sum_e y_dot s_j + y s_dot_j,   B_dot = sum_e 2 f f_dot s_j^2 + 2 f^2 s_j s_dot_j
//   tau_dot = sum_l W_ang[l] (2 sum_m A A_dot - B_dot)
// and of the gradient (Abar = 2 taubar W A, Bbar = -taubar sum_l W):
//   sigma_dot_e = sum_lm (Abar_dot y + Abar y_dot) + 2 Bbar_dot f^2 s_j + 2 Bbar (2 f f_dot s_j + f^2 s_dot_j)
//   dW_ang[l] += taubar_dot (sum_m A^2 - B) + taubar (2 sum_m A A_dot - B_dot)    (per row)
// The channels of a row are split over "slices" (workgroups of the same row)
// so that A and A_dot of 16 harmonics fit the registers; the per-edge
// harmonics are computed once per slice.

// directional derivatives grad S_lm . v of the 16 harmonics at (x, y, z)
__device__ inline void harmonics_dir(float x, float y, float z, float vx, float vy, float vz, float *D) {
  const float r3 = 1.7320508075688772f, r15 = 3.872983346207417f;
  const float a58 = 0.7905694150420949f, a38 = 0.6123724356957945f;
  const float xx = x * x, yy = y * y, zz = z * z;
  D[0] = 0.f;
  D[1] = vx; D[2] = vy; D[3] = vz;
  D[4] = r3 * (y * vx + x * vy);
  D[5] = r3 * (z * vy + y * vz);
  D[6] = 3.f * z * vz;
  D[7] = r3 * (z * vx + x * vz);
  D[8] = r3 * (x * vx - y * vy);
  D[9] = a58 * (6.f * x * y * vx + 3.f * (xx - yy) * vy);
  D[10] = r15 * (y * z * vx + x * z * vy + x * y * vz);
  D[11] = a38 * ((5.f * zz - 1.f) * vy + 10.f * y * z * vz);
  D[12] = 0.5f * (15.f * zz - 3.f) * vz;
  D[13] = a38 * ((5.f * zz - 1.f) * vx + 10.f * x * z * vz);
  D[14] = r15 * (x * z * vx - y * z * vy + 0.5f * (xx - yy) * vz);
  D[15] = a58 * (3.f * (xx - yy) * vx - 6.f * x * y * vy);
}

struct TriTanRow {
  const int32_t *src;
  const float4 *geom;
  const float *s, *s_dot;   // s_dot may be null
  const float *x_dot;
  float x_sign;
  int Dt, c0, i;
  int n_atoms;
};

// y, y_dot, f^2 and 2 f f_dot of the chunk's edges into LDS (lane = edge)
__device__ inline void tan_edge_terms(const TriTanRow &t, const Radial &R, int e, float xi0, float xi1,
                                      float xi2, float (*ysh)[NSH], float (*ydt)[NSH], float *fsq,
                                      float *ffd, int *jj, int lane) {
  const EdgeGeo G = edge_geo(t.geom[e], R);
  const int j = int(MLIP_IDX(t.src[e], t.n_atoms, "sender"));
  const float dx = t.x_sign * (t.x_dot[3 * j] - xi0), dy = t.x_sign * (t.x_dot[3 * j + 1] - xi1),
              dz = t.x_sign * (t.x_dot[3 * j + 2] - xi2);
  const float rd = G.u.x * dx + G.u.y * dy + G.u.z * dz;
  const float vx = (dx - G.u.x * rd) * G.inv_r, vy = (dy - G.u.y * rd) * G.inv_r,
              vz = (dz - G.u.z * rd) * G.inv_r;
  float S[NSH], D[NSH];
  harmonics(G.u.x, G.u.y, G.u.z, S);
  harmonics_dir(G.u.x, G.u.y, G.u.z, vx, vy, vz, D);
  const float fd = G.dfc * rd;
#pragma unroll
  for (int lm = 0; lm < NSH; ++lm) {
    ysh[lane][lm] = G.fc * S[lm];
    ydt[lane][lm] = fd * S[lm] + G.fc * D[lm];
  }
  fsq[lane] = G.fc * G.fc;
  ffd[lane] = 2.f * G.fc * fd;
  jj[lane] = j;
}

template <int CPL>
__device__ inline void tan_accumulate(const TriTanRow &t, int r0, int r1, const Radial &R, float (*ysh)[NSH],
                                      float (*ydt)[NSH], float *fsq, float *ffd, int *jj,
                                      float (&A)[NSH][CPL], float (&Ad)[NSH][CPL], float (&Bs)[CPL],
                                      float (&Bd)[CPL]) {
  const int lane = threadIdx.x;
#pragma unroll
  for (int lm = 0; lm < NSH; ++lm)
#pragma unroll
    for (int c = 0; c < CPL; ++c) A[lm][c] = Ad[lm][c] = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) Bs[c] = Bd[c] = 0.f;
  const float xi0 = t.x_dot[3 * t.i], xi1 = t.x_dot[3 * t.i + 1], xi2 = t.x_dot[3 * t.i + 2];
  for (int e0 = r0; e0 < r1; e0 += CHUNK) {
    const int n = min(CHUNK, r1 - e0);
    if (lane < n) tan_edge_terms(t, R, e0 + lane, xi0, xi1, xi2, ysh, ydt, fsq, ffd, jj, lane);
    __syncthreads();
    for (int me = 0; me < n; ++me) {
      float sj[CPL], sd[CPL];
      const int64_t j = jj[me];
      ldc<CPL>(t.s + j * t.Dt + t.c0, sj);
      if (t.s_dot) ldc<CPL>(t.s_dot + j * t.Dt + t.c0, sd);
      else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) sd[c] = 0.f;
      }
#pragma unroll
      for (int lm = 0; lm < NSH; ++lm) {
        const float y = ysh[me][lm], yd = ydt[me][lm];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          A[lm][c] += y * sj[c];
          Ad[lm][c] += yd * sj[c] + y * sd[c];
        }
      }
      const float fq = fsq[me], fd2 = ffd[me];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        Bs[c] += fq * sj[c] * sj[c];
        Bd[c] += fd2 * sj[c] * sj[c] + 2.f * fq * sj[c] * sd[c];
      }
    }
    __syncthreads();
  }
}

struct TriTanArgs {
  const int32_t *row_ptr, *src, *rev;
  const float *geom;
  int n_atoms;
  const float *x_dot;
  float x_sign;
  const float *s, *s_dot, *W_ang, *taubar, *taubar_dot;
  float *tau_dot, *sigma_dot, *wang_part, *sbar_dot;
  int Dt, n_slices;
  float rc;
};

template <int CPL>
__global__ void __launch_bounds__(64) tri_jvp_kernel(TriTanArgs a) {
  __shared__ float ysh[CHUNK][NSH], ydt[CHUNK][NSH];
  __shared__ float fsq[CHUNK], ffd[CHUNK];
  __shared__ int jj[CHUNK];
  const int lane = threadIdx.x;
  const int64_t blk = xcd_block(int64_t(a.n_atoms) * a.n_slices);
  if (blk < 0) return;
  const int i = int(blk / a.n_slices), slice = int(blk - int64_t(i) * a.n_slices);
  const int cc = (slice * 64 + lane) * CPL;
  const bool active = cc < a.Dt;
  TriTanRow t{a.src, reinterpret_cast<const float4 *>(a.geom), a.s, a.s_dot, a.x_dot, a.x_sign, a.Dt,
              active ? cc : 0, i, a.n_atoms};
  const Radial R = make_radial(a.rc);
  float A[NSH][CPL], Ad[NSH][CPL], Bs[CPL], Bd[CPL];
  tan_accumulate<CPL>(t, a.row_ptr[i], a.row_ptr[i + 1], R, ysh, ydt, fsq, ffd, jj, A, Ad, Bs, Bd);
  if (!active) return;
  float w[NANG][CPL], out[CPL];
#pragma unroll
  for (int l = 0; l < NANG; ++l) ldc<CPL>(a.W_ang + int64_t(l) * a.Dt + t.c0, w[l]);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float qd[NANG] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int lm = 0; lm < NSH; ++lm) qd[l_of(lm)] += 2.f * A[lm][c] * Ad[lm][c];
    float acc = 0.f;
#pragma unroll
    for (int l = 0; l < NANG; ++l) acc += w[l][c] * (qd[l] - Bd[c]);
    out[c] = acc;
  }
  stc<CPL>(a.tau_dot + int64_t(i) * a.Dt + t.c0, out);
}

template <int CPL>
__global__ void __launch_bounds__(64) tri_tvjp_recv_kernel(TriTanArgs a) {
  __shared__ float ysh[CHUNK][NSH], ydt[CHUNK][NSH];
  __shared__ float fsq[CHUNK], ffd[CHUNK];
  __shared__ int jj[CHUNK];
  const int lane = threadIdx.x;
  const int64_t blk = xcd_block(int64_t(a.n_atoms) * a.n_slices);
  if (blk < 0) return;
  const int i = int(blk / a.n_slices), slice = int(blk - int64_t(i) * a.n_slices);
  const int cc = (slice * 64 + lane) * CPL;
  const bool active = cc < a.Dt;
  TriTanRow t{a.src, reinterpret_cast<const float4 *>(a.geom), a.s, a.s_dot, a.x_dot, a.x_sign, a.Dt,
              active ? cc : 0, i, a.n_atoms};
  const Radial R = make_radial(a.rc);
  const int r0 = a.row_ptr[i], r1 = a.row_ptr[i + 1];
  float A[NSH][CPL], Ad[NSH][CPL], Bs[CPL], Bd[CPL];
  tan_accumulate<CPL>(t, r0, r1, R, ysh, ydt, fsq, ffd, jj, A, Ad, Bs, Bd);
  // W_ang gradient share of this row, then Abar / Abar_dot / Bbar / Bbar_dot in place
  {
    float w[NANG][CPL], tb[CPL], tbd[CPL];
#pragma unroll
    for (int l = 0; l < NANG; ++l) ldc<CPL>(a.W_ang + int64_t(l) * a.Dt + t.c0, w[l]);
    ldc<CPL>(a.taubar + int64_t(i) * a.Dt + t.c0, tb);
    ldc<CPL>(a.taubar_dot + int64_t(i) * a.Dt + t.c0, tbd);
    float wp[NANG][CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float q[NANG] = {0.f, 0.f, 0.f, 0.f}, qd[NANG] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int lm = 0; lm < NSH; ++lm) {
        q[l_of(lm)] += A[lm][c] * A[lm][c];
        qd[l_of(lm)] += 2.f * A[lm][c] * Ad[lm][c];
      }
      float wsum = 0.f;
#pragma unroll
      for (int l = 0; l < NANG; ++l) {
        wp[l][c] = tbd[c] * (q[l] - Bs[c]) + tb[c] * (qd[l] - Bd[c]);
        wsum += w[l][c];
      }
#pragma unroll
      for (int lm = 0; lm < NSH; ++lm) {
        const float wl = w[l_of(lm)][c];
        const float ab = 2.f * tb[c] * wl * A[lm][c];
        Ad[lm][c] = active ? 2.f * (tbd[c] * wl * A[lm][c] + tb[c] * wl * Ad[lm][c]) : 0.f;
        A[lm][c] = active ? ab : 0.f;
      }
      Bs[c] = active ? -tb[c] * wsum : 0.f;
      Bd[c] = active ? -tbd[c] * wsum : 0.f;
    }
    if (active) {
#pragma unroll
      for (int l = 0; l < NANG; ++l) stc<CPL>(a.wang_part + (int64_t(i) * NANG + l) * a.Dt + t.c0, wp[l]);
    }
  }
  // edges again: sigma_dot_e
  const float xi0 = a.x_dot[3 * i], xi1 = a.x_dot[3 * i + 1], xi2 = a.x_dot[3 * i + 2];
  for (int e0 = r0; e0 < r1; e0 += CHUNK) {
    const int n = min(CHUNK, r1 - e0);
    if (lane < n) tan_edge_terms(t, R, e0 + lane, xi0, xi1, xi2, ysh, ydt, fsq, ffd, jj, lane);
    __syncthreads();
    for (int me = 0; me < n; ++me) {
      float sj[CPL], sd[CPL], out[CPL];
      const int64_t j = jj[me];
      ldc<CPL>(a.s + j * a.Dt + t.c0, sj);
      if (a.s_dot) ldc<CPL>(a.s_dot + j * a.Dt + t.c0, sd);
      else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) sd[c] = 0.f;
      }
      const float fq = fsq[me], fd2 = ffd[me];
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        out[c] = 2.f * Bd[c] * fq * sj[c] + 2.f * Bs[c] * (fd2 * sj[c] + fq * sd[c]);
#pragma unroll
      for (int lm = 0; lm < NSH; ++lm) {
        const float y = ysh[me][lm], yd = ydt[me][lm];
#pragma unroll
        for (int c = 0; c < CPL; ++c) out[c] += Ad[lm][c] * y + A[lm][c] * yd;
      }
      if (active) stc<CPL>(a.sigma_dot + int64_t(e0 + me) * a.Dt + t.c0, out);
    }
    __syncthreads();
  }
}

// sbar_dot_j = sum over the edges j <- i of sigma_dot of the reverse edge
template <int CPL>
__global__ void __launch_bounds__(64) tri_tvjp_send_kernel(TriTanArgs a) {
  __shared__ int rr[CHUNK];
  const int lane = threadIdx.x;
  const int64_t blk = xcd_block(int64_t(a.n_atoms) * a.n_slices);
  if (blk < 0) return;
  const int j = int(blk / a.n_slices), slice = int(blk - int64_t(j) * a.n_slices);
  const int cc = (slice * 64 + lane) * CPL;
  const bool active = cc < a.Dt;
  const int c0 = active ? cc : 0;
  float sb[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) sb[c] = 0.f;
  const int r0 = a.row_ptr[j], r1 = a.row_ptr[j + 1];
  for (int e0 = r0; e0 < r1; e0 += CHUNK) {
    const int n = min(CHUNK, r1 - e0);
    if (lane < n) rr[lane] = int(MLIP_IDX(a.rev[e0 + lane], a.row_ptr[a.n_atoms], "reverse edge"));
    __syncthreads();
    for (int me = 0; me < n; ++me) {
      float sg[CPL];
      ldc<CPL>(a.sigma_dot + int64_t(rr[me]) * a.Dt + c0, sg);
#pragma unroll
      for (int c = 0; c < CPL; ++c) sb[c] += sg[c];
    }
    __syncthreads();
  }
  if (active) stc<CPL>(a.sbar_dot + int64_t(j) * a.Dt + c0, sb);
}

template <int CPL>
int launch_tan_cpl(int which, const TriTanArgs &a, hipStream_t stream) {
  const dim3 grid(unsigned(padded_grid(int64_t(a.n_atoms) * a.n_slices))), block(64);
  if (which == 0) tri_jvp_kernel<CPL><<<grid, block, 0, stream>>>(a);
  else if (which == 1) tri_tvjp_recv_kernel<CPL><<<grid, block, 0, stream>>>(a);
  else tri_tvjp_send_kernel<CPL><<<grid, block, 0, stream>>>(a);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

// channels per lane of the tangent kernels: at most 4 (A and A_dot in
// registers); wider rows are split into two slices
int tan_layout(int Dt, int *cpl_t, int *n_slices) {
  int cpl = 0;
  if (tri_lane_layout(Dt, &cpl) != MLIP_OK) return MLIP_ERR_UNSUPPORTED;
  *cpl_t = cpl <= 4 ? cpl : cpl / 2;
  *n_slices = int(cdiv(Dt, 64 * *cpl_t));
  return MLIP_OK;
}

int dispatch_tan(int which, TriTanArgs a, hipStream_t stream) {
  int c = 0;
  if (tan_layout(a.Dt, &c, &a.n_slices) != MLIP_OK) {
    set_error("d_tri = %d has no three-body lane layout", a.Dt);
    return MLIP_ERR_UNSUPPORTED;
  }
  switch (c) {
    case 1: return launch_tan_cpl<1>(which, a, stream);
    case 2: return launch_tan_cpl<2>(which, a, stream);
    case 3: return launch_tan_cpl<3>(which, a, stream);
    case 4: return launch_tan_cpl<4>(which, a, stream);
    default: break;
  }
  set_error("no three-body tangent layout for %d channels per lane", c);
  return MLIP_ERR_UNSUPPORTED;
}

}  // namespace

int tri_lane_layout(int Dt, int *cpl) {
  const int options[] = {1, 2, 3, 4, 6, 8};
  for (int c : options) {
    if (Dt % c == 0 && Dt <= 64 * c) {
      *cpl = c;
      return MLIP_OK;
    }
  }
  return MLIP_ERR_UNSUPPORTED;
}

int launch_tri_fwd(const TriArgs &a, hipStream_t stream) {
  if (a.n_atoms <= 0) return MLIP_OK;
  ProfScope ps(K_TRI_FWD, stream);
  return dispatch(0, a, stream);
}

int launch_tri_vjp(const TriArgs &a, hipStream_t stream) {
  if (a.n_atoms <= 0) return MLIP_OK;
  {
    ProfScope ps(K_TRI_VJP_RECV, stream);
    if (int rc = dispatch(1, a, stream)) return rc;
  }
  ProfScope ps(K_TRI_VJP_SEND, stream);
  return dispatch(2, a, stream);
}

int launch_tri_jvp(const int32_t *row_ptr, const int32_t *src, const float *geom, int n_atoms,
                   const float *x_dot, float x_sign, const float *s, const float *s_dot, const float *W_ang,
                   int Dt, float rc, float *tau_dot, hipStream_t stream) {
  if (n_atoms <= 0) return MLIP_OK;
  ProfScope ps(K_TRI_FWD, stream);
  TriTanArgs a{};
  a.row_ptr = row_ptr; a.src = src; a.geom = geom; a.n_atoms = n_atoms;
  a.x_dot = x_dot; a.x_sign = x_sign; a.s = s; a.s_dot = s_dot; a.W_ang = W_ang;
  a.tau_dot = tau_dot; a.Dt = Dt; a.rc = rc;
  return dispatch_tan(0, a, stream);
}

int launch_tri_tvjp(const int32_t *row_ptr, const int32_t *src, const int32_t *rev, const float *geom,
                    int n_atoms, const float *x_dot, float x_sign, const float *s, const float *s_dot,
                    const float *W_ang, const float *taubar, const float *taubar_dot, int Dt, float rc,
                    float *sigma_dot, float *wang_part, float *sbar_dot, hipStream_t stream) {
  if (n_atoms <= 0) return MLIP_OK;
  TriTanArgs a{};
  a.row_ptr = row_ptr; a.src = src; a.rev = rev; a.geom = geom; a.n_atoms = n_atoms;
  a.x_dot = x_dot; a.x_sign = x_sign; a.s = s; a.s_dot = s_dot; a.W_ang = W_ang;
  a.taubar = taubar; a.taubar_dot = taubar_dot; a.sigma_dot = sigma_dot; a.wang_part = wang_part;
  a.sbar_dot = sbar_dot; a.Dt = Dt; a.rc = rc;
  {
    ProfScope ps(K_TRI_VJP_RECV, stream);
    if (int rc2 = dispatch_tan(1, a, stream)) return rc2;
  }
  ProfScope ps(K_TRI_VJP_SEND, stream);
  return dispatch_tan(2, a, stream);
}

}  // namespace mlip
