// Neighbour multi-head attention of the complete interaction block and its
// input gradient.
//
// The paper review of "Breaking the Training Barrier of Billion-Parameter
// Universal MLIPs" (section 3.2) replaces the separable attention of MatRIS
// by multi-head self-attention whose cost stays O(N) at a fixed cutoff, with
// sparse MoE layers before and after it; Table II gives the heads and width
// (S: 8 x 48).  Attention runs over each atom's radius-graph neighbours:
//   e_ij   = f_c(r) (phi(r) @ Wa_e)                    (attention width Da)
//   s_ij^t = sum_{c in head t} q_ic k_jc e_ijc / sqrt(dh)
//   a_ij^t = f_c(r_ij) exp(s_ij^t) / sum_l f_c(r_il) exp(s_il^t)
//   o_ic   = sum_j a_ij^{t(c)} v_jc e_ijc
// with [q | k | v] = h0 @ W_qkv computed by the dense GEMM beforehand.
//
// Layout: one 64-lane workgroup per receiver row, all heads in the one
// wavefront.  Lane l serves head t = l / LPH and the CPL consecutive channels
// t*dh + (l % LPH)*CPL ...; a head's dot products are summed over its LPH
// lanes with xor shuffles (LPH a power of two, so groups never straddle).
// The softmax is accumulated online (running maximum, rescaled sums).  The
// per-edge radial terms are computed once per edge (lane = edge) and read
// from LDS by every lane.  Rows are private to one wavefront: no atomics.
//
// Gradient, in two row passes (dL/do = obar, beta_i^t = <obar_i, o_i>_t):
//   receiver pass (row i): gbar_ij^t = a_ij^t (<obar_i, v_j e_ij>_t - beta_i^t),
//     qbar_i += gbar k_j e / sqrt(dh), dL/dr_ij = ebar . de/dr + fbar f_c'(r)
//     with ebar = gbar q_i k_j / sqrt(dh) + a obar_i v_j and fbar the
//     derivative through the envelope weight; gbar, a and dL/dr are stored
//     per edge.
//   sender pass (row j, edges j <- i): the reverse edge i <- j carries the
//     receiver-pass values, so kbar_j = sum gbar_rev q_i e / sqrt(dh),
//     vbar_j = sum a_rev obar_i e, and the forces and virial take
//     dL/dr_e + dL/dr_rev(e) as in the aggregation's gradient.
#include <cmath>

#include "common.h"

namespace mlip {

namespace {

constexpr int K = MLIP_N_RBF;
constexpr int KQ = K / 4;
constexpr int CHUNK = 64;
constexpr int UNROLL = 2;

// CPL consecutive floats (vector loads where CPL allows; the channel offset
// is a multiple of CPL, and rows are multiples of 4 floats long)
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

// Sum over the lph lanes of one head (aligned power-of-two lane groups); LPH
// is the lane count when it is fixed at compile time, 0 when it is not.
template <int LPH>
__device__ inline float head_sum(float v, int lph) {
  if constexpr (LPH > 0) {
    return group_sum<LPH>(v);
  } else {
    for (int d = lph >> 1; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
  }
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// e_c = sum_k b[k] w[k][c] for the lane's channels, b read from LDS as float4;
// one chain of fused multiply-adds per channel in k order
template <int CPL>
__device__ inline void basis_map(const float4 *b, const float (&w)[K][CPL], float (&e)[CPL]) {
  const float4 p0 = b[0];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    e[c] = p0.x * w[0][c];
    e[c] = p0.y * w[1][c] + e[c];
    e[c] = p0.z * w[2][c] + e[c];
    e[c] = p0.w * w[3][c] + e[c];
  }
#pragma unroll
  for (int kq = 1; kq < KQ; ++kq) {
    const float4 p = b[kq];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      e[c] = p.x * w[4 * kq][c] + e[c];
      e[c] = p.y * w[4 * kq + 1][c] + e[c];
      e[c] = p.z * w[4 * kq + 2][c] + e[c];
      e[c] = p.w * w[4 * kq + 3][c] + e[c];
    }
  }
}

struct Lanes {
  int t, c0;
  bool active;
};

template <int CPL>
__device__ inline Lanes lane_map(int lane, int nh, int lph) {
  Lanes L;
  const int dh = lph * CPL;
  L.t = lane / lph;
  L.active = L.t < nh;
  L.c0 = L.active ? L.t * dh + (lane - L.t * lph) * CPL : 0;
  if (!L.active) L.t = 0;
  return L;
}

// ------------------------------------------------------------- forward ---
// The sender rows of the next UNROLL edges are gathered into a second set of
// registers while the current ones are used (two sets where the register
// budget of two waves per SIMD allows it, i.e. up to 6 channels per lane).
template <int CPL>
constexpr bool kPrefetch = CPL <= 6;

template <int CPL, int LPH>
__global__ void __launch_bounds__(64) attn_fwd_kernel(
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ src,
    const float4 *__restrict__ geom, int n_atoms, const float *__restrict__ Wa_e,
    const float *__restrict__ qkv, int Da, int nh, int lph, float rc, float *__restrict__ o,
    float2 *__restrict__ stats) {
  __shared__ float4 phi[CHUNK][KQ];  // f_c(r) phi_k(r)
  __shared__ float fcs[CHUNK];
  __shared__ int jj[CHUNK];
  const int lane = threadIdx.x;
  const int64_t blk = xcd_block(n_atoms);
  if (blk < 0) return;
  const int i = int(blk);
  const Lanes L = lane_map<CPL>(lane, nh, lph);
  const float isq = 1.f / sqrtf(float(lph * CPL));
  const Radial R = make_radial(rc);
  const int64_t ld = 3 * int64_t(Da);

  float w[K][CPL];
#pragma unroll
  for (int k = 0; k < K; ++k) ldc<CPL>(Wa_e + int64_t(k) * Da + L.c0, w[k]);
  float q[CPL];
  ldc<CPL>(qkv + int64_t(i) * ld + L.c0, q);
#pragma unroll
  for (int c = 0; c < CPL; ++c) q[c] *= isq;

  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  float m = -INFINITY, Z = 0.f;
  constexpr int NB = kPrefetch<CPL> ? 2 : 1;
  float kj[NB][UNROLL][CPL], vj[NB][UNROLL][CPL];
  const int r0 = row_ptr[i], r1 = row_ptr[i + 1];
  for (int e0 = r0; e0 < r1; e0 += CHUNK) {
    const int n = min(CHUNK, r1 - e0);
    if (lane < n) {
      const float r = geom[e0 + lane].w;
      const float fc = r < rc ? 0.5f * (__cosf(r * R.pi_over_rc) + 1.f) : 0.f;
      float ph[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float x = r - float(k) * R.mu_step;
        ph[k] = fc * __expf(-R.gamma * x * x);
      }
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq)
        phi[lane][kq] = make_float4(ph[4 * kq], ph[4 * kq + 1], ph[4 * kq + 2], ph[4 * kq + 3]);
      fcs[lane] = fc;
      jj[lane] = int(MLIP_IDX(src[e0 + lane], n_atoms, "sender"));
    }
    __syncthreads();
    // gather the k and v rows of edges mm .. mm + UNROLL - 1 into set b
    auto fetch = [&](int b, int mm) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const float *row = qkv + int64_t(jj[min(mm + u, n - 1)]) * ld + L.c0;
        ldc<CPL>(row + Da, kj[b][u]);
        ldc<CPL>(row + 2 * Da, vj[b][u]);
      }
    };
    auto edges = [&](int b, int mm) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (mm + u < n) {
          const int me = mm + u;
          float e[CPL];
          basis_map<CPL>(phi[me], w, e);
          float part = 0.f;
#pragma unroll
          for (int c = 0; c < CPL; ++c) part += q[c] * kj[b][u][c] * e[c];
          const float s = head_sum<LPH>(part, lph);
          const float mn = fmaxf(m, s);
          const float sc = __expf(m - mn);
          const float wt = fcs[me] * __expf(s - mn);
          Z = Z * sc + wt;
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[c] = acc[c] * sc + wt * (vj[b][u][c] * e[c]);
          m = mn;
        }
      }
    };
    if constexpr (NB == 2) {
      fetch(0, 0);
      for (int mm = 0; mm < n; mm += 2 * UNROLL) {
        if (mm + UNROLL < n) fetch(1, mm + UNROLL);
        edges(0, mm);
        if (mm + 2 * UNROLL < n) fetch(0, mm + 2 * UNROLL);
        edges(1, mm + UNROLL);
      }
    } else {
      for (int mm = 0; mm < n; mm += UNROLL) {
        fetch(0, mm);
        edges(0, mm);
      }
    }
    __syncthreads();
  }
  if (L.active) {
    const float inv = Z > 0.f ? 1.f / Z : 0.f;
    float out[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) out[c] = acc[c] * inv;
    stc<CPL>(o + int64_t(i) * Da + L.c0, out);
    if (lane == L.t * lph) stats[int64_t(i) * nh + L.t] = make_float2(m, Z);
  }
}

// ------------------------------------------------ gradient: receiver rows --
// dL/dr of an edge sums over all channels: each 16-lane row sums its lanes with
// DPP moves, the row totals go to LDS, and after the chunk lane e adds the four
// totals of its edge and stores them (one coalesced store per chunk).
template <int CPL, int LPH>
__global__ void __launch_bounds__(64) attn_vjp_recv_kernel(
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ src,
    const float4 *__restrict__ geom, int n_atoms, const float *__restrict__ Wa_e,
    const float *__restrict__ qkv, const float *__restrict__ o, const float2 *__restrict__ stats,
    const float *__restrict__ obar, int Da, int nh, int lph, float rc,
    float *__restrict__ qkv_bar, float *__restrict__ edge_g, float *__restrict__ edge_a,
    float *__restrict__ edge_c) {
  __shared__ float4 phi[CHUNK][KQ];   // f_c phi_k
  __shared__ float4 dph[CHUNK][KQ];   // d(f_c phi_k)/dr
  __shared__ float fcs[CHUNK], dfcs[CHUNK];
  __shared__ int jj[CHUNK];
  __shared__ float4 rowc[CHUNK];      // per edge: the four 16-lane rows' dL/dr parts
  const int lane = threadIdx.x;
  const int64_t blk = xcd_block(n_atoms);
  if (blk < 0) return;
  const int i = int(blk);
  const Lanes L = lane_map<CPL>(lane, nh, lph);
  const float isq = 1.f / sqrtf(float(lph * CPL));
  const Radial R = make_radial(rc);
  const int64_t ld = 3 * int64_t(Da);
  const float on = L.active ? 1.f : 0.f;

  float w[K][CPL];
#pragma unroll
  for (int k = 0; k < K; ++k) ldc<CPL>(Wa_e + int64_t(k) * Da + L.c0, w[k]);
  float q[CPL], ob[CPL], oo[CPL];
  ldc<CPL>(qkv + int64_t(i) * ld + L.c0, q);
  ldc<CPL>(obar + int64_t(i) * Da + L.c0, ob);
  ldc<CPL>(o + int64_t(i) * Da + L.c0, oo);
  float bpart = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    q[c] *= isq * on;
    ob[c] *= on;
    bpart += ob[c] * oo[c];
  }
  const float beta = head_sum<LPH>(bpart, lph);
  const float2 st = stats[int64_t(i) * nh + L.t];
  const float m = L.active ? st.x : 0.f;
  const float invZ = (L.active && st.y > 0.f) ? 1.f / st.y : 0.f;
  const bool head_lead = L.active && lane == L.t * lph;
  const bool row_lead = (lane & 15) == 0;
  float *rowc_f = reinterpret_cast<float *>(rowc);

  float qb[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) qb[c] = 0.f;
  constexpr int NB = kPrefetch<CPL> ? 2 : 1;
  float kj[NB][UNROLL][CPL], vj[NB][UNROLL][CPL];
  const int r0 = row_ptr[i], r1 = row_ptr[i + 1];
  for (int e0 = r0; e0 < r1; e0 += CHUNK) {
    const int n = min(CHUNK, r1 - e0);
    if (lane < n) {
      const float r = geom[e0 + lane].w;
      float fc = 0.f, dfc = 0.f;
      if (r < rc) {
        float sn, cs;
        __sincosf(r * R.pi_over_rc, &sn, &cs);
        fc = 0.5f * (cs + 1.f);
        dfc = -0.5f * R.pi_over_rc * sn;
      }
      float ph[K], dp[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float x = r - float(k) * R.mu_step;
        const float p = __expf(-R.gamma * x * x);
        ph[k] = fc * p;
        dp[k] = dfc * p + fc * (-2.f * R.gamma * x * p);
      }
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) {
        phi[lane][kq] = make_float4(ph[4 * kq], ph[4 * kq + 1], ph[4 * kq + 2], ph[4 * kq + 3]);
        dph[lane][kq] = make_float4(dp[4 * kq], dp[4 * kq + 1], dp[4 * kq + 2], dp[4 * kq + 3]);
      }
      fcs[lane] = fc;
      dfcs[lane] = dfc;
      jj[lane] = int(MLIP_IDX(src[e0 + lane], n_atoms, "sender"));
    }
    __syncthreads();
    auto fetch = [&](int b, int mm) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const float *row = qkv + int64_t(jj[min(mm + u, n - 1)]) * ld + L.c0;
        ldc<CPL>(row + Da, kj[b][u]);
        ldc<CPL>(row + 2 * Da, vj[b][u]);
      }
    };
    auto edges = [&](int b, int mm) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (mm + u < n) {
          const int me = mm + u;
          const float *kk = kj[b][u], *vv = vj[b][u];
          float e[CPL], de[CPL];
          basis_map<CPL>(phi[me], w, e);
          basis_map<CPL>(dph[me], w, de);
          float ps = 0.f, pa = 0.f;
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            ps += q[c] * kk[c] * e[c];
            pa += ob[c] * vv[c] * e[c];
          }
          const float s = head_sum<LPH>(ps, lph);
          const float ab = head_sum<LPH>(pa, lph);
          const float wt = __expf(s - m);
          const float alpha = fcs[me] * wt * invZ;
          const float diff = ab - beta;
          const float g = alpha * diff;
          float cp = head_lead ? wt * invZ * diff * dfcs[me] : 0.f;
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            cp += (g * q[c] * kk[c] + alpha * ob[c] * vv[c]) * de[c];
            qb[c] += g * kk[c] * e[c];
          }
          const float cr = group_sum<16>(cp);
          if (row_lead) rowc_f[4 * me + (lane >> 4)] = cr;
          const int64_t eg = int64_t(e0 + me);
          if (head_lead) {
            edge_g[eg * nh + L.t] = g;
            edge_a[eg * nh + L.t] = alpha;
          }
        }
      }
    };
    if constexpr (NB == 2) {
      fetch(0, 0);
      for (int mm = 0; mm < n; mm += 2 * UNROLL) {
        if (mm + UNROLL < n) fetch(1, mm + UNROLL);
        edges(0, mm);
        if (mm + 2 * UNROLL < n) fetch(0, mm + 2 * UNROLL);
        edges(1, mm + UNROLL);
      }
    } else {
      for (int mm = 0; mm < n; mm += UNROLL) {
        fetch(0, mm);
        edges(0, mm);
      }
    }
    __syncthreads();
    if (lane < n) {
      const float4 rc4 = rowc[lane];
      edge_c[e0 + lane] = (rc4.x + rc4.y) + (rc4.z + rc4.w);
    }
  }
  if (L.active) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) qb[c] *= isq;
    stc<CPL>(qkv_bar + int64_t(i) * ld + L.c0, qb);
  }
}

// -------------------------------------------------- gradient: sender rows --
template <int CPL, int LPH>
__global__ void __launch_bounds__(64) attn_vjp_send_kernel(
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ src,
    const int32_t *__restrict__ rev, const float4 *__restrict__ geom, int n_atoms,
    const float *__restrict__ Wa_e, const float *__restrict__ qkv, const float *__restrict__ obar,
    const float *__restrict__ edge_g, const float *__restrict__ edge_a,
    const float *__restrict__ edge_c, int Da, int nh, int lph, float rc, int accumulate,
    float *__restrict__ qkv_bar, float *__restrict__ grad_pos, float *__restrict__ atom_virial) {
  __shared__ float4 phi[CHUNK][KQ];
  __shared__ int jj[CHUNK], rr[CHUNK];
  const int lane = threadIdx.x;
  const int64_t blk = xcd_block(n_atoms);
  if (blk < 0) return;
  const int j = int(blk);
  const Lanes L = lane_map<CPL>(lane, nh, lph);
  const float isq = 1.f / sqrtf(float(lph * CPL));
  const Radial R = make_radial(rc);
  const int64_t ld = 3 * int64_t(Da);

  float w[K][CPL];
#pragma unroll
  for (int k = 0; k < K; ++k) ldc<CPL>(Wa_e + int64_t(k) * Da + L.c0, w[k]);
  float kb[CPL], vb[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) kb[c] = vb[c] = 0.f;
  // lane-private partial force and virial over the edges this lane set up
  float fx = 0.f, fy = 0.f, fz = 0.f;
  float vir[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  constexpr int NB = kPrefetch<CPL> ? 2 : 1;
  float qi[NB][UNROLL][CPL], oi[NB][UNROLL][CPL], gg[NB][UNROLL], aa[NB][UNROLL];
  const int r0 = row_ptr[j], r1 = row_ptr[j + 1];
  for (int e0 = r0; e0 < r1; e0 += CHUNK) {
    const int n = min(CHUNK, r1 - e0);
    if (lane < n) {
      const int e = e0 + lane;
      const float4 gm = geom[e];
      const float r = gm.w;
      const float fc = r < rc ? 0.5f * (__cosf(r * R.pi_over_rc) + 1.f) : 0.f;
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) {
        float b[4];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const float x = r - float(4 * kq + qq) * R.mu_step;
          b[qq] = fc * __expf(-R.gamma * x * x);
        }
        phi[lane][kq] = make_float4(b[0], b[1], b[2], b[3]);
      }
      const int re = int(MLIP_IDX(rev[e], row_ptr[n_atoms], "reverse edge"));
      jj[lane] = int(MLIP_IDX(src[e], n_atoms, "sender"));
      rr[lane] = re;
      const float cc = edge_c[e] + edge_c[re];
      const float inv = r > 0.f ? 1.f / r : 0.f;
      const float p = cc * inv;
      fx += p * gm.x;
      fy += p * gm.y;
      fz += p * gm.z;
      vir[0] += p * gm.x * gm.x;
      vir[1] += p * gm.y * gm.y;
      vir[2] += p * gm.z * gm.z;
      vir[3] += p * gm.y * gm.z;
      vir[4] += p * gm.x * gm.z;
      vir[5] += p * gm.x * gm.y;
    }
    __syncthreads();
    // the q and obar rows of the senders and the reverse edges' weights of
    // edges mm .. mm + UNROLL - 1, into set b
    auto fetch = [&](int b, int mm) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int me = min(mm + u, n - 1);
        const int64_t ii = jj[me];
        ldc<CPL>(qkv + ii * ld + L.c0, qi[b][u]);
        ldc<CPL>(obar + ii * Da + L.c0, oi[b][u]);
        const int64_t re = rr[me];
        gg[b][u] = edge_g[re * nh + L.t];
        aa[b][u] = edge_a[re * nh + L.t];
      }
    };
    auto edges = [&](int b, int mm) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (mm + u < n) {
          float e[CPL];
          basis_map<CPL>(phi[mm + u], w, e);
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            kb[c] += gg[b][u] * qi[b][u][c] * e[c];
            vb[c] += aa[b][u] * oi[b][u][c] * e[c];
          }
        }
      }
    };
    if constexpr (NB == 2) {
      fetch(0, 0);
      for (int mm = 0; mm < n; mm += 2 * UNROLL) {
        if (mm + UNROLL < n) fetch(1, mm + UNROLL);
        edges(0, mm);
        if (mm + 2 * UNROLL < n) fetch(0, mm + 2 * UNROLL);
        edges(1, mm + UNROLL);
      }
    } else {
      for (int mm = 0; mm < n; mm += UNROLL) {
        fetch(0, mm);
        edges(0, mm);
      }
    }
    __syncthreads();
  }
  if (L.active) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) kb[c] *= isq;
    stc<CPL>(qkv_bar + int64_t(j) * ld + Da + L.c0, kb);
    stc<CPL>(qkv_bar + int64_t(j) * ld + 2 * Da + L.c0, vb);
  }
  fx = wave_sum(fx);
  fy = wave_sum(fy);
  fz = wave_sum(fz);
#pragma unroll
  for (int qv = 0; qv < 6; ++qv) vir[qv] = wave_sum(vir[qv]);
  if (lane == 0) {
    float *gp = grad_pos + int64_t(j) * 3;
    float *av = atom_virial + int64_t(j) * 6;
    const float g3[3] = {-fx, -fy, -fz};
#pragma unroll
    for (int q = 0; q < 3; ++q) gp[q] = accumulate ? gp[q] + g3[q] : g3[q];
#pragma unroll
    for (int qv = 0; qv < 6; ++qv) av[qv] = accumulate ? av[qv] + 0.5f * vir[qv] : 0.5f * vir[qv];
  }
}

template <int CPL, int LPH>
int launch_all(int which, const AttnArgs &a, hipStream_t stream) {
  const dim3 grid(unsigned(padded_grid(a.n_atoms))), block(64);
  const float4 *g4 = reinterpret_cast<const float4 *>(a.geom);
  if (which == 0) {
    attn_fwd_kernel<CPL, LPH><<<grid, block, 0, stream>>>(a.row_ptr, a.src, g4, a.n_atoms, a.Wa_e, a.qkv,
                                                     a.Da, a.nh, a.lph, a.rc, a.o,
                                                     reinterpret_cast<float2 *>(a.stats));
  } else if (which == 1) {
    attn_vjp_recv_kernel<CPL, LPH><<<grid, block, 0, stream>>>(
        a.row_ptr, a.src, g4, a.n_atoms, a.Wa_e, a.qkv, a.o,
        reinterpret_cast<const float2 *>(a.stats), a.obar, a.Da, a.nh, a.lph, a.rc, a.qkv_bar,
        a.edge_g, a.edge_a, a.edge_c);
  } else {
    attn_vjp_send_kernel<CPL, LPH><<<grid, block, 0, stream>>>(
        a.row_ptr, a.src, a.rev, g4, a.n_atoms, a.Wa_e, a.qkv, a.obar, a.edge_g, a.edge_a,
        a.edge_c, a.Da, a.nh, a.lph, a.rc, a.accumulate, a.qkv_bar, a.grad_pos, a.atom_virial);
  }
  MLIP_LAUNCHED();
  return MLIP_OK;
}

// Layouts whose head width is fixed at compile time (head sums unrolled into
// DPP moves): 8 heads of 48 channels (6 per lane, 8 lanes per head) and 4
// heads of 128 (8 per lane, 16 lanes per head), the widths of the S and M/L
// models.  Every other layout sums heads in a loop over lph.
int dispatch(int which, const AttnArgs &a, hipStream_t stream) {
  switch (a.cpl) {
    case 1: return launch_all<1, 0>(which, a, stream);
    case 2: return launch_all<2, 0>(which, a, stream);
    case 3: return launch_all<3, 0>(which, a, stream);
    case 4: return launch_all<4, 0>(which, a, stream);
    case 6: return a.lph == 8 ? launch_all<6, 8>(which, a, stream) : launch_all<6, 0>(which, a, stream);
    case 8: return a.lph == 16 ? launch_all<8, 16>(which, a, stream) : launch_all<8, 0>(which, a, stream);
    default: break;
  }
  set_error("no attention lane layout for %d channels per lane", a.cpl);
  return MLIP_ERR_UNSUPPORTED;
}

// ------------------------------------------------------------ tangents ---
// Training gradient: derivatives of the forward and of the gradient above
// along a position direction x_dot (with r_dot_e = dhat_e . (x_dot_j - x_dot_i),
// the same on both directions of an edge) and feature tangents q_dot, k_dot,
// v_dot (from h0_dot W_qkv).  With e_dot = r_dot de/dr and f_dot = r_dot f_c':
//   s_dot = sum_t q_dot k e + q k_dot e + q k e_dot        (q scaled by 1/sqrt(dh))
//   a_dot = a s_dot + f_dot w / Z - a T,   T_i^t = sum_l a_il s_dot_il + f_dot_il w_il / Z_i
//   o_dot = sum_j a_dot v e + a (v_dot e + v e_dot)
//         = sum_j (a s_dot + f_dot w / Z) v e + a (v_dot e + v e_dot) - T o   (one pass)
// and, for the gradient, with beta = <obar, o>_t, gbar = a (<obar, v e>_t - beta):
//   gbar_dot = a_dot (<obar, v e> - beta) + a (<obar_dot, v e> + <obar, v_dot e + v e_dot> - beta_dot)
//   qbar_dot_i = sum_j gbar_dot k e + gbar (k_dot e + k e_dot)              (x 1/sqrt(dh))
//   kbar_dot_j = sum_i gbar_dot q e + gbar (q_dot e + q e_dot)              (x 1/sqrt(dh))
//   vbar_dot_j = sum_i a_dot obar e + a (obar_dot e + obar e_dot)
//   ebar = gbar q k + a obar v,  ebar_dot its tangent (written per edge for the
//   Wa_e gradient).  The position part of the gradient's tangent (a Hessian
//   product) is not formed: parameter gradients do not need it.

// radial terms of the chunk's edges for the tangents (lane = edge)
template <int KK>
__device__ inline void tan_radial(const AttnTanArgs &a, const float4 *geom, const Radial &R, int e, int i,
                                  float xi0, float xi1, float xi2, float4 (*phi)[KQ], float4 (*dph)[KQ],
                                  float *fcs, float *fdot, float *rdot, int lane) {
  const float4 gm = geom[e];
  const float r = gm.w;
  const int j = int(MLIP_IDX(a.src[e], a.n_atoms, "sender"));
  float rd = 0.f;
  if (r > 0.f)
    rd = a.x_sign * (gm.x * (a.x_dot[3 * j] - xi0) + gm.y * (a.x_dot[3 * j + 1] - xi1) +
                     gm.z * (a.x_dot[3 * j + 2] - xi2)) / r;
  float fc = 0.f, dfc = 0.f;
  if (r < a.rc) {
    float sn, cs;
    __sincosf(r * R.pi_over_rc, &sn, &cs);
    fc = 0.5f * (cs + 1.f);
    dfc = -0.5f * R.pi_over_rc * sn;
  }
  float ph[KK], dp[KK];
#pragma unroll
  for (int k = 0; k < KK; ++k) {
    const float x = r - float(k) * R.mu_step;
    const float p = __expf(-R.gamma * x * x);
    ph[k] = fc * p;
    dp[k] = dfc * p + fc * (-2.f * R.gamma * x * p);
  }
#pragma unroll
  for (int kq = 0; kq < KQ; ++kq) {
    phi[lane][kq] = make_float4(ph[4 * kq], ph[4 * kq + 1], ph[4 * kq + 2], ph[4 * kq + 3]);
    dph[lane][kq] = make_float4(dp[4 * kq], dp[4 * kq + 1], dp[4 * kq + 2], dp[4 * kq + 3]);
  }
  fcs[lane] = fc;
  fdot[lane] = dfc * rd;
  rdot[lane] = rd;
}

template <int CPL, int LPH>
__global__ void __launch_bounds__(64) attn_jvp_kernel(AttnTanArgs a) {
  __shared__ float4 phi[CHUNK][KQ], dph[CHUNK][KQ];
  __shared__ float fcs[CHUNK], fdot[CHUNK], rdot[CHUNK];
  __shared__ int jj[CHUNK];
  const int lane = threadIdx.x;
  const int64_t blk = xcd_block(a.n_atoms);
  if (blk < 0) return;
  const int i = int(blk);
  const Lanes L = lane_map<CPL>(lane, a.nh, a.lph);
  const int Da = a.Da, nh = a.nh, lph = a.lph;
  const float isq = 1.f / sqrtf(float(lph * CPL));
  const Radial R = make_radial(a.rc);
  const int64_t ld = 3 * int64_t(Da);
  const float on = L.active ? 1.f : 0.f;
  const float4 *geom = reinterpret_cast<const float4 *>(a.geom);

  float w[K][CPL];
#pragma unroll
  for (int k = 0; k < K; ++k) ldc<CPL>(a.Wa_e + int64_t(k) * Da + L.c0, w[k]);
  float q[CPL], qd[CPL], X[CPL];
  ldc<CPL>(a.qkv + int64_t(i) * ld + L.c0, q);
  ldc<CPL>(a.qkv_dot + int64_t(i) * ld + L.c0, qd);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    q[c] *= isq * on;
    qd[c] *= isq * on;
    X[c] = 0.f;
  }
  const float2 st = reinterpret_cast<const float2 *>(a.stats)[int64_t(i) * nh + L.t];
  const float m = L.active ? st.x : 0.f;
  const float invZ = (L.active && st.y > 0.f) ? 1.f / st.y : 0.f;
  const float xi0 = a.x_dot[3 * i], xi1 = a.x_dot[3 * i + 1], xi2 = a.x_dot[3 * i + 2];
  float Tsum = 0.f;
  const int r0 = a.row_ptr[i], r1 = a.row_ptr[i + 1];
  for (int e0 = r0; e0 < r1; e0 += CHUNK) {
    const int n = min(CHUNK, r1 - e0);
    if (lane < n) {
      tan_radial<K>(a, geom, R, e0 + lane, i, xi0, xi1, xi2, phi, dph, fcs, fdot, rdot, lane);
      jj[lane] = int(MLIP_IDX(a.src[e0 + lane], a.n_atoms, "sender"));
    }
    __syncthreads();
    for (int me = 0; me < n; ++me) {
      float kj[CPL], vj[CPL], kd[CPL], vd[CPL];
      const int64_t j = jj[me];
      ldc<CPL>(a.qkv + j * ld + Da + L.c0, kj);
      ldc<CPL>(a.qkv + j * ld + 2 * Da + L.c0, vj);
      ldc<CPL>(a.qkv_dot + j * ld + Da + L.c0, kd);
      ldc<CPL>(a.qkv_dot + j * ld + 2 * Da + L.c0, vd);
      float e[CPL], de[CPL];
      basis_map<CPL>(phi[me], w, e);
      basis_map<CPL>(dph[me], w, de);
      const float rd = rdot[me];
      float ps = 0.f, psd = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        de[c] *= rd;
        ps += q[c] * kj[c] * e[c];
        psd += qd[c] * kj[c] * e[c] + q[c] * kd[c] * e[c] + q[c] * kj[c] * de[c];
      }
      const float s = head_sum<LPH>(ps, lph);
      const float sd = head_sum<LPH>(psd, lph);
      const float wt = __expf(s - m);
      const float al = fcs[me] * wt * invZ;
      const float fw = fdot[me] * wt * invZ;
      Tsum += al * sd + fw;
      const float cf = al * sd + fw;
#pragma unroll
      for (int c = 0; c < CPL; ++c) X[c] += cf * vj[c] * e[c] + al * (vd[c] * e[c] + vj[c] * de[c]);
    }
    __syncthreads();
  }
  if (L.active) {
    float oo[CPL], od[CPL];
    ldc<CPL>(a.o + int64_t(i) * Da + L.c0, oo);
#pragma unroll
    for (int c = 0; c < CPL; ++c) od[c] = X[c] - Tsum * oo[c];
    stc<CPL>(a.o_dot + int64_t(i) * Da + L.c0, od);
    if (lane == L.t * lph) a.tstat[int64_t(i) * nh + L.t] = Tsum;
  }
}

template <int CPL, int LPH>
__global__ void __launch_bounds__(64) attn_tvjp_recv_kernel(AttnTanArgs a) {
  __shared__ float4 phi[CHUNK][KQ], dph[CHUNK][KQ];
  __shared__ float fcs[CHUNK], fdot[CHUNK], rdot[CHUNK];
  __shared__ int jj[CHUNK];
  const int lane = threadIdx.x;
  const int64_t blk = xcd_block(a.n_atoms);
  if (blk < 0) return;
  const int i = int(blk);
  const Lanes L = lane_map<CPL>(lane, a.nh, a.lph);
  const int Da = a.Da, nh = a.nh, lph = a.lph;
  const float isq = 1.f / sqrtf(float(lph * CPL));
  const Radial R = make_radial(a.rc);
  const int64_t ld = 3 * int64_t(Da);
  const float on = L.active ? 1.f : 0.f;
  const float4 *geom = reinterpret_cast<const float4 *>(a.geom);

  float w[K][CPL];
#pragma unroll
  for (int k = 0; k < K; ++k) ldc<CPL>(a.Wa_e + int64_t(k) * Da + L.c0, w[k]);
  float q[CPL], qd[CPL], ob[CPL], obd[CPL], qbd[CPL];
  float bp = 0.f, bpd = 0.f;
  {
    float oo[CPL], od[CPL];
    ldc<CPL>(a.qkv + int64_t(i) * ld + L.c0, q);
    ldc<CPL>(a.qkv_dot + int64_t(i) * ld + L.c0, qd);
    ldc<CPL>(a.obar + int64_t(i) * Da + L.c0, ob);
    ldc<CPL>(a.obar_dot + int64_t(i) * Da + L.c0, obd);
    ldc<CPL>(a.o + int64_t(i) * Da + L.c0, oo);
    ldc<CPL>(a.o_dot + int64_t(i) * Da + L.c0, od);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      q[c] *= isq * on;
      qd[c] *= isq * on;
      ob[c] *= on;
      obd[c] *= on;
      bp += ob[c] * oo[c];
      bpd += obd[c] * oo[c] + ob[c] * od[c];
      qbd[c] = 0.f;
    }
  }
  const float beta = head_sum<LPH>(bp, lph);
  const float betad = head_sum<LPH>(bpd, lph);
  const float2 st = reinterpret_cast<const float2 *>(a.stats)[int64_t(i) * nh + L.t];
  const float m = L.active ? st.x : 0.f;
  const float invZ = (L.active && st.y > 0.f) ? 1.f / st.y : 0.f;
  const float T = L.active ? a.tstat[int64_t(i) * nh + L.t] : 0.f;
  const bool head_lead = L.active && lane == L.t * lph;
  const float xi0 = a.x_dot[3 * i], xi1 = a.x_dot[3 * i + 1], xi2 = a.x_dot[3 * i + 2];
  const int r0 = a.row_ptr[i], r1 = a.row_ptr[i + 1];
  for (int e0 = r0; e0 < r1; e0 += CHUNK) {
    const int n = min(CHUNK, r1 - e0);
    if (lane < n) {
      tan_radial<K>(a, geom, R, e0 + lane, i, xi0, xi1, xi2, phi, dph, fcs, fdot, rdot, lane);
      jj[lane] = int(MLIP_IDX(a.src[e0 + lane], a.n_atoms, "sender"));
    }
    __syncthreads();
    for (int me = 0; me < n; ++me) {
      float kj[CPL], vj[CPL], kd[CPL], vd[CPL];
      const int64_t j = jj[me];
      ldc<CPL>(a.qkv + j * ld + Da + L.c0, kj);
      ldc<CPL>(a.qkv + j * ld + 2 * Da + L.c0, vj);
      ldc<CPL>(a.qkv_dot + j * ld + Da + L.c0, kd);
      ldc<CPL>(a.qkv_dot + j * ld + 2 * Da + L.c0, vd);
      float e[CPL], de[CPL];
      basis_map<CPL>(phi[me], w, e);
      basis_map<CPL>(dph[me], w, de);
      const float rd = rdot[me];
      float ps = 0.f, psd = 0.f, pa = 0.f, pad = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        de[c] *= rd;
        ps += q[c] * kj[c] * e[c];
        psd += qd[c] * kj[c] * e[c] + q[c] * kd[c] * e[c] + q[c] * kj[c] * de[c];
        pa += ob[c] * vj[c] * e[c];
        pad += obd[c] * vj[c] * e[c] + ob[c] * vd[c] * e[c] + ob[c] * vj[c] * de[c];
      }
      const float s = head_sum<LPH>(ps, lph);
      const float sd = head_sum<LPH>(psd, lph);
      const float ab = head_sum<LPH>(pa, lph);
      const float abd = head_sum<LPH>(pad, lph);
      const float wt = __expf(s - m);
      const float al = fcs[me] * wt * invZ;
      const float ald = al * sd + fdot[me] * wt * invZ - al * T;
      const float diff = ab - beta;
      const float g = al * diff;
      const float gd = ald * diff + al * (abd - betad);
      float eb[CPL], ebd[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        qbd[c] += gd * kj[c] * e[c] + g * (kd[c] * e[c] + kj[c] * de[c]);
        eb[c] = g * q[c] * kj[c] + al * ob[c] * vj[c];
        ebd[c] = gd * q[c] * kj[c] + g * (qd[c] * kj[c] + q[c] * kd[c]) + ald * ob[c] * vj[c] +
                 al * (obd[c] * vj[c] + ob[c] * vd[c]);
      }
      const int64_t eg = int64_t(e0 + me);
      if (L.active) {
        stc<CPL>(a.ebar + eg * Da + L.c0, eb);
        stc<CPL>(a.ebar_dot + eg * Da + L.c0, ebd);
      }
      if (head_lead) {
        a.edge_g[eg * nh + L.t] = g;
        a.edge_gd[eg * nh + L.t] = gd;
        a.edge_a[eg * nh + L.t] = al;
        a.edge_ad[eg * nh + L.t] = ald;
      }
    }
    __syncthreads();
  }
  if (L.active) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) qbd[c] *= isq;
    stc<CPL>(a.qkv_bar_dot + int64_t(i) * ld + L.c0, qbd);
  }
}

template <int CPL, int LPH>
__global__ void __launch_bounds__(64) attn_tvjp_send_kernel(AttnTanArgs a) {
  __shared__ float4 phi[CHUNK][KQ], dph[CHUNK][KQ];
  __shared__ float fcs[CHUNK], fdot[CHUNK], rdot[CHUNK];
  __shared__ int jj[CHUNK], rr[CHUNK];
  const int lane = threadIdx.x;
  const int64_t blk = xcd_block(a.n_atoms);
  if (blk < 0) return;
  const int j = int(blk);
  const Lanes L = lane_map<CPL>(lane, a.nh, a.lph);
  const int Da = a.Da, nh = a.nh, lph = a.lph;
  const float isq = 1.f / sqrtf(float(lph * CPL));
  const Radial R = make_radial(a.rc);
  const int64_t ld = 3 * int64_t(Da);
  const float4 *geom = reinterpret_cast<const float4 *>(a.geom);

  float w[K][CPL];
#pragma unroll
  for (int k = 0; k < K; ++k) ldc<CPL>(a.Wa_e + int64_t(k) * Da + L.c0, w[k]);
  float kbd[CPL], vbd[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) kbd[c] = vbd[c] = 0.f;
  const float xj0 = a.x_dot[3 * j], xj1 = a.x_dot[3 * j + 1], xj2 = a.x_dot[3 * j + 2];
  const int r0 = a.row_ptr[j], r1 = a.row_ptr[j + 1];
  for (int e0 = r0; e0 < r1; e0 += CHUNK) {
    const int n = min(CHUNK, r1 - e0);
    if (lane < n) {
      tan_radial<K>(a, geom, R, e0 + lane, j, xj0, xj1, xj2, phi, dph, fcs, fdot, rdot, lane);
      jj[lane] = int(MLIP_IDX(a.src[e0 + lane], a.n_atoms, "sender"));
      rr[lane] = int(MLIP_IDX(a.rev[e0 + lane], a.row_ptr[a.n_atoms], "reverse edge"));
    }
    __syncthreads();
    for (int me = 0; me < n; ++me) {
      // edge j <- i; its reverse i <- j carries the receiver-pass values
      const int64_t ii = jj[me];
      const int64_t re = rr[me];
      float qi[CPL], qdi[CPL], oi[CPL], odi[CPL];
      ldc<CPL>(a.qkv + ii * ld + L.c0, qi);
      ldc<CPL>(a.qkv_dot + ii * ld + L.c0, qdi);
      ldc<CPL>(a.obar + ii * Da + L.c0, oi);
      ldc<CPL>(a.obar_dot + ii * Da + L.c0, odi);
      const float g = a.edge_g[re * nh + L.t], gd = a.edge_gd[re * nh + L.t];
      const float al = a.edge_a[re * nh + L.t], ald = a.edge_ad[re * nh + L.t];
      float e[CPL], de[CPL];
      basis_map<CPL>(phi[me], w, e);
      basis_map<CPL>(dph[me], w, de);
      const float rd = rdot[me];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        de[c] *= rd;
        kbd[c] += gd * qi[c] * e[c] + g * (qdi[c] * e[c] + qi[c] * de[c]);
        vbd[c] += ald * oi[c] * e[c] + al * (odi[c] * e[c] + oi[c] * de[c]);
      }
    }
    __syncthreads();
  }
  if (L.active) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) kbd[c] *= isq;
    stc<CPL>(a.qkv_bar_dot + int64_t(j) * ld + Da + L.c0, kbd);
    stc<CPL>(a.qkv_bar_dot + int64_t(j) * ld + 2 * Da + L.c0, vbd);
  }
}

template <int CPL, int LPH>
int launch_tan(int which, const AttnTanArgs &a, hipStream_t stream) {
  const dim3 grid(unsigned(padded_grid(a.n_atoms))), block(64);
  if (which == 0) attn_jvp_kernel<CPL, LPH><<<grid, block, 0, stream>>>(a);
  else if (which == 1) attn_tvjp_recv_kernel<CPL, LPH><<<grid, block, 0, stream>>>(a);
  else attn_tvjp_send_kernel<CPL, LPH><<<grid, block, 0, stream>>>(a);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

int dispatch_tan(int which, const AttnTanArgs &a, hipStream_t stream) {
  switch (a.cpl) {
    case 1: return launch_tan<1, 0>(which, a, stream);
    case 2: return launch_tan<2, 0>(which, a, stream);
    case 3: return launch_tan<3, 0>(which, a, stream);
    case 4: return launch_tan<4, 0>(which, a, stream);
    case 6: return a.lph == 8 ? launch_tan<6, 8>(which, a, stream) : launch_tan<6, 0>(which, a, stream);
    case 8: return a.lph == 16 ? launch_tan<8, 16>(which, a, stream) : launch_tan<8, 0>(which, a, stream);
    default: break;
  }
  set_error("no attention lane layout for %d channels per lane", a.cpl);
  return MLIP_ERR_UNSUPPORTED;
}

}  // namespace

int attn_lane_layout(int Da, int nh, int *cpl, int *lph) {
  if (nh < 1 || Da % nh) return MLIP_ERR_INVALID;
  const int dh = Da / nh;
  const int options[] = {1, 2, 3, 4, 6, 8};
  for (int c : options) {
    if (dh % c) continue;
    const int l = dh / c;
    if ((l & (l - 1)) != 0 || int64_t(nh) * l > 64) continue;
    *cpl = c;
    *lph = l;
    return MLIP_OK;
  }
  return MLIP_ERR_UNSUPPORTED;
}

int launch_attn_fwd(const AttnArgs &a, hipStream_t stream) {
  if (a.n_atoms <= 0) return MLIP_OK;
  ProfScope ps(K_ATTN_FWD, stream);
  return dispatch(0, a, stream);
}

int launch_attn_vjp(const AttnArgs &a, hipStream_t stream) {
  if (a.n_atoms <= 0) return MLIP_OK;
  {
    ProfScope ps(K_ATTN_VJP_RECV, stream);
    if (int rc = dispatch(1, a, stream)) return rc;
  }
  ProfScope ps(K_ATTN_VJP_SEND, stream);
  return dispatch(2, a, stream);
}

int launch_attn_jvp(const AttnTanArgs &a, hipStream_t stream) {
  if (a.n_atoms <= 0) return MLIP_OK;
  ProfScope ps(K_ATTN_TAN, stream);
  return dispatch_tan(0, a, stream);
}

int launch_attn_tvjp(const AttnTanArgs &a, hipStream_t stream) {
  if (a.n_atoms <= 0) return MLIP_OK;
  ProfScope ps(K_ATTN_TAN, stream);
  if (int rc = dispatch_tan(1, a, stream)) return rc;
  return dispatch_tan(2, a, stream);
}

}  // namespace mlip
