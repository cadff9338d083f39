// Element-type routing, element-grouped token dispatch, gate-weighted
// combine, and the linear readout.
//
// Routing is static per element type (ScienceAI article, architecture
// section; paper review of "Breaking the Training Barrier of
// Billion-Parameter Universal MLIPs", section 3.2): every atom of type t goes
// to the same k experts with the same gates, so the routing table is T x k
// and the dispatch is a counting sort of atoms by type.  Tokens (atom, rank)
// are laid out by (expert, element, atom) with prefix-sum offsets; the
// positions are computed, not claimed with atomics, so the layout is
// deterministic.  The combine gathers each atom's k expert outputs in rank
// order, so no scatter (and no write contention) is needed at all.
#include "common.h"

namespace mlip {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int RANK_BLOCK = 256;

// top-k per element type (ties -> lower expert index) and softmax gates.
// One wavefront per type: the row of logits sits in registers (up to 16 per
// lane), and each of the k picks is a wavefront arg-max.  A NaN logit ranks
// below every number, so the k picks are always distinct.
constexpr int ROUTE_MAX_X = 1024;
__global__ void __launch_bounds__(64) route_kernel(const float *__restrict__ logits, int T, int X,
                                                   int k, int32_t *__restrict__ topk,
                                                   float *__restrict__ gate) {
  constexpr int PER = ROUTE_MAX_X / 64;
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  if (t >= T) return;
  const float *l = logits + int64_t(t) * X;
  float v[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    const int x = lane + 64 * c;
    float w = x < X ? l[x] : -INFINITY;
    v[c] = (w != w) ? -INFINITY : w;
  }
  unsigned taken = 0;
  float first = 0.f, sum = 0.f;
  for (int r = 0; r < k; ++r) {
    int bx = 0x7fffffff;
    float bv = -INFINITY;
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const int x = lane + 64 * c;
      if (x < X && !((taken >> c) & 1u) && (bx == 0x7fffffff || v[c] > bv)) {
        bv = v[c];
        bx = x;
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const float ov = __shfl_xor(bv, d, 64);
      const int ox = __shfl_xor(bx, d, 64);
      if (ox != 0x7fffffff && (bx == 0x7fffffff || ov > bv || (ov == bv && ox < bx))) {
        bv = ov;
        bx = ox;
      }
    }
    if ((bx & 63) == lane) taken |= 1u << (bx >> 6);
    if (r == 0) first = bv;
    const float w = expf(bv - first);
    sum += w;
    if (lane == 0) {
      topk[int64_t(t) * k + r] = bx;
      gate[int64_t(t) * k + r] = w;
    }
  }
  __syncthreads();
  const float inv = 1.f / sum;
  for (int r = lane; r < k; r += 64) gate[int64_t(t) * k + r] *= inv;
}

__global__ void moe_fill_i32(int32_t *p, int64_t n, int32_t v) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Per block of 256 atoms: rank of each atom among the earlier atoms of the
// same type in the block, and the block's per-type counts.
__global__ void __launch_bounds__(RANK_BLOCK) elem_rank_kernel(const int32_t *__restrict__ z, int N,
                                                               int T, int32_t *__restrict__ local_rank,
                                                               int32_t *__restrict__ blk_count,
                                                               int32_t *__restrict__ flags) {
  __shared__ int zs[RANK_BLOCK];
  extern __shared__ int hist[];
  const int i = blockIdx.x * RANK_BLOCK + threadIdx.x;
  for (int t = threadIdx.x; t < T; t += RANK_BLOCK) hist[t] = 0;
  int zi = -1;
  if (i < N) {
    zi = z[i];
    if (zi < 0 || zi >= T) {
      atomicOr(flags, 1);
      zi = zi < 0 ? 0 : T - 1;
    }
  }
  zs[threadIdx.x] = zi;
  __syncthreads();
  if (i < N) {
    int r = 0;
    for (int q = 0; q < int(threadIdx.x); ++q) r += zs[q] == zi;
    local_rank[i] = r;
    atomicAdd(&hist[zi], 1);
  }
  __syncthreads();
  for (int t = threadIdx.x; t < T; t += RANK_BLOCK) blk_count[int64_t(blockIdx.x) * T + t] = hist[t];
}

// One workgroup: per-type block offsets (in place), type counts, the
// (expert, type) offset table and the expert offsets.
// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ inline int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// One workgroup of 256 threads builds the dispatch tables:
//  1. per type t, the exclusive scan of the per-block type counts over the
//     atom blocks (in place) and the type total n_type[t]; one wavefront per
//     type, 64 blocks per pass;
//  2. per expert x, pre[x][t] = the tokens of types t' < t routed to x, and
//     exp_count[x]; the routing table and n_type are read from LDS when the
//     table fits (TKS entries), else from global memory;
//  3. exp_off = the exclusive scan of exp_count (a block scan).
constexpr int TKS = 4096;
__global__ void __launch_bounds__(256) dispatch_tables_kernel(
    int n_blocks, int T, int X, int k, const int32_t *__restrict__ topk,
    int32_t *__restrict__ blk_count, int32_t *__restrict__ n_type, int32_t *__restrict__ pre,
    int32_t *__restrict__ exp_count, int32_t *__restrict__ exp_off) {
  __shared__ int s_ntype[TKS];
  __shared__ int s_topk[TKS];
  __shared__ int s_wave[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool in_lds = T <= TKS && int64_t(T) * k <= TKS;
  for (int t = wave; t < T; t += 4) {
    int run = 0;
    for (int b0 = 0; b0 < n_blocks; b0 += 64) {
      const int b = b0 + lane;
      const int64_t o = int64_t(b) * T + t;
      const int c = b < n_blocks ? blk_count[o] : 0;
      const int incl = wave_incl_scan(c);
      if (b < n_blocks) blk_count[o] = run + incl - c;
      run += __shfl(incl, 63, 64);
    }
    if (lane == 0) {
      n_type[t] = run;
      if (in_lds) s_ntype[t] = run;
    }
  }
  if (in_lds)
    for (int q = tid; q < T * k; q += 256) s_topk[q] = topk[q];
  __threadfence_block();
  __syncthreads();
  const int32_t *tk = in_lds ? s_topk : topk;
  const int32_t *nt = in_lds ? s_ntype : n_type;
  for (int x = tid; x < X; x += 256) {
    int run = 0;
    for (int t = 0; t < T; ++t) {
      pre[int64_t(x) * T + t] = run;
      bool hit = false;
      for (int r = 0; r < k; ++r) hit |= tk[t * k + r] == x;
      if (hit) run += nt[t];
    }
    exp_count[x] = run;
  }
  __threadfence_block();
  __syncthreads();
  // exclusive scan of exp_count over the experts, 256 at a time
  int base = 0;
  for (int x0 = 0; x0 < X; x0 += 256) {
    const int x = x0 + tid;
    const int c = x < X ? exp_count[x] : 0;
    const int incl = wave_incl_scan(c);
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int before = base;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    if (x < X) exp_off[x] = before + incl - c;
    const int total = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
    __syncthreads();
    base += total;
  }
  if (tid == 0) exp_off[X] = base;
}

__global__ void dispatch_scatter_kernel(const int32_t *__restrict__ z, int N, int T, int k,
                                        const int32_t *__restrict__ topk,
                                        const int32_t *__restrict__ local_rank,
                                        const int32_t *__restrict__ blk_base,
                                        const int32_t *__restrict__ pre,
                                        const int32_t *__restrict__ exp_off,
                                        int32_t *__restrict__ tok_atom, int32_t *__restrict__ slot) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  int t = z[i];
  t = t < 0 ? 0 : (t >= T ? T - 1 : t);
  const int rank = blk_base[int64_t(i / RANK_BLOCK) * T + t] + local_rank[i];
  for (int r = 0; r < k; ++r) {
    const int x = topk[t * k + r];
    const int p = exp_off[x] + pre[int64_t(x) * T + t] + rank;
    tok_atom[p] = i;
    slot[int64_t(i) * k + r] = p;
  }
}

// out_i = base_i + sum_r gate[z_i, r] * rows[slot(i, r)], r in rank order
// (base may be null: 0).  Two wavefronts per atom, each on alternate 64-wide
// float4 column chunks; the atom's k gates and row indices are uniform (scalar
// loads), and all k + 1 rows of a column chunk are loaded before they are
// summed.  KT > 0: k fixed at compile time.
template <int KT>
__global__ void __launch_bounds__(256) combine_kernel(const float *__restrict__ base,
                                                      const float *__restrict__ rows,
                                                      const int32_t *__restrict__ z,
                                                      const float *__restrict__ gate,
                                                      const int32_t *__restrict__ slot, int N, int T,
                                                      int k_rt, int D, float *__restrict__ out) {
  constexpr int KMAX = KT > 0 ? KT : 1;
  const int i = blockIdx.x * 2 + (threadIdx.x >> 7);
  if (i >= N) return;
  const int lane = threadIdx.x & 127;   // column chunk offset of this wavefront pair
  const int k = KT > 0 ? KT : k_rt;
  int t = z[i];
  t = t < 0 ? 0 : (t >= T ? T - 1 : t);
  const int D4 = D >> 2;
  const float4 *b4 = base ? reinterpret_cast<const float4 *>(base + int64_t(i) * D) : nullptr;
  float4 *o4 = reinterpret_cast<float4 *>(out + int64_t(i) * D);
  if (KT > 0) {
    float gv[KMAX];
    const floatx4 *y4[KMAX];
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      gv[r] = gate[t * KMAX + r];
      y4[r] = reinterpret_cast<const floatx4 *>(
          rows + MLIP_IDX(slot[int64_t(i) * KMAX + r], int64_t(N) * KMAX, "dispatch slot") * D);
    }
    for (int c = lane; c < D4; c += 128) {
      float4 acc = b4 ? b4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      floatx4 y[KMAX];
#pragma unroll
      for (int r = 0; r < KMAX; ++r) y[r] = __builtin_nontemporal_load(y4[r] + c);
#pragma unroll
      for (int r = 0; r < KMAX; ++r) {
        acc.x += gv[r] * y[r][0];
        acc.y += gv[r] * y[r][1];
        acc.z += gv[r] * y[r][2];
        acc.w += gv[r] * y[r][3];
      }
      o4[c] = acc;
    }
  } else {
    for (int c = lane; c < D4; c += 128) {
      float4 acc = b4 ? b4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      for (int r = 0; r < k; ++r) {
        const float gv = gate[t * k + r];
        const float4 y = reinterpret_cast<const float4 *>(
            rows + MLIP_IDX(slot[int64_t(i) * k + r], int64_t(N) * k, "dispatch slot") * D)[c];
        acc.x += gv * y.x;
        acc.y += gv * y.y;
        acc.z += gv * y.z;
        acc.w += gv * y.w;
      }
      o4[c] = acc;
    }
  }
}

// eps_i = h_i . w_r (one wavefront per atom).
__global__ void __launch_bounds__(256) readout_eps_kernel(const float *__restrict__ h,
                                                          const float *__restrict__ w, int N, int D,
                                                          float *__restrict__ eps) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= N) return;
  const int lane = threadIdx.x & 63;
  float acc = 0.f;
  const float4 *hr = reinterpret_cast<const float4 *>(h + int64_t(i) * D);
  const float4 *wr = reinterpret_cast<const float4 *>(w);
  for (int c = lane; c < (D >> 2); c += 64) {
    const float4 a = hr[c], b = wr[c];
    acc += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
  if (lane == 0) eps[i] = acc;
}

// E_b = sum of eps over structure b, in float64 with a fixed reduction tree.
__global__ void __launch_bounds__(256) readout_energy_kernel(const float *__restrict__ eps,
                                                             const int32_t *__restrict__ struct_ptr,
                                                             int n_atoms, double *__restrict__ energy) {
  __shared__ double part[256];
  const int b = blockIdx.x;
  // clamped into [0, n_atoms): a malformed struct_ptr cannot read past eps
  const int lo = min(max(struct_ptr[b], 0), n_atoms);
  const int hi = min(max(struct_ptr[b + 1], lo), n_atoms);
  double acc = 0.0;
  for (int i = lo + threadIdx.x; i < hi; i += 256) acc += double(eps[i]);
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s >= 1; s >>= 1) {
    if (int(threadIdx.x) < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) energy[b] = part[0];
}

}  // namespace

int moe_route_dispatch(const int32_t *z, const float *logits, int N, int T, int X, int k,
                       int32_t *topk, float *gate, int32_t *exp_off, int32_t *tok_atom,
                       int32_t *slot, int32_t *local_rank, int32_t *blk_count, int32_t *n_type,
                       int32_t *pre, int32_t *exp_count, int32_t *flags, hipStream_t stream) {
  ProfScope ps(K_ROUTE_DISPATCH, stream);
  route_kernel<<<dim3(unsigned(T)), dim3(64), 0, stream>>>(logits, T, X, k, topk, gate);
  MLIP_LAUNCHED();
  moe_fill_i32<<<1, 64, 0, stream>>>(flags, 1, 0);
  MLIP_LAUNCHED();
  const int n_blocks = int(cdiv(N, RANK_BLOCK));
  if (N > 0) {
    elem_rank_kernel<<<dim3(unsigned(n_blocks)), dim3(RANK_BLOCK), size_t(T) * sizeof(int), stream>>>(
        z, N, T, local_rank, blk_count, flags);
    MLIP_LAUNCHED();
  }
  dispatch_tables_kernel<<<1, 256, 0, stream>>>(n_blocks, T, X, k, topk, blk_count, n_type, pre,
                                                exp_count, exp_off);
  MLIP_LAUNCHED();
  if (N > 0) {
    dispatch_scatter_kernel<<<dim3(unsigned(cdiv(N, 256))), dim3(256), 0, stream>>>(
        z, N, T, k, topk, local_rank, blk_count, pre, exp_off, tok_atom, slot);
    MLIP_LAUNCHED();
  }
  return MLIP_OK;
}

int moe_combine(const float *base, const float *rows, const int32_t *z, const float *gate,
                const int32_t *slot, int N, int T, int k, int D, float *out, hipStream_t stream) {
  if (N <= 0) return MLIP_OK;
  ProfScope ps(K_COMBINE, stream);
  const dim3 grid(unsigned(cdiv(N, 2))), block(256);
#define MLIP_COMBINE(KV) combine_kernel<KV><<<grid, block, 0, stream>>>(base, rows, z, gate, slot, N, T, k, D, out)
  switch (k) {
    case 1: MLIP_COMBINE(1); break;
    case 2: MLIP_COMBINE(2); break;
    case 4: MLIP_COMBINE(4); break;
    case 8: MLIP_COMBINE(8); break;
    case 16: MLIP_COMBINE(16); break;
    default: MLIP_COMBINE(0); break;
  }
#undef MLIP_COMBINE
  MLIP_LAUNCHED();
  return MLIP_OK;
}

// h[i] = table[z[i]] (float4 columns; rows of an out-of-range type are zero).
__global__ void __launch_bounds__(256) embed_atoms_kernel(const int32_t *__restrict__ z,
                                                          const float4 *__restrict__ table, int N, int T,
                                                          int D4, float4 *__restrict__ h) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= int64_t(N) * D4) return;
  const int i = int(idx / D4), c = int(idx - int64_t(i) * D4);
  const int t = z[i];
  h[idx] = (t >= 0 && t < T) ? table[int64_t(t) * D4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
}

int embed_atoms(const int32_t *z, const float *table, int N, int T, int D, float *h,
                hipStream_t stream) {
  const int D4 = D / 4;
  embed_atoms_kernel<<<dim3(unsigned(cdiv(int64_t(N) * D4, 256))), dim3(256), 0, stream>>>(
      z, reinterpret_cast<const float4 *>(table), N, T, D4, reinterpret_cast<float4 *>(h));
  MLIP_LAUNCHED();
  return MLIP_OK;
}

// d_table[t] = sum over atoms with z_i = t of grad_h_i (atoms in index order;
// one thread per (type, float4 column), the type test is uniform per wave).
__global__ void __launch_bounds__(64) embed_grad_kernel(const int32_t *__restrict__ z,
                                                        const float4 *__restrict__ grad_h, int N, int D4,
                                                        float4 *__restrict__ d_table) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * 64 + threadIdx.x;
  if (c >= D4) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i = 0; i < N; ++i) {
    if (z[i] != t) continue;
    const float4 v = grad_h[int64_t(i) * D4 + c];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  d_table[int64_t(t) * D4 + c] = acc;
}

int embed_grad(const int32_t *z, const float *grad_h, int N, int T, int D, float *d_table,
               hipStream_t stream) {
  ProfScope ps(K_MOE_TAN, stream);
  const int D4 = D / 4;
  embed_grad_kernel<<<dim3(unsigned(cdiv(D4, 64)), unsigned(T)), dim3(64), 0, stream>>>(
      z, reinterpret_cast<const float4 *>(grad_h), N, D4, reinterpret_cast<float4 *>(d_table));
  MLIP_LAUNCHED();
  return MLIP_OK;
}

int readout(const float *h, const float *w_r, const int32_t *struct_ptr, int N, int B, int D,
            float *eps, double *energy, hipStream_t stream) {
  ProfScope ps(K_READOUT, stream);
  if (N > 0) {
    readout_eps_kernel<<<dim3(unsigned(cdiv(N, 4))), dim3(256), 0, stream>>>(h, w_r, N, D, eps);
    MLIP_LAUNCHED();
  }
  readout_energy_kernel<<<dim3(unsigned(B)), dim3(256), 0, stream>>>(eps, struct_ptr, N, energy);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

}  // namespace mlip
