// Periodic radius graph on the GPU: cell list, per-receiver neighbour count,
// CSR scan, per-receiver fill in canonical order, reverse-edge index.
//
// The graph follows the paper review of "Breaking the Training Barrier of
// Billion-Parameter Universal MLIPs", section 3.1, Figure 1(a) (graph under
// periodic repetition).  The edge predicate is the float64 formula written
// in mlip.h; every double operation below is an explicit round-to-nearest
// intrinsic so the compiler cannot contract or reorder it, which makes the
// edge set identical to any other evaluation of the same formula.
//
// Cell list in fractional coordinates f = x C^-1 (rows of C are the lattice
// vectors; any cell with non-zero volume, either handedness).  w_a, the distance between the
// lattice planes spanned by the other two vectors, sets the bins along axis
// a: with n_a = floor(w_a / r_c) >= 3 bins every bin is at least r_c thick,
// so the candidates of an atom are the atoms of its own and the two adjacent
// bins per axis (wrapping across the cell with a shift of +-1).  Along an
// axis with fewer than three bins there is one bin, and a candidate's image
// shifts S_a are those with |d . n_a| < r_c for the plane normal n_a, i.e.
// S_a in [-r_c/w_a - (f_j - f_i)_a, r_c/w_a - (f_j - f_i)_a] (widened by 1e-9).
// For orthorhombic cells f_a = x_a / L_a and w_a = L_a.
#include <thread>

#include "common.h"

namespace mlip {

namespace {

constexpr int kMaxDeg = 1024;     // edges per row held in LDS by the fill pass
constexpr int kMaxImages = 8;     // |S| bound along a short axis

enum GraphFlags {
  GF_BAD_CELL = 2,
  GF_POS_OUTSIDE = 4,
  GF_TOO_MANY_IMAGES = 8,
  GF_REV_MISSING = 16,
  GF_BAD_STRUCTS = 32,   // struct_ptr not 0 = p_0 <= p_1 <= ... <= p_B = n_atoms
  GF_BAD_SRC = 64,       // a caller-supplied sender index outside [0, n_atoms)
};

// Every pass after the setup skips its work when the structure table was
// rejected, so a malformed struct_ptr never turns into an index.
__device__ inline bool structs_rejected(const int32_t *flags) {
  return (__atomic_load_n(flags, __ATOMIC_RELAXED) & GF_BAD_STRUCTS) != 0;
}

// accepted rounding of a general cell's fractional coordinates outside [0, 1)
constexpr double kFracTol = 1e-6;

struct StructParams {
  double C[9];     // lattice vectors as rows
  double Ci[9];    // C^-1: fractional coordinates f = x C^-1 (row vectors)
  double w[3];     // lattice-plane spacings (cell edge for orthorhombic cells)
  int ortho;       // diagonal cell: f_a = x_a / C_aa exactly
  int lo, hi;      // atom range
  int nb[3];       // bins per axis (1 = image mode)
  int nimg[3];     // image range for image-mode axes
  int bin_base;    // first global bin id
  int valid;
};

// Zeroes the flags, the degree maximum and the two bin counters in one launch.
__global__ void graph_zero(int32_t *__restrict__ flags, int32_t *__restrict__ maxdeg,
                           int32_t *__restrict__ bin_count, int32_t *__restrict__ bin_fill,
                           int64_t nbins) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < 4) {
    flags[i] = 0;
    maxdeg[i] = 0;
  }
  if (i < nbins) {
    bin_count[i] = 0;
    bin_fill[i] = 0;
  }
}

__global__ void graph_setup(const float *__restrict__ cell, const int32_t *__restrict__ struct_ptr,
                            int n_structs, int n_atoms, float cutoff, StructParams *__restrict__ prm,
                            int32_t *__restrict__ flags) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= n_structs) return;
  StructParams P;
  for (int q = 0; q < 9; ++q) P.C[q] = double(cell[b * 9 + q]);
  P.lo = struct_ptr[b];
  P.hi = struct_ptr[b + 1];
  // the table must run 0 = p_0 <= p_1 <= ... <= p_B = n_atoms; each thread
  // checks its own pair, the first and the last thread the two ends
  if (!(P.lo >= 0 && P.lo <= P.hi && P.hi <= n_atoms) || (b == 0 && P.lo != 0) ||
      (b == n_structs - 1 && P.hi != n_atoms)) {
    P.lo = P.hi = 0;
    atomicOr(flags, GF_BAD_STRUCTS);
  }
  P.bin_base = P.lo + b;
  int f = 0;
  const double rc = double(cutoff);
  const double *C = P.C;
  P.ortho = 1;
  for (int a = 0; a < 3; ++a)
    for (int c = 0; c < 3; ++c) {
      if (c != a && C[a * 3 + c] != 0.0) P.ortho = 0;
      if (!(fabs(C[a * 3 + c]) < 1e30)) f |= GF_BAD_CELL;
    }
  // cross products of the rows: X[a] = C[a+1] x C[a+2]; det = C[0] . X[0]
  double X[9];
  for (int a = 0; a < 3; ++a) {
    const double *u = C + ((a + 1) % 3) * 3, *v = C + ((a + 2) % 3) * 3;
    X[a * 3 + 0] = u[1] * v[2] - u[2] * v[1];
    X[a * 3 + 1] = u[2] * v[0] - u[0] * v[2];
    X[a * 3 + 2] = u[0] * v[1] - u[1] * v[0];
  }
  // either handedness is a valid basis; only a flat (or non-finite) cell is not
  const double det = C[0] * X[0] + C[1] * X[1] + C[2] * X[2];
  if (!(fabs(det) > 0.0) || !(fabs(det) < 1e300)) f |= GF_BAD_CELL;
  for (int a = 0; a < 3; ++a) {
    // C^-1 has the cross products as columns: (C^-1)_{c,a} = X[a]_c / det
    for (int c = 0; c < 3; ++c) P.Ci[c * 3 + a] = X[a * 3 + c] / det;
    const double nx = sqrt(X[a * 3] * X[a * 3] + X[a * 3 + 1] * X[a * 3 + 1] + X[a * 3 + 2] * X[a * 3 + 2]);
    P.w[a] = P.ortho ? C[a * 3 + a] : fabs(det) / nx;
    if (!(P.w[a] > 0.0)) f |= GF_BAD_CELL;
  }
  int n_b = P.hi - P.lo;
  if (f == 0) {
    int64_t cap = n_b > 1 ? n_b : 1;
    // a general cell accepts fractional coordinates up to kFracTol outside
    // [0, 1) and clamps them into the edge bins; the bins are thickened so a
    // pair closer than r_c still lands in adjacent bins after that move
    const double tol = P.ortho ? 0.0 : kFracTol;
    for (int a = 0; a < 3; ++a) {
      double w = P.w[a] / (rc * (1.0 + 1e-5) + 2.0 * tol * P.w[a]);
      int nb = w >= 1024.0 ? 1024 : int(w);
      P.nb[a] = nb >= 3 ? nb : 1;
    }
    // never more bins than atoms: bins only get wider, still >= r_c
    while (int64_t(P.nb[0]) * P.nb[1] * P.nb[2] > cap) {
      int a = 0;
      if (P.nb[1] > P.nb[a]) a = 1;
      if (P.nb[2] > P.nb[a]) a = 2;
      P.nb[a] -= 1;
      if (P.nb[a] < 3) P.nb[a] = 1;
    }
    for (int a = 0; a < 3; ++a) {
      P.nimg[a] = 0;
      if (P.nb[a] == 1) {
        // |S_a| < r_c / w_a + 1 (+ 2 kFracTol for a general cell)
        double n = ceil(rc / P.w[a]) + (P.ortho ? 0.0 : 1.0);
        if (n > kMaxImages) {
          f |= GF_TOO_MANY_IMAGES;
          n = kMaxImages;
        }
        P.nimg[a] = int(n);
      }
    }
  } else {
    for (int a = 0; a < 3; ++a) {
      P.nb[a] = 1;
      P.nimg[a] = 0;
      P.w[a] = 1.0;
    }
  }
  P.valid = f == 0;
  prm[b] = P;
  if (f) atomicOr(flags, f);
}

__device__ inline int cdiv_dev(int a, int b) { return (a + b - 1) / b; }

__device__ inline int find_struct(const int32_t *__restrict__ struct_ptr, int n_structs, int i) {
  int lo = 0, hi = n_structs;  // last b with struct_ptr[b] <= i
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (struct_ptr[mid] <= i) lo = mid;
    else hi = mid;
  }
  return lo;
}

__device__ inline int bin_coord(double x, double L, int nb) {
  int c = int(x * double(nb) / L);
  c = c < 0 ? 0 : c;
  return c >= nb ? nb - 1 : c;
}

// fractional coordinate a of the Cartesian point x (f = x C^-1)
__device__ inline double frac(const StructParams &P, const double *x, int a) {
  return x[0] * P.Ci[0 * 3 + a] + x[1] * P.Ci[1 * 3 + a] + x[2] * P.Ci[2 * 3 + a];
}

__global__ void graph_bin(const float *__restrict__ pos, const int32_t *__restrict__ struct_ptr,
                          int n_structs, int n_atoms, const StructParams *__restrict__ prm,
                          int32_t *__restrict__ atom_struct, int32_t *__restrict__ atom_bin,
                          int32_t *__restrict__ bin_count, int32_t *__restrict__ flags) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_atoms || structs_rejected(flags)) return;
  int b = find_struct(struct_ptr, n_structs, i);
  const StructParams &P = prm[b];
  int c[3];
  bool outside = false;
  const double x[3] = {double(pos[i * 3 + 0]), double(pos[i * 3 + 1]), double(pos[i * 3 + 2])};
  for (int a = 0; a < 3; ++a) {
    if (P.ortho) {
      // orthorhombic: 0 <= x_a < L_a exactly
      if (!(x[a] >= 0.0) || !(x[a] < P.w[a])) outside = true;
      c[a] = bin_coord(x[a], P.w[a], P.nb[a]);
    } else {
      // general cell: fractional coordinates in [0, 1) up to the rounding of
      // float32 positions (the bins' extra 2 kFracTol w_a covers the clamp)
      const double fa = frac(P, x, a);
      if (!(fa >= -kFracTol) || !(fa < 1.0 + kFracTol)) outside = true;
      c[a] = bin_coord(fa, 1.0, P.nb[a]);
    }
  }
  if (outside) atomicOr(flags, GF_POS_OUTSIDE);
  int gb = P.bin_base + (c[2] * P.nb[1] + c[1]) * P.nb[0] + c[0];
  atom_struct[i] = b;
  atom_bin[i] = gb;
  atomicAdd(&bin_count[gb], 1);
}

__global__ void graph_scatter(const float *__restrict__ pos, int n_atoms,
                              const int32_t *__restrict__ atom_bin,
                              const int32_t *__restrict__ bin_start, int32_t *__restrict__ bin_fill,
                              float4 *__restrict__ binned, const int32_t *__restrict__ flags) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_atoms || structs_rejected(flags)) return;
  int gb = atom_bin[i];
  int p = atomicAdd(&bin_fill[gb], 1);
  binned[bin_start[gb] + p] =
      make_float4(pos[i * 3 + 0], pos[i * 3 + 1], pos[i * 3 + 2], __int_as_float(i));
}

// Candidate enumeration shared by the count and fill passes.  The visitor is
// called once per candidate slot with (accept, j, S, d, d2); all lanes of the
// wave call it the same number of times (inactive lanes with accept=false).
//
// Along a binned axis the shift is fixed by the neighbouring bin.  Along an
// image-mode axis only shifts with |x_j - x_i + S L| < r_c can give an edge
// (|d_a| >= r_c implies d2 >= r_c^2 under round-to-nearest), so each
// candidate atom carries the range of such S per axis, widened by 1e-9 of a
// cell length; the (atom, shift) pairs of 64 atoms are then flattened over
// the lanes with a prefix sum, and the exact float64 predicate decides.
__device__ inline int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(v, d, 64);
    if (lane >= d) v += y;
  }
  return v;
}

template <typename Visit>
__device__ inline void visit_candidates(int i, const float *__restrict__ pos,
                                        const StructParams &P, int gbin_i,
                                        const int32_t *__restrict__ bin_start,
                                        const float4 *__restrict__ binned, double rc2,
                                        double rc, Visit &&visit) {
  const int lane = threadIdx.x & 63;
  const double xi[3] = {double(pos[i * 3 + 0]), double(pos[i * 3 + 1]), double(pos[i * 3 + 2])};
  int local = gbin_i - P.bin_base;
  int bc[3];
  bc[0] = local % P.nb[0];
  bc[1] = (local / P.nb[0]) % P.nb[1];
  bc[2] = local / (P.nb[0] * P.nb[1]);
  int cnt[3];
  for (int a = 0; a < 3; ++a) cnt[a] = P.nb[a] == 1 ? 1 : 3;
  for (int e2 = 0; e2 < cnt[2]; ++e2)
    for (int e1 = 0; e1 < cnt[1]; ++e1)
      for (int e0 = 0; e0 < cnt[0]; ++e0) {
        const int ee[3] = {e0, e1, e2};
        int Sb[3], bb[3];
        for (int a = 0; a < 3; ++a) {
          if (P.nb[a] == 1) {
            Sb[a] = 0;
            bb[a] = 0;
          } else {
            const int v = bc[a] + ee[a] - 1;
            Sb[a] = v < 0 ? -1 : (v >= P.nb[a] ? 1 : 0);
            bb[a] = v - Sb[a] * P.nb[a];
          }
        }
        const int gb = P.bin_base + (bb[2] * P.nb[1] + bb[1]) * P.nb[0] + bb[0];
        const int k0 = bin_start[gb], k1 = bin_start[gb + 1];
        for (int kb = k0; kb < k1; kb += 64) {
          // this lane's candidate atom and its shift ranges
          const int kk = kb + lane;
          float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
          int lo[3] = {0, 0, 0}, span[3] = {1, 1, 1};
          int count = 0;
          if (kk < k1) {
            q = binned[kk];
            count = 1;
            const float qc[3] = {q.x, q.y, q.z};
            const double dxyz[3] = {double(qc[0]) - xi[0], double(qc[1]) - xi[1], double(qc[2]) - xi[2]};
            for (int a = 0; a < 3; ++a) {
              if (P.nb[a] != 1) {
                lo[a] = Sb[a];
                continue;
              }
              // (f_j - f_i)_a; the exact predicate below decides, so this
              // range only has to contain every shift that can give an edge
              const double df = frac(P, dxyz, a);
              const double slack = 1e-9;
              int l = int(ceil(-rc / P.w[a] - df - slack));
              int h = int(floor(rc / P.w[a] - df + slack));
              l = l < -P.nimg[a] ? -P.nimg[a] : l;
              h = h > P.nimg[a] ? P.nimg[a] : h;
              lo[a] = l;
              span[a] = h >= l ? h - l + 1 : 0;
              count *= span[a];
            }
          }
          const int incl = wave_incl_scan(count);
          const int total = __shfl(incl, 63, 64);
          for (int f0 = 0; f0 < total; f0 += 64) {
            const int f = f0 + lane;
            // owner lane: number of lanes whose inclusive prefix is <= f
            int o = 0;
#pragma unroll
            for (int step = 32; step >= 1; step >>= 1) {
              const int v = __shfl(incl, o + step - 1, 64);
              if (v <= f) o += step;
            }
            o = o > 63 ? 63 : o;
            // every lane takes part in every shuffle (a lane outside a branch
            // would not supply its value)
            const int prev_in = __shfl(incl, o > 0 ? o - 1 : 0, 64);
            const int prev = o > 0 ? prev_in : 0;
            int r = f - prev;
            const float ox = __shfl(q.x, o, 64), oy = __shfl(q.y, o, 64), oz = __shfl(q.z, o, 64);
            const int j = __float_as_int(__shfl(q.w, o, 64));
            int S[3];
            const int olo0 = __shfl(lo[0], o, 64), olo1 = __shfl(lo[1], o, 64), olo2 = __shfl(lo[2], o, 64);
            // spans are >= 1 for every owner of a real slot; the max() only
            // keeps the decode of padding slots (f >= total) well defined
            const int osp0 = max(1, __shfl(span[0], o, 64)), osp1 = max(1, __shfl(span[1], o, 64));
            S[0] = olo0 + r % osp0;
            r /= osp0;
            S[1] = olo1 + r % osp1;
            r /= osp1;
            S[2] = olo2 + r;
            bool ok = false;
            double d0 = 0, d1 = 0, d2v = 0, dd = 0;
            if (f < total) {
              const double s0 = double(S[0]), s1 = double(S[1]), s2 = double(S[2]);
              double t[3];
              for (int c = 0; c < 3; ++c)
                t[c] = __dadd_rn(__dadd_rn(__dmul_rn(s0, P.C[0 * 3 + c]), __dmul_rn(s1, P.C[1 * 3 + c])),
                                 __dmul_rn(s2, P.C[2 * 3 + c]));
              d0 = __dadd_rn(__dsub_rn(double(ox), xi[0]), t[0]);
              d1 = __dadd_rn(__dsub_rn(double(oy), xi[1]), t[1]);
              d2v = __dadd_rn(__dsub_rn(double(oz), xi[2]), t[2]);
              dd = __dadd_rn(__dadd_rn(__dmul_rn(d0, d0), __dmul_rn(d1, d1)), __dmul_rn(d2v, d2v));
              const bool zero_shift = S[0] == 0 && S[1] == 0 && S[2] == 0;
              ok = dd < rc2 && !(zero_shift && j == i);
            }
            visit(ok, j, S, d0, d1, d2v, dd);
          }
        }
      }
}

// One wave (one workgroup) per receiver: number of neighbours.
__global__ void __launch_bounds__(64) graph_count(const float *__restrict__ pos, int n_atoms,
                                                  const StructParams *__restrict__ prm,
                                                  const int32_t *__restrict__ atom_struct,
                                                  const int32_t *__restrict__ atom_bin,
                                                  const int32_t *__restrict__ bin_start,
                                                  const float4 *__restrict__ binned, double rc2,
                                                  double rc, int32_t *__restrict__ deg,
                                                  int32_t *__restrict__ maxdeg,
                                                  const int32_t *__restrict__ flags) {
  const int64_t blk = xcd_block(n_atoms);
  if (blk < 0) return;
  const int i = int(blk);
  if (structs_rejected(flags)) {
    // no atom has a structure: every row is empty
    if (threadIdx.x == 0) deg[i] = 0;
    return;
  }
  const StructParams &P = prm[atom_struct[i]];
  int count = 0;
  if (P.valid) {
    visit_candidates(i, pos, P, atom_bin[i], bin_start, binned, rc2, rc,
                     [&](bool ok, int, const int *, double, double, double, double) {
                       count += __popcll(__ballot(ok));
                     });
  }
  if (threadIdx.x == 0) {
    deg[i] = count;
    // most rows are not the longest: a plain read skips their atomics
    if (count > __atomic_load_n(maxdeg, __ATOMIC_RELAXED)) atomicMax(maxdeg, count);
  }
}

__global__ void graph_summary(const int32_t *__restrict__ row_ptr, int n_atoms,
                              const int32_t *__restrict__ flags, const int32_t *__restrict__ maxdeg,
                              int32_t *__restrict__ out) {
  out[0] = row_ptr[n_atoms];
  out[1] = *flags;
  out[2] = *maxdeg;
}

// The fill and reverse passes run before the single host read of the
// build: they proceed only when all E edges fit the caller's capacity, no row
// exceeds the LDS row buffer and the structure table was accepted, so that
// every edge slot [0, E) is written with an index in [0, n_atoms).
__device__ inline bool fill_allowed(const int32_t *row_ptr, int n_atoms, int64_t capacity,
                                    const int32_t *maxdeg, const int32_t *flags) {
  return int64_t(row_ptr[n_atoms]) <= capacity && *maxdeg <= kMaxDeg &&
         (__atomic_load_n(flags, __ATOMIC_RELAXED) & GF_BAD_STRUCTS) == 0;
}

__device__ inline uint64_t edge_key(int j, int s0, int s1, int s2) {
  return (uint64_t(uint32_t(j)) << 24) | (uint64_t(s0 + 128) << 16) | (uint64_t(s1 + 128) << 8) |
         uint64_t(s2 + 128);
}

// One wave (one workgroup) per receiver: collect the row in LDS, order it by
// (sender, shift) with a rank count, write it out.
__global__ void __launch_bounds__(64) graph_fill(const float *__restrict__ pos, int n_atoms,
                                                 const StructParams *__restrict__ prm,
                                                 const int32_t *__restrict__ atom_struct,
                                                 const int32_t *__restrict__ atom_bin,
                                                 const int32_t *__restrict__ bin_start,
                                                 const float4 *__restrict__ binned, double rc2,
                                                 double rc, const int32_t *__restrict__ row_ptr,
                                                 int64_t capacity, const int32_t *__restrict__ maxdeg,
                                                 const int32_t *__restrict__ flags,
                                                 int32_t *__restrict__ src, char4 *__restrict__ shift,
                                                 float4 *__restrict__ geom) {
  __shared__ uint64_t keys[kMaxDeg];
  __shared__ float4 gm[kMaxDeg];
  const int64_t blk = xcd_block(n_atoms);
  if (blk < 0) return;
  int i = int(blk);
  // runs before the host has seen the edge count: writes nothing unless all
  // E edges fit the caller's buffers and every row fits the LDS row buffer
  if (!fill_allowed(row_ptr, n_atoms, capacity, maxdeg, flags)) return;
  const int lane = threadIdx.x;
  const StructParams &P = prm[atom_struct[i]];
  if (!P.valid) return;
  int n = 0;
  visit_candidates(i, pos, P, atom_bin[i], bin_start, binned, rc2, rc,
                   [&](bool ok, int j, const int *S, double d0, double d1, double d2v, double dd) {
                     uint64_t m = __ballot(ok);
                     if (ok) {
                       int p = n + __popcll(m & ((uint64_t(1) << lane) - 1));
                       if (p < kMaxDeg) {
                         keys[p] = edge_key(j, S[0], S[1], S[2]);
                         gm[p] = make_float4(__double2float_rn(d0), __double2float_rn(d1),
                                             __double2float_rn(d2v),
                                             __double2float_rn(__dsqrt_rn(dd)));
                       }
                     }
                     n += __popcll(m);
                   });
  __syncthreads();
  const int r0 = row_ptr[i];
  const int deg = min(n, kMaxDeg);
  for (int a = lane; a < deg; a += 64) {
    uint64_t ka = keys[a];
    int rank = 0;
    for (int b = 0; b < deg; ++b) rank += keys[b] < ka;
    int o = r0 + rank;
    src[o] = int(ka >> 24);
    shift[o] = make_char4(char(int((ka >> 16) & 255) - 128), char(int((ka >> 8) & 255) - 128),
                          char(int(ka & 255) - 128), 0);
    geom[o] = gm[a];
  }
}

// One wave per receiver: reverse-edge index by binary search in the sender's
// row.  An edge whose reverse is absent (impossible for a graph of this
// library: the predicate is symmetric, d_rev = -d exactly) raises
// GF_REV_MISSING, which the calling entry point returns as an error; its
// rev entry is then the edge itself, so no later pass indexes out of range.
// In the build (gate >= 0) the pass runs only when fill_allowed; for a
// caller's own CSR (gate < 0, mlip_graph_reverse) every row range and
// sender index is checked against [0, n_edges] and [0, n_atoms) first.
__global__ void __launch_bounds__(256) graph_rev(int n_atoms, int64_t n_edges,
                                                 const int32_t *__restrict__ row_ptr,
                                                 const int32_t *__restrict__ src,
                                                 const char4 *__restrict__ shift,
                                                 int32_t *__restrict__ rev,
                                                 int32_t *__restrict__ flags, int64_t gate,
                                                 const int32_t *__restrict__ maxdeg) {
  int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= n_atoms) return;
  if (gate >= 0 && !fill_allowed(row_ptr, n_atoms, gate, maxdeg, flags)) return;
  const int lane = threadIdx.x & 63;
  const int r0 = row_ptr[i], r1 = row_ptr[i + 1];
  if (!(r0 >= 0 && r0 <= r1 && int64_t(r1) <= n_edges)) {
    if (lane == 0) atomicOr(flags, GF_BAD_SRC);
    return;
  }
  for (int e = r0 + lane; e < r1; e += 64) {
    const int j = src[e];
    bool found = false;
    int lo = 0;
    if (j < 0 || j >= n_atoms) {
      atomicOr(flags, GF_BAD_SRC);
    } else {
      const int j0 = row_ptr[j], j1 = row_ptr[j + 1];
      if (!(j0 >= 0 && j0 <= j1 && int64_t(j1) <= n_edges)) {
        atomicOr(flags, GF_BAD_SRC);
      } else {
        const char4 s = shift[e];
        const uint64_t want = edge_key(i, -int(s.x), -int(s.y), -int(s.z));
        lo = j0;
        int hi = j1;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          const char4 t = shift[mid];
          if (edge_key(src[mid], t.x, t.y, t.z) < want) lo = mid + 1;
          else hi = mid;
        }
        if (lo < j1) {
          const char4 t = shift[lo];
          found = edge_key(src[lo], t.x, t.y, t.z) == want;
        }
        if (!found) atomicOr(flags, GF_REV_MISSING);
      }
    }
    rev[e] = found ? lo : e;
  }
}

struct GraphWs {
  StructParams *prm;
  int32_t *flags, *maxdeg, *readback;
  int32_t *atom_struct, *atom_bin, *bin_count, *bin_start, *bin_fill, *scan_tmp;
  float4 *binned;
};

GraphWs carve_graph(void *base, int64_t N, int64_t B, size_t *bytes) {
  Carver c(base);
  GraphWs w;
  w.prm = c.take<StructParams>(size_t(B));
  w.flags = c.take<int32_t>(4);
  w.maxdeg = c.take<int32_t>(4);
  w.readback = c.take<int32_t>(4);
  int64_t nbins = N + B;
  w.atom_struct = c.take<int32_t>(size_t(N));
  w.atom_bin = c.take<int32_t>(size_t(N));
  w.bin_count = c.take<int32_t>(size_t(nbins));
  w.bin_start = c.take<int32_t>(size_t(nbins + 1));
  w.bin_fill = c.take<int32_t>(size_t(nbins));
  w.scan_tmp = c.take<int32_t>(scan_tmp_elems(std::max<int64_t>(nbins, N) + 1));
  w.binned = c.take<float4>(size_t(N));
  if (bytes) *bytes = c.bytes();
  return w;
}

inline unsigned nblk(int64_t n, int per) { return unsigned(cdiv(n < 1 ? 1 : n, per)); }

}  // namespace
}  // namespace mlip

using namespace mlip;

namespace mlip {
namespace {

// The one host read of a build (or of mlip_graph_reverse): waits for the
// stream, then copies the 4-word summary through a small pinned buffer kept
// per host thread for the life of the process (a pageable target takes the
// staged copy path).  The thread polls rather than sleeps, so the caller's
// next launches go out as soon as the stream drains.
int read_summary(const int32_t *dev, int32_t host[4], hipStream_t stream) {
  static thread_local int32_t *pinned = nullptr;
  if (!pinned)
    MLIP_HIP(hipHostMalloc(reinterpret_cast<void **>(&pinned), 4 * sizeof(int32_t), hipHostMallocPortable));
  MLIP_HIP(hipMemcpyAsync(pinned, dev, 4 * sizeof(int32_t), hipMemcpyDeviceToHost, stream));
  hipError_t q;
  while ((q = hipStreamQuery(stream)) == hipErrorNotReady) std::this_thread::yield();
  MLIP_HIP(q);
  for (int t = 0; t < 4; ++t) host[t] = pinned[t];
  return MLIP_OK;
}

// After the summary is written: when the fill pass did not run (the edges
// exceed the capacity, a row exceeds the LDS row buffer or the structure
// table was rejected), row_ptr becomes an empty graph, so that a caller who
// has not yet read the summary runs every later pass on no edges instead of
// on edge slots that were never written.
__global__ void graph_empty_on_error(int32_t *__restrict__ row_ptr, int n_atoms, int64_t capacity,
                                     const int32_t *__restrict__ summary) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i > n_atoms) return;
  const bool failed = int64_t(summary[0]) > capacity || summary[2] > kMaxDeg || (summary[1] & GF_BAD_STRUCTS);
  if (failed) row_ptr[i] = 0;
}

// Queues every pass of the build on the stream.  The summary (E, flags,
// largest degree, 0) goes to summary_out when given, else to the workspace's
// read-back slot; nothing waits for the device.
int enqueue_build(const float *pos, const float *cell, const int32_t *struct_ptr, int32_t n_atoms,
                  int32_t n_structs, float cutoff, int64_t edge_capacity, int32_t *row_ptr, int32_t *src,
                  int8_t *shift, int32_t *rev, float *geom, int32_t *summary_out, void *ws, size_t ws_bytes,
                  hipStream_t stream) {
  MLIP_CHECK_ARG(n_atoms >= 0 && n_structs >= 1, "n_atoms must be >= 0 and n_structs >= 1");
  MLIP_CHECK_ARG(cell && struct_ptr && row_ptr, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || pos, "pos is null");
  MLIP_CHECK_ARG(cutoff > 0.f && cutoff < 1e30f, "cutoff must be positive and finite");
  MLIP_CHECK_ARG(edge_capacity >= 0 && edge_capacity < (int64_t(1) << 31),
                 "edge_capacity must be in [0, 2^31)");
  MLIP_CHECK_ARG(edge_capacity == 0 || (src && shift && rev && geom), "edge buffers are null");
  size_t need = mlip_graph_workspace_size(n_atoms, n_structs);
  MLIP_CHECK_ARG(ws && ws_bytes >= need, "workspace too small: need %zu bytes, got %zu", need,
                 ws_bytes);
  MLIP_CHECK_ARG((reinterpret_cast<uintptr_t>(ws) & 255) == 0, "workspace must be 256-byte aligned");
  MLIP_CHECK_ARG((reinterpret_cast<uintptr_t>(geom) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(shift) & 3) == 0,
                 "geom must be 16-byte and shift 4-byte aligned");

  GraphWs w = carve_graph(ws, n_atoms, n_structs, nullptr);
  int32_t *summary = summary_out ? summary_out : w.readback;
  const int64_t N = n_atoms, B = n_structs, nbins = N + B;
  const double rc2 = double(cutoff) * double(cutoff);
  graph_zero<<<nblk(nbins, 256), 256, 0, stream>>>(w.flags, w.maxdeg, w.bin_count, w.bin_fill, nbins);
  MLIP_LAUNCHED();
  graph_setup<<<nblk(B, 64), 64, 0, stream>>>(cell, struct_ptr, n_structs, n_atoms, cutoff, w.prm,
                                               w.flags);
  MLIP_LAUNCHED();
  if (N > 0) {
    graph_bin<<<nblk(N, 256), 256, 0, stream>>>(pos, struct_ptr, n_structs, n_atoms, w.prm,
                                                 w.atom_struct, w.atom_bin, w.bin_count, w.flags);
    MLIP_LAUNCHED();
    int rc = exclusive_scan(w.bin_count, w.bin_start, nbins, true, w.scan_tmp, stream);
    if (rc) return rc;
    graph_scatter<<<nblk(N, 256), 256, 0, stream>>>(pos, n_atoms, w.atom_bin, w.bin_start, w.bin_fill,
                                                     w.binned, w.flags);
    MLIP_LAUNCHED();
    graph_count<<<unsigned(padded_grid(N)), 64, 0, stream>>>(pos, n_atoms, w.prm, w.atom_struct,
                                                             w.atom_bin, w.bin_start, w.binned, rc2,
                                                             double(cutoff), row_ptr, w.maxdeg, w.flags);
    MLIP_LAUNCHED();
  }
  int rc = exclusive_scan(row_ptr, row_ptr, N, true, w.scan_tmp, stream);
  if (rc) return rc;
  if (N > 0 && edge_capacity > 0) {
    graph_fill<<<unsigned(padded_grid(N)), 64, 0, stream>>>(
        pos, n_atoms, w.prm, w.atom_struct, w.atom_bin, w.bin_start, w.binned, rc2, double(cutoff),
        row_ptr, edge_capacity, w.maxdeg, w.flags, src, reinterpret_cast<char4 *>(shift),
        reinterpret_cast<float4 *>(geom));
    MLIP_LAUNCHED();
    graph_rev<<<nblk(N, 4), 256, 0, stream>>>(n_atoms, edge_capacity, row_ptr, src,
                                              reinterpret_cast<const char4 *>(shift), rev, w.flags,
                                              edge_capacity, w.maxdeg);
    MLIP_LAUNCHED();
  }
  graph_summary<<<1, 1, 0, stream>>>(row_ptr, n_atoms, w.flags, w.maxdeg, summary);
  MLIP_LAUNCHED();
  graph_empty_on_error<<<nblk(N + 1, 256), 256, 0, stream>>>(row_ptr, n_atoms, edge_capacity, summary);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

// The host's reading of a build summary (E, flags, largest degree).
int check_summary(const int32_t *host, int64_t edge_capacity, int64_t *n_edges) {
  const int64_t E = host[0];
  const int flags = host[1];
  *n_edges = E;
  if (flags & GF_BAD_STRUCTS) {
    *n_edges = 0;
    set_error("struct_ptr rejected: it must run 0 = p_0 <= p_1 <= ... <= p_B = n_atoms");
    return MLIP_ERR_INPUT;
  }
  if (flags & GF_BAD_CELL) {
    set_error("cell rejected: non-finite entries or zero volume (rows must be a lattice basis; "
              "a diagonal cell needs positive edges)");
    return MLIP_ERR_INPUT;
  }
  if (flags & GF_POS_OUTSIDE) {
    set_error("positions must be wrapped into their cell: fractional coordinates x C^-1 in [0, 1) "
              "(0 <= x < L along each axis of an orthorhombic cell)");
    return MLIP_ERR_INPUT;
  }
  if (flags & GF_TOO_MANY_IMAGES) {
    set_error("cutoff spans more than %d lattice-plane spacings of a cell", kMaxImages);
    return MLIP_ERR_UNSUPPORTED;
  }
  if (host[2] > kMaxDeg) {
    set_error("a receiver has %d neighbours; at most %d are supported", host[2], kMaxDeg);
    return MLIP_ERR_UNSUPPORTED;
  }
  if (E > edge_capacity) {
    set_error("edge_capacity %lld < required %lld", (long long)edge_capacity, (long long)E);
    return MLIP_ERR_CAPACITY;
  }
  if (flags & (GF_REV_MISSING | GF_BAD_SRC)) {
    set_error("internal error: an edge of the built graph has no reverse edge");
    return MLIP_ERR_INPUT;
  }
  return MLIP_OK;
}

__global__ void graph_flags_zero(int32_t *__restrict__ flags, int32_t *__restrict__ maxdeg) {
  if (threadIdx.x < 4) {
    flags[threadIdx.x] = 0;
    maxdeg[threadIdx.x] = 0;
  }
}

}  // namespace
}  // namespace mlip

extern "C" {

size_t mlip_graph_workspace_size(int32_t n_atoms, int32_t n_structs) {
  size_t bytes = 0;
  carve_graph(nullptr, n_atoms < 0 ? 0 : n_atoms, n_structs < 1 ? 1 : n_structs, &bytes);
  return bytes;
}

int mlip_build_graph(const float *pos, const float *cell, const int32_t *struct_ptr,
                     int32_t n_atoms, int32_t n_structs, float cutoff, int64_t edge_capacity,
                     int32_t *row_ptr, int32_t *src, int8_t *shift, int32_t *rev, float *geom,
                     int64_t *n_edges, void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_edges, "n_edges is null");
  int32_t host[4] = {0, 0, 0, 0};
  {
    ProfScope ps(K_GRAPH, stream);
    if (int rc = enqueue_build(pos, cell, struct_ptr, n_atoms, n_structs, cutoff, edge_capacity, row_ptr,
                               src, shift, rev, geom, nullptr, ws, ws_bytes, stream))
      return rc;
    // the one host read of the build: E, the error flags and the largest degree
    GraphWs w = carve_graph(ws, n_atoms, n_structs, nullptr);
    if (int rc = read_summary(w.readback, host, stream)) return rc;
  }
  return check_summary(host, edge_capacity, n_edges);
}

int mlip_build_graph_async(const float *pos, const float *cell, const int32_t *struct_ptr,
                           int32_t n_atoms, int32_t n_structs, float cutoff, int64_t edge_capacity,
                           int32_t *row_ptr, int32_t *src, int8_t *shift, int32_t *rev, float *geom,
                           int32_t *summary, void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(summary, "summary is null");
  MLIP_CHECK_ARG((reinterpret_cast<uintptr_t>(summary) & 15) == 0, "summary must be 16-byte aligned");
  ProfScope ps(K_GRAPH, stream);
  return enqueue_build(pos, cell, struct_ptr, n_atoms, n_structs, cutoff, edge_capacity, row_ptr, src,
                       shift, rev, geom, summary, ws, ws_bytes, stream);
}

int mlip_graph_check(const int32_t *summary_host, int64_t edge_capacity, int64_t *n_edges) {
  MLIP_CHECK_ARG(summary_host && n_edges, "null pointer argument");
  return check_summary(summary_host, edge_capacity, n_edges);
}

int mlip_graph_reverse(const int32_t *row_ptr, const int32_t *src, const int8_t *shift,
                       int32_t n_atoms, int64_t n_edges, int32_t *rev, void *ws, size_t ws_bytes,
                       void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0 && n_edges >= 0 && n_edges < (int64_t(1) << 31),
                 "n_atoms/n_edges out of range");
  MLIP_CHECK_ARG(row_ptr, "row_ptr is null");
  MLIP_CHECK_ARG(n_edges == 0 || (src && shift && rev), "edge arrays are null");
  size_t need = mlip_graph_workspace_size(0, 1);
  MLIP_CHECK_ARG(ws && ws_bytes >= need, "workspace too small: need %zu bytes, got %zu", need,
                 ws_bytes);
  MLIP_CHECK_ARG((reinterpret_cast<uintptr_t>(ws) & 255) == 0, "workspace must be 256-byte aligned");
  MLIP_CHECK_ARG((reinterpret_cast<uintptr_t>(shift) & 3) == 0, "shift must be 4-byte aligned");
  GraphWs w = carve_graph(ws, 0, 1, nullptr);
  int32_t host[4] = {0, 0, 0, 0};
  {
    ProfScope ps(K_GRAPH, stream);
    graph_flags_zero<<<1, 64, 0, stream>>>(w.flags, w.maxdeg);
    MLIP_LAUNCHED();
    if (n_atoms > 0 && n_edges > 0) {
      graph_rev<<<nblk(n_atoms, 4), 256, 0, stream>>>(n_atoms, n_edges, row_ptr, src,
                                                      reinterpret_cast<const char4 *>(shift), rev,
                                                      w.flags, -1, w.maxdeg);
      MLIP_LAUNCHED();
    }
    graph_summary<<<1, 1, 0, stream>>>(row_ptr, n_atoms, w.flags, w.maxdeg, w.readback);
    MLIP_LAUNCHED();
    if (int rc = read_summary(w.readback, host, stream)) return rc;
  }
  if (host[1] & GF_BAD_SRC) {
    set_error("row_ptr or src out of range: rows must satisfy 0 <= row_ptr[i] <= row_ptr[i+1] <= "
              "n_edges and senders lie in [0, n_atoms)");
    return MLIP_ERR_INPUT;
  }
  if (host[1] & GF_REV_MISSING) {
    set_error("the graph is not symmetric: some edge (i <- j, S) has no edge (j <- i, -S)");
    return MLIP_ERR_INPUT;
  }
  return MLIP_OK;
}

}  // extern "C"
