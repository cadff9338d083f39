// C ABI entry points of the interaction block (aggregation, mixture of
// experts, readout, input gradient).  The radius graph lives in graph.hip.
// Each entry point validates its arguments on the host, carves its scratch
// buffers out of the caller's workspace and enqueues its kernels on the
// caller's stream.
#include <algorithm>
#include <mutex>

#include "common.h"

namespace mlip {

int launch_embed_aggregate(const int32_t *row_ptr, const int32_t *src, const float *geom,
                           int n_atoms, const float *W_e, const float *s, int De, float rc,
                           float *e, float *a, hipStream_t stream);
int launch_edge_vjp(const int32_t *row_ptr, const int32_t *src, const float *geom, int n_atoms,
                    const float *W_e, const float *e, const float *s, const float *abar, int De,
                    float rc, float *sbar, float *grad_pos, float *atom_virial, hipStream_t stream);
int launch_strain_sum(const float *atom_virial, const int32_t *struct_ptr, int n_structs, int n_atoms,
                      double *grad_strain, hipStream_t stream);
int moe_route_dispatch(const int32_t *z, const float *logits, int N, int T, int X, int k,
                       int32_t *topk, float *gate, int32_t *exp_off, int32_t *tok_atom,
                       int32_t *slot, int32_t *local_rank, int32_t *blk_count, int32_t *n_type,
                       int32_t *pre, int32_t *exp_count, int32_t *flags, hipStream_t stream);
int moe_combine(const float *base, const float *rows, const int32_t *z, const float *gate,
                const int32_t *slot, int N, int T, int k, int D, float *out, hipStream_t stream);
int readout(const float *h, const float *w_r, const int32_t *struct_ptr, int N, int B, int D,
            float *eps, double *energy, hipStream_t stream);
int embed_atoms(const int32_t *z, const float *table, int N, int T, int D, float *h,
                hipStream_t stream);
int embed_grad(const int32_t *z, const float *grad_h, int N, int T, int D, float *d_table,
               hipStream_t stream);
int launch_readout_seed(const float *w_r, const double *Ebar, const int32_t *struct_ptr, int N, int B,
                        int D, float *g, hipStream_t stream);

namespace {

constexpr int kMaxTypes = 4096;
constexpr int kMaxExperts = 1023;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_ws(void *ws, size_t ws_bytes, size_t need) {
  if (need == 0) return MLIP_OK;
  MLIP_CHECK_ARG(ws != nullptr && ws_bytes >= need, "workspace too small: need %zu bytes, got %zu",
                 need, ws_bytes);
  MLIP_CHECK_ARG(aligned(ws, 256), "workspace must be 256-byte aligned");
  return MLIP_OK;
}

int check_width(int32_t d, const char *name) {
  MLIP_CHECK_ARG(d > 0 && d % 4 == 0 && d <= (1 << 20), "%s = %d must be a positive multiple of 4",
                 name, d);
  return MLIP_OK;
}

// ------------------------------------------------------------- workspaces --
struct AggWs {
  float *a, *split;
};
AggWs carve_agg(void *base, int64_t N, int64_t De, int64_t Dn, size_t *bytes) {
  Carver c(base);
  AggWs w;
  w.a = c.take<float>(size_t(N * De));
  w.split = c.take<float>(size_t(dense_split_floats(N, De, Dn)));   // s = h W_d split over K
  if (bytes) *bytes = c.bytes();
  return w;
}

struct MoeWs {
  int32_t *flags, *local_rank, *blk_count, *n_type, *pre, *exp_count;
  float *act, *Y;
};
MoeWs carve_moe(void *base, int64_t N, int64_t T, int64_t X, int64_t k, int64_t Dn, int64_t H,
                size_t *bytes) {
  Carver c(base);
  MoeWs w;
  w.flags = c.take<int32_t>(4);
  w.local_rank = c.take<int32_t>(size_t(std::max<int64_t>(N, 1)));
  w.blk_count = c.take<int32_t>(size_t(cdiv(std::max<int64_t>(N, 1), 256) * T));
  w.n_type = c.take<int32_t>(size_t(T));
  w.pre = c.take<int32_t>(size_t(X * T));
  w.exp_count = c.take<int32_t>(size_t(X));
  w.act = c.take<float>(size_t(N * k * H));
  w.Y = c.take<float>(size_t(N * k * Dn));
  if (bytes) *bytes = c.bytes();
  return w;
}

struct VjpWs {
  float *Q, *Utok, *ubar, *abar, *sbar, *virial, *split;
};
VjpWs carve_vjp(void *base, int64_t N, int64_t k, int64_t De, int64_t Dn, int64_t H, size_t *bytes) {
  Carver c(base);
  VjpWs w;
  w.split = c.take<float>(size_t(dense_split_floats(N, De, Dn)));   // abar = ubar W_u^T split over K
  w.virial = c.take<float>(size_t(N * 6));
  w.Q = c.take<float>(size_t(N * k * H));
  w.Utok = c.take<float>(size_t(N * k * Dn));
  w.ubar = c.take<float>(size_t(N * Dn));
  w.abar = c.take<float>(size_t(N * De));
  w.sbar = c.take<float>(size_t(N * De));
  if (bytes) *bytes = c.bytes();
  return w;
}
struct AggVjpWs {
  float *split, *virial, *abar, *sbar;
};
AggVjpWs carve_agg_vjp(void *base, int64_t N, int64_t De, int64_t Dn, size_t *bytes) {
  Carver c(base);
  AggVjpWs w;
  w.split = c.take<float>(size_t(dense_split_floats(N, De, Dn)));   // abar = ubar W_u^T split over K
  w.virial = c.take<float>(size_t(N * 6));
  w.abar = c.take<float>(size_t(N * De));
  w.sbar = c.take<float>(size_t(N * De));
  if (bytes) *bytes = c.bytes();
  return w;
}

// mlip_moe_forward_vjp: the forward's buffers, then Q [N k, H] (Utok reuses Y)
struct MoeFwdVjpWs {
  MoeWs f;
  float *Q;
};
MoeFwdVjpWs carve_moe_fwd_vjp(void *base, int64_t N, int64_t T, int64_t X, int64_t k, int64_t Dn,
                              int64_t H, size_t *bytes) {
  size_t fb = 0;
  MoeFwdVjpWs w;
  w.f = carve_moe(base, N, T, X, k, Dn, H, &fb);
  Carver c(base ? static_cast<char *>(base) + fb : nullptr);
  w.Q = c.take<float>(size_t(N * k * H));
  if (bytes) *bytes = fb + c.bytes();
  return w;
}


struct MoeVjpWs {
  float *Q, *Utok;
};
MoeVjpWs carve_moe_vjp(void *base, int64_t N, int64_t k, int64_t Dn, int64_t H, size_t *bytes) {
  Carver c(base);
  MoeVjpWs w;
  w.Q = c.take<float>(size_t(N * k * H));
  w.Utok = c.take<float>(size_t(N * k * Dn));
  if (bytes) *bytes = c.bytes();
  return w;
}

struct AttnVjpWs {
  float *obar, *qkv_bar, *edge_g, *edge_a, *edge_c, *virial, *split;
};
AttnVjpWs carve_attn_vjp(void *base, int64_t N, int64_t E, int64_t Da, int64_t nh, size_t *bytes) {
  Carver c(base);
  AttnVjpWs w;
  w.split = c.take<float>(size_t(dense_split_floats_max(N, Da)));   // obar = ubar W_o^T split over K
  w.obar = c.take<float>(size_t(N * Da));
  w.qkv_bar = c.take<float>(size_t(N * 3 * Da));
  w.edge_g = c.take<float>(size_t(E * nh));
  w.edge_a = c.take<float>(size_t(E * nh));
  w.edge_c = c.take<float>(size_t(E));
  w.virial = c.take<float>(size_t(N * 6));
  if (bytes) *bytes = c.bytes();
  return w;
}

struct TriVjpWs {
  float *taubar, *sigma, *gvec, *sbar, *virial, *split;
};
TriVjpWs carve_tri_vjp(void *base, int64_t N, int64_t E, int64_t Dt, size_t *bytes) {
  Carver c(base);
  TriVjpWs w;
  w.split = c.take<float>(size_t(dense_split_floats_max(N, Dt)));   // taubar = grad_hT W_T^T split over K
  w.taubar = c.take<float>(size_t(N * Dt));
  w.sigma = c.take<float>(size_t(E * Dt));
  w.gvec = c.take<float>(size_t(E * 4));
  w.sbar = c.take<float>(size_t(N * Dt));
  w.virial = c.take<float>(size_t(N * 6));
  if (bytes) *bytes = c.bytes();
  return w;
}

struct JvpWs {
  float *act_dot, *Y_dot;
};
JvpWs carve_jvp(void *base, int64_t N, int64_t k, int64_t Dn, int64_t H, size_t *bytes) {
  Carver c(base);
  JvpWs w;
  w.act_dot = c.take<float>(size_t(N * k * H));
  w.Y_dot = c.take<float>(size_t(N * k * Dn));
  if (bytes) *bytes = c.bytes();
  return w;
}

// dL/du = g + sum_r gate * ((g[tok] @ W2_x^T) * silu'(P)) @ W1_x^T, gathered back
// by slot in rank order (two grouped GEMMs and the combine).
// With q_save, the product g[tok] @ W2^T is also kept (before the silu' factor).
int moe_vjp_core(const float *grad_out, const int32_t *z, const float *gate,
                 const int32_t *exp_off, const int32_t *tok_atom, const int32_t *slot,
                 const float *P, const float *W1, const float *W2, int N, int T, int X, int k,
                 int Dn, int H, float *Q, float *Utok, float *grad_in, hipStream_t stream,
                 float *q_save = nullptr) {
  const int M = N * k;
  GemmArgs g1;  // Q = (g[tok] @ W2[x]^T) * silu'(P)
  g1.A = grad_out; g1.lda = Dn; g1.a_rows = tok_atom; g1.a_row_limit = N;
  g1.B = W2; g1.ldb = Dn; g1.b_group_stride = int64_t(H) * Dn;
  g1.C = Q; g1.C2 = q_save; g1.ldc = H; g1.R = P; g1.ldr = H;
  g1.group_off = exp_off; g1.n_groups = X;
  g1.M = M; g1.N = H; g1.K = Dn;
  if (int rc = launch_gemm(g1, true, q_save ? EPI_DSILU_Q : EPI_DSILU, K_GEMM_EXPERT_VJP_DOWN, stream))
    return rc;
  GemmArgs g2;  // U_tok = Q @ W1[x]^T
  g2.A = Q; g2.lda = H;
  g2.B = W1; g2.ldb = H; g2.b_group_stride = int64_t(Dn) * H;
  g2.C = Utok; g2.ldc = Dn;
  g2.group_off = exp_off; g2.n_groups = X;
  g2.M = M; g2.N = Dn; g2.K = H;
  if (int rc = launch_gemm(g2, true, EPI_STORE, K_GEMM_EXPERT_VJP_UP, stream)) return rc;
  return moe_combine(grad_out, Utok, z, gate, slot, N, T, k, Dn, grad_in, stream);
}

// Forward tangent of h' = u + MoE(u): P_dot = u_dot[tok] W1_x (and act_dot =
// silu'(P) P_dot), h_out_dot = u_dot + sum_r gate * act_dot W2_x (when asked).
int moe_jvp_core(const float *u_dot, const int32_t *z, const float *gate, const int32_t *exp_off,
                 const int32_t *tok_atom, const int32_t *slot, const float *P, const float *W1,
                 const float *W2, int N, int T, int X, int k, int Dn, int H, float *P_dot,
                 float *act_dot, float *Y_dot, float *h_out_dot, hipStream_t stream) {
  const int M = N * k;
  GemmArgs g3;  // P_dot = u_dot[tok] @ W1[x], act_dot = silu'(P) * P_dot
  g3.A = u_dot; g3.lda = Dn; g3.a_rows = tok_atom; g3.a_row_limit = N;
  g3.B = W1; g3.ldb = H; g3.b_group_stride = int64_t(Dn) * H;
  g3.C = P_dot; g3.C2 = act_dot; g3.ldc = H; g3.R = P; g3.ldr = H;
  g3.group_off = exp_off; g3.n_groups = X;
  g3.M = M; g3.N = H; g3.K = Dn;
  if (int rc = launch_gemm(g3, false, EPI_TAN, K_GEMM_EXPERT_TAN, stream)) return rc;
  if (!h_out_dot) return MLIP_OK;
  GemmArgs g4;  // Y_dot = act_dot @ W2[x]
  g4.A = act_dot; g4.lda = H;
  g4.B = W2; g4.ldb = Dn; g4.b_group_stride = int64_t(H) * Dn;
  g4.C = Y_dot; g4.ldc = Dn;
  g4.group_off = exp_off; g4.n_groups = X;
  g4.M = M; g4.N = Dn; g4.K = H;
  if (int rc = launch_gemm(g4, false, EPI_STORE, K_GEMM_EXPERT_TAN, stream)) return rc;
  return moe_combine(u_dot, Y_dot, z, gate, slot, N, T, k, Dn, h_out_dot, stream);
}

struct MoeTanWs {
  float *D_dot, *act, *act_dot, *D, *dg, *gt, *U_dot;
  double *G;
};
MoeTanWs carve_moe_tan(Carver &c, int64_t N, int64_t T, int64_t k, int64_t Dn, int64_t H) {
  MoeTanWs w;
  const int64_t M = N * k;
  w.D_dot = c.take<float>(size_t(M * H));
  w.act = c.take<float>(size_t(M * H));
  w.act_dot = c.take<float>(size_t(M * H));
  w.D = c.take<float>(size_t(M * H));
  w.dg = c.take<float>(size_t(std::max<int64_t>(M, 1)));
  w.gt = c.take<float>(size_t(std::max<int64_t>(M, 1)));
  w.U_dot = c.take<float>(size_t(M * Dn));
  w.G = c.take<double>(size_t(T * k));
  return w;
}

// Tangent of the MoE layer's gradient along (u_dot, grad_out_dot): grad_in_dot
// = g_dot + sum_r gate * D_dot W1_x^T and the weight, gate and logit gradients
// (D = silu'(P) Q, Q = g[tok] W2^T kept by the primal gradient).
int moe_tvjp_core(const int32_t *z, const int32_t *topk, const float *gate, const int32_t *exp_off,
                  const int32_t *tok_atom, const int32_t *slot, const float *P, const float *P_dot,
                  const float *W1, const float *W2, int N, int T, int X, int k, int Dn, int H,
                  const float *u, const float *u_dot, const float *grad_out, const float *Q,
                  const float *grad_out_dot, const MoeTanWs &w, float *grad_in_dot, float *d_W1,
                  float *d_W2, float *d_gate, float *d_logits, hipStream_t stream) {
  const int M = N * k;
  if (N > 0) {
    if (grad_out_dot) {
      GemmArgs g;  // Q_dot = g_dot[tok] @ W2^T (into D_dot, turned into D_dot in place below)
      g.A = grad_out_dot; g.lda = Dn; g.a_rows = tok_atom; g.a_row_limit = N;
      g.B = W2; g.ldb = Dn; g.b_group_stride = int64_t(H) * Dn;
      g.C = w.D_dot; g.ldc = H;
      g.group_off = exp_off; g.n_groups = X;
      g.M = M; g.N = H; g.K = Dn;
      if (int rc = launch_gemm(g, true, EPI_STORE, K_GEMM_EXPERT_TAN, stream)) return rc;
    }
    if (int rc = launch_moe_tan(P, P_dot, Q, grad_out_dot ? w.D_dot : nullptr, M, H, w.act, w.act_dot,
                                w.D, w.D_dot, w.dg, stream))
      return rc;
    if (grad_in_dot) {
      GemmArgs g2;  // U_dot = D_dot @ W1^T; grad_in_dot = g_dot + sum_r gate * U_dot[slot]
      g2.A = w.D_dot; g2.lda = H;
      g2.B = W1; g2.ldb = H; g2.b_group_stride = int64_t(Dn) * H;
      g2.C = w.U_dot; g2.ldc = Dn;
      g2.group_off = exp_off; g2.n_groups = X;
      g2.M = M; g2.N = Dn; g2.K = H;
      if (int rc = launch_gemm(g2, true, EPI_STORE, K_GEMM_EXPERT_TAN, stream)) return rc;
      if (int rc = moe_combine(grad_out_dot, w.U_dot, z, gate, slot, N, T, k, Dn, grad_in_dot, stream))
        return rc;
    }
  }
  if (int rc = launch_token_gate(z, gate, slot, N, T, k, w.gt, stream)) return rc;
  {
    WgradArgs q;  // d W1_x = sum_t gate_t (u_dot[i]^T D_t + u[i]^T D_dot_t)
    q.A0 = u_dot; q.B0 = w.D; q.A1 = u; q.B1 = w.D_dot; q.lda = Dn; q.ldb = H;
    q.a_rows = tok_atom; q.row_limit = N; q.scale = w.gt; q.group_off = exp_off; q.n_groups = X;
    q.P = M; q.Mo = Dn; q.No = H; q.C = d_W1;
    if (int rc = launch_wgrad(q, nullptr, stream)) return rc;
  }
  {
    WgradArgs q;  // d W2_x = sum_t gate_t (act_dot_t^T g[i] + act_t^T g_dot[i])
    q.A0 = w.act_dot; q.B0 = grad_out;
    if (grad_out_dot) { q.A1 = w.act; q.B1 = grad_out_dot; }
    q.lda = H; q.ldb = Dn; q.b_rows = tok_atom; q.row_limit = N; q.scale = w.gt; q.group_off = exp_off;
    q.n_groups = X; q.P = M; q.Mo = H; q.No = Dn; q.C = d_W2;
    if (int rc = launch_wgrad(q, nullptr, stream)) return rc;
  }
  return launch_gate_grad(w.dg, z, topk, gate, exp_off, tok_atom, T, X, k, w.G, d_gate, d_logits, stream);
}

struct TanVjpWs {
  float *ubar_dot, *abar, *abar_dot, *sbar, *sbar_dot, *dwe_part, *split;
};
TanVjpWs carve_tan_vjp(void *base, int64_t N, int64_t T, int64_t k, int64_t De, int64_t Dn,
                       int64_t H, size_t *bytes, MoeTanWs *moe) {
  Carver c(base);
  TanVjpWs w;
  MoeTanWs m = carve_moe_tan(c, N, T, k, Dn, H);
  if (moe) *moe = m;
  w.ubar_dot = c.take<float>(size_t(N * Dn));
  w.abar = c.take<float>(size_t(N * De));
  w.abar_dot = c.take<float>(size_t(N * De));
  w.sbar = c.take<float>(size_t(N * De));
  w.sbar_dot = c.take<float>(size_t(N * De));
  w.dwe_part = c.take<float>(size_t(edge_tan_part_floats(int(N), int(De))));
  // split-K scratch, shared in stream order by abar / abar_dot (first) and
  // the two dense weight gradients (last)
  WgradArgs u, d;
  u.P = d.P = int(N);
  u.Mo = int(De); u.No = int(Dn);
  d.Mo = int(Dn); d.No = int(De);
  w.split = c.take<float>(size_t(std::max({wgrad_split_floats(u), wgrad_split_floats(d),
                                           dense_split_floats_max(N, De)})));
  if (bytes) *bytes = c.bytes();
  return w;
}

struct AttnTanWs {
  float *obar, *obar_dot, *qkv_bar_dot, *eg, *egd, *ea, *ead, *ebar, *ebar_dot, *part, *split;
};
AttnTanWs carve_attn_tan(void *base, int64_t N, int64_t E, int64_t Dn, int64_t Da, int64_t nh,
                         size_t *bytes) {
  Carver c(base);
  AttnTanWs w;
  w.obar = c.take<float>(size_t(N * Da));
  w.obar_dot = c.take<float>(size_t(N * Da));
  w.qkv_bar_dot = c.take<float>(size_t(N * 3 * Da));
  w.eg = c.take<float>(size_t(E * nh));
  w.egd = c.take<float>(size_t(E * nh));
  w.ea = c.take<float>(size_t(E * nh));
  w.ead = c.take<float>(size_t(E * nh));
  w.ebar = c.take<float>(size_t(E * Da));
  w.ebar_dot = c.take<float>(size_t(E * Da));
  w.part = c.take<float>(size_t(edge_tan_part_floats(int(N), int(Da))));
  WgradArgs a, b;
  a.P = b.P = int(N);
  a.Mo = int(Dn); a.No = int(3 * Da);
  b.Mo = int(Da); b.No = int(Dn);
  // shared in stream order by the split-K parts of obar / obar_dot (first) and
  // of the dense weight gradients (last)
  w.split = c.take<float>(size_t(std::max({wgrad_split_floats(a), wgrad_split_floats(b),
                                           dense_split_floats_max(N, Da)})));
  if (bytes) *bytes = c.bytes();
  return w;
}

struct TriTanWs {
  float *taubar, *taubar_dot, *sigma_dot, *wang_part, *wang_part2, *sbar_dot, *split;
};
TriTanWs carve_tri_tan(void *base, int64_t N, int64_t E, int64_t Dn, int64_t Dt, size_t *bytes) {
  Carver c(base);
  TriTanWs w;
  w.taubar = c.take<float>(size_t(N * Dt));
  w.taubar_dot = c.take<float>(size_t(N * Dt));
  w.sigma_dot = c.take<float>(size_t(E * Dt));
  w.wang_part = c.take<float>(size_t(N * MLIP_N_ANG * Dt));
  w.wang_part2 = c.take<float>(size_t(std::max<int64_t>(cdiv(N, 32), 1) * MLIP_N_ANG * Dt));
  w.sbar_dot = c.take<float>(size_t(N * Dt));
  WgradArgs a, b;
  a.P = b.P = int(N);
  a.Mo = int(Dn); a.No = int(Dt);
  b.Mo = int(Dt); b.No = int(Dn);
  // shared in stream order by the split-K parts of taubar / taubar_dot (first)
  // and of the dense weight gradients (last)
  w.split = c.take<float>(size_t(std::max({wgrad_split_floats(a), wgrad_split_floats(b),
                                           dense_split_floats_max(N, Dt)})));
  if (bytes) *bytes = c.bytes();
  return w;
}

int check_aggregate_args(const int32_t *row_ptr, const int32_t *src, const float *geom,
                         int32_t n_atoms, int64_t n_edges, const float *h, const float *W_e,
                         const float *W_d, const float *W_u, int32_t n_rbf, int32_t d_edge,
                         int32_t d_node, float cutoff, const float *e, const float *s,
                         const float *u) {
  MLIP_CHECK_ARG(n_atoms >= 0 && n_edges >= 0 && n_edges < (int64_t(1) << 31),
                 "n_atoms/n_edges out of range");
  MLIP_CHECK_ARG(n_rbf == MLIP_N_RBF, "n_rbf must be %d", MLIP_N_RBF);
  if (int rc = check_width(d_edge, "d_edge")) return rc;
  if (int rc = check_width(d_node, "d_node")) return rc;
  MLIP_CHECK_ARG(cutoff > 0.f && cutoff < 1e30f, "cutoff must be positive and finite");
  MLIP_CHECK_ARG(row_ptr && W_e && W_d && W_u, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (h && s && u), "null pointer argument");
  MLIP_CHECK_ARG(n_edges == 0 || (src && geom), "null edge pointer");
  MLIP_CHECK_ARG(aligned(geom, 16) && aligned(h, 16) && aligned(W_e, 16) && aligned(W_d, 16) &&
                     aligned(W_u, 16) && aligned(e, 16) && aligned(s, 16) && aligned(u, 16),
                 "float arrays must be 16-byte aligned");
  return MLIP_OK;
}

// s = h W_d, the edge embedding + aggregation into w.a, u = h + a W_u.
int aggregate_core(const int32_t *row_ptr, const int32_t *src, const float *geom, int32_t n_atoms,
                   const float *h, const float *W_e, const float *W_d, const float *W_u,
                   int32_t d_edge, int32_t d_node, float cutoff, float *e, float *s, float *u,
                   const AggWs &w, hipStream_t stream) {
  GemmArgs g;  // s = h @ W_d
  g.A = h; g.lda = d_node; g.B = W_d; g.ldb = d_edge; g.C = s; g.ldc = d_edge;
  g.M = n_atoms; g.N = d_edge; g.K = d_node;
  g.k_split = dense_k_split(n_atoms, d_edge, d_node); g.split_ws = w.split;
  if (int rc = launch_gemm(g, false, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
  if (int rc = launch_embed_aggregate(row_ptr, src, geom, n_atoms, W_e, s, d_edge, cutoff, e, w.a,
                                      stream))
    return rc;
  GemmArgs g2;  // u = h + a @ W_u
  g2.A = w.a; g2.lda = d_edge; g2.B = W_u; g2.ldb = d_node; g2.C = u; g2.ldc = d_node;
  g2.R = h; g2.ldr = d_node; g2.M = n_atoms; g2.N = d_node; g2.K = d_edge;
  return launch_gemm(g2, false, EPI_RESID, K_GEMM_DENSE, stream);
}

// ------------------------------------------- library-owned scratch memory --
// Scratch of mlip_aggregate_static: a file-scope device array, one copy per
// GPU, held until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is only a stand-in for the symbol): the device
// address of each GPU's copy is looked up once, with that GPU current, and
// kept in g_scratch_addr.
constexpr size_t kAggScratchBytes = MLIP_AGGREGATE_STATIC_MAX_BYTES;
constexpr int kMaxScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kAggScratchBytes];
static std::mutex g_scratch_mu;
static void *g_scratch_addr[kMaxScratchDevices];

int scratch_address(void **out) {
  int dev = -1;
  MLIP_HIP(hipGetDevice(&dev));
  MLIP_CHECK_ARG(dev >= 0 && dev < kMaxScratchDevices, "device %d outside the %d supported", dev,
                 kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    MLIP_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) {
      set_error("hipGetSymbolAddress gave a null address for the scratch array");
      return MLIP_ERR_HIP;
    }
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return MLIP_OK;
}

}  // namespace
}  // namespace mlip

using namespace mlip;

extern "C" {

// ------------------------------------------------------------- aggregate ---
size_t mlip_aggregate_workspace_size(int32_t n_atoms, int32_t d_edge, int32_t d_node) {
  size_t b = 0;
  carve_agg(nullptr, std::max(n_atoms, 0), std::max(d_edge, 0), std::max(d_node, 0), &b);
  return b;
}

int mlip_aggregate(const int32_t *row_ptr, const int32_t *src, const float *geom, int32_t n_atoms,
                   int64_t n_edges, const float *h, const float *W_e, const float *W_d,
                   const float *W_u, int32_t n_rbf, int32_t d_edge, int32_t d_node, float cutoff,
                   float *e, float *s, float *u, void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (int rc = check_aggregate_args(row_ptr, src, geom, n_atoms, n_edges, h, W_e, W_d, W_u, n_rbf,
                                    d_edge, d_node, cutoff, e, s, u))
    return rc;
  if (int rc = check_ws(ws, ws_bytes, mlip_aggregate_workspace_size(n_atoms, d_edge, d_node)))
    return rc;
  if (n_atoms == 0) return MLIP_OK;
  AggWs w = carve_agg(ws, n_atoms, d_edge, d_node, nullptr);
  return aggregate_core(row_ptr, src, geom, n_atoms, h, W_e, W_d, W_u, d_edge, d_node, cutoff, e, s,
                        u, w, stream);
}

int mlip_aggregate_static(const int32_t *row_ptr, const int32_t *src, const float *geom,
                          int32_t n_atoms, int64_t n_edges, const float *h, const float *W_e,
                          const float *W_d, const float *W_u, int32_t n_rbf, int32_t d_edge,
                          int32_t d_node, float cutoff, float *e, float *s, float *u,
                          void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (int rc = check_aggregate_args(row_ptr, src, geom, n_atoms, n_edges, h, W_e, W_d, W_u, n_rbf,
                                    d_edge, d_node, cutoff, e, s, u))
    return rc;
  const size_t need = mlip_aggregate_workspace_size(n_atoms, d_edge, d_node);
  if (need > kAggScratchBytes) {
    set_error("mlip_aggregate_static needs %zu bytes of scratch for %d atoms x d_edge %d; the "
              "library's static scratch holds %zu (use mlip_aggregate with a workspace)",
              need, n_atoms, d_edge, kAggScratchBytes);
    return MLIP_ERR_UNSUPPORTED;
  }
  if (n_atoms == 0) return MLIP_OK;
  void *base = nullptr;
  if (int rc = scratch_address(&base)) return rc;
  AggWs w = carve_agg(base, n_atoms, d_edge, d_node, nullptr);
  return aggregate_core(row_ptr, src, geom, n_atoms, h, W_e, W_d, W_u, d_edge, d_node, cutoff, e, s,
                        u, w, stream);
}

// ------------------------------------------------------------------- MoE ---
size_t mlip_moe_workspace_size(int32_t n_atoms, int32_t n_types, int32_t n_experts, int32_t top_k,
                               int32_t d_node, int32_t d_hidden) {
  size_t b = 0;
  carve_moe(nullptr, std::max(n_atoms, 0), std::max(n_types, 1), std::max(n_experts, 1),
            std::max(top_k, 1), std::max(d_node, 0), std::max(d_hidden, 0), &b);
  return b;
}

int mlip_moe_forward(const float *u, const int32_t *z, const float *logits, const float *W1,
                     const float *W2, int32_t n_atoms, int32_t n_types, int32_t n_experts,
                     int32_t top_k, int32_t d_node, int32_t d_hidden, int32_t *topk, float *gate,
                     int32_t *exp_off, int32_t *tok_atom, int32_t *slot, float *P, float *h_out,
                     void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0, "n_atoms must be >= 0");
  MLIP_CHECK_ARG(n_types >= 1 && n_types <= kMaxTypes, "n_types must be in [1, %d]", kMaxTypes);
  MLIP_CHECK_ARG(n_experts >= 1 && top_k >= 1 && top_k <= n_experts,
                 "need 1 <= top_k <= n_experts");
  MLIP_CHECK_ARG(n_experts <= kMaxExperts, "n_experts must be <= %d", kMaxExperts);
  MLIP_CHECK_ARG(int64_t(n_atoms) * top_k < (int64_t(1) << 31), "n_atoms * top_k too large");
  if (int rc = check_width(d_node, "d_node")) return rc;
  if (int rc = check_width(d_hidden, "d_hidden")) return rc;
  MLIP_CHECK_ARG(logits && W1 && W2 && topk && gate && exp_off, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (u && z && tok_atom && slot && P && h_out), "null pointer argument");
  MLIP_CHECK_ARG(aligned(u, 16) && aligned(W1, 16) && aligned(W2, 16) && aligned(P, 16) &&
                     aligned(h_out, 16),
                 "float arrays must be 16-byte aligned");
  if (int rc = check_ws(ws, ws_bytes, mlip_moe_workspace_size(n_atoms, n_types, n_experts, top_k,
                                                              d_node, d_hidden)))
    return rc;
  MoeWs w = carve_moe(ws, n_atoms, n_types, n_experts, top_k, d_node, d_hidden, nullptr);
  const int M = n_atoms * top_k;
  if (int rc = moe_route_dispatch(z, logits, n_atoms, n_types, n_experts, top_k, topk, gate,
                                  exp_off, tok_atom, slot, w.local_rank, w.blk_count, w.n_type,
                                  w.pre, w.exp_count, w.flags, stream))
    return rc;
  if (n_atoms == 0) return MLIP_OK;
  GemmArgs g;  // P = u[tok] @ W1[x], act = silu(P)
  g.A = u; g.lda = d_node; g.a_rows = tok_atom; g.a_row_limit = n_atoms;
  g.B = W1; g.ldb = d_hidden; g.b_group_stride = int64_t(d_node) * d_hidden;
  g.C = P; g.C2 = w.act; g.ldc = d_hidden;
  g.group_off = exp_off; g.n_groups = n_experts;
  g.M = M; g.N = d_hidden; g.K = d_node;
  if (int rc = launch_gemm(g, false, EPI_SILU, K_GEMM_EXPERT_UP, stream)) return rc;
  GemmArgs g2;  // Y = act @ W2[x]
  g2.A = w.act; g2.lda = d_hidden;
  g2.B = W2; g2.ldb = d_node; g2.b_group_stride = int64_t(d_hidden) * d_node;
  g2.C = w.Y; g2.ldc = d_node;
  g2.group_off = exp_off; g2.n_groups = n_experts;
  g2.M = M; g2.N = d_node; g2.K = d_hidden;
  if (int rc = launch_gemm(g2, false, EPI_STORE, K_GEMM_EXPERT_DOWN, stream)) return rc;
  return moe_combine(u, w.Y, z, gate, slot, n_atoms, n_types, top_k, d_node, h_out, stream);
}

int mlip_moe_status(const void *ws, int32_t *bad_types, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(ws && bad_types, "null pointer argument");
  int32_t f = 0;
  MLIP_HIP(hipMemcpyAsync(&f, ws, sizeof(f), hipMemcpyDeviceToHost, stream));
  MLIP_HIP(hipStreamSynchronize(stream));
  *bad_types = (f & 1) ? 1 : 0;
  return MLIP_OK;
}

// --------------------------------------------------------------- readout ---
int mlip_readout(const float *h_out, const float *w_r, const int32_t *struct_ptr, int32_t n_atoms,
                 int32_t n_structs, int32_t d_node, float *eps, double *energy, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0 && n_structs >= 1, "n_atoms >= 0 and n_structs >= 1 required");
  if (int rc = check_width(d_node, "d_node")) return rc;
  MLIP_CHECK_ARG(w_r && struct_ptr && energy, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (h_out && eps), "null pointer argument");
  MLIP_CHECK_ARG(aligned(h_out, 16) && aligned(w_r, 16), "float arrays must be 16-byte aligned");
  return readout(h_out, w_r, struct_ptr, n_atoms, n_structs, d_node, eps, energy, stream);
}

// ------------------------------------------------------------------- VJP ---
size_t mlip_vjp_workspace_size(int32_t n_atoms, int32_t top_k, int32_t d_edge, int32_t d_node,
                               int32_t d_hidden) {
  size_t b = 0;
  carve_vjp(nullptr, std::max(n_atoms, 0), std::max(top_k, 1), std::max(d_edge, 0),
            std::max(d_node, 0), std::max(d_hidden, 0), &b);
  return b;
}

int mlip_block_vjp(const int32_t *row_ptr, const int32_t *src, const float *geom, int32_t n_atoms,
                   int64_t n_edges, const float *e, const float *s, const int32_t *z,
                   const float *gate, const int32_t *exp_off, const int32_t *tok_atom,
                   const int32_t *slot, const float *P, const float *W_e, const float *W_d,
                   const float *W_u, const float *W1, const float *W2, int32_t n_rbf,
                   int32_t d_edge, int32_t d_node, int32_t d_hidden, int32_t n_types,
                   int32_t n_experts, int32_t top_k, float cutoff, const float *grad_out,
                   float *grad_h, float *grad_pos, const int32_t *struct_ptr, int32_t n_structs,
                   float *atom_virial, double *grad_strain, float *ubar_out, float *q_out,
                   void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0 && n_edges >= 0 && n_edges < (int64_t(1) << 31),
                 "n_atoms/n_edges out of range");
  MLIP_CHECK_ARG(n_rbf == MLIP_N_RBF, "n_rbf must be %d", MLIP_N_RBF);
  MLIP_CHECK_ARG(n_types >= 1 && n_types <= kMaxTypes, "n_types must be in [1, %d]", kMaxTypes);
  MLIP_CHECK_ARG(n_experts >= 1 && top_k >= 1 && top_k <= n_experts,
                 "need 1 <= top_k <= n_experts");
  MLIP_CHECK_ARG(n_experts <= kMaxExperts, "n_experts must be <= %d", kMaxExperts);
  MLIP_CHECK_ARG(int64_t(n_atoms) * top_k < (int64_t(1) << 31), "n_atoms * top_k too large");
  if (int rc = check_width(d_edge, "d_edge")) return rc;
  if (int rc = check_width(d_node, "d_node")) return rc;
  if (int rc = check_width(d_hidden, "d_hidden")) return rc;
  MLIP_CHECK_ARG(cutoff > 0.f && cutoff < 1e30f, "cutoff must be positive and finite");
  MLIP_CHECK_ARG(row_ptr && W_e && W_d && W_u && W1 && W2 && gate && exp_off, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (s && z && tok_atom && slot && P && grad_out && grad_h && grad_pos),
                 "null pointer argument");
  MLIP_CHECK_ARG(n_edges == 0 || (src && geom), "null edge pointer");
  MLIP_CHECK_ARG(!grad_strain || (struct_ptr && n_structs >= 1),
                 "grad_strain needs struct_ptr and n_structs >= 1");
  MLIP_CHECK_ARG(aligned(e, 16) && aligned(s, 16) && aligned(P, 16) && aligned(grad_out, 16) &&
                     aligned(grad_h, 16) && aligned(geom, 16),
                 "float arrays must be 16-byte aligned");
  if (int rc = check_ws(ws, ws_bytes,
                        mlip_vjp_workspace_size(n_atoms, top_k, d_edge, d_node, d_hidden)))
    return rc;
  if (n_atoms == 0) {
    if (grad_strain) return launch_strain_sum(nullptr, struct_ptr, n_structs, 0, grad_strain, stream);
    return MLIP_OK;
  }
  MLIP_CHECK_ARG(aligned(ubar_out, 16) && aligned(q_out, 16), "float arrays must be 16-byte aligned");
  VjpWs w = carve_vjp(ws, n_atoms, top_k, d_edge, d_node, d_hidden, nullptr);
  float *vir = atom_virial ? atom_virial : w.virial;
  if (ubar_out) w.ubar = ubar_out;

  if (int rc = moe_vjp_core(grad_out, z, gate, exp_off, tok_atom, slot, P, W1, W2, n_atoms,
                            n_types, n_experts, top_k, d_node, d_hidden, w.Q, w.Utok, w.ubar,
                            stream, q_out))
    return rc;
  GemmArgs g3;  // abar = ubar @ W_u^T
  g3.A = w.ubar; g3.lda = d_node; g3.B = W_u; g3.ldb = d_node; g3.C = w.abar; g3.ldc = d_edge;
  g3.M = n_atoms; g3.N = d_edge; g3.K = d_node;
  g3.k_split = dense_k_split(n_atoms, d_edge, d_node); g3.split_ws = w.split;
  if (int rc = launch_gemm(g3, true, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
  if (int rc = launch_edge_vjp(row_ptr, src, geom, n_atoms, W_e, e, s, w.abar, d_edge, cutoff,
                               w.sbar, grad_pos, vir, stream))
    return rc;
  if (grad_strain) {
    if (int rc = launch_strain_sum(vir, struct_ptr, n_structs, n_atoms, grad_strain, stream)) return rc;
  }
  GemmArgs g4;  // grad_h = ubar + sbar @ W_d^T
  g4.A = w.sbar; g4.lda = d_edge; g4.B = W_d; g4.ldb = d_edge; g4.C = grad_h; g4.ldc = d_node;
  g4.R = w.ubar; g4.ldr = d_node; g4.M = n_atoms; g4.N = d_node; g4.K = d_edge;
  return launch_gemm(g4, true, EPI_RESID, K_GEMM_DENSE, stream);
}

// ------------------------------------------------------------ MoE VJP ----
size_t mlip_moe_vjp_workspace_size(int32_t n_atoms, int32_t top_k, int32_t d_node,
                                   int32_t d_hidden) {
  size_t b = 0;
  carve_moe_vjp(nullptr, std::max(n_atoms, 0), std::max(top_k, 1), std::max(d_node, 0),
                std::max(d_hidden, 0), &b);
  return b;
}

size_t mlip_moe_forward_vjp_workspace_size(int32_t n_atoms, int32_t n_types, int32_t n_experts,
                                           int32_t top_k, int32_t d_node, int32_t d_hidden) {
  size_t b = 0;
  carve_moe_fwd_vjp(nullptr, std::max(n_atoms, 0), std::max(n_types, 1), std::max(n_experts, 1),
                    std::max(top_k, 1), std::max(d_node, 0), std::max(d_hidden, 0), &b);
  return b;
}

size_t mlip_struct_size(int32_t which) {
  switch (which) {
    case 0: return sizeof(mlip_graph);
    case 1: return sizeof(mlip_moe_state);
    default: return 0;
  }
}

int mlip_moe_forward_vjp(const float *u, const int32_t *z, const float *logits, const float *W1,
                         const float *W2, int32_t n_atoms, int32_t n_types, int32_t n_experts,
                         int32_t top_k, int32_t d_node, int32_t d_hidden, const float *grad_out,
                         const mlip_moe_state *state, float *h_out, float *grad_u, float *q_out,
                         void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(state, "null MoE state");
  int32_t *topk = state->topk, *exp_off = state->exp_off, *tok_atom = state->tok_atom, *slot = state->slot;
  float *gate = state->gate, *P = state->P;
  MLIP_CHECK_ARG(n_atoms >= 0, "n_atoms must be >= 0");
  MLIP_CHECK_ARG(n_types >= 1 && n_types <= kMaxTypes, "n_types must be in [1, %d]", kMaxTypes);
  MLIP_CHECK_ARG(n_experts >= 1 && top_k >= 1 && top_k <= n_experts,
                 "need 1 <= top_k <= n_experts");
  MLIP_CHECK_ARG(n_experts <= kMaxExperts, "n_experts must be <= %d", kMaxExperts);
  MLIP_CHECK_ARG(int64_t(n_atoms) * top_k < (int64_t(1) << 31), "n_atoms * top_k too large");
  if (int rc = check_width(d_node, "d_node")) return rc;
  if (int rc = check_width(d_hidden, "d_hidden")) return rc;
  MLIP_CHECK_ARG(logits && W1 && W2 && topk && gate && exp_off, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (u && z && tok_atom && slot && P && h_out && grad_out && grad_u),
                 "null pointer argument");
  MLIP_CHECK_ARG(aligned(u, 16) && aligned(W1, 16) && aligned(W2, 16) && aligned(P, 16) &&
                     aligned(h_out, 16) && aligned(grad_out, 16) && aligned(grad_u, 16) &&
                     aligned(q_out, 16),
                 "float arrays must be 16-byte aligned");
  if (int rc = check_ws(ws, ws_bytes, mlip_moe_forward_vjp_workspace_size(n_atoms, n_types, n_experts,
                                                                          top_k, d_node, d_hidden)))
    return rc;
  MoeFwdVjpWs w = carve_moe_fwd_vjp(ws, n_atoms, n_types, n_experts, top_k, d_node, d_hidden, nullptr);
  const int M = n_atoms * top_k;
  if (int rc = moe_route_dispatch(z, logits, n_atoms, n_types, n_experts, top_k, topk, gate, exp_off,
                                  tok_atom, slot, w.f.local_rank, w.f.blk_count, w.f.n_type, w.f.pre,
                                  w.f.exp_count, w.f.flags, stream))
    return rc;
  if (n_atoms == 0) return MLIP_OK;
  GemmArgs g;  // P = u[tok] @ W1[x], act = silu(P)
  g.A = u; g.lda = d_node; g.a_rows = tok_atom; g.a_row_limit = n_atoms;
  g.B = W1; g.ldb = d_hidden; g.b_group_stride = int64_t(d_node) * d_hidden;
  g.C = P; g.C2 = w.f.act; g.ldc = d_hidden;
  g.group_off = exp_off; g.n_groups = n_experts;
  g.M = M; g.N = d_hidden; g.K = d_node;
  if (int rc = launch_gemm(g, false, EPI_SILU, K_GEMM_EXPERT_UP, stream)) return rc;
  // Y = act @ W2[x] (forward) and Q = (grad_out[tok] @ W2[x]^T) * silu'(P) (gradient) need only
  // P and grad_out: one launch
  GemmArgs g2;
  g2.A = w.f.act; g2.lda = d_hidden;
  g2.B = W2; g2.ldb = d_node; g2.b_group_stride = int64_t(d_hidden) * d_node;
  g2.C = w.f.Y; g2.ldc = d_node;
  g2.group_off = exp_off; g2.n_groups = n_experts;
  g2.M = M; g2.N = d_node; g2.K = d_hidden;
  GemmArgs g3;
  g3.A = grad_out; g3.lda = d_node; g3.a_rows = tok_atom; g3.a_row_limit = n_atoms;
  g3.B = W2; g3.ldb = d_node; g3.b_group_stride = int64_t(d_hidden) * d_node;
  g3.C = w.Q; g3.C2 = q_out; g3.ldc = d_hidden; g3.R = P; g3.ldr = d_hidden;
  g3.group_off = exp_off; g3.n_groups = n_experts;
  g3.M = M; g3.N = d_hidden; g3.K = d_node;
  if (int rc = launch_expert_pair(g2, false, EPI_STORE, g3, true, q_out ? EPI_DSILU_Q : EPI_DSILU,
                                  K_GEMM_EXPERT_PAIR, stream))
    return rc;
  if (int rc = moe_combine(u, w.f.Y, z, gate, slot, n_atoms, n_types, top_k, d_node, h_out, stream))
    return rc;
  GemmArgs g4;  // U_tok = Q @ W1[x]^T, into Y (the forward's combine has read it)
  g4.A = w.Q; g4.lda = d_hidden;
  g4.B = W1; g4.ldb = d_hidden; g4.b_group_stride = int64_t(d_node) * d_hidden;
  g4.C = w.f.Y; g4.ldc = d_node;
  g4.group_off = exp_off; g4.n_groups = n_experts;
  g4.M = M; g4.N = d_node; g4.K = d_hidden;
  if (int rc = launch_gemm(g4, true, EPI_STORE, K_GEMM_EXPERT_VJP_UP, stream)) return rc;
  return moe_combine(grad_out, w.f.Y, z, gate, slot, n_atoms, n_types, top_k, d_node, grad_u, stream);
}

size_t mlip_aggregate_vjp_workspace_size(int32_t n_atoms, int32_t d_edge, int32_t d_node) {
  size_t b = 0;
  carve_agg_vjp(nullptr, std::max(n_atoms, 0), std::max(d_edge, 0), std::max(d_node, 0), &b);
  return b;
}

int mlip_aggregate_vjp(const mlip_graph *graph, const float *e, const float *s, const float *W_e,
                       const float *W_d, const float *W_u, int32_t n_rbf, int32_t d_edge, int32_t d_node,
                       float cutoff, const float *grad_u, float *grad_h, float *grad_pos,
                       const int32_t *struct_ptr, int32_t n_structs, float *atom_virial,
                       double *grad_strain, void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(graph, "null graph");
  const int32_t *row_ptr = graph->row_ptr, *src = graph->src;
  const float *geom = graph->geom;
  const int32_t n_atoms = graph->n_atoms;
  const int64_t n_edges = graph->n_edges;
  MLIP_CHECK_ARG(n_atoms >= 0 && n_edges >= 0 && n_edges < (int64_t(1) << 31),
                 "n_atoms/n_edges out of range");
  MLIP_CHECK_ARG(n_rbf == MLIP_N_RBF, "n_rbf must be %d", MLIP_N_RBF);
  if (int rc = check_width(d_edge, "d_edge")) return rc;
  if (int rc = check_width(d_node, "d_node")) return rc;
  MLIP_CHECK_ARG(cutoff > 0.f && cutoff < 1e30f, "cutoff must be positive and finite");
  MLIP_CHECK_ARG(row_ptr && W_e && W_d && W_u, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (s && grad_u && grad_h && grad_pos), "null pointer argument");
  MLIP_CHECK_ARG(n_edges == 0 || (src && geom), "null edge pointer");
  MLIP_CHECK_ARG(!grad_strain || (struct_ptr && n_structs >= 1),
                 "grad_strain needs struct_ptr and n_structs >= 1");
  MLIP_CHECK_ARG(aligned(e, 16) && aligned(s, 16) && aligned(grad_u, 16) && aligned(grad_h, 16) &&
                     aligned(geom, 16),
                 "float arrays must be 16-byte aligned");
  if (int rc = check_ws(ws, ws_bytes, mlip_aggregate_vjp_workspace_size(n_atoms, d_edge, d_node)))
    return rc;
  if (n_atoms == 0) {
    if (grad_strain) return launch_strain_sum(nullptr, struct_ptr, n_structs, 0, grad_strain, stream);
    return MLIP_OK;
  }
  AggVjpWs w = carve_agg_vjp(ws, n_atoms, d_edge, d_node, nullptr);
  float *vir = atom_virial ? atom_virial : w.virial;
  GemmArgs g3;  // abar = ubar @ W_u^T
  g3.A = grad_u; g3.lda = d_node; g3.B = W_u; g3.ldb = d_node; g3.C = w.abar; g3.ldc = d_edge;
  g3.M = n_atoms; g3.N = d_edge; g3.K = d_node;
  g3.k_split = dense_k_split(n_atoms, d_edge, d_node); g3.split_ws = w.split;
  if (int rc = launch_gemm(g3, true, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
  if (int rc = launch_edge_vjp(row_ptr, src, geom, n_atoms, W_e, e, s, w.abar, d_edge, cutoff, w.sbar,
                               grad_pos, vir, stream))
    return rc;
  if (grad_strain) {
    if (int rc = launch_strain_sum(vir, struct_ptr, n_structs, n_atoms, grad_strain, stream)) return rc;
  }
  GemmArgs g4;  // grad_h = ubar + sbar @ W_d^T
  g4.A = w.sbar; g4.lda = d_edge; g4.B = W_d; g4.ldb = d_edge; g4.C = grad_h; g4.ldc = d_node;
  g4.R = grad_u; g4.ldr = d_node; g4.M = n_atoms; g4.N = d_node; g4.K = d_edge;
  return launch_gemm(g4, true, EPI_RESID, K_GEMM_DENSE, stream);
}

int mlip_moe_vjp(const int32_t *z, const float *gate, const int32_t *exp_off,
                 const int32_t *tok_atom, const int32_t *slot, const float *P, const float *W1,
                 const float *W2, int32_t n_atoms, int32_t n_types, int32_t n_experts,
                 int32_t top_k, int32_t d_node, int32_t d_hidden, const float *grad_out,
                 float *grad_in, float *q_out, void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0, "n_atoms must be >= 0");
  MLIP_CHECK_ARG(n_types >= 1 && n_types <= kMaxTypes, "n_types must be in [1, %d]", kMaxTypes);
  MLIP_CHECK_ARG(n_experts >= 1 && top_k >= 1 && top_k <= n_experts,
                 "need 1 <= top_k <= n_experts");
  MLIP_CHECK_ARG(n_experts <= kMaxExperts, "n_experts must be <= %d", kMaxExperts);
  MLIP_CHECK_ARG(int64_t(n_atoms) * top_k < (int64_t(1) << 31), "n_atoms * top_k too large");
  if (int rc = check_width(d_node, "d_node")) return rc;
  if (int rc = check_width(d_hidden, "d_hidden")) return rc;
  MLIP_CHECK_ARG(W1 && W2 && gate && exp_off, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (z && tok_atom && slot && P && grad_out && grad_in),
                 "null pointer argument");
  MLIP_CHECK_ARG(aligned(P, 16) && aligned(grad_out, 16) && aligned(grad_in, 16) &&
                     aligned(W1, 16) && aligned(W2, 16),
                 "float arrays must be 16-byte aligned");
  if (int rc = check_ws(ws, ws_bytes, mlip_moe_vjp_workspace_size(n_atoms, top_k, d_node, d_hidden)))
    return rc;
  if (n_atoms == 0) return MLIP_OK;
  MLIP_CHECK_ARG(aligned(q_out, 16), "float arrays must be 16-byte aligned");
  MoeVjpWs w = carve_moe_vjp(ws, n_atoms, top_k, d_node, d_hidden, nullptr);
  return moe_vjp_core(grad_out, z, gate, exp_off, tok_atom, slot, P, W1, W2, n_atoms, n_types,
                      n_experts, top_k, d_node, d_hidden, w.Q, w.Utok, grad_in, stream, q_out);
}

// ---------------------------------------------------------- attention ----
static int check_attn_dims(int32_t d_node, int32_t d_attn, int32_t n_heads, float cutoff,
                           int32_t n_rbf, int *cpl, int *lph) {
  MLIP_CHECK_ARG(n_rbf == MLIP_N_RBF, "n_rbf must be %d", MLIP_N_RBF);
  if (int rc = check_width(d_node, "d_node")) return rc;
  if (int rc = check_width(d_attn, "d_attn")) return rc;
  MLIP_CHECK_ARG(n_heads >= 1 && d_attn % n_heads == 0, "d_attn = %d must be a multiple of "
                 "n_heads = %d", d_attn, n_heads);
  MLIP_CHECK_ARG(cutoff > 0.f && cutoff < 1e30f, "cutoff must be positive and finite");
  if (attn_lane_layout(d_attn, n_heads, cpl, lph) != MLIP_OK) {
    set_error("unsupported attention shape: %d heads of width %d (need a width dh = c * 2^j, "
              "c in {1,2,3,4,6,8}, with n_heads * 2^j <= 64)", n_heads, d_attn / n_heads);
    return MLIP_ERR_UNSUPPORTED;
  }
  return MLIP_OK;
}

size_t mlip_attention_workspace_size(int32_t n_atoms, int32_t d_attn) {
  return size_t(dense_split_floats_max(std::max(n_atoms, 0), 3 * int64_t(std::max(d_attn, 0)))) * sizeof(float);
}

int mlip_attention(const int32_t *row_ptr, const int32_t *src, const float *geom, int32_t n_atoms,
                   int64_t n_edges, const float *h0, const float *W_qkv, const float *Wa_e,
                   const float *W_o, int32_t n_rbf, int32_t d_node, int32_t d_attn,
                   int32_t n_heads, float cutoff, float *qkv, float *o, float *stats, float *u,
                   void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0 && n_edges >= 0 && n_edges < (int64_t(1) << 31),
                 "n_atoms/n_edges out of range");
  int cpl = 0, lph = 0;
  if (int rc = check_attn_dims(d_node, d_attn, n_heads, cutoff, n_rbf, &cpl, &lph)) return rc;
  MLIP_CHECK_ARG(row_ptr && W_qkv && Wa_e && W_o, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (h0 && qkv && o && stats && u), "null pointer argument");
  MLIP_CHECK_ARG(n_edges == 0 || (src && geom), "null edge pointer");
  MLIP_CHECK_ARG(aligned(geom, 16) && aligned(h0, 16) && aligned(W_qkv, 16) && aligned(Wa_e, 16) &&
                     aligned(W_o, 16) && aligned(qkv, 16) && aligned(o, 16) && aligned(u, 16) &&
                     aligned(stats, 8),
                 "float arrays must be 16-byte aligned (stats 8-byte)");
  if (ws) {
    if (int rc = check_ws(ws, ws_bytes, mlip_attention_workspace_size(n_atoms, d_attn))) return rc;
  }
  if (n_atoms == 0) return MLIP_OK;
  GemmArgs g;  // [q | k | v] = h0 @ W_qkv
  g.A = h0; g.lda = d_node; g.B = W_qkv; g.ldb = 3 * int64_t(d_attn);
  g.C = qkv; g.ldc = 3 * int64_t(d_attn);
  g.M = n_atoms; g.N = 3 * d_attn; g.K = d_node;
  if (ws) {   // K split over the workspace when the output has few tiles
    g.k_split = dense_k_split(n_atoms, 3 * int64_t(d_attn), d_node);
    g.split_ws = static_cast<float *>(ws);
  }
  if (int rc = launch_gemm(g, false, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
  AttnArgs a;
  a.row_ptr = row_ptr; a.src = src; a.geom = geom; a.n_atoms = n_atoms;
  a.Wa_e = Wa_e; a.qkv = qkv; a.o = o; a.stats = stats;
  a.Da = d_attn; a.nh = n_heads; a.cpl = cpl; a.lph = lph; a.rc = cutoff;
  if (int rc = launch_attn_fwd(a, stream)) return rc;
  GemmArgs g2;  // u = h0 + o @ W_o
  g2.A = o; g2.lda = d_attn; g2.B = W_o; g2.ldb = d_node; g2.C = u; g2.ldc = d_node;
  g2.R = h0; g2.ldr = d_node; g2.M = n_atoms; g2.N = d_node; g2.K = d_attn;
  return launch_gemm(g2, false, EPI_RESID, K_GEMM_DENSE, stream);
}

size_t mlip_attention_vjp_workspace_size(int32_t n_atoms, int64_t n_edges, int32_t d_attn,
                                         int32_t n_heads) {
  size_t b = 0;
  carve_attn_vjp(nullptr, std::max(n_atoms, 0), std::max<int64_t>(n_edges, 0),
                 std::max(d_attn, 0), std::max(n_heads, 1), &b);
  return b;
}

int mlip_attention_vjp(const int32_t *row_ptr, const int32_t *src, const int32_t *rev,
                       const float *geom, int32_t n_atoms, int64_t n_edges, const float *qkv,
                       const float *o, const float *stats, const float *W_qkv, const float *Wa_e,
                       const float *W_o, int32_t n_rbf, int32_t d_node, int32_t d_attn,
                       int32_t n_heads, float cutoff, const float *grad_u, float *grad_h0,
                       float *grad_pos, const int32_t *struct_ptr, int32_t n_structs,
                       float *atom_virial, double *grad_strain, int32_t accumulate,
                       float *qkv_bar_out, void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0 && n_edges >= 0 && n_edges < (int64_t(1) << 31),
                 "n_atoms/n_edges out of range");
  MLIP_CHECK_ARG(aligned(qkv_bar_out, 16), "float arrays must be 16-byte aligned");
  int cpl = 0, lph = 0;
  if (int rc = check_attn_dims(d_node, d_attn, n_heads, cutoff, n_rbf, &cpl, &lph)) return rc;
  MLIP_CHECK_ARG(!accumulate || atom_virial || !grad_strain || n_atoms == 0,
                 "accumulating into grad_strain needs the accumulated atom_virial");
  MLIP_CHECK_ARG(row_ptr && W_qkv && Wa_e && W_o, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (qkv && o && stats && grad_u && grad_h0 && grad_pos),
                 "null pointer argument");
  MLIP_CHECK_ARG(n_edges == 0 || (src && rev && geom), "null edge pointer");
  MLIP_CHECK_ARG(!grad_strain || (struct_ptr && n_structs >= 1),
                 "grad_strain needs struct_ptr and n_structs >= 1");
  MLIP_CHECK_ARG(aligned(geom, 16) && aligned(qkv, 16) && aligned(o, 16) && aligned(stats, 8) &&
                     aligned(W_qkv, 16) && aligned(Wa_e, 16) && aligned(W_o, 16) &&
                     aligned(grad_u, 16) && aligned(grad_h0, 16),
                 "float arrays must be 16-byte aligned (stats 8-byte)");
  if (int rc = check_ws(ws, ws_bytes,
                        mlip_attention_vjp_workspace_size(n_atoms, n_edges, d_attn, n_heads)))
    return rc;
  if (n_atoms == 0) {
    if (grad_strain) return launch_strain_sum(nullptr, struct_ptr, n_structs, 0, grad_strain, stream);
    return MLIP_OK;
  }
  AttnVjpWs w = carve_attn_vjp(ws, n_atoms, n_edges, d_attn, n_heads, nullptr);
  float *vir = atom_virial ? atom_virial : w.virial;
  if (qkv_bar_out) w.qkv_bar = qkv_bar_out;
  GemmArgs g1;  // obar = ubar @ W_o^T
  g1.A = grad_u; g1.lda = d_node; g1.B = W_o; g1.ldb = d_node; g1.C = w.obar; g1.ldc = d_attn;
  g1.M = n_atoms; g1.N = d_attn; g1.K = d_node;
  g1.k_split = dense_k_split(n_atoms, d_attn, d_node); g1.split_ws = w.split;
  if (int rc = launch_gemm(g1, true, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
  AttnArgs a;
  a.row_ptr = row_ptr; a.src = src; a.rev = rev; a.geom = geom; a.n_atoms = n_atoms;
  a.Wa_e = Wa_e; a.qkv = qkv; a.o = const_cast<float *>(o);
  a.stats = const_cast<float *>(stats); a.obar = w.obar; a.qkv_bar = w.qkv_bar;
  a.edge_g = w.edge_g; a.edge_a = w.edge_a; a.edge_c = w.edge_c;
  a.grad_pos = grad_pos; a.atom_virial = vir; a.accumulate = accumulate ? 1 : 0;
  a.Da = d_attn; a.nh = n_heads; a.cpl = cpl; a.lph = lph; a.rc = cutoff;
  if (int rc = launch_attn_vjp(a, stream)) return rc;
  if (grad_strain) {
    if (int rc = launch_strain_sum(vir, struct_ptr, n_structs, n_atoms, grad_strain, stream)) return rc;
  }
  GemmArgs g2;  // grad_h0 = ubar + [qbar | kbar | vbar] @ W_qkv^T
  g2.A = w.qkv_bar; g2.lda = 3 * int64_t(d_attn); g2.B = W_qkv; g2.ldb = 3 * int64_t(d_attn);
  g2.C = grad_h0; g2.ldc = d_node; g2.R = grad_u; g2.ldr = d_node;
  g2.M = n_atoms; g2.N = d_node; g2.K = 3 * d_attn;
  return launch_gemm(g2, true, EPI_RESID, K_GEMM_DENSE, stream);
}

// --------------------------------------------------- three-body update ----
static int check_tri_dims(int32_t d_node, int32_t d_tri, int32_t n_ang, float cutoff, int *cpl) {
  MLIP_CHECK_ARG(n_ang == MLIP_N_ANG, "n_ang must be %d", MLIP_N_ANG);
  if (int rc = check_width(d_node, "d_node")) return rc;
  if (int rc = check_width(d_tri, "d_tri")) return rc;
  MLIP_CHECK_ARG(cutoff > 0.f && cutoff < 1e30f, "cutoff must be positive and finite");
  if (tri_lane_layout(d_tri, cpl) != MLIP_OK) {
    set_error("d_tri = %d too wide for one wavefront per row (at most 512)", d_tri);
    return MLIP_ERR_UNSUPPORTED;
  }
  return MLIP_OK;
}

size_t mlip_tri_workspace_size(int32_t n_atoms, int32_t d_tri) {
  return size_t(dense_split_floats_max(std::max(n_atoms, 0), std::max(d_tri, 0))) * sizeof(float);
}

int mlip_tri(const int32_t *row_ptr, const int32_t *src, const float *geom, int32_t n_atoms,
             int64_t n_edges, const float *h, const float *W_s, const float *W_ang, const float *W_T,
             int32_t n_ang, int32_t d_node, int32_t d_tri, float cutoff, float *s, float *tau,
             float *h_T, void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0 && n_edges >= 0 && n_edges < (int64_t(1) << 31),
                 "n_atoms/n_edges out of range");
  int cpl = 0;
  if (int rc = check_tri_dims(d_node, d_tri, n_ang, cutoff, &cpl)) return rc;
  MLIP_CHECK_ARG(row_ptr && W_s && W_ang && W_T, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (h && s && tau && h_T), "null pointer argument");
  MLIP_CHECK_ARG(n_edges == 0 || (src && geom), "null edge pointer");
  MLIP_CHECK_ARG(aligned(geom, 16) && aligned(h, 16) && aligned(W_s, 16) && aligned(W_ang, 16) &&
                     aligned(W_T, 16) && aligned(s, 16) && aligned(tau, 16) && aligned(h_T, 16),
                 "float arrays must be 16-byte aligned");
  if (ws) {
    if (int rc = check_ws(ws, ws_bytes, mlip_tri_workspace_size(n_atoms, d_tri))) return rc;
  }
  if (n_atoms == 0) return MLIP_OK;
  GemmArgs g;  // s = h @ W_s
  g.A = h; g.lda = d_node; g.B = W_s; g.ldb = d_tri; g.C = s; g.ldc = d_tri;
  g.M = n_atoms; g.N = d_tri; g.K = d_node;
  if (ws) {   // K split over the workspace when the output has few tiles
    g.k_split = dense_k_split(n_atoms, d_tri, d_node);
    g.split_ws = static_cast<float *>(ws);
  }
  if (int rc = launch_gemm(g, false, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
  TriArgs a;
  a.row_ptr = row_ptr; a.src = src; a.geom = geom; a.n_atoms = n_atoms;
  a.s = s; a.W_ang = W_ang; a.tau = tau; a.Dt = d_tri; a.cpl = cpl; a.rc = cutoff;
  if (int rc = launch_tri_fwd(a, stream)) return rc;
  GemmArgs g2;  // h_T = h + tau @ W_T
  g2.A = tau; g2.lda = d_tri; g2.B = W_T; g2.ldb = d_node; g2.C = h_T; g2.ldc = d_node;
  g2.R = h; g2.ldr = d_node; g2.M = n_atoms; g2.N = d_node; g2.K = d_tri;
  return launch_gemm(g2, false, EPI_RESID, K_GEMM_DENSE, stream);
}

size_t mlip_tri_vjp_workspace_size(int32_t n_atoms, int64_t n_edges, int32_t d_tri) {
  size_t b = 0;
  carve_tri_vjp(nullptr, std::max(n_atoms, 0), std::max<int64_t>(n_edges, 0), std::max(d_tri, 0),
                &b);
  return b;
}

int mlip_tri_vjp(const int32_t *row_ptr, const int32_t *src, const int32_t *rev, const float *geom,
                 int32_t n_atoms, int64_t n_edges, const float *s, const float *W_s,
                 const float *W_ang, const float *W_T, int32_t n_ang, int32_t d_node,
                 int32_t d_tri, float cutoff, const float *grad_hT, float *grad_h,
                 float *grad_pos, const int32_t *struct_ptr, int32_t n_structs,
                 float *atom_virial, double *grad_strain, int32_t accumulate, float *sbar_out,
                 void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0 && n_edges >= 0 && n_edges < (int64_t(1) << 31),
                 "n_atoms/n_edges out of range");
  MLIP_CHECK_ARG(aligned(sbar_out, 16), "float arrays must be 16-byte aligned");
  int cpl = 0;
  if (int rc = check_tri_dims(d_node, d_tri, n_ang, cutoff, &cpl)) return rc;
  MLIP_CHECK_ARG(row_ptr && W_s && W_ang && W_T, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (s && grad_hT && grad_h && grad_pos), "null pointer argument");
  MLIP_CHECK_ARG(n_edges == 0 || (src && rev && geom), "null edge pointer");
  MLIP_CHECK_ARG(!grad_strain || (struct_ptr && n_structs >= 1),
                 "grad_strain needs struct_ptr and n_structs >= 1");
  MLIP_CHECK_ARG(!accumulate || atom_virial || !grad_strain || n_atoms == 0,
                 "accumulating into grad_strain needs the accumulated atom_virial");
  MLIP_CHECK_ARG(aligned(geom, 16) && aligned(s, 16) && aligned(W_s, 16) && aligned(W_ang, 16) &&
                     aligned(W_T, 16) && aligned(grad_hT, 16) && aligned(grad_h, 16),
                 "float arrays must be 16-byte aligned");
  if (int rc = check_ws(ws, ws_bytes, mlip_tri_vjp_workspace_size(n_atoms, n_edges, d_tri)))
    return rc;
  if (n_atoms == 0) {
    if (grad_strain) return launch_strain_sum(nullptr, struct_ptr, n_structs, 0, grad_strain, stream);
    return MLIP_OK;
  }
  TriVjpWs w = carve_tri_vjp(ws, n_atoms, n_edges, d_tri, nullptr);
  float *vir = atom_virial ? atom_virial : w.virial;
  if (sbar_out) w.sbar = sbar_out;
  GemmArgs g1;  // taubar = grad_hT @ W_T^T
  g1.A = grad_hT; g1.lda = d_node; g1.B = W_T; g1.ldb = d_node; g1.C = w.taubar; g1.ldc = d_tri;
  g1.M = n_atoms; g1.N = d_tri; g1.K = d_node;
  g1.k_split = dense_k_split(n_atoms, d_tri, d_node); g1.split_ws = w.split;
  if (int rc = launch_gemm(g1, true, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
  TriArgs a;
  a.row_ptr = row_ptr; a.src = src; a.rev = rev; a.geom = geom; a.n_atoms = n_atoms;
  a.s = s; a.W_ang = W_ang; a.taubar = w.taubar; a.sigma = w.sigma; a.gvec = w.gvec;
  a.sbar = w.sbar; a.grad_pos = grad_pos; a.atom_virial = vir;
  a.accumulate = accumulate ? 1 : 0; a.Dt = d_tri; a.cpl = cpl; a.rc = cutoff;
  if (int rc = launch_tri_vjp(a, stream)) return rc;
  if (grad_strain) {
    if (int rc = launch_strain_sum(vir, struct_ptr, n_structs, n_atoms, grad_strain, stream)) return rc;
  }
  GemmArgs g2;  // grad_h = grad_hT + sbar @ W_s^T
  g2.A = w.sbar; g2.lda = d_tri; g2.B = W_s; g2.ldb = d_tri; g2.C = grad_h; g2.ldc = d_node;
  g2.R = grad_hT; g2.ldr = d_node; g2.M = n_atoms; g2.N = d_node; g2.K = d_tri;
  return launch_gemm(g2, true, EPI_RESID, K_GEMM_DENSE, stream);
}

// ----------------------------------------------- training gradient: JVP ---
size_t mlip_block_jvp_workspace_size(int32_t n_atoms, int32_t top_k, int32_t d_node,
                                     int32_t d_hidden) {
  size_t b = 0;
  carve_jvp(nullptr, std::max(n_atoms, 0), std::max(top_k, 1), std::max(d_node, 0),
            std::max(d_hidden, 0), &b);
  return b;
}

static int check_block_dims(int32_t n_atoms, int64_t n_edges, int32_t n_rbf, int32_t d_edge,
                            int32_t d_node, int32_t d_hidden, int32_t n_types, int32_t n_experts,
                            int32_t top_k, float cutoff) {
  MLIP_CHECK_ARG(n_atoms >= 0 && n_edges >= 0 && n_edges < (int64_t(1) << 31),
                 "n_atoms/n_edges out of range");
  MLIP_CHECK_ARG(n_rbf == MLIP_N_RBF, "n_rbf must be %d", MLIP_N_RBF);
  MLIP_CHECK_ARG(n_types >= 1 && n_types <= kMaxTypes, "n_types must be in [1, %d]", kMaxTypes);
  MLIP_CHECK_ARG(n_experts >= 1 && top_k >= 1 && top_k <= n_experts,
                 "need 1 <= top_k <= n_experts");
  MLIP_CHECK_ARG(n_experts <= kMaxExperts, "n_experts must be <= %d", kMaxExperts);
  MLIP_CHECK_ARG(int64_t(n_atoms) * top_k < (int64_t(1) << 31), "n_atoms * top_k too large");
  if (int rc = check_width(d_edge, "d_edge")) return rc;
  if (int rc = check_width(d_node, "d_node")) return rc;
  if (int rc = check_width(d_hidden, "d_hidden")) return rc;
  MLIP_CHECK_ARG(cutoff > 0.f && cutoff < 1e30f, "cutoff must be positive and finite");
  return MLIP_OK;
}

int mlip_block_jvp(const int32_t *row_ptr, const int32_t *src, const float *geom, int32_t n_atoms,
                   int64_t n_edges, const float *grad_forces, const float *h_dot, const float *s,
                   const int32_t *z, const float *gate, const int32_t *exp_off,
                   const int32_t *tok_atom, const int32_t *slot, const float *P, const float *W_e,
                   const float *W_d, const float *W_u, const float *W1, const float *W2,
                   int32_t n_rbf, int32_t d_edge, int32_t d_node, int32_t d_hidden,
                   int32_t n_types, int32_t n_experts, int32_t top_k, float cutoff, float *a,
                   float *s_dot, float *a_dot, float *u_dot, float *P_dot, float *h_out_dot,
                   void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (int rc = check_block_dims(n_atoms, n_edges, n_rbf, d_edge, d_node, d_hidden, n_types,
                                n_experts, top_k, cutoff))
    return rc;
  MLIP_CHECK_ARG(row_ptr && W_e && W_d && W_u && W1 && W2 && gate && exp_off, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (grad_forces && s && z && tok_atom && slot && P && a_dot && u_dot &&
                                  P_dot),
                 "null pointer argument");
  MLIP_CHECK_ARG(!h_dot || s_dot, "h_dot needs s_dot");
  MLIP_CHECK_ARG(n_edges == 0 || (src && geom), "null edge pointer");
  MLIP_CHECK_ARG(aligned(geom, 16) && aligned(h_dot, 16) && aligned(s, 16) && aligned(P, 16) &&
                     aligned(a, 16) && aligned(s_dot, 16) && aligned(a_dot, 16) &&
                     aligned(u_dot, 16) && aligned(P_dot, 16) && aligned(h_out_dot, 16) &&
                     aligned(W_e, 16) && aligned(W_d, 16) && aligned(W_u, 16) && aligned(W1, 16) &&
                     aligned(W2, 16),
                 "float arrays must be 16-byte aligned");
  if (int rc = check_ws(ws, ws_bytes, mlip_block_jvp_workspace_size(n_atoms, top_k, d_node, d_hidden)))
    return rc;
  if (n_atoms == 0) return MLIP_OK;
  JvpWs w = carve_jvp(ws, n_atoms, top_k, d_node, d_hidden, nullptr);
  const int M = n_atoms * top_k;
  if (h_dot) {
    GemmArgs g;  // s_dot = h_dot @ W_d
    g.A = h_dot; g.lda = d_node; g.B = W_d; g.ldb = d_edge; g.C = s_dot; g.ldc = d_edge;
    g.M = n_atoms; g.N = d_edge; g.K = d_node;
    if (int rc = launch_gemm(g, false, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
  }
  EdgeTanArgs et;  // a_dot = sum_e e_dot * s_src + e * s_dot_src, a = sum_e e * s_src
  et.row_ptr = row_ptr; et.src = src; et.geom = geom; et.n_atoms = n_atoms;
  et.x_dot = grad_forces; et.x_sign = -1.f; et.W_e = W_e;
  et.X = s; et.Y = h_dot ? s_dot : nullptr; et.out1 = a_dot; et.out2 = a;
  et.De = d_edge; et.rc = cutoff;
  if (int rc = launch_edge_tan(et, stream)) return rc;
  GemmArgs g2;  // u_dot = h_dot + a_dot @ W_u
  g2.A = a_dot; g2.lda = d_edge; g2.B = W_u; g2.ldb = d_node; g2.C = u_dot; g2.ldc = d_node;
  g2.R = h_dot; g2.ldr = d_node; g2.M = n_atoms; g2.N = d_node; g2.K = d_edge;
  if (int rc = launch_gemm(g2, false, h_dot ? EPI_RESID : EPI_STORE, K_GEMM_DENSE, stream)) return rc;
  return moe_jvp_core(u_dot, z, gate, exp_off, tok_atom, slot, P, W1, W2, n_atoms, n_types, n_experts,
                      top_k, d_node, d_hidden, P_dot, w.act_dot, w.Y_dot, h_out_dot, stream);
}

// ------------------------------------- training gradient: tangent of VJP ---
size_t mlip_block_tangent_vjp_workspace_size(int32_t n_atoms, int32_t n_types, int32_t top_k,
                                             int32_t d_edge, int32_t d_node, int32_t d_hidden) {
  size_t b = 0;
  carve_tan_vjp(nullptr, std::max(n_atoms, 0), std::max(n_types, 1), std::max(top_k, 1),
                std::max(d_edge, 0), std::max(d_node, 0), std::max(d_hidden, 0), &b, nullptr);
  return b;
}

int mlip_block_tangent_vjp(
    const int32_t *row_ptr, const int32_t *src, const float *geom, int32_t n_atoms, int64_t n_edges,
    const float *grad_forces, const float *h_dot, const float *h, const float *s,
    const float *s_dot, const float *a, const float *a_dot, const float *u, const float *u_dot,
    const int32_t *z, const int32_t *topk, const float *gate, const int32_t *exp_off,
    const int32_t *tok_atom, const int32_t *slot, const float *P, const float *P_dot,
    const float *grad_out, const float *ubar, const float *Q, const float *grad_out_dot,
    const float *W_e, const float *W_d, const float *W_u, const float *W1, const float *W2,
    int32_t n_rbf, int32_t d_edge, int32_t d_node, int32_t d_hidden, int32_t n_types,
    int32_t n_experts, int32_t top_k, float cutoff, float *grad_h_dot, float *d_W_e,
    float *d_W_d, float *d_W_u, float *d_W1, float *d_W2, float *d_gate, float *d_logits,
    void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (int rc = check_block_dims(n_atoms, n_edges, n_rbf, d_edge, d_node, d_hidden, n_types,
                                n_experts, top_k, cutoff))
    return rc;
  MLIP_CHECK_ARG(row_ptr && W_e && W_d && W_u && W1 && W2 && topk && gate && exp_off && d_W_e &&
                     d_W_d && d_W_u && d_W1 && d_W2,
                 "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (grad_forces && h && s && a && a_dot && u && u_dot && z &&
                                  tok_atom && slot && P && P_dot && grad_out && ubar && Q),
                 "null pointer argument");
  MLIP_CHECK_ARG(!h_dot || s_dot, "h_dot needs s_dot");
  MLIP_CHECK_ARG(n_edges == 0 || (src && geom), "null edge pointer");
  MLIP_CHECK_ARG(aligned(geom, 16) && aligned(h_dot, 16) && aligned(h, 16) && aligned(s, 16) &&
                     aligned(s_dot, 16) && aligned(a, 16) && aligned(a_dot, 16) && aligned(u, 16) &&
                     aligned(u_dot, 16) && aligned(P, 16) && aligned(P_dot, 16) &&
                     aligned(grad_out, 16) && aligned(ubar, 16) && aligned(Q, 16) &&
                     aligned(grad_out_dot, 16) && aligned(grad_h_dot, 16) && aligned(W_e, 16) &&
                     aligned(W_d, 16) && aligned(W_u, 16) && aligned(W1, 16) && aligned(W2, 16) &&
                     aligned(d_W_e, 16) && aligned(d_W_d, 16) && aligned(d_W_u, 16) &&
                     aligned(d_W1, 16) && aligned(d_W2, 16),
                 "float arrays must be 16-byte aligned");
  if (int rc = check_ws(ws, ws_bytes, mlip_block_tangent_vjp_workspace_size(
                                          n_atoms, n_types, top_k, d_edge, d_node, d_hidden)))
    return rc;
  MoeTanWs mw;
  TanVjpWs w = carve_tan_vjp(ws, n_atoms, n_types, top_k, d_edge, d_node, d_hidden, nullptr, &mw);
  const int N = n_atoms;
  const int De = d_edge, Dn = d_node;

  // MoE: gradient tangent into ubar_dot, W1 / W2 / gate / logit gradients
  if (int rc = moe_tvjp_core(z, topk, gate, exp_off, tok_atom, slot, P, P_dot, W1, W2, N, n_types,
                             n_experts, top_k, Dn, d_hidden, u, u_dot, grad_out, Q, grad_out_dot, mw,
                             w.ubar_dot, d_W1, d_W2, d_gate, d_logits, stream))
    return rc;
  if (N > 0) {
    // ---- projections: abar = ubar W_u^T, abar_dot = ubar_dot W_u^T ----
    GemmArgs g3;
    g3.A = ubar; g3.lda = Dn; g3.B = W_u; g3.ldb = Dn; g3.C = w.abar; g3.ldc = De;
    g3.M = N; g3.N = De; g3.K = Dn;
    g3.k_split = dense_k_split(N, De, Dn); g3.split_ws = w.split;
    if (int rc = launch_gemm(g3, true, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
    g3.A = w.ubar_dot; g3.C = w.abar_dot;
    if (int rc = launch_gemm(g3, true, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
  }
  // ---- edges: sbar_dot, sbar (with h_dot) and the W_e gradient ----
  EdgeTanArgs et;
  et.row_ptr = row_ptr; et.src = src; et.geom = geom; et.n_atoms = N;
  et.x_dot = grad_forces; et.x_sign = -1.f; et.W_e = W_e;
  et.X = w.abar; et.Y = w.abar_dot; et.out1 = w.sbar_dot; et.out2 = h_dot ? w.sbar : nullptr;
  et.R1 = s; et.R2 = h_dot ? s_dot : nullptr; et.dwe = d_W_e; et.dwe_part = w.dwe_part;
  et.De = De; et.rc = cutoff;
  if (int rc = launch_edge_tan(et, stream)) return rc;
  if (grad_h_dot && N > 0) {
    GemmArgs g;  // grad_h_dot = ubar_dot + sbar_dot W_d^T
    g.A = w.sbar_dot; g.lda = De; g.B = W_d; g.ldb = De; g.C = grad_h_dot; g.ldc = Dn;
    g.R = w.ubar_dot; g.ldr = Dn; g.M = N; g.N = Dn; g.K = De;
    if (int rc = launch_gemm(g, true, EPI_RESID, K_GEMM_DENSE, stream)) return rc;
  }
  {
    WgradArgs q;  // d W_u = sum_i a_dot_i^T ubar_i + a_i^T ubar_dot_i
    q.A0 = a_dot; q.B0 = ubar; q.A1 = a; q.B1 = w.ubar_dot; q.lda = De; q.ldb = Dn;
    q.P = N; q.Mo = De; q.No = Dn; q.C = d_W_u;
    if (int rc = launch_wgrad(q, w.split, stream)) return rc;
  }
  WgradArgs q;  // d W_d = sum_i h_dot_i^T sbar_i + h_i^T sbar_dot_i
  q.A0 = h; q.B0 = w.sbar_dot;
  if (h_dot) { q.A1 = h_dot; q.B1 = w.sbar; }
  q.lda = Dn; q.ldb = De; q.P = N; q.Mo = Dn; q.No = De; q.C = d_W_d;
  return launch_wgrad(q, w.split, stream);
}

// ------------------------------------------------------- readout grads ---
int mlip_readout_vjp(const float *w_r, const double *grad_energy, const int32_t *struct_ptr,
                     int32_t n_atoms, int32_t n_structs, int32_t d_node, float *grad_h_out,
                     void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0 && n_structs >= 1, "n_atoms >= 0 and n_structs >= 1 required");
  if (int rc = check_width(d_node, "d_node")) return rc;
  MLIP_CHECK_ARG(w_r && struct_ptr && (n_atoms == 0 || grad_h_out), "null pointer argument");
  MLIP_CHECK_ARG(aligned(w_r, 16) && aligned(grad_h_out, 16), "float arrays must be 16-byte aligned");
  if (n_atoms == 0) return MLIP_OK;
  return launch_readout_seed(w_r, grad_energy, struct_ptr, n_atoms, n_structs, d_node, grad_h_out,
                             stream);
}

size_t mlip_readout_grad_workspace_size(int32_t n_atoms, int32_t d_node) {
  return size_t(readout_grad_part_floats(std::max(n_atoms, 0), std::max(d_node, 0))) * sizeof(float);
}

int mlip_readout_grad(const float *h_out, const float *h_out_dot, const double *grad_energy,
                      const int32_t *struct_ptr, int32_t n_atoms, int32_t n_structs, int32_t d_node,
                      float *d_w_r, void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0 && n_structs >= 1, "n_atoms >= 0 and n_structs >= 1 required");
  if (int rc = check_width(d_node, "d_node")) return rc;
  MLIP_CHECK_ARG(struct_ptr && d_w_r && (n_atoms == 0 || h_out), "null pointer argument");
  MLIP_CHECK_ARG(aligned(h_out, 16) && aligned(h_out_dot, 16), "float arrays must be 16-byte aligned");
  if (int rc = check_ws(ws, ws_bytes, mlip_readout_grad_workspace_size(n_atoms, d_node))) return rc;
  return launch_readout_grad(h_out, h_out_dot, grad_energy, struct_ptr, n_atoms, n_structs, d_node,
                             static_cast<float *>(ws), d_w_r, stream);
}

// ------------------------------------------- MoE layer: training tangents ---
size_t mlip_moe_jvp_workspace_size(int32_t n_atoms, int32_t top_k, int32_t d_node, int32_t d_hidden) {
  return mlip_block_jvp_workspace_size(n_atoms, top_k, d_node, d_hidden);
}

static int check_moe_dims(int32_t n_atoms, int32_t n_types, int32_t n_experts, int32_t top_k,
                          int32_t d_node, int32_t d_hidden) {
  MLIP_CHECK_ARG(n_atoms >= 0, "n_atoms must be >= 0");
  MLIP_CHECK_ARG(n_types >= 1 && n_types <= kMaxTypes, "n_types must be in [1, %d]", kMaxTypes);
  MLIP_CHECK_ARG(n_experts >= 1 && top_k >= 1 && top_k <= n_experts,
                 "need 1 <= top_k <= n_experts");
  MLIP_CHECK_ARG(n_experts <= kMaxExperts, "n_experts must be <= %d", kMaxExperts);
  MLIP_CHECK_ARG(int64_t(n_atoms) * top_k < (int64_t(1) << 31), "n_atoms * top_k too large");
  if (int rc = check_width(d_node, "d_node")) return rc;
  return check_width(d_hidden, "d_hidden");
}

int mlip_moe_jvp(const int32_t *z, const float *gate, const int32_t *exp_off, const int32_t *tok_atom,
                 const int32_t *slot, const float *P, const float *W1, const float *W2, int32_t n_atoms,
                 int32_t n_types, int32_t n_experts, int32_t top_k, int32_t d_node, int32_t d_hidden,
                 const float *u_dot, float *P_dot, float *h_out_dot, void *ws, size_t ws_bytes,
                 void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (int rc = check_moe_dims(n_atoms, n_types, n_experts, top_k, d_node, d_hidden)) return rc;
  MLIP_CHECK_ARG(W1 && W2 && gate && exp_off, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (z && tok_atom && slot && P && u_dot && P_dot), "null pointer argument");
  MLIP_CHECK_ARG(aligned(P, 16) && aligned(u_dot, 16) && aligned(P_dot, 16) && aligned(h_out_dot, 16) &&
                     aligned(W1, 16) && aligned(W2, 16),
                 "float arrays must be 16-byte aligned");
  if (int rc = check_ws(ws, ws_bytes, mlip_moe_jvp_workspace_size(n_atoms, top_k, d_node, d_hidden)))
    return rc;
  if (n_atoms == 0) return MLIP_OK;
  JvpWs w = carve_jvp(ws, n_atoms, top_k, d_node, d_hidden, nullptr);
  return moe_jvp_core(u_dot, z, gate, exp_off, tok_atom, slot, P, W1, W2, n_atoms, n_types, n_experts,
                      top_k, d_node, d_hidden, P_dot, w.act_dot, w.Y_dot, h_out_dot, stream);
}

size_t mlip_moe_tangent_vjp_workspace_size(int32_t n_atoms, int32_t n_types, int32_t top_k,
                                           int32_t d_node, int32_t d_hidden) {
  Carver c(nullptr);
  carve_moe_tan(c, std::max(n_atoms, 0), std::max(n_types, 1), std::max(top_k, 1), std::max(d_node, 0),
                std::max(d_hidden, 0));
  return c.bytes();
}

int mlip_moe_tangent_vjp(const int32_t *z, const int32_t *topk, const float *gate,
                         const int32_t *exp_off, const int32_t *tok_atom, const int32_t *slot,
                         const float *P, const float *P_dot, const float *W1, const float *W2,
                         int32_t n_atoms, int32_t n_types, int32_t n_experts, int32_t top_k,
                         int32_t d_node, int32_t d_hidden, const float *u, const float *u_dot,
                         const float *grad_out, const float *Q, const float *grad_out_dot,
                         float *grad_in_dot, float *d_W1, float *d_W2, float *d_gate, float *d_logits,
                         void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (int rc = check_moe_dims(n_atoms, n_types, n_experts, top_k, d_node, d_hidden)) return rc;
  MLIP_CHECK_ARG(W1 && W2 && topk && gate && exp_off && d_W1 && d_W2, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (z && tok_atom && slot && P && P_dot && u && u_dot && grad_out && Q),
                 "null pointer argument");
  MLIP_CHECK_ARG(aligned(P, 16) && aligned(P_dot, 16) && aligned(u, 16) && aligned(u_dot, 16) &&
                     aligned(grad_out, 16) && aligned(Q, 16) && aligned(grad_out_dot, 16) &&
                     aligned(grad_in_dot, 16) && aligned(W1, 16) && aligned(W2, 16) &&
                     aligned(d_W1, 16) && aligned(d_W2, 16),
                 "float arrays must be 16-byte aligned");
  if (int rc = check_ws(ws, ws_bytes, mlip_moe_tangent_vjp_workspace_size(n_atoms, n_types, top_k,
                                                                          d_node, d_hidden)))
    return rc;
  Carver c(ws);
  MoeTanWs w = carve_moe_tan(c, n_atoms, n_types, top_k, d_node, d_hidden);
  return moe_tvjp_core(z, topk, gate, exp_off, tok_atom, slot, P, P_dot, W1, W2, n_atoms, n_types,
                       n_experts, top_k, d_node, d_hidden, u, u_dot, grad_out, Q, grad_out_dot, w,
                       grad_in_dot, d_W1, d_W2, d_gate, d_logits, stream);
}

// ------------------------------------------- attention: training tangents ---
int mlip_attention_jvp(const int32_t *row_ptr, const int32_t *src, const float *geom, int32_t n_atoms,
                       int64_t n_edges, const float *grad_forces, const float *h0_dot, const float *qkv,
                       const float *o, const float *stats, const float *W_qkv, const float *Wa_e,
                       const float *W_o, int32_t n_rbf, int32_t d_node, int32_t d_attn, int32_t n_heads,
                       float cutoff, float *qkv_dot, float *o_dot, float *tstat, float *u_dot,
                       void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0 && n_edges >= 0 && n_edges < (int64_t(1) << 31),
                 "n_atoms/n_edges out of range");
  int cpl = 0, lph = 0;
  if (int rc = check_attn_dims(d_node, d_attn, n_heads, cutoff, n_rbf, &cpl, &lph)) return rc;
  MLIP_CHECK_ARG(row_ptr && W_qkv && Wa_e && W_o, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (grad_forces && h0_dot && qkv && o && stats && qkv_dot && o_dot &&
                                  tstat && u_dot),
                 "null pointer argument");
  MLIP_CHECK_ARG(n_edges == 0 || (src && geom), "null edge pointer");
  MLIP_CHECK_ARG(aligned(geom, 16) && aligned(h0_dot, 16) && aligned(qkv, 16) && aligned(o, 16) &&
                     aligned(stats, 8) && aligned(W_qkv, 16) && aligned(Wa_e, 16) && aligned(W_o, 16) &&
                     aligned(qkv_dot, 16) && aligned(o_dot, 16) && aligned(u_dot, 16),
                 "float arrays must be 16-byte aligned (stats 8-byte)");
  if (n_atoms == 0) return MLIP_OK;
  GemmArgs g;  // [q_dot | k_dot | v_dot] = h0_dot W_qkv
  g.A = h0_dot; g.lda = d_node; g.B = W_qkv; g.ldb = 3 * int64_t(d_attn); g.C = qkv_dot;
  g.ldc = 3 * int64_t(d_attn); g.M = n_atoms; g.N = 3 * d_attn; g.K = d_node;
  if (int rc = launch_gemm(g, false, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
  AttnTanArgs a;
  a.row_ptr = row_ptr; a.src = src; a.geom = geom; a.n_atoms = n_atoms;
  a.x_dot = grad_forces; a.x_sign = -1.f; a.Wa_e = Wa_e; a.qkv = qkv; a.qkv_dot = qkv_dot;
  a.o = o; a.o_dot = o_dot; a.stats = stats; a.tstat = tstat;
  a.Da = d_attn; a.nh = n_heads; a.cpl = cpl; a.lph = lph; a.rc = cutoff;
  if (int rc = launch_attn_jvp(a, stream)) return rc;
  GemmArgs g2;  // u_dot = h0_dot + o_dot W_o
  g2.A = o_dot; g2.lda = d_attn; g2.B = W_o; g2.ldb = d_node; g2.C = u_dot; g2.ldc = d_node;
  g2.R = h0_dot; g2.ldr = d_node; g2.M = n_atoms; g2.N = d_node; g2.K = d_attn;
  return launch_gemm(g2, false, EPI_RESID, K_GEMM_DENSE, stream);
}

size_t mlip_attention_tangent_vjp_workspace_size(int32_t n_atoms, int64_t n_edges, int32_t d_node,
                                                 int32_t d_attn, int32_t n_heads) {
  size_t b = 0;
  carve_attn_tan(nullptr, std::max(n_atoms, 0), std::max<int64_t>(n_edges, 0), std::max(d_node, 0),
                 std::max(d_attn, 0), std::max(n_heads, 1), &b);
  return b;
}

int mlip_attention_tangent_vjp(
    const int32_t *row_ptr, const int32_t *src, const int32_t *rev, const float *geom, int32_t n_atoms,
    int64_t n_edges, const float *grad_forces, const float *h0, const float *h0_dot, const float *qkv,
    const float *qkv_dot, const float *o, const float *o_dot, const float *stats, const float *tstat,
    const float *qkv_bar, const float *W_qkv, const float *Wa_e, const float *W_o, int32_t n_rbf,
    int32_t d_node, int32_t d_attn, int32_t n_heads, float cutoff, const float *grad_u,
    const float *grad_u_dot, float *grad_h0_dot, float *d_W_qkv, float *d_Wa_e, float *d_W_o, void *ws,
    size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0 && n_edges >= 0 && n_edges < (int64_t(1) << 31),
                 "n_atoms/n_edges out of range");
  int cpl = 0, lph = 0;
  if (int rc = check_attn_dims(d_node, d_attn, n_heads, cutoff, n_rbf, &cpl, &lph)) return rc;
  MLIP_CHECK_ARG(row_ptr && W_qkv && Wa_e && W_o && d_W_qkv && d_Wa_e && d_W_o, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (grad_forces && h0 && h0_dot && qkv && qkv_dot && o && o_dot && stats &&
                                  tstat && qkv_bar && grad_u && grad_u_dot),
                 "null pointer argument");
  MLIP_CHECK_ARG(n_edges == 0 || (src && rev && geom), "null edge pointer");
  MLIP_CHECK_ARG(aligned(geom, 16) && aligned(h0, 16) && aligned(h0_dot, 16) && aligned(qkv, 16) &&
                     aligned(qkv_dot, 16) && aligned(o, 16) && aligned(o_dot, 16) && aligned(stats, 8) &&
                     aligned(qkv_bar, 16) && aligned(W_qkv, 16) && aligned(Wa_e, 16) && aligned(W_o, 16) &&
                     aligned(grad_u, 16) && aligned(grad_u_dot, 16) && aligned(grad_h0_dot, 16) &&
                     aligned(d_W_qkv, 16) && aligned(d_Wa_e, 16) && aligned(d_W_o, 16),
                 "float arrays must be 16-byte aligned (stats 8-byte)");
  if (int rc = check_ws(ws, ws_bytes, mlip_attention_tangent_vjp_workspace_size(n_atoms, n_edges, d_node,
                                                                                d_attn, n_heads)))
    return rc;
  AttnTanWs w = carve_attn_tan(ws, n_atoms, n_edges, d_node, d_attn, n_heads, nullptr);
  const int N = n_atoms, Da = d_attn, Dn = d_node;
  if (N > 0) {
    GemmArgs g;  // obar = ubar W_o^T, obar_dot = ubar_dot W_o^T
    g.A = grad_u; g.lda = Dn; g.B = W_o; g.ldb = Dn; g.C = w.obar; g.ldc = Da;
    g.M = N; g.N = Da; g.K = Dn;
    g.k_split = dense_k_split(N, Da, Dn); g.split_ws = w.split;
    if (int rc = launch_gemm(g, true, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
    g.A = grad_u_dot; g.C = w.obar_dot;
    if (int rc = launch_gemm(g, true, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
    AttnTanArgs a;
    a.row_ptr = row_ptr; a.src = src; a.rev = rev; a.geom = geom; a.n_atoms = N;
    a.x_dot = grad_forces; a.x_sign = -1.f; a.Wa_e = Wa_e; a.qkv = qkv; a.qkv_dot = qkv_dot;
    a.o = o; a.o_dot = const_cast<float *>(o_dot); a.stats = stats; a.tstat = const_cast<float *>(tstat);
    a.obar = w.obar; a.obar_dot = w.obar_dot; a.qkv_bar_dot = w.qkv_bar_dot;
    a.edge_g = w.eg; a.edge_gd = w.egd; a.edge_a = w.ea; a.edge_ad = w.ead;
    a.ebar = w.ebar; a.ebar_dot = w.ebar_dot;
    a.Da = Da; a.nh = n_heads; a.cpl = cpl; a.lph = lph; a.rc = cutoff;
    if (int rc = launch_attn_tvjp(a, stream)) return rc;
  }
  if (int rc = launch_edge_basis_grad(row_ptr, src, geom, N, grad_forces, -1.f, w.ebar, w.ebar_dot, Da,
                                      cutoff, w.part, d_Wa_e, stream))
    return rc;
  if (grad_h0_dot && N > 0) {
    GemmArgs g;  // grad_h0_dot = ubar_dot + [q|k|v]bar_dot W_qkv^T
    g.A = w.qkv_bar_dot; g.lda = 3 * int64_t(Da); g.B = W_qkv; g.ldb = 3 * int64_t(Da);
    g.C = grad_h0_dot; g.ldc = Dn; g.R = grad_u_dot; g.ldr = Dn; g.M = N; g.N = Dn; g.K = 3 * Da;
    if (int rc = launch_gemm(g, true, EPI_RESID, K_GEMM_DENSE, stream)) return rc;
  }
  {
    WgradArgs q;  // d W_qkv = sum_i h0_dot_i^T [q|k|v]bar_i + h0_i^T [q|k|v]bar_dot_i
    q.A0 = h0_dot; q.B0 = qkv_bar; q.A1 = h0; q.B1 = w.qkv_bar_dot; q.lda = Dn; q.ldb = 3 * int64_t(Da);
    q.P = N; q.Mo = Dn; q.No = 3 * Da; q.C = d_W_qkv;
    if (int rc = launch_wgrad(q, w.split, stream)) return rc;
  }
  WgradArgs q;  // d W_o = sum_i o_dot_i^T ubar_i + o_i^T ubar_dot_i
  q.A0 = o_dot; q.B0 = grad_u; q.A1 = o; q.B1 = grad_u_dot; q.lda = Da; q.ldb = Dn;
  q.P = N; q.Mo = Da; q.No = Dn; q.C = d_W_o;
  return launch_wgrad(q, w.split, stream);
}

// ------------------------------------ three-body update: training tangents ---
int mlip_tri_jvp(const int32_t *row_ptr, const int32_t *src, const float *geom, int32_t n_atoms,
                 int64_t n_edges, const float *grad_forces, const float *h_dot, const float *s,
                 const float *W_s, const float *W_ang, const float *W_T, int32_t n_ang, int32_t d_node,
                 int32_t d_tri, float cutoff, float *s_dot, float *tau_dot, float *hT_dot, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0 && n_edges >= 0 && n_edges < (int64_t(1) << 31),
                 "n_atoms/n_edges out of range");
  int cpl = 0;
  if (int rc = check_tri_dims(d_node, d_tri, n_ang, cutoff, &cpl)) return rc;
  MLIP_CHECK_ARG(row_ptr && W_s && W_ang && W_T, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (grad_forces && s && tau_dot && hT_dot), "null pointer argument");
  MLIP_CHECK_ARG(!h_dot || s_dot, "h_dot needs s_dot");
  MLIP_CHECK_ARG(n_edges == 0 || (src && geom), "null edge pointer");
  MLIP_CHECK_ARG(aligned(geom, 16) && aligned(h_dot, 16) && aligned(s, 16) && aligned(W_s, 16) &&
                     aligned(W_ang, 16) && aligned(W_T, 16) && aligned(s_dot, 16) && aligned(tau_dot, 16) &&
                     aligned(hT_dot, 16),
                 "float arrays must be 16-byte aligned");
  if (n_atoms == 0) return MLIP_OK;
  if (h_dot) {
    GemmArgs g;  // s_dot = h_dot W_s
    g.A = h_dot; g.lda = d_node; g.B = W_s; g.ldb = d_tri; g.C = s_dot; g.ldc = d_tri;
    g.M = n_atoms; g.N = d_tri; g.K = d_node;
    if (int rc = launch_gemm(g, false, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
  }
  if (int rc = launch_tri_jvp(row_ptr, src, geom, n_atoms, grad_forces, -1.f, s, h_dot ? s_dot : nullptr, W_ang,
                              d_tri, cutoff, tau_dot, stream))
    return rc;
  GemmArgs g2;  // hT_dot = h_dot + tau_dot W_T
  g2.A = tau_dot; g2.lda = d_tri; g2.B = W_T; g2.ldb = d_node; g2.C = hT_dot; g2.ldc = d_node;
  g2.R = h_dot; g2.ldr = d_node; g2.M = n_atoms; g2.N = d_node; g2.K = d_tri;
  return launch_gemm(g2, false, h_dot ? EPI_RESID : EPI_STORE, K_GEMM_DENSE, stream);
}

size_t mlip_tri_tangent_vjp_workspace_size(int32_t n_atoms, int64_t n_edges, int32_t d_node, int32_t d_tri) {
  size_t b = 0;
  carve_tri_tan(nullptr, std::max(n_atoms, 0), std::max<int64_t>(n_edges, 0), std::max(d_node, 0),
                std::max(d_tri, 0), &b);
  return b;
}

int mlip_tri_tangent_vjp(const int32_t *row_ptr, const int32_t *src, const int32_t *rev, const float *geom,
                         int32_t n_atoms, int64_t n_edges, const float *grad_forces, const float *h,
                         const float *h_dot, const float *s, const float *s_dot, const float *tau,
                         const float *tau_dot, const float *sbar, const float *W_s, const float *W_ang,
                         const float *W_T, int32_t n_ang, int32_t d_node, int32_t d_tri, float cutoff,
                         const float *grad_hT, const float *grad_hT_dot, float *grad_h_dot, float *d_W_s,
                         float *d_W_ang, float *d_W_T, void *ws, size_t ws_bytes, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0 && n_edges >= 0 && n_edges < (int64_t(1) << 31),
                 "n_atoms/n_edges out of range");
  int cpl = 0;
  if (int rc = check_tri_dims(d_node, d_tri, n_ang, cutoff, &cpl)) return rc;
  MLIP_CHECK_ARG(row_ptr && W_s && W_ang && W_T && d_W_s && d_W_ang && d_W_T, "null pointer argument");
  MLIP_CHECK_ARG(n_atoms == 0 || (grad_forces && h && s && tau && tau_dot && sbar && grad_hT && grad_hT_dot),
                 "null pointer argument");
  MLIP_CHECK_ARG(!h_dot || s_dot, "h_dot needs s_dot");
  MLIP_CHECK_ARG(n_edges == 0 || (src && rev && geom), "null edge pointer");
  MLIP_CHECK_ARG(aligned(geom, 16) && aligned(h, 16) && aligned(h_dot, 16) && aligned(s, 16) &&
                     aligned(s_dot, 16) && aligned(tau, 16) && aligned(tau_dot, 16) && aligned(sbar, 16) &&
                     aligned(W_s, 16) && aligned(W_ang, 16) && aligned(W_T, 16) && aligned(grad_hT, 16) &&
                     aligned(grad_hT_dot, 16) && aligned(grad_h_dot, 16) && aligned(d_W_s, 16) &&
                     aligned(d_W_ang, 16) && aligned(d_W_T, 16),
                 "float arrays must be 16-byte aligned");
  if (int rc = check_ws(ws, ws_bytes, mlip_tri_tangent_vjp_workspace_size(n_atoms, n_edges, d_node, d_tri)))
    return rc;
  TriTanWs w = carve_tri_tan(ws, n_atoms, n_edges, d_node, d_tri, nullptr);
  const int N = n_atoms, Dt = d_tri, Dn = d_node;
  if (N > 0) {
    GemmArgs g;  // taubar = grad_hT W_T^T, taubar_dot = grad_hT_dot W_T^T
    g.A = grad_hT; g.lda = Dn; g.B = W_T; g.ldb = Dn; g.C = w.taubar; g.ldc = Dt;
    g.M = N; g.N = Dt; g.K = Dn;
    g.k_split = dense_k_split(N, Dt, Dn); g.split_ws = w.split;
    if (int rc = launch_gemm(g, true, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
    g.A = grad_hT_dot; g.C = w.taubar_dot;
    if (int rc = launch_gemm(g, true, EPI_STORE, K_GEMM_DENSE, stream)) return rc;
    if (int rc = launch_tri_tvjp(row_ptr, src, rev, geom, N, grad_forces, -1.f, s, h_dot ? s_dot : nullptr,
                                 W_ang, w.taubar, w.taubar_dot, Dt, cutoff, w.sigma_dot, w.wang_part,
                                 w.sbar_dot, stream))
      return rc;
  }
  if (int rc = launch_row_sum(w.wang_part, N, MLIP_N_ANG * Dt, w.wang_part2, d_W_ang, stream)) return rc;
  if (grad_h_dot && N > 0) {
    GemmArgs g;  // grad_h_dot = grad_hT_dot + sbar_dot W_s^T
    g.A = w.sbar_dot; g.lda = Dt; g.B = W_s; g.ldb = Dt; g.C = grad_h_dot; g.ldc = Dn;
    g.R = grad_hT_dot; g.ldr = Dn; g.M = N; g.N = Dn; g.K = Dt;
    if (int rc = launch_gemm(g, true, EPI_RESID, K_GEMM_DENSE, stream)) return rc;
  }
  {
    WgradArgs q;  // d W_s = sum_i h_i^T sbar_dot_i + h_dot_i^T sbar_i
    q.A0 = h; q.B0 = w.sbar_dot;
    if (h_dot) { q.A1 = h_dot; q.B1 = sbar; }
    q.lda = Dn; q.ldb = Dt; q.P = N; q.Mo = Dn; q.No = Dt; q.C = d_W_s;
    if (int rc = launch_wgrad(q, w.split, stream)) return rc;
  }
  WgradArgs q;  // d W_T = sum_i tau_dot_i^T grad_hT_i + tau_i^T grad_hT_dot_i
  q.A0 = tau_dot; q.B0 = grad_hT; q.A1 = tau; q.B1 = grad_hT_dot; q.lda = Dt; q.ldb = Dn;
  q.P = N; q.Mo = Dt; q.No = Dn; q.C = d_W_T;
  return launch_wgrad(q, w.split, stream);
}

// ------------------------------------------------------ atom embedding ----
int mlip_embed_atoms(const int32_t *z, const float *table, int32_t n_atoms, int32_t n_types,
                     int32_t d_node, float *h, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0, "n_atoms must be >= 0");
  MLIP_CHECK_ARG(n_types >= 1 && n_types <= kMaxTypes, "n_types must be in [1, %d]", kMaxTypes);
  if (int rc = check_width(d_node, "d_node")) return rc;
  MLIP_CHECK_ARG(table && (n_atoms == 0 || (z && h)), "null pointer argument");
  MLIP_CHECK_ARG(aligned(table, 16) && aligned(h, 16), "float arrays must be 16-byte aligned");
  if (n_atoms == 0) return MLIP_OK;
  return embed_atoms(z, table, n_atoms, n_types, d_node, h, stream);
}

int mlip_embed_grad(const int32_t *z, const float *grad_h, int32_t n_atoms, int32_t n_types, int32_t d_node,
                    float *d_table, void *stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  MLIP_CHECK_ARG(n_atoms >= 0, "n_atoms must be >= 0");
  MLIP_CHECK_ARG(n_types >= 1 && n_types <= kMaxTypes, "n_types must be in [1, %d]", kMaxTypes);
  if (int rc = check_width(d_node, "d_node")) return rc;
  MLIP_CHECK_ARG(d_table && (n_atoms == 0 || (z && grad_h)), "null pointer argument");
  MLIP_CHECK_ARG(aligned(grad_h, 16) && aligned(d_table, 16), "float arrays must be 16-byte aligned");
  return embed_grad(z, grad_h, n_atoms, n_types, d_node, d_table, stream);
}

}  // extern "C"
