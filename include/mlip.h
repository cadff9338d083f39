/*
 * mlip.h - C ABI of the MI355X (gfx950) library for one MatRIS-MoE
 * interaction block: periodic radius graph, neighbour aggregation,
 * element-routed top-k mixture of experts, readout, and the input gradient
 * (VJP) that conservative forces and stresses need; plus the three-body
 * update, the neighbour multi-head attention and the stand-alone MoE
 * gradient that the complete block (Tri, MoE0, attention, MoE1) is built
 * from.
 *
 * Sources (cited by page title and section):
 *   [news]   ScienceAI news article on MatRIS-MoE and Janus, sections on the
 *            model architecture and on conservative training.
 *   [review] xllm-io review of "Breaking the Training Barrier of
 *            Billion-Parameter Universal Machine Learning Interatomic
 *            Potentials": 3.1 (architecture, Fig. 1, Table II),
 *            3.2 (sparse MoE design), 3.3 (forces and stresses),
 *            3.4 (Fig. 3, operators of one block), 3.5 (kernel notes).
 *
 * Conventions for every entry point
 *   - Array arguments are DEVICE pointers unless marked (host).  The caller
 *     owns every buffer; the library allocates no device memory.  Scratch
 *     memory is passed as (ws, ws_bytes); its size comes from the matching
 *     mlip_*_workspace_size() call and it must be 256-byte aligned.
 *   - stream is a hipStream_t passed as void* (NULL = default stream).  All
 *     work is enqueued asynchronously on it; only mlip_build_graph,
 *     mlip_graph_reverse and mlip_moe_status wait for the stream (once each,
 *     to read a count or a device-side check); mlip_build_graph_async is the
 *     graph build without that wait.
 *   - Floating point data are float32, row-major.  Weight matrices are
 *     stored "in x out": y = x @ W.
 *   - Feature widths (d_edge, d_node, d_hidden) must be multiples of 4 and
 *     n_rbf must be 16.
 *   - Return value: MLIP_OK or a negative MLIP_ERR_* code; then
 *     mlip_last_error() returns a message (thread-local).  Arguments are
 *     validated on the host before anything is enqueued, so an error return
 *     leaves the outputs untouched unless stated otherwise.
 *   - Calls on one stream are ordered; calls that share a workspace must
 *     not run concurrently on different streams.
 */
#ifndef MLIP_H
#define MLIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLIP_OK 0
#define MLIP_ERR_INVALID (-1)     /* bad argument (null pointer, bad size, ...) */
#define MLIP_ERR_CAPACITY (-2)    /* output buffer too small; required size reported */
#define MLIP_ERR_UNSUPPORTED (-3) /* valid input outside what the kernels handle */
#define MLIP_ERR_HIP (-4)         /* HIP runtime error */
#define MLIP_ERR_INPUT (-5)       /* input data rejected by a device-side check */

#define MLIP_N_RBF 16
#define MLIP_N_ANG 4   /* Legendre orders l = 0..3 of the three-body update */

const char *mlip_last_error(void);
int mlip_version(void);

/* ------------------------------------------------------------------------
 * Periodic radius graph ([review] 3.1, Fig. 1(a): the structure is turned
 * into a graph under periodic repetition of its cell).
 *
 * An edge i <- j with integer lattice shift S = (S0,S1,S2) exists when i and
 * j belong to the same structure, (j,S) != (i,0) and
 *     d  = (x_j - x_i) + ((S0*C[0] + S1*C[1]) + S2*C[2])      (float64)
 *     d2 = (d.x*d.x + d.y*d.y) + d.z*d.z  <  cutoff*cutoff    (float64)
 * evaluated in float64 from the float32 inputs in exactly this order with
 * no fused multiply-add, so the edge set is reproducible bit for bit.
 *
 * pos        [n_atoms,3]      Cartesian positions, wrapped into their cell:
 *                             fractional coordinates f = x C_b^-1 in [0, 1)
 *                             (for a diagonal cell exactly 0 <= x_a < C_b[a][a];
 *                             for any other cell up to 1e-6 outside, i.e. the
 *                             rounding of float32 positions).
 * cell       [n_structs,3,3]  rows are the lattice vectors: any basis with
 *                             det != 0 (triclinic included); a diagonal cell
 *                             needs positive diagonal entries.
 * struct_ptr [n_structs+1]    atoms of structure b are struct_ptr[b] ..
 *                             struct_ptr[b+1]-1 (non-decreasing, 0 .. n_atoms).
 * cutoff     r_c > 0 in the units of pos.
 * edge_capacity              length of src/rev (and /4 of shift, geom).
 *
 * Outputs (edges sorted by receiver i, then sender j, then S0, S1, S2):
 * row_ptr [n_atoms+1]  CSR offsets, row i = edges with receiver i.
 * src     [E]          sender j of each edge.
 * shift   [E,4] int8   (S0, S1, S2, 0).
 * rev     [E]          index of the reverse edge (j <- i, -S).
 * geom    [E,4] f32    (d.x, d.y, d.z, |d|) rounded to float32.
 * n_edges (host)       E.
 *
 * Errors: MLIP_ERR_CAPACITY when E > edge_capacity (then *n_edges = E, the
 * edge arrays are untouched and row_ptr describes an empty graph, all
 * zeros); MLIP_ERR_INPUT for a struct_ptr that does
 * not run 0 = p_0 <= p_1 <= ... <= p_B = n_atoms (then *n_edges = 0 and
 * nothing is indexed through it), positions outside their cell or a cell
 * with non-finite entries or det = 0 (host message says which), and for an
 * edge without its reverse edge (cannot happen: the predicate is exactly
 * symmetric; reported rather than passed on, with rev[e] = e for that edge);
 * MLIP_ERR_UNSUPPORTED when a row has more than 1024 edges or a cell is so
 * thin that more than 8 images per axis reach the cutoff (shifts then stay
 * within +-8, well inside int8).  All passes are queued before one
 * synchronisation: the calling thread polls the stream (yielding between
 * polls) until all work queued on it, earlier work included, has finished,
 * then reads E, the error flags and the largest degree; the passes that
 * write the edge arrays check on the device that the edges fit, so on any
 * error return the edge arrays are untouched.  The read goes through a
 * small pinned host buffer allocated on a thread's first call and kept for
 * the life of the process.
 * ------------------------------------------------------------------------ */
size_t mlip_graph_workspace_size(int32_t n_atoms, int32_t n_structs);
int mlip_build_graph(const float *pos, const float *cell, const int32_t *struct_ptr,
                     int32_t n_atoms, int32_t n_structs, float cutoff,
                     int64_t edge_capacity, int32_t *row_ptr, int32_t *src,
                     int8_t *shift, int32_t *rev, float *geom, int64_t *n_edges,
                     void *ws, size_t ws_bytes, void *stream);

/* The same build without any wait, for step loops that must not stall the
 * host (and can be captured in a HIP graph): every pass is queued on the
 * stream and the summary (E, error flags, largest degree, 0) is written to
 * the caller's device array summary [4] (16-byte aligned).  When the edges
 * do not fit edge_capacity, a row exceeds 1024 edges or struct_ptr is
 * rejected, the edge arrays are untouched and row_ptr becomes an empty graph
 * (all zeros), so later calls on this graph touch no unwritten edge slot;
 * their results are then meaningless until the caller, having copied the
 * summary to the host, passes it to mlip_graph_check, which returns what
 * mlip_build_graph would have returned (and E).  Later calls may take
 * n_edges = edge_capacity: every pass over the edges is bounded by row_ptr. */
int mlip_build_graph_async(const float *pos, const float *cell, const int32_t *struct_ptr,
                           int32_t n_atoms, int32_t n_structs, float cutoff,
                           int64_t edge_capacity, int32_t *row_ptr, int32_t *src,
                           int8_t *shift, int32_t *rev, float *geom, int32_t *summary,
                           void *ws, size_t ws_bytes, void *stream);
/* Reads a build summary copied to the host (summary_host [4]); *n_edges = E. */
int mlip_graph_check(const int32_t *summary_host, int64_t edge_capacity, int64_t *n_edges);

/* ------------------------------------------------------------------------
 * Reverse-edge index of a caller's receiver-sorted CSR graph ([review] 3.1,
 * Fig. 1(a): the periodic graph is symmetric, every edge i <- j with shift
 * S has the edge j <- i with shift -S).  mlip_build_graph fills rev itself;
 * this entry point serves graphs built elsewhere (or edited) before they go
 * to the attention and three-body passes, which read rev.
 *
 * row_ptr [n_atoms+1], src [n_edges], shift [n_edges,4] int8 as written by
 * mlip_build_graph: rows sorted by (sender, S0, S1, S2).
 * rev     [n_edges]  output: index of the reverse edge.
 * ws      mlip_graph_workspace_size(0, 1) bytes.
 *
 * Errors: MLIP_ERR_INPUT when a row range leaves [0, n_edges] or a sender
 * leaves [0, n_atoms) (those edges are skipped), or when some edge has no
 * reverse edge (its rev entry is then the edge itself, so the array stays a
 * valid index array).  Synchronises the stream once to read the check.
 * ------------------------------------------------------------------------ */
int mlip_graph_reverse(const int32_t *row_ptr, const int32_t *src, const int8_t *shift,
                       int32_t n_atoms, int64_t n_edges, int32_t *rev, void *ws, size_t ws_bytes,
                       void *stream);

/* ------------------------------------------------------------------------
 * Edge embedding + neighbour aggregation + projections ([news] pair
 * distances are embedded; [review] 3.5: gather neighbour features, modulate
 * them, reduce onto the receiver).
 *
 *   e_e = f_c(r_e) * (phi(r_e) @ W_e)              [E, d_edge]
 *        phi_k(r) = exp(-gamma (r - mu_k)^2), mu_k = k r_c/15,
 *        gamma = 15^2/(2 r_c^2), f_c(r) = (cos(pi r/r_c)+1)/2 for r < r_c,
 *        else 0 (r = geom[e].w)
 *   s   = h @ W_d                                  [N, d_edge]
 *   a_i = sum_{e in row i} e_e * s_src(e)          (elementwise)
 *   u   = h + a @ W_u                              [N, d_node]
 *
 * row_ptr/src/geom: graph from mlip_build_graph (n_edges = row_ptr[N]).
 * h [N,d_node], W_e [16,d_edge], W_d [d_node,d_edge], W_u [d_edge,d_node].
 * Outputs s (kept for the VJP), u and, if e is not NULL, the edge features
 * e [E, d_edge].  e is optional: mlip_block_vjp rebuilds it from the
 * geometry when it is not kept (16 multiply-adds per element against an
 * E x d_edge write and read: 312 MB each way at the S widths, 24 GB at the
 * 262144-atom share).  Workspace holds a [N, d_edge].
 * ------------------------------------------------------------------------ */
size_t mlip_aggregate_workspace_size(int32_t n_atoms, int32_t d_edge, int32_t d_node);
int mlip_aggregate(const int32_t *row_ptr, const int32_t *src, const float *geom,
                   int32_t n_atoms, int64_t n_edges, const float *h, const float *W_e,
                   const float *W_d, const float *W_u, int32_t n_rbf, int32_t d_edge,
                   int32_t d_node, float cutoff, float *e, float *s, float *u,
                   void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * mlip_aggregate without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * mlip_aggregate, minus (ws, ws_bytes): the scratch (the aggregated edge
 * messages a and the split-K parts of h @ W_d) lives in a device array of
 * the library, MLIP_AGGREGATE_STATIC_MAX_BYTES per GPU, held from the first
 * call on that GPU until the process ends.  The call allocates nothing and
 * never clears the array: every byte a call reads it has written itself.
 *
 * The array is one per GPU and shared by every call on it: calls that
 * overlap on one GPU (different streams or host threads) race on it.  Call
 * with the stream's device current.
 *
 * Errors: as mlip_aggregate, plus MLIP_ERR_UNSUPPORTED, before any device
 * call, when the scratch the call needs (mlip_aggregate_workspace_size(
 * n_atoms, d_edge, d_node)) exceeds MLIP_AGGREGATE_STATIC_MAX_BYTES.  The
 * S workload (4096 atoms, d_edge 384, d_node 2560) needs 18 MiB.
 * ------------------------------------------------------------------------ */
#define MLIP_AGGREGATE_STATIC_MAX_BYTES ((size_t)32 << 20)
int mlip_aggregate_static(const int32_t *row_ptr, const int32_t *src, const float *geom,
                          int32_t n_atoms, int64_t n_edges, const float *h, const float *W_e,
                          const float *W_d, const float *W_u, int32_t n_rbf, int32_t d_edge,
                          int32_t d_node, float cutoff, float *e, float *s, float *u,
                          void *stream);

/* ------------------------------------------------------------------------
 * Feature-update mixture of experts with static element-type routing
 * ([news], [review] 3.2: each element type activates its own top-k experts,
 * independently of the coordinates).
 *
 *   topk[t,:] = the k experts with the largest logits[t,:] (ties -> lower
 *               index), in decreasing order; gate[t,:] = softmax of those k
 *               logits.
 *   tokens (i, r) are grouped by (expert, element, atom):
 *     exp_off [X+1]  start of each expert's tokens,
 *     tok_atom[N*k]  atom of each token in that order,
 *     slot    [N,k]  position of token (i, r).
 *   P = u[tok_atom] @ W1[x]  per expert x         [N*k, d_hidden] (kept)
 *   h_out_i = u_i + sum_r gate[z_i,r] * (silu(P) @ W2[x])[slot(i,r)]
 *
 * u [N,d_node], z [N] element types in [0,n_types), logits [T,X],
 * W1 [X,d_node,d_hidden], W2 [X,d_hidden,d_node].  Outputs topk [T,k] i32,
 * gate [T,k], exp_off, tok_atom, slot, P (all kept for the VJP) and h_out.
 * Element types outside [0,n_types) are clamped on the device and reported
 * by mlip_moe_status().
 * ------------------------------------------------------------------------ */
size_t mlip_moe_workspace_size(int32_t n_atoms, int32_t n_types, int32_t n_experts,
                               int32_t top_k, int32_t d_node, int32_t d_hidden);
int mlip_moe_forward(const float *u, const int32_t *z, const float *logits,
                     const float *W1, const float *W2, int32_t n_atoms, int32_t n_types,
                     int32_t n_experts, int32_t top_k, int32_t d_node, int32_t d_hidden,
                     int32_t *topk, float *gate, int32_t *exp_off, int32_t *tok_atom,
                     int32_t *slot, float *P, float *h_out, void *ws, size_t ws_bytes,
                     void *stream);
/* Waits for the stream; *bad_types (host) = 1 if the last mlip_moe_forward
 * with this workspace saw an element type outside [0,n_types), else 0. */
int mlip_moe_status(const void *ws, int32_t *bad_types, void *stream);

/* ------------------------------------------------------------------------
 * Structured arguments of the step's hot-path calls (mlip_moe_forward_vjp,
 * mlip_aggregate_vjp): a radius graph and a MoE layer's kept state, as
 * mlip_build_graph(_async) and the MoE forward write them, bundled so that a
 * call takes one pointer each instead of five or six arrays.  The structs
 * hold device pointers and counts only; the caller owns every buffer they
 * point to and the struct itself (read during the call, not kept).
 * mlip_struct_size(0) / (1) return sizeof(mlip_graph) / sizeof(mlip_moe_state)
 * so that a binding can check its own layout.
 * ------------------------------------------------------------------------ */
typedef struct mlip_graph {
  const int32_t *row_ptr; /* [n_atoms+1] receiver-sorted CSR row offsets */
  const int32_t *src;     /* [n_edges] sender of each edge */
  const int8_t *shift;    /* [n_edges][4] periodic image (sx, sy, sz, 0); unused by the calls below */
  const int32_t *rev;     /* [n_edges] reverse edge; unused by the calls below */
  const float *geom;      /* [n_edges] float4 (dx, dy, dz, r), 16-byte aligned */
  int32_t n_atoms;
  int64_t n_edges;
} mlip_graph;

typedef struct mlip_moe_state {
  int32_t *topk;     /* [n_types, top_k] experts of each element type */
  float *gate;       /* [n_types, top_k] their gates */
  int32_t *exp_off;  /* [n_experts+1] token offsets of the experts (dispatch order) */
  int32_t *tok_atom; /* [n_atoms*top_k] atom of each token */
  int32_t *slot;     /* [n_atoms, top_k] token of each (atom, rank) */
  float *P;          /* [n_atoms*top_k, d_hidden] hidden pre-activations, dispatch order */
} mlip_moe_state;

size_t mlip_struct_size(int32_t which);

/* ------------------------------------------------------------------------
 * The MoE forward and its input gradient in one call, for an upstream
 * gradient known before the forward runs: forces of the energy ([news]
 * conservative training, [review] 3.3) have grad_out = dE/dh_out = w_r for
 * every atom when the readout follows, and any fixed upstream works.
 * Outputs and tables as mlip_moe_forward (the tables and P into the buffers
 * *state points to), plus grad_u = dL/du as
 * mlip_moe_vjp returns it (and, if q_out is not NULL, grad_out[tok] @ W2^T
 * per token, as mlip_moe_vjp's q_out).
 *
 * The forward's second expert GEMM (silu(P) @ W2) and the gradient's first
 * ((grad_out[tok] @ W2^T) * silu'(P)) need only P and grad_out, so they run
 * as one launch whose second GEMM fills the slots the first leaves idle at
 * its end.  Results equal mlip_moe_forward followed by mlip_moe_vjp bit for
 * bit.  Workspace: mlip_moe_forward_vjp_workspace_size(); mlip_moe_status()
 * reads its type check.
 * ------------------------------------------------------------------------ */
size_t mlip_moe_forward_vjp_workspace_size(int32_t n_atoms, int32_t n_types, int32_t n_experts,
                                           int32_t top_k, int32_t d_node, int32_t d_hidden);
int mlip_moe_forward_vjp(const float *u, const int32_t *z, const float *logits, const float *W1,
                         const float *W2, int32_t n_atoms, int32_t n_types, int32_t n_experts,
                         int32_t top_k, int32_t d_node, int32_t d_hidden, const float *grad_out,
                         const mlip_moe_state *state, float *h_out, float *grad_u, float *q_out,
                         void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Readout ([review] 3.1 Fig. 1(b) names a readout; the reading here is
 * linear): eps_i = h_out_i . w_r, energy_b = sum_{i in b} eps_i in float64.
 * eps [N] f32, energy [n_structs] f64.  struct_ptr as for mlip_build_graph;
 * its entries are clamped into [0, n_atoms] on the device, so a malformed
 * table gives wrong sums but no access outside eps.
 * ------------------------------------------------------------------------ */
int mlip_readout(const float *h_out, const float *w_r, const int32_t *struct_ptr,
                 int32_t n_atoms, int32_t n_structs, int32_t d_node, float *eps,
                 double *energy, void *stream);

/* ------------------------------------------------------------------------
 * Input gradient of the block ([news] conservative training; [review] 3.3:
 * forces and stresses are obtained by differentiating the energy).  Given
 * grad_out = dL/dh_out [N,d_node]:
 *   ubar = grad_out + sum_r gate * ((grad_out @ W2^T) * silu'(P)) @ W1^T
 *   abar = ubar @ W_u^T
 *   grad_h = ubar + sbar @ W_d^T,  sbar_j = sum_{e: src(e)=j} e_e * abar_recv(e)
 *   c_e = sum_c (abar_recv * s_src)_c * d e_e,c / d r_e
 *   grad_pos_i = dL/dx_i = -sum_{e in row i} (c_e + c_rev(e)) d_e/|d_e|
 *   dL/d(eps) = sum_e c_e (d_e/|d_e|) (x) d_e   for the homogeneous strain
 *               x -> (I + eps) x of positions and cell vectors
 *   atom_virial_i = half of the strain terms of the edges touching atom i
 * Routing depends only on the element types, so gates carry no gradient.
 * With grad_out rows all equal to w_r, grad_pos = dE/dx (forces are
 * -grad_pos) and grad_strain_b / V_b is the stress of structure b.
 *
 * Inputs are the graph, s and (optional, may be NULL: then rebuilt from
 * geom and W_e) e from mlip_aggregate, the kept MoE state from
 * mlip_moe_forward and the weights.  Outputs grad_h [N,d_node],
 * grad_pos [N,3]; optional (may be NULL) atom_virial [N,6] f32 and
 * grad_strain [n_structs,6] f64, both in the order xx, yy, zz, yz, xz, xy;
 * struct_ptr/n_structs are read only when grad_strain is requested.
 * For the training gradient (mlip_block_tangent_vjp) two intermediates can
 * be kept (may be NULL): ubar_out [N,d_node] = ubar above and
 * q_out [N*top_k, d_hidden] = grad_out[tok] @ W2_x^T in dispatch order
 * (before the silu' factor).
 * ------------------------------------------------------------------------ */
size_t mlip_vjp_workspace_size(int32_t n_atoms, int32_t top_k, int32_t d_edge,
                               int32_t d_node, int32_t d_hidden);
int mlip_block_vjp(const int32_t *row_ptr, const int32_t *src, const float *geom,
                   int32_t n_atoms, int64_t n_edges, const float *e, const float *s,
                   const int32_t *z, const float *gate, const int32_t *exp_off,
                   const int32_t *tok_atom, const int32_t *slot, const float *P,
                   const float *W_e, const float *W_d, const float *W_u, const float *W1,
                   const float *W2, int32_t n_rbf, int32_t d_edge, int32_t d_node,
                   int32_t d_hidden, int32_t n_types, int32_t n_experts, int32_t top_k,
                   float cutoff, const float *grad_out, float *grad_h, float *grad_pos,
                   const int32_t *struct_ptr, int32_t n_structs, float *atom_virial,
                   double *grad_strain, float *ubar_out, float *q_out, void *ws,
                   size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * The input gradient of mlip_aggregate alone (a13, a14), from grad_u = dL/du:
 *   abar = grad_u @ W_u^T,  sbar_j = sum_{e: src = j} e_e * abar_recv(e),
 *   grad_h = grad_u + sbar @ W_d^T,  and dL/dr_e -> grad_pos, atom_virial,
 *   grad_strain exactly as mlip_block_vjp computes them.
 * mlip_block_vjp = mlip_moe_vjp followed by this call; after
 * mlip_moe_forward_vjp it completes the block's gradient.  The graph is read
 * from *graph (row_ptr, src, geom, n_atoms, n_edges).  e may be NULL (the
 * edge features are then rebuilt from the geometry).  atom_virial and
 * grad_strain as in mlip_block_vjp.
 * ------------------------------------------------------------------------ */
size_t mlip_aggregate_vjp_workspace_size(int32_t n_atoms, int32_t d_edge, int32_t d_node);
int mlip_aggregate_vjp(const mlip_graph *graph, const float *e, const float *s, const float *W_e,
                       const float *W_d, const float *W_u, int32_t n_rbf, int32_t d_edge, int32_t d_node,
                       float cutoff, const float *grad_u, float *grad_h, float *grad_pos,
                       const int32_t *struct_ptr, int32_t n_structs, float *atom_virial,
                       double *grad_strain, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Training gradient of the block: parameter gradients of a loss on energies
 * and forces ([review] 3.3: the potential is fitted to energies and to the
 * forces obtained by differentiating the energy, so training differentiates
 * the force once more).  For L(E, F) with grad_energy = dL/dE [n_structs]
 * (f64) and grad_forces = dL/dF [N,3]:
 *   dL/dtheta = sum_b dL/dE_b dE_b/dtheta + sum_i dL/dF_i . dF_i/dtheta,
 * computed as the derivative of the reverse-mode gradient along the
 * position direction x_dot = -grad_forces (forward over reverse), with the
 * reverse pass seeded by grad_out = w_r (the force seed) and its tangent by
 * grad_out_dot = dL/dE_b(i) w_r (mlip_readout_vjp).  Sequence for one block:
 *   forward (mlip_aggregate, mlip_moe_forward, mlip_readout), then
 *   mlip_block_vjp with grad_out = w_r keeping ubar_out and q_out (F = -grad_pos),
 *   the caller's loss gives grad_energy and grad_forces, then
 *   mlip_block_jvp (forward tangents), mlip_readout_vjp (grad_out_dot),
 *   mlip_block_tangent_vjp (weight gradients, dL/dh) and
 *   mlip_readout_grad (dL/dw_r).
 * A stack passes h_dot upward (h_out_dot of the block below) in the JVPs
 * and grad_out_dot downward (grad_h_dot of the block above) in the tangent
 * VJPs, top block first.
 *
 * mlip_block_jvp: tangents of the forward along x_dot = -grad_forces [N,3]
 * and h_dot [N,d_node] (may be NULL: 0).  With r_dot_e = dhat_e .
 * (x_dot_src - x_dot_recv), e_dot = r_dot d e/d r:
 *   s_dot = h_dot W_d;  a_dot_i = sum_{e in row i} e_dot_e * s_src + e_e * s_dot_src
 *   u_dot = h_dot + a_dot W_u;  P_dot = u_dot[tok] W1_x (dispatch order)
 *   h_out_dot = u_dot + sum_r gate * (silu'(P) * P_dot) W2_x   (may be NULL)
 * and the primal aggregate a (may be NULL) of the same sweep.  s, z, gate,
 * exp_off, tok_atom, slot, P: the forward's.  Outputs a, s_dot (needed when
 * h_dot is given), a_dot, u_dot [N,d_node], P_dot [N*top_k, d_hidden].
 * Workspace: mlip_block_jvp_workspace_size().
 *
 * mlip_block_tangent_vjp: the derivative, along (x_dot, h_dot, grad_out_dot),
 * of the block's reverse-mode gradient for the upstream grad_out.  Inputs:
 * the graph, grad_forces and h_dot as in the JVP; h, s, u from the forward
 * (u = mlip_aggregate's output), s_dot, a, a_dot, u_dot, P_dot from the JVP;
 * the forward's z, topk, gate, exp_off, tok_atom, slot, P; grad_out, ubar
 * and Q (ubar_out, q_out of mlip_block_vjp); grad_out_dot [N,d_node] (may
 * be NULL: 0).  Outputs (dense row-major, written, not accumulated):
 *   d_W_e [n_rbf,d_edge], d_W_d [d_node,d_edge], d_W_u [d_edge,d_node],
 *   d_W1 [n_experts,d_node,d_hidden], d_W2 [n_experts,d_hidden,d_node]
 *   (experts without tokens get 0), d_gate [n_types,top_k] (may be NULL),
 *   d_logits [n_types,n_experts] (may be NULL; gates are the softmax of the
 *   chosen logits, the others get 0), grad_h_dot [N,d_node] = dL/dh of the
 *   block input (may be NULL).
 * Workspace: mlip_block_tangent_vjp_workspace_size().
 *
 * mlip_readout_vjp: grad_h_out_i = grad_energy[b(i)] w_r (grad_energy NULL:
 * 1, the force seed).  mlip_readout_grad: d_w_r = sum_i grad_energy[b(i)]
 * h_out_i + h_out_dot_i (either term may be NULL); workspace:
 * mlip_readout_grad_workspace_size().
 * Every reduction runs in a fixed order: results are reproducible.
 * ------------------------------------------------------------------------ */
size_t mlip_block_jvp_workspace_size(int32_t n_atoms, int32_t top_k, int32_t d_node,
                                     int32_t d_hidden);
int mlip_block_jvp(const int32_t *row_ptr, const int32_t *src, const float *geom, int32_t n_atoms,
                   int64_t n_edges, const float *grad_forces, const float *h_dot, const float *s,
                   const int32_t *z, const float *gate, const int32_t *exp_off,
                   const int32_t *tok_atom, const int32_t *slot, const float *P, const float *W_e,
                   const float *W_d, const float *W_u, const float *W1, const float *W2,
                   int32_t n_rbf, int32_t d_edge, int32_t d_node, int32_t d_hidden,
                   int32_t n_types, int32_t n_experts, int32_t top_k, float cutoff, float *a,
                   float *s_dot, float *a_dot, float *u_dot, float *P_dot, float *h_out_dot,
                   void *ws, size_t ws_bytes, void *stream);
size_t mlip_block_tangent_vjp_workspace_size(int32_t n_atoms, int32_t n_types, int32_t top_k,
                                             int32_t d_edge, int32_t d_node, int32_t d_hidden);
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
    void *ws, size_t ws_bytes, void *stream);
int mlip_readout_vjp(const float *w_r, const double *grad_energy, const int32_t *struct_ptr,
                     int32_t n_atoms, int32_t n_structs, int32_t d_node, float *grad_h_out,
                     void *stream);
size_t mlip_readout_grad_workspace_size(int32_t n_atoms, int32_t d_node);
int mlip_readout_grad(const float *h_out, const float *h_out_dot, const double *grad_energy,
                      const int32_t *struct_ptr, int32_t n_atoms, int32_t n_structs, int32_t d_node,
                      float *d_w_r, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Input gradient of one mixture-of-experts layer on its own ([news],
 * [review] 3.3: forces from differentiating the energy), for blocks that
 * stack several MoE layers (the complete block below has one before and one
 * after the attention).  With g = grad_out = dL/dh' for h' = u + MoE(u):
 *     grad_in = g + sum_r gate[z_i,r] ((g @ W2_x^T) * silu'(P)) @ W1_x^T
 * Gates carry no gradient (routing depends on z only).  z, gate, exp_off,
 * tok_atom, slot and P are those written by the mlip_moe_forward call of
 * this layer; W1, W2 as there.  grad_in [n_atoms, d_node] may not alias
 * grad_out.  Workspace: mlip_moe_vjp_workspace_size().  q_out (may be NULL)
 * keeps Q = grad_out[tok] @ W2_x^T [n_atoms*top_k, d_hidden] in dispatch
 * order for mlip_moe_tangent_vjp.
 * ------------------------------------------------------------------------ */
size_t mlip_moe_vjp_workspace_size(int32_t n_atoms, int32_t top_k, int32_t d_node,
                                   int32_t d_hidden);
int mlip_moe_vjp(const int32_t *z, const float *gate, const int32_t *exp_off,
                 const int32_t *tok_atom, const int32_t *slot, const float *P, const float *W1,
                 const float *W2, int32_t n_atoms, int32_t n_types, int32_t n_experts,
                 int32_t top_k, int32_t d_node, int32_t d_hidden, const float *grad_out,
                 float *grad_in, float *q_out, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Neighbour multi-head attention of the complete interaction block
 * ([review] 3.4 Fig. 3: a block is Tri, MoE0, Attn, MoE1; 3.2: MoE layers
 * before and after a multi-head self-attention whose cost stays O(N) at a
 * fixed cutoff; Table II: S = 8 heads, width 384; M, L = 4 heads, 512).
 * The pages give no formula; the reading implemented (heads are contiguous
 * channel blocks of width dh = d_attn / n_heads, t(c) the head of channel c):
 *     [q | k | v] = h0 @ W_qkv                         (each d_attn wide)
 *     e_ij   = f_c(r) (phi(r) @ Wa_e)                   (basis as in mlip_aggregate)
 *     s_ij^t = sum_{c in head t} q_ic k_jc e_ijc / sqrt(dh)
 *     a_ij^t = f_c(r_ij) exp(s_ij^t) / sum_{l in row i} f_c(r_il) exp(s_il^t)
 *              (0 when that sum is 0: rows without neighbours)
 *     o_ic   = sum_{j in row i} a_ij^{t(c)} v_jc e_ijc
 *     u      = h0 + o @ W_o
 * The envelope weights the softmax so that a pair crossing r_c changes the
 * energy continuously.  The caller's graph is a mlip_build_graph result.
 *
 * h0     [n_atoms, d_node]      input node features (after MoE0).
 * W_qkv  [d_node, 3*d_attn]     columns q | k | v.
 * Wa_e   [n_rbf, d_attn]        pair embedding in attention width.
 * W_o    [d_attn, d_node].
 * n_heads: d_attn = n_heads * dh; a layout must exist with dh = c * 2^j,
 *        c in {1,2,3,4,6,8} and n_heads * 2^j <= 64 (else MLIP_ERR_UNSUPPORTED):
 *        e.g. 8 x 48, 4 x 128, 4 x 8, 2 x 32.
 * Outputs: qkv [n_atoms, 3*d_attn], o [n_atoms, d_attn] and
 *        stats [n_atoms, n_heads, 2] (running max of the scores, sum of the
 *        weights exp(s - max) f_c) are kept for mlip_attention_vjp;
 *        u [n_atoms, d_node] (may not alias h0).
 * ws: optional workspace of mlip_attention_workspace_size(n_atoms, d_attn)
 *        bytes (256-byte aligned; null, or a size of 0 bytes, is allowed).  With
 *        it, the q|k|v projection splits its K = d_node loop when the output
 *        has too few tiles to fill the GPU and sums the parts in a fixed order;
 *        without it the projection runs unsplit.  The results are the same up
 *        to rounding order.
 * ------------------------------------------------------------------------ */
int mlip_attention(const int32_t *row_ptr, const int32_t *src, const float *geom, int32_t n_atoms,
                   int64_t n_edges, const float *h0, const float *W_qkv, const float *Wa_e,
                   const float *W_o, int32_t n_rbf, int32_t d_node, int32_t d_attn,
                   int32_t n_heads, float cutoff, float *qkv, float *o, float *stats, float *u,
                   void *ws, size_t ws_bytes, void *stream);
size_t mlip_attention_workspace_size(int32_t n_atoms, int32_t d_attn);

/* Input gradient of mlip_attention for grad_u = dL/du [n_atoms, d_node]:
 *   grad_h0 [n_atoms, d_node]  = dL/dh0 (through the residual, q, k and v);
 *   grad_pos [n_atoms, 3]      = dL/dx through the pair distances (forces are
 *                               -grad_pos when L is the energy);
 *   atom_virial [n_atoms, 6]   (optional) per-atom virial, Voigt order
 *                               xx yy zz yz xz xy, as in mlip_block_vjp;
 *   grad_strain [n_structs, 6] (optional, float64) dL/d(strain) per structure.
 * rev is the reverse-edge index of the graph; qkv, o, stats come from the
 * mlip_attention call of the same step.  accumulate != 0 adds to grad_pos and
 * atom_virial instead of writing them (grad_strain, if given, is then
 * recomputed from the accumulated atom_virial, which must be given unless
 * n_atoms is 0), so the
 * forces of several blocks on one graph can be collected.  Per-edge
 * intermediates live in the workspace (mlip_attention_vjp_workspace_size,
 * which grows with n_edges).  Rows are reduced by one wavefront each; no
 * atomics, so the result does not depend on scheduling. */
size_t mlip_attention_vjp_workspace_size(int32_t n_atoms, int64_t n_edges, int32_t d_attn,
                                         int32_t n_heads);
int mlip_attention_vjp(const int32_t *row_ptr, const int32_t *src, const int32_t *rev,
                       const float *geom, int32_t n_atoms, int64_t n_edges, const float *qkv,
                       const float *o, const float *stats, const float *W_qkv, const float *Wa_e,
                       const float *W_o, int32_t n_rbf, int32_t d_node, int32_t d_attn,
                       int32_t n_heads, float cutoff, const float *grad_u, float *grad_h0,
                       float *grad_pos, const int32_t *struct_ptr, int32_t n_structs,
                       float *atom_virial, double *grad_strain, int32_t accumulate,
                       float *qkv_bar_out, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Training tangents of the complete block's layers ([review] 3.3: training
 * differentiates the force once more; see the training gradient of the
 * core block below for the scheme).  x_dot = -grad_forces throughout.
 *
 * mlip_moe_jvp: for h' = u + MoE(u) (state of its mlip_moe_forward),
 *   P_dot = u_dot[tok] W1_x (dispatch order), h_out_dot = u_dot + sum_r gate
 *   * (silu'(P) * P_dot) W2_x (may be NULL).  Workspace:
 *   mlip_moe_jvp_workspace_size().
 * mlip_moe_tangent_vjp: the derivative along (u_dot, grad_out_dot) of the
 *   layer's gradient for the upstream grad_out (Q = q_out of its
 *   mlip_moe_vjp): grad_in_dot = grad_out_dot + sum_r gate * D_dot W1_x^T
 *   (may be NULL), d_W1 [X,d_node,d_hidden], d_W2 [X,d_hidden,d_node],
 *   d_gate [T,k] and d_logits [T,X] (both may be NULL).  grad_out_dot may be
 *   NULL (0).  Workspace: mlip_moe_tangent_vjp_workspace_size().
 * mlip_attention_jvp: [q|k|v]_dot = h0_dot W_qkv, o_dot (with the pair
 *   embedding and envelope moving with r_dot) and u_dot = h0_dot + o_dot W_o;
 *   also tstat [N,n_heads] = sum_j a s_dot + f_dot w / Z, which the tangent
 *   VJP reads.  qkv, o, stats: the forward's.  No workspace.
 * mlip_attention_tangent_vjp: the derivative along (x_dot, h0_dot,
 *   grad_u_dot) of the attention's gradient for the upstream grad_u (qkv_bar
 *   = qkv_bar_out of its mlip_attention_vjp): grad_h0_dot [N,d_node] (may be
 *   NULL), d_W_qkv [d_node,3 d_attn], d_Wa_e [n_rbf,d_attn], d_W_o
 *   [d_attn,d_node].  Workspace: mlip_attention_tangent_vjp_workspace_size().
 * ------------------------------------------------------------------------ */
size_t mlip_moe_jvp_workspace_size(int32_t n_atoms, int32_t top_k, int32_t d_node, int32_t d_hidden);
int mlip_moe_jvp(const int32_t *z, const float *gate, const int32_t *exp_off, const int32_t *tok_atom,
                 const int32_t *slot, const float *P, const float *W1, const float *W2, int32_t n_atoms,
                 int32_t n_types, int32_t n_experts, int32_t top_k, int32_t d_node, int32_t d_hidden,
                 const float *u_dot, float *P_dot, float *h_out_dot, void *ws, size_t ws_bytes,
                 void *stream);
size_t mlip_moe_tangent_vjp_workspace_size(int32_t n_atoms, int32_t n_types, int32_t top_k,
                                           int32_t d_node, int32_t d_hidden);
int mlip_moe_tangent_vjp(const int32_t *z, const int32_t *topk, const float *gate,
                         const int32_t *exp_off, const int32_t *tok_atom, const int32_t *slot,
                         const float *P, const float *P_dot, const float *W1, const float *W2,
                         int32_t n_atoms, int32_t n_types, int32_t n_experts, int32_t top_k,
                         int32_t d_node, int32_t d_hidden, const float *u, const float *u_dot,
                         const float *grad_out, const float *Q, const float *grad_out_dot,
                         float *grad_in_dot, float *d_W1, float *d_W2, float *d_gate, float *d_logits,
                         void *ws, size_t ws_bytes, void *stream);
int mlip_attention_jvp(const int32_t *row_ptr, const int32_t *src, const float *geom, int32_t n_atoms,
                       int64_t n_edges, const float *grad_forces, const float *h0_dot, const float *qkv,
                       const float *o, const float *stats, const float *W_qkv, const float *Wa_e,
                       const float *W_o, int32_t n_rbf, int32_t d_node, int32_t d_attn, int32_t n_heads,
                       float cutoff, float *qkv_dot, float *o_dot, float *tstat, float *u_dot,
                       void *stream);
size_t mlip_attention_tangent_vjp_workspace_size(int32_t n_atoms, int64_t n_edges, int32_t d_node,
                                                 int32_t d_attn, int32_t n_heads);
int mlip_attention_tangent_vjp(
    const int32_t *row_ptr, const int32_t *src, const int32_t *rev, const float *geom, int32_t n_atoms,
    int64_t n_edges, const float *grad_forces, const float *h0, const float *h0_dot, const float *qkv,
    const float *qkv_dot, const float *o, const float *o_dot, const float *stats, const float *tstat,
    const float *qkv_bar, const float *W_qkv, const float *Wa_e, const float *W_o, int32_t n_rbf,
    int32_t d_node, int32_t d_attn, int32_t n_heads, float cutoff, const float *grad_u,
    const float *grad_u_dot, float *grad_h0_dot, float *d_W_qkv, float *d_Wa_e, float *d_W_o, void *ws,
    size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Three-body angular update ("Tri") of the complete block ([news]
 * architecture section: three-body angles are embedded; [review] 3.4 Fig. 3:
 * Tri is the first operator of every block).  The pages give no formula; the
 * reading implemented, for receiver i with edges e (unit vectors dhat_e,
 * envelopes f_e = f_c(r_e) as in mlip_aggregate, senders j(e)):
 *     s      = h @ W_s                                    [n_atoms, d_tri]
 *     tau_ic = sum over ordered pairs e != e' of row i of
 *              f_e f_e' (sum_l P_l(dhat_e . dhat_e') W_ang[l,c]) s_j(e),c s_j(e'),c
 *     h_T    = h + tau @ W_T
 * with P_l the Legendre polynomials, l = 0 .. n_ang-1 (n_ang must be
 * MLIP_N_ANG).  The pair sum is evaluated exactly through the addition
 * theorem of the Legendre polynomials (16 real spherical harmonics per edge),
 * so the cost is O(edges), not O(edges x degree).  Edges of zero length are
 * outside the contract.
 *
 * W_s [d_node, d_tri], W_ang [n_ang, d_tri], W_T [d_tri, d_node];
 * d_tri <= 512 (one wavefront per row).  Outputs s (kept for mlip_tri_vjp),
 * tau [n_atoms, d_tri] and h_T [n_atoms, d_node] (may not alias h).
 * ws: optional workspace of mlip_tri_workspace_size(n_atoms, d_tri) bytes
 * (256-byte aligned; null is allowed): with it the s projection splits its
 * K = d_node loop when the output has too few tiles to fill the GPU, the
 * parts summed in a fixed order; without it the projection runs unsplit.
 * ------------------------------------------------------------------------ */
int mlip_tri(const int32_t *row_ptr, const int32_t *src, const float *geom, int32_t n_atoms,
             int64_t n_edges, const float *h, const float *W_s, const float *W_ang, const float *W_T,
             int32_t n_ang, int32_t d_node, int32_t d_tri, float cutoff, float *s, float *tau,
             float *h_T, void *ws, size_t ws_bytes, void *stream);
size_t mlip_tri_workspace_size(int32_t n_atoms, int32_t d_tri);

/* Input gradient of mlip_tri for grad_hT = dL/dh_T:
 *   grad_h [n_atoms, d_node] = dL/dh;
 *   grad_pos [n_atoms, 3], atom_virial [n_atoms, 6] (optional, Voigt order,
 *     each edge's symmetrised dL/dd_e (x) d_e shared half and half by its two
 *     atoms), grad_strain [n_structs, 6] (optional, float64, the per-structure
 *     sum of atom_virial) as in mlip_block_vjp;
 *   accumulate != 0: grad_pos and atom_virial are ADDED to (so the forces of
 *     a whole block can be collected, e.g. after mlip_attention_vjp), and
 *     grad_strain, if given, is recomputed from the accumulated atom_virial
 *     (which must then be given unless n_atoms is 0).
 * rev is the reverse-edge index; s comes from the mlip_tri call of the step.
 * Per-edge intermediates (d_tri floats per edge) live in the workspace
 * (mlip_tri_vjp_workspace_size).  No atomics. */
size_t mlip_tri_vjp_workspace_size(int32_t n_atoms, int64_t n_edges, int32_t d_tri);
int mlip_tri_vjp(const int32_t *row_ptr, const int32_t *src, const int32_t *rev, const float *geom,
                 int32_t n_atoms, int64_t n_edges, const float *s, const float *W_s,
                 const float *W_ang, const float *W_T, int32_t n_ang, int32_t d_node,
                 int32_t d_tri, float cutoff, const float *grad_hT, float *grad_h,
                 float *grad_pos, const int32_t *struct_ptr, int32_t n_structs,
                 float *atom_virial, double *grad_strain, int32_t accumulate, float *sbar_out, void *ws,
                 size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Training tangents of the three-body update ([review] 3.3; the scheme of
 * the core block's training gradient), x_dot = -grad_forces.  sbar_out of
 * mlip_tri_vjp (may be NULL) keeps sbar = dL/ds [N,d_tri] for them.
 *
 * mlip_tri_jvp: s_dot = h_dot W_s (when h_dot, may be NULL: 0),
 *   tau_dot [N,d_tri] (with r_dot, dhat_dot and the harmonics' directional
 *   derivatives), hT_dot = h_dot + tau_dot W_T.  s: mlip_tri's.
 * mlip_tri_tangent_vjp: the derivative along (x_dot, h_dot, grad_hT_dot) of
 *   the update's gradient for the upstream grad_hT: grad_h_dot (may be
 *   NULL), d_W_s [d_node,d_tri], d_W_ang [n_ang,d_tri], d_W_T [d_tri,d_node].
 *   Inputs h, s, tau (forward), s_dot, tau_dot (JVP), sbar (sbar_out).
 *   Workspace: mlip_tri_tangent_vjp_workspace_size().
 * ------------------------------------------------------------------------ */
int mlip_tri_jvp(const int32_t *row_ptr, const int32_t *src, const float *geom, int32_t n_atoms,
                 int64_t n_edges, const float *grad_forces, const float *h_dot, const float *s,
                 const float *W_s, const float *W_ang, const float *W_T, int32_t n_ang, int32_t d_node,
                 int32_t d_tri, float cutoff, float *s_dot, float *tau_dot, float *hT_dot, void *stream);
size_t mlip_tri_tangent_vjp_workspace_size(int32_t n_atoms, int64_t n_edges, int32_t d_node, int32_t d_tri);
int mlip_tri_tangent_vjp(const int32_t *row_ptr, const int32_t *src, const int32_t *rev, const float *geom,
                         int32_t n_atoms, int64_t n_edges, const float *grad_forces, const float *h,
                         const float *h_dot, const float *s, const float *s_dot, const float *tau,
                         const float *tau_dot, const float *sbar, const float *W_s, const float *W_ang,
                         const float *W_T, int32_t n_ang, int32_t d_node, int32_t d_tri, float cutoff,
                         const float *grad_hT, const float *grad_hT_dot, float *grad_h_dot, float *d_W_s,
                         float *d_W_ang, float *d_W_T, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Element embedding of the input node features ([news] architecture
 * section: atoms are embedded; [review] 3.1 Fig. 1(b): feature embedding
 * before the interaction blocks): h[i] = table[z[i]] for table
 * [n_types, d_node].  Rows of atoms whose type is outside [0, n_types) are
 * set to zero (the MoE routing of the same step reports such types through
 * mlip_moe_status).
 * ------------------------------------------------------------------------ */
int mlip_embed_atoms(const int32_t *z, const float *table, int32_t n_atoms, int32_t n_types,
                     int32_t d_node, float *h, void *stream);

/* Gradient of the element embedding h_i = table[z_i] for grad_h = dL/dh
 * [n_atoms, d_node]: d_table[t] = sum over atoms with z_i = t of grad_h_i
 * ([n_types, d_node], written; types without atoms get 0).  For a stack's
 * training gradient grad_h is the first block's dL/dh.  Atoms are summed in
 * index order (reproducible); out-of-range types are skipped. */
int mlip_embed_grad(const int32_t *z, const float *grad_h, int32_t n_atoms, int32_t n_types, int32_t d_node,
                    float *d_table, void *stream);

/* ------------------------------------------------------------------------
 * Kernel timing.  When enabled, every kernel launch of the library is
 * bracketed by HIP events on its stream; mlip_profile_get() waits for the
 * recorded events and returns, for the kernel class with index idx, its name
 * (static string), the number of launches and their summed duration in
 * milliseconds.  Classes are numbered 0 .. mlip_profile_count()-1.  The
 * timing state is process-wide and guarded by a lock, so several host
 * threads may call the library while profiling is on; their launches then
 * add to the same per-class totals.  Event pairs are created on first use
 * and reused for the life of the process; meant for benchmarks.
 * mlip_profile_select(class_mask) restricts the timing to the classes whose
 * bit (1 << idx) is set in class_mask (all classes until it is called): each
 * timed launch costs two event records on its stream, so a benchmark can time
 * only the kernels it needs.  Launches of other classes are not counted.
 * ------------------------------------------------------------------------ */
int mlip_profile_enable(int enable);
int mlip_profile_select(uint64_t class_mask);
int mlip_profile_reset(void);
int mlip_profile_count(void);
int mlip_profile_get(int idx, const char **name, int64_t *launches, double *total_ms);

#ifdef __cplusplus
}
#endif
#endif /* MLIP_H */
