"""One MatRIS-MoE interaction block, forward and input-gradient, in float64
(oracle; test infrastructure only).

What the pages fix, and the readings taken where they are silent:

* Edge embedding ([news] architecture section: pair distances are embedded).
  The basis is not given.  Reading: K Gaussians on a uniform grid,
  mu_k = k r_c/(K-1), gamma = (K-1)^2/(2 r_c^2), phi_k(r) = exp(-gamma (r-mu_k)^2),
  times a cosine envelope f_c(r) = (cos(pi r/r_c) + 1)/2 for r < r_c, else 0,
  then a linear map:  e = f_c(r) * (phi(r) @ W_e).  The envelope is there
  because the pages require a continuous, smooth energy surface ([news],
  [review] 3.2); without it the energy jumps when a pair crosses r_c.
* Neighbour aggregation ([review] 3.5: gather neighbour features, modulate,
  reduce onto the receiving atom).  Reading: s = h @ W_d,
  a_i = sum over edges e of row i of e_e * s_src(e) (elementwise, no degree
  normalisation), u = h + a @ W_u.
* Feature-update MoE ([news], [review] 3.2: experts chosen per element type,
  top-K, independent of coordinates).  Reading: for each element type t the
  experts are ordered by (-logit[t, x], x) and the first k are taken;
  gates are the softmax of the chosen logits.  Each expert is a bias-free
  SiLU MLP (y = silu(u @ W1_x) @ W2_x) and h' = u + sum_r gate_r * y_r.
  Nothing is dropped: every atom reaches its k experts.
* Readout ([review] 3.1 Fig. 1(b) names a readout without a form).  Reading:
  eps_i = h'_i . w_r and E_b = sum of eps over the atoms of structure b.
* Forces are minus the gradient of the energy ([news] conservative training,
  [review] 3.3).  Routing depends only on z, so gates carry no gradient.
"""
from __future__ import annotations

import contextlib
from typing import Dict, Optional

import numpy as np

# Working precision of every array this module creates.  float64 is the
# reference; ``working_precision(np.float32)`` re-runs the same steps in
# float32, which is how the tests check that the float32 arithmetic the pages
# prescribe can meet the comparison tolerance at all.
f64 = np.float64


@contextlib.contextmanager
def working_precision(dtype):
    """Evaluate this module's functions with arrays of ``dtype`` inside the block."""
    global f64
    saved = f64
    f64 = dtype
    try:
        yield
    finally:
        f64 = saved


# ----------------------------------------------------------------- basis ----
def rbf_params(K: int, rc: float):
    mu = np.arange(K, dtype=f64) * rc / (K - 1)
    gamma = (K - 1) ** 2 / (2.0 * rc * rc)
    return mu, gamma


def rbf(r: np.ndarray, K: int, rc: float) -> np.ndarray:
    """phi_k(r) = exp(-gamma (r - mu_k)^2), shape [..., K]."""
    mu, gamma = rbf_params(K, rc)
    x = np.asarray(r, f64)[..., None] - mu
    return np.exp(-gamma * x * x)


def rbf_dr(r: np.ndarray, K: int, rc: float) -> np.ndarray:
    """d phi_k / d r = -2 gamma (r - mu_k) phi_k."""
    mu, gamma = rbf_params(K, rc)
    x = np.asarray(r, f64)[..., None] - mu
    return -2.0 * gamma * x * np.exp(-gamma * x * x)


def envelope(r: np.ndarray, rc: float) -> np.ndarray:
    r = np.asarray(r, f64)
    return np.where(r < rc, 0.5 * (np.cos(np.pi * r / rc) + 1.0), 0.0)


def envelope_dr(r: np.ndarray, rc: float) -> np.ndarray:
    r = np.asarray(r, f64)
    return np.where(r < rc, -0.5 * np.pi / rc * np.sin(np.pi * r / rc), 0.0)


def silu(p: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return p / (1.0 + np.exp(-p))


def silu_dp(p: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-p))
    return sig * (1.0 + p * (1.0 - sig))


# ------------------------------------------------------------- edge part ----
def edge_embedding(r: np.ndarray, W_e: np.ndarray, rc: float) -> np.ndarray:
    """e = f_c(r) * (phi(r) @ W_e), [E, De]."""
    K = W_e.shape[0]
    return envelope(r, rc)[:, None] * (rbf(r, K, rc) @ np.asarray(W_e, f64))


def edge_embedding_dr(r: np.ndarray, W_e: np.ndarray, rc: float) -> np.ndarray:
    """d e / d r = f_c'(r) (phi @ W_e) + f_c(r) (phi' @ W_e), [E, De]."""
    K = W_e.shape[0]
    W = np.asarray(W_e, f64)
    return (envelope_dr(r, rc)[:, None] * (rbf(r, K, rc) @ W)
            + envelope(r, rc)[:, None] * (rbf_dr(r, K, rc) @ W))


def aggregate(e: np.ndarray, s: np.ndarray, recv: np.ndarray, src: np.ndarray,
              n_atoms: int) -> np.ndarray:
    """a_i = sum over edges with receiver i of e_e * s_src(e) (plain scatter-add)."""
    a = np.zeros((n_atoms, e.shape[1]), f64)
    np.add.at(a, recv, e * s[src])
    return a


# ----------------------------------------------------------------- MoE ------
def route(logits: np.ndarray, k: int):
    """Static per-element routing: top-k experts of each element type.

    Experts are taken in order of decreasing logit; equal logits go to the
    lower expert index.  Gates are the softmax over the k chosen logits
    (max-subtracted), in rank order.  Returns topk [T,k] int64, gate [T,k] f64.
    """
    L = np.asarray(logits, f64)
    T, X = L.shape
    topk = np.zeros((T, k), np.int64)
    gate = np.zeros((T, k), f64)
    for t in range(T):
        taken = []
        for _ in range(k):
            best = -1
            for x in range(X):
                if x in taken:
                    continue
                if best < 0 or L[t, x] > L[t, best]:
                    best = x
            taken.append(best)
        topk[t] = taken
        chosen = L[t, taken]
        w = np.exp(chosen - chosen.max())
        gate[t] = w / w.sum()
    return topk, gate


def dispatch_tables(z: np.ndarray, topk: np.ndarray, n_experts: int):
    """Expert-grouped token order (only used to compare the GPU's tables).

    Tokens are the pairs (atom i, rank r); they are ordered by
    (expert topk[z_i, r], element z_i, atom i).  Returns exp_off [X+1],
    tok_atom [N*k] (atom of each token in that order) and slot [N, k]
    (position of token (i, r) in that order).
    """
    z = np.asarray(z, np.int64)
    N, k = z.size, topk.shape[1]
    atoms = np.repeat(np.arange(N), k)
    ranks = np.tile(np.arange(k), N)
    experts = topk[z[atoms], ranks]
    order = np.lexsort((atoms, z[atoms], experts))
    counts = np.bincount(experts, minlength=n_experts)
    exp_off = np.zeros(n_experts + 1, np.int64)
    exp_off[1:] = np.cumsum(counts)
    slot = np.zeros((N, k), np.int64)
    slot[atoms[order], ranks[order]] = np.arange(N * k)
    return exp_off, atoms[order], slot


def _expert_members(z, topk, x):
    sel = topk[z] == x                 # [N, k]; at most one True per row (ids distinct)
    return np.nonzero(sel)


def moe_forward(u: np.ndarray, z: np.ndarray, topk: np.ndarray, gate: np.ndarray,
                W1: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """h' = u + sum_r gate[z_i, r] * silu(u_i @ W1_x) @ W2_x, x = topk[z_i, r]."""
    z = np.asarray(z, np.int64)
    out = np.array(u, f64, copy=True)
    for x in range(W1.shape[0]):
        atoms, ranks = _expert_members(z, topk, x)
        if atoms.size == 0:
            continue
        p = u[atoms] @ np.asarray(W1[x], f64)
        y = silu(p) @ np.asarray(W2[x], f64)
        out[atoms] += gate[z[atoms], ranks][:, None] * y
    return out


def moe_preactivations(u: np.ndarray, z: np.ndarray, topk: np.ndarray, W1: np.ndarray) -> np.ndarray:
    """First-layer outputs of the chosen experts before SiLU, [N, k, H]:
    p[i, r] = u_i @ W1_x with x = topk[z_i, r] (the hidden state of token (i, r))."""
    z = np.asarray(z, np.int64)
    N, k = z.size, topk.shape[1]
    p = np.zeros((N, k, W1.shape[2]), f64)
    for x in range(W1.shape[0]):
        atoms, ranks = _expert_members(z, topk, x)
        if atoms.size:
            p[atoms, ranks] = np.asarray(u, f64)[atoms] @ np.asarray(W1[x], f64)
    return p


def moe_vjp(u: np.ndarray, g: np.ndarray, z: np.ndarray, topk: np.ndarray,
            gate: np.ndarray, W1: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """dL/du given g = dL/dh'.

    dL/du_i = g_i + sum_r gate * ((g_i @ W2_x^T) * silu'(u_i @ W1_x)) @ W1_x^T.
    """
    z = np.asarray(z, np.int64)
    ubar = np.array(g, f64, copy=True)
    for x in range(W1.shape[0]):
        atoms, ranks = _expert_members(z, topk, x)
        if atoms.size == 0:
            continue
        W1x = np.asarray(W1[x], f64)
        W2x = np.asarray(W2[x], f64)
        p = u[atoms] @ W1x
        q = (g[atoms] @ W2x.T) * silu_dp(p)
        ubar[atoms] += gate[z[atoms], ranks][:, None] * (q @ W1x.T)
    return ubar


def readout(h2: np.ndarray, w_r: np.ndarray, struct_ptr: np.ndarray):
    """eps_i = h'_i . w_r; E_b = sum of eps over structure b."""
    eps = h2 @ np.asarray(w_r, f64)
    sp = np.asarray(struct_ptr, np.int64)
    E = np.array([eps[sp[b]:sp[b + 1]].sum() for b in range(len(sp) - 1)], f64)
    return eps, E


# --------------------------------------------------------------- block ------
def _cutoff(inp) -> float:
    return float(np.float64(np.float32(inp["cutoff"])))


def block_forward(inp: Dict[str, np.ndarray], graph: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """Forward pass of one block on a prebuilt radius graph."""
    rc = _cutoff(inp)
    h = np.asarray(inp["h"], f64)
    N = h.shape[0]
    recv, src, r = graph["recv"], graph["src"], graph["r"]
    e = edge_embedding(r, inp["W_e"], rc)
    s = h @ np.asarray(inp["W_d"], f64)
    a = aggregate(e, s, recv, src, N)
    u = h + a @ np.asarray(inp["W_u"], f64)
    k = int(inp["top_k"]) if "top_k" in inp else None
    if k is None:
        raise KeyError("inputs need 'top_k'")
    topk, gate = route(inp["logits"], k)
    h2 = moe_forward(u, inp["z"], topk, gate, inp["W1"], inp["W2"])
    eps, E = readout(h2, inp["w_r"], inp["struct_ptr"])
    return dict(e=e, s=s, a=a, u=u, topk=topk, gate=gate, h2=h2, eps=eps, E=E)


def block_vjp(inp: Dict[str, np.ndarray], graph: Dict[str, np.ndarray],
              fwd: Dict[str, np.ndarray], g: np.ndarray) -> Dict[str, np.ndarray]:
    """Input gradient of one block: given g = dL/dh', return dL/dh, dL/dx and
    dL/d(strain).

    With g_i = w_r for every atom, dL/dx is dE/dx and the forces are -dL/dx;
    dL/d(strain) per structure divided by the cell volume is the stress
    ([review] 3.3: forces and stresses both come from differentiating the
    energy).  The strain is the homogeneous deformation x -> (I + eps) x of
    positions and cell vectors.  The chain rule is applied step by step in
    reverse; edge sums are plain scatters over both endpoints of every edge.
    """
    rc = _cutoff(inp)
    N = fwd["u"].shape[0]
    recv, src, r = graph["recv"], graph["src"], graph["r"]
    g = np.asarray(g, f64)
    ubar = moe_vjp(fwd["u"], g, inp["z"], fwd["topk"], fwd["gate"], inp["W1"], inp["W2"])
    abar = ubar @ np.asarray(inp["W_u"], f64).T
    # a_i = sum_e e_e * s_src  ->  dL/ds_j = sum over edges with sender j of e_e * abar_recv
    sbar = np.zeros_like(fwd["s"])
    np.add.at(sbar, src, fwd["e"] * abar[recv])
    hbar = ubar + sbar @ np.asarray(inp["W_d"], f64).T
    # dL/dr_e = sum_c (abar_recv * s_src)_c * (d e_e / d r)_c
    ebar = abar[recv] * fwd["s"][src]
    c = np.sum(ebar * edge_embedding_dr(r, inp["W_e"], rc), axis=1)
    gpos, gstrain, av = edge_forces(c, graph, N, inp["struct_ptr"])
    return dict(ubar=ubar, abar=abar, sbar=sbar, grad_h=hbar, c=c, grad_pos=gpos,
                grad_strain=gstrain, atom_virial=av)


def edge_forces(c: np.ndarray, graph: Dict[str, np.ndarray], n_atoms: int,
                struct_ptr: np.ndarray):
    """Position gradient, strain gradient and per-atom virial from c_e = dL/dr_e.

    r = |d|, d = x_src - x_recv + S.C, so dL/dd_e = c_e dhat_e (see ``edge_forces_vec``).
    """
    r, d = graph["r"], graph["d"]
    with np.errstate(invalid="ignore", divide="ignore"):
        dhat = np.where(r[:, None] > 0, d / r[:, None], 0.0)
    return edge_forces_vec(c[:, None] * dhat, graph, n_atoms, struct_ptr)


def edge_forces_vec(gvec: np.ndarray, graph: Dict[str, np.ndarray], n_atoms: int,
                    struct_ptr: np.ndarray):
    """Position gradient, strain gradient and per-atom virial from g_e = dL/dd_e.

    d_e = x_src - x_recv + S.C, so dL/dx_src += g_e and dL/dx_recv -= g_e.
    Under the homogeneous strain x -> (I + eps) x of positions and cell,
    d_e -> (I + eps) d_e and dL/deps_ab = sum_e g_e,a d_e,b.  Each atom of an
    edge gets half of the symmetric part of that edge's term in its virial
    (Voigt order).
    """
    recv, src, d = graph["recv"], graph["src"], graph["d"]
    gpos = np.zeros((n_atoms, 3), f64)
    np.add.at(gpos, src, gvec)
    np.add.at(gpos, recv, -gvec)
    outer = gvec[:, :, None] * d[:, None, :]                            # [E, 3, 3]
    sp = np.asarray(struct_ptr, np.int64)
    nb = len(sp) - 1
    sb_of_edge = np.searchsorted(sp, recv, side="right") - 1
    gstrain = np.zeros((nb, 3, 3), f64)
    np.add.at(gstrain, sb_of_edge, outer)
    sym = 0.5 * (outer + outer.transpose(0, 2, 1))
    av = np.zeros((n_atoms, 3, 3), f64)
    np.add.at(av, recv, 0.5 * sym)
    np.add.at(av, src, 0.5 * sym)
    return gpos, gstrain, voigt(av)


def voigt(t: np.ndarray) -> np.ndarray:
    """[..., 3, 3] -> [..., 6] in the order xx, yy, zz, yz, xz, xy."""
    return np.stack([t[..., 0, 0], t[..., 1, 1], t[..., 2, 2],
                     t[..., 1, 2], t[..., 0, 2], t[..., 0, 1]], axis=-1)


def energy(inp: Dict[str, np.ndarray], pos: Optional[np.ndarray] = None,
           cell: Optional[np.ndarray] = None, h: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-structure energies after rebuilding the graph (positions may be float64)."""
    from .graph import radius_graph
    q = dict(inp)
    if pos is not None:
        q["pos"] = pos
    if cell is not None:
        q["cell"] = cell
    if h is not None:
        q["h"] = h
    gr = radius_graph(q["pos"], q["cell"], q["struct_ptr"], _cutoff(q))
    return block_forward(q, gr)["E"]
