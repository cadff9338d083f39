"""Three-body angular update ("Tri") of the complete interaction block
(oracle; test infrastructure only).

The ScienceAI article (architecture section) says the model embeds atoms,
pair distances and three-body angles; the paper review (section 3.4, Fig. 3)
lists Tri as the first operator of every interaction block, before MoE0,
attention and MoE1, and section 3.1 (Fig. 1(d)) names a graph refinement
module.  No formula is given.  Reading taken here: a node update from the
angles between pairs of edges that share a receiver,

    s      = h @ W_s                                     (width Dt)
    tau_ic = sum over ordered pairs (e, e') of distinct edges of row i of
             f_c(r_e) f_c(r_e') * (sum_l P_l(cos theta_ee') W_ang[l, c])
             * s_{src(e), c} * s_{src(e'), c}
    h_T    = h + tau @ W_T

with cos theta_ee' = dhat_e . dhat_e' (the angle at atom i between its two
neighbours, periodic images counted as separate neighbours), P_l the
Legendre polynomials l = 0 .. L-1, and f_c the cosine envelope of
``oracle.block`` (so that a neighbour crossing r_c enters continuously).
The update keeps the O(N deg^2) triplet structure the pages' timeline
implies; it depends on positions only through distances and angles, so the
energy stays invariant under rotations and translations.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from . import block as B

f64 = np.float64


def legendre(x: np.ndarray, L: int) -> np.ndarray:
    """P_0 .. P_{L-1} at x by Bonnet's recurrence (l+1) P_{l+1} = (2l+1) x P_l - l P_{l-1}."""
    x = np.asarray(x, f64)
    P = np.zeros((L,) + x.shape, f64)
    P[0] = 1.0
    if L > 1:
        P[1] = x
    for l in range(1, L - 1):
        P[l + 1] = ((2 * l + 1) * x * P[l] - l * P[l - 1]) / (l + 1)
    return P


def legendre_dx(x: np.ndarray, L: int) -> np.ndarray:
    """dP_l/dx by the recurrence P'_{l+1} = P'_{l-1} + (2l+1) P_l."""
    P = legendre(x, L)
    D = np.zeros_like(P)
    if L > 1:
        D[1] = 1.0
    for l in range(1, L - 1):
        D[l + 1] = D[l - 1] + (2 * l + 1) * P[l]
    return D


def _unit(graph):
    r, d = graph["r"], graph["d"]
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(r[:, None] > 0, d / r[:, None], 0.0)


def tri_row(U: np.ndarray, f: np.ndarray, S: np.ndarray, W_ang: np.ndarray) -> np.ndarray:
    """tau of one receiver from its edges' unit vectors U [deg,3], envelopes f [deg]
    and sender features S [deg, Dt] (sum over ordered pairs of distinct edges)."""
    L = W_ang.shape[0]
    if U.shape[0] < 2:
        return np.zeros(W_ang.shape[1], f64)
    X = U @ U.T                                            # cosines, [deg, deg]
    G = np.einsum("lab,lc->abc", legendre(X, L), W_ang)   # [deg, deg, Dt]
    F = np.outer(f, f)
    np.fill_diagonal(F, 0.0)                              # distinct edges only
    # sum_ab F_ab G_abc S_ac S_bc, the pair weights folded into G first
    return np.einsum("abc,ac,bc->c", F[:, :, None] * G, S, S)


def tri_row_vjp(U: np.ndarray, r: np.ndarray, f: np.ndarray, df: np.ndarray, S: np.ndarray,
                W_ang: np.ndarray, tb: np.ndarray):
    """Gradient of one receiver's tau for taubar = tb [Dt].

    With K_ab,c = f_a f_b G_ab,c (a != b, symmetric in a, b):
      dL/dS_a,c   = 2 sum_b K_ab,c tb_c S_b,c               (to the sender of edge a)
      dL/df_a     = 2 sum_b f_b sum_c tb_c G_ab,c S_a,c S_b,c
      dL/dx_ab    = f_a f_b sum_c tb_c S_a,c S_b,c sum_l P_l'(x_ab) W_ang[l, c]
      dL/ddhat_a  = 2 sum_b dL/dx_ab dhat_b
      dL/dd_a     = dL/df_a f_c'(r_a) dhat_a + (I - dhat_a dhat_a^T) dL/ddhat_a / r_a.
    Returns (dL/dS [deg, Dt], dL/dd [deg, 3]).
    """
    L = W_ang.shape[0]
    deg = U.shape[0]
    if deg < 2:
        return np.zeros_like(S), np.zeros((deg, 3), f64)
    X = U @ U.T
    G = np.einsum("lab,lc->abc", legendre(X, L), W_ang)
    Gd = np.einsum("lab,lc->abc", legendre_dx(X, L), W_ang)
    off = 1.0 - np.eye(deg)
    F = np.outer(f, f) * off
    St = S * tb                                            # tb_c S_b,c
    sbar = 2.0 * np.einsum("abc,bc->ac", F[:, :, None] * G, St)
    # T_ab = sum_c tb_c G_ab,c S_a,c S_b,c
    T = np.einsum("abc,ac,bc->ab", G, St, S)
    fbar = 2.0 * ((off * T) @ f)
    xbar = F * np.einsum("abc,ac,bc->ab", Gd, St, S)
    ubar = 2.0 * xbar @ U
    with np.errstate(invalid="ignore", divide="ignore"):
        inv_r = np.where(r > 0, 1.0 / r, 0.0)
    radial = np.sum(ubar * U, axis=1)
    gvec = (fbar * df)[:, None] * U + (ubar - radial[:, None] * U) * inv_r[:, None]
    return sbar, gvec


def tri_forward(h: np.ndarray, graph: Dict[str, np.ndarray], W_s: np.ndarray,
                W_ang: np.ndarray, W_T: np.ndarray, rc: float) -> Dict[str, np.ndarray]:
    """h_T = h + tau @ W_T with the pair sum of the module docstring."""
    h = np.asarray(h, f64)
    N = h.shape[0]
    W_ang = np.asarray(W_ang, f64)
    s = h @ np.asarray(W_s, f64)
    recv, src = graph["recv"], graph["src"]
    U = _unit(graph)
    f = B.envelope(graph["r"], rc)
    starts = np.searchsorted(recv, np.arange(N + 1))
    tau = np.zeros((N, W_ang.shape[1]), f64)
    for i in range(N):
        lo, hi = starts[i], starts[i + 1]
        tau[i] = tri_row(U[lo:hi], f[lo:hi], s[src[lo:hi]], W_ang)
    hT = h + tau @ np.asarray(W_T, f64)
    return dict(s=s, tau=tau, hT=hT)


def tri_vjp(fw: Dict[str, np.ndarray], graph: Dict[str, np.ndarray], W_s: np.ndarray,
            W_ang: np.ndarray, W_T: np.ndarray, rc: float, hT_bar: np.ndarray) -> Dict:
    """dL/dh and the per-edge vector gradient dL/dd_e of Tri, for hT_bar = dL/dh_T:
    taubar = hT_bar W_T^T, then ``tri_row_vjp`` per receiver, sender gradients
    scattered to their atoms, and dL/dh = hT_bar + sbar W_s^T."""
    W_ang = np.asarray(W_ang, f64)
    hT_bar = np.asarray(hT_bar, f64)
    N = hT_bar.shape[0]
    tb = hT_bar @ np.asarray(W_T, f64).T
    s = fw["s"]
    recv, src, r = graph["recv"], graph["src"], graph["r"]
    U = _unit(graph)
    f = B.envelope(r, rc)
    df = B.envelope_dr(r, rc)
    sbar = np.zeros_like(s)
    gvec = np.zeros((r.size, 3), f64)
    starts = np.searchsorted(recv, np.arange(N + 1))
    for i in range(N):
        lo, hi = starts[i], starts[i + 1]
        sb, gv = tri_row_vjp(U[lo:hi], r[lo:hi], f[lo:hi], df[lo:hi], s[src[lo:hi]], W_ang, tb[i])
        np.add.at(sbar, src[lo:hi], sb)
        gvec[lo:hi] = gv
    hbar = hT_bar + sbar @ np.asarray(W_s, f64).T
    return dict(taubar=tb, sbar=sbar, gvec=gvec, grad_h=hbar)
