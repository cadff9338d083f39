"""The complete interaction block: message-update MoE, neighbour multi-head
attention, feature-update MoE (oracle; test infrastructure only).

The paper review ("Breaking the Training Barrier of Billion-Parameter
Universal MLIPs", section 3.4, Fig. 3) lists the operators of one interaction
block as Tri, MoE0, Attn and MoE1; section 3.2 puts sparse MoE layers before
and after the self-attention (one for message construction, one for the
refinement after attention) and replaces the original separable attention by
multi-head self-attention whose cost stays O(N) at a fixed cutoff; Table II
gives the heads and the attention width (S: 8 heads, 384; M and L: 4, 512).
The pages give no formula for any of it.  Readings taken here:

* MoE0 is the same element-routed top-k SiLU MoE as the feature-update MoE
  (see ``oracle.block``), with its own logit table and expert weights, on
  the incoming node features:  h0 = h + MoE0(h).
* Attention is self-attention restricted to each atom's neighbours inside
  r_c (the radius graph), which is what keeps it O(N).  With
  [q | k | v] = h0 @ W_qkv (width Da each, heads = contiguous channel blocks
  of width dh = Da / n_heads) and the pair embedding in attention width
  e_ij = f_c(r) (phi(r) @ Wa_e)  (the basis and envelope of ``oracle.block``):
      score   s_ij^t = sum_{c in head t} q_ic k_jc e_ijc / sqrt(dh)
      weight  alpha_ij^t = f_c(r_ij) exp(s_ij^t) / sum_l f_c(r_il) exp(s_il^t)
              (0 for an atom whose weights all vanish)
      output  o_ic = sum_j alpha_ij^{t(c)} v_jc e_ijc
      u = h0 + o @ W_o.
  The pair distance enters keys and values through e, as the edge features
  do in the aggregation of ``oracle.block``.  The envelope also weights the
  softmax terms: without it a neighbour crossing r_c would change the
  softmax denominator by a finite amount and the energy would jump, which
  the smooth energy surface the pages require rules out.
* MoE1 and the readout are those of ``oracle.block``:  h' = u + MoE1(u).
* Tri, the three-body update of ``oracle.tri``, runs first when the inputs
  carry its weights (``W_ang``): h_T = Tri(h) feeds MoE0.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from . import block as B
from . import tri as TR

f64 = np.float64


def heads_of(d_attn: int, n_heads: int) -> np.ndarray:
    """Head index of every attention channel (contiguous blocks of dh)."""
    if n_heads < 1 or d_attn % n_heads:
        raise ValueError("d_attn must be a multiple of n_heads")
    return np.repeat(np.arange(n_heads), d_attn // n_heads)


def head_sum(x: np.ndarray, n_heads: int) -> np.ndarray:
    """[E, Da] -> [E, n_heads]: sum of each head's channels."""
    E, Da = x.shape
    return x.reshape(E, n_heads, Da // n_heads).sum(axis=2)


def neighbour_softmax(s: np.ndarray, f: np.ndarray, recv: np.ndarray, n_atoms: int):
    """Envelope-weighted softmax over each receiver's edges, per head.

    alpha[e, t] = f[e] exp(s[e, t]) / sum over edges l of the same receiver of
    f[l] exp(s[l, t]), evaluated with the receiver's maximum score m
    subtracted.  Returns alpha [E, H], w = exp(s - m) [E, H], m and
    Z = sum f w [N, H] (alpha is 0 where Z is 0).
    """
    E, H = s.shape
    alpha = np.zeros((E, H), f64)
    w = np.zeros((E, H), f64)
    m = np.zeros((n_atoms, H), f64)
    Z = np.zeros((n_atoms, H), f64)
    starts = np.searchsorted(recv, np.arange(n_atoms + 1))
    for i in range(n_atoms):
        lo, hi = starts[i], starts[i + 1]
        if hi == lo:
            continue
        mi = s[lo:hi].max(axis=0)
        wi = np.exp(s[lo:hi] - mi)
        Zi = (f[lo:hi, None] * wi).sum(axis=0)
        w[lo:hi] = wi
        m[i] = mi
        Z[i] = Zi
        with np.errstate(invalid="ignore", divide="ignore"):
            alpha[lo:hi] = np.where(Zi > 0, f[lo:hi, None] * wi / Zi, 0.0)
    return alpha, w, m, Z


def attention_forward(h0: np.ndarray, graph: Dict[str, np.ndarray], W_qkv: np.ndarray,
                      Wa_e: np.ndarray, W_o: np.ndarray, n_heads: int, rc: float) -> Dict:
    """Neighbour multi-head attention of one block (module docstring)."""
    h0 = np.asarray(h0, f64)
    N = h0.shape[0]
    Da = W_o.shape[0]
    dh = Da // n_heads
    recv, src, r = graph["recv"], graph["src"], graph["r"]
    qkv = h0 @ np.asarray(W_qkv, f64)
    q, k, v = qkv[:, :Da], qkv[:, Da:2 * Da], qkv[:, 2 * Da:]
    e = B.edge_embedding(r, Wa_e, rc)
    f = B.envelope(r, rc)
    s = head_sum(q[recv] * k[src] * e, n_heads) / math.sqrt(dh)
    alpha, w, m, Z = neighbour_softmax(s, f, recv, N)
    ht = heads_of(Da, n_heads)
    o = np.zeros((N, Da), f64)
    np.add.at(o, recv, alpha[:, ht] * v[src] * e)
    u = h0 + o @ np.asarray(W_o, f64)
    return dict(h0=h0, q=q, k=k, v=v, e=e, f=f, s=s, alpha=alpha, w=w, m=m, Z=Z, o=o, u=u)


def attention_vjp(fw: Dict, graph: Dict[str, np.ndarray], W_qkv: np.ndarray, Wa_e: np.ndarray,
                  W_o: np.ndarray, n_heads: int, rc: float, ubar: np.ndarray) -> Dict:
    """dL/dh0 and dL/dr_e of the attention, given ubar = dL/du.

    Reverse of the forward, step by step:
      obar = ubar W_o^T;  abar_ij^t = sum_{c in t} obar_ic v_jc e_ijc;
      beta_i^t = sum_{c in t} obar_ic o_ic  (= sum_l alpha_il^t abar_il^t);
      gbar_ij^t = alpha_ij^t (abar_ij^t - beta_i^t)   (dL/d(s + log f));
      dL/df_ij = sum_t w_ij^t / Z_i^t (abar_ij^t - beta_i^t)   (gbar / f, finite at f = 0);
      qbar_i += gbar k_j e / sqrt(dh);  kbar_j += gbar q_i e / sqrt(dh);
      vbar_j += alpha obar_i e;  ebar_ij = gbar q_i k_j / sqrt(dh) + alpha obar_i v_j;
      dL/dr_ij = ebar . de/dr + dL/df_ij f_c'(r);
      dL/dh0 = ubar + [qbar | kbar | vbar] W_qkv^T.
    """
    recv, src, r = graph["recv"], graph["src"], graph["r"]
    N, Da = fw["o"].shape
    dh = Da // n_heads
    sq = 1.0 / math.sqrt(dh)
    ht = heads_of(Da, n_heads)
    ubar = np.asarray(ubar, f64)
    obar = ubar @ np.asarray(W_o, f64).T
    q, k, v, e, alpha, w, Z = fw["q"], fw["k"], fw["v"], fw["e"], fw["alpha"], fw["w"], fw["Z"]
    abar = head_sum(obar[recv] * v[src] * e, n_heads)
    beta = head_sum(obar * fw["o"], n_heads)                     # [N, H]
    diff = abar - beta[recv]
    gbar = alpha * diff
    with np.errstate(invalid="ignore", divide="ignore"):
        Zr = Z[recv]
        fbar = np.sum(np.where(Zr > 0, w / Zr, 0.0) * diff, axis=1)
    G = gbar[:, ht]
    A = alpha[:, ht]
    qbar = np.zeros((N, Da), f64)
    kbar = np.zeros((N, Da), f64)
    vbar = np.zeros((N, Da), f64)
    np.add.at(qbar, recv, G * k[src] * e * sq)
    np.add.at(kbar, src, G * q[recv] * e * sq)
    np.add.at(vbar, src, A * obar[recv] * e)
    ebar = G * q[recv] * k[src] * sq + A * obar[recv] * v[src]
    c = np.sum(ebar * B.edge_embedding_dr(r, Wa_e, rc), axis=1) + fbar * B.envelope_dr(r, rc)
    h0bar = ubar + np.concatenate([qbar, kbar, vbar], axis=1) @ np.asarray(W_qkv, f64).T
    return dict(obar=obar, gbar=gbar, fbar=fbar, qbar=qbar, kbar=kbar, vbar=vbar, c=c,
                grad_h0=h0bar)


# ------------------------------------------------------- complete block ----
def full_block_forward(inp: Dict[str, np.ndarray], graph: Dict[str, np.ndarray]) -> Dict:
    """h -> (Tri) -> MoE0 -> attention -> MoE1 -> readout, on a prebuilt radius graph."""
    rc = B._cutoff(inp)
    h_in = np.asarray(inp["h"], f64)
    k = int(inp["top_k"])
    nh = int(inp["n_heads"])
    tri = None
    if "W_ang" in inp:
        tri = TR.tri_forward(h_in, graph, inp["W_s"], inp["W_ang"], inp["W_T"], rc)
        h = tri["hT"]
    else:
        h = h_in
    topk0, gate0 = B.route(inp["logits0"], k)
    h0 = B.moe_forward(h, inp["z"], topk0, gate0, inp["W1_0"], inp["W2_0"])
    att = attention_forward(h0, graph, inp["W_qkv"], inp["Wa_e"], inp["W_o"], nh, rc)
    topk, gate = B.route(inp["logits"], k)
    h2 = B.moe_forward(att["u"], inp["z"], topk, gate, inp["W1"], inp["W2"])
    eps, E = B.readout(h2, inp["w_r"], inp["struct_ptr"])
    return dict(h=h, tri=tri, topk0=topk0, gate0=gate0, att=att, u=att["u"], topk=topk,
                gate=gate, h2=h2, eps=eps, E=E)


def full_block_vjp(inp: Dict[str, np.ndarray], graph: Dict[str, np.ndarray], fwd: Dict,
                   g: np.ndarray) -> Dict[str, np.ndarray]:
    """Input gradient of the complete block for g = dL/dh': dL/dh, dL/dx,
    dL/d(strain) per structure and the per-atom virial (as ``oracle.block``)."""
    rc = B._cutoff(inp)
    nh = int(inp["n_heads"])
    g = np.asarray(g, f64)
    ubar = B.moe_vjp(fwd["u"], g, inp["z"], fwd["topk"], fwd["gate"], inp["W1"], inp["W2"])
    ab = attention_vjp(fwd["att"], graph, inp["W_qkv"], inp["Wa_e"], inp["W_o"], nh, rc, ubar)
    hbar = B.moe_vjp(fwd["h"], ab["grad_h0"], inp["z"], fwd["topk0"], fwd["gate0"],
                     inp["W1_0"], inp["W2_0"])
    N = hbar.shape[0]
    r, d = graph["r"], graph["d"]
    with np.errstate(invalid="ignore", divide="ignore"):
        dhat = np.where(r[:, None] > 0, d / r[:, None], 0.0)
    gvec = ab["c"][:, None] * dhat
    tb = None
    hT_bar = hbar
    if fwd["tri"] is not None:
        tb = TR.tri_vjp(fwd["tri"], graph, inp["W_s"], inp["W_ang"], inp["W_T"], rc, hT_bar)
        hbar = tb["grad_h"]
        gvec = gvec + tb["gvec"]
    gpos, gstrain, av = B.edge_forces_vec(gvec, graph, N, inp["struct_ptr"])
    return dict(ubar=ubar, grad_h0=ab["grad_h0"], grad_hT=hT_bar, c=ab["c"], gvec=gvec,
                grad_h=hbar, grad_pos=gpos, grad_strain=gstrain, atom_virial=av, att=ab,
                tri=tb)


def full_energy(inp: Dict[str, np.ndarray], pos: Optional[np.ndarray] = None,
                cell: Optional[np.ndarray] = None, h: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-structure energies of the complete block after rebuilding the graph."""
    from .graph import radius_graph
    q = dict(inp)
    if pos is not None:
        q["pos"] = pos
    if cell is not None:
        q["cell"] = cell
    if h is not None:
        q["h"] = h
    gr = radius_graph(q["pos"], q["cell"], q["struct_ptr"], B._cutoff(q))
    return full_block_forward(q, gr)["E"]
