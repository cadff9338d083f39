"""Parameter gradients of an energy + force loss through one interaction
block (oracle; test infrastructure only).

[review] 3.3: the forces are the negative gradient of the energy, and the
potential is trained on energies and forces together, so the training
gradient differentiates the force once more ("double backward").  The pages
name no loss form.  Reading taken: the loss is any scalar L(E, F) of the
per-structure energies and the forces; what the block has to deliver is

    dL/dtheta = sum_b Ebar_b dE_b/dtheta + sum_i Fbar_i . dF_i/dtheta,

with Ebar = dL/dE and Fbar = dL/dF supplied by the caller (for a squared
error, Ebar = 2 w_E (E - E_ref), Fbar = 2 w_F (F - F_ref)).  theta covers
every parameter of the block (W_e, W_d, W_u, W1, W2, the routing logits, the
readout w_r) and the input node features h.

This module writes the block's energy as plain float64 PyTorch CPU
operations on the same radius graph as ``oracle.block`` and takes both
derivatives with torch.autograd: first F = -dE/dx with the graph of that
derivative kept, then the gradient of L.  The block's steps are restated
here from their definitions (``oracle.block`` holds the readings); the two
implementations are checked against each other in the tests, and the
second derivatives against central finite differences of L built from
``oracle.block``'s energies and forces.
"""
from __future__ import annotations

from typing import Dict

import numpy as np
import torch

from . import block as B

f64 = torch.float64
PARAMS = ("W_e", "W_d", "W_u", "W1", "W2", "logits", "w_r", "h")


def _t(x):
    return torch.as_tensor(np.asarray(x, np.float64), dtype=f64)


def _vectors(inp: Dict, graph: Dict, pos: torch.Tensor) -> torch.Tensor:
    """d_e = x_src - x_recv + S . C (cell of the receiver's structure)."""
    recv = torch.as_tensor(graph["recv"], dtype=torch.long)
    src = torch.as_tensor(graph["src"], dtype=torch.long)
    sp = np.asarray(inp["struct_ptr"], np.int64)
    sb = np.searchsorted(sp, np.asarray(graph["recv"]), side="right") - 1
    cell = _t(inp["cell"])[torch.as_tensor(sb, dtype=torch.long)]            # [E, 3, 3]
    return pos[src] - pos[recv] + torch.einsum("ea,eab->eb", _t(graph["shift"]), cell)


def _distances(inp: Dict, graph: Dict, pos: torch.Tensor) -> torch.Tensor:
    """r_e = |x_src - x_recv + S . C| (cell of the receiver's structure)."""
    recv = torch.as_tensor(graph["recv"], dtype=torch.long)
    src = torch.as_tensor(graph["src"], dtype=torch.long)
    sp = np.asarray(inp["struct_ptr"], np.int64)
    sb = np.searchsorted(sp, np.asarray(graph["recv"]), side="right") - 1
    cell = _t(inp["cell"])[torch.as_tensor(sb, dtype=torch.long)]            # [E, 3, 3]
    S = _t(graph["shift"])
    d = pos[src] - pos[recv] + torch.einsum("ea,eab->eb", S, cell)
    return torch.sqrt((d * d).sum(1))


def _block(inp: Dict, graph: Dict, r: torch.Tensor, prm: Dict, h: torch.Tensor) -> torch.Tensor:
    """h' of one block (aggregation + MoE) for node features h."""
    rc = B._cutoff(inp)
    K = prm["W_e"].shape[0]
    recv = torch.as_tensor(graph["recv"], dtype=torch.long)
    src = torch.as_tensor(graph["src"], dtype=torch.long)
    N = h.shape[0]
    # e = f_c(r) (phi(r) @ W_e)
    mu = torch.arange(K, dtype=f64) * rc / (K - 1)
    gamma = (K - 1) ** 2 / (2.0 * rc * rc)
    phi = torch.exp(-gamma * (r[:, None] - mu) ** 2)
    fc = torch.where(r < rc, 0.5 * (torch.cos(np.pi * r / rc) + 1.0), torch.zeros_like(r))
    e = fc[:, None] * (phi @ prm["W_e"])
    # aggregation and up projection
    s = h @ prm["W_d"]
    a = torch.zeros(N, e.shape[1], dtype=f64).index_add(0, recv, e * s[src])
    u = h + a @ prm["W_u"]
    # static element routing: the chosen experts depend on the logits' order
    # only, the gates are the softmax of the chosen logits
    k = int(inp["top_k"])
    topk, _ = B.route(prm["logits"].detach().numpy(), k)
    z = torch.as_tensor(np.asarray(inp["z"], np.int64))
    T = prm["logits"].shape[0]
    chosen = prm["logits"][torch.arange(T)[:, None], torch.as_tensor(topk)]
    gate = torch.softmax(chosen, dim=1)                                       # [T, k]
    h2 = u
    for r_ in range(k):
        x_of_atom = torch.as_tensor(topk)[z, r_]
        g_of_atom = gate[z, r_]
        for x in range(len(prm["W1"])):
            idx = torch.nonzero(x_of_atom == x).flatten()
            if idx.numel() == 0:
                continue
            y = torch.nn.functional.silu(u[idx] @ prm["W1"][x]) @ prm["W2"][x]
            h2 = h2.index_add(0, idx, g_of_atom[idx, None] * y)
    return h2


def _readout(inp: Dict, h2: torch.Tensor, w_r: torch.Tensor) -> torch.Tensor:
    """E_b = sum over structure b of h'_i . w_r."""
    sp = np.asarray(inp["struct_ptr"], np.int64)
    N = h2.shape[0]
    eps = h2 @ w_r
    sbat = torch.as_tensor(np.searchsorted(sp, np.arange(N), side="right") - 1, dtype=torch.long)
    return torch.zeros(len(sp) - 1, dtype=f64).index_add(0, sbat, eps)


def _energy(inp: Dict, graph: Dict, prm: Dict[str, torch.Tensor], pos: torch.Tensor) -> torch.Tensor:
    """E_b of one block as a differentiable function of positions and parameters."""
    r = _distances(inp, graph, pos)
    return _readout(inp, _block(inp, graph, r, prm, prm["h"]), prm["w_r"])


def loss_grads(inp: Dict, graph: Dict, Ebar: np.ndarray, Fbar: np.ndarray,
               experts=None) -> Dict[str, np.ndarray]:
    """E, F and dL/dtheta for L with dL/dE = Ebar [B], dL/dF = Fbar [N, 3].

    With ``experts`` (a list of expert indices) the W1 / W2 gradients are
    taken for those experts only, returned in that order as d_W1 [len, Dn, H]
    and d_W2 [len, H, Dn] (for very wide layers)."""
    names = [n for n in PARAMS if experts is None or n not in ("W1", "W2")]
    prm = {name: _t(inp[name]).requires_grad_(True) for name in names}
    wrt = [prm[n] for n in names]
    if experts is not None:
        for n in ("W1", "W2"):
            full = _t(inp[n])
            leaves = {int(x): full[int(x)].clone().requires_grad_(True) for x in experts}
            prm[n] = [leaves[x] if x in leaves else full[x] for x in range(full.shape[0])]
            wrt += [leaves[int(x)] for x in experts]
    pos = _t(inp["pos"]).requires_grad_(True)
    E = _energy(inp, graph, prm, pos)
    (dEdx,) = torch.autograd.grad(E.sum(), pos, create_graph=True)
    F = -dEdx
    L = (E * _t(Ebar)).sum() + (F * _t(Fbar)).sum()
    grads = torch.autograd.grad(L, wrt, allow_unused=True)
    out = {"E": E.detach().numpy(), "F": F.detach().numpy()}
    for n, g, t in zip(names, grads, wrt):
        out["d_" + n] = np.zeros(t.shape) if g is None else g.detach().numpy()
    if experts is not None:
        rest = list(zip(grads[len(names):], wrt[len(names):]))
        m = len(experts)
        for q, n in enumerate(("W1", "W2")):
            out["d_" + n] = np.stack([np.zeros(t.shape) if g is None else g.detach().numpy()
                                      for g, t in rest[q * m:(q + 1) * m]])
    return out


def loss_value(inp: Dict, Ebar: np.ndarray, Fbar: np.ndarray, **override) -> float:
    """L = Ebar . E + Fbar . F with E and F from ``oracle.block`` (no autograd);
    keyword arguments replace inputs (for finite differences)."""
    from .graph import radius_graph
    q = dict(inp)
    q.update(override)
    g = radius_graph(q["pos"], q["cell"], q["struct_ptr"], B._cutoff(q))
    f = B.block_forward(q, g)
    N = f["u"].shape[0]
    gup = np.broadcast_to(np.asarray(q["w_r"], np.float64), (N, f["u"].shape[1]))
    v = B.block_vjp(q, g, f, gup)
    return float(np.dot(f["E"], Ebar) + np.sum(-v["grad_pos"] * Fbar))


BLOCK_PARAMS = ("W_e", "W_d", "W_u", "W1", "W2", "logits")


def stack_loss_grads(inp: Dict, graph: Dict, blocks, Ebar: np.ndarray, Fbar: np.ndarray) -> Dict:
    """The same loss through blocks chained on one graph, h^(b+1) = Block_b(h^(b)),
    h^(0) = inp["h"], readout on the last.  Returns E, F, d_h, d_w_r and
    ``blocks``: one dict of d_<param> per block."""
    h0 = _t(inp["h"]).requires_grad_(True)
    w_r = _t(inp["w_r"]).requires_grad_(True)
    prms = [{n: _t(b[n]).requires_grad_(True) for n in BLOCK_PARAMS} for b in blocks]
    pos = _t(inp["pos"]).requires_grad_(True)
    r = _distances(inp, graph, pos)
    h = h0
    for prm in prms:
        h = _block(inp, graph, r, prm, h)
    E = _readout(inp, h, w_r)
    (dEdx,) = torch.autograd.grad(E.sum(), pos, create_graph=True)
    F = -dEdx
    L = (E * _t(Ebar)).sum() + (F * _t(Fbar)).sum()
    wrt = [h0, w_r] + [prm[n] for prm in prms for n in BLOCK_PARAMS]
    grads = torch.autograd.grad(L, wrt, allow_unused=True)
    np_ = lambda g, t: np.zeros(t.shape) if g is None else g.detach().numpy()
    out = {"E": E.detach().numpy(), "F": F.detach().numpy(), "d_h": np_(grads[0], h0),
           "d_w_r": np_(grads[1], w_r), "blocks": []}
    q = 2
    for prm in prms:
        out["blocks"].append({"d_" + n: np_(grads[q + j], prm[n]) for j, n in enumerate(BLOCK_PARAMS)})
        q += len(BLOCK_PARAMS)
    return out


def stack_loss_value(inp: Dict, blocks, Ebar: np.ndarray, Fbar: np.ndarray, h=None, w_r=None) -> float:
    """L of chained blocks with E and F from ``oracle.block`` (no autograd):
    forwards in order, input gradients in reverse, forces summed over blocks."""
    from .graph import radius_graph
    q = dict(inp)
    if h is not None:
        q["h"] = h
    if w_r is not None:
        q["w_r"] = w_r
    g = radius_graph(q["pos"], q["cell"], q["struct_ptr"], B._cutoff(q))
    hcur = np.asarray(q["h"], np.float64)
    ins, fwds = [], []
    for b in blocks:
        qb = dict(q)
        qb.update(b)
        qb["h"] = hcur
        f = B.block_forward(qb, g)
        ins.append(qb)
        fwds.append(f)
        hcur = f["h2"]
    N = hcur.shape[0]
    gup = np.broadcast_to(np.asarray(q["w_r"], np.float64), (N, hcur.shape[1])).copy()
    gpos = np.zeros((N, 3))
    for qb, f in zip(reversed(ins), reversed(fwds)):
        v = B.block_vjp(qb, g, f, gup)
        gpos += v["grad_pos"]
        gup = v["grad_h"]
    E = fwds[-1]["E"]
    return float(np.dot(E, Ebar) + np.sum(-gpos * Fbar))


# ------------------------------------------------------- complete block ----
# The readings of oracle.attention and oracle.tri, restated in PyTorch:
# Tri as the plain sum over ordered pairs of distinct edges of a row, MoE0,
# neighbour attention with the envelope-weighted softmax, MoE1.

FULL_PARAMS = ("W_s", "W_ang", "W_T", "logits0", "W1_0", "W2_0", "W_qkv", "Wa_e", "W_o",
               "logits", "W1", "W2")


def _basis(r: torch.Tensor, K: int, rc: float):
    mu = torch.arange(K, dtype=f64) * rc / (K - 1)
    gamma = (K - 1) ** 2 / (2.0 * rc * rc)
    phi = torch.exp(-gamma * (r[:, None] - mu) ** 2)
    fc = torch.where(r < rc, 0.5 * (torch.cos(np.pi * r / rc) + 1.0), torch.zeros_like(r))
    return phi, fc


def _moe(u: torch.Tensor, z: np.ndarray, logits: torch.Tensor, W1, W2, k: int) -> torch.Tensor:
    """u + sum_r gate_r silu(u W1_x) W2_x with element routing (as in _block)."""
    topk, _ = B.route(logits.detach().numpy(), k)
    zt = torch.as_tensor(np.asarray(z, np.int64))
    T = logits.shape[0]
    gate = torch.softmax(logits[torch.arange(T)[:, None], torch.as_tensor(topk)], dim=1)
    out = u
    for r_ in range(k):
        x_of_atom = torch.as_tensor(topk)[zt, r_]
        g_of_atom = gate[zt, r_]
        for x in range(len(W1)):
            idx = torch.nonzero(x_of_atom == x).flatten()
            if idx.numel():
                y = torch.nn.functional.silu(u[idx] @ W1[x]) @ W2[x]
                out = out.index_add(0, idx, g_of_atom[idx, None] * y)
    return out


def _row_pairs(recv: np.ndarray):
    """Ordered pairs (e, e') of distinct edges with the same receiver."""
    E = recv.size
    starts = np.searchsorted(recv, np.arange(recv.max() + 2 if E else 1))
    a, b = [], []
    for i in range(len(starts) - 1):
        lo, hi = starts[i], starts[i + 1]
        if hi - lo < 2:
            continue
        ee = np.arange(lo, hi)
        A, Bm = np.meshgrid(ee, ee, indexing="ij")
        m = A != Bm
        a.append(A[m])
        b.append(Bm[m])
    if not a:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    return np.concatenate(a), np.concatenate(b)


def _full_block(inp: Dict, graph: Dict, d: torch.Tensor, prm: Dict, h: torch.Tensor) -> torch.Tensor:
    rc = B._cutoff(inp)
    recv_np = np.asarray(graph["recv"])
    recv = torch.as_tensor(recv_np, dtype=torch.long)
    src = torch.as_tensor(graph["src"], dtype=torch.long)
    N = h.shape[0]
    k = int(inp["top_k"])
    r = torch.sqrt((d * d).sum(1))
    dhat = d / torch.where(r > 0, r, torch.ones_like(r))[:, None]
    if "W_ang" in prm:
        s = h @ prm["W_s"]
        _, fc = _basis(r, prm["Wa_e"].shape[0], rc)
        pa, pb = _row_pairs(recv_np)
        pa_t, pb_t = torch.as_tensor(pa), torch.as_tensor(pb)
        x = (dhat[pa_t] * dhat[pb_t]).sum(1)
        L = prm["W_ang"].shape[0]
        P = [torch.ones_like(x), x]
        for l in range(1, L - 1):
            P.append(((2 * l + 1) * x * P[l] - l * P[l - 1]) / (l + 1))
        G = sum(P[l][:, None] * prm["W_ang"][l][None, :] for l in range(L))
        term = (fc[pa_t] * fc[pb_t])[:, None] * G * s[src[pa_t]] * s[src[pb_t]]
        tau = torch.zeros(N, s.shape[1], dtype=f64).index_add(0, recv[pa_t], term)
        h = h + tau @ prm["W_T"]
    h0 = _moe(h, inp["z"], prm["logits0"], prm["W1_0"], prm["W2_0"], k)
    nh = int(inp["n_heads"])
    Da = prm["W_o"].shape[0]
    dh = Da // nh
    qkv = h0 @ prm["W_qkv"]
    q, kk, v = qkv[:, :Da], qkv[:, Da:2 * Da], qkv[:, 2 * Da:]
    phi, fc = _basis(r, prm["Wa_e"].shape[0], rc)
    e = fc[:, None] * (phi @ prm["Wa_e"])
    sc = (q[recv] * kk[src] * e).reshape(-1, nh, dh).sum(2) / np.sqrt(dh)     # [E, nh]
    # envelope-weighted softmax per receiver and head (the per-row maximum is
    # a constant shift: it changes nothing but the range of exp)
    m = torch.full((N, nh), -np.inf, dtype=f64).scatter_reduce(
        0, recv[:, None].expand(-1, nh), sc.detach(), reduce="amax", include_self=False)
    w = torch.exp(sc - m[recv])
    Z = torch.zeros(N, nh, dtype=f64).index_add(0, recv, fc[:, None] * w)
    Zr = Z[recv]
    alpha = torch.where(Zr > 0, fc[:, None] * w / torch.where(Zr > 0, Zr, torch.ones_like(Zr)),
                        torch.zeros_like(w))
    A = alpha.repeat_interleave(dh, dim=1)
    o = torch.zeros(N, Da, dtype=f64).index_add(0, recv, A * v[src] * e)
    u = h0 + o @ prm["W_o"]
    return _moe(u, inp["z"], prm["logits"], prm["W1"], prm["W2"], k)


def full_loss_grads(inp: Dict, graph: Dict, Ebar: np.ndarray, Fbar: np.ndarray,
                    experts=None) -> Dict[str, np.ndarray]:
    """E, F and dL/dtheta of L = Ebar . E + Fbar . F through one complete block
    (Tri when the inputs carry W_ang), for every parameter, w_r and h.

    With ``experts = (sel1, sel0)`` the expert weights of MoE1 (W1, W2) and
    MoE0 (W1_0, W2_0) get gradients for those experts only, stacked in that
    order (for very wide layers)."""
    big = {"W1": 0, "W2": 0, "W1_0": 1, "W2_0": 1}
    names = [n for n in FULL_PARAMS if n in inp and (experts is None or n not in big)] + ["w_r", "h"]
    prm = {n: _t(inp[n]).requires_grad_(True) for n in names}
    wrt = [prm[n] for n in names]
    extra = []
    if experts is not None:
        for n, which in big.items():
            full = _t(inp[n])
            sel = [int(x) for x in experts[which]]
            leaves = {x: full[x].clone().requires_grad_(True) for x in sel}
            prm[n] = [leaves[x] if x in leaves else full[x] for x in range(full.shape[0])]
            extra.append((n, [leaves[x] for x in sel]))
            wrt += extra[-1][1]
    pos = _t(inp["pos"]).requires_grad_(True)
    d = _vectors(inp, graph, pos)
    E = _readout(inp, _full_block(inp, graph, d, prm, prm["h"]), prm["w_r"])
    (dEdx,) = torch.autograd.grad(E.sum(), pos, create_graph=True)
    F = -dEdx
    L = (E * _t(Ebar)).sum() + (F * _t(Fbar)).sum()
    grads = torch.autograd.grad(L, wrt, allow_unused=True)
    out = {"E": E.detach().numpy(), "F": F.detach().numpy()}
    np_ = lambda g, t: np.zeros(t.shape) if g is None else g.detach().numpy()
    for n, g in zip(names, grads):
        out["d_" + n] = np_(g, prm[n])
    q = len(names)
    for n, leaves in extra:
        out["d_" + n] = np.stack([np_(grads[q + j], t) for j, t in enumerate(leaves)])
        q += len(leaves)
    return out


def full_loss_value(inp: Dict, Ebar: np.ndarray, Fbar: np.ndarray, **override) -> float:
    """L with E and F from oracle.attention's complete block (no autograd)."""
    from . import attention as A
    from .graph import radius_graph
    q = dict(inp)
    q.update(override)
    g = radius_graph(q["pos"], q["cell"], q["struct_ptr"], B._cutoff(q))
    f = A.full_block_forward(q, g)
    N = f["h2"].shape[0]
    gup = np.broadcast_to(np.asarray(q["w_r"], np.float64), (N, f["h2"].shape[1]))
    v = A.full_block_vjp(q, g, f, gup)
    return float(np.dot(f["E"], Ebar) + np.sum(-v["grad_pos"] * Fbar))


# ------------------------------------------------------------- the stack ----
def stack_full_loss_grads(shared: Dict, blocks, graph: Dict, Ebar: np.ndarray, Fbar: np.ndarray) -> Dict:
    """The loss through a stack of complete blocks (``oracle.stack``): h^(0) =
    Emb[z], blocks in order, readout of the last.  Returns E, F, d_emb, d_w_r
    and ``blocks``: one dict of d_<param> per block."""
    emb = _t(shared["emb"]).requires_grad_(True)
    w_r = _t(shared["w_r"]).requires_grad_(True)
    names = [[n for n in FULL_PARAMS if n in b] for b in blocks]
    prms = [{n: _t(b[n]).requires_grad_(True) for n in nm} for b, nm in zip(blocks, names)]
    pos = _t(shared["pos"]).requires_grad_(True)
    d = _vectors(shared, graph, pos)
    h = emb[torch.as_tensor(np.asarray(shared["z"], np.int64))]
    for prm in prms:
        h = _full_block(shared, graph, d, prm, h)
    E = _readout(shared, h, w_r)
    (dEdx,) = torch.autograd.grad(E.sum(), pos, create_graph=True)
    F = -dEdx
    L = (E * _t(Ebar)).sum() + (F * _t(Fbar)).sum()
    wrt = [emb, w_r] + [prm[n] for prm, nm in zip(prms, names) for n in nm]
    grads = torch.autograd.grad(L, wrt, allow_unused=True)
    np_ = lambda g, t: np.zeros(t.shape) if g is None else g.detach().numpy()
    out = {"E": E.detach().numpy(), "F": F.detach().numpy(), "d_emb": np_(grads[0], emb),
           "d_w_r": np_(grads[1], w_r), "blocks": []}
    q = 2
    for prm, nm in zip(prms, names):
        out["blocks"].append({"d_" + n: np_(grads[q + j], prm[n]) for j, n in enumerate(nm)})
        q += len(nm)
    return out


def stack_full_loss_value(shared: Dict, blocks, Ebar: np.ndarray, Fbar: np.ndarray, **override) -> float:
    """L of the stack with E and F from ``oracle.stack`` (no autograd)."""
    from . import stack as ST
    from .graph import radius_graph
    q = dict(shared)
    q.update(override)
    g = radius_graph(q["pos"], q["cell"], q["struct_ptr"], B._cutoff(q))
    f = ST.stack_forward(q, blocks, g)
    N = f["h_out"].shape[0]
    gup = np.broadcast_to(np.asarray(q["w_r"], np.float64), (N, f["h_out"].shape[1]))
    v = ST.stack_vjp(q, g, f, gup)
    return float(np.dot(f["E"], Ebar) + np.sum(-v["grad_pos"] * Fbar))
