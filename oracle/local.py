"""Block outputs for a few sampled atoms of a large system (oracle; test
infrastructure only).

The same step functions as ``oracle.block`` applied to the neighbourhood of
each sampled atom, so that outputs at full workload sizes can be checked one
atom at a time:

* forward at atom i needs row i (edges with receiver i) and s_j = h_j @ W_d of
  its senders;
* the input gradient at atom i needs, for i and for every atom sharing an edge
  with it, u (hence their rows) and dL/du; the edges with sender i are
  enumerated by brute force with the roles of the two endpoints swapped.

For large orthorhombic cells the candidate partners of an atom are narrowed
with a periodic k-d tree (scipy) at r_c + 1e-3 under the minimum-image
convention; every candidate is then tested with the exact float64 predicate
of ``oracle.graph`` under every lattice shift.  Since every image inside r_c
is at least as far as the minimum image, the candidate set is a superset of
the true partners.
"""
from __future__ import annotations

import itertools
from typing import Dict, Iterable, List, Optional

import numpy as np

from . import block as B
from .graph import shift_range, _rc2

f64 = np.float64


class LocalBlock:
    def __init__(self, inp: Dict[str, np.ndarray], use_tree: Optional[bool] = None):
        self.inp = inp
        self.rc = float(np.float64(np.float32(inp["cutoff"])))
        self.rc2 = _rc2(inp["cutoff"])
        self.pos = np.asarray(inp["pos"]).astype(f64)
        self.cell = np.asarray(inp["cell"]).astype(f64)
        self.sp = np.asarray(inp["struct_ptr"], np.int64)
        self.z = np.asarray(inp["z"], np.int64)
        self.topk, self.gate = B.route(inp["logits"], int(inp["top_k"]))
        self.W_d = np.asarray(inp["W_d"], f64)
        self.W_u = np.asarray(inp["W_u"], f64)
        self._rows: Dict[int, Dict] = {}
        self._cols: Dict[int, Dict] = {}
        self._trees = {}
        self.use_tree = use_tree

    # ------------------------------------------------------------ edges ---
    def _struct(self, i: int) -> int:
        return int(np.searchsorted(self.sp, i, side="right") - 1)

    def _candidates(self, b: int, i: int) -> np.ndarray:
        lo, hi = int(self.sp[b]), int(self.sp[b + 1])
        C = self.cell[b]
        ortho = np.all(C == np.diag(np.diag(C)))
        use = self.use_tree if self.use_tree is not None else (hi - lo > 4096)
        if not (use and ortho):
            return np.arange(lo, hi)
        if b not in self._trees:
            from scipy.spatial import cKDTree
            box = np.diag(C).copy()
            self._trees[b] = cKDTree(self.pos[lo:hi], boxsize=box)
        cand = self._trees[b].query_ball_point(self.pos[i], self.rc + 1e-3)
        return np.sort(np.asarray(cand, np.int64)) + lo

    def _edges(self, i: int, as_sender: bool) -> Dict[str, np.ndarray]:
        """Edges with receiver i (as_sender False) or with sender i (True)."""
        b = self._struct(i)
        C = self.cell[b]
        nr = shift_range(C, self.rc)
        cand = self._candidates(b, i)
        xi = self.pos[i]
        other, shifts, ds, d2s = [], [], [], []
        for S in itertools.product(*[range(-n, n + 1) for n in nr]):
            t = (S[0] * C[0] + S[1] * C[1]) + S[2] * C[2]
            if as_sender:     # edge (j <- i, S): d = (x_i - x_j) + t
                d = (xi[None, :] - self.pos[cand]) + t
            else:             # edge (i <- j, S): d = (x_j - x_i) + t
                d = (self.pos[cand] - xi[None, :]) + t
            d2 = (d[:, 0] * d[:, 0] + d[:, 1] * d[:, 1]) + d[:, 2] * d[:, 2]
            m = d2 < self.rc2
            if S == (0, 0, 0):
                m &= cand != i
            if m.any():
                other.append(cand[m])
                shifts.append(np.broadcast_to(np.array(S, np.int64), (int(m.sum()), 3)))
                ds.append(d[m])
                d2s.append(d2[m])
        if other:
            other = np.concatenate(other)
            shifts = np.concatenate(shifts)
            ds = np.concatenate(ds)
            d2s = np.concatenate(d2s)
        else:
            other = np.zeros(0, np.int64)
            shifts = np.zeros((0, 3), np.int64)
            ds = np.zeros((0, 3))
            d2s = np.zeros(0)
        order = np.lexsort((shifts[:, 2], shifts[:, 1], shifts[:, 0], other))
        r = np.sqrt(d2s[order])
        return dict(other=other[order], shift=shifts[order], d=ds[order], d2=d2s[order], r=r)

    def row(self, i: int) -> Dict[str, np.ndarray]:
        if i not in self._rows:
            self._rows[i] = self._edges(i, as_sender=False)
        return self._rows[i]

    def col(self, i: int) -> Dict[str, np.ndarray]:
        if i not in self._cols:
            self._cols[i] = self._edges(i, as_sender=True)
        return self._cols[i]

    # ---------------------------------------------------------- forward ---
    def s(self, atoms: np.ndarray) -> np.ndarray:
        return np.asarray(self.inp["h"][atoms], f64) @ self.W_d

    def u(self, atoms: Iterable[int]) -> np.ndarray:
        atoms = list(atoms)
        out = np.zeros((len(atoms), self.W_u.shape[1]), f64)
        for n, i in enumerate(atoms):
            rw = self.row(i)
            e = B.edge_embedding(rw["r"], self.inp["W_e"], self.rc)
            a = (e * self.s(rw["other"])).sum(axis=0)
            out[n] = np.asarray(self.inp["h"][i], f64) + a @ self.W_u
        return out

    def forward(self, atoms: Iterable[int]) -> Dict[str, np.ndarray]:
        atoms = np.asarray(list(atoms), np.int64)
        u = self.u(atoms)
        h2 = B.moe_forward(u, self.z[atoms], self.topk, self.gate, self.inp["W1"], self.inp["W2"])
        eps = h2 @ np.asarray(self.inp["w_r"], f64)
        return dict(u=u, h2=h2, eps=eps)

    # -------------------------------------------------------------- VJP ---
    def vjp(self, atoms: Iterable[int], g_all: np.ndarray) -> Dict[str, np.ndarray]:
        """grad_h and grad_pos at the sampled atoms, for upstream g = dL/dh' [N, Dn]."""
        atoms = [int(i) for i in atoms]
        need = set(atoms)
        for i in atoms:
            need.update(int(j) for j in self.row(i)["other"])
            need.update(int(j) for j in self.col(i)["other"])
        need = sorted(need)
        idx = {a: n for n, a in enumerate(need)}
        need_arr = np.asarray(need, np.int64)
        u = self.u(need)
        g = np.asarray(g_all[need_arr], f64)
        ubar = B.moe_vjp(u, g, self.z[need_arr], self.topk, self.gate, self.inp["W1"], self.inp["W2"])
        abar = ubar @ self.W_u.T
        s_need = self.s(need_arr)
        Dn = self.W_u.shape[1]
        grad_h = np.zeros((len(atoms), Dn), f64)
        grad_pos = np.zeros((len(atoms), 3), f64)
        virial = np.zeros((len(atoms), 3, 3), f64)
        for n, i in enumerate(atoms):
            ii = idx[i]
            rw, cl = self.row(i), self.col(i)
            # edges with receiver i: c = sum((abar_i * s_j) * de/dr); contributes -c dhat
            if rw["r"].size:
                js = np.array([idx[int(j)] for j in rw["other"]])
                de = B.edge_embedding_dr(rw["r"], self.inp["W_e"], self.rc)
                c = np.sum(abar[ii][None, :] * s_need[js] * de, axis=1)
                dhat = np.where(rw["r"][:, None] > 0, rw["d"] / np.maximum(rw["r"], 1e-300)[:, None], 0.0)
                grad_pos[n] -= (c[:, None] * dhat).sum(axis=0)
                virial[n] += 0.5 * np.einsum("e,ea,eb->ab", c, dhat, rw["d"])
            # edges with sender i: sbar_i += e * abar_recv; contributes +c dhat
            sbar = np.zeros(self.W_u.shape[0], f64)
            if cl["r"].size:
                js = np.array([idx[int(j)] for j in cl["other"]])
                e = B.edge_embedding(cl["r"], self.inp["W_e"], self.rc)
                sbar = (e * abar[js]).sum(axis=0)
                de = B.edge_embedding_dr(cl["r"], self.inp["W_e"], self.rc)
                c = np.sum(abar[js] * s_need[ii][None, :] * de, axis=1)
                dhat = np.where(cl["r"][:, None] > 0, cl["d"] / np.maximum(cl["r"], 1e-300)[:, None], 0.0)
                grad_pos[n] += (c[:, None] * dhat).sum(axis=0)
                virial[n] += 0.5 * np.einsum("e,ea,eb->ab", c, dhat, cl["d"])
            grad_h[n] = ubar[ii] + sbar @ self.W_d.T
        return dict(grad_h=grad_h, grad_pos=grad_pos, atom_virial=B.voigt(virial))


class LocalFullBlock(LocalBlock):
    """The complete block (``oracle.attention``, with ``oracle.tri`` first) at a
    few sampled atoms.

    The forward at atom i needs Tri and MoE0 at i and at its neighbours
    (q_i, k_j, v_j) and the softmax over row i.  The input gradient at i needs
    the attention's receiver-side quantities of every row within two hops
    (for the reverse edges and for kbar, vbar of the neighbours), hence Tri
    and MoE0 up to three hops out.  Every per-atom step is the oracle's own
    step function on a subset of atoms; MoE layers act atom by atom, and the
    Tri and attention rows are per receiver, so subsets give the same rows.
    """

    def __init__(self, inp: Dict[str, np.ndarray], use_tree: Optional[bool] = None):
        super().__init__(inp, use_tree)
        from . import attention as A
        from . import tri as TR
        self.A = A
        self.TR = TR
        k = int(inp["top_k"])
        self.topk0, self.gate0 = B.route(inp["logits0"], k)
        self.nh = int(inp["n_heads"])
        self.W_qkv = np.asarray(inp["W_qkv"], f64)
        self.W_o = np.asarray(inp["W_o"], f64)
        self.Da = self.W_o.shape[0]
        self.dh = self.Da // self.nh
        self.has_tri = "W_ang" in inp
        if self.has_tri:
            self.W_s = np.asarray(inp["W_s"], f64)
            self.W_ang = np.asarray(inp["W_ang"], f64)
            self.W_T = np.asarray(inp["W_T"], f64)
        self._hT: Dict[int, np.ndarray] = {}
        self._h0: Dict[int, np.ndarray] = {}
        self._att: Dict[int, Dict] = {}

    # ---------------------------------------------------------------- Tri ---
    def _unit_row(self, rw):
        r = rw["r"]
        with np.errstate(invalid="ignore", divide="ignore"):
            return np.where(r[:, None] > 0, rw["d"] / r[:, None], 0.0)

    def s_tri(self, atoms) -> np.ndarray:
        return np.asarray(self.inp["h"][np.asarray(atoms, np.int64)], f64) @ self.W_s

    def hT(self, atoms) -> np.ndarray:
        atoms = [int(a) for a in atoms]
        for a in atoms:
            if a in self._hT:
                continue
            h = np.asarray(self.inp["h"][a], f64)
            if self.has_tri:
                rw = self.row(a)
                tau = self.TR.tri_row(self._unit_row(rw), B.envelope(rw["r"], self.rc),
                                      self.s_tri(rw["other"]), self.W_ang)
                h = h + tau @ self.W_T
            self._hT[a] = h
        return np.stack([self._hT[a] for a in atoms])

    def h0(self, atoms) -> np.ndarray:
        atoms = [int(a) for a in atoms]
        todo = sorted(set(a for a in atoms if a not in self._h0))
        if todo:
            t = np.asarray(todo, np.int64)
            out = B.moe_forward(self.hT(todo), self.z[t], self.topk0, self.gate0,
                                self.inp["W1_0"], self.inp["W2_0"])
            for n, a in enumerate(todo):
                self._h0[a] = out[n]
        return np.stack([self._h0[a] for a in atoms]) if atoms else np.zeros((0, self.W_qkv.shape[0]))

    def qkv(self, atoms) -> np.ndarray:
        return self.h0(atoms) @ self.W_qkv

    def att_row(self, i: int) -> Dict:
        """Softmax and output of row i (edges with receiver i)."""
        if i in self._att:
            return self._att[i]
        rw = self.row(i)
        Da, nh = self.Da, self.nh
        qi = self.qkv([i])[0, :Da]
        kv = self.qkv(rw["other"]) if rw["other"].size else np.zeros((0, 3 * Da))
        kj, vj = kv[:, Da:2 * Da], kv[:, 2 * Da:]
        e = B.edge_embedding(rw["r"], self.inp["Wa_e"], self.rc)
        f = B.envelope(rw["r"], self.rc)
        s = self.A.head_sum(qi[None, :] * kj * e, nh) / np.sqrt(self.dh)
        recv = np.zeros(rw["r"].size, np.int64)
        alpha, w, m, Z = self.A.neighbour_softmax(s, f, recv, 1)
        ht = self.A.heads_of(Da, nh)
        o = (alpha[:, ht] * vj * e).sum(axis=0) if rw["r"].size else np.zeros(Da)
        u = self.h0([i])[0] + o @ self.W_o
        res = dict(q=qi, k=kj, v=vj, e=e, f=f, s=s, alpha=alpha, w=w, Z=Z[0], o=o, u=u)
        self._att[i] = res
        return res

    def forward(self, atoms: Iterable[int]) -> Dict[str, np.ndarray]:
        atoms = np.asarray(list(atoms), np.int64)
        u = np.stack([self.att_row(int(i))["u"] for i in atoms])
        h2 = B.moe_forward(u, self.z[atoms], self.topk, self.gate, self.inp["W1"], self.inp["W2"])
        eps = h2 @ np.asarray(self.inp["w_r"], f64)
        return dict(u=u, h2=h2, eps=eps)

    def _nbrs(self, atoms):
        out = set(int(a) for a in atoms)
        for a in atoms:
            out.update(int(j) for j in self.row(int(a))["other"])
        return sorted(out)

    def vjp(self, atoms: Iterable[int], g_all: np.ndarray) -> Dict[str, np.ndarray]:
        """grad_h, grad_pos and the per-atom virial at the sampled atoms."""
        atoms = [int(i) for i in atoms]
        J1 = self._nbrs(atoms)          # rows whose edge gradients reach the samples
        J2 = self._nbrs(J1)             # rows whose attention terms reach J1
        J2arr = np.asarray(J2, np.int64)
        u = np.stack([self.att_row(j)["u"] for j in J2])
        ubar = B.moe_vjp(u, np.asarray(g_all[J2arr], f64), self.z[J2arr], self.topk, self.gate,
                         self.inp["W1"], self.inp["W2"])
        ub = {j: ubar[n] for n, j in enumerate(J2)}
        ht = self.A.heads_of(self.Da, self.nh)
        sq = 1.0 / np.sqrt(self.dh)
        Wa_e = self.inp["Wa_e"]
        rowq = {}
        for j in J2:           # attention receiver-side quantities
            a = self.att_row(j)
            rw = self.row(j)
            ob = ub[j] @ self.W_o.T
            abar = self.A.head_sum(ob[None, :] * a["v"] * a["e"], self.nh)
            beta = self.A.head_sum((ob * a["o"])[None, :], self.nh)[0]
            diff = abar - beta[None, :]
            gbar = a["alpha"] * diff
            with np.errstate(invalid="ignore", divide="ignore"):
                fbar = np.sum(np.where(a["Z"][None, :] > 0, a["w"] / a["Z"][None, :], 0.0) * diff, axis=1)
            ebar = gbar[:, ht] * a["q"][None, :] * a["k"] * sq + a["alpha"][:, ht] * ob[None, :] * a["v"]
            c = (np.sum(ebar * B.edge_embedding_dr(rw["r"], Wa_e, self.rc), axis=1)
                 + fbar * B.envelope_dr(rw["r"], self.rc))
            key = {(int(o), int(s[0]), int(s[1]), int(s[2])): n
                   for n, (o, s) in enumerate(zip(rw["other"], rw["shift"]))}
            rowq[j] = dict(ob=ob, gbar=gbar, c=c, key=key, gvec=c[:, None] * self._unit_row(rw))
        Da = self.Da
        h0bar = {}
        for m in J1:            # dL/dh0 through the residual, q, k and v
            a, rw, qm = self.att_row(m), self.row(m), rowq[m]
            qbar = (qm["gbar"][:, ht] * a["k"] * a["e"]).sum(axis=0) * sq if rw["r"].size else np.zeros(Da)
            kbar = np.zeros(Da)
            vbar = np.zeros(Da)
            for n, (j, S) in enumerate(zip(rw["other"], rw["shift"])):
                j = int(j)
                rj, aj = rowq[j], self.att_row(j)
                r_idx = rj["key"][(m, -int(S[0]), -int(S[1]), -int(S[2]))]
                kbar += rj["gbar"][r_idx][ht] * aj["q"] * a["e"][n] * sq
                vbar += aj["alpha"][r_idx][ht] * rj["ob"] * a["e"][n]
            h0bar[m] = ub[m] + np.concatenate([qbar, kbar, vbar]) @ self.W_qkv.T
        J1arr = np.asarray(J1, np.int64)
        hTb = B.moe_vjp(self.hT(J1), np.stack([h0bar[m] for m in J1]), self.z[J1arr],
                        self.topk0, self.gate0, self.inp["W1_0"], self.inp["W2_0"])
        hT_bar = {m: hTb[n] for n, m in enumerate(J1)}
        sbar_tri = {}
        if self.has_tri:        # Tri rows of J1: sender gradients and edge vectors
            for m in J1:
                rw = self.row(m)
                r = rw["r"]
                sb, gv = self.TR.tri_row_vjp(self._unit_row(rw), r, B.envelope(r, self.rc),
                                             B.envelope_dr(r, self.rc), self.s_tri(rw["other"]),
                                             self.W_ang, hT_bar[m] @ self.W_T.T)
                rowq[m]["gvec"] = rowq[m]["gvec"] + gv
                for n, j in enumerate(rw["other"]):
                    sbar_tri[int(j)] = sbar_tri.get(int(j), 0.0) + sb[n]
        Dn = self.W_o.shape[1]
        grad_h = np.zeros((len(atoms), Dn), f64)
        grad_pos = np.zeros((len(atoms), 3), f64)
        virial = np.zeros((len(atoms), 3, 3), f64)
        for n, i in enumerate(atoms):
            rw, ri = self.row(i), rowq[i]
            for m, (j, S) in enumerate(zip(rw["other"], rw["shift"])):
                rj = rowq[int(j)]
                r_idx = rj["key"][(i, -int(S[0]), -int(S[1]), -int(S[2]))]
                g = ri["gvec"][m] - rj["gvec"][r_idx]       # d_rev = -d
                grad_pos[n] -= g
                t = np.outer(g, rw["d"][m])
                virial[n] += 0.25 * (t + t.T)
            gh = hT_bar[i]
            if self.has_tri and i in sbar_tri:
                gh = gh + sbar_tri[i] @ self.W_s.T
            grad_h[n] = gh
        return dict(grad_h=grad_h, grad_pos=grad_pos, atom_virial=B.voigt(virial))
