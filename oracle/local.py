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
