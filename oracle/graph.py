"""Periodic radius graph by brute force (oracle; test infrastructure only).

[review] section 3.1, Figure 1(a): the atomic system is turned into a graph
under periodic repetition of the cell.  The pages give no further detail, so
the plain reading is used: an edge i <- j with lattice shift S exists when j
and i belong to the same structure, (j, S) is not (i, 0), and the image of j
shifted by S lies strictly inside the cutoff sphere of i.

Readings where the pages are silent (each is also what the GPU must match
bit for bit):
  * the predicate is evaluated in float64 from the float32 inputs, in this
    exact order and without fused multiply-adds:
        t  = (S0*C[0] + S1*C[1]) + S2*C[2]          (C rows = lattice vectors)
        d  = (x_j - x_i) + t
        d2 = (d.x*d.x + d.y*d.y) + d.z*d.z
        edge  iff  d2 < r_c*r_c   (strict)
  * edges are ordered by (receiver i, sender j, S0, S1, S2);
  * rev[e] is the index of the reverse edge (j <- i, -S);
  * geom[e] = (float32(d), float32(sqrt(d2))).

The enumeration visits every atom of the structure under every shift with
|S_a| <= ceil(r_c / w_a) + 1, w_a being the spacing of the lattice planes
normal to axis a.  For positions wrapped into the cell, |S_a| <= ceil(r_c/w_a)
already reaches every image inside the cutoff; the extra shell only costs
time and keeps the brute force independent of that argument.
"""
from __future__ import annotations

import itertools
from typing import Dict, Iterable, List

import numpy as np


def plane_spacings(cell64: np.ndarray) -> np.ndarray:
    """Spacing of lattice planes along each cell vector: V / |b x c| etc."""
    a, b, c = cell64
    vol = abs(float(np.dot(a, np.cross(b, c))))
    return np.array([vol / np.linalg.norm(np.cross(b, c)),
                     vol / np.linalg.norm(np.cross(c, a)),
                     vol / np.linalg.norm(np.cross(a, b))])


def shift_range(cell64: np.ndarray, cutoff: float) -> List[int]:
    return [int(np.ceil(cutoff / w)) + 1 for w in plane_spacings(cell64)]


def _rc2(cutoff) -> float:
    rc = float(np.float64(np.float32(cutoff))) if not isinstance(cutoff, np.float64) else float(cutoff)
    return rc * rc


def _pairs_for_receivers(X: np.ndarray, recv_local: np.ndarray, cell64: np.ndarray,
                         rc2: float, nr: List[int]):
    """All (i, j, S, d, d2) with i in recv_local, j in the structure, by brute force."""
    out_i, out_j, out_s, out_d, out_d2 = [], [], [], [], []
    Xi = X[recv_local]                                   # [m, 3]
    diff = X[None, :, :] - Xi[:, None, :]                # diff[i, j] = x_j - x_i
    for S in itertools.product(range(-nr[0], nr[0] + 1),
                               range(-nr[1], nr[1] + 1),
                               range(-nr[2], nr[2] + 1)):
        t = (S[0] * cell64[0] + S[1] * cell64[1]) + S[2] * cell64[2]
        d = diff + t
        d2 = (d[..., 0] * d[..., 0] + d[..., 1] * d[..., 1]) + d[..., 2] * d[..., 2]
        m = d2 < rc2
        if S == (0, 0, 0):
            m[np.arange(len(recv_local)), recv_local] = False
        ii, jj = np.nonzero(m)
        if ii.size == 0:
            continue
        out_i.append(recv_local[ii])
        out_j.append(jj)
        out_s.append(np.broadcast_to(np.array(S, np.int64), (ii.size, 3)))
        out_d.append(d[ii, jj])
        out_d2.append(d2[ii, jj])
    return out_i, out_j, out_s, out_d, out_d2


def _finish(N: int, recv, src, shift, d, d2) -> Dict[str, np.ndarray]:
    if len(recv):
        recv = np.concatenate(recv)
        src = np.concatenate(src)
        shift = np.concatenate(shift).astype(np.int64)
        d = np.concatenate(d)
        d2 = np.concatenate(d2)
    else:
        recv = np.zeros(0, np.int64)
        src = np.zeros(0, np.int64)
        shift = np.zeros((0, 3), np.int64)
        d = np.zeros((0, 3))
        d2 = np.zeros(0)
    order = np.lexsort((shift[:, 2], shift[:, 1], shift[:, 0], src, recv))
    recv, src, shift, d, d2 = recv[order], src[order], shift[order], d[order], d2[order]
    return dict(recv=recv, src=src, shift=shift, d=d, d2=d2)


def radius_graph(pos, cell, struct_ptr, cutoff, chunk: int = 256) -> Dict[str, np.ndarray]:
    """Full periodic radius graph of a batch of structures.

    pos [N,3] (float32 or float64, Cartesian), cell [B,3,3] (rows are lattice
    vectors), struct_ptr [B+1].  Returns row_ptr [N+1], src [E], shift [E,3],
    rev [E], d [E,3] (float64), d2 [E], r [E] (float64), geom [E,4] (float32).
    """
    pos64 = np.asarray(pos).astype(np.float64)
    struct_ptr = np.asarray(struct_ptr, np.int64)
    N = pos64.shape[0]
    rc2 = _rc2(cutoff)
    R, S_, J, D, D2 = [], [], [], [], []
    for b in range(len(struct_ptr) - 1):
        lo, hi = int(struct_ptr[b]), int(struct_ptr[b + 1])
        if hi <= lo:
            continue
        C = np.asarray(cell[b]).astype(np.float64)
        nr = shift_range(C, np.sqrt(rc2))
        X = pos64[lo:hi]
        for c0 in range(0, hi - lo, chunk):
            loc = np.arange(c0, min(hi - lo, c0 + chunk))
            i_, j_, s_, d_, d2_ = _pairs_for_receivers(X, loc, C, rc2, nr)
            R += [v + lo for v in i_]
            J += [v + lo for v in j_]
            S_ += s_
            D += d_
            D2 += d2_
    g = _finish(N, R, J, S_, D, D2)
    return _complete(N, g)


def _complete(N: int, g: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    recv, src, shift = g["recv"], g["src"], g["shift"]
    E = recv.size
    row_ptr = np.zeros(N + 1, np.int64)
    row_ptr[1:] = np.cumsum(np.bincount(recv, minlength=N))
    # reverse edge: (j <- i, -S); found by an exact search over integer keys
    W = 2 * (int(np.abs(shift).max()) if E else 0) + 1
    off = W // 2

    def key(i, j, s):
        return (((i * N + j) * W + (s[:, 0] + off)) * W + (s[:, 1] + off)) * W + (s[:, 2] + off)

    k_fwd = key(recv, src, shift)
    k_rev = key(src, recv, -shift)
    rev = np.searchsorted(k_fwd, k_rev)
    if E:
        assert np.all(k_fwd[np.minimum(rev, E - 1)] == k_rev), "radius graph is not symmetric"
    r = np.sqrt(g["d2"])
    geom = np.zeros((E, 4), np.float32)
    geom[:, :3] = g["d"].astype(np.float32)
    geom[:, 3] = r.astype(np.float32)
    return dict(row_ptr=row_ptr, recv=recv, src=src, shift=shift, rev=rev,
                d=g["d"], d2=g["d2"], r=r, geom=geom)


def radius_graph_rows(pos, cell, struct_ptr, cutoff, atoms: Iterable[int]) -> Dict[int, Dict]:
    """Rows of the same graph for a few receivers only (for very large cells).

    Returns {i: dict(src, shift, d, d2, r, geom)} with each row in the canonical
    (sender, shift) order.
    """
    pos64 = np.asarray(pos).astype(np.float64)
    struct_ptr = np.asarray(struct_ptr, np.int64)
    rc2 = _rc2(cutoff)
    out = {}
    for i in atoms:
        i = int(i)
        b = int(np.searchsorted(struct_ptr, i, side="right") - 1)
        lo, hi = int(struct_ptr[b]), int(struct_ptr[b + 1])
        C = np.asarray(cell[b]).astype(np.float64)
        nr = shift_range(C, np.sqrt(rc2))
        X = pos64[lo:hi]
        i_, j_, s_, d_, d2_ = _pairs_for_receivers(X, np.array([i - lo]), C, rc2, nr)
        g = _finish(0, [v + lo for v in i_], [v + lo for v in j_], s_, d_, d2_)
        r = np.sqrt(g["d2"])
        geom = np.zeros((r.size, 4), np.float32)
        geom[:, :3] = g["d"].astype(np.float32)
        geom[:, 3] = r.astype(np.float32)
        out[i] = dict(src=g["src"], shift=g["shift"], d=g["d"], d2=g["d2"], r=r, geom=geom)
    return out
