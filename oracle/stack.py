"""A stack of complete interaction blocks on one radius graph (oracle; test
infrastructure only).

The paper review (section 3.1, Table II) gives 6 layers for every model size;
Fig. 1(b) shows feature embedding, then the interaction blocks, then the
readout.  Reading taken here: the node features start as a learned per-element
embedding, h^(0)_i = Emb[z_i]; every block b is the complete block of
``oracle.attention`` (Tri, MoE0, attention, MoE1) with its own parameters;
the readout of ``oracle.block`` is applied to the last block's output only:

    h^(b+1) = Block_b(h^(b)),   eps_i = h^(B)_i . w_r,   E_s = sum of eps over structure s.

Forces and the strain gradient collect the edge gradients of every block
(all blocks share the positions, hence the graph).
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np

from . import attention as A
from . import block as B

f64 = np.float64


def block_inputs(inp: Dict, params: Dict, h: np.ndarray) -> Dict:
    """The input dict of one complete block: shared geometry and readout, the
    block's own parameters, and its incoming node features."""
    q = {k: inp[k] for k in ("pos", "cell", "struct_ptr", "z", "cutoff", "top_k", "w_r", "n_heads")}
    q.update(params)
    q["h"] = h
    return q


def stack_forward(inp: Dict, blocks: List[Dict], graph: Dict[str, np.ndarray]) -> Dict:
    h = np.asarray(inp["emb"], f64)[np.asarray(inp["z"], np.int64)]
    fwds, ins = [], []
    for params in blocks:
        q = block_inputs(inp, params, h)
        f = A.full_block_forward(q, graph)
        fwds.append(f)
        ins.append(q)
        h = f["h2"]
    eps, E = B.readout(h, inp["w_r"], inp["struct_ptr"])
    return dict(h0=np.asarray(inp["emb"], f64)[np.asarray(inp["z"], np.int64)], fwds=fwds, ins=ins,
                h_out=h, eps=eps, E=E)


def stack_vjp(inp: Dict, graph: Dict[str, np.ndarray], fwd: Dict, g: np.ndarray) -> Dict:
    """dL/dh^(0), dL/dx, dL/d(strain) and per-atom virial for g = dL/dh^(B)."""
    g = np.asarray(g, f64)
    gvec = np.zeros((graph["r"].size, 3), f64)
    for q, f in zip(reversed(fwd["ins"]), reversed(fwd["fwds"])):
        v = A.full_block_vjp(q, graph, f, g)
        gvec += v["gvec"]
        g = v["grad_h"]
    N = g.shape[0]
    gpos, gstrain, av = B.edge_forces_vec(gvec, graph, N, inp["struct_ptr"])
    return dict(grad_h0=g, gvec=gvec, grad_pos=gpos, grad_strain=gstrain, atom_virial=av)


def stack_energy(inp: Dict, blocks: List[Dict], pos=None, cell=None) -> np.ndarray:
    from .graph import radius_graph
    q = dict(inp)
    if pos is not None:
        q["pos"] = pos
    if cell is not None:
        q["cell"] = cell
    gr = radius_graph(q["pos"], q["cell"], q["struct_ptr"], B._cutoff(q))
    return stack_forward(q, blocks, gr)["E"]
