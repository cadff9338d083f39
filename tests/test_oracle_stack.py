"""Pins of the oracle's block stack (``oracle.stack``), CPU only: float64
central differences of the energy through 2 and 6 chained complete blocks
(positions and strain), the sum of forces, and rotation invariance.  The
blocks themselves are pinned in test_oracle_attention / test_oracle_tri;
these tests pin the chaining (edge gradients of every block collected, node
gradients passed down)."""
import numpy as np
import pytest

from element_routed_moe_amd import synth
from oracle import block as B
from oracle import graph as G
from oracle import stack as ST


def _graph(inp):
    return G.radius_graph(inp["pos"], inp["cell"], inp["struct_ptr"], inp["cutoff"])


@pytest.mark.parametrize("n_blocks", [2, 6])
def test_stack_forces_fd(n_blocks):
    cfg = synth.CONFIGS["tiny"]
    shared, blocks = synth.make_stack_inputs(cfg, n_blocks)
    g = _graph(shared)
    f = ST.stack_forward(shared, blocks, g)
    g_up = np.broadcast_to(shared["w_r"], (cfg.n_atoms, cfg.d_node)).astype(np.float64)
    v = ST.stack_vjp(shared, g, f, g_up)
    pos = shared["pos"].astype(np.float64)
    step = 1e-5
    rng = np.random.default_rng(n_blocks)
    idx = [(int(i), int(c)) for i, c in zip(rng.integers(0, cfg.n_atoms, 12), rng.integers(0, 3, 12))]
    ref, got = [], []
    for i, c in idx:
        p1 = pos.copy(); p1[i, c] += step
        p2 = pos.copy(); p2[i, c] -= step
        ref.append((ST.stack_energy(shared, blocks, pos=p1)[0] - ST.stack_energy(shared, blocks, pos=p2)[0])
                   / (2 * step))
        got.append(v["grad_pos"][i, c])
    ref, got = np.array(ref), np.array(got)
    assert np.max(np.abs(got - ref)) <= 1e-6 * np.max(np.abs(ref))
    assert np.max(np.abs(v["grad_pos"].sum(0))) < 1e-11 * np.max(np.abs(v["grad_pos"]))


def test_stack_strain_fd_and_rotation():
    cfg = synth.CONFIGS["tiny"]
    shared, blocks = synth.make_stack_inputs(cfg, 2)
    g = _graph(shared)
    f = ST.stack_forward(shared, blocks, g)
    g_up = np.broadcast_to(shared["w_r"], (cfg.n_atoms, cfg.d_node)).astype(np.float64)
    v = ST.stack_vjp(shared, g, f, g_up)
    gs = v["grad_strain"][0]
    pos = shared["pos"].astype(np.float64)
    cell = shared["cell"].astype(np.float64)
    fd = np.zeros((3, 3))
    for a in range(3):
        for b in range(3):
            vals = []
            for sgn in (1.0, -1.0):
                F = np.eye(3)
                F[a, b] += sgn * 1e-6
                vals.append(ST.stack_energy(shared, blocks, pos=pos @ F.T, cell=cell @ F.T)[0])
            fd[a, b] = (vals[0] - vals[1]) / 2e-6
    assert np.max(np.abs(fd - gs)) <= 1e-6 * np.max(np.abs(gs))
    assert np.allclose(gs, gs.T, atol=1e-10 * np.abs(gs).max())
    assert np.allclose(v["atom_virial"].sum(0), B.voigt(gs), atol=1e-10 * np.abs(gs).max())
    Q, _ = np.linalg.qr(np.random.default_rng(9).standard_normal((3, 3)))
    E0 = f["E"][0]
    assert abs(ST.stack_energy(shared, blocks, pos=pos @ Q.T, cell=cell @ Q.T)[0] - E0) <= 1e-12 * abs(E0)
