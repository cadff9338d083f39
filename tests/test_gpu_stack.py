"""GPU parity of a stack of complete blocks on one radius graph (element
embedding -> B x (Tri, MoE0, attention, MoE1) -> readout, and the input
gradient through all blocks) against the CPU oracle (``oracle.stack``).

Small cases run the oracle on the whole batch; at the S widths the GPU runs
all 32 cells and the oracle checks the first cell completely (cells are
independent structures).  Floating-point tensors must satisfy
max|gpu - oracle| / max|oracle| <= 2e-4.
"""
import sys

import numpy as np
import pytest

from element_routed_moe_amd import synth
from oracle import block as OB
from oracle import graph as OG
from oracle import stack as OS

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-4


def _say(msg):
    print(f"[gpu-stack] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mlip():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from element_routed_moe_amd import mlip as m
    return m


def rel(a, b):
    a = a.detach().cpu().numpy().astype(np.float64) if hasattr(a, "detach") else np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _first_structure(shared):
    n = int(shared["struct_ptr"][1])
    q = dict(shared)
    q["pos"] = shared["pos"][:n]
    q["cell"] = shared["cell"][:1]
    q["struct_ptr"] = shared["struct_ptr"][:2]
    q["z"] = shared["z"][:n]
    return q, n


@pytest.mark.parametrize("name,n_blocks", [("tiny", 6), ("ragged", 6), ("sparse", 2), ("top1", 3),
                                           ("S", 2)])
def test_stack_matches_oracle(mlip, name, n_blocks):
    cfg = synth.CONFIGS[name]
    _say(f"{name} x {n_blocks} blocks: inputs")
    shared, blocks = synth.make_stack_inputs(cfg, n_blocks)
    _say(f"{name}: GPU step")
    st = mlip.Stack(shared, blocks, device="cuda").step()
    torch.cuda.synchronize()
    ref_in, n = (_first_structure(shared) if name == "S" else (shared, cfg.n_atoms))
    _say(f"{name}: oracle on {n} atoms")
    g = OG.radius_graph(ref_in["pos"], ref_in["cell"], ref_in["struct_ptr"], ref_in["cutoff"])
    f = OS.stack_forward(ref_in, blocks, g)
    g_up = np.broadcast_to(shared["w_r"], (n, cfg.d_node)).astype(np.float64)
    v = OS.stack_vjp(ref_in, g, f, g_up)
    nb = len(ref_in["struct_ptr"]) - 1
    errs = {"h_out": rel(st.layers[-1].moe["h_out"][:n], f["h_out"]),
            "eps": rel(st.ro["eps"][:n], f["eps"]),
            "energy": rel(st.ro["energy"][:nb], f["E"]),
            "grad_h0": rel(st.grad_h0[:n], v["grad_h0"]),
            "grad_pos": rel(st.forces["grad_pos"][:n], v["grad_pos"]),
            "atom_virial": rel(st.forces["atom_virial"][:n], v["atom_virial"]),
            "grad_strain": rel(st.forces["grad_strain"][:nb], OB.voigt(v["grad_strain"]))}
    _say(f"{name}: errors {errs}")
    bad = {k: e for k, e in errs.items() if not e <= TOL}
    assert not bad, bad


def test_stack_deterministic(mlip):
    cfg = synth.CONFIGS["ragged"]
    shared, blocks = synth.make_stack_inputs(cfg, 3)
    _say("determinism: ragged x 3 blocks, two steps")
    st = mlip.Stack(shared, blocks, device="cuda")
    st.step()
    torch.cuda.synchronize()
    first = {k: t.clone() for k, t in st.forces.items()}
    e1 = st.ro["energy"].clone()
    st.step()
    torch.cuda.synchronize()
    for k in first:
        assert torch.equal(first[k], st.forces[k]), k
    assert torch.equal(e1, st.ro["energy"])
