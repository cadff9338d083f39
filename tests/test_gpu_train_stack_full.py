"""GPU parity of the training gradient through a stack of complete blocks
(element embedding, blocks with Tri, MoE0, attention and MoE1, readout of the
last) against ``oracle.train.stack_full_loss_grads``: the embedding and w_r
gradients and every parameter gradient of every block, max|gpu - oracle| /
max|oracle| <= 2e-4 per tensor, for seeded loss upstreams dL/dE and dL/dF.
"""
import sys

import numpy as np
import pytest

from element_routed_moe_amd import synth
from oracle import graph as OG
from oracle import train as TR

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-4


def _say(msg):
    print(f"[gpu-train-stack-full] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mlip():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from element_routed_moe_amd import mlip as m
    return m


def rel(a, b):
    a = a.detach().cpu().numpy().astype(np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    m = np.max(np.abs(b)) if b.size else 0.0
    return float(np.max(np.abs(a))) if m == 0 else float(np.max(np.abs(a - b)) / m)


@pytest.mark.parametrize("name,n_blocks", [("tiny", 2), ("top1", 3), ("sparse", 2), ("tiny", 6)])
def test_stack_train_grad(mlip, name, n_blocks):
    cfg = synth.CONFIGS[name]
    shared, blocks = synth.make_stack_inputs(cfg, n_blocks)
    rng = np.random.default_rng(37)
    Ebar = rng.standard_normal(cfg.n_structs)
    Fbar = rng.standard_normal((cfg.n_atoms, 3)).astype(np.float32)
    _say(f"{name} x {n_blocks}: oracle")
    g = OG.radius_graph(shared["pos"], shared["cell"], shared["struct_ptr"], shared["cutoff"])
    ref = TR.stack_full_loss_grads(shared, blocks, g, Ebar, Fbar.astype(np.float64))
    _say(f"{name} x {n_blocks}: GPU")
    st = mlip.Stack(shared, blocks, device="cuda", train=True).step()
    res = st.train_grad(torch.tensor(Ebar, dtype=torch.float64, device="cuda"),
                        torch.from_numpy(Fbar).to("cuda"))
    torch.cuda.synchronize()
    errs = {"F": rel(-st.forces["grad_pos"], ref["F"]), "d_emb": rel(res["d_emb"], ref["d_emb"]),
            "d_w_r": rel(res["d_w_r"], ref["d_w_r"])}
    for b in range(n_blocks):
        for k, v in ref["blocks"][b].items():
            errs[f"{b}:{k}"] = rel(res["blocks"][b][k], v)
    worst = sorted(errs.items(), key=lambda kv: -kv[1])[:6]
    _say(f"{name} x {n_blocks}: {len(errs)} tensors, worst {worst}")
    bad = {k: e for k, e in errs.items() if not e <= TOL}
    assert not bad, bad
