"""GPU parity of the training gradient (parameter gradients of an energy +
force loss through one block) against the float64 oracle ``oracle.train``.

The loss upstreams are seeded random: dL/dE ~ N(0,1) per structure and
dL/dF ~ N(0,1) per force component.  Each gradient tensor must satisfy
max|gpu - oracle| / max|oracle| <= 2e-4.  The cases cover ragged widths
(partial 128-wide weight-gradient tiles), split-K dense weight gradients
(celllist, wide_ragged), isolated atoms, top-1 routing, triclinic cells and
an empty system.
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
KEYS = ["d_W_e", "d_W_d", "d_W_u", "d_W1", "d_W2", "d_logits", "d_w_r", "d_h"]


def _say(msg):
    print(f"[gpu-train] {msg}", flush=True)
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
    if b.size == 0 or np.max(np.abs(b)) == 0:
        return float(np.max(np.abs(a))) if a.size else 0.0
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


def _upstreams(cfg, seed=21):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(cfg.n_structs), rng.standard_normal((cfg.n_atoms, 3)).astype(np.float32)


def _gpu(mlip, inp, Ebar, Fbar):
    blk = mlip.Block(inp, device="cuda", train=True).step()
    res = blk.train_grad(torch.tensor(Ebar, dtype=torch.float64, device="cuda"),
                         torch.from_numpy(Fbar).to("cuda"))
    torch.cuda.synchronize()
    return blk, res


@pytest.mark.parametrize("name", ["tiny", "ragged", "sparse", "top1", "wide_ragged", "triclinic",
                                  "celllist"])
def test_train_grad_matches_oracle(mlip, name):
    cfg = synth.CONFIGS[name]
    inp = synth.make_inputs(cfg)
    Ebar, Fbar = _upstreams(cfg)
    _say(f"{name}: oracle (N={cfg.n_atoms})")
    g = OG.radius_graph(inp["pos"], inp["cell"], inp["struct_ptr"], inp["cutoff"])
    ref = TR.loss_grads(inp, g, Ebar, Fbar.astype(np.float64))
    _say(f"{name}: GPU (E={g['src'].size}, De={cfg.d_edge}, Dn={cfg.d_node}, H={cfg.d_hidden}, "
         f"X={cfg.n_experts}, k={cfg.top_k})")
    blk, res = _gpu(mlip, inp, Ebar, Fbar)
    errs = {k: rel(res[k], ref[k]) for k in KEYS}
    errs["F"] = rel(-blk.vjp["grad_pos"], ref["F"])
    _say(f"{name}: errors {errs}")
    bad = {k: e for k, e in errs.items() if not e <= TOL}
    assert not bad, bad


def test_train_grad_deterministic(mlip):
    cfg = synth.CONFIGS["ragged"]
    inp = synth.make_inputs(cfg)
    Ebar, Fbar = _upstreams(cfg)
    _say("determinism: ragged, two calls")
    blk, res = _gpu(mlip, inp, Ebar, Fbar)
    first = {k: res[k].clone() for k in KEYS}
    res2 = blk.train_grad(torch.tensor(Ebar, dtype=torch.float64, device="cuda"),
                          torch.from_numpy(Fbar).to("cuda"))
    torch.cuda.synchronize()
    for k in KEYS:
        assert torch.equal(first[k], res2[k]), k


def test_train_grad_empty_system(mlip):
    cfg = synth.CONFIGS["tiny"]
    inp = synth.make_inputs(cfg)
    inp["pos"] = inp["pos"][:0]
    inp["z"] = inp["z"][:0]
    inp["h"] = inp["h"][:0]
    inp["struct_ptr"] = np.array([0, 0], np.int32)
    _say("empty system")
    blk, res = _gpu(mlip, inp, np.array([1.5]), np.zeros((0, 3), np.float32))
    for k in KEYS:
        assert not torch.any(res[k] != 0), k
    assert res["d_W1"].shape == tuple(inp["W1"].shape)
