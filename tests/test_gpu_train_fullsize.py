"""GPU parity of the training gradient at the full S, M and L widths, in the
launch configuration the benchmark times (every structure of the batch).

Weight gradients are sums over the whole batch, so the loss is placed on the
first structure alone: dL/dE and dL/dF are seeded random there and zero on
every other structure, which then contributes exactly nothing.  The oracle
(``oracle.train``) runs that one structure and is compared with the GPU on
W_e, W_d, W_u, the routing logits, w_r, dL/dh (first structure; zero
elsewhere), the forces, and W1 / W2 of four experts: the most loaded in the
structure, the lowest- and highest-numbered used ones and one it does not use
(gradient 0).  Tolerance: max|gpu - oracle| / max|oracle| <= 2e-4 per tensor.
"""
import sys

import numpy as np
import pytest

from element_routed_moe_amd import synth
from oracle import block as OB
from oracle import graph as OG
from oracle import train as TR

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-4


def _say(msg):
    print(f"[gpu-train-fullsize] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mlip():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from element_routed_moe_amd import mlip as m
    return m


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    m = np.max(np.abs(b))
    return float(np.max(np.abs(a))) if m == 0 else float(np.max(np.abs(a - b)) / m)


@pytest.mark.parametrize("name", ["S", "M", "L"])
def test_train_grad_fullsize(mlip, name):
    cfg = synth.CONFIGS[name]
    _say(f"{name}: inputs")
    inp = synth.make_inputs(cfg)
    n0 = int(inp["struct_ptr"][1])
    rng = np.random.default_rng(31)
    Ebar = np.zeros(cfg.n_structs)
    Ebar[0] = 1.3
    Fbar = np.zeros((cfg.n_atoms, 3), np.float32)
    Fbar[:n0] = rng.standard_normal((n0, 3))
    _say(f"{name}: GPU (N={cfg.n_atoms}, {cfg.n_structs} structures)")
    blk = mlip.Block(inp, device="cuda", train=True).step()
    res = blk.train_grad(torch.tensor(Ebar, dtype=torch.float64, device="cuda"),
                         torch.from_numpy(Fbar).to("cuda"))
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in res.items()}
    F_gpu = -blk.vjp["grad_pos"][:n0].cpu().numpy()
    del blk, res
    torch.cuda.empty_cache()

    q = dict(inp)
    q["pos"], q["z"], q["h"] = inp["pos"][:n0], inp["z"][:n0], inp["h"][:n0]
    q["cell"], q["struct_ptr"] = inp["cell"][:1], inp["struct_ptr"][:2]
    g = OG.radius_graph(q["pos"], q["cell"], q["struct_ptr"], q["cutoff"])
    topk, _ = OB.route(inp["logits"], cfg.top_k)
    load = np.bincount(topk[q["z"]].ravel(), minlength=cfg.n_experts)
    used = np.nonzero(load)[0]
    sel = [int(np.argmax(load)), int(used[0]), int(used[-1])]
    if np.any(load == 0):
        sel.append(int(np.nonzero(load == 0)[0][0]))
    _say(f"{name}: oracle on structure 0 ({n0} atoms, {g['src'].size} edges), experts {sel}")
    ref = TR.loss_grads(q, g, Ebar[:1], Fbar[:n0].astype(np.float64), experts=sel)

    errs = {k: rel(got[k], ref[k]) for k in ("d_W_e", "d_W_d", "d_W_u", "d_logits", "d_w_r")}
    errs["d_h"] = rel(got["d_h"][:n0], ref["d_h"])
    errs["d_h_rest"] = float(np.max(np.abs(got["d_h"][n0:]))) if cfg.n_atoms > n0 else 0.0
    errs["F"] = rel(F_gpu, ref["F"])
    for n in ("W1", "W2"):
        for q_, x in enumerate(sel):
            errs[f"d_{n}[{x}]"] = rel(got["d_" + n][x], ref["d_" + n][q_])
    _say(f"{name}: errors {errs}")
    assert errs.pop("d_h_rest") == 0.0
    bad = {k: e for k, e in errs.items() if not e <= TOL}
    assert not bad, bad
