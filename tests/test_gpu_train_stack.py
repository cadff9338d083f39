"""GPU parity of the training gradient through two chained blocks on one
graph (h^(1) = Block_0(h^(0)), h^(2) = Block_1(h^(1)), readout on h^(2)),
against ``oracle.train.stack_loss_grads``.

This drives the entry points the way a stack uses them: forwards in order,
input gradients in reverse with the force seed (the lower block's upstream is
the upper block's input gradient), forward tangents in order (the upper
block's h_dot is the lower block's h_out_dot), tangents of the input
gradients in reverse (the lower block's grad_out_dot is the upper block's
grad_h_dot).  It covers the paths a single block never takes: a non-zero
h_dot (s_dot, the second sum of the aggregation tangent, the two-term W_d
gradient) and a primal upstream that varies per atom.  Forces are the sum of
both blocks' position gradients (added here, on the host).
Tolerance: max|gpu - oracle| / max|oracle| <= 2e-4 per tensor.
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
    print(f"[gpu-train-stack] {msg}", flush=True)
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
    m = np.max(np.abs(b)) if b.size else 0.0
    return float(np.max(np.abs(a))) if m == 0 else float(np.max(np.abs(a - b)) / m)


@pytest.mark.parametrize("name", ["tiny", "ragged", "wide_ragged"])
def test_two_block_train_grad(mlip, name):
    cfg = synth.CONFIGS[name]
    inp = synth.make_inputs(cfg)
    other = synth.make_inputs(cfg, seed=cfg.seed + 1000)
    blocks = [{n: inp[n] for n in TR.BLOCK_PARAMS}, {n: other[n] for n in TR.BLOCK_PARAMS}]
    rng = np.random.default_rng(23)
    Ebar = rng.standard_normal(cfg.n_structs)
    Fbar = rng.standard_normal((cfg.n_atoms, 3)).astype(np.float32)
    _say(f"{name}: oracle (N={cfg.n_atoms})")
    g_ref = OG.radius_graph(inp["pos"], inp["cell"], inp["struct_ptr"], inp["cutoff"])
    ref = TR.stack_loss_grads(inp, g_ref, blocks, Ebar, Fbar.astype(np.float64))

    dev = "cuda"
    f32 = torch.float32
    up = lambda x, dt=f32: torch.from_numpy(np.ascontiguousarray(x)).to(device=dev, dtype=dt)
    pos, cell, sp, z = up(inp["pos"]), up(inp["cell"]), up(inp["struct_ptr"], torch.int32), up(inp["z"], torch.int32)
    w_r = up(inp["w_r"])
    P = [{n: up(b[n]) for n in TR.BLOCK_PARAMS} for b in blocks]
    rc, k = float(inp["cutoff"]), cfg.top_k
    _say(f"{name}: GPU forward / forces")
    g = mlip.mlip_build_graph(pos, cell, sp, rc)
    hs, aggs, moes = [up(inp["h"])], [], []
    for p in P:
        agg = mlip.mlip_aggregate(g, hs[-1], p["W_e"], p["W_d"], p["W_u"], rc, store_e=False)
        moe = mlip.mlip_moe_forward(agg["u"], z, p["logits"], p["W1"], p["W2"], k)
        aggs.append(agg)
        moes.append(moe)
        hs.append(moe["h_out"])
    seed = mlip.mlip_readout_vjp(w_r, sp, cfg.n_atoms)          # the force seed: w_r on every atom
    wt = lambda b: (P[b]["W_e"], P[b]["W_d"], P[b]["W_u"], P[b]["W1"], P[b]["W2"])
    vjp1 = mlip.mlip_block_vjp(g, aggs[1], moes[1], z, *wt(1), rc, k, seed, struct_ptr=sp, keep=True)
    # the lower block's upstream is the upper block's input gradient
    vjp0 = mlip.mlip_block_vjp(g, aggs[0], moes[0], z, *wt(0), rc, k, vjp1["grad_h"], struct_ptr=sp, keep=True)
    vjps = [vjp0, vjp1]
    grad_out = [vjp1["grad_h"], seed]
    F = -(vjps[0]["grad_pos"] + vjps[1]["grad_pos"])

    _say(f"{name}: GPU tangents")
    Fb = up(Fbar)
    Eb = torch.tensor(Ebar, dtype=torch.float64, device=dev)
    jvps, h_dot = [], None
    for b in (0, 1):
        jvps.append(mlip.mlip_block_jvp(g, aggs[b], moes[b], z, *wt(b), rc, k, Fb, h_dot=h_dot))
        h_dot = jvps[-1]["h_out_dot"]
    g_dot = mlip.mlip_readout_vjp(w_r, sp, cfg.n_atoms, grad_energy=Eb)
    tans = [None, None]
    for b in (1, 0):
        tans[b] = mlip.mlip_block_tangent_vjp(g, hs[b], aggs[b], moes[b], jvps[b], vjps[b], z, *wt(b), rc, k, Fb,
                                              grad_out[b], grad_out_dot=g_dot,
                                              h_dot=jvps[0]["h_out_dot"] if b == 1 else None)
        g_dot = tans[b]["grad_h_dot"]
    d_w_r = mlip.mlip_readout_grad(hs[-1], sp, grad_energy=Eb, h_out_dot=jvps[1]["h_out_dot"])
    torch.cuda.synchronize()

    errs = {"F": rel(F, ref["F"]), "d_h": rel(tans[0]["grad_h_dot"], ref["d_h"]), "d_w_r": rel(d_w_r, ref["d_w_r"])}
    for b in (0, 1):
        for n in TR.BLOCK_PARAMS:
            errs[f"{b}:d_{n}"] = rel(tans[b]["d_" + n], ref["blocks"][b]["d_" + n])
    _say(f"{name}: errors {errs}")
    bad = {kk: e for kk, e in errs.items() if not e <= TOL}
    assert not bad, bad
