"""GPU parity of the complete block (Tri -> MoE0 -> neighbour attention -> MoE1) at
the full workload sizes (S, M, L widths and the 262144-atom share), in the
launch configuration the benchmark times.

The oracle cannot run these end to end, so it checks the MoE0 routing and
dispatch tables bit for bit (cheap at any size), and sampled atoms of h0, u,
h', eps, dL/dh, dL/dx and the per-atom virial, each computed by the oracle
from the atom's own two-hop neighbourhood (``oracle.local.LocalFullBlock``),
within 2e-4 of the sample's max-abs; per-structure energies and strain
gradients are checked as float64 sums of the per-atom values.
"""
import sys

import numpy as np
import pytest

from element_routed_moe_amd import synth
from oracle import block as OB
from oracle.local import LocalFullBlock

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-4


def _say(msg):
    print(f"[gpu-full-block-fullsize] {msg}", flush=True)
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
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _sample_atoms(cfg, z, n, seed):
    rng = np.random.default_rng(seed)
    picks = {0, cfg.n_atoms - 1}
    counts = np.bincount(z, minlength=cfg.n_types)
    present = np.nonzero(counts)[0]
    for t in (present[np.argmax(counts[present])], present[np.argmin(counts[present])]):
        picks.add(int(np.nonzero(z == t)[0][0]))
    while len(picks) < n:
        picks.add(int(rng.integers(0, cfg.n_atoms)))
    return sorted(picks)[:n]


@pytest.mark.parametrize("name", ["S", "M", "L", "share"])
def test_full_block_fullsize(mlip, name):
    cfg = synth.CONFIGS[name]
    _say(f"{name}: generating inputs ({cfg.n_atoms} atoms, {cfg.n_heads} heads x "
         f"{cfg.d_attn // cfg.n_heads})")
    inp = synth.make_full_inputs(cfg)
    gup = synth.upstream_grad(cfg, inp, "energy")
    _say(f"{name}: GPU step")
    blk = mlip.FullBlock(inp, device="cuda", grad_out=gup).step()
    torch.cuda.synchronize()
    _say(f"{name}: {blk.graph['n_edges']} edges; MoE0 tables")
    topk0, gate0 = OB.route(inp["logits0"], cfg.top_k)
    exp_off, tok_atom, slot = OB.dispatch_tables(inp["z"], topk0, cfg.n_experts)
    assert np.array_equal(blk.moe0["topk"].cpu().numpy(), topk0)
    assert rel(blk.moe0["gate"].cpu().numpy(), gate0) <= 1e-6
    assert np.array_equal(blk.moe0["exp_off"].cpu().numpy(), exp_off)
    assert np.array_equal(blk.moe0["tok_atom"].cpu().numpy(), tok_atom)
    assert np.array_equal(blk.moe0["slot"].cpu().numpy(), slot)

    lb = LocalFullBlock(inp)
    fwd_atoms = _sample_atoms(cfg, inp["z"], 8, seed=2)
    _say(f"{name}: oracle forward at {len(fwd_atoms)} atoms")
    lf = lb.forward(fwd_atoms)
    errs = {"h_T": rel(blk.tri["h_T"].cpu().numpy()[fwd_atoms], lb.hT(fwd_atoms)),
            "h0": rel(blk.moe0["h_out"].cpu().numpy()[fwd_atoms], lb.h0(fwd_atoms)),
            "u": rel(blk.att["u"].cpu().numpy()[fwd_atoms], lf["u"]),
            "h_out": rel(blk.moe["h_out"].cpu().numpy()[fwd_atoms], lf["h2"]),
            "eps": rel(blk.ro["eps"].cpu().numpy()[fwd_atoms], lf["eps"])}
    # one VJP sample at the share size: its neighbourhood reaches three hops
    # (thousands of MoE0 rows in the float64 oracle)
    vjp_atoms = _sample_atoms(cfg, inp["z"], 1 if name == "share" else 3, seed=3)
    _say(f"{name}: oracle VJP at {len(vjp_atoms)} atoms")
    lv = lb.vjp(vjp_atoms, gup)
    errs["grad_h"] = rel(blk.grad_h.cpu().numpy()[vjp_atoms], lv["grad_h"])
    errs["grad_pos"] = rel(blk.avjp["grad_pos"].cpu().numpy()[vjp_atoms], lv["grad_pos"])
    errs["atom_virial"] = rel(blk.avjp["atom_virial"].cpu().numpy()[vjp_atoms], lv["atom_virial"])
    sp = inp["struct_ptr"]
    eps = blk.ro["eps"].cpu().numpy().astype(np.float64)
    e_ref = np.array([eps[sp[b]:sp[b + 1]].sum() for b in range(cfg.n_structs)])
    errs["energy_sum"] = rel(blk.ro["energy"].cpu().numpy(), e_ref)
    av = blk.avjp["atom_virial"].cpu().numpy().astype(np.float64)
    gs_ref = np.stack([av[sp[b]:sp[b + 1]].sum(0) for b in range(cfg.n_structs)])
    errs["strain_sum"] = rel(blk.avjp["grad_strain"].cpu().numpy(), gs_ref)
    _say(f"{name}: errors {errs}")
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, bad
    # forces of each periodic structure sum to zero (translation invariance)
    gp = blk.avjp["grad_pos"].cpu().numpy().astype(np.float64)
    tot = np.stack([gp[sp[b]:sp[b + 1]].sum(0) for b in range(cfg.n_structs)])
    assert np.max(np.abs(tot)) <= 1e-4 * np.max(np.abs(gp)) * np.sqrt(np.max(np.diff(sp)))
