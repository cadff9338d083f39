"""Pins of the oracle's complete block: MoE0, neighbour attention, MoE1 (CPU only).

What fixes each piece independently of the oracle itself:
  * the envelope-weighted softmax equals scipy's softmax of (score + log f_c);
  * one neighbour per atom (a dimer) makes every weight 1, and a zero query
    makes the weights f_c / sum f_c: both reduce the attention to the plain
    aggregation of ``oracle.block`` (itself pinned by a closed form);
  * relabelling heads (consistently in W_qkv, Wa_e and W_o) and permuting
    channels inside a head change nothing, while moving one channel to another
    head does: the head split is where the definition puts it;
  * float64 central differences of the energy and of a random loss pin the
    whole hand-derived VJP (positions, node features, strain);
  * translation, rotation and permutation invariance; sum of forces = 0;
  * a neighbour crossing r_c changes the energy continuously.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

from element_routed_moe_amd import synth
from oracle import attention as A
from oracle import block as B
from oracle import graph as G


def _inputs(name="tiny", q_scale=6.0):
    """Complete-block inputs; the query weights are scaled up so that the
    softmax is far from uniform (otherwise the weights are close to f_c / sum)."""
    cfg = synth.CONFIGS[name]
    inp = synth.make_full_inputs(cfg)
    Da = cfg.d_attn
    W = inp["W_qkv"].astype(np.float64)
    W[:, :Da] *= q_scale
    inp["W_qkv"] = W
    return cfg, inp


def _graph(inp):
    return G.radius_graph(inp["pos"], inp["cell"], inp["struct_ptr"], inp["cutoff"])


def _loss(inp, g_up, **kw):
    q = dict(inp)
    q.update({k: v for k, v in kw.items() if v is not None})
    gr = _graph(q)
    return float(np.sum(A.full_block_forward(q, gr)["h2"] * g_up))


# ------------------------------------------------------------ softmax ----
def test_weighted_softmax_is_softmax_of_score_plus_log_envelope():
    cfg, inp = _inputs()
    g = _graph(inp)
    fw = A.full_block_forward(inp, g)["att"]
    assert np.all(fw["f"] > 0)          # every pair strictly inside r_c here
    s, f, alpha = fw["s"], fw["f"], fw["alpha"]
    spread = 0.0
    for i in range(cfg.n_atoms):
        rows = np.nonzero(g["recv"] == i)[0]
        ref = softmax(s[rows] + np.log(f[rows])[:, None], axis=0)
        assert np.allclose(alpha[rows], ref, rtol=0, atol=1e-14)
        spread = max(spread, float(alpha[rows].max() / alpha[rows].mean()))
    assert spread > 5.0                 # the test case is far from uniform weights


def test_empty_rows_give_zero_output():
    cfg = synth.CONFIGS["sparse"]
    inp = synth.make_full_inputs(cfg)
    g = _graph(inp)
    fw = A.full_block_forward(inp, g)
    deg = np.bincount(g["recv"], minlength=cfg.n_atoms)
    assert np.any(deg == 0)
    iso = deg == 0
    assert np.all(fw["att"]["o"][iso] == 0.0)
    assert np.allclose(fw["att"]["u"][iso], fw["att"]["h0"][iso], atol=0)


# ---------------------------------------------------- special cases ------
def _dimer_inputs(r):
    cfg = synth.CONFIGS["tiny"]
    inp = synth.make_full_inputs(cfg)
    L = 30.0
    pos = np.array([[10.0, 10.0, 10.0], [10.0 + r, 10.0, 10.0]], np.float64)
    q = dict(inp, pos=pos, cell=np.diag([L, L, L])[None].astype(np.float64),
             struct_ptr=np.array([0, 2], np.int32), z=inp["z"][:2], h=inp["h"][:2])
    return q


def test_single_neighbour_reduces_to_aggregation():
    inp = _dimer_inputs(2.7)
    g = _graph(inp)
    assert g["src"].size == 2
    rc = B._cutoff(inp)
    fw = A.attention_forward(inp["h"].astype(np.float64), g, inp["W_qkv"], inp["Wa_e"],
                             inp["W_o"], int(inp["n_heads"]), rc)
    assert np.allclose(fw["alpha"], 1.0, atol=1e-15)
    v = fw["v"]
    e = B.edge_embedding(g["r"], inp["Wa_e"], rc)
    ref = B.aggregate(e, v, g["recv"], g["src"], 2)
    assert np.allclose(fw["o"], ref, atol=1e-14)


def test_zero_query_is_envelope_weighted_mean():
    cfg, inp = _inputs()
    Da = cfg.d_attn
    W = inp["W_qkv"].copy()
    W[:, :Da] = 0.0
    inp["W_qkv"] = W
    g = _graph(inp)
    rc = B._cutoff(inp)
    h0 = np.asarray(inp["h"], np.float64)
    fw = A.attention_forward(h0, g, W, inp["Wa_e"], inp["W_o"], cfg.n_heads, rc)
    f = B.envelope(g["r"], rc)
    Z = np.bincount(g["recv"], weights=f, minlength=cfg.n_atoms)
    e = B.edge_embedding(g["r"], inp["Wa_e"], rc) * (f / Z[g["recv"]])[:, None]
    ref = B.aggregate(e, fw["v"], g["recv"], g["src"], cfg.n_atoms)
    assert np.allclose(fw["o"], ref, atol=1e-13)


def test_head_relabelling_and_in_head_permutation():
    cfg, inp = _inputs()
    g = _graph(inp)
    rc = B._cutoff(inp)
    nh, Da = cfg.n_heads, cfg.d_attn
    dh = Da // nh
    h0 = np.asarray(inp["h"], np.float64)

    def run(perm):
        W = inp["W_qkv"]
        Wp = np.concatenate([W[:, :Da][:, perm], W[:, Da:2 * Da][:, perm], W[:, 2 * Da:][:, perm]], 1)
        return A.attention_forward(h0, g, Wp, inp["Wa_e"][:, perm], inp["W_o"][perm], nh, rc)["u"]

    u0 = run(np.arange(Da))
    rng = np.random.default_rng(3)
    heads = rng.permutation(nh)
    within = np.concatenate([h * dh + rng.permutation(dh) for h in heads])
    assert np.allclose(run(within), u0, atol=1e-12)
    # moving one channel into another head is a different model
    cross = np.arange(Da)
    cross[[0, dh]] = cross[[dh, 0]]
    cross[[1, dh + 1]] = cross[[dh + 1, 1]]
    assert np.max(np.abs(run(cross) - u0)) > 1e-6


# ------------------------------------------------------------- gradient ---
@pytest.mark.parametrize("kind", ["energy", "random"])
def test_vjp_positions_fd(kind):
    cfg, inp = _inputs()
    g = _graph(inp)
    fw = A.full_block_forward(inp, g)
    g_up = synth.upstream_grad(cfg, inp, kind).astype(np.float64)
    v = A.full_block_vjp(inp, g, fw, g_up)
    pos = inp["pos"].astype(np.float64)
    step = 1e-5
    idx = [(i, c) for i in range(cfg.n_atoms) for c in range(3)]
    if kind == "random":
        idx = idx[::5]
    ref, got = [], []
    for i, c in idx:
        p1 = pos.copy(); p1[i, c] += step
        p2 = pos.copy(); p2[i, c] -= step
        ref.append((_loss(inp, g_up, pos=p1) - _loss(inp, g_up, pos=p2)) / (2 * step))
        got.append(v["grad_pos"][i, c])
    ref, got = np.array(ref), np.array(got)
    assert np.max(np.abs(got - ref)) <= 1e-6 * np.max(np.abs(ref))
    assert np.max(np.abs(v["grad_pos"].sum(0))) < 1e-11 * np.max(np.abs(v["grad_pos"]))


def test_vjp_features_directional_fd():
    cfg, inp = _inputs()
    g = _graph(inp)
    fw = A.full_block_forward(inp, g)
    g_up = synth.upstream_grad(cfg, inp, "random").astype(np.float64)
    v = A.full_block_vjp(inp, g, fw, g_up)
    rng = np.random.default_rng(6)
    h = inp["h"].astype(np.float64)
    for _ in range(3):
        dirn = rng.standard_normal(h.shape)
        step = 1e-5
        fd = (_loss(inp, g_up, h=h + step * dirn) - _loss(inp, g_up, h=h - step * dirn)) / (2 * step)
        an = float(np.sum(v["grad_h"] * dirn))
        assert abs(fd - an) <= 1e-7 * abs(an)


@pytest.mark.parametrize("name", ["tiny", "ragged"])
def test_strain_gradient_fd(name):
    cfg, inp = _inputs(name)
    g = _graph(inp)
    fw = A.full_block_forward(inp, g)
    g_up = synth.upstream_grad(cfg, inp, "random").astype(np.float64)
    v = A.full_block_vjp(inp, g, fw, g_up)
    pos = inp["pos"].astype(np.float64)
    cell = inp["cell"].astype(np.float64)
    sp = inp["struct_ptr"]
    step = 1e-6
    for b in range(cfg.n_structs):
        if sp[b + 1] - sp[b] < 2:
            continue
        gs = v["grad_strain"][b]
        fd = np.zeros((3, 3))
        for a in range(3):
            for c in range(3):
                vals = []
                for sgn in (1.0, -1.0):
                    F = np.eye(3)
                    F[a, c] += sgn * step
                    p = pos.copy()
                    p[sp[b]:sp[b + 1]] = pos[sp[b]:sp[b + 1]] @ F.T
                    cl = cell.copy()
                    cl[b] = cell[b] @ F.T
                    vals.append(_loss(inp, g_up, pos=p, cell=cl))
                fd[a, c] = (vals[0] - vals[1]) / (2 * step)
        assert np.max(np.abs(fd - gs)) <= 2e-6 * np.max(np.abs(gs)), (b, fd, gs)
    assert np.allclose(
        np.stack([v["atom_virial"][sp[b]:sp[b + 1]].sum(0) for b in range(cfg.n_structs)]),
        B.voigt(v["grad_strain"]), atol=1e-10 * np.max(np.abs(v["grad_strain"])))


def test_invariances():
    cfg, inp = _inputs()
    E0 = A.full_energy(inp)[0]
    N = cfg.n_atoms
    L = float(inp["cell"][0, 0, 0])
    pos = np.mod(inp["pos"].astype(np.float64) + np.array([1.25, -2.5, 3.0625]), L)
    assert abs(A.full_energy(inp, pos=pos)[0] - E0) <= 1e-12 * abs(E0)
    Q, _ = np.linalg.qr(np.random.default_rng(9).standard_normal((3, 3)))
    posR = inp["pos"].astype(np.float64) @ Q.T
    cellR = inp["cell"].astype(np.float64) @ Q.T
    assert abs(A.full_energy(inp, pos=posR, cell=cellR)[0] - E0) <= 1e-12 * abs(E0)
    perm = np.random.default_rng(10).permutation(N)
    q = dict(inp, pos=inp["pos"][perm], z=inp["z"][perm], h=inp["h"][perm])
    gq, g0 = _graph(q), _graph(inp)
    fq, f0 = A.full_block_forward(q, gq), A.full_block_forward(inp, g0)
    assert abs(fq["E"][0] - E0) <= 1e-12 * abs(E0)
    assert np.allclose(fq["eps"], f0["eps"][perm], atol=1e-12)
    vq = A.full_block_vjp(q, gq, fq, synth.upstream_grad(cfg, q, "energy").astype(np.float64))
    v0 = A.full_block_vjp(inp, g0, f0, synth.upstream_grad(cfg, inp, "energy").astype(np.float64))
    assert np.allclose(vq["grad_pos"], v0["grad_pos"][perm], atol=1e-10)


def test_energy_continuous_across_cutoff():
    """A third atom moved through r_c of the first: the energy changes by
    O(delta^2) across the cutoff (envelope-weighted softmax), while the same
    move inside the sphere changes it by O(delta)."""
    cfg = synth.CONFIGS["tiny"]
    inp = synth.make_full_inputs(cfg)
    rc = float(np.float32(inp["cutoff"]))
    L = 40.0
    base = np.array([[10.0, 10.0, 10.0], [12.5, 10.0, 10.0], [0.0, 10.0, 10.0]])

    def energy(x):
        pos = base.copy()
        pos[2, 0] = 10.0 - x           # distance x from atom 0, > r_c from atom 1
        q = dict(inp, pos=pos, cell=np.diag([L, L, L])[None].astype(np.float64),
                 struct_ptr=np.array([0, 3], np.int32), z=inp["z"][:3], h=inp["h"][:3])
        return A.full_energy(q)[0]

    d = 1e-4
    jump = abs(energy(rc + d) - energy(rc - d))
    jump10 = abs(energy(rc + 10 * d) - energy(rc - 10 * d))
    inside = abs(energy(rc - 0.3 + d) - energy(rc - 0.3 - d))
    assert inside > 0
    assert jump < 1e-3 * inside
    # quadratic in the distance to r_c (f_c ~ (pi delta / r_c)^2 / 4 there)
    assert 50 < jump10 / jump < 200


@pytest.mark.parametrize("name", ["tiny", "ragged", "top1"])
def test_local_full_oracle_matches_full(name):
    from oracle.local import LocalFullBlock
    cfg = synth.CONFIGS[name]
    inp = synth.make_full_inputs(cfg)
    g = _graph(inp)
    f = A.full_block_forward(inp, g)
    g_up = synth.upstream_grad(cfg, inp, "random").astype(np.float64)
    v = A.full_block_vjp(inp, g, f, g_up)
    atoms = np.random.default_rng(0).choice(cfg.n_atoms, size=min(8, cfg.n_atoms), replace=False)
    lb = LocalFullBlock(inp)
    lf = lb.forward(atoms)
    assert np.allclose(lf["h2"], f["h2"][atoms], atol=1e-10)
    assert np.allclose(lf["eps"], f["eps"][atoms], atol=1e-10)
    lv = lb.vjp(atoms, g_up)
    assert np.allclose(lv["grad_h"], v["grad_h"][atoms], atol=1e-10)
    assert np.allclose(lv["grad_pos"], v["grad_pos"][atoms], atol=1e-10)
    assert np.allclose(lv["atom_virial"], v["atom_virial"][atoms], atol=1e-10)
