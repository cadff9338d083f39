"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer outputs (graph, routing table, dispatch tables) must match bit for
bit.  Floating-point outputs must satisfy
    max |gpu - oracle| / max |oracle|  <=  2e-4
per tensor, the bound the block is specified to (float32 arithmetic against
a float64 oracle).
"""
import functools
import sys

import numpy as np
import pytest

from element_routed_moe_amd import synth
from oracle import block as OB
from oracle import graph as OG

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-4
SMALL = ["tiny", "ragged", "celllist", "sparse", "top1", "wide_ragged", "triclinic", "triclinic_cl"]


def _say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mlip():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from element_routed_moe_amd import mlip as m
    return m


def rel(gpu, ref):
    a = gpu.detach().cpu().numpy().astype(np.float64) if hasattr(gpu, "detach") else np.asarray(gpu, np.float64)
    b = np.asarray(ref, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if b.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@functools.lru_cache(maxsize=None)
def oracle_full(name, upstream):
    cfg = synth.CONFIGS[name]
    inp = synth.make_inputs(cfg)
    g = OG.radius_graph(inp["pos"], inp["cell"], inp["struct_ptr"], inp["cutoff"])
    f = OB.block_forward(inp, g)
    gup = synth.upstream_grad(cfg, inp, upstream)
    v = OB.block_vjp(inp, g, f, gup.astype(np.float64))
    tables = OB.dispatch_tables(inp["z"], f["topk"], cfg.n_experts)
    return cfg, inp, g, f, v, gup, tables


def run_gpu(mlip, inp, gup, store_e=True):
    blk = mlip.Block(inp, device="cuda", grad_out=gup, store_edge_features=store_e).step()
    torch.cuda.synchronize()
    return blk


@pytest.mark.parametrize("name", SMALL + ["S_slice"])
def test_graph_bit_exact(mlip, name):
    cfg, inp, g, *_ = oracle_full(name, "energy")
    _say(f"graph {name}: N={cfg.n_atoms} E={g['src'].size}")
    dev = "cuda"
    out = mlip.mlip_build_graph(torch.from_numpy(inp["pos"]).to(dev), torch.from_numpy(inp["cell"]).to(dev),
                                torch.from_numpy(inp["struct_ptr"]).to(dev), float(inp["cutoff"]))
    torch.cuda.synchronize()
    assert out["n_edges"] == g["src"].size
    assert np.array_equal(out["row_ptr"].cpu().numpy(), g["row_ptr"])
    assert np.array_equal(out["src"].cpu().numpy(), g["src"])
    sh = out["shift"].cpu().numpy()
    assert np.array_equal(sh[:, :3].astype(np.int64), g["shift"]) and np.all(sh[:, 3] == 0)
    assert np.array_equal(out["rev"].cpu().numpy(), g["rev"])
    geo = out["geom"].cpu().numpy()
    assert np.array_equal(geo, g["geom"]), np.max(np.abs(geo - g["geom"]))


@pytest.mark.parametrize("name", SMALL + ["S_slice"])
@pytest.mark.parametrize("upstream,store_e", [("energy", True), ("random", False)])
def test_block_parity(mlip, name, upstream, store_e):
    """store_e: the edge features are kept and compared, else the VJP rebuilds them."""
    cfg, inp, g, f, v, gup, (exp_off, tok_atom, slot) = oracle_full(name, upstream)
    _say(f"block {name} upstream={upstream} store_e={store_e}: N={cfg.n_atoms} E={g['src'].size} "
         f"De={cfg.d_edge} Dn={cfg.d_node} H={cfg.d_hidden} X={cfg.n_experts} k={cfg.top_k}")
    blk = run_gpu(mlip, inp, gup, store_e)
    # integer tables
    assert np.array_equal(blk.moe["topk"].cpu().numpy(), f["topk"])
    assert np.array_equal(blk.moe["exp_off"].cpu().numpy(), exp_off)
    assert np.array_equal(blk.moe["tok_atom"].cpu().numpy(), tok_atom)
    assert np.array_equal(blk.moe["slot"].cpu().numpy(), slot)
    assert not mlip.mlip_moe_status(blk.ws_moe)
    errs = {
        "gate": rel(blk.moe["gate"], f["gate"]),
        "s": rel(blk.agg["s"], f["s"]),
        "u": rel(blk.agg["u"], f["u"]),
        "h_out": rel(blk.moe["h_out"], f["h2"]),
        "eps": rel(blk.ro["eps"], f["eps"]),
        "energy": rel(blk.ro["energy"], f["E"]),
        "grad_h": rel(blk.vjp["grad_h"], v["grad_h"]),
        "grad_pos": rel(blk.vjp["grad_pos"], v["grad_pos"]),
        "atom_virial": rel(blk.vjp["atom_virial"], v["atom_virial"]),
        "grad_strain": rel(blk.vjp["grad_strain"], OB.voigt(v["grad_strain"])),
    }
    if store_e:
        errs["e"] = rel(blk.agg["e"], f["e"])
    else:
        assert blk.agg["e"] is None
    # the kept pre-activations, in dispatch order
    P_ref = np.concatenate([
        (np.asarray(f["u"])[tok_atom[exp_off[x]:exp_off[x + 1]]] @ inp["W1"][x].astype(np.float64))
        for x in range(cfg.n_experts)], axis=0) if cfg.n_atoms else np.zeros((0, cfg.d_hidden))
    errs["P"] = rel(blk.moe["P"], P_ref)
    _say(f"  errors {errs}")
    bad = {k: e for k, e in errs.items() if not e <= TOL}
    assert not bad, bad


def _rotated(inp, seed):
    """The same structures turned by a random rotation (cell rows and positions)."""
    Q, _ = np.linalg.qr(np.random.default_rng(seed).standard_normal((3, 3)))
    Q *= np.sign(np.linalg.det(Q))
    q = dict(inp)
    q["pos"] = (inp["pos"].astype(np.float64) @ Q.T).astype(np.float32)
    q["cell"] = (inp["cell"].astype(np.float64) @ Q.T).astype(np.float32)
    return q


@pytest.mark.parametrize("name,hand", [("tiny", 1), ("ragged", 1), ("celllist", -1)])
def test_general_cell_graph_and_rotation(mlip, name, hand):
    """Rotated cubic cells (nine non-zero entries; hand=-1 also reverses the
    row order, a left-handed basis): the graph matches the oracle bit for bit
    and the edge multiset and energy match those of the unrotated cells."""
    cfg = synth.CONFIGS[name]
    inp = synth.make_inputs(cfg)
    q = _rotated(inp, 7)
    if hand < 0:
        q["cell"] = np.ascontiguousarray(q["cell"][:, ::-1, :])
    _say(f"rotated {name} (hand {hand}): N={cfg.n_atoms}")
    g = OG.radius_graph(q["pos"], q["cell"], q["struct_ptr"], q["cutoff"])
    dev = "cuda"
    out = mlip.mlip_build_graph(torch.from_numpy(q["pos"]).to(dev), torch.from_numpy(q["cell"]).to(dev),
                                torch.from_numpy(q["struct_ptr"]).to(dev), float(q["cutoff"]))
    torch.cuda.synchronize()
    assert out["n_edges"] == g["src"].size
    assert np.array_equal(out["row_ptr"].cpu().numpy(), g["row_ptr"])
    assert np.array_equal(out["src"].cpu().numpy(), g["src"])
    assert np.array_equal(out["shift"].cpu().numpy()[:, :3].astype(np.int64), g["shift"])
    assert np.array_equal(out["rev"].cpu().numpy(), g["rev"])
    assert np.array_equal(out["geom"].cpu().numpy(), g["geom"])
    # same edges as the unrotated cell up to pairs within rounding of r_c
    g0 = OG.radius_graph(inp["pos"], inp["cell"], inp["struct_ptr"], inp["cutoff"])
    assert abs(g0["src"].size - g["src"].size) <= max(2, g0["src"].size // 10000)
    e0 = run_gpu(mlip, inp, None).ro["energy"].cpu().numpy()
    e1 = run_gpu(mlip, q, None).ro["energy"].cpu().numpy()
    assert np.max(np.abs(e1 - e0)) <= TOL * max(np.max(np.abs(e0)), 1e-30)


@pytest.mark.parametrize("name", ["ragged", "S_slice"])
def test_deterministic(mlip, name):
    """Two runs give the same bits (S_slice takes the full-width kernels: the tall paired expert GEMM,
    the split-K projections)."""
    cfg = synth.CONFIGS[name]
    inp = synth.make_inputs(cfg)
    gup = synth.upstream_grad(cfg, inp, "random")
    _say(f"determinism {name}")
    a = run_gpu(mlip, inp, gup)
    outs_a = [t.cpu().clone() for t in (a.agg["e"], a.agg["u"], a.moe["h_out"], a.vjp["grad_h"],
                                        a.vjp["grad_pos"], a.ro["energy"])]
    b = run_gpu(mlip, inp, gup)
    outs_b = [t.cpu() for t in (b.agg["e"], b.agg["u"], b.moe["h_out"], b.vjp["grad_h"],
                                b.vjp["grad_pos"], b.ro["energy"])]
    for x, y in zip(outs_a, outs_b):
        assert torch.equal(x, y)


def test_empty_system(mlip):
    _say("empty system")
    cfg = synth.CONFIGS["tiny"]
    inp = synth.make_inputs(cfg)
    q = dict(inp)
    q["pos"] = np.zeros((0, 3), np.float32)
    q["struct_ptr"] = np.array([0, 0], np.int32)
    q["z"] = np.zeros(0, np.int32)
    q["h"] = np.zeros((0, cfg.d_node), np.float32)
    blk = mlip.Block(q, device="cuda").step()
    torch.cuda.synchronize()
    assert blk.graph["n_edges"] == 0
    assert blk.ro["energy"].cpu().numpy().tolist() == [0.0]
    assert blk.vjp["grad_pos"].shape == (0, 3)


def test_input_errors(mlip):
    _say("input errors")
    cfg = synth.CONFIGS["tiny"]
    inp = synth.make_inputs(cfg)
    dev = "cuda"
    pos = torch.from_numpy(inp["pos"]).to(dev)
    cell = torch.from_numpy(inp["cell"]).to(dev)
    sp = torch.from_numpy(inp["struct_ptr"]).to(dev)
    bad = pos.clone()
    bad[3, 1] = 8.5                                # outside the 8 A cell
    with pytest.raises(mlip.MlipError) as ei:
        mlip.mlip_build_graph(bad, cell, sp, 5.0)
    assert ei.value.code == mlip.MLIP_ERR_INPUT
    flat = cell.clone()
    flat[0, 2] = flat[0, 0] + flat[0, 1]           # third row in the plane of the first two
    with pytest.raises(mlip.MlipError) as ei:
        mlip.mlip_build_graph(pos, flat, sp, 5.0)
    assert ei.value.code == mlip.MLIP_ERR_INPUT
    neg = cell.clone()
    neg[0, 1, 1] = -8.0                            # diagonal cell with a negative edge
    with pytest.raises(mlip.MlipError) as ei:
        mlip.mlip_build_graph(pos, neg, sp, 5.0)
    assert ei.value.code == mlip.MLIP_ERR_INPUT
    skew = cell.clone()
    skew[0, 1, 0] = 4.0                            # atoms with f_0 = x/8 - y/16 < 0 leave the cell
    with pytest.raises(mlip.MlipError) as ei:
        mlip.mlip_build_graph(pos, skew, sp, 5.0)
    assert ei.value.code == mlip.MLIP_ERR_INPUT
    # a too-small edge capacity is reported with the required count, then met
    g = mlip.mlip_build_graph(pos, cell, sp, 5.0, edge_capacity=10)
    assert g["n_edges"] > 10
    # element types outside [0, T) are clamped and reported
    q = dict(inp)
    q["z"] = inp["z"].copy()
    q["z"][5] = 17
    blk = mlip.Block(q, device="cuda").step()
    assert mlip.mlip_moe_status(blk.ws_moe)


def test_struct_ptr_errors(mlip):
    """A malformed structure table is rejected before it indexes anything; a
    valid build afterwards (same workspace) is unaffected."""
    _say("struct_ptr errors")
    cfg = synth.CONFIGS["ragged"]
    inp = synth.make_inputs(cfg)
    dev = "cuda"
    pos = torch.from_numpy(inp["pos"]).to(dev)
    cell = torch.from_numpy(inp["cell"]).to(dev)
    sp_ok = inp["struct_ptr"].astype(np.int32)
    N, B = cfg.n_atoms, cfg.n_structs
    ws = mlip._ws(mlip._lib.mlip_graph_workspace_size(N, B), dev)
    bads = []
    s = sp_ok.copy(); s[0] = 1; bads.append(s)                    # does not start at 0
    s = sp_ok.copy(); s[-1] = N - 1; bads.append(s)               # does not end at N
    s = sp_ok.copy(); s[-1] = N + 1000; bads.append(s)            # runs past the atoms
    s = sp_ok.copy(); s[1], s[2] = s[2] + 1, s[1]; bads.append(s)  # decreasing step
    s = sp_ok.copy(); s[2] = -5; bads.append(s)                   # negative entry
    for bad in bads:
        with pytest.raises(mlip.MlipError) as ei:
            mlip.mlip_build_graph(pos, cell, torch.from_numpy(bad).to(dev), float(inp["cutoff"]), ws=ws)
        assert ei.value.code == mlip.MLIP_ERR_INPUT
        assert "struct_ptr" in str(ei.value)
    g = OG.radius_graph(inp["pos"], inp["cell"], inp["struct_ptr"], inp["cutoff"])
    out = mlip.mlip_build_graph(pos, cell, torch.from_numpy(sp_ok).to(dev), float(inp["cutoff"]), ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(out["src"].cpu().numpy(), g["src"])
    assert np.array_equal(out["rev"].cpu().numpy(), g["rev"])
    # the readout clamps a table that runs past the atoms: same energies as the
    # clamped table, no read past eps
    h = torch.randn(N, 8, device=dev)
    w_r = torch.randn(8, device=dev)
    over = sp_ok.copy(); over[-1] = N + 77
    r1 = mlip.mlip_readout(h, w_r, torch.from_numpy(over).to(dev))
    r0 = mlip.mlip_readout(h, w_r, torch.from_numpy(sp_ok).to(dev))
    assert torch.equal(r1["energy"], r0["energy"])


def test_capacity_error_leaves_edges_untouched(mlip):
    """With too small an edge capacity the build writes only row_ptr: the fill
    and reverse passes check the capacity on the device."""
    _say("capacity error")
    import ctypes as C
    cfg = synth.CONFIGS["tiny"]
    inp = synth.make_inputs(cfg)
    dev = "cuda"
    pos = torch.from_numpy(inp["pos"]).to(dev)
    cell = torch.from_numpy(inp["cell"]).to(dev)
    sp = torch.from_numpy(inp["struct_ptr"]).to(dev)
    N = cfg.n_atoms
    cap = 100
    row_ptr = torch.empty(N + 1, dtype=torch.int32, device=dev)
    src = torch.full((cap,), -7, dtype=torch.int32, device=dev)
    shift = torch.full((cap, 4), 9, dtype=torch.int8, device=dev)
    rev = torch.full((cap,), -3, dtype=torch.int32, device=dev)
    geom = torch.full((cap, 4), 2.5, dtype=torch.float32, device=dev)
    ws = mlip._ws(mlip._lib.mlip_graph_workspace_size(N, 1), dev)
    ne = C.c_int64(0)
    rc = mlip._lib.mlip_build_graph(pos.data_ptr(), cell.data_ptr(), sp.data_ptr(), N, 1,
                                    float(inp["cutoff"]), cap, row_ptr.data_ptr(), src.data_ptr(),
                                    shift.data_ptr(), rev.data_ptr(), geom.data_ptr(), C.byref(ne),
                                    ws.data_ptr(), ws.numel(), mlip._stream())
    torch.cuda.synchronize()
    assert rc == mlip.MLIP_ERR_CAPACITY
    g = OG.radius_graph(inp["pos"], inp["cell"], inp["struct_ptr"], inp["cutoff"])
    assert ne.value == g["src"].size
    assert torch.all(row_ptr == 0)                 # an empty graph until the build succeeds
    assert torch.all(src == -7) and torch.all(shift == 9) and torch.all(rev == -3) and torch.all(geom == 2.5)


def test_async_graph_build(mlip):
    """mlip_build_graph_async gives the synchronous build's graph; on overflow the
    summary reports the count, the edges stay untouched and row_ptr is an empty
    graph, on which the aggregation runs as on a graph without edges."""
    _say("async graph build")
    cfg = synth.CONFIGS["ragged"]
    inp = synth.make_inputs(cfg)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    pos, cell, sp = t(inp["pos"]), t(inp["cell"]), t(inp["struct_ptr"])
    ref = mlip.mlip_build_graph(pos, cell, sp, float(inp["cutoff"]))
    E = ref["n_edges"]
    ws = mlip._ws(mlip._lib.mlip_graph_workspace_size(cfg.n_atoms, cfg.n_structs), "cuda")
    summary = torch.zeros(4, dtype=torch.int32, device="cuda")

    def buffers(cap):
        return dict(row_ptr=torch.full((cfg.n_atoms + 1,), -1, dtype=torch.int32, device="cuda"),
                    src=torch.full((cap,), -7, dtype=torch.int32, device="cuda"),
                    shift=torch.zeros((cap, 4), dtype=torch.int8, device="cuda"),
                    rev=torch.zeros(cap, dtype=torch.int32, device="cuda"),
                    geom=torch.zeros((cap, 4), dtype=torch.float32, device="cuda"))
    g = mlip.mlip_build_graph_async(pos, cell, sp, float(inp["cutoff"]), buffers(E + 100), summary, ws)
    torch.cuda.synchronize()
    assert mlip.mlip_graph_check(summary.cpu(), E + 100) == E
    for k in ("row_ptr", "src", "shift", "rev", "geom"):
        assert torch.equal(g[k][:E] if k != "row_ptr" else g[k], ref[k]), k
    small = buffers(E // 2)
    g2 = mlip.mlip_build_graph_async(pos, cell, sp, float(inp["cutoff"]), small, summary, ws)
    torch.cuda.synchronize()
    with pytest.raises(mlip.MlipError) as ei:
        mlip.mlip_graph_check(summary.cpu(), E // 2)
    assert ei.value.code == mlip.MLIP_ERR_CAPACITY and int(summary[0]) == E
    assert torch.all(g2["row_ptr"] == 0) and torch.all(g2["src"] == -7)
    h = t(inp["h"])
    agg = mlip.mlip_aggregate(g2, h, t(inp["W_e"]), t(inp["W_d"]), t(inp["W_u"]), float(inp["cutoff"]))
    torch.cuda.synchronize()
    assert torch.equal(agg["u"], h)                # no edges: no messages, u = h + 0 @ W_u


def test_block_steps_reuse_and_regrow_the_graph(mlip):
    """Step loops: the first step's build waits, later ones are queued without a
    wait; a later graph that outgrows its buffers is detected and the step is
    run again on a rebuilt graph.  Every step gives the first step's results."""
    cfg, inp, g, f, v, gup, _ = oracle_full("ragged", "random")
    _say("block step loop")
    blk = mlip.Block(inp, device="cuda", grad_out=gup).step()
    torch.cuda.synchronize()
    first = {k: blk.vjp[k].clone() for k in ("grad_h", "grad_pos")}
    first["h_out"] = blk.moe["h_out"].clone()
    assert blk.graph["n_edges"] == g["src"].size
    for it in range(3):
        if it == 1:   # shrink the kept buffers below the edge count: the queued build overflows
            st = blk.graph_state
            cap = st.graph["n_edges"] // 2
            st.graph["buffers"] = {k: (v[:cap] if k != "row_ptr" else v) for k, v in st.graph["buffers"].items()}
        blk.step()
        torch.cuda.synchronize()
        assert blk.graph["n_edges"] == g["src"].size
        assert np.array_equal(blk.graph["src"].cpu().numpy(), g["src"])
        assert torch.equal(blk.moe["h_out"], first["h_out"])
        for k in ("grad_h", "grad_pos"):
            assert torch.equal(blk.vjp[k], first[k]), (it, k)
    assert rel(blk.vjp["grad_pos"], v["grad_pos"]) <= TOL


def test_graph_reverse(mlip):
    """mlip_graph_reverse reproduces the build's reverse index, and reports a
    graph that is not symmetric or holds an out-of-range sender."""
    _say("graph reverse")
    cfg = synth.CONFIGS["ragged"]
    inp = synth.make_inputs(cfg)
    dev = "cuda"
    out = mlip.mlip_build_graph(torch.from_numpy(inp["pos"]).to(dev), torch.from_numpy(inp["cell"]).to(dev),
                                torch.from_numpy(inp["struct_ptr"]).to(dev), float(inp["cutoff"]))
    rev = mlip.mlip_graph_reverse(out["row_ptr"], out["src"], out["shift"])
    torch.cuda.synchronize()
    assert torch.equal(rev, out["rev"])
    rp = out["row_ptr"].cpu().numpy().astype(np.int64)
    src = out["src"].cpu().numpy()
    sh = out["shift"].cpu().numpy()
    # drop one edge of the longest row: its partner loses its reverse
    i = int(np.argmax(np.diff(rp)))
    e0 = int(rp[i])
    keep = np.ones(src.size, bool)
    keep[e0] = False
    rp2 = rp.copy()
    rp2[i + 1:] -= 1
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    with pytest.raises(mlip.MlipError) as ei:
        mlip.mlip_graph_reverse(t(rp2.astype(np.int32)), t(src[keep]), t(sh[keep]))
    assert ei.value.code == mlip.MLIP_ERR_INPUT and "symmetric" in str(ei.value)
    # a sender outside [0, N)
    src3 = src.copy()
    src3[e0] = cfg.n_atoms + 5
    with pytest.raises(mlip.MlipError) as ei:
        mlip.mlip_graph_reverse(out["row_ptr"], t(src3), out["shift"])
    assert ei.value.code == mlip.MLIP_ERR_INPUT and "range" in str(ei.value)
    # a row range past the edges
    rp4 = rp.copy().astype(np.int32)
    rp4[-1] = src.size + 100
    with pytest.raises(mlip.MlipError) as ei:
        mlip.mlip_graph_reverse(t(rp4), out["src"], out["shift"])
    assert ei.value.code == mlip.MLIP_ERR_INPUT


@pytest.mark.parametrize("name", ["ragged", "S_slice", "sparse"])
def test_fused_moe_forward_vjp_matches_separate_calls(mlip, name):
    """mlip_moe_forward_vjp (the forward's second expert GEMM and the gradient's
    first in one launch) + mlip_aggregate_vjp, as Block.step runs them, give
    bit for bit what mlip_moe_forward + mlip_block_vjp (and mlip_moe_vjp) give."""
    cfg = synth.CONFIGS[name]
    inp = synth.make_inputs(cfg)
    gup = synth.upstream_grad(cfg, inp, "random")
    _say(f"fused MoE forward+VJP {name}")
    blk = mlip.Block(inp, device="cuda", grad_out=gup, train=True).step()
    g, agg = blk.graph, blk.agg
    moe = mlip.mlip_moe_forward(agg["u"], blk.z, blk.logits, blk.W1, blk.W2, blk.top_k)
    vjp = mlip.mlip_block_vjp(g, agg, moe, blk.z, blk.W_e, blk.W_d, blk.W_u, blk.W1, blk.W2, blk.cutoff,
                              blk.top_k, blk.grad_out, struct_ptr=blk.struct_ptr, keep=True)
    ubar = mlip.mlip_moe_vjp(moe, blk.z, blk.W1, blk.W2, blk.grad_out)
    torch.cuda.synchronize()
    for k in ("topk", "gate", "exp_off", "tok_atom", "slot", "P", "h_out"):
        assert torch.equal(blk.moe[k], moe[k]), k
    assert torch.equal(blk.moe["grad_u"], ubar)
    assert torch.equal(blk.moe["grad_u"], vjp["ubar"]) and torch.equal(blk.moe["Q"], vjp["Q"])
    for k in ("grad_h", "grad_pos", "atom_virial", "grad_strain"):
        assert torch.equal(blk.vjp[k], vjp[k]), k
