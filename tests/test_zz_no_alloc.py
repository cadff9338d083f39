"""mlip_aggregate_static (library-owned scratch, no workspace argument) against
mlip_aggregate (caller workspace): the same kernels run on the same inputs, so
the outputs must agree bit for bit.  Two calls in a row on one GPU, the
second on a smaller input, show that the shared scratch carries nothing
from one call into the next."""
import sys

import numpy as np
import pytest

from element_routed_moe_amd import synth
from oracle import block as OB
from oracle import graph as OG

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mlip():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from element_routed_moe_amd import mlip as m
    return m


def _inputs(mlip, name):
    cfg = synth.CONFIGS[name]
    inp = synth.make_inputs(cfg)
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    g = mlip.mlip_build_graph(t(inp["pos"]), t(inp["cell"]), t(inp["struct_ptr"]), float(inp["cutoff"]))
    w = {k: t(inp[k]) for k in ("h", "W_e", "W_d", "W_u")}
    return cfg, inp, g, w


def _outputs(N, E, De, Dn, fill):
    dev = "cuda"
    return dict(e=torch.full((E, De), fill, dtype=torch.float32, device=dev),
                s=torch.full((N, De), fill, dtype=torch.float32, device=dev),
                u=torch.full((N, Dn), fill, dtype=torch.float32, device=dev))


@pytest.mark.parametrize("order", [("S", "ragged"), ("S_slice", "tiny")])
def test_static_matches_workspace(mlip, order):
    for name in order:
        cfg, inp, g, w = _inputs(mlip, name)
        N, E, De, Dn = cfg.n_atoms, g["n_edges"], cfg.d_edge, cfg.d_node
        _say(f"{name}: N={N} E={E} De={De} Dn={Dn}, scratch "
             f"{mlip._lib.mlip_aggregate_workspace_size(N, De, Dn)} bytes")
        ref = mlip.mlip_aggregate(g, w["h"], w["W_e"], w["W_d"], w["W_u"], cfg.cutoff,
                                  out=_outputs(N, E, De, Dn, 0.0))
        out = mlip.mlip_aggregate_static(g, w["h"], w["W_e"], w["W_d"], w["W_u"], cfg.cutoff,
                                         out=_outputs(N, E, De, Dn, float("nan")))
        torch.cuda.synchronize()
        for k in ("e", "s", "u"):
            assert torch.equal(out[k], ref[k]), (name, k)
        if N <= 512:
            # and both against the float64 oracle of s and u
            og = OG.radius_graph(inp["pos"], inp["cell"], inp["struct_ptr"], inp["cutoff"])
            f = OB.block_forward(inp, og)
            for k, key in (("s", "s"), ("u", "u"), ("e", "e")):
                a = out[k].cpu().numpy().astype(np.float64)
                assert np.max(np.abs(a - f[key])) <= 2e-4 * np.max(np.abs(f[key])), (name, k)


def test_static_rejects_oversize(mlip):
    """More scratch than the library holds: an error before any device work."""
    cfg, inp, g, w = _inputs(mlip, "tiny")
    N = 8192
    assert mlip._lib.mlip_aggregate_workspace_size(N, 384, 2560) > mlip.AGGREGATE_STATIC_MAX_BYTES
    dev = "cuda"
    h = torch.zeros((N, 2560), device=dev)
    W_e = torch.zeros((16, 384), device=dev)
    W_d = torch.zeros((2560, 384), device=dev)
    W_u = torch.zeros((384, 2560), device=dev)
    rp = torch.zeros(N + 1, dtype=torch.int32, device=dev)
    graph = dict(row_ptr=rp, src=None, geom=None, n_edges=0)
    out = dict(e=None, s=torch.zeros((N, 384), device=dev), u=torch.zeros((N, 2560), device=dev))
    with pytest.raises(mlip.MlipError) as ei:
        mlip.mlip_aggregate_static(graph, h, W_e, W_d, W_u, 5.0, out=out)
    assert ei.value.code == mlip.MLIP_ERR_UNSUPPORTED
    assert "scratch" in str(ei.value)
