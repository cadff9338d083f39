"""GPU checks of the split-K dense projections.

mlip_attention and mlip_tri take an optional workspace: with it their
K = d_node projection ([q|k|v] = h0 W_qkv, s = h W_s) is split over K when the
output has few tiles, the parts summed in a fixed order; without it the
projection runs in one pass.  On the S widths with 256 atoms (few tiles, so
the split applies) both calls must agree to FP32 rounding, repeat bit for bit,
and each agree with the float64 product to the usual 2e-4 of max-abs.  The
two sum the same 2560 products in different groupings (4 parts of 640, or one
pass), so they differ by rounding only: a few 1e-6 of max-abs was observed;
the bound used is 2e-5 for the projection and the outputs built on it.
"""
import ctypes as C
import sys

import numpy as np
import pytest

from element_routed_moe_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-split-k] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mlip():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from element_routed_moe_amd import mlip as m
    return m


def _rel(a, b):
    a = a.detach().cpu().numpy().astype(np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


@pytest.fixture(scope="module")
def setup(mlip):
    cfg = synth.CONFIGS["S_slice"]
    inp = synth.make_full_inputs(cfg)
    dev = "cuda"
    up = lambda x, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(x)).to(device=dev, dtype=dt)
    _say(f"S_slice: {cfg.n_atoms} atoms, d_node {cfg.d_node}, d_attn {cfg.d_attn}")
    g = mlip.mlip_build_graph(up(inp["pos"]), up(inp["cell"]), up(inp["struct_ptr"], torch.int32),
                              float(inp["cutoff"]))
    return cfg, inp, g, up


def _attention(mlip, g, h0, W_qkv, Wa_e, W_o, n_heads, rc, ws):
    N, Dn = h0.shape
    Da = W_o.shape[0]
    dev = h0.device
    out = dict(qkv=torch.empty((N, 3 * Da), device=dev), o=torch.empty((N, Da), device=dev),
               stats=torch.empty((N, n_heads, 2), device=dev), u=torch.empty((N, Dn), device=dev))
    p = lambda t: C.c_void_p(t.data_ptr())
    rc_ = mlip._lib.mlip_attention(p(g["row_ptr"]), p(g["src"]), p(g["geom"]), N, g["n_edges"], p(h0), p(W_qkv),
                                   p(Wa_e), p(W_o), Wa_e.shape[0], Dn, Da, n_heads, rc, p(out["qkv"]), p(out["o"]),
                                   p(out["stats"]), p(out["u"]), None if ws is None else p(ws),
                                   0 if ws is None else ws.numel(), C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc_ == 0, mlip._lib.mlip_last_error()
    return out


def _tri(mlip, g, h, W_s, W_ang, W_T, rc, ws):
    N, Dn = h.shape
    Dt = W_s.shape[1]
    dev = h.device
    out = dict(s=torch.empty((N, Dt), device=dev), tau=torch.empty((N, Dt), device=dev),
               h_T=torch.empty((N, Dn), device=dev))
    p = lambda t: C.c_void_p(t.data_ptr())
    rc_ = mlip._lib.mlip_tri(p(g["row_ptr"]), p(g["src"]), p(g["geom"]), N, g["n_edges"], p(h), p(W_s), p(W_ang),
                             p(W_T), W_ang.shape[0], Dn, Dt, rc, p(out["s"]), p(out["tau"]), p(out["h_T"]),
                             None if ws is None else p(ws), 0 if ws is None else ws.numel(),
                             C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc_ == 0, mlip._lib.mlip_last_error()
    return out


def test_attention_split_matches_unsplit(mlip, setup):
    cfg, inp, g, up = setup
    h0, W_qkv, Wa_e, W_o = up(inp["h"]), up(inp["W_qkv"]), up(inp["Wa_e"]), up(inp["W_o"])
    need = mlip._lib.mlip_attention_workspace_size(cfg.n_atoms, cfg.d_attn)
    assert need > 0, "S widths with 256 atoms have few tiles: the projection must be split"
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rc = float(inp["cutoff"])
    _say("attention with and without the split workspace")
    a = _attention(mlip, g, h0, W_qkv, Wa_e, W_o, cfg.n_heads, rc, ws)
    b = _attention(mlip, g, h0, W_qkv, Wa_e, W_o, cfg.n_heads, rc, None)
    a2 = _attention(mlip, g, h0, W_qkv, Wa_e, W_o, cfg.n_heads, rc, ws)
    torch.cuda.synchronize()
    ref = inp["h"].astype(np.float64) @ inp["W_qkv"].astype(np.float64)
    errs = {k: _rel(a[k], b[k].cpu().numpy()) for k in ("qkv", "o", "u")}
    errs["split_vs_float64"] = _rel(a["qkv"], ref)
    errs["unsplit_vs_float64"] = _rel(b["qkv"], ref)
    _say(f"errors {errs}")
    assert max(errs["qkv"], errs["o"], errs["u"]) <= 2e-5, errs
    assert max(errs["split_vs_float64"], errs["unsplit_vs_float64"]) <= 2e-4, errs
    for k in a:
        assert torch.equal(a[k], a2[k]), k


def test_tri_split_matches_unsplit(mlip, setup):
    cfg, inp, g, up = setup
    h, W_s, W_ang, W_T = up(inp["h"]), up(inp["W_s"]), up(inp["W_ang"]), up(inp["W_T"])
    Dt = int(inp["W_s"].shape[1])
    need = mlip._lib.mlip_tri_workspace_size(cfg.n_atoms, Dt)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rc = float(inp["cutoff"])
    _say("Tri with and without the split workspace")
    a = _tri(mlip, g, h, W_s, W_ang, W_T, rc, ws)
    b = _tri(mlip, g, h, W_s, W_ang, W_T, rc, None)
    torch.cuda.synchronize()
    ref = inp["h"].astype(np.float64) @ inp["W_s"].astype(np.float64)
    errs = {k: _rel(a[k], b[k].cpu().numpy()) for k in ("s", "tau", "h_T")}
    errs["split_vs_float64"] = _rel(a["s"], ref)
    errs["unsplit_vs_float64"] = _rel(b["s"], ref)
    _say(f"errors {errs}")
    assert max(errs["s"], errs["tau"], errs["h_T"]) <= 2e-5, errs
    assert max(errs["split_vs_float64"], errs["unsplit_vs_float64"]) <= 2e-4, errs
