"""GPU parity of the MoE forward and input gradient at the grouped GEMM's tile
boundaries.

The expert GEMMs cut each expert's token rows into 128-row tiles.  A
remainder of at most 32 rows gets a 32-row tile, at most 64 rows a 64-row
tile, and a longer one a padded full tile.  Each test crafts the per-expert
token counts directly: top-1 routing, with element type t sent to expert t by
a diagonal logit table, so that count_x is the number of atoms of type x.
The counts sit on every boundary (0, 1, 31, 32, 33, 63, 64, 65, 127, 128,
129, ...), and cover a case with short tiles only and a case with a single
busy expert.

Widths such as Dn = 148 and H = 260 leave a K tail (K mod 16 = 4) and a ragged
last 128-wide column tile.  h_out and dL/du are compared with the float64
oracle (moe_forward, moe_vjp) to 2e-4 of max-abs; the dispatch tables must
match exactly.

The fused call (forward and input gradient in one paired expert launch) runs
the same counts, once at widths that are multiples of 256 and once at the
ragged widths; it must equal the separate calls bit for bit and the oracle to
2e-4.  At the wide widths the launch takes 128 x 256 tiles and folds short
remainders into tall tiles: 129, 160 and 257 rows give one tall tile, 300 two
(a remainder of 44 split 22 + 22), 161 and every count up to 64 short tiles,
and 96, 255 a padded full tile.
"""
import sys

import numpy as np
import pytest

from oracle import block as OB

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = [
    # name, per-expert token counts, Dn, H
    ("boundaries", [0, 1, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 160, 161, 192, 255, 256, 257, 300, 0, 5],
     148, 260),
    ("short_only", [1, 2, 32, 33, 40, 64, 0, 7], 64, 128),
    ("one_expert", [0, 0, 1000, 0], 132, 196),
]


def _say(msg):
    print(f"[gpu-moe-tiles] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mlip():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from element_routed_moe_amd import mlip as m
    return m


def _inputs(counts, Dn, H, seed):
    rng = np.random.default_rng(seed)
    X = len(counts)
    z = np.concatenate([np.full(c, t, np.int32) for t, c in enumerate(counts)])
    z = z[rng.permutation(z.size)]                       # types interleaved over the atoms
    logits = (rng.standard_normal((X, X)) + 10.0 * np.eye(X)).astype(np.float32)
    u = rng.standard_normal((z.size, Dn)).astype(np.float32)
    W1 = (rng.standard_normal((X, Dn, H)) / np.sqrt(Dn)).astype(np.float32)
    W2 = (rng.standard_normal((X, H, Dn)) / np.sqrt(H)).astype(np.float32)
    g = rng.standard_normal((z.size, Dn)).astype(np.float32)
    return z, logits, u, W1, W2, g


def _rel(a, b):
    a = a.detach().cpu().numpy().astype(np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


@pytest.mark.parametrize("name,counts,Dn,H", CASES)
def test_moe_tile_boundaries(mlip, name, counts, Dn, H):
    z, logits, u, W1, W2, g = _inputs(counts, Dn, H, seed=len(counts) * 1000 + Dn)
    X = len(counts)
    _say(f"{name}: {z.size} atoms, {X} experts, counts {counts}, Dn {Dn}, H {H}")
    dev = "cuda"
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    moe = mlip.mlip_moe_forward(up(u), up(z), up(logits), up(W1), up(W2), 1)
    ubar = mlip.mlip_moe_vjp(moe, up(z), up(W1), up(W2), up(g))
    torch.cuda.synchronize()

    topk, gate = OB.route(logits, 1)
    assert np.array_equal(topk[:, 0], np.arange(X)), "the diagonal logits route type t to expert t"
    exp_off, tok_atom, slot = OB.dispatch_tables(z, topk, X)
    assert np.array_equal(np.diff(exp_off), np.asarray(counts)), "crafted per-expert counts"
    assert np.array_equal(moe["exp_off"].cpu().numpy(), exp_off)
    assert np.array_equal(moe["tok_atom"].cpu().numpy(), tok_atom)
    assert np.array_equal(moe["slot"].cpu().numpy(), slot)

    u64 = u.astype(np.float64)
    h_ref = OB.moe_forward(u64, z, topk, gate, W1, W2)
    ubar_ref = OB.moe_vjp(u64, g.astype(np.float64), z, topk, gate, W1, W2)
    errs = dict(h_out=_rel(moe["h_out"], h_ref), ubar=_rel(ubar, ubar_ref))
    # the MoE part alone (h_out - u), so that the residual does not mask it
    errs["moe_part"] = _rel(moe["h_out"] - up(u), h_ref - u64)
    errs["moe_vjp_part"] = _rel(ubar - up(g), ubar_ref - g.astype(np.float64))
    _say(f"{name}: errors {errs}")
    bad = {k: e for k, e in errs.items() if not e <= 2e-4}
    assert not bad, bad


def _many_experts():
    """1023 experts (the most the library takes), every eighth with a tile-boundary count and the last one
    busy: the expert lookup then spans every thread of the workgroup."""
    marks = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 160, 161, 192, 255, 256, 257, 300]
    counts = [marks[(e // 8) % len(marks)] if e % 8 == 7 else 0 for e in range(1023)]
    counts[-1] = 300
    return counts


FUSED_CASES = [
    # widths that are multiples of 256 take the paired launch's 128 x 256 tiles (tall 160 x 256 tiles for
    # the remainders, 32 x 256 and 64 x 256 short tiles for the smallest experts); the others its 128 x 128 tiles
    ("boundaries_wide", CASES[0][1], 256, 512),
    ("short_only_wide", CASES[1][1], 512, 256),
    ("boundaries", CASES[0][1], 148, 260),
    ("many_experts_wide", _many_experts(), 256, 256),
]


@pytest.mark.parametrize("name,counts,Dn,H", FUSED_CASES)
def test_fused_moe_tile_boundaries(mlip, name, counts, Dn, H):
    """mlip_moe_forward_vjp (the paired launch) at the same tile boundaries: the
    oracle to 2e-4, and the separate forward + VJP calls bit for bit."""
    z, logits, u, W1, W2, g = _inputs(counts, Dn, H, seed=len(counts) * 1000 + Dn + 7)
    X = len(counts)
    _say(f"fused {name}: {z.size} atoms, {X} experts, Dn {Dn}, H {H}")
    dev = "cuda"
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    fused = mlip.mlip_moe_forward_vjp(up(u), up(z), up(logits), up(W1), up(W2), 1, up(g), keep=True)
    moe = mlip.mlip_moe_forward(up(u), up(z), up(logits), up(W1), up(W2), 1)
    q = torch.empty_like(fused["Q"])
    ubar = mlip.mlip_moe_vjp(moe, up(z), up(W1), up(W2), up(g), q_out=q)
    torch.cuda.synchronize()
    for k in ("topk", "gate", "exp_off", "tok_atom", "slot", "P", "h_out"):
        assert torch.equal(fused[k], moe[k]), (name, k)
    assert torch.equal(fused["grad_u"], ubar), name
    assert torch.equal(fused["Q"], q), name
    topk, gate = OB.route(logits, 1)
    u64 = u.astype(np.float64)
    errs = dict(h_out=_rel(fused["h_out"], OB.moe_forward(u64, z, topk, gate, W1, W2)),
                ubar=_rel(fused["grad_u"], OB.moe_vjp(u64, g.astype(np.float64), z, topk, gate, W1, W2)))
    _say(f"fused {name}: errors {errs}")
    bad = {k: e for k, e in errs.items() if not e <= 2e-4}
    assert not bad, bad
