"""The bounds-checked build (libmlip_debug.so, -DMLIP_DEBUG_BOUNDS) on the GPU.

Each case runs in a child process that loads the debug build through
MLIP_LIBRARY (the parent has the release build loaded):
  * on valid inputs the checks stay silent and the block, the complete block
    and its training gradient still match the float64 oracle;
  * a sender index past the atoms, handed to the aggregation, is reported by
    the check (and clamped by it, so the kernel reads nothing out of range);
  * the fused MoE call at widths that are multiples of 256 (the paired launch
    on 128 x 256 tiles with tall and short tiles), with expert sizes on every
    tile-class boundary, stays silent and matches the oracle.
"""
import json
import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEBUG_LIB = os.path.join(ROOT, "element_routed_moe_amd", "libmlip_debug.so")

VALID = r'''
import json, sys
import numpy as np, torch
sys.path.insert(0, ROOT)
from element_routed_moe_amd import mlip, synth
from oracle import attention as OA, block as OB, graph as OG
assert mlip.LIB_PATH.endswith("libmlip_debug.so")
def rel(a, b):
    a = a.detach().cpu().numpy().astype(np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))
errs = {}
for name in ("tiny", "ragged"):
    cfg = synth.CONFIGS[name]
    inp = synth.make_full_inputs(cfg)
    g = OG.radius_graph(inp["pos"], inp["cell"], inp["struct_ptr"], inp["cutoff"])
    gup = synth.upstream_grad(cfg, inp, "energy").astype(np.float64)
    blk = mlip.Block(inp, device="cuda").step()
    f = OB.block_forward(inp, g); v = OB.block_vjp(inp, g, f, gup)
    fb = mlip.FullBlock(inp, device="cuda", train=True).step()
    ff = OA.full_block_forward(inp, g); fv = OA.full_block_vjp(inp, g, ff, gup)
    rng = np.random.default_rng(3)
    tg = fb.train_grad(torch.tensor(rng.standard_normal(cfg.n_structs), dtype=torch.float64, device="cuda"),
                       torch.from_numpy(rng.standard_normal((cfg.n_atoms, 3)).astype(np.float32)).cuda())
    torch.cuda.synchronize()
    errs[name] = dict(h_out=rel(blk.moe["h_out"], f["h2"]), grad_pos=rel(blk.vjp["grad_pos"], v["grad_pos"]),
                      full_h_out=rel(fb.moe["h_out"], ff["h2"]), full_grad_pos=rel(fb.avjp["grad_pos"], fv["grad_pos"]),
                      train_finite=bool(all(torch.isfinite(t).all() for t in tg.values() if t is not None)))
print("RESULT " + json.dumps(errs), flush=True)
'''

CORRUPT = r'''
import sys
import numpy as np, torch
sys.path.insert(0, ROOT)
from element_routed_moe_amd import mlip, synth
cfg = synth.CONFIGS["tiny"]
inp = synth.make_inputs(cfg)
t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
g = mlip.mlip_build_graph(t(inp["pos"]), t(inp["cell"]), t(inp["struct_ptr"]), float(inp["cutoff"]))
bad = dict(g)
bad["src"] = g["src"].clone()
bad["src"][5] = cfg.n_atoms + 7          # one sender past the atoms
out = mlip.mlip_aggregate(bad, t(inp["h"]), t(inp["W_e"]), t(inp["W_d"]), t(inp["W_u"]), float(inp["cutoff"]))
torch.cuda.synchronize()
print("RESULT finite=%d" % int(torch.isfinite(out["u"]).all().item()), flush=True)
'''


WIDE = r'''
import json, sys
import numpy as np, torch
sys.path.insert(0, ROOT)
from element_routed_moe_amd import mlip
from oracle import block as OB
assert mlip.LIB_PATH.endswith("libmlip_debug.so")
counts = [0, 1, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 160, 161, 192, 255, 256, 257, 300, 0, 5]
X, Dn, H = len(counts), 256, 512
rng = np.random.default_rng(5)
z = np.concatenate([np.full(c, t, np.int32) for t, c in enumerate(counts)])
z = z[rng.permutation(z.size)]
logits = (rng.standard_normal((X, X)) + 10.0 * np.eye(X)).astype(np.float32)   # type t -> expert t
u = rng.standard_normal((z.size, Dn)).astype(np.float32)
W1 = (rng.standard_normal((X, Dn, H)) / np.sqrt(Dn)).astype(np.float32)
W2 = (rng.standard_normal((X, H, Dn)) / np.sqrt(H)).astype(np.float32)
g = rng.standard_normal((z.size, Dn)).astype(np.float32)
up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
out = mlip.mlip_moe_forward_vjp(up(u), up(z), up(logits), up(W1), up(W2), 1, up(g))
torch.cuda.synchronize()
topk, gate = OB.route(logits, 1)
def rel(a, b):
    a = a.detach().cpu().numpy().astype(np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))
u64 = u.astype(np.float64)
errs = dict(h_out=rel(out["h_out"], OB.moe_forward(u64, z, topk, gate, W1, W2)),
            ubar=rel(out["grad_u"], OB.moe_vjp(u64, g.astype(np.float64), z, topk, gate, W1, W2)))
print("RESULT " + json.dumps(errs), flush=True)
'''


def _run(code):
    env = dict(os.environ, MLIP_LIBRARY=DEBUG_LIB)
    r = subprocess.run([sys.executable, "-c", f"ROOT = {ROOT!r}\n" + code], env=env, capture_output=True,
                       text=True, timeout=300)
    print(r.stdout[-4000:], r.stderr[-4000:], flush=True)
    return r


@pytest.fixture(scope="module")
def debug_lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    if not os.path.exists(DEBUG_LIB):
        pytest.skip("libmlip_debug.so is not built (python -m element_routed_moe_amd.build --debug-bounds)")
    return DEBUG_LIB


def test_debug_build_silent_and_exact_on_valid_input(debug_lib):
    r = _run(VALID)
    assert r.returncode == 0
    assert "mlip bounds" not in r.stdout + r.stderr
    line = [x for x in r.stdout.splitlines() if x.startswith("RESULT ")][-1]
    errs = json.loads(line[len("RESULT "):])
    for name, e in errs.items():
        assert e.pop("train_finite"), name
        assert max(e.values()) <= 2e-4, (name, e)


def test_debug_build_reports_a_bad_sender(debug_lib):
    r = _run(CORRUPT)
    assert r.returncode == 0
    assert "mlip bounds: sender index" in r.stdout + r.stderr
    assert "RESULT finite=1" in r.stdout


def test_debug_build_silent_on_the_tall_paired_launch(debug_lib):
    r = _run(WIDE)
    assert r.returncode == 0
    assert "mlip bounds" not in r.stdout + r.stderr
    line = [x for x in r.stdout.splitlines() if x.startswith("RESULT ")][-1]
    errs = json.loads(line[len("RESULT "):])
    assert max(errs.values()) <= 2e-4, errs
