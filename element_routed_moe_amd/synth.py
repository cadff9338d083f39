"""Seeded synthetic inputs for one MatRIS-MoE interaction block.

This module only draws random numbers and lays them out in the shapes the
block takes.  It holds none of the method's arithmetic, so both the GPU path
and the CPU oracle can be fed from it.

Workloads follow the model widths of Table II in the paper review
"Breaking the Training Barrier of Billion-Parameter Universal Machine Learning
Interatomic Potentials" (xllm-io, section 3.1): S = node 2560 / edge 384 /
hidden 2560 / 72 experts / top-4; M = 1536 / 1536 / 1536 / 40 / top-8;
L = 1920 / 1920 / 1920 / 72 / top-16.  Structures are periodic cubic cells of
uniformly random atoms; the cell edge is chosen so that the expected number of
neighbours inside the cutoff hits a target degree.  The pages train on public
datasets that are not available here; these synthetic cells stand in for
them (about 128 atoms and 50 neighbours per atom, the same order of edges per
configuration as the pages' training corpus).

Draw order for a config with seed s (numpy PCG64 ``default_rng(s)``):
  1. positions, one structure after another: ``rng.random((n, 3)) * L``
     rounded to float32 (a value that rounds up to L is wrapped to 0);
  2. element types z: uniform integers, or a Zipf(s) law over T types;
  3. node features h ~ N(0, 1), float32 [N, Dn];
  4. the routing logit table ~ N(0, 1), float32 [T, X];
  5. weights ~ N(0, 1/fan_in), float32: W_e [K, De], W_d [Dn, De],
     W_u [De, Dn], W1 [X, Dn, H], W2 [X, H, Dn], w_r [Dn].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Union

import numpy as np

IntOrList = Union[int, Sequence[int]]
N_ANG = 4          # Legendre orders l = 0..3 of the three-body update
FloatOrList = Union[float, Sequence[float]]


@dataclasses.dataclass(frozen=True)
class BlockConfig:
    """Shape of one synthetic interaction-block workload."""

    name: str
    atoms_per_struct: IntOrList      # int (same for all) or one entry per structure
    n_structs: int
    cutoff: float                    # r_c in Angstrom
    n_types: int                     # T
    n_rbf: int                       # K
    d_edge: int                      # De
    d_node: int                      # Dn
    d_hidden: int                    # H
    n_experts: int                   # X
    top_k: int                       # k
    seed: int
    box: Optional[FloatOrList] = None        # cubic cell edge; None -> from target_degree
    target_degree: Optional[float] = None
    zipf: Optional[float] = None             # None -> uniform element types
    description: str = ""
    n_heads: int = 0                         # attention heads of the complete block
    d_attn: int = 0                          # attention width Da (0: no complete block)
    shape: Optional[Sequence[Sequence[float]]] = None  # lattice rows in units of the box edge

    def atoms_list(self) -> List[int]:
        if isinstance(self.atoms_per_struct, int):
            return [self.atoms_per_struct] * self.n_structs
        out = [int(v) for v in self.atoms_per_struct]
        assert len(out) == self.n_structs
        return out

    def boxes(self) -> List[float]:
        n = self.atoms_list()
        if self.box is None:
            assert self.target_degree is not None
            # expected neighbours = n * (4/3) pi r_c^3 / L^3  ->  solve for L
            vol_sphere = 4.0 / 3.0 * math.pi * self.cutoff ** 3
            det = 1.0 if self.shape is None else float(np.linalg.det(np.asarray(self.shape, np.float64)))
            return [(max(m, 1) * vol_sphere / (self.target_degree * det)) ** (1.0 / 3.0) for m in n]
        if isinstance(self.box, (int, float)):
            return [float(self.box)] * self.n_structs
        out = [float(v) for v in self.box]
        assert len(out) == self.n_structs
        return out

    @property
    def n_atoms(self) -> int:
        return int(sum(self.atoms_list()))

    @property
    def n_tokens(self) -> int:
        return self.n_atoms * self.top_k


CONFIGS: Dict[str, BlockConfig] = {}


def _reg(c: BlockConfig) -> BlockConfig:
    CONFIGS[c.name] = c
    return c


# The five workloads of the block: a tiny reference case, the S/M/L widths of
# Table II, and one GPU's graph-partition share at S widths.
TINY = _reg(BlockConfig(
    "tiny", 64, 1, 5.0, 4, 16, 32, 64, 128, 8, 2, seed=0, box=8.0, n_heads=4, d_attn=32,
    description="1 cubic cell of edge 8 A, 64 atoms, 4 uniform types, r_c 5 A, "
                "De 32, Dn 64, 8 experts top-2, MLP 64->128->64"))
S = _reg(BlockConfig(
    "S", 128, 32, 6.0, 16, 16, 384, 2560, 2560, 72, 4, seed=1, target_degree=50.0,
    n_heads=8, d_attn=384,
    description="32 cells x 128 atoms, ~50 nbrs at 6 A, 16 uniform types, De 384, "
                "Dn 2560, 72 experts top-4, MLP 2560->2560->2560"))
M = _reg(BlockConfig(
    "M", 128, 128, 6.0, 32, 16, 1536, 1536, 1536, 40, 8, seed=2, target_degree=50.0,
    zipf=1.1, n_heads=4, d_attn=512,
    description="128 cells x 128 atoms, 32 Zipf(1.1) types, De=Dn=H=1536, 40 experts top-8"))
L = _reg(BlockConfig(
    "L", 128, 64, 6.0, 64, 16, 1920, 1920, 1920, 72, 16, seed=3, target_degree=50.0,
    zipf=1.1, n_heads=4, d_attn=512,
    description="64 cells x 128 atoms, 64 Zipf(1.1) types, De=Dn=H=1920, 72 experts top-16"))
SHARE = _reg(BlockConfig(
    "share", 262144, 1, 6.0, 89, 16, 384, 2560, 2560, 72, 4, seed=4, target_degree=60.0,
    zipf=1.3, n_heads=8, d_attn=384,
    description="one periodic supercell of 262144 atoms, ~60 nbrs at 6 A, 89 Zipf(1.3) "
                "types, S widths"))

# Parity cases sized so the oracle finishes in seconds while the kernels still
# see several tiles, ragged tails and uneven structures.
RAGGED = _reg(BlockConfig(
    "ragged", [97, 130, 61, 1, 0, 200], 6, 5.5, 5, 16, 100, 132, 196, 7, 3, seed=11,
    box=[10.5, 11.0, 9.25, 12.0, 7.0, 14.5], n_heads=3, d_attn=72,
    description="6 uneven cells (incl. a 1-atom and an empty one), dims not tile multiples"))
CELLLIST = _reg(BlockConfig(
    "celllist", 3000, 1, 5.0, 6, 16, 64, 96, 160, 9, 2, seed=12, target_degree=45.0,
    zipf=1.2, n_heads=2, d_attn=64,
    description="one 3000-atom cell large enough for a >=3 bins/axis cell list"))
S_SLICE = _reg(BlockConfig(
    "S_slice", 128, 2, 6.0, 16, 16, 384, 2560, 2560, 72, 4, seed=13, target_degree=50.0,
    n_heads=8, d_attn=384,
    description="two cells at the full S widths (production tiles at oracle-friendly size)"))
SPARSE = _reg(BlockConfig(
    "sparse", [5, 3, 9], 3, 3.0, 3, 16, 36, 40, 44, 3, 3, seed=14, box=[30.0, 25.0, 28.0],
    n_heads=3, d_attn=36,
    description="dilute cells with isolated atoms (degree 0 rows), k = X"))
WIDE_RAGGED = _reg(BlockConfig(
    "wide_ragged", [150, 139], 2, 5.0, 5, 16, 100, 1028, 260, 5, 2, seed=16, box=[11.0, 10.5],
    n_heads=5, d_attn=80,
    description="wide node features with ragged K/N tails (K-sliced projections)"))
TOP1 = _reg(BlockConfig(
    "top1", [40, 33], 2, 4.0, 2, 16, 48, 68, 72, 5, 1, seed=15, box=[7.0, 6.5],
    n_heads=1, d_attn=48,
    description="top-1 routing (gate exactly 1), images because r_c > L/2"))


TRICLINIC_SHAPE = ((1.0, 0.1, -0.05), (0.35, 0.95, 0.08), (-0.3, 0.25, 0.9))
TRICLINIC = _reg(BlockConfig(
    "triclinic", [90, 120, 75], 3, 5.0, 5, 16, 40, 72, 96, 6, 2, seed=17, box=[9.0, 10.5, 8.5],
    n_heads=2, d_attn=32, shape=TRICLINIC_SHAPE,
    description="3 triclinic cells (all nine cell entries non-zero), one image bin per axis"))
TRICLINIC_CL = _reg(BlockConfig(
    "triclinic_cl", 2000, 1, 4.5, 4, 16, 40, 72, 96, 6, 2, seed=18, target_degree=45.0,
    n_heads=2, d_attn=32, shape=TRICLINIC_SHAPE,
    description="one 2000-atom triclinic cell with >= 3 bins per axis (fractional cell list)"))


def make_positions(cfg: BlockConfig, rng: np.random.Generator):
    """Positions [N,3] f32 (wrapped into the cell), cells [B,3,3] f32, struct_ptr [B+1] i32.

    Cubic cells: x = U[0,1)^3 * L rounded to float32.  A config with a
    ``shape`` uses the cell L * shape (rows = lattice vectors, rounded to
    float32) and x = f C with f ~ U[0,1)^3, rounded to float32."""
    counts = cfg.atoms_list()
    boxes = cfg.boxes()
    pos_parts = []
    cells = np.zeros((cfg.n_structs, 3, 3), dtype=np.float32)
    for b, (n, L_b) in enumerate(zip(counts, boxes)):
        Lf = np.float32(L_b)
        if cfg.shape is None:
            cells[b] = np.diag([Lf, Lf, Lf])
            p = (rng.random((n, 3)) * L_b).astype(np.float32)
            p[p >= Lf] = np.float32(0.0)
        else:
            cells[b] = (np.asarray(cfg.shape, np.float64) * L_b).astype(np.float32)
            p = (rng.random((n, 3)) @ cells[b].astype(np.float64)).astype(np.float32)
        pos_parts.append(p)
    pos = np.concatenate(pos_parts, axis=0) if pos_parts else np.zeros((0, 3), np.float32)
    struct_ptr = np.zeros(cfg.n_structs + 1, dtype=np.int32)
    struct_ptr[1:] = np.cumsum(counts)
    return pos, cells, struct_ptr


def make_types(cfg: BlockConfig, rng: np.random.Generator) -> np.ndarray:
    N, T = cfg.n_atoms, cfg.n_types
    if cfg.zipf is None:
        return rng.integers(0, T, N).astype(np.int32)
    p = (np.arange(T, dtype=np.float64) + 1.0) ** (-cfg.zipf)
    p /= p.sum()
    return rng.choice(T, N, p=p).astype(np.int32)


def _normal(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def make_inputs(cfg: BlockConfig, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """All host-side inputs of one block, in the fixed draw order of the module doc."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    pos, cells, struct_ptr = make_positions(cfg, rng)
    z = make_types(cfg, rng)
    N, T, X = cfg.n_atoms, cfg.n_types, cfg.n_experts
    K, De, Dn, H = cfg.n_rbf, cfg.d_edge, cfg.d_node, cfg.d_hidden
    out = dict(pos=pos, cell=cells, struct_ptr=struct_ptr, z=z)
    out["h"] = _normal(rng, (N, Dn), 1.0)
    out["logits"] = _normal(rng, (T, X), 1.0)
    out["W_e"] = _normal(rng, (K, De), 1.0 / math.sqrt(K))
    out["W_d"] = _normal(rng, (Dn, De), 1.0 / math.sqrt(Dn))
    out["W_u"] = _normal(rng, (De, Dn), 1.0 / math.sqrt(De))
    out["W1"] = _normal(rng, (X, Dn, H), 1.0 / math.sqrt(Dn))
    out["W2"] = _normal(rng, (X, H, Dn), 1.0 / math.sqrt(H))
    out["w_r"] = _normal(rng, (Dn,), 1.0 / math.sqrt(Dn))
    out["cutoff"] = np.float32(cfg.cutoff)
    out["top_k"] = int(cfg.top_k)
    return out


def make_full_inputs(cfg: BlockConfig, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of the complete block (MoE0, attention, MoE1): ``make_inputs``
    plus the extra parameters, drawn from a second generator seeded with
    (seed, 1) in this order: the MoE0 logit table logits0 ~ N(0,1) [T, X];
    Wa_e [K, Da]; W_qkv [Dn, 3 Da] (columns q | k | v); W_o [Da, Dn];
    W1_0 [X, Dn, H]; W2_0 [X, H, Dn] (weights ~ N(0, 1/fan_in)); then the
    three-body update: W_s [Dn, Dt] ~ N(0, 1/Dn), W_ang [L, Dt] ~ N(0, 1/L)
    scaled by 1/50 (about one over the number of neighbour pairs' square
    root, so that the pair sum stays of order one), W_T [Dt, Dn] ~ N(0, 1/Dt),
    with Dt = Da and L = N_ANG.  MoE1 uses ``logits``, ``W1``, ``W2`` and the
    readout ``w_r`` of ``make_inputs``."""
    if cfg.d_attn <= 0 or cfg.n_heads <= 0:
        raise ValueError(f"config {cfg.name} has no attention width")
    out = make_inputs(cfg, seed)
    base = cfg.seed if seed is None else seed
    rng = np.random.default_rng([base, 1])
    T, X, K = cfg.n_types, cfg.n_experts, cfg.n_rbf
    Dn, H, Da = cfg.d_node, cfg.d_hidden, cfg.d_attn
    out["logits0"] = _normal(rng, (T, X), 1.0)
    out["Wa_e"] = _normal(rng, (K, Da), 1.0 / math.sqrt(K))
    out["W_qkv"] = _normal(rng, (Dn, 3 * Da), 1.0 / math.sqrt(Dn))
    out["W_o"] = _normal(rng, (Da, Dn), 1.0 / math.sqrt(Da))
    out["W1_0"] = _normal(rng, (X, Dn, H), 1.0 / math.sqrt(Dn))
    out["W2_0"] = _normal(rng, (X, H, Dn), 1.0 / math.sqrt(H))
    out["W_s"] = _normal(rng, (Dn, Da), 1.0 / math.sqrt(Dn))
    out["W_ang"] = _normal(rng, (N_ANG, Da), 1.0 / (math.sqrt(N_ANG) * 50.0))
    out["W_T"] = _normal(rng, (Da, Dn), 1.0 / math.sqrt(Da))
    out["n_heads"] = int(cfg.n_heads)
    return out


N_BLOCKS = 6       # interaction blocks per model (Table II: 6 layers at every size)

# Without any normalisation layer (the pages name none) a deep stack of
# random-init residual blocks grows its features geometrically (the three-body
# term is quadratic in them); the stack therefore draws the output weight of
# every residual branch at RESID_SCALE times N(0, 1/fan_in), which keeps six
# blocks at feature scale ~1.
RESID_SCALE = 0.3

_BLOCK_PARAM_SHAPES = (   # (name, shape(cfg), fan_in(cfg) or None for N(0, 1), extra scale), in draw order
    ("logits0", lambda c: (c.n_types, c.n_experts), None, 1.0),
    ("logits", lambda c: (c.n_types, c.n_experts), None, 1.0),
    ("Wa_e", lambda c: (c.n_rbf, c.d_attn), lambda c: c.n_rbf, 1.0),
    ("W_qkv", lambda c: (c.d_node, 3 * c.d_attn), lambda c: c.d_node, 1.0),
    ("W_o", lambda c: (c.d_attn, c.d_node), lambda c: c.d_attn, RESID_SCALE),
    ("W1_0", lambda c: (c.n_experts, c.d_node, c.d_hidden), lambda c: c.d_node, 1.0),
    ("W2_0", lambda c: (c.n_experts, c.d_hidden, c.d_node), lambda c: c.d_hidden, RESID_SCALE),
    ("W_s", lambda c: (c.d_node, c.d_attn), lambda c: c.d_node, 1.0),
    ("W_ang", lambda c: (N_ANG, c.d_attn), lambda c: N_ANG * 2500.0, 1.0),
    ("W_T", lambda c: (c.d_attn, c.d_node), lambda c: c.d_attn, RESID_SCALE),
    ("W1", lambda c: (c.n_experts, c.d_node, c.d_hidden), lambda c: c.d_node, 1.0),
    ("W2", lambda c: (c.n_experts, c.d_hidden, c.d_node), lambda c: c.d_hidden, RESID_SCALE),
)


def make_stack_inputs(cfg: BlockConfig, n_blocks: int = N_BLOCKS, seed: Optional[int] = None):
    """Inputs of a stack of complete blocks on one graph: (shared, blocks).

    shared: positions, cells, struct_ptr and z drawn exactly as in
    ``make_inputs`` (same generator, same first two draws); then, from a
    generator seeded (seed, 2): the element embedding emb ~ N(0,1) [T, Dn]
    and the readout w_r ~ N(0, 1/Dn).  blocks[b]: the parameters of block b
    from a generator seeded (seed, 100 + b), drawn in the order of
    ``_BLOCK_PARAM_SHAPES`` (weights ~ N(0, 1/fan_in), residual-branch
    outputs times RESID_SCALE; W_ang as in ``make_full_inputs``)."""
    base = cfg.seed if seed is None else seed
    rng = np.random.default_rng(base)
    pos, cells, struct_ptr = make_positions(cfg, rng)
    z = make_types(cfg, rng)
    shared = dict(pos=pos, cell=cells, struct_ptr=struct_ptr, z=z, cutoff=np.float32(cfg.cutoff),
                  top_k=int(cfg.top_k), n_heads=int(cfg.n_heads))
    r2 = np.random.default_rng([base, 2])
    shared["emb"] = _normal(r2, (cfg.n_types, cfg.d_node), 1.0)
    shared["w_r"] = _normal(r2, (cfg.d_node,), 1.0 / math.sqrt(cfg.d_node))
    blocks = []
    for b in range(n_blocks):
        rb = np.random.default_rng([base, 100 + b])
        blocks.append({name: _normal(rb, shape(cfg), sc if fan is None else sc / math.sqrt(fan(cfg)))
                       for name, shape, fan, sc in _BLOCK_PARAM_SHAPES})
    return shared, blocks


def device_stack_params(cfg: BlockConfig, n_blocks: int, device, seed: Optional[int] = None):
    """Block parameters of a stack generated on the GPU (the S-width stack holds
    about 45 GB of expert weights, too much to draw on the host): a seeded
    torch generator on the device, seeded with seed * 1000 + 100 + b for block
    b, same names, shapes, order and scales as ``make_stack_inputs``.  The two
    logit tables (routing, drawn first) come from the host generator exactly
    as there, so routing and expert loads match the host-drawn stack."""
    import torch
    base = cfg.seed if seed is None else seed
    blocks = []
    for b in range(n_blocks):
        g = torch.Generator(device=device)
        g.manual_seed(base * 1000 + 100 + b)
        rb = np.random.default_rng([base, 100 + b])
        p = {}
        for name, shape, fan, sc in _BLOCK_PARAM_SHAPES:
            if name in ("logits0", "logits"):
                p[name] = torch.from_numpy(_normal(rb, shape(cfg), 1.0)).to(device)
                continue
            t = torch.randn(shape(cfg), generator=g, device=device, dtype=torch.float32)
            p[name] = t.mul_(sc / math.sqrt(fan(cfg)))
        blocks.append(p)
    return blocks


def upstream_grad(cfg: BlockConfig, inputs: Dict[str, np.ndarray], kind: str = "energy",
                  seed: int = 99) -> np.ndarray:
    """Upstream gradient dL/dh' [N, Dn] f32 for the block's VJP.

    ``energy``: every row is the readout vector w_r, so the VJP returns dE/d(inputs)
    of a one-block model.  ``random``: N(0,1) rows, the general upstream a later
    block would send.
    """
    N, Dn = cfg.n_atoms, cfg.d_node
    if kind == "energy":
        return np.broadcast_to(inputs["w_r"], (N, Dn)).astype(np.float32, copy=True)
    rng = np.random.default_rng(seed)
    return rng.standard_normal((N, Dn), dtype=np.float32)
