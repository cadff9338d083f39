"""Python binding of libmlip.so (the C ABI in include/mlip.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their device pointers and the current HIP stream to
the C entry point of the same name, and turns a negative status into an
exception.  Nothing here computes any part of the block; when the library is
missing, importing this module fails.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLIP_LIBRARY selects another build of the same library (e.g. libmlip_debug.so,
# the bounds-checked build); by default the release build next to this file.
LIB_PATH = os.environ.get("MLIP_LIBRARY") or os.path.join(_HERE, "libmlip.so")

MLIP_OK = 0
MLIP_ERR_INVALID = -1
MLIP_ERR_CAPACITY = -2
MLIP_ERR_UNSUPPORTED = -3
MLIP_ERR_HIP = -4
MLIP_ERR_INPUT = -5
N_RBF = 16
N_ANG = 4


class MlipError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mlip error {code}: {msg}")
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing; build it with "
                      f"`python -m element_routed_moe_amd.build`")
_lib = C.CDLL(LIB_PATH)

_p, _i32, _i64, _f32, _sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
_SIGS = {
    "mlip_last_error": (C.c_char_p, []),
    "mlip_version": (C.c_int, []),
    "mlip_graph_workspace_size": (_sz, [_i32, _i32]),
    "mlip_build_graph": (C.c_int, [_p, _p, _p, _i32, _i32, _f32, _i64, _p, _p, _p, _p, _p,
                                   C.POINTER(C.c_int64), _p, _sz, _p]),
    "mlip_graph_reverse": (C.c_int, [_p, _p, _p, _i32, _i64, _p, _p, _sz, _p]),
    "mlip_build_graph_async": (C.c_int, [_p, _p, _p, _i32, _i32, _f32, _i64, _p, _p, _p, _p, _p, _p, _p,
                                         _sz, _p]),
    "mlip_graph_check": (C.c_int, [_p, _i64, C.POINTER(C.c_int64)]),
    "mlip_aggregate_workspace_size": (_sz, [_i32, _i32, _i32]),
    "mlip_aggregate": (C.c_int, [_p, _p, _p, _i32, _i64, _p, _p, _p, _p, _i32, _i32, _i32, _f32,
                                 _p, _p, _p, _p, _sz, _p]),
    "mlip_aggregate_static": (C.c_int, [_p, _p, _p, _i32, _i64, _p, _p, _p, _p, _i32, _i32, _i32, _f32,
                                        _p, _p, _p, _p]),
    "mlip_moe_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "mlip_moe_forward": (C.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                   _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "mlip_moe_status": (C.c_int, [_p, C.POINTER(C.c_int32), _p]),
    "mlip_moe_forward_vjp_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "mlip_struct_size": (_sz, [_i32]),
    "mlip_moe_forward_vjp": (C.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p,
                                       _p, _p, _p, _p, _p, _sz, _p]),
    "mlip_aggregate_vjp_workspace_size": (_sz, [_i32, _i32, _i32]),
    "mlip_aggregate_vjp": (C.c_int, [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _f32,
                                     _p, _p, _p, _p, _i32, _p, _p, _p, _sz, _p]),
    "mlip_readout": (C.c_int, [_p, _p, _p, _i32, _i32, _i32, _p, _p, _p]),
    "mlip_vjp_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "mlip_block_vjp": (C.c_int, [_p, _p, _p, _i32, _i64, _p, _p, _p, _p, _p, _p, _p, _p,
                                 _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                 _f32, _p, _p, _p, _p, _i32, _p, _p, _p, _p, _p, _sz, _p]),
    "mlip_block_jvp_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "mlip_block_jvp": (C.c_int, [_p, _p, _p, _i32, _i64, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                 _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                 _f32, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "mlip_block_tangent_vjp_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "mlip_block_tangent_vjp": (C.c_int, [_p, _p, _p, _i32, _i64, _p, _p, _p, _p, _p, _p, _p, _p,
                                         _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                         _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                         _i32, _f32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "mlip_readout_vjp": (C.c_int, [_p, _p, _p, _i32, _i32, _i32, _p, _p]),
    "mlip_readout_grad_workspace_size": (_sz, [_i32, _i32]),
    "mlip_readout_grad": (C.c_int, [_p, _p, _p, _p, _i32, _i32, _i32, _p, _p, _sz, _p]),
    "mlip_moe_vjp_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "mlip_moe_vjp": (C.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                               _p, _p, _p, _p, _sz, _p]),
    "mlip_moe_jvp_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "mlip_moe_jvp": (C.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                               _p, _p, _p, _p, _sz, _p]),
    "mlip_moe_tangent_vjp_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "mlip_moe_tangent_vjp": (C.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                                       _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "mlip_attention_jvp": (C.c_int, [_p, _p, _p, _i32, _i64, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32,
                                     _i32, _i32, _f32, _p, _p, _p, _p, _p]),
    "mlip_attention_tangent_vjp_workspace_size": (_sz, [_i32, _i64, _i32, _i32, _i32]),
    "mlip_attention_tangent_vjp": (C.c_int, [_p, _p, _p, _p, _i32, _i64, _p, _p, _p, _p, _p, _p, _p, _p,
                                             _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _f32, _p, _p, _p,
                                             _p, _p, _p, _p, _sz, _p]),
    "mlip_attention": (C.c_int, [_p, _p, _p, _i32, _i64, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                                 _f32, _p, _p, _p, _p, _p, _sz, _p]),
    "mlip_attention_workspace_size": (_sz, [_i32, _i32]),
    "mlip_attention_vjp_workspace_size": (_sz, [_i32, _i64, _i32, _i32]),
    "mlip_attention_vjp": (C.c_int, [_p, _p, _p, _p, _i32, _i64, _p, _p, _p, _p, _p, _p, _i32,
                                     _i32, _i32, _i32, _f32, _p, _p, _p, _p, _i32, _p, _p, _i32,
                                     _p, _p, _sz, _p]),
    "mlip_embed_atoms": (C.c_int, [_p, _p, _i32, _i32, _i32, _p, _p]),
    "mlip_embed_grad": (C.c_int, [_p, _p, _i32, _i32, _i32, _p, _p]),
    "mlip_tri": (C.c_int, [_p, _p, _p, _i32, _i64, _p, _p, _p, _p, _i32, _i32, _i32, _f32, _p, _p,
                           _p, _p, _sz, _p]),
    "mlip_tri_workspace_size": (_sz, [_i32, _i32]),
    "mlip_tri_vjp_workspace_size": (_sz, [_i32, _i64, _i32]),
    "mlip_tri_vjp": (C.c_int, [_p, _p, _p, _p, _i32, _i64, _p, _p, _p, _p, _i32, _i32, _i32, _f32,
                               _p, _p, _p, _p, _i32, _p, _p, _i32, _p, _p, _sz, _p]),
    "mlip_tri_jvp": (C.c_int, [_p, _p, _p, _i32, _i64, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _f32,
                               _p, _p, _p, _p]),
    "mlip_tri_tangent_vjp_workspace_size": (_sz, [_i32, _i64, _i32, _i32]),
    "mlip_tri_tangent_vjp": (C.c_int, [_p, _p, _p, _p, _i32, _i64, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                       _p, _i32, _i32, _i32, _f32, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "mlip_profile_enable": (C.c_int, [C.c_int]),
    "mlip_profile_select": (C.c_int, [C.c_uint64]),
    "mlip_profile_reset": (C.c_int, []),
    "mlip_profile_count": (C.c_int, []),
    "mlip_profile_get": (C.c_int, [C.c_int, C.POINTER(C.c_char_p), C.POINTER(C.c_int64),
                                   C.POINTER(C.c_double)]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class _Graph(C.Structure):
    """mlip_graph of include/mlip.h: device pointers of a receiver-sorted CSR graph."""
    _fields_ = [("row_ptr", C.c_void_p), ("src", C.c_void_p), ("shift", C.c_void_p), ("rev", C.c_void_p),
                ("geom", C.c_void_p), ("n_atoms", C.c_int32), ("n_edges", C.c_int64)]


class _MoeState(C.Structure):
    """mlip_moe_state of include/mlip.h: a MoE layer's routing tables and hidden pre-activations."""
    _fields_ = [("topk", C.c_void_p), ("gate", C.c_void_p), ("exp_off", C.c_void_p),
                ("tok_atom", C.c_void_p), ("slot", C.c_void_p), ("P", C.c_void_p)]


if _lib.mlip_struct_size(0) != C.sizeof(_Graph) or _lib.mlip_struct_size(1) != C.sizeof(_MoeState):
    raise ImportError("libmlip's mlip_graph / mlip_moe_state layout differs from this binding's")


def _graph_struct(graph) -> _Graph:
    return _Graph(_ptr(graph["row_ptr"]), _ptr(graph.get("src")), _ptr(graph.get("shift")),
                  _ptr(graph.get("rev")), _ptr(graph.get("geom")), int(graph["row_ptr"].shape[0]) - 1,
                  int(graph["n_edges"]))


def _moe_struct(moe) -> _MoeState:
    return _MoeState(_ptr(moe["topk"]), _ptr(moe["gate"]), _ptr(moe["exp_off"]), _ptr(moe["tok_atom"]),
                     _ptr(moe["slot"]), _ptr(moe["P"]))


def _check(rc: int):
    if rc != MLIP_OK:
        raise MlipError(rc, _lib.mlip_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmlip must be contiguous")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# --------------------------------------------------------------- entry points
def mlip_build_graph(pos, cell, struct_ptr, cutoff: float, edge_capacity: Optional[int] = None,
                     ws: Optional[torch.Tensor] = None, buffers: Optional[Dict] = None) -> Dict[str, torch.Tensor]:
    """Periodic radius graph (CSR by receiver).  Returns row_ptr, src, shift, rev, geom, n_edges.

    ``buffers`` (the "buffers" entry of an earlier result) lends its arrays
    when their capacity suffices, so a repeated build allocates nothing; the
    earlier result's tensors are then overwritten."""
    dev = pos.device
    N, B = int(pos.shape[0]), int(cell.shape[0])
    if ws is None:
        ws = _ws(_lib.mlip_graph_workspace_size(N, B), dev)
    cap = int(edge_capacity) if edge_capacity is not None else max(64 * N, 1)
    for _ in range(2):
        if buffers is not None and buffers["src"].shape[0] >= cap and buffers["row_ptr"].shape[0] == N + 1:
            row_ptr, src, shift, rev, geom = (buffers[k] for k in ("row_ptr", "src", "shift", "rev", "geom"))
            cap = int(src.shape[0])
        else:
            row_ptr = torch.empty(N + 1, dtype=torch.int32, device=dev)
            src = torch.empty(cap, dtype=torch.int32, device=dev)
            shift = torch.empty((cap, 4), dtype=torch.int8, device=dev)
            rev = torch.empty(cap, dtype=torch.int32, device=dev)
            geom = torch.empty((cap, 4), dtype=torch.float32, device=dev)
            buffers = dict(row_ptr=row_ptr, src=src, shift=shift, rev=rev, geom=geom)
        ne = C.c_int64(0)
        rc = _lib.mlip_build_graph(_ptr(pos), _ptr(cell), _ptr(struct_ptr), N, B, float(cutoff), cap,
                                   _ptr(row_ptr), _ptr(src), _ptr(shift), _ptr(rev), _ptr(geom),
                                   C.byref(ne), _ptr(ws), ws.numel(), _stream())
        if rc == MLIP_ERR_CAPACITY:
            cap = int(ne.value)
            buffers = None
            continue
        _check(rc)
        E = int(ne.value)
        return dict(row_ptr=row_ptr, src=src[:E], shift=shift[:E], rev=rev[:E], geom=geom[:E],
                    n_edges=E, buffers=buffers)
    raise MlipError(MLIP_ERR_CAPACITY, "edge capacity could not be met")


def mlip_build_graph_async(pos, cell, struct_ptr, cutoff: float, buffers: Dict, summary: torch.Tensor,
                           ws: torch.Tensor) -> Dict[str, torch.Tensor]:
    """The graph build queued with no wait, into ``buffers`` (the "buffers" of an
    earlier mlip_build_graph result, whose length is the edge capacity).  The
    summary (E, flags, largest degree) goes to the device tensor ``summary``
    [4]; read it with mlip_graph_check once copied to the host.  The result's
    n_edges is the capacity (an upper bound every later call may use)."""
    N, B = int(pos.shape[0]), int(cell.shape[0])
    row_ptr, src, shift, rev, geom = (buffers[k] for k in ("row_ptr", "src", "shift", "rev", "geom"))
    cap = int(src.shape[0])
    _check(_lib.mlip_build_graph_async(_ptr(pos), _ptr(cell), _ptr(struct_ptr), N, B, float(cutoff), cap,
                                       _ptr(row_ptr), _ptr(src), _ptr(shift), _ptr(rev), _ptr(geom),
                                       _ptr(summary), _ptr(ws), ws.numel(), _stream()))
    return dict(row_ptr=row_ptr, src=src, shift=shift, rev=rev, geom=geom, n_edges=cap, buffers=buffers)


def mlip_graph_check(summary_host: torch.Tensor, edge_capacity: int) -> int:
    """Status of an asynchronous build from its summary on the host: returns E,
    raises MlipError for what mlip_build_graph would have returned as an error."""
    ne = C.c_int64(0)
    _check(_lib.mlip_graph_check(_ptr(summary_host), int(edge_capacity), C.byref(ne)))
    return int(ne.value)


class GraphState:
    """The radius graph of a step loop.  The first build waits for the edge
    count and sizes the buffers; later builds are queued without a wait
    (mlip_build_graph_async) into those buffers, and their summary is read by
    ``check()`` after the rest of the step has been queued, waiting only for
    the build itself.  When the edges outgrow the buffers, ``check()`` says so
    and the next build is again a waiting one, with room to spare."""

    def __init__(self, pos, cell, struct_ptr, cutoff: float, device):
        self.pos, self.cell, self.struct_ptr, self.cutoff = pos, cell, struct_ptr, float(cutoff)
        N, B = int(pos.shape[0]), int(cell.shape[0])
        self.ws = _ws(_lib.mlip_graph_workspace_size(N, B), device)
        self.summary_dev = torch.zeros(4, dtype=torch.int32, device=device)
        self.summary_host = torch.zeros(4, dtype=torch.int32).pin_memory()
        self.event = torch.cuda.Event()
        self.graph = None
        self.pending = False
        self.min_capacity = None

    def build(self):
        if self.graph is None:
            self.graph = mlip_build_graph(self.pos, self.cell, self.struct_ptr, self.cutoff,
                                          edge_capacity=self.min_capacity, ws=self.ws)
            return self.graph
        self.graph = mlip_build_graph_async(self.pos, self.cell, self.struct_ptr, self.cutoff,
                                            self.graph["buffers"], self.summary_dev, self.ws)
        self.summary_host.copy_(self.summary_dev, non_blocking=True)
        self.event.record()
        self.pending = True
        return self.graph

    def check(self) -> bool:
        """False when the last build's edges did not fit: the step must be run again."""
        if not self.pending:
            return True
        self.pending = False
        self.event.synchronize()
        buf = self.graph["buffers"]
        cap = int(buf["src"].shape[0])
        try:
            E = mlip_graph_check(self.summary_host, cap)
        except MlipError as err:
            if err.code != MLIP_ERR_CAPACITY:
                raise
            need = int(self.summary_host[0])
            self.min_capacity = need + need // 4 + 64
            self.graph = None
            return False
        self.graph.update(src=buf["src"][:E], shift=buf["shift"][:E], rev=buf["rev"][:E],
                          geom=buf["geom"][:E], n_edges=E)
        return True


def mlip_graph_reverse(row_ptr, src, shift, rev: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Reverse-edge index of a receiver-sorted CSR graph (rows ordered by
    sender and shift, as mlip_build_graph writes them)."""
    N = int(row_ptr.shape[0]) - 1
    E = int(src.shape[0])
    dev = row_ptr.device
    if rev is None:
        rev = torch.empty(max(E, 1), dtype=torch.int32, device=dev)[:E]
    if ws is None:
        ws = _ws(_lib.mlip_graph_workspace_size(0, 1), dev)
    _check(_lib.mlip_graph_reverse(_ptr(row_ptr), _ptr(src), _ptr(shift), N, E, _ptr(rev), _ptr(ws),
                                   ws.numel(), _stream()))
    return rev


def mlip_aggregate(graph, h, W_e, W_d, W_u, cutoff: float, out: Optional[Dict] = None,
                   ws: Optional[torch.Tensor] = None, store_e: bool = True) -> Dict[str, torch.Tensor]:
    """Edge embedding + aggregation; out["e"] is None when the edge features are
    not kept (the VJP then rebuilds them)."""
    N, Dn = int(h.shape[0]), int(h.shape[1])
    De = int(W_e.shape[1])
    E = int(graph["n_edges"])
    dev = h.device
    if out is None:
        out = dict(e=torch.empty((E, De), dtype=torch.float32, device=dev) if store_e else None,
                   s=torch.empty((N, De), dtype=torch.float32, device=dev),
                   u=torch.empty((N, Dn), dtype=torch.float32, device=dev))
    if ws is None:
        ws = _ws(_lib.mlip_aggregate_workspace_size(N, De, Dn), dev)
    _check(_lib.mlip_aggregate(_ptr(graph["row_ptr"]), _ptr(graph["src"]), _ptr(graph["geom"]), N, E,
                               _ptr(h), _ptr(W_e), _ptr(W_d), _ptr(W_u), int(W_e.shape[0]), De, Dn,
                               float(cutoff), _ptr(out["e"]), _ptr(out["s"]), _ptr(out["u"]),
                               _ptr(ws), ws.numel(), _stream()))
    return out


AGGREGATE_STATIC_MAX_BYTES = 32 << 20    # MLIP_AGGREGATE_STATIC_MAX_BYTES of mlip.h


def mlip_aggregate_static(graph, h, W_e, W_d, W_u, cutoff: float, out: Dict) -> Dict[str, torch.Tensor]:
    """mlip_aggregate on the library's own scratch (no workspace): the caller
    passes preallocated outputs out["e"] (or None), out["s"], out["u"]."""
    N, Dn = int(h.shape[0]), int(h.shape[1])
    De = int(W_e.shape[1])
    E = int(graph["n_edges"])
    _check(_lib.mlip_aggregate_static(_ptr(graph["row_ptr"]), _ptr(graph["src"]), _ptr(graph["geom"]), N,
                                      E, _ptr(h), _ptr(W_e), _ptr(W_d), _ptr(W_u), int(W_e.shape[0]), De,
                                      Dn, float(cutoff), _ptr(out.get("e")), _ptr(out["s"]),
                                      _ptr(out["u"]), _stream()))
    return out


def mlip_moe_forward(u, z, logits, W1, W2, top_k: int, out: Optional[Dict] = None,
                     ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    N, Dn = int(u.shape[0]), int(u.shape[1])
    T, X = int(logits.shape[0]), int(logits.shape[1])
    H = int(W1.shape[2])
    k = int(top_k)
    dev = u.device
    if out is None:
        out = dict(topk=torch.empty((T, k), dtype=torch.int32, device=dev),
                   gate=torch.empty((T, k), dtype=torch.float32, device=dev),
                   exp_off=torch.empty(X + 1, dtype=torch.int32, device=dev),
                   tok_atom=torch.empty(N * k, dtype=torch.int32, device=dev),
                   slot=torch.empty((N, k), dtype=torch.int32, device=dev),
                   P=torch.empty((N * k, H), dtype=torch.float32, device=dev),
                   h_out=torch.empty((N, Dn), dtype=torch.float32, device=dev))
    if ws is None:
        ws = _ws(_lib.mlip_moe_workspace_size(N, T, X, k, Dn, H), dev)
    out["ws"] = ws
    _check(_lib.mlip_moe_forward(_ptr(u), _ptr(z), _ptr(logits), _ptr(W1), _ptr(W2), N, T, X, k, Dn, H,
                                 _ptr(out["topk"]), _ptr(out["gate"]), _ptr(out["exp_off"]),
                                 _ptr(out["tok_atom"]), _ptr(out["slot"]), _ptr(out["P"]),
                                 _ptr(out["h_out"]), _ptr(ws), ws.numel(), _stream()))
    return out


def mlip_moe_forward_vjp(u, z, logits, W1, W2, top_k: int, grad_out, out: Optional[Dict] = None,
                         ws: Optional[torch.Tensor] = None, keep: bool = False) -> Dict[str, torch.Tensor]:
    """MoE forward and its input gradient for a known upstream grad_out: the
    tables, P and h_out of mlip_moe_forward plus grad_u (and, with ``keep``,
    Q = grad_out[tok] @ W2^T per token for the training gradient)."""
    N, Dn = int(u.shape[0]), int(u.shape[1])
    T, X = int(logits.shape[0]), int(logits.shape[1])
    H = int(W1.shape[2])
    k = int(top_k)
    dev = u.device
    if out is None:
        out = dict(topk=torch.empty((T, k), dtype=torch.int32, device=dev),
                   gate=torch.empty((T, k), dtype=torch.float32, device=dev),
                   exp_off=torch.empty(X + 1, dtype=torch.int32, device=dev),
                   tok_atom=torch.empty(N * k, dtype=torch.int32, device=dev),
                   slot=torch.empty((N, k), dtype=torch.int32, device=dev),
                   P=torch.empty((N * k, H), dtype=torch.float32, device=dev),
                   h_out=torch.empty((N, Dn), dtype=torch.float32, device=dev),
                   grad_u=torch.empty((N, Dn), dtype=torch.float32, device=dev))
    if keep and out.get("Q") is None:
        out["Q"] = torch.empty((N * k, H), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _ws(_lib.mlip_moe_forward_vjp_workspace_size(N, T, X, k, Dn, H), dev)
    out["ws"] = ws
    st = _moe_struct(out)
    _check(_lib.mlip_moe_forward_vjp(_ptr(u), _ptr(z), _ptr(logits), _ptr(W1), _ptr(W2), N, T, X, k, Dn, H,
                                     _ptr(grad_out), C.byref(st), _ptr(out["h_out"]), _ptr(out["grad_u"]),
                                     _ptr(out.get("Q") if keep else None), _ptr(ws), ws.numel(), _stream()))
    return out


def mlip_aggregate_vjp(graph, agg, W_e, W_d, W_u, cutoff: float, grad_u, struct_ptr=None,
                       out: Optional[Dict] = None, ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Input gradient of the aggregation step from grad_u = dL/du: grad_h, grad_pos,
    atom_virial and (with struct_ptr) grad_strain."""
    N, Dn = int(grad_u.shape[0]), int(grad_u.shape[1])
    De = int(W_e.shape[1])
    E = int(graph["n_edges"])
    dev = grad_u.device
    B = int(struct_ptr.shape[0]) - 1 if struct_ptr is not None else 0
    if out is None:
        out = dict(grad_h=torch.empty((N, Dn), dtype=torch.float32, device=dev),
                   grad_pos=torch.empty((N, 3), dtype=torch.float32, device=dev),
                   atom_virial=torch.empty((N, 6), dtype=torch.float32, device=dev))
        if struct_ptr is not None:
            out["grad_strain"] = torch.empty((B, 6), dtype=torch.float64, device=dev)
    if ws is None:
        ws = _ws(_lib.mlip_aggregate_vjp_workspace_size(N, De, Dn), dev)
    g = _graph_struct(graph)
    if g.n_atoms != N or g.n_edges != E:
        raise ValueError("the graph and grad_u disagree on the atom count")
    _check(_lib.mlip_aggregate_vjp(C.byref(g), _ptr(agg["e"]), _ptr(agg["s"]), _ptr(W_e), _ptr(W_d), _ptr(W_u),
                                   int(W_e.shape[0]), De, Dn, float(cutoff), _ptr(grad_u), _ptr(out["grad_h"]),
                                   _ptr(out["grad_pos"]), _ptr(struct_ptr), B, _ptr(out.get("atom_virial")),
                                   _ptr(out.get("grad_strain")), _ptr(ws), ws.numel(), _stream()))
    return out


def mlip_moe_status(ws: torch.Tensor) -> bool:
    """True when the last MoE forward with this workspace saw an out-of-range element type."""
    bad = C.c_int32(0)
    _check(_lib.mlip_moe_status(_ptr(ws), C.byref(bad), _stream()))
    return bool(bad.value)


def mlip_readout(h_out, w_r, struct_ptr, out: Optional[Dict] = None) -> Dict[str, torch.Tensor]:
    N, Dn = int(h_out.shape[0]), int(h_out.shape[1])
    B = int(struct_ptr.shape[0]) - 1
    dev = h_out.device
    if out is None:
        out = dict(eps=torch.empty(N, dtype=torch.float32, device=dev),
                   energy=torch.empty(B, dtype=torch.float64, device=dev))
    _check(_lib.mlip_readout(_ptr(h_out), _ptr(w_r), _ptr(struct_ptr), N, B, Dn, _ptr(out["eps"]),
                             _ptr(out["energy"]), _stream()))
    return out


def mlip_block_vjp(graph, agg, moe, z, W_e, W_d, W_u, W1, W2, cutoff: float, top_k: int,
                   grad_out, struct_ptr=None, out: Optional[Dict] = None,
                   ws: Optional[torch.Tensor] = None, keep: bool = False) -> Dict[str, torch.Tensor]:
    """Input gradient; with ``keep`` also out["ubar"] and out["Q"] for the training gradient."""
    N, Dn = int(grad_out.shape[0]), int(grad_out.shape[1])
    De = int(W_e.shape[1])
    H = int(W1.shape[2])
    X = int(W1.shape[0])
    T = int(moe["gate"].shape[0])
    E = int(graph["n_edges"])
    dev = grad_out.device
    B = int(struct_ptr.shape[0]) - 1 if struct_ptr is not None else 0
    if out is None:
        out = dict(grad_h=torch.empty((N, Dn), dtype=torch.float32, device=dev),
                   grad_pos=torch.empty((N, 3), dtype=torch.float32, device=dev),
                   atom_virial=torch.empty((N, 6), dtype=torch.float32, device=dev))
        if struct_ptr is not None:
            out["grad_strain"] = torch.empty((B, 6), dtype=torch.float64, device=dev)
    if keep and "ubar" not in out:
        out["ubar"] = torch.empty((N, Dn), dtype=torch.float32, device=dev)
        out["Q"] = torch.empty((N * int(top_k), H), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _ws(_lib.mlip_vjp_workspace_size(N, top_k, De, Dn, H), dev)
    _check(_lib.mlip_block_vjp(_ptr(graph["row_ptr"]), _ptr(graph["src"]), _ptr(graph["geom"]), N, E,
                               _ptr(agg["e"]), _ptr(agg["s"]), _ptr(z), _ptr(moe["gate"]),
                               _ptr(moe["exp_off"]), _ptr(moe["tok_atom"]), _ptr(moe["slot"]),
                               _ptr(moe["P"]), _ptr(W_e), _ptr(W_d), _ptr(W_u), _ptr(W1), _ptr(W2),
                               int(W_e.shape[0]), De, Dn, H, T, X, int(top_k), float(cutoff),
                               _ptr(grad_out), _ptr(out["grad_h"]), _ptr(out["grad_pos"]),
                               _ptr(struct_ptr), B, _ptr(out.get("atom_virial")),
                               _ptr(out.get("grad_strain")), _ptr(out.get("ubar") if keep else None),
                               _ptr(out.get("Q") if keep else None), _ptr(ws), ws.numel(), _stream()))
    return out


def mlip_block_jvp(graph, agg, moe, z, W_e, W_d, W_u, W1, W2, cutoff: float, top_k: int,
                   grad_forces, h_dot=None, want_h_out_dot: bool = True, out: Optional[Dict] = None,
                   ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Forward tangents along x_dot = -grad_forces (and h_dot): a, s_dot, a_dot, u_dot, P_dot, h_out_dot."""
    N, De = int(agg["s"].shape[0]), int(W_e.shape[1])
    Dn, H, X = int(W_u.shape[1]), int(W1.shape[2]), int(W1.shape[0])
    T, k = int(moe["gate"].shape[0]), int(top_k)
    E = int(graph["n_edges"])
    dev = agg["s"].device
    f32 = torch.float32
    if out is None:
        out = dict(a=torch.empty((N, De), dtype=f32, device=dev),
                   s_dot=torch.empty((N, De), dtype=f32, device=dev) if h_dot is not None else None,
                   a_dot=torch.empty((N, De), dtype=f32, device=dev),
                   u_dot=torch.empty((N, Dn), dtype=f32, device=dev),
                   P_dot=torch.empty((N * k, H), dtype=f32, device=dev),
                   h_out_dot=torch.empty((N, Dn), dtype=f32, device=dev) if want_h_out_dot else None)
    need = _lib.mlip_block_jvp_workspace_size(N, k, Dn, H)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    _check(_lib.mlip_block_jvp(_ptr(graph["row_ptr"]), _ptr(graph["src"]), _ptr(graph["geom"]), N, E,
                               _ptr(grad_forces), _ptr(h_dot), _ptr(agg["s"]), _ptr(z), _ptr(moe["gate"]),
                               _ptr(moe["exp_off"]), _ptr(moe["tok_atom"]), _ptr(moe["slot"]),
                               _ptr(moe["P"]), _ptr(W_e), _ptr(W_d), _ptr(W_u), _ptr(W1), _ptr(W2),
                               int(W_e.shape[0]), De, Dn, H, T, X, k, float(cutoff), _ptr(out["a"]),
                               _ptr(out["s_dot"]), _ptr(out["a_dot"]), _ptr(out["u_dot"]),
                               _ptr(out["P_dot"]), _ptr(out["h_out_dot"]), _ptr(ws), ws.numel(),
                               _stream()))
    out["ws"] = ws
    return out


def mlip_block_tangent_vjp(graph, h, agg, moe, jvp, vjp, z, W_e, W_d, W_u, W1, W2, cutoff: float,
                           top_k: int, grad_forces, grad_out, grad_out_dot=None, h_dot=None,
                           want_grad_h_dot: bool = True, out: Optional[Dict] = None,
                           ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Weight gradients (and dL/dh) of the tangent of the block's VJP; ``vjp`` holds ubar and Q."""
    N, De = int(h.shape[0]), int(W_e.shape[1])
    Dn, H, X = int(h.shape[1]), int(W1.shape[2]), int(W1.shape[0])
    T, k = int(moe["gate"].shape[0]), int(top_k)
    E = int(graph["n_edges"])
    dev = h.device
    f32 = torch.float32
    if out is None:
        out = dict(d_W_e=torch.empty(tuple(W_e.shape), dtype=f32, device=dev),
                   d_W_d=torch.empty(tuple(W_d.shape), dtype=f32, device=dev),
                   d_W_u=torch.empty(tuple(W_u.shape), dtype=f32, device=dev),
                   d_W1=torch.empty(tuple(W1.shape), dtype=f32, device=dev),
                   d_W2=torch.empty(tuple(W2.shape), dtype=f32, device=dev),
                   d_gate=torch.empty((T, k), dtype=f32, device=dev),
                   d_logits=torch.empty((T, X), dtype=f32, device=dev),
                   grad_h_dot=torch.empty((N, Dn), dtype=f32, device=dev) if want_grad_h_dot else None)
    need = _lib.mlip_block_tangent_vjp_workspace_size(N, T, k, De, Dn, H)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    _check(_lib.mlip_block_tangent_vjp(
        _ptr(graph["row_ptr"]), _ptr(graph["src"]), _ptr(graph["geom"]), N, E, _ptr(grad_forces),
        _ptr(h_dot), _ptr(h), _ptr(agg["s"]), _ptr(jvp["s_dot"]), _ptr(jvp["a"]), _ptr(jvp["a_dot"]),
        _ptr(agg["u"]), _ptr(jvp["u_dot"]), _ptr(z), _ptr(moe["topk"]), _ptr(moe["gate"]),
        _ptr(moe["exp_off"]), _ptr(moe["tok_atom"]), _ptr(moe["slot"]), _ptr(moe["P"]), _ptr(jvp["P_dot"]),
        _ptr(grad_out), _ptr(vjp["ubar"]), _ptr(vjp["Q"]), _ptr(grad_out_dot), _ptr(W_e), _ptr(W_d),
        _ptr(W_u), _ptr(W1), _ptr(W2), int(W_e.shape[0]), De, Dn, H, T, X, k, float(cutoff),
        _ptr(out["grad_h_dot"]), _ptr(out["d_W_e"]), _ptr(out["d_W_d"]), _ptr(out["d_W_u"]),
        _ptr(out["d_W1"]), _ptr(out["d_W2"]), _ptr(out["d_gate"]), _ptr(out["d_logits"]), _ptr(ws),
        ws.numel(), _stream()))
    out["ws"] = ws
    return out


def mlip_readout_vjp(w_r, struct_ptr, n_atoms: int, grad_energy=None,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """grad_h_out_i = grad_energy[b(i)] w_r (grad_energy None: w_r)."""
    Dn = int(w_r.shape[0])
    B = int(struct_ptr.shape[0]) - 1
    if out is None:
        out = torch.empty((int(n_atoms), Dn), dtype=torch.float32, device=w_r.device)
    _check(_lib.mlip_readout_vjp(_ptr(w_r), _ptr(grad_energy), _ptr(struct_ptr), int(n_atoms), B, Dn,
                                 _ptr(out), _stream()))
    return out


def mlip_readout_grad(h_out, struct_ptr, grad_energy=None, h_out_dot=None,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """d_w_r = sum_i grad_energy[b(i)] h_out_i + h_out_dot_i."""
    N, Dn = int(h_out.shape[0]), int(h_out.shape[1])
    B = int(struct_ptr.shape[0]) - 1
    if out is None:
        out = torch.empty(Dn, dtype=torch.float32, device=h_out.device)
    ws = _ws(_lib.mlip_readout_grad_workspace_size(N, Dn), h_out.device)
    _check(_lib.mlip_readout_grad(_ptr(h_out), _ptr(h_out_dot), _ptr(grad_energy), _ptr(struct_ptr), N, B,
                                  Dn, _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out


def mlip_moe_vjp(moe, z, W1, W2, grad_out, out: Optional[torch.Tensor] = None,
                 ws: Optional[torch.Tensor] = None, q_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dL/du of h' = u + MoE(u) for grad_out = dL/dh' (moe: the layer's forward state);
    q_out (optional) keeps Q = grad_out[tok] W2^T for the training tangents."""
    N, Dn = int(grad_out.shape[0]), int(grad_out.shape[1])
    X, H = int(W1.shape[0]), int(W1.shape[2])
    T, k = int(moe["gate"].shape[0]), int(moe["gate"].shape[1])
    dev = grad_out.device
    if out is None:
        out = torch.empty((N, Dn), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _ws(_lib.mlip_moe_vjp_workspace_size(N, k, Dn, H), dev)
    _check(_lib.mlip_moe_vjp(_ptr(z), _ptr(moe["gate"]), _ptr(moe["exp_off"]), _ptr(moe["tok_atom"]),
                             _ptr(moe["slot"]), _ptr(moe["P"]), _ptr(W1), _ptr(W2), N, T, X, k, Dn, H,
                             _ptr(grad_out), _ptr(out), _ptr(q_out), _ptr(ws), ws.numel(), _stream()))
    return out


def mlip_moe_jvp(moe, z, W1, W2, u_dot, want_h_out_dot: bool = True, out: Optional[Dict] = None,
                 ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Forward tangent of one MoE layer: P_dot and h_out_dot = u_dot + sum gate silu'(P) P_dot W2."""
    N, Dn = int(u_dot.shape[0]), int(u_dot.shape[1])
    X, H = int(W1.shape[0]), int(W1.shape[2])
    T, k = int(moe["gate"].shape[0]), int(moe["gate"].shape[1])
    dev = u_dot.device
    if out is None:
        out = dict(P_dot=torch.empty((N * k, H), dtype=torch.float32, device=dev),
                   h_out_dot=torch.empty((N, Dn), dtype=torch.float32, device=dev) if want_h_out_dot else None)
    need = _lib.mlip_moe_jvp_workspace_size(N, k, Dn, H)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    _check(_lib.mlip_moe_jvp(_ptr(z), _ptr(moe["gate"]), _ptr(moe["exp_off"]), _ptr(moe["tok_atom"]),
                             _ptr(moe["slot"]), _ptr(moe["P"]), _ptr(W1), _ptr(W2), N, T, X, k, Dn, H,
                             _ptr(u_dot), _ptr(out["P_dot"]), _ptr(out["h_out_dot"]), _ptr(ws), ws.numel(),
                             _stream()))
    out["ws"] = ws
    return out


def mlip_moe_tangent_vjp(moe, z, W1, W2, u, u_dot, P_dot, grad_out, Q, grad_out_dot=None,
                         want_grad_in_dot: bool = True, out: Optional[Dict] = None,
                         ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Tangent of one MoE layer's gradient: grad_in_dot, d_W1, d_W2, d_gate, d_logits."""
    N, Dn = int(u.shape[0]), int(u.shape[1])
    X, H = int(W1.shape[0]), int(W1.shape[2])
    T, k = int(moe["gate"].shape[0]), int(moe["gate"].shape[1])
    dev = u.device
    f32 = torch.float32
    if out is None:
        out = dict(grad_in_dot=torch.empty((N, Dn), dtype=f32, device=dev) if want_grad_in_dot else None,
                   d_W1=torch.empty(tuple(W1.shape), dtype=f32, device=dev),
                   d_W2=torch.empty(tuple(W2.shape), dtype=f32, device=dev),
                   d_gate=torch.empty((T, k), dtype=f32, device=dev),
                   d_logits=torch.empty((T, X), dtype=f32, device=dev))
    need = _lib.mlip_moe_tangent_vjp_workspace_size(N, T, k, Dn, H)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    _check(_lib.mlip_moe_tangent_vjp(_ptr(z), _ptr(moe["topk"]), _ptr(moe["gate"]), _ptr(moe["exp_off"]),
                                     _ptr(moe["tok_atom"]), _ptr(moe["slot"]), _ptr(moe["P"]), _ptr(P_dot),
                                     _ptr(W1), _ptr(W2), N, T, X, k, Dn, H, _ptr(u), _ptr(u_dot),
                                     _ptr(grad_out), _ptr(Q), _ptr(grad_out_dot), _ptr(out["grad_in_dot"]),
                                     _ptr(out["d_W1"]), _ptr(out["d_W2"]), _ptr(out["d_gate"]),
                                     _ptr(out["d_logits"]), _ptr(ws), ws.numel(), _stream()))
    out["ws"] = ws
    return out


def mlip_attention_jvp(graph, att, h0_dot, W_qkv, Wa_e, W_o, n_heads: int, cutoff: float, grad_forces,
                       out: Optional[Dict] = None) -> Dict[str, torch.Tensor]:
    """Forward tangent of the attention: qkv_dot, o_dot, tstat, u_dot."""
    N, Dn = int(h0_dot.shape[0]), int(h0_dot.shape[1])
    Da = int(W_o.shape[0])
    E = int(graph["n_edges"])
    dev = h0_dot.device
    f32 = torch.float32
    if out is None:
        out = dict(qkv_dot=torch.empty((N, 3 * Da), dtype=f32, device=dev),
                   o_dot=torch.empty((N, Da), dtype=f32, device=dev),
                   tstat=torch.empty((N, int(n_heads)), dtype=f32, device=dev),
                   u_dot=torch.empty((N, Dn), dtype=f32, device=dev))
    _check(_lib.mlip_attention_jvp(_ptr(graph["row_ptr"]), _ptr(graph["src"]), _ptr(graph["geom"]), N, E,
                                   _ptr(grad_forces), _ptr(h0_dot), _ptr(att["qkv"]), _ptr(att["o"]),
                                   _ptr(att["stats"]), _ptr(W_qkv), _ptr(Wa_e), _ptr(W_o), int(Wa_e.shape[0]),
                                   Dn, Da, int(n_heads), float(cutoff), _ptr(out["qkv_dot"]),
                                   _ptr(out["o_dot"]), _ptr(out["tstat"]), _ptr(out["u_dot"]), _stream()))
    return out


def mlip_attention_tangent_vjp(graph, att, ajvp, h0, h0_dot, qkv_bar, W_qkv, Wa_e, W_o, n_heads: int,
                               cutoff: float, grad_forces, grad_u, grad_u_dot, want_grad_h0_dot: bool = True,
                               out: Optional[Dict] = None, ws: Optional[torch.Tensor] = None):
    """Tangent of the attention's gradient: grad_h0_dot, d_W_qkv, d_Wa_e, d_W_o."""
    N, Dn = int(h0.shape[0]), int(h0.shape[1])
    Da = int(W_o.shape[0])
    E = int(graph["n_edges"])
    dev = h0.device
    f32 = torch.float32
    if out is None:
        out = dict(grad_h0_dot=torch.empty((N, Dn), dtype=f32, device=dev) if want_grad_h0_dot else None,
                   d_W_qkv=torch.empty(tuple(W_qkv.shape), dtype=f32, device=dev),
                   d_Wa_e=torch.empty(tuple(Wa_e.shape), dtype=f32, device=dev),
                   d_W_o=torch.empty(tuple(W_o.shape), dtype=f32, device=dev))
    need = _lib.mlip_attention_tangent_vjp_workspace_size(N, E, Dn, Da, int(n_heads))
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    _check(_lib.mlip_attention_tangent_vjp(
        _ptr(graph["row_ptr"]), _ptr(graph["src"]), _ptr(graph["rev"]), _ptr(graph["geom"]), N, E,
        _ptr(grad_forces), _ptr(h0), _ptr(h0_dot), _ptr(att["qkv"]), _ptr(ajvp["qkv_dot"]), _ptr(att["o"]),
        _ptr(ajvp["o_dot"]), _ptr(att["stats"]), _ptr(ajvp["tstat"]), _ptr(qkv_bar), _ptr(W_qkv), _ptr(Wa_e),
        _ptr(W_o), int(Wa_e.shape[0]), Dn, Da, int(n_heads), float(cutoff), _ptr(grad_u), _ptr(grad_u_dot),
        _ptr(out["grad_h0_dot"]), _ptr(out["d_W_qkv"]), _ptr(out["d_Wa_e"]), _ptr(out["d_W_o"]), _ptr(ws),
        ws.numel(), _stream()))
    out["ws"] = ws
    return out


def mlip_attention(graph, h0, W_qkv, Wa_e, W_o, n_heads: int, cutoff: float,
                   out: Optional[Dict] = None, ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    N, Dn = int(h0.shape[0]), int(h0.shape[1])
    Da = int(W_o.shape[0])
    E = int(graph["n_edges"])
    dev = h0.device
    need = _lib.mlip_attention_workspace_size(N, Da)
    if ws is None and out is not None:
        ws = out.get("ws")
    if need and (ws is None or ws.numel() < need):
        ws = _ws(need, dev)
    if out is None:
        out = dict(qkv=torch.empty((N, 3 * Da), dtype=torch.float32, device=dev),
                   o=torch.empty((N, Da), dtype=torch.float32, device=dev),
                   stats=torch.empty((N, int(n_heads), 2), dtype=torch.float32, device=dev),
                   u=torch.empty((N, Dn), dtype=torch.float32, device=dev))
    _check(_lib.mlip_attention(_ptr(graph["row_ptr"]), _ptr(graph["src"]), _ptr(graph["geom"]), N, E,
                               _ptr(h0), _ptr(W_qkv), _ptr(Wa_e), _ptr(W_o), int(Wa_e.shape[0]), Dn,
                               Da, int(n_heads), float(cutoff), _ptr(out["qkv"]), _ptr(out["o"]),
                               _ptr(out["stats"]), _ptr(out["u"]), _ptr(ws) if need else None,
                               ws.numel() if need else 0, _stream()))
    out["ws"] = ws if need else None
    return out


def mlip_attention_vjp(graph, att, W_qkv, Wa_e, W_o, n_heads: int, cutoff: float, grad_u,
                       struct_ptr=None, out: Optional[Dict] = None,
                       ws: Optional[torch.Tensor] = None,
                       accumulate: bool = False, keep: bool = False) -> Dict[str, torch.Tensor]:
    """Attention gradient; with ``keep`` also out["qkv_bar"] for the training tangents."""
    N, Dn = int(grad_u.shape[0]), int(grad_u.shape[1])
    Da = int(W_o.shape[0])
    E = int(graph["n_edges"])
    dev = grad_u.device
    B = int(struct_ptr.shape[0]) - 1 if struct_ptr is not None else 0
    if out is None:
        out = dict(grad_h0=torch.empty((N, Dn), dtype=torch.float32, device=dev),
                   grad_pos=torch.empty((N, 3), dtype=torch.float32, device=dev),
                   atom_virial=torch.empty((N, 6), dtype=torch.float32, device=dev))
        if struct_ptr is not None:
            out["grad_strain"] = torch.empty((B, 6), dtype=torch.float64, device=dev)
    if ws is None or ws.numel() < _lib.mlip_attention_vjp_workspace_size(N, E, Da, int(n_heads)):
        ws = _ws(_lib.mlip_attention_vjp_workspace_size(N, E, Da, int(n_heads)), dev)
    out["ws"] = ws
    if keep and out.get("qkv_bar") is None:
        out["qkv_bar"] = torch.empty((N, 3 * Da), dtype=torch.float32, device=dev)
    _check(_lib.mlip_attention_vjp(_ptr(graph["row_ptr"]), _ptr(graph["src"]), _ptr(graph["rev"]),
                                   _ptr(graph["geom"]), N, E, _ptr(att["qkv"]), _ptr(att["o"]),
                                   _ptr(att["stats"]), _ptr(W_qkv), _ptr(Wa_e), _ptr(W_o),
                                   int(Wa_e.shape[0]), Dn, Da, int(n_heads), float(cutoff),
                                   _ptr(grad_u), _ptr(out["grad_h0"]), _ptr(out["grad_pos"]),
                                   _ptr(struct_ptr), B, _ptr(out.get("atom_virial")),
                                   _ptr(out.get("grad_strain")), 1 if accumulate else 0,
                                   _ptr(out.get("qkv_bar") if keep else None), _ptr(ws),
                                   ws.numel(), _stream()))
    return out


def mlip_embed_atoms(z, table, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    N = int(z.shape[0])
    T, Dn = int(table.shape[0]), int(table.shape[1])
    if out is None:
        out = torch.empty((N, Dn), dtype=torch.float32, device=table.device)
    _check(_lib.mlip_embed_atoms(_ptr(z), _ptr(table), N, T, Dn, _ptr(out), _stream()))
    return out


def mlip_embed_grad(z, grad_h, n_types: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """d_table[t] = sum of grad_h over the atoms of type t."""
    N, Dn = int(grad_h.shape[0]), int(grad_h.shape[1])
    if out is None:
        out = torch.empty((int(n_types), Dn), dtype=torch.float32, device=grad_h.device)
    _check(_lib.mlip_embed_grad(_ptr(z), _ptr(grad_h), N, int(n_types), Dn, _ptr(out), _stream()))
    return out


def mlip_tri(graph, h, W_s, W_ang, W_T, cutoff: float, out: Optional[Dict] = None,
             ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    N, Dn = int(h.shape[0]), int(h.shape[1])
    Dt = int(W_s.shape[1])
    E = int(graph["n_edges"])
    dev = h.device
    need = _lib.mlip_tri_workspace_size(N, Dt)
    if ws is None and out is not None:
        ws = out.get("ws")
    if need and (ws is None or ws.numel() < need):
        ws = _ws(need, dev)
    if out is None:
        out = dict(s=torch.empty((N, Dt), dtype=torch.float32, device=dev),
                   tau=torch.empty((N, Dt), dtype=torch.float32, device=dev),
                   h_T=torch.empty((N, Dn), dtype=torch.float32, device=dev))
    _check(_lib.mlip_tri(_ptr(graph["row_ptr"]), _ptr(graph["src"]), _ptr(graph["geom"]), N, E, _ptr(h),
                         _ptr(W_s), _ptr(W_ang), _ptr(W_T), int(W_ang.shape[0]), Dn, Dt, float(cutoff),
                         _ptr(out["s"]), _ptr(out["tau"]), _ptr(out["h_T"]), _ptr(ws) if need else None,
                         ws.numel() if need else 0, _stream()))
    out["ws"] = ws if need else None
    return out


def mlip_tri_vjp(graph, tri, W_s, W_ang, W_T, cutoff: float, grad_hT, grad_pos, atom_virial=None,
                 grad_strain=None, struct_ptr=None, accumulate: bool = False,
                 out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                 sbar_out: Optional[torch.Tensor] = None):
    """dL/dh of the three-body update; grad_pos / atom_virial are written, or added
    to when ``accumulate`` (then grad_strain is recomputed from atom_virial)."""
    N, Dn = int(grad_hT.shape[0]), int(grad_hT.shape[1])
    Dt = int(W_s.shape[1])
    E = int(graph["n_edges"])
    dev = grad_hT.device
    B = int(struct_ptr.shape[0]) - 1 if struct_ptr is not None else 0
    if out is None:
        out = torch.empty((N, Dn), dtype=torch.float32, device=dev)
    need = _lib.mlip_tri_vjp_workspace_size(N, E, Dt)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    _check(_lib.mlip_tri_vjp(_ptr(graph["row_ptr"]), _ptr(graph["src"]), _ptr(graph["rev"]),
                             _ptr(graph["geom"]), N, E, _ptr(tri["s"]), _ptr(W_s), _ptr(W_ang), _ptr(W_T),
                             int(W_ang.shape[0]), Dn, Dt, float(cutoff), _ptr(grad_hT), _ptr(out),
                             _ptr(grad_pos), _ptr(struct_ptr), B, _ptr(atom_virial), _ptr(grad_strain),
                             1 if accumulate else 0, _ptr(sbar_out), _ptr(ws), ws.numel(), _stream()))
    return out, ws


def mlip_tri_jvp(graph, tri, W_s, W_ang, W_T, cutoff: float, grad_forces, h_dot=None,
                 out: Optional[Dict] = None) -> Dict[str, torch.Tensor]:
    """Forward tangent of the three-body update: s_dot (with h_dot), tau_dot, hT_dot."""
    N, Dt = int(tri["s"].shape[0]), int(W_s.shape[1])
    Dn = int(W_s.shape[0])
    E = int(graph["n_edges"])
    dev = tri["s"].device
    f32 = torch.float32
    if out is None:
        out = dict(s_dot=torch.empty((N, Dt), dtype=f32, device=dev) if h_dot is not None else None,
                   tau_dot=torch.empty((N, Dt), dtype=f32, device=dev),
                   hT_dot=torch.empty((N, Dn), dtype=f32, device=dev))
    _check(_lib.mlip_tri_jvp(_ptr(graph["row_ptr"]), _ptr(graph["src"]), _ptr(graph["geom"]), N, E,
                             _ptr(grad_forces), _ptr(h_dot), _ptr(tri["s"]), _ptr(W_s), _ptr(W_ang), _ptr(W_T),
                             int(W_ang.shape[0]), Dn, Dt, float(cutoff), _ptr(out["s_dot"]), _ptr(out["tau_dot"]),
                             _ptr(out["hT_dot"]), _stream()))
    return out


def mlip_tri_tangent_vjp(graph, tri, tjvp, h, sbar, W_s, W_ang, W_T, cutoff: float, grad_forces, grad_hT,
                         grad_hT_dot, h_dot=None, want_grad_h_dot: bool = True, out: Optional[Dict] = None,
                         ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Tangent of the three-body update's gradient: grad_h_dot, d_W_s, d_W_ang, d_W_T."""
    N, Dn = int(h.shape[0]), int(h.shape[1])
    Dt = int(W_s.shape[1])
    E = int(graph["n_edges"])
    dev = h.device
    f32 = torch.float32
    if out is None:
        out = dict(grad_h_dot=torch.empty((N, Dn), dtype=f32, device=dev) if want_grad_h_dot else None,
                   d_W_s=torch.empty(tuple(W_s.shape), dtype=f32, device=dev),
                   d_W_ang=torch.empty(tuple(W_ang.shape), dtype=f32, device=dev),
                   d_W_T=torch.empty(tuple(W_T.shape), dtype=f32, device=dev))
    need = _lib.mlip_tri_tangent_vjp_workspace_size(N, E, Dn, Dt)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    _check(_lib.mlip_tri_tangent_vjp(
        _ptr(graph["row_ptr"]), _ptr(graph["src"]), _ptr(graph["rev"]), _ptr(graph["geom"]), N, E,
        _ptr(grad_forces), _ptr(h), _ptr(h_dot), _ptr(tri["s"]), _ptr(tjvp["s_dot"]), _ptr(tri["tau"]),
        _ptr(tjvp["tau_dot"]), _ptr(sbar), _ptr(W_s), _ptr(W_ang), _ptr(W_T), int(W_ang.shape[0]), Dn, Dt,
        float(cutoff), _ptr(grad_hT), _ptr(grad_hT_dot), _ptr(out["grad_h_dot"]), _ptr(out["d_W_s"]),
        _ptr(out["d_W_ang"]), _ptr(out["d_W_T"]), _ptr(ws), ws.numel(), _stream()))
    out["ws"] = ws
    return out


# ------------------------------------------------------------------ timing
def profile_enable(on: bool = True):
    _check(_lib.mlip_profile_enable(1 if on else 0))


def profile_select(names=None):
    """Time only the kernel classes named (None: every class)."""
    if names is None:
        mask = (1 << 64) - 1
    else:
        idx = {}
        for i in range(_lib.mlip_profile_count()):
            nm = C.c_char_p()
            _check(_lib.mlip_profile_get(i, C.byref(nm), None, None))
            idx[nm.value.decode()] = i
        mask = 0
        for n in names:
            mask |= 1 << idx[n]
    _check(_lib.mlip_profile_select(C.c_uint64(mask)))


def profile_reset():
    _check(_lib.mlip_profile_reset())


def profile_read() -> Dict[str, Dict[str, float]]:
    res = {}
    for i in range(_lib.mlip_profile_count()):
        name = C.c_char_p()
        n = C.c_int64()
        ms = C.c_double()
        _check(_lib.mlip_profile_get(i, C.byref(name), C.byref(n), C.byref(ms)))
        res[name.value.decode()] = dict(launches=int(n.value), total_ms=float(ms.value))
    return res


# ------------------------------------------------------------ one block step
class Block:
    """Device-resident inputs and buffers of one interaction block.

    ``step()`` runs the whole path on the current stream: radius graph,
    aggregation, mixture of experts, readout and the input gradient for the
    given upstream gradient (node features, positions and strain).  The edge
    features are kept in memory only with ``store_edge_features`` (the input
    gradient rebuilds them otherwise).
    """

    def __init__(self, inputs: Dict, device="cuda", grad_out=None, store_edge_features: bool = False,
                 train: bool = False):
        def dev(x, dt=None):
            t = torch.from_numpy(x) if not isinstance(x, torch.Tensor) else x
            return t.to(device=device, dtype=dt or t.dtype).contiguous()

        self.device = device
        self.pos = dev(inputs["pos"], torch.float32)
        self.cell = dev(inputs["cell"], torch.float32)
        self.struct_ptr = dev(inputs["struct_ptr"], torch.int32)
        self.z = dev(inputs["z"], torch.int32)
        self.h = dev(inputs["h"], torch.float32)
        self.logits = dev(inputs["logits"], torch.float32)
        self.W_e = dev(inputs["W_e"], torch.float32)
        self.W_d = dev(inputs["W_d"], torch.float32)
        self.W_u = dev(inputs["W_u"], torch.float32)
        self.W1 = dev(inputs["W1"], torch.float32)
        self.W2 = dev(inputs["W2"], torch.float32)
        self.w_r = dev(inputs["w_r"], torch.float32)
        self.cutoff = float(inputs["cutoff"])
        self.top_k = int(inputs["top_k"])
        if grad_out is None:
            grad_out = self.w_r.expand(self.h.shape[0], -1)
        self.grad_out = dev(grad_out, torch.float32)
        N, Dn = self.h.shape
        De, H = self.W_e.shape[1], self.W1.shape[2]
        T, X = self.logits.shape
        B = self.cell.shape[0]
        self.graph_state = None      # made on the first build
        self.ws_agg = _ws(_lib.mlip_aggregate_workspace_size(N, De, Dn), device)
        self.ws_moe = _ws(_lib.mlip_moe_forward_vjp_workspace_size(N, T, X, self.top_k, Dn, H), device)
        self.ws_vjp = _ws(_lib.mlip_aggregate_vjp_workspace_size(N, De, Dn), device)
        self.store_e = bool(store_edge_features)
        self.train = bool(train)
        self.graph = self.agg = self.moe = self.ro = self.vjp = None
        self.jvp = self.tan = None

    def _graph(self, build_graph: bool):
        """The radius graph of this step: rebuilt, or (build_graph=False, as a
        model of several blocks on one graph does) the previous step's."""
        if not build_graph and self.graph is not None:
            return self.graph
        if self.graph_state is None:
            self.graph_state = GraphState(self.pos, self.cell, self.struct_ptr, self.cutoff, self.pos.device)
        return self.graph_state.build()

    def _graph_done(self, build_graph: bool) -> bool:
        """After the step is queued: False when its graph build overflowed (the
        step is then run again on a rebuilt graph)."""
        if self.graph_state is None:
            return True
        ok = self.graph_state.check()
        self.graph = self.graph_state.graph if ok else None
        return ok

    def step(self, build_graph: bool = True):
        g = self._graph(build_graph)
        reuse = self.agg
        if reuse is not None and reuse["e"] is not None and reuse["e"].shape[0] != g["n_edges"]:
            reuse = None
        self.graph = g
        self.agg = mlip_aggregate(g, self.h, self.W_e, self.W_d, self.W_u, self.cutoff,
                                  out=reuse, ws=self.ws_agg, store_e=self.store_e)
        # the upstream gradient is known before the forward: the MoE forward and
        # its gradient run in one call (the forward's second expert GEMM and the
        # gradient's first share a launch), then the aggregation's gradient
        self.moe = mlip_moe_forward_vjp(self.agg["u"], self.z, self.logits, self.W1, self.W2, self.top_k,
                                        self.grad_out, out=self.moe, ws=self.ws_moe, keep=self.train)
        self.ro = mlip_readout(self.moe["h_out"], self.w_r, self.struct_ptr, out=self.ro)
        self.vjp = mlip_aggregate_vjp(g, self.agg, self.W_e, self.W_d, self.W_u, self.cutoff,
                                      self.moe["grad_u"], struct_ptr=self.struct_ptr, out=self.vjp,
                                      ws=self.ws_vjp)
        if self.train:
            self.vjp["ubar"], self.vjp["Q"] = self.moe["grad_u"], self.moe["Q"]
        if not self._graph_done(build_graph):
            self.agg = None
            return self.step(True)
        return self

    def train_grad(self, grad_energy, grad_forces) -> Dict[str, torch.Tensor]:
        """Parameter gradients of a loss L(E, F) after ``step()`` (built with
        ``train=True`` and the force seed grad_out = w_r): grad_energy = dL/dE
        [B] float64, grad_forces = dL/dF [N, 3] float32, both on the device.
        Returns d_W_e, d_W_d, d_W_u, d_W1, d_W2, d_logits, d_gate, d_w_r and
        d_h (= dL/dh of the input features)."""
        if not self.train or self.vjp is None:
            raise RuntimeError("train_grad needs Block(train=True) and a step() first")
        g = self.graph
        self.jvp = mlip_block_jvp(g, self.agg, self.moe, self.z, self.W_e, self.W_d, self.W_u, self.W1,
                                  self.W2, self.cutoff, self.top_k, grad_forces,
                                  out=self.jvp, ws=None if self.jvp is None else self.jvp["ws"])
        seed_dot = mlip_readout_vjp(self.w_r, self.struct_ptr, self.h.shape[0], grad_energy=grad_energy)
        self.tan = mlip_block_tangent_vjp(g, self.h, self.agg, self.moe, self.jvp, self.vjp, self.z, self.W_e,
                                          self.W_d, self.W_u, self.W1, self.W2, self.cutoff, self.top_k,
                                          grad_forces, self.grad_out, grad_out_dot=seed_dot, out=self.tan,
                                          ws=None if self.tan is None else self.tan["ws"])
        d_w_r = mlip_readout_grad(self.moe["h_out"], self.struct_ptr, grad_energy=grad_energy,
                                  h_out_dot=self.jvp["h_out_dot"])
        res = {k: v for k, v in self.tan.items() if k not in ("ws", "grad_h_dot")}
        res["d_h"] = self.tan["grad_h_dot"]
        res["d_w_r"] = d_w_r
        return res


class FullBlock:
    """The complete interaction block: Tri -> MoE0 -> neighbour attention -> MoE1.

    ``step()`` runs on the current stream: radius graph, the three-body update
    (when the parameters include it), MoE0, attention, MoE1, readout, then
    the input gradient back through MoE1, the attention, MoE0 and Tri
    (forces and virial of both geometric operators) for the given upstream
    gradient dL/dh'.  ``forward`` / ``backward`` run one block on a given
    graph, as the layers of a ``Stack`` do.
    """

    def __init__(self, inputs: Dict, device="cuda", grad_out=None, params: Optional[Dict] = None,
                 train: bool = False):
        def dev(x, dt=None):
            t = torch.from_numpy(x) if not isinstance(x, torch.Tensor) else x
            return t.to(device=device, dtype=dt or t.dtype).contiguous()

        self.device = device
        self.train = bool(train)
        f32 = torch.float32
        params = inputs if params is None else params
        self.pos = dev(inputs["pos"], f32)
        self.cell = dev(inputs["cell"], f32)
        self.struct_ptr = dev(inputs["struct_ptr"], torch.int32)
        self.z = dev(inputs["z"], torch.int32)
        self.h = dev(inputs["h"], f32) if "h" in inputs else None
        self.logits0 = dev(params["logits0"], f32)
        self.W1_0 = dev(params["W1_0"], f32)
        self.W2_0 = dev(params["W2_0"], f32)
        self.W_qkv = dev(params["W_qkv"], f32)
        self.Wa_e = dev(params["Wa_e"], f32)
        self.W_o = dev(params["W_o"], f32)
        self.logits = dev(params["logits"], f32)
        self.W1 = dev(params["W1"], f32)
        self.W2 = dev(params["W2"], f32)
        self.w_r = dev(inputs["w_r"], f32)
        self.cutoff = float(inputs["cutoff"])
        self.top_k = int(inputs["top_k"])
        self.n_heads = int(inputs["n_heads"])
        self.has_tri = "W_ang" in params
        if self.has_tri:
            self.W_s = dev(params["W_s"], f32)
            self.W_ang = dev(params["W_ang"], f32)
            self.W_T = dev(params["W_T"], f32)
        N = int(self.z.shape[0])
        Dn = int(self.W_o.shape[1])
        if grad_out is None:
            grad_out = self.w_r.expand(N, -1)
        self.grad_out = dev(grad_out, f32)
        H = self.W1.shape[2]
        T, X = self.logits.shape
        B = self.cell.shape[0]
        self.graph_state = None      # made on the first build
        self.ws_moe0 = _ws(_lib.mlip_moe_workspace_size(N, T, X, self.top_k, Dn, H), device)
        self.ws_moe1 = _ws(_lib.mlip_moe_workspace_size(N, T, X, self.top_k, Dn, H), device)
        self.ws_mvjp = _ws(_lib.mlip_moe_vjp_workspace_size(N, self.top_k, Dn, H), device)
        self.ws_moe1f = None         # MoE1 forward + gradient in one call (made on first use)
        self.ubar_ready = False
        self.ws_avjp = self.ws_tvjp = None
        self.graph = self.tri = self.moe0 = self.att = self.moe = self.ro = None
        self.ubar = self.avjp = self.grad_hT = self.grad_h = None
        self.g_up = self.Q0 = self.Q1 = self.tri_sbar = None
        self.h_in = None
        if self.train:
            M = N * self.top_k
            self.Q0 = torch.empty((M, H), dtype=f32, device=device)
            self.Q1 = torch.empty((M, H), dtype=f32, device=device)
            if self.has_tri:
                self.tri_sbar = torch.empty((N, int(self.W_s.shape[1])), dtype=f32, device=device)

    def forward(self, g, h, grad_out=None):
        """One block on graph g for input features h; returns h' (MoE1 output).
        With grad_out (dL/dh', known before the forward under a linear
        readout) MoE1's input gradient is formed in the same call, and
        ``backward`` with that grad_out starts from it."""
        self.h_in = h
        if self.has_tri:
            self.tri = mlip_tri(g, h, self.W_s, self.W_ang, self.W_T, self.cutoff, out=self.tri)
            h = self.tri["h_T"]
        self.moe0 = mlip_moe_forward(h, self.z, self.logits0, self.W1_0, self.W2_0, self.top_k,
                                     out=self.moe0, ws=self.ws_moe0)
        self.att = mlip_attention(g, self.moe0["h_out"], self.W_qkv, self.Wa_e, self.W_o,
                                  self.n_heads, self.cutoff, out=self.att)
        if grad_out is None:
            self.moe = mlip_moe_forward(self.att["u"], self.z, self.logits, self.W1, self.W2, self.top_k,
                                        out=self.moe, ws=self.ws_moe1)
            self.ubar_ready = False
            return self.moe["h_out"]
        if self.ws_moe1f is None:
            N, Dn = int(self.z.shape[0]), int(self.W1.shape[1])
            T, X = int(self.logits.shape[0]), int(self.logits.shape[1])
            self.ws_moe1f = _ws(_lib.mlip_moe_forward_vjp_workspace_size(
                N, T, X, self.top_k, Dn, int(self.W1.shape[2])), grad_out.device)
        out = self.moe if self.moe is not None and "grad_u" in self.moe else None
        self.moe = mlip_moe_forward_vjp(self.att["u"], self.z, self.logits, self.W1, self.W2, self.top_k,
                                        grad_out, out=out, ws=self.ws_moe1f, keep=self.train)
        self.g_up = grad_out
        self.ubar = self.moe["grad_u"]
        if self.train:
            self.Q1 = self.moe["Q"]
        self.ubar_ready = True
        return self.moe["h_out"]

    def backward(self, g, grad_out, forces: Optional[Dict] = None, accumulate: bool = False):
        """Input gradient for grad_out = dL/dh'; forces (grad_pos, atom_virial,
        grad_strain) are written, or added to the given buffers when accumulate."""
        if not (self.ubar_ready and grad_out is self.g_up):
            self.g_up = grad_out
            self.ubar = mlip_moe_vjp(self.moe, self.z, self.W1, self.W2, grad_out, out=self.ubar,
                                     ws=self.ws_mvjp, q_out=self.Q1)
        self.ubar_ready = False
        out = None
        if forces is not None:
            gh0 = self.avjp["grad_h0"] if self.avjp is not None else torch.empty_like(grad_out)
            out = dict(forces, grad_h0=gh0)
        self.avjp = mlip_attention_vjp(g, self.att, self.W_qkv, self.Wa_e, self.W_o, self.n_heads,
                                       self.cutoff, self.ubar, struct_ptr=self.struct_ptr,
                                       out=out if out is not None else self.avjp, ws=self.ws_avjp,
                                       accumulate=accumulate, keep=self.train)
        self.ws_avjp = self.avjp["ws"]
        if self.has_tri:
            self.grad_hT = mlip_moe_vjp(self.moe0, self.z, self.W1_0, self.W2_0, self.avjp["grad_h0"],
                                        out=self.grad_hT, ws=self.ws_mvjp, q_out=self.Q0)
            self.grad_h, self.ws_tvjp = mlip_tri_vjp(
                g, self.tri, self.W_s, self.W_ang, self.W_T, self.cutoff, self.grad_hT,
                self.avjp["grad_pos"], atom_virial=self.avjp["atom_virial"],
                grad_strain=self.avjp["grad_strain"], struct_ptr=self.struct_ptr, accumulate=True,
                out=self.grad_h, ws=self.ws_tvjp, sbar_out=self.tri_sbar)
        else:
            self.grad_h = mlip_moe_vjp(self.moe0, self.z, self.W1_0, self.W2_0, self.avjp["grad_h0"],
                                       out=self.grad_h, ws=self.ws_mvjp, q_out=self.Q0)
        return self.grad_h

    def jvp(self, g, grad_forces, h_dot=None):
        """Forward tangents along x_dot = -grad_forces and h_dot (None: 0) after
        ``forward``; returns h_out_dot."""
        if not self.train:
            raise RuntimeError("tangents need FullBlock(train=True)")
        self.h_dot = h_dot
        if self.has_tri:
            self.tjvp = mlip_tri_jvp(g, self.tri, self.W_s, self.W_ang, self.W_T, self.cutoff, grad_forces,
                                     h_dot=h_dot, out=getattr(self, "tjvp", None))
            hT_dot = self.tjvp["hT_dot"]
        else:
            hT_dot = h_dot if h_dot is not None else torch.zeros_like(self.h_in)
        self.hT_dot = hT_dot
        self.m0jvp = mlip_moe_jvp(self.moe0, self.z, self.W1_0, self.W2_0, hT_dot,
                                  out=getattr(self, "m0jvp", None))
        self.ajvp = mlip_attention_jvp(g, self.att, self.m0jvp["h_out_dot"], self.W_qkv, self.Wa_e, self.W_o,
                                       self.n_heads, self.cutoff, grad_forces, out=getattr(self, "ajvp", None))
        self.m1jvp = mlip_moe_jvp(self.moe, self.z, self.W1, self.W2, self.ajvp["u_dot"],
                                  out=getattr(self, "m1jvp", None))
        return self.m1jvp["h_out_dot"]

    def tangent_vjp(self, g, grad_forces, grad_out_dot) -> Dict[str, torch.Tensor]:
        """Tangent of ``backward`` along (x_dot, h_dot, grad_out_dot) after
        ``jvp``: the parameter gradients of the block and d_h (the tangent of
        dL/dh, i.e. the upstream of the block below)."""
        m1 = mlip_moe_tangent_vjp(self.moe, self.z, self.W1, self.W2, self.att["u"], self.ajvp["u_dot"],
                                  self.m1jvp["P_dot"], self.g_up, self.Q1, grad_out_dot=grad_out_dot,
                                  out=getattr(self, "m1tan", None))
        self.m1tan = m1
        at = mlip_attention_tangent_vjp(g, self.att, self.ajvp, self.moe0["h_out"], self.m0jvp["h_out_dot"],
                                        self.avjp["qkv_bar"], self.W_qkv, self.Wa_e, self.W_o, self.n_heads,
                                        self.cutoff, grad_forces, self.ubar, m1["grad_in_dot"],
                                        out=getattr(self, "atan", None))
        self.atan = at
        hT = self.tri["h_T"] if self.has_tri else self.h_in
        m0 = mlip_moe_tangent_vjp(self.moe0, self.z, self.W1_0, self.W2_0, hT, self.hT_dot,
                                  self.m0jvp["P_dot"], self.avjp["grad_h0"], self.Q0,
                                  grad_out_dot=at["grad_h0_dot"], out=getattr(self, "m0tan", None))
        self.m0tan = m0
        res = dict(d_W1=m1["d_W1"], d_W2=m1["d_W2"], d_logits=m1["d_logits"],
                   d_W_qkv=at["d_W_qkv"], d_Wa_e=at["d_Wa_e"], d_W_o=at["d_W_o"],
                   d_W1_0=m0["d_W1"], d_W2_0=m0["d_W2"], d_logits0=m0["d_logits"], d_h=m0["grad_in_dot"])
        if self.has_tri:
            tt = mlip_tri_tangent_vjp(g, self.tri, self.tjvp, self.h_in, self.tri_sbar, self.W_s, self.W_ang,
                                      self.W_T, self.cutoff, grad_forces, self.grad_hT, m0["grad_in_dot"],
                                      h_dot=self.h_dot, out=getattr(self, "ttan", None))
            self.ttan = tt
            res.update(d_W_s=tt["d_W_s"], d_W_ang=tt["d_W_ang"], d_W_T=tt["d_W_T"], d_h=tt["grad_h_dot"])
        return res

    def train_grad(self, grad_energy, grad_forces) -> Dict[str, torch.Tensor]:
        """Parameter gradients of a loss L(E, F) after ``step()`` (built with
        ``train=True`` and the force seed): grad_energy = dL/dE [B] float64,
        grad_forces = dL/dF [N, 3] float32 on the device."""
        g = self.graph
        h_out_dot = self.jvp(g, grad_forces)
        seed_dot = mlip_readout_vjp(self.w_r, self.struct_ptr, int(self.z.shape[0]), grad_energy=grad_energy)
        res = self.tangent_vjp(g, grad_forces, seed_dot)
        res["d_w_r"] = mlip_readout_grad(self.moe["h_out"], self.struct_ptr, grad_energy=grad_energy,
                                         h_out_dot=h_out_dot)
        return res

    _graph = Block._graph
    _graph_done = Block._graph_done

    def step(self, build_graph: bool = True):
        g = self._graph(build_graph)
        self.graph = g
        h_out = self.forward(g, self.h, grad_out=self.grad_out)
        self.ro = mlip_readout(h_out, self.w_r, self.struct_ptr, out=self.ro)
        self.backward(g, self.grad_out)
        if not self._graph_done(build_graph):
            return self.step(True)
        return self


class Stack:
    """A model of several complete blocks on one radius graph.

    ``step()``: radius graph; h^(0) = element embedding of z; the blocks in
    order; readout of the last block; then the input gradient of the energy
    (or of the given upstream gradient) back through every block, collecting
    forces, per-atom virials and the strain gradient of all blocks.
    Workspaces are shared between blocks (they run one after another).
    """

    def __init__(self, shared: Dict, blocks, device="cuda", grad_out=None, train: bool = False):
        f32 = torch.float32

        def dev(x, dt=None):
            t = torch.from_numpy(x) if not isinstance(x, torch.Tensor) else x
            return t.to(device=device, dtype=dt or t.dtype).contiguous()

        self.layers = [FullBlock(shared, device=device, params=p, grad_out=grad_out, train=train)
                       for p in blocks]
        first = self.layers[0]
        for L in self.layers[1:]:        # one set of workspaces for all layers
            L.ws_moe0, L.ws_moe1, L.ws_mvjp = first.ws_moe0, first.ws_moe1, first.ws_mvjp
        self.emb = dev(shared["emb"], f32)
        self.first = first
        N = int(first.z.shape[0])
        B = int(first.cell.shape[0])
        self.forces = dict(grad_pos=torch.empty((N, 3), dtype=f32, device=device),
                           atom_virial=torch.empty((N, 6), dtype=f32, device=device),
                           grad_strain=torch.empty((B, 6), dtype=torch.float64, device=device))
        self.graph = self.h0 = self.ro = self.grad_h0 = None
        self.graph_state = GraphState(first.pos, first.cell, first.struct_ptr, first.cutoff, device)

    def step(self, build_graph: bool = True):
        L0 = self.first
        g = self.graph_state.build() if (build_graph or self.graph is None) else self.graph
        self.graph = g
        self.h0 = mlip_embed_atoms(L0.z, self.emb, out=self.h0)
        h = self.h0
        for L in self.layers:
            h = L.forward(g, h)
        self.ro = mlip_readout(h, L0.w_r, L0.struct_ptr, out=self.ro)
        grad = L0.grad_out
        for n, L in enumerate(reversed(self.layers)):
            ws_a, ws_t = self.layers[-1].ws_avjp, self.layers[-1].ws_tvjp
            if L is not self.layers[-1]:
                L.ws_avjp, L.ws_tvjp = ws_a, ws_t      # share the per-edge workspaces
            grad = L.backward(g, grad, forces=self.forces, accumulate=n > 0)
        self.grad_h0 = grad
        ok = self.graph_state.check()
        self.graph = self.graph_state.graph if ok else None
        if not ok:
            return self.step(True)
        return self

    def train_grad(self, grad_energy, grad_forces):
        """Parameter gradients of a loss L(E, F) after ``step()`` (built with
        ``train=True`` and the force seed): forward tangents block by block
        (h_dot of a block = h_out_dot of the one below; the embedding does
        not move), then the tangents of the input gradients from the top
        (grad_out_dot of a block = d_h of the one above).  Returns a list of
        per-block gradient dicts and d_emb, d_w_r."""
        g = self.graph
        L0 = self.first
        h_dot = None
        for L in self.layers:
            h_dot = L.jvp(g, grad_forces, h_dot)
        g_dot = mlip_readout_vjp(L0.w_r, L0.struct_ptr, int(L0.z.shape[0]), grad_energy=grad_energy)
        per_block = [None] * len(self.layers)
        for b in range(len(self.layers) - 1, -1, -1):
            per_block[b] = self.layers[b].tangent_vjp(g, grad_forces, g_dot)
            g_dot = per_block[b]["d_h"]
        d_emb = mlip_embed_grad(L0.z, g_dot, int(self.emb.shape[0]))
        d_w_r = mlip_readout_grad(self.layers[-1].moe["h_out"], L0.struct_ptr, grad_energy=grad_energy,
                                  h_out_dot=h_dot)
        return dict(blocks=per_block, d_emb=d_emb, d_w_r=d_w_r)
