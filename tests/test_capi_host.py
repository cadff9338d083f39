"""Host-side checks of the C ABI: the library loads without a GPU, exports
every entry point declared in include/mlip.h, and rejects bad arguments
before touching the device (no kernel is launched by these tests)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlip.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mlip_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def mlip():
    from element_routed_moe_amd import mlip as m
    return m


def test_exports_every_declared_symbol(mlip):
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(mlip._lib, n), n
        assert n in mlip.EXPORTED, n
    assert mlip._lib.mlip_version() == 1


def test_debug_build_exports_the_same_symbols(mlip):
    """The bounds-checked build (libmlip_debug.so) is the same library: it loads
    without a GPU and exports every declared entry point."""
    path = os.path.join(ROOT, "element_routed_moe_amd", "libmlip_debug.so")
    if not os.path.exists(path):
        pytest.skip("debug build not present")
    lib = C.CDLL(path)
    for n in _declared():
        assert hasattr(lib, n), n


def test_workspace_sizes_are_monotone(mlip):
    L = mlip._lib
    assert L.mlip_graph_workspace_size(4096, 32) < L.mlip_graph_workspace_size(8192, 32)
    a = L.mlip_aggregate_workspace_size(4096, 384, 2560)
    assert a >= 4096 * 384 * 4
    m = L.mlip_moe_workspace_size(4096, 16, 72, 4, 2560, 2560)
    assert m >= 2 * 4096 * 4 * 2560 * 4          # SiLU activations + expert outputs
    v = L.mlip_vjp_workspace_size(4096, 4, 384, 2560, 2560)
    assert v >= 2 * 4096 * 4 * 2560 * 4
    for s in (a, m, v):
        assert s % 256 == 0


def _err(mlip, rc, code):
    assert rc == code, (rc, mlip._lib.mlip_last_error())
    return mlip._lib.mlip_last_error().decode()


def test_build_graph_rejects_bad_args(mlip):
    L = mlip._lib
    ne = C.c_int64(0)
    fake = C.c_void_p(256)        # never dereferenced: validation fails first
    rc = L.mlip_build_graph(fake, fake, fake, 10, 0, 5.0, 100, fake, fake, fake, fake, fake,
                            C.byref(ne), fake, 1 << 20, None)
    assert "n_structs" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_build_graph(fake, fake, fake, 10, 1, -1.0, 100, fake, fake, fake, fake, fake,
                            C.byref(ne), fake, 1 << 20, None)
    assert "cutoff" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_build_graph(fake, fake, fake, 10, 1, 5.0, 100, fake, fake, fake, fake, fake,
                            C.byref(ne), fake, 16, None)
    assert "workspace" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)


def test_graph_reverse_rejects_bad_args(mlip):
    L = mlip._lib
    fake = C.c_void_p(256)
    rc = L.mlip_graph_reverse(None, fake, fake, 4, 10, fake, fake, 1 << 20, None)
    assert "row_ptr" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_graph_reverse(fake, None, fake, 4, 10, fake, fake, 1 << 20, None)
    assert "edge arrays" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_graph_reverse(fake, fake, fake, 4, -1, fake, fake, 1 << 20, None)
    assert "out of range" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_graph_reverse(fake, fake, fake, 4, 10, fake, fake, 8, None)
    assert "workspace" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_graph_reverse(fake, fake, C.c_void_p(258), 4, 10, fake, fake, 1 << 20, None)
    assert "aligned" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)


def test_aggregate_static_rejects_oversize_on_host(mlip):
    """The scratch limit is checked before any device call (runs without a GPU)."""
    L = mlip._lib
    f = C.c_void_p(256)
    N, De, Dn = 8192, 384, 2560
    assert L.mlip_aggregate_workspace_size(N, De, Dn) > mlip.AGGREGATE_STATIC_MAX_BYTES
    rc = L.mlip_aggregate_static(f, f, f, N, 1000, f, f, f, f, 16, De, Dn, 6.0, f, f, f, None)
    assert "scratch" in _err(mlip, rc, mlip.MLIP_ERR_UNSUPPORTED)
    rc = L.mlip_aggregate_static(None, f, f, N, 1000, f, f, f, f, 16, De, Dn, 6.0, f, f, f, None)
    _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    hdr = open(HEADER).read()
    assert "#define MLIP_AGGREGATE_STATIC_MAX_BYTES ((size_t)32 << 20)" in hdr
    assert mlip.AGGREGATE_STATIC_MAX_BYTES == 32 << 20


def test_aggregate_and_moe_reject_bad_args(mlip):
    L = mlip._lib
    f = C.c_void_p(256)
    rc = L.mlip_aggregate(f, f, f, 10, 20, f, f, f, f, 8, 32, 64, 5.0, f, f, f, f, 1 << 30, None)
    assert "n_rbf" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_aggregate(f, f, f, 10, 20, f, f, f, f, 16, 30, 64, 5.0, f, f, f, f, 1 << 30, None)
    assert "d_edge" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_moe_forward(f, f, f, f, f, 10, 4, 3, 4, 64, 128, f, f, f, f, f, f, f, f, 1 << 30, None)
    assert "top_k" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_moe_forward(f, f, f, f, f, 10, 4, 8, 2, 64, 128, f, f, f, f, f, f, f, None, 0, None)
    assert "workspace" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    def vjp(d_hidden, struct_ptr, n_structs, grad_strain):
        # graph (3), sizes (2), saved state (8), weights (5), dims (7), cutoff,
        # grad_out/grad_h/grad_pos, struct_ptr/n_structs, atom_virial/grad_strain, ws
        return L.mlip_block_vjp(f, f, f, 10, 20, f, f, f, f, f, f, f, f, f, f, f, f, f,
                                16, 32, 64, d_hidden, 4, 8, 2, 5.0, f, f, f,
                                struct_ptr, n_structs, None, grad_strain, None, None, f, 1 << 30, None)
    rc = vjp(130, None, 0, None)
    assert "d_hidden" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = vjp(128, None, 0, f)
    assert "grad_strain" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)


def test_struct_arguments(mlip):
    """mlip_graph / mlip_moe_state: the binding's ctypes layout matches the
    library's, the fields sit where the header declares them, and a NULL
    struct or a bad field is rejected on the host."""
    L = mlip._lib
    assert L.mlip_struct_size(0) == C.sizeof(mlip._Graph) == 6 * 8 + 8
    assert L.mlip_struct_size(1) == C.sizeof(mlip._MoeState) == 6 * 8
    assert L.mlip_struct_size(2) == 0
    assert mlip._Graph.n_edges.offset == 48 and mlip._Graph.n_atoms.offset == 40
    hdr = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    g_fields = re.search(r"typedef struct mlip_graph \{(.*?)\} mlip_graph;", hdr, re.S).group(1)
    assert re.findall(r"(\w+);", g_fields) == [n for n, _ in mlip._Graph._fields_]
    m_fields = re.search(r"typedef struct mlip_moe_state \{(.*?)\} mlip_moe_state;", hdr, re.S).group(1)
    assert re.findall(r"(\w+);", m_fields) == [n for n, _ in mlip._MoeState._fields_]
    f = C.c_void_p(256)
    rc = L.mlip_aggregate_vjp(None, f, f, f, f, f, 16, 32, 64, 5.0, f, f, f, None, 0, None, None, f, 1 << 30, None)
    assert "graph" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    g = mlip._Graph(256, 256, None, None, 256, 10, -1)
    rc = L.mlip_aggregate_vjp(C.byref(g), f, f, f, f, f, 16, 32, 64, 5.0, f, f, f, None, 0, None, None, f,
                              1 << 30, None)
    assert "out of range" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_moe_forward_vjp(f, f, f, f, f, 10, 4, 8, 2, 64, 128, f, None, f, f, None, f, 1 << 30, None)
    assert "MoE state" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    st = mlip._MoeState(256, 256, 256, 256, 256, 256)
    rc = L.mlip_moe_forward_vjp(f, f, f, f, f, 10, 4, 3, 4, 64, 128, f, C.byref(st), f, f, None, f, 1 << 30,
                                None)
    assert "top_k" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)


def test_attention_and_moe_vjp_reject_bad_args(mlip):
    L = mlip._lib
    f = C.c_void_p(256)

    def att(d_attn, n_heads, cutoff=5.0):
        return L.mlip_attention(f, f, f, 10, 20, f, f, f, f, 16, 64, d_attn, n_heads, cutoff,
                                f, f, f, f, None, 0, None)
    assert "n_heads" in _err(mlip, att(32, 3), mlip.MLIP_ERR_INVALID)
    assert "d_attn" in _err(mlip, att(30, 3), mlip.MLIP_ERR_INVALID)
    assert "cutoff" in _err(mlip, att(32, 4, cutoff=0.0), mlip.MLIP_ERR_INVALID)
    # 5 heads of width 20: 20 is not c * 2^j with c in {1, 2, 3, 4, 6, 8}
    assert "unsupported attention shape" in _err(mlip, att(100, 5), mlip.MLIP_ERR_UNSUPPORTED)
    # an optional workspace, when given, must have the size the query reports
    need = L.mlip_attention_workspace_size(4096, 384)
    assert need >= 2 * 4096 * 3 * 384 * 4      # 576 tiles of 64 x 128: the K loop is split
    assert L.mlip_attention_workspace_size(262144, 384) == 0   # enough tiles: never split
    rc = L.mlip_attention(f, f, f, 4096, 20, f, f, f, f, 16, 2560, 384, 8, 5.0, f, f, f, f, f, need - 1, None)
    assert "workspace" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_attention_vjp(f, f, f, f, 10, 20, f, f, f, f, f, f, 16, 64, 32, 4, 5.0, f, f, f,
                              None, 0, None, f, 0, None, f, 1 << 30, None)
    assert "grad_strain" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_attention_vjp(f, f, f, f, 10, 20, f, f, f, f, f, f, 16, 64, 32, 4, 5.0, f, f, f,
                              f, 1, None, f, 1, None, f, 1 << 30, None)
    assert "accumulated atom_virial" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_attention_vjp(f, f, f, f, 10, 20, f, f, f, f, f, f, 16, 64, 32, 4, 5.0, f, f, f,
                              None, 0, None, None, 0, None, f, 16, None)
    assert "workspace" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_embed_atoms(f, f, 10, 0, 64, f, None)
    assert "n_types" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    assert (L.mlip_attention_vjp_workspace_size(4096, 200000, 384, 8)
            >= (200000 * (2 * 8 + 1) + 4096 * 4 * 384) * 4)
    rc = L.mlip_moe_vjp(f, f, f, f, f, f, f, f, 10, 4, 3, 4, 64, 128, f, f, None, f, 1 << 30, None)
    assert "top_k" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_moe_vjp(f, f, f, f, f, f, f, f, 10, 4, 8, 2, 64, 128, f, f, None, f, 16, None)
    assert "workspace" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)


def test_tri_rejects_bad_args(mlip):
    L = mlip._lib
    f = C.c_void_p(256)

    def tri(n_ang=4, d_tri=32, cutoff=5.0):
        return L.mlip_tri(f, f, f, 10, 20, f, f, f, f, n_ang, 64, d_tri, cutoff, f, f, f, None, 0, None)
    assert "n_ang" in _err(mlip, tri(n_ang=3), mlip.MLIP_ERR_INVALID)
    assert "d_tri" in _err(mlip, tri(d_tri=30), mlip.MLIP_ERR_INVALID)
    assert "too wide" in _err(mlip, tri(d_tri=516), mlip.MLIP_ERR_UNSUPPORTED)
    need = L.mlip_tri_workspace_size(4096, 384)
    assert need > 0 and L.mlip_tri_workspace_size(262144, 384) == 0
    rc = L.mlip_tri(f, f, f, 4096, 20, f, f, f, f, 4, 2560, 384, 5.0, f, f, f, f, need - 1, None)
    assert "workspace" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)

    def vjp(accumulate, atom_virial, grad_strain, ws_bytes=1 << 30):
        return L.mlip_tri_vjp(f, f, f, f, 10, 20, f, f, f, f, 4, 64, 32, 5.0, f, f, f, f, 1,
                              atom_virial, grad_strain, accumulate, None, f, ws_bytes, None)
    assert "accumulated atom_virial" in _err(mlip, vjp(1, None, f), mlip.MLIP_ERR_INVALID)
    assert "workspace" in _err(mlip, vjp(0, f, f, 16), mlip.MLIP_ERR_INVALID)
    assert L.mlip_tri_vjp_workspace_size(4096, 200000, 384) >= 200000 * (384 + 4) * 4


def test_profile_api_without_gpu(mlip):
    names = list(mlip.profile_read())
    assert "gemm_expert_up" in names and "edge_vjp" in names and "attn_fwd" in names
    assert "tri_fwd" in names and "tri_vjp_send" in names
    assert "gemm_wgrad" in names and "edge_tan" in names and "moe_tan" in names
    assert "gemm_expert_pair" in names
    assert len(names) == 23


def test_training_entry_points_reject_bad_args(mlip):
    L = mlip._lib
    f = C.c_void_p(256)

    def jvp(h_dot, s_dot, d_hidden=128, ws_bytes=1 << 30):
        # graph (3), sizes (2), grad_forces, h_dot, s, z, gate, exp_off, tok_atom, slot, P,
        # weights (5), dims (7), cutoff, a, s_dot, a_dot, u_dot, P_dot, h_out_dot, ws
        return L.mlip_block_jvp(f, f, f, 10, 20, f, h_dot, f, f, f, f, f, f, f, f, f, f, f, f,
                                16, 32, 64, d_hidden, 4, 8, 2, 5.0, f, s_dot, f, f, f, None, f,
                                ws_bytes, None)
    assert "h_dot needs s_dot" in _err(mlip, jvp(f, None), mlip.MLIP_ERR_INVALID)
    assert "d_hidden" in _err(mlip, jvp(None, None, d_hidden=130), mlip.MLIP_ERR_INVALID)
    assert "workspace" in _err(mlip, jvp(None, None, ws_bytes=16), mlip.MLIP_ERR_INVALID)

    def tan(top_k=2, d_W1=f, ws_bytes=1 << 30):
        return L.mlip_block_tangent_vjp(f, f, f, 10, 20, f, None, f, f, None, f, f, f, f, f, f, f, f,
                                        f, f, f, f, f, f, f, None, f, f, f, f, f, 16, 32, 64, 128, 4,
                                        8, top_k, 5.0, f, f, f, f, d_W1, f, None, None, f, ws_bytes,
                                        None)
    assert "top_k" in _err(mlip, tan(top_k=9), mlip.MLIP_ERR_INVALID)
    assert "null pointer" in _err(mlip, tan(d_W1=None), mlip.MLIP_ERR_INVALID)
    assert "workspace" in _err(mlip, tan(ws_bytes=16), mlip.MLIP_ERR_INVALID)
    t = L.mlip_block_tangent_vjp_workspace_size(4096, 16, 4, 384, 2560, 2560)
    assert t >= 4 * (4096 * 4 * 2560 * 4)          # four token-order [M, H] buffers
    assert L.mlip_block_jvp_workspace_size(4096, 4, 2560, 2560) >= 2 * 4096 * 4 * 2560 * 4
    rc = L.mlip_readout_grad(f, None, None, f, 10, 1, 64, f, f, 16, None)
    assert "workspace" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_readout_vjp(f, None, f, 10, 0, 64, f, None)
    assert "n_structs" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    # layer tangents of the complete block
    rc = L.mlip_moe_jvp(f, f, f, f, f, f, f, f, 10, 4, 8, 9, 64, 128, f, f, None, f, 1 << 30, None)
    assert "top_k" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_moe_tangent_vjp(f, f, f, f, f, f, f, f, f, f, 10, 4, 8, 2, 64, 128, f, f, f, f, None,
                                None, f, f, None, None, f, 16, None)
    assert "workspace" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_attention_jvp(f, f, f, 10, 20, f, None, f, f, f, f, f, f, 16, 64, 32, 4, 5.0, f, f, f, f, None)
    assert "null pointer" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_attention_tangent_vjp(f, f, f, f, 10, 20, f, f, f, f, f, f, f, f, f, f, f, f, f, 16, 64, 100,
                                      5, 5.0, f, f, None, f, f, f, f, 1 << 30, None)
    assert "unsupported attention shape" in _err(mlip, rc, mlip.MLIP_ERR_UNSUPPORTED)
    rc = L.mlip_tri_jvp(f, f, f, 10, 20, f, f, f, f, f, f, 4, 64, 32, 5.0, None, f, f, None)
    assert "h_dot needs s_dot" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
    rc = L.mlip_tri_tangent_vjp(f, f, f, f, 10, 20, f, f, None, f, None, f, f, f, f, f, f, 4, 64, 32, 5.0,
                                f, f, None, f, f, f, f, 16, None)
    assert "workspace" in _err(mlip, rc, mlip.MLIP_ERR_INVALID)
