"""Host-only checks of the C ABI: the library loads and exports every function include/equitp.h
declares; handles, irreps parsing and argument validation behave as documented; the GPU-side
CG table (built by sphere quadrature) matches the oracle's Racah-formula CG.  No compute calls."""
import ctypes
import subprocess

import numpy as np
import pytest

import tensor_product_gnn_amd as tp
from oracle import so3
from tensor_product_gnn_amd import workloads


def test_library_exports_every_declared_function():
    names = tp.header_functions()
    assert len(names) >= 12
    L = tp.lib()
    for n in names:
        assert hasattr(L, n), n
    syms = subprocess.run(["nm", "-D", "--defined-only", tp.LIB_PATH], capture_output=True,
                          text=True).stdout
    for n in names:
        assert f" T {n}\n" in syms, n


@pytest.mark.parametrize("L,n_paths", [(0, 1), (1, 4), (2, 11), (3, 23)])
def test_create_query_and_path_order(L, n_paths):
    ir = "+".join(f"32x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(L + 1))
    sh = "+".join(f"1x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(L + 1))
    c = tp.Conv(ir, sh, ir, n_radial=8, hidden=64, r_cut=5.0)
    assert c.n_paths == n_paths == workloads.N_PATHS_FOR_L[L]
    assert c.channels == 32 and c.f_in == c.f_out == c.f_sh == (L + 1) ** 2
    assert c.w1_numel == 8 * 64 and c.w2_numel == 64 * n_paths * 32
    assert c.paths() == so3.paths(L, L, L)


@pytest.mark.parametrize("bad,status", [
    ("16x0e+16x1e", -3),          # wrong parity for l = 1
    ("16x0e+32x1o", -3),          # mixed multiplicities
    ("16x0e+16x2e", -3),          # missing l = 1
    ("16x0e+16x1o+16x2e+16x3o+16x4e", -3),  # l > 3
    ("12x0e+12x1o", -3),          # C not a multiple of 16
    ("16x0q", -2),                # parse error
    ("", -2),
    ("16x0e++16x1o", -2),
])
def test_create_rejects(bad, status):
    h = ctypes.c_void_p()
    st = tp.lib().equitp_create(bad.encode(), b"1x0e+1x1o", bad.encode(), 8, ctypes.byref(h))
    assert st == status
    assert not h.value


def test_create_accepts_implicit_sh_multiplicity_and_rejects_bad_radial():
    h = ctypes.c_void_p()
    assert tp.lib().equitp_create(b"16x0e + 16x1o", b"0e+1o", b"16x0e+16x1o", 8, ctypes.byref(h)) == 0
    assert tp.lib().equitp_set_radial(h, 32, 5.0) == -3
    assert tp.lib().equitp_set_radial(h, 64, -1.0) == -1
    assert tp.lib().equitp_set_radial(h, 16, 4.0) == 0
    tp.lib().equitp_destroy(h)
    h2 = ctypes.c_void_p()
    assert tp.lib().equitp_create(b"16x0e", b"0e", b"16x0e", 6, ctypes.byref(h2)) == -3
    assert tp.lib().equitp_create(b"16x0e", b"0e", b"16x0e", 0, ctypes.byref(h2)) == -1


def test_status_strings_and_null_handles():
    L = tp.lib()
    for s in (0, -1, -2, -3, -4, -5):
        assert L.equitp_status_string(s)
    assert L.equitp_forward(None, None, None, None, None, None, None, None) == -1
    assert L.equitp_query(None, None, None, None, None, None, None, None) == -1
    assert L.equitp_linear(-1, 2, 128, None, None, 0, None, None) == -1
    L.equitp_destroy(None)


def test_forward_validates_arguments_without_touching_the_gpu():
    c = tp.Conv("16x0e+16x1o", "1x0e+1x1o", "16x0e+16x1o", hidden=16)
    g = tp.GraphStruct(4, 3, 256, 512, 768, 0, 0)
    L = tp.lib()
    # null x / out
    assert L.equitp_forward(c._h, ctypes.byref(g), 1024, None, 2048, 4096, 8192, None) == -1
    # misaligned feature pointers
    assert L.equitp_forward(c._h, ctypes.byref(g), 1024, 1028, 2048, 4096, 8192, None) == -1
    # negative sizes
    bad = tp.GraphStruct(4, -1, 256, 512, 768, 0, 0)
    assert L.equitp_forward(c._h, ctypes.byref(bad), 1024, 2048, 2048, 4096, 8192, None) == -1
    # no nodes: nothing to do
    empty = tp.GraphStruct(0, 0, 0, 0, 0, 0, 0)
    assert L.equitp_forward(c._h, ctypes.byref(empty), 0, 0, 0, 0, 0, None) == 0
    # grad_x requested without the sender CSR
    assert L.equitp_backward(c._h, ctypes.byref(g), 1024, 2048, 4096, 4096, 8192, 0, 16384, 0, 0,
                             0, 0, None) == -1


def test_backward_workspace_grows_with_edges():
    c = tp.Conv("128x0e+128x1o+128x2e+128x3o", "1x0e+1x1o+1x2e+1x3o", "128x0e+128x1o+128x2e+128x3o")
    a, b = c.workspace_bytes(1024, 1000), c.workspace_bytes(1024, 131072)
    assert b > a > 0
    assert b >= 8 * 131072 * 3 * 4   # one dL/dvec partial per channel slice and edge


@pytest.mark.parametrize("path", so3.paths(3, 3, 3))
def test_gpu_side_cg_table_matches_oracle(path):
    got = tp.cg_block(*path)
    ref = so3.real_cg(*path)
    assert np.abs(got - ref).max() < 1e-7
    assert (np.abs(got) > 0).sum() == (np.abs(ref) > 1e-12).sum()


def test_cg_block_rejects_odd_paths():
    d = np.zeros(27, dtype=np.float32)
    assert tp.lib().equitp_cg_block(1, 1, 1, d.ctypes.data_as(ctypes.POINTER(ctypes.c_float))) == -3


@pytest.mark.parametrize("L", [0, 1, 2, 3])
def test_ladder_path_count_matches_oracle(L):
    from oracle import ladder
    assert tp.ladder_num_paths(L) == len(ladder.paths(L)) == workloads.N_PATHS_FOR_L[L]


def test_ladder_validates_arguments_without_touching_the_gpu():
    L = tp.lib()
    # unsupported order, rank or channel count
    assert L.equitp_ladder_forward(3, 6, 4, 64, 256, 512, 1024, None, None) == -3
    assert L.equitp_ladder_forward(4, 3, 4, 64, 256, 512, 1024, None, None) == -3
    assert L.equitp_ladder_forward(3, 3, 4, 40, 256, 512, 1024, None, None) == -3
    assert L.equitp_ladder_forward(3, 1, 4, 64, 256, 512, 1024, None, None) == -3
    # negative sizes, null or aliased pointers
    assert L.equitp_ladder_forward(3, 3, -1, 64, 256, 512, 1024, None, None) == -1
    assert L.equitp_ladder_forward(3, 3, 4, 64, None, 512, 1024, None, None) == -1
    assert L.equitp_ladder_forward(3, 3, 4, 64, 256, 512, 256, None, None) == -1
    assert L.equitp_ladder_forward(3, 3, 4, 64, 256, 512, 1024, 1024, None) == -1
    # no nodes: nothing to do
    assert L.equitp_ladder_forward(3, 3, 0, 64, None, None, None, None, None) == 0
    assert L.equitp_ladder_backward(3, 3, 0, 64, None, None, None, None, None, None, None, 0,
                                    None) == 0
    # grad_w without a large enough workspace
    ws = ctypes.c_size_t(0)
    assert L.equitp_ladder_backward_workspace(3, 5, 4096, 128, ctypes.byref(ws)) == 0
    assert ws.value >= 4 * 23 * 128 * 4
    assert L.equitp_ladder_backward(3, 5, 4096, 128, 256, 512, None, 1024, 2048, 4096, 8192,
                                    ws.value - 4, None) == -5
    # outputs aliasing inputs
    assert L.equitp_ladder_backward(3, 5, 4096, 128, 256, 512, None, 1024, 256, None, None, 0,
                                    None) == -1
    assert L.equitp_ladder_backward(3, 5, 4096, 128, 256, 512, 3072, 1024, 3072, None, None, 0,
                                    None) == -1


def test_full_ladder_validates_arguments_without_touching_the_gpu():
    L = tp.lib()
    ws = ctypes.c_size_t(0)
    # unsupported order, rank or channel count (the kernels take 32, 64 or 128 channels)
    for lmax, nu, C in [(3, 6, 64), (4, 3, 64), (3, 3, 48), (3, 3, 16), (3, 1, 64), (3, 3, 256)]:
        assert L.equitp_full_ladder_workspace(lmax, nu, 4, C, 0, ctypes.byref(ws)) == -3
        assert L.equitp_full_ladder_forward(lmax, nu, 4, C, 256, 512, 1024, None, None, 4096,
                                            1 << 30, None) == -3
    assert L.equitp_full_ladder_workspace(3, 3, -1, 64, 0, ctypes.byref(ws)) == -1
    # workspace: one step's path outputs (+ two rungs when none are kept) in the forward; the
    # rungs, the next step's output gradient and one partial map per dL/dW work-group backward
    N, C, D, F = 4096, 128, 99, 16
    assert L.equitp_full_ladder_workspace(3, 5, N, C, 0, ctypes.byref(ws)) == 0
    assert ws.value == 4 * (N * D * C + 2 * N * F * C)
    fwd = ws.value
    assert L.equitp_full_ladder_workspace(3, 5, N, C, 1, ctypes.byref(ws)) == 0
    # dL/dW row ranges: about 1024 work-groups in all, multiples of 32 rows, 256..4096 rows
    rows = min(4096, max(256, -(-(-(-N * D // 1024)) // 32) * 32))
    assert rows == 416
    blocks = sum(-(-N * (2 * l3 + 1) // rows) for (_, _, l3) in so3.paths(3, 3, 3))
    assert ws.value == 4 * (N * D * C + 3 * N * F * C + N * F * C + blocks * C * C)
    bwd = ws.value
    # kept path outputs: every step's, [nu-1][N * D][C]
    n = ctypes.c_size_t(0)
    assert L.equitp_full_ladder_saved_floats(3, 5, N, C, ctypes.byref(n)) == 0
    assert n.value == 4 * N * D * C
    # null, aliased or misaligned pointers, workspace too small
    fl, bl = L.equitp_full_ladder_forward, L.equitp_full_ladder_backward
    assert fl(3, 5, N, C, None, 512, 1024, None, None, 4096, fwd, None) == -1
    assert fl(3, 5, N, C, 256, 512, 256, None, None, 4096, fwd, None) == -1
    assert fl(3, 5, N, C, 256, 512, 1024, 1024, None, 4096, fwd, None) == -1
    assert fl(3, 5, N, C, 256, 512, 1024, None, 1024, 4096, fwd, None) == -1
    assert fl(3, 5, N, C, 256, 512, 1024, None, 2052, 4096, fwd, None) == -1
    assert fl(3, 5, N, C, 260, 512, 1024, None, None, 4096, fwd, None) == -1
    assert fl(3, 5, N, C, 256, 512, 1024, None, None, 4096, fwd - 4, None) == -5
    assert bl(3, 5, N, C, 256, 512, None, None, 1024, 256, None, 4096, bwd, None) == -1
    assert bl(3, 5, N, C, 256, 512, 3072, None, 1024, 3072, None, 4096, bwd, None) == -1
    assert bl(3, 5, N, C, 256, 512, None, 2052, 1024, 2048, 8192, 4096, bwd, None) == -1
    assert bl(3, 5, N, C, 256, 512, None, None, 1024, 2048, 8192, 4096, bwd - 4, None) == -5
    # nothing requested, or no nodes: nothing to do
    assert bl(3, 5, N, C, 256, 512, None, None, 1024, None, None, None, 0, None) == 0
    assert fl(3, 3, 0, 64, None, None, None, None, None, None, 0, None) == 0


def test_mixed_multiplicities_create_query_and_validation():
    L = tp.lib()
    h = ctypes.c_void_p()
    big = b"128x0e+64x1o+32x2e+32x3o"
    # multiplicities must be multiples of 32 up to 128, parity (-1)^l, the same ranks in and out,
    # l >= 1, 8 Bessel functions, MLP width 64
    for a, b, nr, hid, st in [(b"48x0e+32x1o", b"48x0e+32x1o", 8, 64, -3),
                              (b"256x0e+32x1o", b"256x0e+32x1o", 8, 64, -3),
                              (b"128x0e+64x1e", b"128x0e+64x1e", 8, 64, -3),
                              (big, b"128x0e+64x1o+32x2e", 8, 64, -3),
                              (b"128x0e", b"128x0e", 8, 64, -3),
                              (big, big, 8, 16, -3), (big, big, 4, 64, -3),
                              (b"128x0e+", big, 8, 64, -2)]:
        assert L.equitp_mixed_create(a, b, nr, hid, 5.0, ctypes.byref(h)) == st, (a, b, nr, hid)
    assert L.equitp_mixed_create(big, big, 8, 64, 0.0, ctypes.byref(h)) == -1
    m = tp.MixedConv(big.decode(), big.decode(), r_cut=35.0)
    # 23 paths; 3 channel slices (32 channels of l <= 3, 32 of l <= 1, 64 of l = 0) with 7, 3 and 1
    # launches (the most paths into one output rank among the paths each slice carries)
    assert (m.n_paths, m.f_in, m.f_out, m.n_slices, m.n_launches) == (23, 704, 704, 3, 11)
    widths = [128, 64, 32, 32]
    assert m.w2_numel == 64 * sum(widths[l1] for (l1, _, _) in so3.paths(3, 3, 3))
    assert m.wlin_numel == sum(widths[l1] * widths[l3] for (l1, _, l3) in so3.paths(3, 3, 3))
    # graphs that carry path masks are refused (the call sets its own)
    g = tp.GraphStruct(4, 3, 256, 512, 768, 0, 0, 1024)
    assert L.equitp_mixed_forward(m._h, ctypes.byref(g), 2048, 4096, 8192, 8192, 8192, 16384, None,
                                  4096, 1 << 30, None) == -1
    # kept path outputs: one row of 128 (padded) channels per path-output component and node
    n = ctypes.c_size_t(0)
    assert L.equitp_mixed_saved_floats(m._h, 1000, ctypes.byref(n)) == 0
    assert n.value == 1000 * sum(2 * l3 + 1 for (_, _, l3) in so3.paths(3, 3, 3)) * 128


@pytest.mark.parametrize("L", [1, 2, 3])
def test_bench_ladder_flop_count_matches_oracle(L):
    import bench
    from oracle import ladder
    assert bench.ladder_flops(tp, L) == ladder.flops_per_node_channel_step(L)


@pytest.mark.parametrize("L", [1, 2, 3])
def test_bench_full_ladder_flop_count_matches_oracle(L):
    """GEMM: 2 C^2 per row of path outputs; products: the path-reduced count less its weight FMA."""
    import bench
    from oracle import ladder
    C = 64
    rows = sum(2 * l3 + 1 for (_, _, l3) in ladder.paths(L))
    f = bench.full_ladder_flops(tp, L, C)
    assert f["mix_fwd"] == f["mix_dt"] == f["mix_dw"] == 2 * rows * C * C
    assert f["full_tp"] == (ladder.flops_per_node_channel_step(L) - 2 * rows) * C


def test_path_masks_rejected_where_unsupported():
    L = tp.lib()
    g = tp.GraphStruct(4, 3, 256, 512, 768, 0, 0, 1024)
    # l = 0: no masked kernels
    c0 = tp.Conv("16x0e", "1x0e", "16x0e")
    assert L.equitp_forward(c0._h, ctypes.byref(g), 2048, 4096, 8192, 8192, 16384, None) == -3
    # bf16 MLP operands with masks
    c = tp.Conv("16x0e+16x1o", "1x0e+1x1o", "16x0e+16x1o", mlp_bf16=True)
    assert L.equitp_forward(c._h, ctypes.byref(g), 2048, 4096, 8192, 8192, 16384, None) == -3
    # hidden 16 with masks
    c16 = tp.Conv("16x0e+16x1o", "1x0e+1x1o", "16x0e+16x1o", hidden=16)
    assert L.equitp_backward(c16._h, ctypes.byref(g), 2048, 4096, 8192, 8192, 16384, 0, 0, 0, 0,
                             0, 0, None) == -3


def test_profile_filter_is_host_only_and_resets():
    # the timing filter takes names, an empty string or NULL, and records nothing by itself
    tp.profile_reset()
    tp.profile_only(["bwd", "seg_fwd"])
    tp.profile_only(None)
    assert tp.lib().equitp_profile_only(b"") == 0
    assert tp.profile_read() == {}


def test_traffic_record_hash_ignores_comments_only():
    import bench
    code = "int f(int a) {\n  // sum\n  return a + 1; /* one */\n}\n"
    assert bench.code_tokens(code) == bench.code_tokens("int f(int a) {\n  return a + 1;\n}")
    assert bench.code_tokens(code) != bench.code_tokens(code.replace("a + 1", "a + 2"))
    # every recorded traffic figure is keyed on a hash this function can reproduce
    for unit in bench.KERNEL_SOURCES:
        assert len(bench.kernel_source_hash(unit)) == 16
