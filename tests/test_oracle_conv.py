"""Pins for the oracle's edge convolution: closed forms of the radial part, equivariance under
random rotations (Wigner-D), the scalar-only special case against numpy's scatter-add, brute-force
finite-difference gradients, force invariants and the diamond-cell neighbour count.  CPU only."""
import numpy as np
import pytest
import scipy.special as sp

from oracle import conv, so3
from tensor_product_gnn_amd import workloads


def _tiny(L, C=3, H=5, n_nodes=6, n_edges=10, seed=0, r_cut=4.0, n_radial=4):
    rng = np.random.default_rng(seed)
    pos = rng.uniform(0, 3.0, size=(n_nodes, 3))
    src, dst = [], []
    while len(src) < n_edges:
        s, d = rng.integers(0, n_nodes, 2)
        if s != d:
            src.append(s)
            dst.append(d)
    src, dst = np.array(src), np.array(dst)
    vec = pos[src] - pos[dst]
    P = len(so3.paths(L, L, L))
    F = (L + 1) ** 2
    x = rng.standard_normal((n_nodes, F, C))
    W1 = rng.standard_normal((n_radial, H)) / np.sqrt(n_radial)
    W2 = rng.standard_normal((H, P * C)) / np.sqrt(H)
    G = rng.standard_normal((n_nodes, F, C))
    pb = conv.Problem(vec, src, dst, n_nodes, x, W1, W2, L, L, L, r_cut, G=G)
    return pb, pos


def _rotate_features(feat, a, L):
    out = np.empty_like(feat)
    for l in range(L + 1):
        D = so3.wigner_d_real(l, *a)
        out[:, l * l:(l + 1) ** 2, :] = np.einsum("mk,nkc->nmc", D, feat[:, l * l:(l + 1) ** 2, :])
    return out


# ---------------------------------------------------------------- radial part
def test_cutoff_closed_form():
    t = np.array([0.0, 1.0, 1.5])
    assert np.allclose(conv.cutoff(t), [1.0, 0.0, 0.0], atol=1e-15)
    assert np.allclose(conv.cutoff_deriv(np.array([0.0, 1.0])), [0.0, 0.0], atol=1e-15)
    # recover the degree-8 polynomial from samples inside the cutoff: value 1 at 0, and value,
    # slope and curvature all 0 at 1 (the envelope is C^2 at the cutoff)
    ts = np.linspace(0.0, 0.99, 12)
    poly = np.polynomial.Polynomial.fit(ts, conv.cutoff(ts), 8).convert()
    assert abs(poly(0.0) - 1.0) < 1e-10
    for k in range(3):
        assert abs(poly.deriv(k)(1.0)) < 1e-8
    tt = np.linspace(0.05, 0.95, 7)
    fd = (conv.cutoff(tt + 1e-6) - conv.cutoff(tt - 1e-6)) / 2e-6
    assert np.allclose(conv.cutoff_deriv(tt), fd, atol=1e-7)


def test_bessel_basis_is_spherical_j0():
    r_cut, nr = 5.0, 8
    r = np.linspace(0.1, 4.9, 17)
    e, de = conv.radial_basis(r, nr, r_cut)
    n = np.arange(1, nr + 1)
    k = n * np.pi / r_cut
    # B_n(r) = sqrt(2/r_c) sin(k r) / r = sqrt(2/r_c) k j0(k r)
    B = np.sqrt(2 / r_cut) * k[None, :] * sp.spherical_jn(0, k[None, :] * r[:, None])
    assert np.allclose(e, B * conv.cutoff(r / r_cut)[:, None], atol=1e-13)
    fd = (conv.radial_basis(r + 1e-6, nr, r_cut)[0] - conv.radial_basis(r - 1e-6, nr, r_cut)[0]) / 2e-6
    assert np.allclose(de, fd, atol=1e-6)


def test_messages_vanish_beyond_cutoff():
    pb, _ = _tiny(2, r_cut=1.0)
    r = np.linalg.norm(pb.vec, axis=1)
    assert np.any(r >= 1.0)
    st = pb.edge_state(np.arange(len(pb.src)))
    assert np.all(st["w"][r >= 1.0] == 0.0)


# ---------------------------------------------------------------- whole convolution
@pytest.mark.parametrize("L", [1, 2, 3])
def test_equivariance_under_rotation(L):
    pb, _ = _tiny(L, C=4, n_nodes=7, n_edges=16, seed=L)
    out = conv.forward(pb)
    rng = np.random.default_rng(100 + L)
    a = (rng.uniform(0, 2 * np.pi), rng.uniform(0, np.pi), rng.uniform(0, 2 * np.pi))
    R = so3.rotation_zyz(*a)
    pb_r = conv.Problem(pb.vec @ R.T, pb.src, pb.dst, pb.n_nodes, _rotate_features(pb.x, a, L),
                        pb.W1, pb.W2, L, L, L, pb.r_cut)
    out_r = conv.forward(pb_r)
    assert np.allclose(out_r, _rotate_features(out, a, L), atol=1e-10 * np.abs(out).max())
    # scalar outputs are invariant
    assert np.allclose(out_r[:, 0, :], out[:, 0, :], atol=1e-10 * np.abs(out).max())


def test_linear_in_x_and_edge_order():
    pb, _ = _tiny(2, C=3, n_edges=14, seed=3)
    out = conv.forward(pb)
    pb2 = conv.Problem(pb.vec, pb.src, pb.dst, pb.n_nodes, 2.5 * pb.x, pb.W1, pb.W2, 2, 2, 2, pb.r_cut)
    assert np.allclose(conv.forward(pb2), 2.5 * out, atol=1e-12)
    perm = np.random.default_rng(0).permutation(len(pb.src))
    pb3 = conv.Problem(pb.vec[perm], pb.src[perm], pb.dst[perm], pb.n_nodes, pb.x, pb.W1, pb.W2,
                       2, 2, 2, pb.r_cut)
    assert np.allclose(conv.forward(pb3), out, atol=1e-12)


def test_scalar_only_reduces_to_gather_scale_scatter():
    wl = workloads.generate("l0")
    pb = conv.Problem.from_workload(wl)
    out = conv.forward(pb)
    # library-routine reference: w from the MLP, then numpy's unbuffered scatter-add
    r = np.linalg.norm(pb.vec, axis=1)
    n = np.arange(1, pb.W1.shape[0] + 1)[None, :]
    e = np.sqrt(2 / pb.r_cut) * np.sin(n * np.pi * r[:, None] / pb.r_cut) / r[:, None] \
        * conv.cutoff(r / pb.r_cut)[:, None]
    z = e @ pb.W1
    w = (z * sp.expit(z)) @ pb.W2
    ref = np.zeros((pb.n_nodes, pb.C))
    np.add.at(ref, pb.dst, w * pb.x[pb.src, 0, :])
    assert np.allclose(out[:, 0, :], ref, atol=1e-13)


# ---------------------------------------------------------------- gradients by brute force
def _loss(pb):
    return float(np.sum(pb.G * conv.forward(pb)))


@pytest.mark.parametrize("L", [1, 2, 3])
def test_backward_matches_central_differences(L):
    pb, _ = _tiny(L, C=3, H=5, n_nodes=5, n_edges=9, seed=10 + L)
    g = conv.backward(pb)
    h = 1e-6

    def fd(arr, idx):
        old = arr[idx]
        arr[idx] = old + h
        lp = _loss(pb)
        arr[idx] = old - h
        lm = _loss(pb)
        arr[idx] = old
        return (lp - lm) / (2 * h)

    rng = np.random.default_rng(0)
    for name, arr, grad in (("vec", pb.vec, g["dvec"]), ("x", pb.x, g["dx"]),
                            ("W1", pb.W1, g["dW1"]), ("W2", pb.W2, g["dW2"])):
        scale = np.abs(grad).max()
        for _ in range(12):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            assert abs(fd(arr, idx) - grad[idx]) <= 1e-7 * max(scale, 1.0), name


def test_backward_on_c0_matches_central_differences():
    wl = workloads.generate("c0")
    pb = conv.Problem.from_workload(wl)
    g = conv.backward(pb)
    h = 1e-6
    rng = np.random.default_rng(1)
    for arr, grad in ((pb.vec, g["dvec"]), (pb.W2, g["dW2"]), (pb.W1, g["dW1"]), (pb.x, g["dx"])):
        scale = np.abs(grad).max()
        for _ in range(4):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(pb)
            arr[idx] = old - h
            lm = _loss(pb)
            arr[idx] = old
            assert abs((lp - lm) / (2 * h) - grad[idx]) <= 1e-7 * scale


def test_backward_of_block_with_linear():
    pb, _ = _tiny(2, C=4, n_edges=12, seed=4)
    rng = np.random.default_rng(2)
    W_lin = [rng.standard_normal((4, 4)) / 2 for _ in range(3)]
    dy = rng.standard_normal((pb.n_nodes, 9, 4))

    def loss():
        return float(np.sum(dy * conv.linear(conv.forward(pb), W_lin, 2)))
    g = conv.backward(pb, G=conv.linear_backward_data(dy, W_lin, 2))
    h = 1e-6
    for _ in range(6):
        idx = tuple(rng.integers(0, s) for s in pb.vec.shape)
        old = pb.vec[idx]
        pb.vec[idx] = old + h
        lp = loss()
        pb.vec[idx] = old - h
        lm = loss()
        pb.vec[idx] = old
        assert abs((lp - lm) / (2 * h) - g["dvec"][idx]) <= 1e-7 * np.abs(g["dvec"]).max()
    dW = conv.linear_backward_weight(conv.forward(pb), dy, 2)
    for l in range(3):
        i, j = rng.integers(0, 4, 2)
        old = W_lin[l][i, j]
        W_lin[l][i, j] = old + h
        lp = loss()
        W_lin[l][i, j] = old - h
        lm = loss()
        W_lin[l][i, j] = old
        assert abs((lp - lm) / (2 * h) - dW[l][i, j]) <= 1e-7 * np.abs(dW[l]).max()


# ---------------------------------------------------------------- forces
def test_force_invariants_on_c0():
    wl = workloads.generate("c0")
    pb = conv.Problem.from_workload(wl)
    a = np.asarray(wl.readout, dtype=np.float64)
    G = np.zeros_like(pb.x)
    G[:, 0, :] = a[None, :]                 # E = sum_n a . out[n, 0e, :]
    g = conv.backward(pb, G=G, want_dx=False)
    F = conv.forces(g["dvec"], pb.src, pb.dst, pb.n_nodes)
    pos = wl.pos
    scale = np.abs(F).max()
    assert np.allclose(F.sum(0), 0.0, atol=1e-12 * scale * len(F))
    # zero torque needs an energy invariant in positions alone: keep only scalar input features
    xs = pb.x.copy()
    xs[:, 1:, :] = 0.0
    pb_s = conv.Problem(pb.vec, pb.src, pb.dst, pb.n_nodes, xs, pb.W1, pb.W2, 1, 1, 1, pb.r_cut)
    F_s = conv.forces(conv.backward(pb_s, G=G, want_dx=False)["dvec"], pb.src, pb.dst, pb.n_nodes)
    assert np.abs(F_s).max() > 1e-3
    # sum_i pos_i x F_i = -sum_e vec_e x dE/dvec_e; checked on the edge vectors actually used
    # (the float32 inputs), since positions only fix them up to float32 rounding
    dv = conv.backward(pb_s, G=G, want_dx=False)["dvec"]
    assert np.allclose(np.cross(pb.vec, dv).sum(0), 0.0, atol=1e-12 * np.abs(dv).max() * len(dv))
    assert np.allclose(np.cross(pos, F_s).sum(0), 0.0, atol=1e-6 * np.abs(F_s).max() * len(F))
    # covariance: F(R pos) = R F(pos)
    rng = np.random.default_rng(3)
    ang = (rng.uniform(0, 2 * np.pi), rng.uniform(0, np.pi), rng.uniform(0, 2 * np.pi))
    R = so3.rotation_zyz(*ang)
    pb_r = conv.Problem(pb.vec @ R.T, pb.src, pb.dst, pb.n_nodes, _rotate_features(pb.x, ang, 1),
                        pb.W1, pb.W2, 1, 1, 1, pb.r_cut)
    F_r = conv.forces(conv.backward(pb_r, G=G, want_dx=False)["dvec"], pb.src, pb.dst, pb.n_nodes)
    assert np.allclose(F_r, F @ R.T, atol=1e-10 * scale)


def test_diamond_neighbour_count_without_noise():
    spec = dict(workloads.SPECS["c3"])
    spec["sigma"] = 0.0
    wl = workloads.generate("c3", spec=spec)
    deg = np.diff(wl.row_ptr)
    assert wl.n_edges == 86000 and deg.min() == 86 and deg.max() == 86
    # shells 4, 12, 12, 6, 12, 24, 16 inside 5 A; the next (12 at 5.044 A) lies outside
    r = np.sort(np.linalg.norm(wl.vec[wl.dst == 0].astype(np.float64), axis=1))
    shells = np.split(r, np.where(np.diff(r) > 1e-3)[0] + 1)
    assert [len(s) for s in shells] == [4, 12, 12, 6, 12, 24, 16]


# ---------------------------------------------------------------- the pins have teeth
def test_planted_mistakes_are_caught(monkeypatch):
    """Plant plausible mistakes in the oracle and check that a pin above fails for each."""
    pb, _ = _tiny(2, C=3, n_nodes=6, n_edges=12, seed=5)
    rng = np.random.default_rng(9)
    a = (rng.uniform(0, 2 * np.pi), rng.uniform(0, np.pi), rng.uniform(0, 2 * np.pi))
    R = so3.rotation_zyz(*a)

    def equivariance_error(p):
        out = conv.forward(p)
        p_r = conv.Problem(p.vec @ R.T, p.src, p.dst, p.n_nodes, _rotate_features(p.x, a, 2),
                           p.W1, p.W2, 2, 2, 2, p.r_cut)
        return np.abs(conv.forward(p_r) - _rotate_features(out, a, 2)).max() / np.abs(out).max()

    assert equivariance_error(pb) < 1e-12
    # (1) a transposed CG operand (m1 <-> m3) on a path with l1 == l3
    bad = conv.Problem(pb.vec, pb.src, pb.dst, pb.n_nodes, pb.x, pb.W1, pb.W2, 2, 2, 2, pb.r_cut)
    k = bad.paths.index((2, 2, 2))
    bad.cg[k] = bad.cg[k].transpose(2, 1, 0).copy()
    bad.cg[k][0, 0, 1] += 0.3
    assert equivariance_error(bad) > 1e-3
    # (2) a sign flip inside one CG block
    bad = conv.Problem(pb.vec, pb.src, pb.dst, pb.n_nodes, pb.x, pb.W1, pb.W2, 2, 2, 2, pb.r_cut)
    k = bad.paths.index((1, 1, 2))
    bad.cg[k] = bad.cg[k].copy()
    bad.cg[k][:, :, 0] *= -1
    assert equivariance_error(bad) > 1e-3
    # (3) a dropped cutoff-derivative term is caught by the finite-difference check
    g_good = conv.backward(pb)["dvec"]
    monkeypatch.setattr(conv, "cutoff_deriv", lambda t: np.zeros_like(t))
    g_bad = conv.backward(pb)["dvec"]
    assert np.abs(g_bad - g_good).max() > 1e-6 * np.abs(g_good).max()


# ---------------------------------------------------------------- bf16 operands of the MLP

def test_round_bf16_ties_to_even_and_matches_torch():
    import torch
    e = 2.0 ** -8  # half an ulp of bf16 at 1
    got = conv.round_bf16([1 + e, 1 + 3 * e, 1 + e + 2 ** -20, -(1 + 3 * e), 3.0, 0.0])
    assert list(got) == [1.0, 1 + 4 * e, 1 + 2 * e, -(1 + 4 * e), 3.0, 0.0]
    rng = np.random.default_rng(0)
    x = rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))
    lib = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(conv.round_bf16(x), lib)


def test_bf16_operands_stay_within_the_rounding_bound():
    """Each bf16 operand is within 2^-8 (relative) of its fp32 value, so a product of two is within
    2^-7 + 2^-16, and a sum of products within that times the sum of absolute products."""
    pb, _ = _tiny(2, C=3, n_nodes=6, n_edges=12, seed=3)
    pbb = conv.Problem(pb.vec, pb.src, pb.dst, pb.n_nodes, pb.x, pb.W1, pb.W2, 2, 2, 2, pb.r_cut,
                       G=pb.G, mlp_bf16=True)
    edges = np.arange(len(pb.src))
    st, stb = pb.edge_state(edges), pbb.edge_state(edges)
    rel = 2.0 ** -7 + 2.0 ** -15
    bound = (np.abs(st["h"]) @ np.abs(pb.W2)).reshape(st["w"].shape) * rel
    assert np.all(np.abs(stb["w"] - st["w"]) <= bound)
    assert np.abs(stb["w"] - st["w"]).max() > 0  # the rounding is active
    g, gb = conv.backward(pb), conv.backward(pbb)
    # dL/dw does not involve w, so dL/dW2 differs only through the rounding of h and dL/dw
    assert np.abs(gb["dW2"] - g["dW2"]).max() <= rel * (np.abs(st["h"]).T @ np.abs(
        _dw_rows(pb, st))).max() + 1e-15
    for k in ("dvec", "dx", "dW1", "dW2"):
        assert np.all(np.isfinite(gb[k]))
        assert np.abs(gb[k] - g[k]).max() <= 0.05 * np.abs(g[k]).max(), k


def _dw_rows(pb, st):
    """dL/dw per edge [E, P*C] (independent of w), for the bound above."""
    xs, Gd = pb.x[pb.src], pb.G[pb.dst]
    cols = []
    for p, (l1, l2, l3) in enumerate(pb.paths):
        t = np.einsum("ijk,eic,ej->ekc", pb.cg[p], xs[:, l1 * l1:(l1 + 1) ** 2, :], st["Y"][l2])
        cols.append(np.einsum("ekc,ekc->ec", Gd[:, l3 * l3:(l3 + 1) ** 2, :], t))
    return np.concatenate(cols, axis=1)


# ---------------------------------------------------------------- per-edge path subsets
def _masked(pb, mask):
    return conv.Problem(pb.vec, pb.src, pb.dst, pb.n_nodes, pb.x, pb.W1, pb.W2, pb.L_in, pb.L_sh,
                        pb.L_out, pb.r_cut, G=pb.G, path_mask=mask)


@pytest.mark.parametrize("d", [0, 1, 2])
def test_degree_mask_equals_lower_sh_degree_convolution(d):
    """Masking every edge to the paths with l2 <= d is the convolution with spherical harmonics
    up to degree d (an independent path table, W2 restricted to those paths' columns)."""
    pb, _ = _tiny(3, C=2, n_nodes=6, n_edges=14, seed=30 + d)
    mask = np.full(len(pb.src), workloads.degree_masks(3)[d], dtype=np.uint32)
    got = conv.forward(_masked(pb, mask))
    sub = [i for i, p in enumerate(pb.paths) if p[1] <= d]
    assert [pb.paths[i] for i in sub] == so3.paths(3, d, 3)
    cols = np.concatenate([np.arange(i * pb.C, (i + 1) * pb.C) for i in sub])
    low = conv.Problem(pb.vec, pb.src, pb.dst, pb.n_nodes, pb.x, pb.W1, pb.W2[:, cols], 3, d, 3,
                       pb.r_cut, G=pb.G)
    ref = conv.forward(low)
    assert np.abs(got - ref).max() < 1e-12 * max(1.0, np.abs(ref).max())
    g_got, g_ref = conv.backward(_masked(pb, mask)), conv.backward(low)
    assert np.abs(g_got["dvec"] - g_ref["dvec"]).max() < 1e-12 * np.abs(g_ref["dvec"]).max()
    assert np.abs(g_got["dx"] - g_ref["dx"]).max() < 1e-12 * np.abs(g_ref["dx"]).max()
    assert np.abs(g_got["dW1"] - g_ref["dW1"]).max() < 1e-12 * np.abs(g_ref["dW1"]).max()
    # dL/dW2 of the masked convolution is zero in the columns of the paths that are off
    off_cols = np.setdiff1d(np.arange(pb.W2.shape[1]), cols)
    assert np.abs(g_got["dW2"][:, off_cols]).max() == 0.0
    assert np.abs(g_got["dW2"][:, cols] - g_ref["dW2"]).max() < 1e-12 * np.abs(g_ref["dW2"]).max()


def test_empty_mask_removes_the_edge():
    pb, _ = _tiny(2, C=3, n_nodes=6, n_edges=12, seed=41)
    mask = np.full(len(pb.src), 0xFFFFFFFF, dtype=np.uint32)
    k = 5
    mask[k] = 0
    keep = np.setdiff1d(np.arange(len(pb.src)), [k])
    red = conv.Problem(pb.vec[keep], pb.src[keep], pb.dst[keep], pb.n_nodes, pb.x, pb.W1, pb.W2,
                       2, 2, 2, pb.r_cut, G=pb.G)
    assert np.abs(conv.forward(_masked(pb, mask)) - conv.forward(red)).max() < 1e-13
    g, gr = conv.backward(_masked(pb, mask)), conv.backward(red)
    assert np.abs(g["dvec"][k]).max() == 0.0
    assert np.abs(g["dvec"][keep] - gr["dvec"]).max() < 1e-13
    for key in ("dx", "dW1", "dW2"):
        assert np.abs(g[key] - gr[key]).max() < 1e-12, key


def test_masked_backward_matches_central_differences():
    pb, _ = _tiny(2, C=2, n_nodes=5, n_edges=9, seed=43)
    rng = np.random.default_rng(3)
    mask = rng.integers(0, 1 << 11, size=len(pb.src)).astype(np.uint32)
    mp = _masked(pb, mask)
    g = conv.backward(mp)

    def loss(**kw):
        args = dict(vec=pb.vec, x=pb.x, W1=pb.W1, W2=pb.W2)
        args.update(kw)
        q = conv.Problem(args["vec"], pb.src, pb.dst, pb.n_nodes, args["x"], args["W1"],
                         args["W2"], 2, 2, 2, pb.r_cut, G=pb.G, path_mask=mask)
        return float(np.sum(pb.G * conv.forward(q)))
    h = 1e-6
    for name, arr, key in (("vec", pb.vec, "dvec"), ("x", pb.x, "dx"), ("W2", pb.W2, "dW2"),
                           ("W1", pb.W1, "dW1")):
        for _ in range(6):
            i = tuple(rng.integers(0, s) for s in arr.shape)
            a, b = arr.copy(), arr.copy()
            a[i] += h
            b[i] -= h
            fd = (loss(**{name: a}) - loss(**{name: b})) / (2 * h)
            assert abs(fd - g[key][i]) < 1e-6 * max(1.0, abs(fd)), (name, i)


def test_adaptive_workload_masks_follow_distance():
    wl = workloads.generate("c2as")
    dm = workloads.degree_masks(3)
    r = np.linalg.norm(wl.vec.astype(np.float64), axis=1)
    deg = np.array([dm.index(int(m)) for m in wl.path_mask])
    assert np.bincount(deg).tolist() == [len(r) // 4] * 4
    assert r[deg == 3].max() <= r[deg == 0].min()          # shorter edges, higher degree
    for d in range(wl.n_nodes):                              # descending degree within a receiver
        seg = deg[wl.row_ptr[d]:wl.row_ptr[d + 1]]
        assert np.all(np.diff(seg) <= 0)
    assert [p for p in workloads.path_list(3)] == so3.paths(3, 3, 3)


def test_planted_mask_mistakes_are_caught():
    """A mask applied to the forward's w but not to dL/dw, or path bits read in reverse order,
    fail the pins above."""
    pb, _ = _tiny(3, C=2, n_nodes=6, n_edges=14, seed=31)
    mask = np.full(len(pb.src), workloads.degree_masks(3)[1], dtype=np.uint32)
    # bits in reverse path order: no longer the l2 <= 1 convolution
    P = len(pb.paths)
    rev = np.array([int(f"{int(m):0{P}b}"[::-1], 2) for m in mask], dtype=np.uint32)
    sub = [i for i, p in enumerate(pb.paths) if p[1] <= 1]
    cols = np.concatenate([np.arange(i * pb.C, (i + 1) * pb.C) for i in sub])
    low = conv.Problem(pb.vec, pb.src, pb.dst, pb.n_nodes, pb.x, pb.W1, pb.W2[:, cols], 3, 1, 3,
                       pb.r_cut, G=pb.G)
    assert np.abs(conv.forward(_masked(pb, rev)) - conv.forward(low)).max() > 1e-3
    # dL/dW2 without the mask on dL/dw: nonzero columns for paths that are off
    g = conv.backward(_masked(pb, mask))
    full = conv.backward(pb)
    off_cols = np.setdiff1d(np.arange(pb.W2.shape[1]), cols)
    assert np.abs(full["dW2"][:, off_cols]).max() > 1e-3 and np.abs(g["dW2"][:, off_cols]).max() == 0
