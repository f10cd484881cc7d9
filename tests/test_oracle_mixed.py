"""Pins of the mixed-multiplicity convolution oracle (oracle/mixed.py) to things other than itself:
  * uniform multiplicities with identity maps = the path-reduced convolution oracle (forward and
    every gradient), itself pinned in test_oracle_conv.py;
  * any multiplicities = a composition through the masked convolution oracle: one path at a time
    (a path mask with that path alone), inputs zero-padded to the largest multiplicity, the
    path's block cut to its own channels and mapped by its linear;
  * rotation equivariance of the output;
  * gradients against central differences;
  * a planted mistake (the outputs of two paths into one rank swapped) is caught."""
import numpy as np
import pytest

from oracle import conv, mixed, so3


def _graph(n_nodes, n_edges, rng):
    pos = rng.uniform(0, 3.0, size=(n_nodes, 3))
    src, dst = [], []
    while len(src) < n_edges:
        s, d = rng.integers(0, n_nodes, 2)
        if s != d:
            src.append(s)
            dst.append(d)
    src, dst = np.array(src), np.array(dst)
    return pos, src, dst


def _tiny(mult_in, mult_out, H=5, n_nodes=6, n_edges=11, seed=0, r_cut=4.0, n_radial=4):
    rng = np.random.default_rng(seed)
    pos, src, dst = _graph(n_nodes, n_edges, rng)
    L = len(mult_in) - 1
    paths = so3.paths(L, L, L)
    f_in = sum((2 * l + 1) * m for l, m in enumerate(mult_in))
    f_out = sum((2 * l + 1) * m for l, m in enumerate(mult_out))
    x = rng.standard_normal((n_nodes, f_in))
    W1 = rng.standard_normal((n_radial, H)) / np.sqrt(n_radial)
    W2 = rng.standard_normal((H, sum(mult_in[l1] for (l1, _, _) in paths))) / np.sqrt(H)
    Wlin = [rng.standard_normal((mult_in[l1], mult_out[l3])) for (l1, _, l3) in paths]
    G = rng.standard_normal((n_nodes, f_out))
    return mixed.Problem(pos[src] - pos[dst], src, dst, n_nodes, x, W1, W2, Wlin, mult_in,
                         mult_out, r_cut, G=G)


def _padded(pb):
    """The same inputs in the uniform layout of oracle.conv, zero-padded to C = max m_in."""
    C, L = max(pb.mult_in), pb.L
    F = (L + 1) ** 2
    x = np.zeros((pb.n_nodes, F, C))
    for l, b in enumerate(pb.x):
        x[:, l * l:(l + 1) ** 2, :b.shape[2]] = b
    W2 = np.zeros((pb.W1.shape[1], len(pb.paths) * C))
    for p, (l1, _, _) in enumerate(pb.paths):
        W2[:, p * C:p * C + pb.mult_in[l1]] = pb.W2[:, pb.wcol[p]:pb.wcol[p] + pb.mult_in[l1]]
    return x, W2, C


@pytest.mark.parametrize("L", [1, 2, 3])
def test_uniform_multiplicities_with_identity_maps_are_the_convolution(L):
    C = 3
    pb = _tiny([C] * (L + 1), [C] * (L + 1), seed=L)
    pb.Wlin = [np.eye(C) for _ in pb.paths]
    F = (L + 1) ** 2
    x_u = np.concatenate([b.reshape(pb.n_nodes, -1) for b in pb.x], axis=1).reshape(pb.n_nodes, F, C)
    G_u = mixed.join(pb.G).reshape(pb.n_nodes, F, C)
    cp = conv.Problem(pb.vec, pb.src, pb.dst, pb.n_nodes, x_u, pb.W1, pb.W2, L, L, L, pb.r_cut, G=G_u)
    out = mixed.forward(pb).reshape(pb.n_nodes, F, C)
    ref = conv.forward(cp)
    assert np.abs(out - ref).max() < 1e-12 * np.abs(ref).max()
    g, gc = mixed.backward(pb), conv.backward(cp)
    for k in ("dvec", "dW1", "dW2"):
        assert np.abs(g[k] - gc[k]).max() < 1e-11 * np.abs(gc[k]).max(), k
    dx = g["dx"].reshape(pb.n_nodes, F, C)
    assert np.abs(dx - gc["dx"]).max() < 1e-11 * np.abs(gc["dx"]).max()


@pytest.mark.parametrize("mult_in,mult_out", [([4, 3, 2], [3, 2, 4]), ([6, 4, 2, 2], [6, 4, 2, 2]),
                                              ([2, 5], [3, 1])])
def test_composition_through_the_masked_convolution(mult_in, mult_out):
    pb = _tiny(mult_in, mult_out, seed=len(mult_in) + mult_in[0])
    L = pb.L
    x, W2, C = _padded(pb)
    out = [np.zeros((pb.n_nodes, 2 * l + 1, m)) for l, m in enumerate(mult_out)]
    for p, (l1, _, l3) in enumerate(pb.paths):
        mask = np.full(len(pb.src), 1 << p, dtype=np.int64)
        cp = conv.Problem(pb.vec, pb.src, pb.dst, pb.n_nodes, x, pb.W1, W2, L, L, L, pb.r_cut,
                          path_mask=mask)
        Mp = conv.forward(cp)[:, l3 * l3:(l3 + 1) ** 2, :mult_in[l1]]
        out[l3] += Mp @ pb.Wlin[p]
    ref = mixed.join(out)
    got = mixed.forward(pb)
    assert np.abs(got - ref).max() < 1e-12 * np.abs(ref).max()


def test_equivariance_under_rotation():
    pb = _tiny([4, 3, 2, 2], [3, 3, 2, 1], seed=21)
    out = mixed.forward(pb)
    a = (0.7, 1.1, -0.4)
    pb.vec = pb.vec @ so3.rotation_zyz(*a).T
    pb.x = [np.einsum("mk,nkc->nmc", so3.wigner_d_real(l, *a), b) for l, b in enumerate(pb.x)]
    out_r = mixed.forward(pb)
    rot = mixed.join([np.einsum("mk,nkc->nmc", so3.wigner_d_real(l, *a), b)
                      for l, b in enumerate(mixed.split(out, pb.mult_out))])
    assert np.abs(out_r - rot).max() < 1e-10 * np.abs(out).max()


def _loss(pb):
    return float(np.sum(mixed.join(pb.G) * mixed.forward(pb)))


@pytest.mark.parametrize("mult_in,mult_out", [([3, 2, 2], [2, 3, 1]), ([4, 2, 1, 1], [2, 2, 1, 1])])
def test_backward_matches_central_differences(mult_in, mult_out):
    pb = _tiny(mult_in, mult_out, n_nodes=5, n_edges=9, seed=40 + len(mult_in))
    g = mixed.backward(pb)
    h = 1e-6

    def fd(arr, idx):
        old = arr[idx]
        arr[idx] = old + h
        lp = _loss(pb)
        arr[idx] = old - h
        lm = _loss(pb)
        arr[idx] = old
        return (lp - lm) / (2 * h)

    rng = np.random.default_rng(1)
    dx = mixed.split(g["dx"], pb.mult_in)
    cases = [("vec", pb.vec, g["dvec"]), ("W1", pb.W1, g["dW1"]), ("W2", pb.W2, g["dW2"])]
    cases += [(f"x{l}", pb.x[l], dx[l]) for l in range(pb.L + 1)]
    cases += [(f"Wlin{p}", pb.Wlin[p], g["dWlin"][p]) for p in rng.choice(len(pb.paths), 4, replace=False)]
    for name, arr, grad in cases:
        scale = max(np.abs(grad).max(), 1.0)
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            assert abs(fd(arr, idx) - grad[idx]) <= 1e-7 * scale, name


def test_planted_mistake_is_caught(monkeypatch):
    """Swapping the receiver sums of two paths into the same rank changes the output."""
    pb = _tiny([3, 3, 2], [3, 3, 2], seed=5)
    good = mixed.forward(pb)
    orig = mixed.path_sums

    def wrong(pb_, chunk=2048, edges=None):
        M = orig(pb_, chunk, edges)
        # swap the outputs of two paths into l3 = 1 (both carry 3 channels there)
        i, j = [p for p, (l1, _, l3) in enumerate(pb_.paths) if l3 == 1 and pb_.mult_in[l1] == 3][:2]
        M[i], M[j] = M[j], M[i]
        return M
    monkeypatch.setattr(mixed, "path_sums", wrong)
    assert np.abs(mixed.forward(pb) - good).max() > 1e-3 * np.abs(good).max()
