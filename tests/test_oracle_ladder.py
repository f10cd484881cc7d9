"""Pins for the oracle's node-local product ladder: closed forms for the scalar-only and l <= 1
ladders, equivariance under random rotations (Wigner-D), homogeneity in the atomic basis, and
central finite differences of the backward.  Planted mistakes show the pins have teeth.  CPU only."""
import numpy as np
import pytest

from oracle import ladder, so3


def _rand(L, nu, N=5, C=3, seed=0):
    rng = np.random.default_rng(seed)
    P = len(ladder.paths(L))
    A = rng.standard_normal((N, (L + 1) ** 2, C))
    w = rng.standard_normal((nu - 1, P, C))
    G = rng.standard_normal((N, (L + 1) ** 2, C))
    return A, w, G


def _rotate(feat, a, L):
    out = np.empty_like(feat)
    for l in range(L + 1):
        D = so3.wigner_d_real(l, *a)
        out[:, l * l:(l + 1) ** 2, :] = np.einsum("mk,nkc->nmc", D, feat[:, l * l:(l + 1) ** 2, :])
    return out


# ---------------------------------------------------------------- closed forms
def _scalar_error(nu):
    """L = 0: one path (0,0,0), so B_s = (w_2 ... w_s) A^s and out = sum_{s>=2} B_s."""
    A, w, _ = _rand(0, nu, N=7, C=4, seed=nu)
    ref = np.zeros_like(A)
    coef = np.ones_like(A[:, 0, :])
    for s in range(2, nu + 1):
        coef = coef * w[s - 2, 0][None, :]
        ref[:, 0, :] += coef * A[:, 0, :] ** s
    return np.abs(ladder.forward(A, w, 0, nu) - ref).max() / np.abs(ref).max()


@pytest.mark.parametrize("nu", [2, 3, 4, 5])
def test_scalar_ladder_is_a_weighted_power_sum(nu):
    assert _scalar_error(nu) < 1e-13


def _l1_error():
    """L = 1, paths (0,0,0), (0,1,1), (1,0,1), (1,1,0).  With the unitary real CG blocks the
    (0,l,l) and (l,0,l) couplings are identities and (1,1,0) is -delta/sqrt(3), so one product of
    B (scalar b0, vector b) with A (a0, a) is
        out0 = w000 b0 a0 - w110 (b . a) / sqrt(3),    out1 = w011 b0 a + w101 a0 b.
    Two steps (nu = 3) fix which factor is the previous rung: B_3 uses B_2 as b and A as a."""
    A, w, _ = _rand(1, 3, N=6, C=2, seed=11)

    def step(B, wq):
        b0, b = B[:, 0, :], B[:, 1:4, :]
        a0, a = A[:, 0, :], A[:, 1:4, :]
        out = np.empty_like(A)
        out[:, 0, :] = wq[0] * b0 * a0 - wq[3] * np.sum(b * a, axis=1) / np.sqrt(3.0)
        out[:, 1:4, :] = wq[1][None, None, :] * b0[:, None, :] * a + \
            wq[2][None, None, :] * a0[:, None, :] * b
        return out

    B2 = step(A, w[0])
    B3 = step(B2, w[1])
    got = ladder.levels(A, w, 1, 3)
    scale = np.abs(B3).max()
    return max(np.abs(got[1] - B2).max(), np.abs(got[2] - B3).max(),
               np.abs(ladder.forward(A, w, 1, 3) - (B2 + B3)).max()) / scale


def test_l1_ladder_closed_form():
    assert ladder.paths(1) == [(0, 0, 0), (0, 1, 1), (1, 0, 1), (1, 1, 0)]
    assert _l1_error() < 1e-13


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("L,nu", [(2, 3), (3, 2), (3, 4)])
def test_equivariance_under_rotation(L, nu):
    A, w, _ = _rand(L, nu, N=4, C=3, seed=L * 10 + nu)
    rng = np.random.default_rng(L + nu)
    a = (rng.uniform(0, 2 * np.pi), rng.uniform(0, np.pi), rng.uniform(0, 2 * np.pi))
    out = ladder.forward(A, w, L, nu)
    out_r = ladder.forward(_rotate(A, a, L), w, L, nu)
    assert np.abs(out_r - _rotate(out, a, L)).max() < 1e-11 * np.abs(out).max()


def test_rungs_are_homogeneous_in_the_basis():
    """B_s is a degree-s polynomial in A: B_s(lambda A) = lambda^s B_s(A)."""
    A, w, _ = _rand(3, 5, N=3, C=2, seed=3)
    lam = 1.7
    B = ladder.levels(A, w, 3, 5)
    Bl = ladder.levels(lam * A, w, 3, 5)
    for s in range(1, 6):
        assert np.allclose(Bl[s - 1], lam ** s * B[s - 1], rtol=1e-12, atol=1e-12)


def test_linear_in_each_steps_weights():
    A, w, _ = _rand(2, 3, N=3, C=2, seed=4)
    w2 = w.copy()
    w2[1] *= 2.5                      # last step's weights enter B_3 linearly and B_2 not at all
    B = ladder.levels(A, w, 2, 3)
    B2 = ladder.levels(A, w2, 2, 3)
    assert np.allclose(B2[1], B[1], rtol=1e-14, atol=1e-14)
    assert np.allclose(B2[2], 2.5 * B[2], rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- backward
def _fd_error(dA, dw, A, w, G, L, nu, n=12):
    """Largest disagreement between (dA, dw) and central differences of <G, forward>."""
    def loss(A_, w_):
        return float(np.sum(G * ladder.forward(A_, w_, L, nu)))
    h = 1e-6
    rng = np.random.default_rng(1)
    err = 0.0
    for _ in range(n):
        for X, dX, is_A in ((A, dA, True), (w, dw, False)):
            i = tuple(rng.integers(0, s) for s in X.shape)
            Xp, Xm = X.copy(), X.copy()
            Xp[i] += h
            Xm[i] -= h
            fd = (loss(Xp, w) - loss(Xm, w)) / (2 * h) if is_A else \
                (loss(A, Xp) - loss(A, Xm)) / (2 * h)
            err = max(err, abs(fd - dX[i]) / max(1.0, abs(fd)))
    return err


@pytest.mark.parametrize("L,nu", [(1, 2), (2, 4), (3, 3)])
def test_backward_matches_central_differences(L, nu):
    A, w, G = _rand(L, nu, N=3, C=2, seed=20 + L + nu)
    dA, dw = ladder.backward(A, w, G, L, nu)
    assert _fd_error(dA, dw, A, w, G, L, nu) < 1e-6


# ---------------------------------------------------------------- the pins have teeth
def test_planted_mistakes_are_caught(monkeypatch):
    # (1) the factors of each product swapped (A first, previous rung second)
    orig = ladder.product
    monkeypatch.setattr(ladder, "product", lambda B, A_, w_, L: orig(A_, B, w_, L))
    assert _l1_error() > 1e-3
    monkeypatch.setattr(ladder, "product", orig)

    # (2) the sign of the (1,1,0) block flipped: equivariance cannot see it, the closed form does
    orig_cg = ladder._cg

    def flipped(L):
        cg = [c.copy() for c in orig_cg(L)]
        cg[ladder.paths(L).index((1, 1, 0))] *= -1
        return cg
    monkeypatch.setattr(ladder, "_cg", flipped)
    assert _l1_error() > 1e-3
    monkeypatch.setattr(ladder, "_cg", orig_cg)

    # (3) A itself added to the final sum
    monkeypatch.setattr(ladder, "forward",
                        lambda A_, w_, L, nu: np.sum(ladder.levels(A_, w_, L, nu), axis=0))
    assert _scalar_error(3) > 1e-3
    monkeypatch.undo()

    # (4) a backward that drops the gradient flowing into the previous rung
    L, nu = 2, 3
    A, w, G = _rand(L, nu, N=3, C=2, seed=7)
    B = ladder.levels(A, w, L, nu)
    dA_wrong = np.zeros_like(A)
    for s in (3, 2):
        for p, ((l1, l2, l3), Cp) in enumerate(zip(ladder.paths(L), ladder._cg(L))):
            wg = w[s - 2, p][None, None, :] * G[:, l3 * l3:l3 * l3 + 2 * l3 + 1, :]
            dA_wrong[:, l2 * l2:l2 * l2 + 2 * l2 + 1, :] += np.einsum(
                "ijk,nic,nkc->njc", Cp, B[s - 2][:, l1 * l1:l1 * l1 + 2 * l1 + 1, :], wg)
    _, dw = ladder.backward(A, w, G, L, nu)
    assert _fd_error(dA_wrong, dw, A, w, G, L, nu) > 1e-3


# ---------------------------------------------------------------- full ladder
def _rand_full(L, nu, N=4, C=3, seed=0):
    rng = np.random.default_rng(seed)
    P = len(ladder.paths(L))
    A = rng.standard_normal((N, (L + 1) ** 2, C))
    W = rng.standard_normal((nu - 1, P, C, C)) / np.sqrt(C)
    G = rng.standard_normal((N, (L + 1) ** 2, C))
    return A, W, G


@pytest.mark.parametrize("L,nu", [(1, 3), (2, 4), (3, 5)])
def test_full_ladder_with_diagonal_maps_is_the_path_reduced_ladder(L, nu):
    A, w, G = _rand(L, nu, N=4, C=3, seed=L + nu)
    W = np.zeros(w.shape + (w.shape[-1],))
    for q in range(nu - 1):
        for p in range(w.shape[1]):
            W[q, p] = np.diag(w[q, p])
    ref = ladder.forward(A, w, L, nu)
    assert np.abs(ladder.full_forward(A, W, L, nu) - ref).max() < 1e-12 * np.abs(ref).max()
    dA, dw = ladder.backward(A, w, G, L, nu)
    fA, fW = ladder.full_backward(A, W, G, L, nu)
    assert np.abs(fA - dA).max() < 1e-12 * np.abs(dA).max()
    # the diagonal of dL/dW is dL/dw
    diag = np.einsum("qpuu->qpu", fW)
    assert np.abs(diag - dw).max() < 1e-12 * np.abs(dw).max()


@pytest.mark.parametrize("L,nu", [(2, 3), (3, 2)])
def test_full_ladder_equivariance(L, nu):
    A, W, _ = _rand_full(L, nu, seed=5 + L)
    rng = np.random.default_rng(L)
    a = (rng.uniform(0, 2 * np.pi), rng.uniform(0, np.pi), rng.uniform(0, 2 * np.pi))
    out = ladder.full_forward(A, W, L, nu)
    out_r = ladder.full_forward(_rotate(A, a, L), W, L, nu)
    assert np.abs(out_r - _rotate(out, a, L)).max() < 1e-11 * np.abs(out).max()


def test_full_ladder_maps_mix_channels():
    """A map that moves channel 0 to channel 1 on one path moves that path's output alone."""
    L, nu, C = 1, 2, 3
    A, _, _ = _rand_full(L, nu, C=C, seed=9)
    P = len(ladder.paths(L))
    W = np.zeros((1, P, C, C))
    k = ladder.paths(L).index((0, 1, 1))
    W[0, k, 0, 1] = 1.0
    out = ladder.full_forward(A, W, L, nu)
    ref = np.zeros_like(out)
    ref[:, 1:4, 1] = A[:, 0, 0][:, None] * A[:, 1:4, 0]     # (0,1,1) is the identity coupling
    assert np.abs(out - ref).max() < 1e-13


@pytest.mark.parametrize("L,nu", [(1, 3), (2, 3)])
def test_full_ladder_backward_matches_central_differences(L, nu):
    A, W, G = _rand_full(L, nu, N=2, C=2, seed=30 + L)
    dA, dW = ladder.full_backward(A, W, G, L, nu)

    def loss(A_, W_):
        return float(np.sum(G * ladder.full_forward(A_, W_, L, nu)))
    h = 1e-6
    rng = np.random.default_rng(2)
    for _ in range(10):
        i = tuple(rng.integers(0, s) for s in A.shape)
        Ap, Am = A.copy(), A.copy()
        Ap[i] += h
        Am[i] -= h
        fd = (loss(Ap, W) - loss(Am, W)) / (2 * h)
        assert abs(fd - dA[i]) < 1e-6 * max(1.0, abs(fd))
        j = tuple(rng.integers(0, s) for s in W.shape)
        Wp, Wm = W.copy(), W.copy()
        Wp[j] += h
        Wm[j] -= h
        fd = (loss(A, Wp) - loss(A, Wm)) / (2 * h)
        assert abs(fd - dW[j]) < 1e-6 * max(1.0, abs(fd))
