"""Pins for the oracle's SO(3) pieces: printed values (FlashCart Table C1), closed forms, library
routines (scipy spherical harmonics) and invariants.  CPU only."""
import json
import os

import numpy as np
import pytest
import scipy.special as sp

from oracle import so3
from tensor_product_gnn_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(rng, n):
    u = rng.standard_normal((n, 3))
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def _couplings(L):
    return [(l1, l2, l3) for l1 in range(L + 1) for l2 in range(l1, L + 1) for l3 in range(L + 1)
            if abs(l1 - l2) <= l3 <= l1 + l2 and (l1 + l2 + l3) % 2 == 0]


# ---------------------------------------------------------------- printed values: Table C1
def test_table_c1_couplings_and_sparse_cg_ops():
    with open(os.path.join(GOLDEN, "table_c1.json")) as f:
        tab = json.load(f)
    for L, n_coup, _full, _indep, sparse in tab["rows"]:
        cps = _couplings(L)
        assert len(cps) == n_coup
        ops = sum(3 * int(np.count_nonzero(np.abs(so3.real_cg(*p)) > 1e-12)) - (2 * p[2] + 1)
                  for p in cps) - 1
        assert ops == sparse


def test_path_counts_match_configs():
    for L, n in workloads.N_PATHS_FOR_L.items():
        assert len(so3.paths(L, L, L)) == n
    assert so3.paths(1, 1, 1) == [(0, 0, 0), (0, 1, 1), (1, 0, 1), (1, 1, 0)]
    # every path obeys parity: l1 + l2 + l3 even (parity-restricted irreps)
    assert all((a + b + c) % 2 == 0 for a, b, c in so3.paths(3, 3, 3))


def test_cg_nnz_per_path():
    # Nonzero counts of the real-basis CG for the 23 lmax-3 paths (sum 353); the 11 lmax-2 paths
    # sum to 83 and the 4 lmax-1 paths to 10.
    nnz = [int(np.count_nonzero(np.abs(so3.real_cg(*p)) > 1e-12)) for p in so3.paths(3, 3, 3)]
    assert nnz == [1, 3, 5, 7, 3, 3, 11, 11, 21, 21, 5, 11, 21, 5, 25, 21, 41, 7, 21, 21, 41, 7, 41]
    assert sum(int(np.count_nonzero(np.abs(so3.real_cg(*p)) > 1e-12)) for p in so3.paths(2, 2, 2)) == 83
    assert sum(int(np.count_nonzero(np.abs(so3.real_cg(*p)) > 1e-12)) for p in so3.paths(1, 1, 1)) == 10


# ---------------------------------------------------------------- real SH
def test_sh_closed_forms():
    u = _unit(np.random.default_rng(0), 50)
    x, y, z = u.T
    assert np.allclose(so3.real_sh(0, u), 1.0, atol=1e-15)
    assert np.allclose(so3.real_sh(1, u), np.sqrt(3) * np.stack([y, z, x], -1), atol=1e-14)
    s15 = np.sqrt(15)
    Y2 = np.stack([s15 * x * y, s15 * y * z, np.sqrt(5) / 2 * (3 * z * z - 1), s15 * x * z,
                   s15 / 2 * (x * x - y * y)], -1)
    assert np.allclose(so3.real_sh(2, u), Y2, atol=1e-13)


@pytest.mark.parametrize("l", [0, 1, 2, 3, 4])
def test_sh_against_scipy_condon_shortley(l):
    u = _unit(np.random.default_rng(1), 40)
    th, ph = np.arccos(u[:, 2]), np.arctan2(u[:, 1], u[:, 0])
    Yc = np.stack([sp.sph_harm_y(l, m, th, ph) for m in range(-l, l + 1)], -1)
    Yr = np.sqrt(4 * np.pi) * (Yc @ so3.q_matrix(l).T)
    assert np.max(np.abs(Yr.imag)) < 1e-13
    assert np.allclose(Yr.real, so3.real_sh(l, u), atol=1e-13)


@pytest.mark.parametrize("l", [0, 1, 2, 3])
def test_sh_addition_theorem(l):
    rng = np.random.default_rng(2)
    u, v = _unit(rng, 30), _unit(rng, 30)
    assert np.allclose(np.sum(so3.real_sh(l, u) ** 2, -1), 2 * l + 1, atol=1e-13)
    # sum_m Y_lm(u) Y_lm(v) = (2l + 1) P_l(u . v)
    lhs = np.sum(so3.real_sh(l, u) * so3.real_sh(l, v), -1)
    rhs = (2 * l + 1) * sp.eval_legendre(l, np.sum(u * v, -1))
    assert np.allclose(lhs, rhs, atol=1e-13)


@pytest.mark.parametrize("l", [1, 2, 3])
def test_sh_gradient_finite_difference(l):
    # the polynomial gradient against central differences of the polynomial itself
    rng = np.random.default_rng(3)
    u = _unit(rng, 10)
    g = so3.real_sh_grad(l, u)
    h = 1e-6
    for k in range(3):
        d = np.zeros(3)
        d[k] = h
        fd = (np.stack([so3._eval_poly(so3.sh_polynomial(l, m), u + d) for m in range(-l, l + 1)], -1)
              - np.stack([so3._eval_poly(so3.sh_polynomial(l, m), u - d) for m in range(-l, l + 1)], -1)) / (2 * h)
        assert np.allclose(g[..., k], fd, atol=1e-8)


# ---------------------------------------------------------------- Wigner-D
def _angles(rng):
    return rng.uniform(0, 2 * np.pi), rng.uniform(0, np.pi), rng.uniform(0, 2 * np.pi)


def test_wigner_l1_is_permuted_rotation():
    rng = np.random.default_rng(4)
    P = np.array([[0, 1, 0], [0, 0, 1], [1, 0, 0.0]])  # (x, y, z) -> (y, z, x)
    for _ in range(5):
        a = _angles(rng)
        assert np.allclose(so3.wigner_d_real(1, *a), P @ so3.rotation_zyz(*a) @ P.T, atol=1e-14)


@pytest.mark.parametrize("l", [0, 1, 2, 3])
def test_wigner_orthogonal_homomorphism_and_sh(l):
    rng = np.random.default_rng(5 + l)
    a1, a2 = _angles(rng), _angles(rng)
    D1, D2 = so3.wigner_d_real(l, *a1), so3.wigner_d_real(l, *a2)
    R1, R2 = so3.rotation_zyz(*a1), so3.rotation_zyz(*a2)
    assert np.allclose(D1 @ D1.T, np.eye(2 * l + 1), atol=1e-13)
    # D(R1 R2) = D(R1) D(R2): recover Euler angles of R1 R2 from the matrix
    R = R1 @ R2
    b = np.arccos(np.clip(R[2, 2], -1, 1))
    a = np.arctan2(R[1, 2], R[0, 2])
    c = np.arctan2(R[2, 1], -R[2, 0])
    assert np.allclose(so3.rotation_zyz(a, b, c), R, atol=1e-12)
    assert np.allclose(so3.wigner_d_real(l, a, b, c), D1 @ D2, atol=1e-12)
    # Y(R u) = D(R) Y(u)
    u = _unit(rng, 20)
    assert np.allclose(so3.real_sh(l, u @ R1.T), so3.real_sh(l, u) @ D1.T, atol=1e-13)
    # least-squares D from samples agrees with the Wigner formula
    Yu, YRu = so3.real_sh(l, u), so3.real_sh(l, u @ R1.T)
    Dls = np.linalg.lstsq(Yu, YRu, rcond=None)[0].T
    assert np.allclose(Dls, D1, atol=1e-12)


# ---------------------------------------------------------------- Clebsch-Gordan
def test_cg_orthonormal_per_output():
    for p in so3.paths(3, 3, 3):
        C = so3.real_cg(*p)
        assert np.allclose(np.einsum("abk,abn->kn", C, C), np.eye(2 * p[2] + 1), atol=1e-13)


def test_cg_full_orthogonality_over_even_outputs():
    # For fixed (l1, l2), the CG blocks of all l3 (both parities) form an orthogonal change of
    # basis of the (2l1+1)(2l2+1) product space.
    for l1 in range(4):
        for l2 in range(4):
            blocks = [so3.real_cg(l1, l2, l3).reshape((2 * l1 + 1) * (2 * l2 + 1), -1)
                      for l3 in range(abs(l1 - l2), l1 + l2 + 1)]
            U = np.concatenate(blocks, axis=1)
            assert U.shape[0] == U.shape[1]
            assert np.allclose(U.conj().T @ U, np.eye(U.shape[0]), atol=1e-12)


def test_cg_special_cases():
    for l in range(4):
        assert np.allclose(so3.real_cg(0, l, l)[0], np.eye(2 * l + 1), atol=1e-14)
        assert np.allclose(so3.real_cg(l, 0, l)[:, 0, :], np.eye(2 * l + 1), atol=1e-14)
    # (1,1,0): the dot product, -1/sqrt(3) delta (Condon-Shortley sign of <1 0 1 0|0 0>)
    assert np.allclose(so3.real_cg(1, 1, 0)[:, :, 0], -np.eye(3) / np.sqrt(3), atol=1e-14)
    # (1,1,2): the output of two vectors is the symmetric traceless part of their outer product:
    # antisymmetric inputs and the identity give zero.
    C112 = so3.real_cg(1, 1, 2)
    assert np.allclose(C112 - C112.transpose(1, 0, 2), 0, atol=1e-14)
    assert np.allclose(np.einsum("aak->k", C112), 0, atol=1e-14)


def test_cg_equivariance():
    rng = np.random.default_rng(6)
    a = _angles(rng)
    for (l1, l2, l3) in so3.paths(3, 3, 3):
        C = so3.real_cg(l1, l2, l3)
        D1, D2, D3 = (so3.wigner_d_real(l, *a) for l in (l1, l2, l3))
        assert np.allclose(np.einsum("kn,abn->abk", D3, C),
                           np.einsum("ia,jb,ijk->abk", D1, D2, C), atol=1e-12)


def test_gaunt_identity():
    # sum_{m1,m2} C Y_l1 Y_l2 = sqrt((2l1+1)(2l2+1)/(2l3+1)) <l1 0 l2 0|l3 0> Y_l3
    u = _unit(np.random.default_rng(7), 25)
    for (l1, l2, l3) in so3.paths(3, 3, 3):
        lhs = np.einsum("abk,ea,eb->ek", so3.real_cg(l1, l2, l3), so3.real_sh(l1, u), so3.real_sh(l2, u))
        c = np.sqrt((2 * l1 + 1) * (2 * l2 + 1) / (2 * l3 + 1)) * so3.cg_complex(l1, 0, l2, 0, l3, 0)
        assert np.allclose(lhs, c * so3.real_sh(l3, u), atol=1e-12)


def test_racah_known_values():
    # textbook values
    assert np.isclose(so3.cg_complex(1, 0, 1, 0, 0, 0), -1 / np.sqrt(3), atol=1e-15)
    assert np.isclose(so3.cg_complex(1, 0, 1, 0, 2, 0), np.sqrt(2 / 3), atol=1e-15)
    assert np.isclose(so3.cg_complex(1, 1, 1, -1, 0, 0), 1 / np.sqrt(3), atol=1e-15)
    assert np.isclose(so3.cg_complex(1, 1, 1, 0, 2, 1), 1 / np.sqrt(2), atol=1e-15)
    assert np.isclose(so3.cg_complex(2, 2, 1, -1, 2, 1), np.sqrt(1 / 3), atol=1e-15)
    assert so3.cg_complex(1, 0, 1, 0, 1, 0) == 0.0
