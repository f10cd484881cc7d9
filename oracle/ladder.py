"""ORACLE (test infrastructure only).  The node-local product ladder with path-reduced products,
and its exact vector-Jacobian product, in float64 with plain numpy, one path at a time.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this module.  The
library never imports it; it shares no code with the HIP path.

Source: "FlashCart: Fast Cartesian Tensor Products for Equivariant Interatomic Potentials",
Fig. 3(b) (node-local tensor products as a function of the correlation order; path-reduced
products that sum contributions inside the kernel with one scalar weight per path and feature
channel) and Fig. E1(b) (the same atomic basis A enters every product; the output of each step
feeds the next product and is also added to the final sum).

What is computed, per node n and feature channel c, for correlation order nu >= 2:
    B_1 = A
    B_s[l3, m3] = sum_{p = (l1, l2, l3)} w[s-2, p, c] sum_{m1, m2} C_p[m1, m2, m3] B_{s-1}[l1, m1] A[l2, m2]
                  for s = 2..nu
    out = B_2 + B_3 + ... + B_nu
over the parity-allowed paths with l1, l2, l3 <= L (oracle.so3.paths(L, L, L) order).  A, B and out
are [N, (L+1)^2, C] (m-major blocks per l, channels innermost); w is [nu-1, P, C].

Readings where the pages are silent: B_{s-1} is the first factor and A the second; the final sum
holds the products' outputs B_2..B_nu (not A itself); weights are per (step, path, channel).

The second half of this module (full_forward, full_backward) is the full ladder the same figure
compares against: each path's output is mixed over channels by its own C x C map before the paths
into one l3 are summed.  Pins: with diagonal maps it equals the path-reduced ladder (forward, dA and
the diagonal of dW), it is equivariant under rotations, a single off-diagonal entry moves one path's
output to another channel, and its gradients match central differences.
"""
from __future__ import annotations

import numpy as np

from . import so3


def feat_dim(L: int) -> int:
    return (L + 1) ** 2


def _blk(l: int) -> slice:
    return slice(l * l, l * l + 2 * l + 1)


def paths(L: int):
    return so3.paths(L, L, L)


def _cg(L: int):
    return [so3.real_cg(*p) for p in paths(L)]


def product(B: np.ndarray, A: np.ndarray, w: np.ndarray, L: int) -> np.ndarray:
    """One path-reduced product: out[n, l3 m3, c] = sum_p w[p, c] sum C_p B[l1 m1] A[l2 m2]."""
    out = np.zeros((A.shape[0], feat_dim(L), A.shape[2]))
    for p, ((l1, l2, l3), Cp) in enumerate(zip(paths(L), _cg(L))):
        t = np.einsum("ijk,nic,njc->nkc", Cp, B[:, _blk(l1), :], A[:, _blk(l2), :])
        out[:, _blk(l3), :] += w[p][None, None, :] * t
    return out


def levels(A, w, L: int, nu: int):
    """[B_1, B_2, ..., B_nu]."""
    A = np.asarray(A, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    assert nu >= 2 and w.shape[0] == nu - 1 and w.shape[1] == len(paths(L))
    B = [A]
    for s in range(2, nu + 1):
        B.append(product(B[-1], A, w[s - 2], L))
    return B


def forward(A, w, L: int, nu: int) -> np.ndarray:
    B = levels(A, w, L, nu)
    return np.sum(B[1:], axis=0)


def backward(A, w, G, L: int, nu: int):
    """dA [N, F, C] and dw [nu-1, P, C] for the loss <G, forward(A, w)>."""
    A = np.asarray(A, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    B = levels(A, w, L, nu)
    dA = np.zeros_like(A)
    dw = np.zeros(w.shape)
    g_next = np.zeros_like(A)          # gradient reaching B_s through step s+1
    for s in range(nu, 1, -1):
        Gs = G + g_next                # B_s is in the sum and feeds step s+1
        Bp = B[s - 2]                  # B_{s-1}
        dB = np.zeros_like(A)
        for p, ((l1, l2, l3), Cp) in enumerate(zip(paths(L), _cg(L))):
            b1, a2, g3 = Bp[:, _blk(l1), :], A[:, _blk(l2), :], Gs[:, _blk(l3), :]
            t = np.einsum("ijk,nic,njc->nkc", Cp, b1, a2)
            dw[s - 2, p] += np.einsum("nkc,nkc->c", g3, t)
            wg = w[s - 2, p][None, None, :] * g3
            dB[:, _blk(l1), :] += np.einsum("ijk,njc,nkc->nic", Cp, a2, wg)
            dA[:, _blk(l2), :] += np.einsum("ijk,nic,nkc->njc", Cp, b1, wg)
        g_next = dB
    dA += g_next                       # B_1 = A
    return dA, dw


def flops_per_node_channel_step(L: int) -> int:
    """Algorithmic FLOP of one product per (node, channel): for each path, the sums over m2 for
    every (m1, m3) pair that has entries (one FMA per CG entry), one FMA per (m1, m3) pair to
    contract with B, and one FMA per output component to apply the path weight."""
    n = 0
    for (l1, l2, l3), Cp in zip(paths(L), _cg(L)):
        nz = np.abs(Cp) > 1e-12
        n += int(nz.sum()) + int(nz.any(axis=1).sum()) + (2 * l3 + 1)
    return 2 * n


# ----------------------------------------------------------------------------------------------
# Full ladder: the products' per-path outputs mixed by linear maps between steps
# ----------------------------------------------------------------------------------------------
# FlashCart, Fig. 3(b) (dashed curves: the full ladder, with the linear maps that mix paths and
# channels between steps) and Fig. E1(b) (the products' outputs over the retained coupling paths
# are compressed by W^(q) to d channels per retained rank).  Reading: every rank up to L is kept,
# d = C (the same channels as A, so the products stay channelwise), and W^(q) is one C x C map
# per path, the maps of the paths into the same l3 summed:
#     T_p[n, m3, u] = sum_{m1, m2} C_p[m1, m2, m3] B_{s-1}[n, l1, m1, u] A[n, l2, m2, u]
#     B_s[n, l3, m3, v] = sum_{p -> l3} sum_u T_p[n, m3, u] W[s-2, p, u, v]
# out = B_2 + ... + B_nu as before; W is [nu-1, P, C, C].  With W[s-2, p] = diag(w[s-2, p]) this
# is the path-reduced ladder above.

def path_outputs(B: np.ndarray, A: np.ndarray, L: int):
    """[T_p] for every path p, each [N, 2l3+1, C]."""
    return [np.einsum("ijk,nic,njc->nkc", Cp, B[:, _blk(l1), :], A[:, _blk(l2), :])
            for (l1, l2, l3), Cp in zip(paths(L), _cg(L))]


def full_product(B: np.ndarray, A: np.ndarray, W: np.ndarray, L: int) -> np.ndarray:
    out = np.zeros((A.shape[0], feat_dim(L), A.shape[2]))
    for p, ((l1, l2, l3), T) in enumerate(zip(paths(L), path_outputs(B, A, L))):
        out[:, _blk(l3), :] += T @ W[p]
    return out


def full_levels(A, W, L: int, nu: int):
    A = np.asarray(A, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    assert nu >= 2 and W.shape[:2] == (nu - 1, len(paths(L)))
    B = [A]
    for s in range(2, nu + 1):
        B.append(full_product(B[-1], A, W[s - 2], L))
    return B


def full_forward(A, W, L: int, nu: int) -> np.ndarray:
    return np.sum(full_levels(A, W, L, nu)[1:], axis=0)


def full_backward(A, W, G, L: int, nu: int):
    """dA [N, F, C] and dW [nu-1, P, C, C] for the loss <G, full_forward(A, W)>."""
    A = np.asarray(A, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    B = full_levels(A, W, L, nu)
    dA = np.zeros_like(A)
    dW = np.zeros(W.shape)
    g_next = np.zeros_like(A)
    for s in range(nu, 1, -1):
        Gs = G + g_next
        Bp = B[s - 2]
        dB = np.zeros_like(A)
        for p, ((l1, l2, l3), Cp) in enumerate(zip(paths(L), _cg(L))):
            b1, a2, g3 = Bp[:, _blk(l1), :], A[:, _blk(l2), :], Gs[:, _blk(l3), :]
            T = np.einsum("ijk,nic,njc->nkc", Cp, b1, a2)
            dW[s - 2, p] += np.einsum("nku,nkv->uv", T, g3)
            dT = g3 @ W[s - 2, p].T                                   # [N, 2l3+1, C]
            dB[:, _blk(l1), :] += np.einsum("ijk,njc,nkc->nic", Cp, a2, dT)
            dA[:, _blk(l2), :] += np.einsum("ijk,nic,nkc->njc", Cp, b1, dT)
        g_next = dB
    dA += g_next
    return dA, dW
