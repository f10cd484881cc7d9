"""ORACLE (test infrastructure only).  The E(3)-equivariant edge convolution and its exact
vector-Jacobian product, in float64 with plain numpy, one path at a time.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this module.  The
library never imports it; it shares no code with the HIP path (see oracle/so3.py).

What is computed, per edge e = (s -> d) with edge vector v_e:
    r = |v_e|,  u = v_e / r
    Y_l = real SH of u, l = 0..L_sh                       (oracle/so3.py)
    e_n = sqrt(2/r_c) sin(n pi r / r_c) / r * f(r / r_c),  n = 1..n_radial
    f(t) = 1 - 28 t^6 + 48 t^7 - 21 t^8 for t < 1, else 0
    h   = SiLU(e W1)                   (W1 [n_radial, H], no bias)
    w   = h W2                         (W2 [H, P*C], column p*C + c, no bias)
    out[d, l3, m3, c] += w[p, c] * sum_{m1, m2} C_p[m1, m2, m3] x[s, l1, m1, c] Y_l2[m2]
for every path p = (l1, l2, l3) (oracle.so3.paths order).  Paths with the same l3 are summed:
FlashCart, Fig. 3 caption, describes path-reduced products that sum contributions inside the
kernel with one scalar weight per path and feature channel.  Tensor products run in fp32 in the
library ("Fast and Accurate Foundation Models for Equivariant MLIPs", Sec. II: fp32 for tensor
products and scatter sums); the oracle is fp64.

The pages give neither the radial basis, the cutoff polynomial, nor the MLP shape; the readings
taken (Bessel basis, p = 6 polynomial envelope, two bias-free layers, plain scatter sum) are listed
with the other readings in the design notes.

Per-edge path subsets (optional): "BranchIP: Learning Adaptive Equivariant Computation for
Interatomic Potentials" (abstract) computes the tensor product adaptively, with a learned choice of
how much of it each interaction needs.  Here the choice is an input: a bitmask per edge, bit p set
when path p is computed for that edge.  A path that is off contributes nothing to that edge's
message, i.e. its radial weight is taken as zero:  w_eff[e, p, c] = mask[e, p] * w[e, p, c].
"""
from __future__ import annotations

import numpy as np

from . import so3


def feat_dim(L: int) -> int:
    return (L + 1) ** 2


def off(l: int) -> int:
    return l * l


# ----------------------------------------------------------------------------------------------
# Radial part
# ----------------------------------------------------------------------------------------------

def cutoff(t: np.ndarray) -> np.ndarray:
    return np.where(t < 1.0, 1.0 - 28.0 * t ** 6 + 48.0 * t ** 7 - 21.0 * t ** 8, 0.0)


def cutoff_deriv(t: np.ndarray) -> np.ndarray:
    return np.where(t < 1.0, -168.0 * t ** 5 + 336.0 * t ** 6 - 168.0 * t ** 7, 0.0)


def radial_basis(r: np.ndarray, n_radial: int, r_cut: float):
    """e [E, n_radial] and de/dr [E, n_radial]."""
    n = np.arange(1, n_radial + 1)[None, :]
    k = n * np.pi / r_cut
    A = np.sqrt(2.0 / r_cut)
    rr = r[:, None]
    B = A * np.sin(k * rr) / rr
    dB = A * (k * np.cos(k * rr) / rr - np.sin(k * rr) / rr ** 2)
    t = rr / r_cut
    f = cutoff(t)
    df = cutoff_deriv(t) / r_cut
    return B * f, dB * f + B * df


def round_bf16(a) -> np.ndarray:
    """a rounded to fp32, then to the nearest bfloat16 (8-bit significand, ties to even), returned
    as float64.  The operand precision of the mixed-precision variant of the radial-MLP
    contractions (bf16 operands, fp32 accumulation: the training precision of "High-performance
    training and inference for deep equivariant interatomic potentials"); the library holds
    fp32 values there, so the oracle rounds through fp32 too."""
    u = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32)).view(np.uint32)
    u = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def silu(z):
    return z / (1.0 + np.exp(-z))


def silu_deriv(z):
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


# ----------------------------------------------------------------------------------------------
# Per-edge state
# ----------------------------------------------------------------------------------------------

class Problem:
    """fp64 copy of one workload's inputs plus its path table."""

    def __init__(self, vec, src, dst, n_nodes, x, W1, W2, L_in, L_sh, L_out, r_cut, G=None,
                 W_lin=None, mlp_bf16=False, path_mask=None):
        self.vec = np.asarray(vec, dtype=np.float64)
        self.src = np.asarray(src, dtype=np.int64)
        self.dst = np.asarray(dst, dtype=np.int64)
        self.n_nodes = int(n_nodes)
        self.x = np.asarray(x, dtype=np.float64)
        self.W1 = np.asarray(W1, dtype=np.float64)
        self.W2 = np.asarray(W2, dtype=np.float64)
        self.L_in, self.L_sh, self.L_out = L_in, L_sh, L_out
        self.r_cut = float(r_cut)
        self.C = self.x.shape[2]
        self.paths = so3.paths(L_in, L_sh, L_out)
        self.cg = [so3.real_cg(*p) for p in self.paths]
        self.G = None if G is None else np.asarray(G, dtype=np.float64)
        self.W_lin = None if W_lin is None else [np.asarray(w, dtype=np.float64) for w in W_lin]
        assert self.W2.shape[1] == len(self.paths) * self.C
        # bf16 operands for the three W2 contractions (w = h W2, dL/dh = dL/dw W2^T,
        # dL/dW2 = h^T dL/dw); every sum and every other step stays at full precision
        self.mlp_bf16 = bool(mlp_bf16)
        # per-edge path bitmask (bit p = path p is computed for the edge), or None for all paths
        if path_mask is None:
            self.mask = None
        else:
            pm = np.asarray(path_mask).astype(np.int64) & 0xFFFFFFFF
            self.mask = ((pm[:, None] >> np.arange(len(self.paths))[None, :]) & 1).astype(np.float64)

    def mlp_operand(self, a):
        return round_bf16(a) if self.mlp_bf16 else a

    @classmethod
    def from_workload(cls, wl, mlp_bf16=False):
        return cls(wl.vec, wl.src, wl.dst, wl.n_nodes, wl.x, wl.W1, wl.W2, wl.L, wl.L, wl.L,
                   wl.spec["r_cut"], G=wl.G, W_lin=wl.W_lin, mlp_bf16=mlp_bf16,
                   path_mask=getattr(wl, "path_mask", None))

    def edge_mask(self, edges: np.ndarray):
        """[len(edges), P] 0/1 factors of the paths computed for these edges."""
        if self.mask is None:
            return np.ones((len(edges), len(self.paths)))
        return self.mask[edges]

    def edge_state(self, edges: np.ndarray):
        v = self.vec[edges]
        r = np.linalg.norm(v, axis=1)
        u = v / r[:, None]
        Y = [so3.real_sh(l, u) for l in range(self.L_sh + 1)]
        e, de = radial_basis(r, self.W1.shape[0], self.r_cut)
        pre = e @ self.W1
        h = silu(pre)
        w = (self.mlp_operand(h) @ self.mlp_operand(self.W2)).reshape(len(edges), len(self.paths),
                                                                      self.C)
        w = w * self.edge_mask(edges)[:, :, None]
        return dict(v=v, r=r, u=u, Y=Y, e=e, de=de, pre=pre, h=h, w=w)


def _chunks(n: int, size: int):
    for a in range(0, n, size):
        yield np.arange(a, min(n, a + size))


# ----------------------------------------------------------------------------------------------
# Forward
# ----------------------------------------------------------------------------------------------

def forward(pb: Problem, edges=None, chunk: int = 2048) -> np.ndarray:
    """out [N, (L_out+1)^2, C] summed over the given edges (default: all)."""
    if edges is None:
        edges = np.arange(len(pb.src))
    edges = np.asarray(edges, dtype=np.int64)
    out = np.zeros((pb.n_nodes, feat_dim(pb.L_out), pb.C))
    for idx in _chunks(len(edges), chunk):
        ed = edges[idx]
        st = pb.edge_state(ed)
        xs = pb.x[pb.src[ed]]
        msg = np.zeros((len(ed), feat_dim(pb.L_out), pb.C))
        for p, (l1, l2, l3) in enumerate(pb.paths):
            x1 = xs[:, off(l1):off(l1) + 2 * l1 + 1, :]
            t = np.einsum("ijk,eic,ej->ekc", pb.cg[p], x1, st["Y"][l2])
            msg[:, off(l3):off(l3) + 2 * l3 + 1, :] += st["w"][:, p, None, :] * t
        np.add.at(out, pb.dst[ed], msg)
    return out


# ----------------------------------------------------------------------------------------------
# Backward: exact vector-Jacobian product of forward() for upstream gradient G.
# ----------------------------------------------------------------------------------------------

def backward(pb: Problem, G=None, edges=None, chunk: int = 2048, want_dx: bool = True):
    """Returns dict with
        dvec [E, 3]   (rows outside `edges` are zero)
        dx   [N, F_in, C]
        dW1  [n_radial, H]
        dW2  [H, P*C]
    for the loss <G, forward(edges)>."""
    G = pb.G if G is None else np.asarray(G, dtype=np.float64)
    if edges is None:
        edges = np.arange(len(pb.src))
    edges = np.asarray(edges, dtype=np.int64)
    P, C = len(pb.paths), pb.C
    dvec = np.zeros((len(pb.src), 3))
    dx = np.zeros_like(pb.x) if want_dx else None
    dW1 = np.zeros_like(pb.W1)
    dW2 = np.zeros_like(pb.W2)
    for idx in _chunks(len(edges), chunk):
        ed = edges[idx]
        st = pb.edge_state(ed)
        st["mask"] = pb.edge_mask(ed)
        xs = pb.x[pb.src[ed]]
        Gd = G[pb.dst[ed]]
        dw = np.zeros((len(ed), P, C))
        dY = [np.zeros_like(y) for y in st["Y"]]
        dxs = np.zeros_like(xs)
        for p, (l1, l2, l3) in enumerate(pb.paths):
            Cp = pb.cg[p]
            x1 = xs[:, off(l1):off(l1) + 2 * l1 + 1, :]
            g3 = Gd[:, off(l3):off(l3) + 2 * l3 + 1, :]
            Y2 = st["Y"][l2]
            t = np.einsum("ijk,eic,ej->ekc", Cp, x1, Y2)
            dw[:, p, :] = np.einsum("ekc,ekc->ec", g3, t) * st["mask"][:, p, None]
            wg = st["w"][:, p, None, :] * g3
            dY[l2] += np.einsum("ijk,eic,ekc->ej", Cp, x1, wg)
            dxs[:, off(l1):off(l1) + 2 * l1 + 1, :] += np.einsum("ijk,ej,ekc->eic", Cp, Y2, wg)
        dwf = dw.reshape(len(ed), P * C)
        dW2 += pb.mlp_operand(st["h"]).T @ pb.mlp_operand(dwf)
        dh = pb.mlp_operand(dwf) @ pb.mlp_operand(pb.W2).T
        dpre = dh * silu_deriv(st["pre"])
        dW1 += st["e"].T @ dpre
        de = dpre @ pb.W1.T
        dr = np.sum(de * st["de"], axis=1)
        # r = |v|: dr/dv = u.   Y(u), u = v / r: dY/dv = (I - u u^T) / r * grad P_l(u).
        gv = dr[:, None] * st["u"]
        u = st["u"]
        for l in range(pb.L_sh + 1):
            gp = so3.real_sh_grad(l, u)                       # [E, 2l+1, 3]
            gu = np.einsum("em,emk->ek", dY[l], gp)
            gu = gu - np.sum(gu * u, axis=1, keepdims=True) * u
            gv += gu / st["r"][:, None]
        dvec[ed] = gv
        if want_dx:
            np.add.at(dx, pb.src[ed], dxs)
    return dict(dvec=dvec, dx=dx, dW1=dW1, dW2=dW2)


# ----------------------------------------------------------------------------------------------
# Interaction block: convolution then a per-irrep channel-mixing linear y[n,l,m,:] = out[n,l,m,:] W_l
# ----------------------------------------------------------------------------------------------

def linear(feat: np.ndarray, W_lin, L: int) -> np.ndarray:
    y = np.empty_like(feat)
    for l in range(L + 1):
        y[:, off(l):off(l) + 2 * l + 1, :] = feat[:, off(l):off(l) + 2 * l + 1, :] @ W_lin[l]
    return y


def linear_backward_data(dy: np.ndarray, W_lin, L: int) -> np.ndarray:
    d = np.empty_like(dy)
    for l in range(L + 1):
        d[:, off(l):off(l) + 2 * l + 1, :] = dy[:, off(l):off(l) + 2 * l + 1, :] @ W_lin[l].T
    return d


def linear_backward_weight(feat: np.ndarray, dy: np.ndarray, L: int):
    return [np.einsum("nmu,nmv->uv", feat[:, off(l):off(l) + 2 * l + 1, :],
                      dy[:, off(l):off(l) + 2 * l + 1, :]) for l in range(L + 1)]


def forces(dvec: np.ndarray, src: np.ndarray, dst: np.ndarray, n_nodes: int) -> np.ndarray:
    """F = -dE/dpos with vec = pos[src] - pos[dst]:  F[dst] += dE/dvec,  F[src] -= dE/dvec."""
    F = np.zeros((n_nodes, 3))
    np.add.at(F, dst, dvec)
    np.add.at(F, src, -dvec)
    return F
