"""ORACLE (test infrastructure only).  The edge convolution with a different number of channels
per rotation order: per-path channelwise products, receiver sums kept per path, then one
channel-mixing linear map per output rank.  float64, plain numpy, one path at a time.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this module.  The
library never imports it; it shares no code with the HIP path.

Source: "Fast and Accurate Foundation Models for Equivariant MLIPs", Sec. III, Table 1: the NequIP
models' tensor features have their own channel count per rotation order (the large model 128,
64, 32 and 32 channels for l = 0..3).  The page gives the counts only.  Reading (the same edge
convolution as oracle.conv, written for per-l multiplicities):
  * a path p = (l1, l2, l3) is channelwise over the m_in[l1] channels of its input rank, so its
    output has m_in[l1] channels at rank l3; paths with different l1 cannot be summed channel by
    channel, so their receiver sums stay separate per path;
  * one linear map per path, Wlin_p [m_in[l1], m_out[l3]], takes them to the m_out[l3] output
    channels, and the maps of the paths into one l3 are summed (a channel-mixing linear per output
    rank over the concatenated path outputs);
  * the radial MLP gives one weight per (path, channel): W2 [H, sum_p m_in[l1(p)]], a block of
    m_in[l1] columns per path in path order.
Per edge e = (s -> d), with r, Y, the radial basis e and h = SiLU(e W1) exactly as in oracle.conv:
    w = h W2
    M_p[d, m3, u] += w[e, p, u] sum_{m1, m2} C_p[m1, m2, m3] x[s, l1 m1, u] Y_l2[m2]    (u < m_in[l1])
    out[d, l3 m3, v] = sum_{p -> l3} sum_u M_p[d, m3, u] Wlin_p[u, v]                  (v < m_out[l3])
With every multiplicity equal to C and every Wlin_p the identity this is oracle.conv.forward.

Node tensors with mixed multiplicities are stored [N, sum_l (2l+1) m[l]]: the blocks of l = 0, 1,
... in order, block l holding 2l+1 rows of m[l] channels (m-major, channels innermost).
"""
from __future__ import annotations

import numpy as np

from . import so3
from .conv import radial_basis, silu, silu_deriv


def block_offsets(mult):
    """Start of each l block in a mixed node tensor, and the row length."""
    offs, o = [], 0
    for l, m in enumerate(mult):
        offs.append(o)
        o += (2 * l + 1) * m
    return offs, o


def split(feat: np.ndarray, mult):
    """Mixed node tensor [N, sum] -> list over l of [N, 2l+1, m[l]]."""
    offs, _ = block_offsets(mult)
    return [feat[:, offs[l]:offs[l] + (2 * l + 1) * m].reshape(len(feat), 2 * l + 1, m)
            for l, m in enumerate(mult)]


def join(blocks) -> np.ndarray:
    return np.concatenate([b.reshape(len(b), -1) for b in blocks], axis=1)


class Problem:
    @classmethod
    def from_workload(cls, wl):
        g = wl.graph
        return cls(g.vec, g.src, g.dst, g.x.shape[0], wl.x, g.W1, wl.W2, wl.wlin_blocks(),
                   wl.mult_in, wl.mult_out, g.spec["r_cut"], G=wl.G)

    def __init__(self, vec, src, dst, n_nodes, x, W1, W2, Wlin, mult_in, mult_out, r_cut, G=None):
        self.vec = np.asarray(vec, dtype=np.float64)
        self.src = np.asarray(src, dtype=np.int64)
        self.dst = np.asarray(dst, dtype=np.int64)
        self.n_nodes = int(n_nodes)
        self.mult_in, self.mult_out = list(mult_in), list(mult_out)
        self.L = len(self.mult_in) - 1
        assert len(self.mult_out) == self.L + 1
        self.x = split(np.asarray(x, dtype=np.float64), self.mult_in)
        self.W1 = np.asarray(W1, dtype=np.float64)
        self.W2 = np.asarray(W2, dtype=np.float64)
        self.Wlin = [np.asarray(w, dtype=np.float64) for w in Wlin]
        self.r_cut = float(r_cut)
        self.paths = so3.paths(self.L, self.L, self.L)
        self.cg = [so3.real_cg(*p) for p in self.paths]
        self.wcol = []                         # first W2 column of each path
        o = 0
        for (l1, _, _) in self.paths:
            self.wcol.append(o)
            o += self.mult_in[l1]
        assert self.W2.shape[1] == o
        for p, (l1, _, l3) in enumerate(self.paths):
            assert self.Wlin[p].shape == (self.mult_in[l1], self.mult_out[l3])
        self.G = None if G is None else split(np.asarray(G, dtype=np.float64), self.mult_out)

    def edge_state(self, edges):
        v = self.vec[edges]
        r = np.linalg.norm(v, axis=1)
        u = v / r[:, None]
        Y = [so3.real_sh(l, u) for l in range(self.L + 1)]
        e, de = radial_basis(r, self.W1.shape[0], self.r_cut)
        pre = e @ self.W1
        h = silu(pre)
        return dict(v=v, r=r, u=u, Y=Y, e=e, de=de, pre=pre, h=h, w=h @ self.W2)

    def wp(self, w, p):
        l1 = self.paths[p][0]
        return w[:, self.wcol[p]:self.wcol[p] + self.mult_in[l1]]


def _chunks(n, size):
    for a in range(0, n, size):
        yield np.arange(a, min(n, a + size))


def _edge_list(pb, edges):
    return np.arange(len(pb.src)) if edges is None else np.asarray(edges, dtype=np.int64)


def path_sums(pb: Problem, chunk: int = 2048, edges=None):
    """M_p [N, 2l3+1, m_in[l1]] for every path: the receiver sums of the per-path messages over
    the given edges (default: all)."""
    M = [np.zeros((pb.n_nodes, 2 * l3 + 1, pb.mult_in[l1])) for (l1, _, l3) in pb.paths]
    edges = _edge_list(pb, edges)
    for idx in _chunks(len(edges), chunk):
        ed = edges[idx]
        st = pb.edge_state(ed)
        for p, (l1, l2, l3) in enumerate(pb.paths):
            t = np.einsum("ijk,eic,ej->ekc", pb.cg[p], pb.x[l1][pb.src[ed]], st["Y"][l2])
            np.add.at(M[p], pb.dst[ed], pb.wp(st["w"], p)[:, None, :] * t)
    return M


def forward(pb: Problem, edges=None) -> np.ndarray:
    """out [N, sum_l (2l+1) m_out[l]] summed over the given edges (default: all)."""
    M = path_sums(pb, edges=edges)
    out = [np.zeros((pb.n_nodes, 2 * l + 1, m)) for l, m in enumerate(pb.mult_out)]
    for p, (_, _, l3) in enumerate(pb.paths):
        out[l3] += M[p] @ pb.Wlin[p]
    return join(out)


def backward(pb: Problem, G=None, chunk: int = 2048, edges=None):
    """dvec [E, 3] (rows outside `edges` are zero), dx (mixed layout), dW1, dW2, dWlin (list per
    path) for <G, forward(edges)>."""
    G = pb.G if G is None else split(np.asarray(G, dtype=np.float64), pb.mult_out)
    M = path_sums(pb, edges=edges)
    dWlin = [M[p].reshape(-1, M[p].shape[2]).T @ G[l3].reshape(-1, G[l3].shape[2])
             for p, (_, _, l3) in enumerate(pb.paths)]
    dM = [G[l3] @ pb.Wlin[p].T for p, (_, _, l3) in enumerate(pb.paths)]   # dL/dM_p
    dvec = np.zeros((len(pb.src), 3))
    dx = [np.zeros_like(b) for b in pb.x]
    dW1 = np.zeros_like(pb.W1)
    dW2 = np.zeros_like(pb.W2)
    edges = _edge_list(pb, edges)
    for idx in _chunks(len(edges), chunk):
        ed = edges[idx]
        st = pb.edge_state(ed)
        dw = np.zeros_like(st["w"])
        dY = [np.zeros_like(y) for y in st["Y"]]
        for p, (l1, l2, l3) in enumerate(pb.paths):
            Cp, x1, Y2 = pb.cg[p], pb.x[l1][pb.src[ed]], st["Y"][l2]
            g3 = dM[p][pb.dst[ed]]                                       # [E, 2l3+1, m_in[l1]]
            t = np.einsum("ijk,eic,ej->ekc", Cp, x1, Y2)
            c0 = pb.wcol[p]
            dw[:, c0:c0 + pb.mult_in[l1]] = np.einsum("ekc,ekc->ec", g3, t)
            wg = pb.wp(st["w"], p)[:, None, :] * g3
            dY[l2] += np.einsum("ijk,eic,ekc->ej", Cp, x1, wg)
            np.add.at(dx[l1], pb.src[ed], np.einsum("ijk,ej,ekc->eic", Cp, Y2, wg))
        dW2 += st["h"].T @ dw
        dpre = (dw @ pb.W2.T) * silu_deriv(st["pre"])
        dW1 += st["e"].T @ dpre
        dr = np.sum((dpre @ pb.W1.T) * st["de"], axis=1)
        # r = |v|: dr/dv = u.  Y(u), u = v / r: dY/dv = (I - u u^T) / r * grad P_l(u)
        gv = dr[:, None] * st["u"]
        u = st["u"]
        for l in range(pb.L + 1):
            gu = np.einsum("em,emk->ek", dY[l], so3.real_sh_grad(l, u))
            gu = gu - np.sum(gu * u, axis=1, keepdims=True) * u
            gv += gu / st["r"][:, None]
        dvec[ed] = gv
    return dict(dvec=dvec, dx=join(dx), dW1=dW1, dW2=dW2, dWlin=dWlin)


def flops_per_edge(mult_in, mult_out, n_radial: int, hidden: int, n_nodes: int, n_edges: int):
    """Algorithmic FLOP of one forward per edge: products (per path and channel, one FMA per CG
    entry of the sums over m2 and one per (m1, m3) pair, plus the radial weight per output
    component), the radial MLP, and the linear maps (per node, spread over the edges)."""
    L = len(mult_in) - 1
    tp = mlp = lin = 0
    for (l1, l2, l3) in so3.paths(L, L, L):
        nz = np.abs(so3.real_cg(l1, l2, l3)) > 1e-12
        m = mult_in[l1]
        tp += 2 * (m * (int(nz.any(axis=1).sum()) + 2 * l3 + 1) + int(nz.sum()))
        mlp += 2 * hidden * m
        lin += 2 * (2 * l3 + 1) * m * mult_out[l3]
    mlp += 2 * n_radial * hidden
    return tp, mlp, lin * n_nodes / n_edges
