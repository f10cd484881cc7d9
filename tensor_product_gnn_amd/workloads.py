"""Seeded synthetic inputs for the equivariant edge convolution.

This module only draws inputs: positions, graphs, edge vectors, node features, radial-MLP
weights, per-irrep linear weights and upstream gradients.  It holds none of the convolution's
arithmetic (no spherical harmonics, no Clebsch-Gordan coefficients, no radial basis), so that the
fp64 oracle and the HIP path can both consume it without sharing any of the method's code.

Workload shapes follow the pages:
  * "Fast and Accurate Foundation Models for Equivariant MLIPs" (arXiv 2607.28461), Sec. II:
    tensor products run in fp32; Table 1: irreps multiplicities and cutoffs of NequIP models.
  * "FlashCart: Fast Cartesian Tensor Products for Equivariant Interatomic Potentials", Fig. 3(a):
    edge convolutions on 1024 nodes with 128 edges per node, 128 channels, single precision;
    Fig. 1 / Table G1: a periodic 1000-atom diamond cell as the evaluation system.

All floating-point arrays are returned as float32 (the library's precision).  The oracle promotes
those exact float32 values to float64, so both sides see bit-identical inputs.

Conventions that are inputs rather than arithmetic:
  * edges are directed sender -> receiver, sorted by (receiver, sender); vec = pos[src] - pos[dst]
    (minimum image for periodic cells);
  * node tensors are laid out [node][l*l + (m + l)][channel] for l = 0..L (channels innermost);
  * W1 is [n_radial][hidden]; W2 is [hidden][n_paths * C] (path-major, channel-minor).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

# Each spec is data only.  "n_paths" is the number of Clebsch-Gordan paths the irreps imply
# (l1, l2, l3 <= L, triangle rule, l1 + l2 + l3 even): 1 / 4 / 11 / 23 for L = 0 / 1 / 2 / 3.
# It is stored here only to size W2; both the oracle and the library enumerate paths themselves
# and the tests assert they agree with this number.
N_PATHS_FOR_L = {0: 1, 1: 4, 2: 11, 3: 23}

SPECS: Dict[str, dict] = {
    # Tiny edge conv: 64 nodes in a 10 A cube, 8 distinct senders per receiver, 16x(0e+1o).
    "c0": dict(kind="random_in", n_nodes=64, box=10.0, k=8, L=1, C=16, n_radial=8, r_cut=5.0,
               hidden=16),
    # Kernel-benchmark shape: 1024 nodes, each sends to 128 distinct receivers, 128x(0e+1o+2e).
    "c1": dict(kind="random_out", n_nodes=1024, box=20.0, k=128, L=2, C=128, n_radial=8,
               r_cut=35.0, hidden=64),
    # Same graph as c1 with L = 3.
    "c2": dict(kind="random_out", n_nodes=1024, box=20.0, k=128, L=3, C=128, n_radial=8,
               r_cut=35.0, hidden=64),
    # 1000-atom periodic diamond cell (5x5x5 conventional cells), 5 A cutoff, L = 2, + linear.
    "c3": dict(kind="diamond", cells=5, a=3.567, sigma=0.05, L=2, C=128, n_radial=8, r_cut=5.0,
               hidden=64, linear=True),
    # 32768 atoms, random sequential addition at 0.1 atoms/A^3, 6 A cutoff, L = 3.
    "c4": dict(kind="rsa", n_nodes=32768, density=0.1, d_min=1.5, L=3, C=128, n_radial=8,
               r_cut=6.0, hidden=64),
    # Small parity cases with the shapes of c1..c4 (several 16-edge tiles and ragged tails).
    "c1s": dict(kind="random_out", n_nodes=48, box=20.0, k=40, L=2, C=128, n_radial=8,
                r_cut=35.0, hidden=64),
    "c2s": dict(kind="random_out", n_nodes=48, box=20.0, k=40, L=3, C=128, n_radial=8,
                r_cut=35.0, hidden=64),
    "c3s": dict(kind="diamond", cells=3, a=3.567, sigma=0.05, L=2, C=128, n_radial=8, r_cut=5.0,
                hidden=64, linear=True),
    "c4s": dict(kind="rsa", n_nodes=300, density=0.1, d_min=1.5, L=3, C=128, n_radial=8,
                r_cut=6.0, hidden=64),
    # Per-edge adaptive path subsets on c2's graph: each edge computes only the paths whose
    # spherical-harmonic degree l2 is at most its own degree, 3 for the shortest quarter of the
    # edges down to 0 for the longest quarter; edges sorted by (receiver, degree descending, sender).
    "c2a": dict(kind="random_out", n_nodes=1024, box=20.0, k=128, L=3, C=128, n_radial=8,
                r_cut=35.0, hidden=64, adaptive=True),
    "c2as": dict(kind="random_out", n_nodes=48, box=20.0, k=40, L=3, C=128, n_radial=8,
                 r_cut=35.0, hidden=64, adaptive=True),
    # Scalar-only case (irreps 0e): the convolution reduces to gather-scale-scatter.
    "l0": dict(kind="random_in", n_nodes=40, box=10.0, k=12, L=0, C=32, n_radial=8, r_cut=8.0,
               hidden=16),
}


@dataclasses.dataclass
class Workload:
    name: str
    spec: dict
    pos: np.ndarray          # [N, 3] float64 positions (A)
    box: Optional[float]     # periodic box edge (A) or None
    src: np.ndarray          # [E] int32 sender of each edge, edges sorted by (dst, src)
    dst: np.ndarray          # [E] int32 receiver of each edge
    row_ptr: np.ndarray      # [N + 1] int32 receiver CSR
    vec: np.ndarray          # [E, 3] float32 edge vectors pos[src] - pos[dst]
    x: np.ndarray            # [N, (L+1)^2, C] float32 node features
    W1: np.ndarray           # [n_radial, hidden] float32
    W2: np.ndarray           # [hidden, n_paths * C] float32
    W_lin: Optional[list]    # per l: [C, C] float32 (block workloads only)
    G: np.ndarray            # [N, (L+1)^2, C] float32 upstream gradient
    readout: np.ndarray      # [C] float32 invariant readout weights
    path_mask: Optional[np.ndarray] = None   # [E] uint32 per-edge path bitmask (adaptive only)

    @property
    def n_nodes(self) -> int:
        return int(self.pos.shape[0])

    @property
    def n_edges(self) -> int:
        return int(self.src.shape[0])

    @property
    def L(self) -> int:
        return int(self.spec["L"])

    @property
    def C(self) -> int:
        return int(self.spec["C"])

    def irreps(self) -> str:
        """Irreps string with parity (-1)^l, e.g. '128x0e+128x1o+128x2e'."""
        return "+".join(f"{self.C}x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(self.L + 1))

    def irreps_sh(self) -> str:
        return "+".join(f"1x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(self.L + 1))


def path_list(L: int):
    """The path order of W2's columns and of the path-mask bits: (l1, l2, l3) with every l <= L,
    |l1 - l2| <= l3 <= l1 + l2 and l1 + l2 + l3 even, lexicographic.  (An indexing convention of
    the inputs; the oracle and the library each enumerate it themselves.)"""
    return [(a, b, c) for a in range(L + 1) for b in range(L + 1) for c in range(L + 1)
            if abs(a - b) <= c <= a + b and (a + b + c) % 2 == 0]


def degree_masks(L: int) -> list:
    """mask[d]: bits of the paths with spherical-harmonic degree l2 <= d."""
    pl = path_list(L)
    return [sum(1 << i for i, (_, l2, _) in enumerate(pl) if l2 <= d) for d in range(L + 1)]


def _sort_edges(src: np.ndarray, dst: np.ndarray, n_nodes: int, key2=None):
    """Edges sorted by (receiver, key2, sender); key2 defaults to none."""
    order = np.lexsort((src, dst)) if key2 is None else np.lexsort((src, key2, dst))
    src = src[order].astype(np.int32)
    dst = dst[order].astype(np.int32)
    counts = np.bincount(dst, minlength=n_nodes)
    row_ptr = np.zeros(n_nodes + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    return src, dst, row_ptr.astype(np.int32), order


def _min_image(d: np.ndarray, box: Optional[float]) -> np.ndarray:
    if box is None:
        return d
    return d - box * np.round(d / box)


def _random_graph(rng, n: int, k: int, direction: str):
    """k distinct partners (never the node itself) per node, drawn node by node in index order.

    direction 'in': each node receives from k senders; 'out': each node sends to k receivers."""
    a = np.repeat(np.arange(n), k)
    b = np.empty(n * k, dtype=np.int64)
    for i in range(n):
        pick = rng.choice(n - 1, size=k, replace=False)
        pick = pick + (pick >= i)   # skip the node itself
        b[i * k:(i + 1) * k] = pick
    if direction == "in":
        return b, a   # src, dst
    return a, b


def _diamond_positions(rng, cells: int, a: float, sigma: float):
    basis = np.array([[0, 0, 0], [0, .5, .5], [.5, 0, .5], [.5, .5, 0],
                      [.25, .25, .25], [.25, .75, .75], [.75, .25, .75], [.75, .75, .25]])
    grid = np.stack(np.meshgrid(np.arange(cells), np.arange(cells), np.arange(cells),
                                indexing="ij"), -1).reshape(-1, 3)
    pos = (grid[:, None, :] + basis[None, :, :]).reshape(-1, 3) * a
    box = cells * a
    if sigma > 0:
        pos = pos + rng.normal(0.0, sigma, size=pos.shape)
    return np.mod(pos, box), box


def _rsa_positions(rng, n: int, box: float, d_min: float):
    """Random sequential addition in a periodic cube; a proposal is kept if it is at least d_min
    (minimum image) from every atom kept so far."""
    ncell = max(3, int(np.floor(box / d_min)))
    csize = box / ncell
    cap = 8
    cell_pos = np.zeros((ncell, ncell, ncell, cap, 3))
    cell_cnt = np.zeros((ncell, ncell, ncell), dtype=np.int64)
    out = np.empty((n, 3))
    got = 0
    offs = np.stack(np.meshgrid([-1, 0, 1], [-1, 0, 1], [-1, 0, 1], indexing="ij"), -1).reshape(-1, 3)
    d2min = d_min * d_min
    while got < n:
        batch = rng.uniform(0.0, box, size=(256, 3))
        for p in batch:
            c = np.minimum((p / csize).astype(np.int64), ncell - 1)
            nb = np.mod(c[None, :] + offs, ncell)
            cnt = cell_cnt[nb[:, 0], nb[:, 1], nb[:, 2]]
            if cnt.any():
                cand = cell_pos[nb[:, 0], nb[:, 1], nb[:, 2]]           # [27, cap, 3]
                mask = np.arange(cap)[None, :] < cnt[:, None]
                d = _min_image(cand[mask] - p[None, :], box)
                if np.min(np.einsum("ij,ij->i", d, d)) < d2min:
                    continue
            k = cell_cnt[c[0], c[1], c[2]]
            if k >= cap:
                continue
            cell_pos[c[0], c[1], c[2], k] = p
            cell_cnt[c[0], c[1], c[2]] = k + 1
            out[got] = p
            got += 1
            if got == n:
                break
    return out


def _cell_order(pos: np.ndarray, box: float, cell: float) -> np.ndarray:
    """Permutation that lists atoms cell by cell (x-major), for gather locality."""
    nc = max(1, int(np.floor(box / cell)))
    c = np.minimum((pos / (box / nc)).astype(np.int64), nc - 1)
    key = (c[:, 0] * nc + c[:, 1]) * nc + c[:, 2]
    return np.argsort(key, kind="stable")


def _radius_graph(pos: np.ndarray, box: float, r_cut: float):
    from scipy.spatial import cKDTree
    tree = cKDTree(pos, boxsize=box)
    pairs = tree.query_pairs(r_cut, output_type="ndarray").astype(np.int64)
    src = np.concatenate([pairs[:, 0], pairs[:, 1]])
    dst = np.concatenate([pairs[:, 1], pairs[:, 0]])
    return src, dst


def generate(name: str, seed: int = 0, spec: Optional[dict] = None) -> Workload:
    """Draw one workload.  Draw order with numpy.random.default_rng(seed): positions, graph, x,
    W1, W2, W_lin (block workloads), G, readout."""
    spec = dict(SPECS[name] if spec is None else spec)
    rng = np.random.default_rng(seed)
    kind = spec["kind"]
    box = None
    if kind in ("random_in", "random_out"):
        n = spec["n_nodes"]
        pos = rng.uniform(0.0, spec["box"], size=(n, 3))
        src, dst = _random_graph(rng, n, spec["k"], "in" if kind == "random_in" else "out")
    elif kind == "diamond":
        pos, box = _diamond_positions(rng, spec["cells"], spec["a"], spec["sigma"])
        src, dst = _radius_graph(pos, box, spec["r_cut"])
    elif kind == "rsa":
        n = spec["n_nodes"]
        box = float((n / spec["density"]) ** (1.0 / 3.0))
        pos = _rsa_positions(rng, n, box, spec["d_min"])
        pos = pos[_cell_order(pos, box, spec["r_cut"])]
        src, dst = _radius_graph(pos, box, spec["r_cut"])
    else:
        raise ValueError(kind)
    n = pos.shape[0]
    src, dst = np.asarray(src), np.asarray(dst)
    depth = None
    if spec.get("adaptive"):
        # per-edge spherical-harmonic degree from the distance rank: quarters of the edges, the
        # shortest get degree L, the longest degree 0
        dist = np.linalg.norm(_min_image(pos[src] - pos[dst], box), axis=1)
        rank = np.argsort(np.argsort(dist, kind="stable"), kind="stable")
        depth = spec["L"] - (rank * (spec["L"] + 1)) // len(dist)
    src, dst, row_ptr, order = _sort_edges(src, dst, n, None if depth is None else -depth)
    vec = _min_image(pos[src] - pos[dst], box).astype(np.float32)
    path_mask = None
    if depth is not None:
        path_mask = np.asarray(degree_masks(spec["L"]), dtype=np.uint32)[depth[order]]

    L, C, H, nr = spec["L"], spec["C"], spec["hidden"], spec["n_radial"]
    F = (L + 1) ** 2
    P = N_PATHS_FOR_L[L]
    x = rng.standard_normal((n, F, C)).astype(np.float32)
    W1 = (rng.standard_normal((nr, H)) / np.sqrt(nr)).astype(np.float32)
    W2 = (rng.standard_normal((H, P * C)) / np.sqrt(H)).astype(np.float32)
    W_lin = None
    if spec.get("linear"):
        W_lin = [(rng.standard_normal((C, C)) / np.sqrt(C)).astype(np.float32) for _ in range(L + 1)]
    G = rng.standard_normal((n, F, C)).astype(np.float32)
    readout = (rng.standard_normal(C) / np.sqrt(C)).astype(np.float32)
    return Workload(name=name, spec=spec, pos=pos, box=box, src=src, dst=dst, row_ptr=row_ptr,
                    vec=vec, x=x, W1=W1, W2=W2, W_lin=W_lin, G=G, readout=readout,
                    path_mask=path_mask)


def sender_csr(src: np.ndarray, n_nodes: int):
    """Edges grouped by sender: (t_row_ptr [N+1], t_perm [E]) with t_perm listing edge ids in
    (sender, edge id) order.  Graph bookkeeping only."""
    perm = np.argsort(src, kind="stable").astype(np.int32)
    counts = np.bincount(src, minlength=n_nodes)
    t_row_ptr = np.zeros(n_nodes + 1, dtype=np.int64)
    np.cumsum(counts, out=t_row_ptr[1:])
    return t_row_ptr.astype(np.int32), perm


# ------------------------------------------------------------------ node-local product ladder
# "FlashCart: Fast Cartesian Tensor Products for Equivariant Interatomic Potentials", Fig. 3(b):
# node-local tensor products on 4096 nodes, 128 channels, single precision, correlation order
# nu = 2..5.  Inputs: the atomic basis A [N, (L+1)^2, C], per-step path weights w [nu-1, P, C]
# and an upstream gradient G [N, (L+1)^2, C].
LADDER_SPECS: Dict[str, dict] = {
    "ladder": dict(n_nodes=4096, L=3, C=128, nu=5),
    # small parity cases: ragged node counts, every channel width the kernels take
    "ladder_s": dict(n_nodes=37, L=3, C=128, nu=5),
}


@dataclasses.dataclass
class LadderWorkload:
    name: str
    spec: dict
    A: np.ndarray            # [N, (L+1)^2, C] float32 atomic basis
    w: np.ndarray            # [nu-1, n_paths, C] float32 path weights per step
    G: np.ndarray            # [N, (L+1)^2, C] float32 upstream gradient

    @property
    def n_nodes(self) -> int:
        return int(self.A.shape[0])

    @property
    def L(self) -> int:
        return int(self.spec["L"])

    @property
    def C(self) -> int:
        return int(self.spec["C"])

    @property
    def nu(self) -> int:
        return int(self.spec["nu"])


def generate_ladder(name: str = "ladder", seed: int = 0, spec: Optional[dict] = None) -> LadderWorkload:
    """Draw order with numpy.random.default_rng(seed): A ~ N(0, 1), w ~ N(0, 1/P), G ~ N(0, 1)."""
    spec = dict(LADDER_SPECS[name] if spec is None else spec)
    rng = np.random.default_rng(seed)
    n, L, C, nu = spec["n_nodes"], spec["L"], spec["C"], spec["nu"]
    F = (L + 1) ** 2
    P = N_PATHS_FOR_L[L]
    A = rng.standard_normal((n, F, C)).astype(np.float32)
    w = (rng.standard_normal((nu - 1, P, C)) / np.sqrt(P)).astype(np.float32)
    G = rng.standard_normal((n, F, C)).astype(np.float32)
    return LadderWorkload(name=name, spec=spec, A=A, w=w, G=G)


@dataclasses.dataclass
class FullLadderWorkload:
    name: str
    spec: dict
    A: np.ndarray            # [N, (L+1)^2, C] float32 atomic basis
    W: np.ndarray            # [nu-1, n_paths, C, C] float32 channel-mixing map per step and path
    G: np.ndarray            # [N, (L+1)^2, C] float32 upstream gradient

    @property
    def n_nodes(self) -> int:
        return int(self.A.shape[0])

    @property
    def L(self) -> int:
        return int(self.spec["L"])

    @property
    def C(self) -> int:
        return int(self.spec["C"])

    @property
    def nu(self) -> int:
        return int(self.spec["nu"])


def generate_full_ladder(name: str = "ladder", seed: int = 0,
                         spec: Optional[dict] = None) -> FullLadderWorkload:
    """Same shapes as the path-reduced ladder's workloads, with one C x C map per step and path.
    Draw order with numpy.random.default_rng(seed): A ~ N(0, 1), W ~ N(0, 1/(P C)), G ~ N(0, 1)
    (a map's C inputs and a rank's paths each add a term, so 1/(P C) keeps the rungs at the scale
    of the path-reduced ladder's, whose weights are N(0, 1/P))."""
    spec = dict(LADDER_SPECS[name] if spec is None else spec)
    rng = np.random.default_rng(seed)
    n, L, C, nu = spec["n_nodes"], spec["L"], spec["C"], spec["nu"]
    F = (L + 1) ** 2
    P = N_PATHS_FOR_L[L]
    A = rng.standard_normal((n, F, C)).astype(np.float32)
    W = (rng.standard_normal((nu - 1, P, C, C)) / np.sqrt(P * C)).astype(np.float32)
    G = rng.standard_normal((n, F, C)).astype(np.float32)
    return FullLadderWorkload(name=name, spec=spec, A=A, W=W, G=G)


# Mixed multiplicities per rotation order ("Fast and Accurate Foundation Models for Equivariant
# MLIPs", Sec. III, Table 1: NequIP S 128,64; M 128,64,32; L 128,64,32,32) on the graphs above.
MIXED_SPECS: Dict[str, dict] = {
    "c2m": dict(graph="c2", mult_in=[128, 64, 32, 32], mult_out=[128, 64, 32, 32]),
    "c2ms": dict(graph="c2s", mult_in=[128, 64, 32, 32], mult_out=[128, 64, 32, 32]),
}


@dataclasses.dataclass
class MixedWorkload:
    name: str
    spec: dict
    graph: "Workload"         # the graph, edge vectors, W1 (the uniform workload's)
    mult_in: list
    mult_out: list
    x: np.ndarray             # [N, sum_l (2l+1) m_in[l]] float32
    W2: np.ndarray            # [H, sum_p m_in[l1(p)]]
    Wlin: np.ndarray          # concatenation over paths of [m_in[l1], m_out[l3]] (flat)
    G: np.ndarray             # [N, sum_l (2l+1) m_out[l]]

    @property
    def L(self) -> int:
        return len(self.mult_in) - 1

    def wlin_blocks(self):
        out, o = [], 0
        for (l1, _, l3) in path_list(self.L):
            a, b = self.mult_in[l1], self.mult_out[l3]
            out.append(self.Wlin[o:o + a * b].reshape(a, b))
            o += a * b
        return out

    @staticmethod
    def irreps(mult) -> str:
        return "+".join(f"{m}x{l}{'e' if l % 2 == 0 else 'o'}" for l, m in enumerate(mult))


def generate_mixed(name: str = "c2m", seed: int = 0, spec: Optional[dict] = None) -> MixedWorkload:
    """The graph, edge vectors and W1 of the named uniform workload; then, with
    numpy.random.default_rng(seed + 1): x ~ N(0, 1), W2 ~ N(0, 1/H), Wlin_p ~ N(0, 1/K(l3)) with
    K(l3) = sum over the paths into l3 of m_in[l1] (unit-scale outputs), G ~ N(0, 1)."""
    spec = dict(MIXED_SPECS[name] if spec is None else spec)
    g = generate(spec["graph"], seed=seed, spec=spec.get("graph_spec"))
    rng = np.random.default_rng(seed + 1)
    mi, mo = list(spec["mult_in"]), list(spec["mult_out"])
    L = len(mi) - 1
    assert g.spec["L"] == L
    n = g.x.shape[0]
    H = g.W1.shape[1]
    paths = path_list(L)
    f_in = sum((2 * l + 1) * m for l, m in enumerate(mi))
    f_out = sum((2 * l + 1) * m for l, m in enumerate(mo))
    x = rng.standard_normal((n, f_in)).astype(np.float32)
    W2 = (rng.standard_normal((H, sum(mi[l1] for (l1, _, _) in paths))) / np.sqrt(H)).astype(np.float32)
    K = [sum(mi[l1] for (l1, _, l3) in paths if l3 == t) for t in range(L + 1)]
    Wlin = np.concatenate([(rng.standard_normal((mi[l1], mo[l3])) / np.sqrt(K[l3])).ravel()
                           for (l1, _, l3) in paths]).astype(np.float32)
    G = rng.standard_normal((n, f_out)).astype(np.float32)
    return MixedWorkload(name=name, spec=spec, graph=g, mult_in=mi, mult_out=mo, x=x, W2=W2,
                         Wlin=Wlin, G=G)
