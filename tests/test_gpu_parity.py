"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle, element by element.

Small cases (every output, forward and all gradients) span several 16-edge tiles, ragged tails
and every channel slice; full-size cases (the configurations the benchmark times) are checked on
sampled receivers and sampled edges the oracle computes one by one.  Tolerance: max relative
error 1e-4 per output tensor (fp32 path vs fp64 oracle), metric in gpu_harness.rel_err."""
import numpy as np
import pytest

import tensor_product_gnn_amd as tp

from gpu_harness import (TOL, TOL_BF16, Device, problem, receiver_edges, rel_err, sample_edges,
                         sample_receivers)
from oracle import conv
from tensor_product_gnn_amd import workloads

pytestmark = pytest.mark.gpu


def _full_check(name):
    wl = workloads.generate(name)
    dev = Device(wl)
    out = dev.forward().cpu().numpy()
    grads = {k: v.cpu().numpy() for k, v in dev.backward().items()}
    pb = problem(wl)
    ref = conv.forward(pb)
    refg = conv.backward(pb)
    errs = {"out": rel_err(out, ref), "vec": rel_err(grads["vec"], refg["dvec"]),
            "x": rel_err(grads["x"], refg["dx"]), "W1": rel_err(grads["W1"], refg["dW1"]),
            "W2": rel_err(grads["W2"], refg["dW2"])}
    print(name, {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (name, k, v)


@pytest.mark.parametrize("name", ["c0", "l0", "c1s", "c2s"])
def test_small_full_parity(name):
    _full_check(name)


@pytest.mark.parametrize("name,n_recv,n_edge", [("c1", 12, 48), ("c2", 8, 32), ("c3", 12, 48),
                                                ("c4", 12, 48), ("c3s", 12, 64), ("c4s", 12, 64)])
def test_sampled_parity_at_benchmark_size(name, n_recv, n_edge):
    wl = workloads.generate(name)
    dev = Device(wl, sender_csr=False)
    out = dev.forward().cpu().numpy()
    g = dev.backward(want_x=False, want_W=False)["vec"].cpu().numpy()
    pb = problem(wl)
    recv = sample_receivers(wl, n_recv, seed=1)
    ref = conv.forward(pb, edges=receiver_edges(wl, recv))[recv]
    e = sample_edges(wl, n_edge, seed=2)
    refv = conv.backward(pb, edges=e, want_dx=False)["dvec"][e]
    eo, ev = rel_err(out[recv], ref), rel_err(g[e], refv)
    print(name, f"out {eo:.2e} dvec {ev:.2e}")
    assert eo <= TOL and ev <= TOL


# Relative tolerance of the linearity identities below, against sum_i |g_i d_i|: both sides are
# fp32 results summed in fp64, so they agree to rounding (~1e-7 of that scale); a gradient block
# that is wrong for a whole path or channel slice moves them apart by far more than 1e-5.
LIN_RTOL = 1e-5


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_linear_gradients_at_benchmark_size(name):
    """<G, out> is linear and homogeneous in W2 and in x, so for any d, <dL/dW2, d> equals
    <G, out> with W2 replaced by d, and <dL/dx, d> equals <G, out> with x replaced by d: the
    full-size weight and feature gradients (every edge, every work-group partial) checked against
    the library's own forward, without the oracle.  One path's W2 columns at a time, so that a
    block of the gradient landing in the wrong path group cannot hide (l <= 2: two backward
    launches; l <= 3: four)."""
    import torch
    wl = workloads.generate(name)
    dev = Device(wl)
    grads = dev.backward(want_x=True, want_W=True)
    gW2, gx = grads["W2"].double(), grads["x"].double()
    G = dev.G.double()
    H, PC = wl.W2.shape
    C = wl.spec["C"]
    rng = np.random.default_rng(5)
    worst = 0.0
    for p in range(PC // C):
        d = np.zeros((H, PC), np.float32)
        d[:, p * C:(p + 1) * C] = rng.standard_normal((H, C))
        dt = torch.from_numpy(d).cuda()
        lhs = float((gW2 * dt.double()).sum())
        scale = float((gW2 * dt.double()).abs().sum())
        rhs = float((G * dev.conv.forward(dev.g, dev.vec, dev.x, dev.W1, dt).double()).sum())
        err = abs(lhs - rhs) / scale
        worst = max(worst, err)
        assert err <= LIN_RTOL, (name, "W2 path", p, lhs, rhs, err)
    dx = torch.from_numpy(rng.standard_normal(wl.x.shape).astype(np.float32)).cuda()
    lhs = float((gx * dx.double()).sum())
    scale = float((gx * dx.double()).abs().sum())
    rhs = float((G * dev.conv.forward(dev.g, dev.vec, dx, dev.W1, dev.W2).double()).sum())
    errx = abs(lhs - rhs) / scale
    print(name, f"W2 (worst path) {worst:.2e} x {errx:.2e}")
    assert errx <= LIN_RTOL, (name, "x", lhs, rhs, errx)


def test_dx_sampled_senders_c2():
    wl = workloads.generate("c2")
    dev = Device(wl)
    dx = dev.backward(want_x=True, want_W=False)["x"].cpu().numpy()
    pb = problem(wl)
    senders = sample_receivers(wl, 6, seed=3)
    edges = np.nonzero(np.isin(wl.src, senders))[0]
    ref = conv.backward(pb, edges=edges)["dx"][senders]
    err = rel_err(dx[senders], ref)
    print("c2 dx", f"{err:.2e}")
    assert err <= TOL


def test_block_with_linear_c3s():
    """Interaction block: convolution, then the per-irrep 128x128 linear; forces via backward."""
    import torch
    import tensor_product_gnn_amd as tp
    wl = workloads.generate("c3s")
    dev = Device(wl, sender_csr=False)
    out = dev.forward()
    y = tp.linear(out, dev.W_lin, wl.L).cpu().numpy()
    dy = torch.from_numpy(wl.G).cuda()
    G = tp.linear(dy, dev.W_lin, wl.L, transpose=True)
    gv = dev.backward(G=G, want_x=False, want_W=False)["vec"].cpu().numpy()
    pb = problem(wl)
    recv = sample_receivers(wl, 10, seed=4)
    ref_out = conv.forward(pb, edges=receiver_edges(wl, recv))
    ref_y = conv.linear(ref_out, pb.W_lin, wl.L)[recv]
    Gref = conv.linear_backward_data(wl.G.astype(np.float64), pb.W_lin, wl.L)
    assert rel_err(G.cpu().numpy(), Gref) <= TOL
    e = sample_edges(wl, 48, seed=5)
    refv = conv.backward(pb, G=Gref, edges=e, want_dx=False)["dvec"][e]
    ey, ev = rel_err(y[recv], ref_y), rel_err(gv[e], refv)
    print("c3s block", f"y {ey:.2e} dvec {ev:.2e}")
    assert ey <= TOL and ev <= TOL


@pytest.mark.parametrize("C,lmax,n_nodes", [(16, 1, 37), (32, 3, 5), (64, 2, 100), (128, 2, 1000),
                                             (128, 3, 11)])
def test_linear_against_oracle(C, lmax, n_nodes):
    """Per-irrep linear and its data gradient on ragged row counts (several work-groups per l and
    partial last tiles), every supported channel count."""
    import torch
    import tensor_product_gnn_amd as tp
    rng = np.random.default_rng(C + lmax)
    F = (lmax + 1) ** 2
    feat = rng.standard_normal((n_nodes, F, C)).astype(np.float32)
    W = [(rng.standard_normal((C, C)) / np.sqrt(C)).astype(np.float32) for _ in range(lmax + 1)]
    tf, tW = torch.from_numpy(feat).cuda(), torch.from_numpy(np.stack(W)).cuda()
    y = tp.linear(tf, tW, lmax).cpu().numpy()
    yt = tp.linear(tf, tW, lmax, transpose=True).cpu().numpy()
    W64 = [w.astype(np.float64) for w in W]
    ey = rel_err(y, conv.linear(feat.astype(np.float64), W64, lmax))
    et = rel_err(yt, conv.linear_backward_data(feat.astype(np.float64), W64, lmax))
    print(f"linear C={C} l<={lmax} n={n_nodes}: {ey:.2e} {et:.2e}")
    assert ey <= TOL and et <= TOL


@pytest.mark.parametrize("name", ["c1s", "c2s"])
def test_bf16_mlp_operands_small_full_parity(name):
    """The mixed-precision variant (bf16 operands for the W2 contractions, fp32 elsewhere) against
    the oracle rounding the same operands, every output and gradient."""
    wl = workloads.generate(name)
    dev = Device(wl, mlp_bf16=True)
    out = dev.forward().cpu().numpy()
    g = {k: v.cpu().numpy() for k, v in dev.backward().items()}
    pb = problem(wl, mlp_bf16=True)
    ref, refg = conv.forward(pb), conv.backward(pb)
    errs = {"out": rel_err(out, ref), "vec": rel_err(g["vec"], refg["dvec"]),
            "x": rel_err(g["x"], refg["dx"]), "W1": rel_err(g["W1"], refg["dW1"]),
            "W2": rel_err(g["W2"], refg["dW2"])}
    exact = conv.forward(problem(wl))
    print(name, "bf16", {k: f"{v:.2e}" for k, v in errs.items()},
          f"(out vs fp64 without rounding {rel_err(out, exact):.2e})")
    for k, v in errs.items():
        assert v <= TOL_BF16, (name, k, v)


def test_bf16_mlp_operands_sampled_c2():
    wl = workloads.generate("c2")
    dev = Device(wl, sender_csr=False, mlp_bf16=True)
    out = dev.forward().cpu().numpy()
    gv = dev.backward(want_x=False)["vec"].cpu().numpy()
    pb = problem(wl, mlp_bf16=True)
    recv = sample_receivers(wl, 8, seed=6)
    ref = conv.forward(pb, edges=receiver_edges(wl, recv))[recv]
    e = sample_edges(wl, 32, seed=7)
    refv = conv.backward(pb, edges=e, want_dx=False)["dvec"][e]
    eo, ev = rel_err(out[recv], ref), rel_err(gv[e], refv)
    print(f"c2 bf16 out {eo:.2e} dvec {ev:.2e}")
    assert eo <= TOL_BF16 and ev <= TOL_BF16


def test_deterministic_reruns():
    wl = workloads.generate("c2s")
    dev = Device(wl)
    a = dev.forward().cpu().numpy()
    b = dev.forward().cpu().numpy()
    ga = {k: v.cpu().numpy() for k, v in dev.backward().items()}
    gb = {k: v.cpu().numpy() for k, v in dev.backward().items()}
    assert np.array_equal(a, b)
    for k in ga:
        assert np.array_equal(ga[k], gb[k]), k


@pytest.mark.parametrize("subset", [("vec",), ("W1",), ("W2",), ("vec", "W2"), ("x", "W1")])
def test_gradient_subsets_match_full_backward(subset):
    """Only the requested gradients are produced, and they equal those of a full backward (the
    kernels without weight-gradient accumulation compute dL/dvec the same way)."""
    import torch
    wl = workloads.generate("c2s")
    dev = Device(wl)
    full = {k: v.cpu().numpy() for k, v in dev.backward().items()}
    flags = {f"want_{k}": (k in subset) for k in ("vec", "x", "W1", "W2")}
    sentinel = {k: torch.full_like(v, float("nan")) for k, v in dev.backward().items()}
    got = dev.conv.backward(dev.g, dev.vec, dev.x, dev.W1, dev.W2, dev.G, outs=sentinel, **flags)
    assert sorted(got) == sorted(subset)
    for k in ("vec", "x", "W1", "W2"):
        if k in subset:
            assert rel_err(got[k].cpu().numpy(), full[k]) <= 1e-6, k
        else:  # not requested: the caller's tensor is left untouched
            assert torch.isnan(sentinel[k]).all(), k


def test_equivariance_of_gpu_output():
    import torch
    from oracle import so3
    wl = workloads.generate("c2s")
    dev = Device(wl, sender_csr=False)
    out = dev.forward().cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(7)
    ang = (rng.uniform(0, 2 * np.pi), rng.uniform(0, np.pi), rng.uniform(0, 2 * np.pi))
    R = so3.rotation_zyz(*ang)

    def rot(f):
        o = np.empty_like(f)
        for l in range(wl.L + 1):
            D = so3.wigner_d_real(l, *ang)
            o[:, l * l:(l + 1) ** 2, :] = np.einsum("mk,nkc->nmc", D, f[:, l * l:(l + 1) ** 2, :])
        return o
    dev.vec = torch.from_numpy((wl.vec.astype(np.float64) @ R.T).astype(np.float32)).cuda()
    dev.x = torch.from_numpy(rot(wl.x.astype(np.float64)).astype(np.float32)).cuda()
    out_r = dev.forward().cpu().numpy()
    assert rel_err(out_r, rot(out)) <= 1e-4


def test_edge_cases_empty_isolated_and_ragged():
    """No edges; receivers with 0, 1, 15, 16, 17, 33 edges; edges beyond the cutoff."""
    import torch
    import tensor_product_gnn_amd as tp
    rng = np.random.default_rng(11)
    degs = [0, 1, 15, 16, 17, 0, 33, 2]
    n = len(degs) + 3
    src, dst = [], []
    for d, k in enumerate(degs):
        s = rng.choice([i for i in range(n) if i != d], size=k, replace=True)
        src += list(s)
        dst += [d] * k
    src, dst = np.array(src, dtype=np.int32), np.array(dst, dtype=np.int32)
    row_ptr = np.concatenate([[0], np.cumsum(np.bincount(dst, minlength=n))]).astype(np.int32)
    pos = rng.uniform(0, 6.0, size=(n, 3))
    vec = (pos[src] - pos[dst]).astype(np.float32)
    spec = dict(workloads.SPECS["c2s"])
    base = workloads.generate("c2s")
    wl = workloads.Workload(name="edge", spec=spec, pos=pos, box=None, src=src, dst=dst,
                            row_ptr=row_ptr, vec=vec, x=base.x[:n].copy(), W1=base.W1, W2=base.W2,
                            W_lin=None, G=base.G[:n].copy(), readout=base.readout)
    wl.spec["r_cut"] = 4.0   # some edges are beyond the cutoff
    assert np.any(np.linalg.norm(vec, axis=1) >= 4.0)
    _check_workload(wl)
    # no edges at all
    empty = workloads.Workload(name="empty", spec=spec, pos=pos, box=None,
                               src=np.zeros(0, np.int32), dst=np.zeros(0, np.int32),
                               row_ptr=np.zeros(n + 1, np.int32), vec=np.zeros((0, 3), np.float32),
                               x=wl.x, W1=wl.W1, W2=wl.W2, W_lin=None, G=wl.G, readout=wl.readout)
    dev = Device(empty)
    assert np.all(dev.forward().cpu().numpy() == 0)
    gr = dev.backward()
    assert np.all(gr["x"].cpu().numpy() == 0)
    assert np.all(gr["W1"].cpu().numpy() == 0) and np.all(gr["W2"].cpu().numpy() == 0)
    assert gr["vec"].numel() == 0


def _check_workload(wl):
    dev = Device(wl)
    out = dev.forward().cpu().numpy()
    grads = {k: v.cpu().numpy() for k, v in dev.backward().items()}
    pb = problem(wl)
    ref = conv.forward(pb)
    refg = conv.backward(pb)
    assert np.all(out[np.diff(wl.row_ptr) == 0] == 0)
    for k, a, b in (("out", out, ref), ("vec", grads["vec"], refg["dvec"]),
                    ("x", grads["x"], refg["dx"]), ("W1", grads["W1"], refg["dW1"]),
                    ("W2", grads["W2"], refg["dW2"])):
        e = rel_err(a, b)
        print(wl.name, k, f"{e:.2e}")
        assert e <= TOL, (k, e)


def test_build_csr_matches_stable_argsort():
    import torch
    import tensor_product_gnn_amd as tp
    wl = workloads.generate("c1")
    key = torch.from_numpy(wl.src).cuda()
    row_ptr, perm = tp.build_csr(key, wl.n_nodes)
    ref_rp, ref_perm = workloads.sender_csr(wl.src, wl.n_nodes)
    assert np.array_equal(row_ptr.cpu().numpy(), ref_rp)
    assert np.array_equal(perm.cpu().numpy(), ref_perm)


# ---------------------------------------------------------------- per-edge path subsets
def _mask_device(wl, mask, sender_csr=True):
    dev = Device(wl, sender_csr=sender_csr)
    dev.g = tp.Graph.from_arrays(wl.n_nodes, wl.row_ptr, wl.src, wl.dst, sender_csr=sender_csr,
                                 path_mask=mask)
    return dev


@pytest.mark.parametrize("name,kind", [("c1s", "random"), ("c2s", "random"), ("c2as", "degree"),
                                       ("c2s", "ones")])
def test_path_subsets_small_full_parity(name, kind):
    """Arbitrary per-edge masks (random bits: tiles mix every pattern), the distance-ranked degree
    masks of the adaptive workload, and the all-paths mask, against the oracle on every output."""
    wl = workloads.generate(name)
    P = workloads.N_PATHS_FOR_L[wl.L]
    if kind == "random":
        mask = np.random.default_rng(7).integers(0, 1 << P, size=wl.n_edges).astype(np.uint32)
    elif kind == "ones":
        mask = np.full(wl.n_edges, (1 << P) - 1, dtype=np.uint32)
    else:
        mask = wl.path_mask
    dev = _mask_device(wl, mask)
    out = dev.forward().cpu().numpy()
    grads = {k: v.cpu().numpy() for k, v in dev.backward().items()}
    pb = conv.Problem(wl.vec, wl.src, wl.dst, wl.n_nodes, wl.x, wl.W1, wl.W2, wl.L, wl.L, wl.L,
                      wl.spec["r_cut"], G=wl.G, path_mask=mask)
    ref = conv.forward(pb)
    refg = conv.backward(pb)
    errs = {"out": rel_err(out, ref), "vec": rel_err(grads["vec"], refg["dvec"]),
            "x": rel_err(grads["x"], refg["dx"]), "W1": rel_err(grads["W1"], refg["dW1"]),
            "W2": rel_err(grads["W2"], refg["dW2"])}
    print(name, kind, {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (name, kind, k, v)
    if kind == "ones":
        # the masked kernels with every path on agree with the plain kernels
        plain = Device(wl)
        assert rel_err(out, plain.forward().cpu().numpy()) <= 1e-6


def test_path_subsets_sampled_c2a():
    wl = workloads.generate("c2a")
    dev = _mask_device(wl, wl.path_mask, sender_csr=False)
    out = dev.forward().cpu().numpy()
    g = dev.backward(want_x=False, want_W=False)["vec"].cpu().numpy()
    pb = problem(wl)
    assert pb.mask is not None
    recv = sample_receivers(wl, 10, seed=3)
    ref = conv.forward(pb, edges=receiver_edges(wl, recv))[recv]
    e = sample_edges(wl, 40, seed=4)
    refv = conv.backward(pb, edges=e, want_dx=False)["dvec"][e]
    eo, ev = rel_err(out[recv], ref), rel_err(g[e], refv)
    print("c2a", f"out {eo:.2e} dvec {ev:.2e}")
    assert eo <= TOL and ev <= TOL


def test_empty_masks_give_zero_messages():
    wl = workloads.generate("c1s")
    dev = _mask_device(wl, np.zeros(wl.n_edges, dtype=np.uint32))
    out = dev.forward().cpu().numpy()
    g = dev.backward()
    assert np.abs(out).max() == 0.0
    for k in ("vec", "x", "W2"):
        assert float(g[k].abs().max()) == 0.0, k


@pytest.mark.parametrize("L,C,H", [(2, 48, 64), (3, 64, 64), (3, 32, 16), (1, 80, 64)])
def test_small_full_parity_channel_counts(L, C, H):
    """Channel counts other than 128 (3, 4, 2 and 5 channel slices) and the width-16 MLP at
    l = 3, on a 48-node graph with 40 edges per sender (several tiles, ragged tails)."""
    spec = dict(kind="random_out", n_nodes=48, box=20.0, k=40, L=L, C=C, n_radial=8,
                r_cut=35.0, hidden=H)
    wl = workloads.generate("c1s", seed=L * 100 + C, spec=spec)
    dev = Device(wl)
    out = dev.forward().cpu().numpy()
    grads = {k: v.cpu().numpy() for k, v in dev.backward().items()}
    pb = problem(wl)
    ref = conv.forward(pb)
    refg = conv.backward(pb)
    errs = {"out": rel_err(out, ref), "vec": rel_err(grads["vec"], refg["dvec"]),
            "x": rel_err(grads["x"], refg["dx"]), "W1": rel_err(grads["W1"], refg["dW1"]),
            "W2": rel_err(grads["W2"], refg["dW2"])}
    print(f"L={L} C={C} H={H}", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (L, C, H, k, v)


def test_path_subsets_channel_count_64():
    spec = dict(kind="random_out", n_nodes=48, box=20.0, k=40, L=3, C=64, n_radial=8,
                r_cut=35.0, hidden=64, adaptive=True)
    wl = workloads.generate("c2as", seed=5, spec=spec)
    dev = _mask_device(wl, wl.path_mask)
    out = dev.forward().cpu().numpy()
    grads = {k: v.cpu().numpy() for k, v in dev.backward().items()}
    pb = problem(wl)
    ref = conv.forward(pb)
    refg = conv.backward(pb)
    errs = {"out": rel_err(out, ref), "vec": rel_err(grads["vec"], refg["dvec"]),
            "x": rel_err(grads["x"], refg["dx"]), "W2": rel_err(grads["W2"], refg["dW2"])}
    print("masked C=64", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (k, v)
