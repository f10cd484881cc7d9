"""GPU parity of the edge convolution with mixed per-l multiplicities (equitp_mixed_*): the HIP
library through its C ABI against the fp64 oracle (oracle/mixed.py), element by element.

Small graphs carry the NequIP large-model multiplicities (128, 64, 32, 32 for l = 0..3, three
channel slices and 11 masked launches), the medium and small ones (128, 64, 32 and 128, 64 on
l <= 2 and l <= 1 graphs) and input and output multiplicities that differ; forward and every
gradient compared in full.  Uniform multiplicities with identity maps are compared with the
uniform convolution.  At the benchmark size (1024 nodes x 128 edges) the forward and dL/dvec are
checked on the edges into sampled receivers (the oracle computes them exactly there) and the
weight gradients and dL/dx with an upstream gradient that is zero outside the sample.  Tolerance:
max relative error 1e-4 per output tensor (gpu_harness.rel_err)."""
import numpy as np
import pytest

import tensor_product_gnn_amd as tp
from gpu_harness import TOL, rel_err
from oracle import mixed
from tensor_product_gnn_amd import workloads

pytestmark = pytest.mark.gpu


def _dev(*arrays):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrays]


def _setup(wl):
    g0 = wl.graph
    conv = tp.MixedConv(wl.irreps(wl.mult_in), wl.irreps(wl.mult_out), n_radial=8, hidden=64,
                        r_cut=g0.spec["r_cut"])
    g = tp.Graph.from_arrays(g0.x.shape[0], g0.row_ptr, g0.src, g0.dst)
    vec, x, W1, W2, Wlin, G = _dev(g0.vec, wl.x, g0.W1, wl.W2, wl.Wlin, wl.G)
    return conv, g, vec, x, W1, W2, Wlin, G


def _check_full(wl):
    conv, g, vec, x, W1, W2, Wlin, G = _setup(wl)
    out = conv.forward(g, vec, x, W1, W2, Wlin).cpu().numpy()
    gr = conv.backward(g, vec, x, W1, W2, Wlin, G)
    pb = mixed.Problem.from_workload(wl)
    ref = mixed.forward(pb)
    rg = mixed.backward(pb)
    errs = {"out": rel_err(out, ref), "vec": rel_err(gr["vec"].cpu().numpy(), rg["dvec"]),
            "x": rel_err(gr["x"].cpu().numpy(), rg["dx"]),
            "W1": rel_err(gr["W1"].cpu().numpy(), rg["dW1"]),
            "W2": rel_err(gr["W2"].cpu().numpy(), rg["dW2"]),
            "Wlin": rel_err(gr["Wlin"].cpu().numpy(), np.concatenate([w.ravel() for w in rg["dWlin"]]))}
    print(f"mixed {wl.name} in={wl.mult_in} out={wl.mult_out}",
          {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= TOL, (k, v)


def test_nequip_large_multiplicities_small_graph():
    _check_full(workloads.generate_mixed("c2ms"))


@pytest.mark.parametrize("graph,mult_in,mult_out", [
    ("c1s", [128, 64, 32], [128, 64, 32]),          # NequIP medium (l <= 2)
    ("c0h", [128, 64], [128, 64]),                  # NequIP small (l <= 1)
    ("c2s", [64, 128, 32, 64], [32, 64, 128, 32]),  # input and output multiplicities differ
    ("c2s", [32, 32, 32, 32], [64, 32, 32, 128]),   # one slice, mixed outputs
])
def test_other_multiplicities(graph, mult_in, mult_out):
    spec = dict(graph=graph, mult_in=mult_in, mult_out=mult_out)
    if graph == "c0h":   # the 64-node l <= 1 graph with the radial MLP width these kernels take
        spec.update(graph="c0", graph_spec=dict(workloads.SPECS["c0"], hidden=64))
    _check_full(workloads.generate_mixed(spec=spec, seed=3))


def test_uniform_with_identity_maps_is_the_uniform_convolution():
    import torch
    wl = workloads.generate_mixed(spec=dict(graph="c2s", mult_in=[64] * 4, mult_out=[64] * 4), seed=4)
    conv, g, vec, x, W1, W2, Wlin, G = _setup(wl)
    Wl = torch.cat([torch.eye(64, device="cuda").ravel() for _ in range(23)])
    out = conv.forward(g, vec, x, W1, W2, Wl)
    u = tp.Conv(wl.irreps([64] * 4), "0e+1o+2e+3o", wl.irreps([64] * 4), n_radial=8, hidden=64,
                r_cut=wl.graph.spec["r_cut"])
    ref = u.forward(g, vec, x.view(-1, 16, 64), W1, W2).reshape(out.shape)
    e = rel_err(out.cpu().numpy(), ref.cpu().numpy().astype(np.float64))
    print(f"uniform via mixed vs uniform kernel: {e:.2e}")
    assert e <= TOL


def test_gradient_subsets_and_determinism():
    wl = workloads.generate_mixed("c2ms", seed=5)
    conv, g, vec, x, W1, W2, Wlin, G = _setup(wl)
    full = conv.backward(g, vec, x, W1, W2, Wlin, G)
    again = conv.backward(g, vec, x, W1, W2, Wlin, G)
    for k in full:
        assert bool((full[k] == again[k]).all()), k
    for want in (("vec",), ("x",), ("W1", "W2"), ("Wlin",)):
        part = conv.backward(g, vec, x, W1, W2, Wlin, G, want=want)
        assert set(part) == set(want)
        for k in want:
            assert bool((part[k] == full[k]).all()), k
    o1 = conv.forward(g, vec, x, W1, W2, Wlin)
    o2 = conv.forward(g, vec, x, W1, W2, Wlin)
    assert bool((o1 == o2).all())


def test_kept_path_outputs_match_recompute():
    """A backward reading the path outputs the forward kept equals the recomputing one bitwise."""
    wl = workloads.generate_mixed("c2ms", seed=8)
    conv, g, vec, x, W1, W2, Wlin, G = _setup(wl)
    saved = conv.saved_tensor(wl.graph.x.shape[0])
    o1 = conv.forward(g, vec, x, W1, W2, Wlin, saved=saved)
    o2 = conv.forward(g, vec, x, W1, W2, Wlin)
    assert bool((o1 == o2).all())
    a = conv.backward(g, vec, x, W1, W2, Wlin, G, saved=saved)
    b = conv.backward(g, vec, x, W1, W2, Wlin, G)
    for k in a:
        assert bool((a[k] == b[k]).all()), k


def test_no_edges():
    import torch
    wl = workloads.generate_mixed("c2ms", seed=6)
    conv, _, vec, x, W1, W2, Wlin, G = _setup(wl)
    n = wl.graph.x.shape[0]
    g = tp.Graph.from_arrays(n, np.zeros(n + 1, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32))
    out = conv.forward(g, vec[:0], x, W1, W2, Wlin)
    gr = conv.backward(g, vec[:0], x, W1, W2, Wlin, G)
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0
    for k in ("x", "W1", "W2", "Wlin"):
        assert float(gr[k].abs().max()) == 0.0, k


def test_benchmark_size_sampled():
    wl = workloads.generate_mixed("c2m")
    g0 = wl.graph
    conv, g, vec, x, W1, W2, Wlin, G = _setup(wl)
    n = g0.x.shape[0]
    rng = np.random.default_rng(7)
    S = np.sort(rng.choice(n, size=4, replace=False))
    edges = np.concatenate([np.arange(g0.row_ptr[d], g0.row_ptr[d + 1]) for d in S])
    pb = mixed.Problem.from_workload(wl)
    out = conv.forward(g, vec, x, W1, W2, Wlin).cpu().numpy()
    ref = mixed.forward(pb, edges=edges)
    offs, _ = mixed.block_offsets(wl.mult_out)
    e_out = rel_err(out[S], ref[S])
    Gm = np.zeros_like(wl.G)
    Gm[S] = wl.G[S]
    (Gm_d,) = _dev(Gm)
    gr = conv.backward(g, vec, x, W1, W2, Wlin, Gm_d)
    rg = mixed.backward(pb, G=Gm, edges=edges)
    errs = {"out": e_out, "vec": rel_err(gr["vec"].cpu().numpy()[edges], rg["dvec"][edges]),
            "x": rel_err(gr["x"].cpu().numpy(), rg["dx"]),
            "W1": rel_err(gr["W1"].cpu().numpy(), rg["dW1"]),
            "W2": rel_err(gr["W2"].cpu().numpy(), rg["dW2"]),
            "Wlin": rel_err(gr["Wlin"].cpu().numpy(), np.concatenate([w.ravel() for w in rg["dWlin"]]))}
    rest = np.setdiff1d(np.arange(len(g0.src)), edges)
    assert float(np.abs(gr["vec"].cpu().numpy()[rest]).max()) == 0.0
    print("mixed c2m sampled", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= TOL, (k, v)
