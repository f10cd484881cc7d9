"""GPU parity of the node-local product ladder: the HIP library (through its C ABI) against the
fp64 oracle (oracle/ladder.py), element by element.

Small cases cover every lmax (0..3), correlation order (2..5) and channel width class (16, 32,
48, 64, 128: one, two or four nodes per wave and several channel groups) with node counts that
leave partly filled waves.  At the benchmark size (4096 nodes, 128 channels, lmax 3, nu 5) the
forward and dL/dA are checked on sampled nodes (both are node-local, so the oracle computes them
exactly on the sample), and dL/dw, a sum over all nodes, with an upstream gradient that is zero
outside the sampled nodes (so the oracle's sum over the sample is the whole sum), plus the
linearity of dL/dw in the upstream gradient at full size.  Tolerance as for the convolution:
max relative error 1e-4 per output tensor (gpu_harness.rel_err)."""
import numpy as np
import pytest

import tensor_product_gnn_amd as tp
from gpu_harness import TOL, rel_err
from oracle import ladder
from tensor_product_gnn_amd import workloads

pytestmark = pytest.mark.gpu


def _dev(*arrays):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrays]


def _check_small(n, L, C, nu, seed):
    wl = workloads.generate_ladder(spec=dict(n_nodes=n, L=L, C=C, nu=nu), seed=seed)
    A, w, G = _dev(wl.A, wl.w, wl.G)
    out = tp.ladder_forward(A, w, L, nu).cpu().numpy()
    g = tp.ladder_backward(A, w, G, L, nu)
    ref = ladder.forward(wl.A, wl.w, L, nu)
    dA, dw = ladder.backward(wl.A, wl.w, wl.G, L, nu)
    errs = {"out": rel_err(out, ref), "A": rel_err(g["A"].cpu().numpy(), dA),
            "w": rel_err(g["w"].cpu().numpy(), dw)}
    print(f"ladder n={n} L={L} C={C} nu={nu}", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (k, v)


@pytest.mark.parametrize("L", [0, 1, 2, 3])
@pytest.mark.parametrize("nu", [2, 3, 4, 5])
def test_small_full_parity_every_order(L, nu):
    _check_small(n=37, L=L, C=64, nu=nu, seed=10 * L + nu)


@pytest.mark.parametrize("C,n", [(16, 13), (32, 7), (48, 9), (128, 37)])
def test_small_full_parity_channel_widths(C, n):
    _check_small(n=n, L=3, C=C, nu=5, seed=C)


def test_gradient_subsets_and_determinism():
    wl = workloads.generate_ladder("ladder_s", seed=3)
    L, nu = wl.L, wl.nu
    A, w, G = _dev(wl.A, wl.w, wl.G)
    full = tp.ladder_backward(A, w, G, L, nu)
    again = tp.ladder_backward(A, w, G, L, nu)
    only_A = tp.ladder_backward(A, w, G, L, nu, want_w=False)
    only_w = tp.ladder_backward(A, w, G, L, nu, want_A=False)
    assert set(only_A) == {"A"} and set(only_w) == {"w"}
    for k in ("A", "w"):
        assert bool((full[k] == again[k]).all()), k            # bitwise reproducible
    assert bool((only_A["A"] == full["A"]).all())
    assert bool((only_w["w"] == full["w"]).all())
    o1 = tp.ladder_forward(A, w, L, nu)
    o2 = tp.ladder_forward(A, w, L, nu)
    assert bool((o1 == o2).all())


def test_no_nodes_zeroes_dw():
    import torch
    L, nu, C = 2, 3, 32
    P = tp.ladder_num_paths(L)
    A = torch.zeros((0, (L + 1) ** 2, C), device="cuda")
    w = torch.randn((nu - 1, P, C), device="cuda")
    G = torch.zeros_like(A)
    dw = torch.full_like(w, 7.0)
    res = tp.ladder_backward(A, w, G, L, nu, outs={"w": dw})
    torch.cuda.synchronize()
    assert float(res["w"].abs().max()) == 0.0
    assert tp.ladder_forward(A, w, L, nu).shape == A.shape


def test_benchmark_size_sampled():
    wl = workloads.generate_ladder("ladder")
    L, nu = wl.L, wl.nu
    A, w, G = _dev(wl.A, wl.w, wl.G)
    rng = np.random.default_rng(5)
    S = np.sort(rng.choice(wl.n_nodes, size=24, replace=False))
    out = tp.ladder_forward(A, w, L, nu).cpu().numpy()
    g = tp.ladder_backward(A, w, G, L, nu)
    ref = ladder.forward(wl.A[S], wl.w, L, nu)
    dA_ref, _ = ladder.backward(wl.A[S], wl.w, wl.G[S], L, nu)
    e_out = rel_err(out[S], ref)
    e_dA = rel_err(g["A"].cpu().numpy()[S], dA_ref)
    # dL/dw with the upstream gradient restricted to the sample
    Gm = np.zeros_like(wl.G)
    Gm[S] = wl.G[S]
    (Gm_d,) = _dev(Gm)
    gm = tp.ladder_backward(A, w, Gm_d, L, nu)
    dA_m, dw_m = ladder.backward(wl.A[S], wl.w, wl.G[S], L, nu)
    e_dw = rel_err(gm["w"].cpu().numpy(), dw_m)
    dA_gm = gm["A"].cpu().numpy()
    rest = np.setdiff1d(np.arange(wl.n_nodes), S)
    assert float(np.abs(dA_gm[rest]).max()) == 0.0       # no upstream gradient, no dL/dA
    # linearity in the upstream gradient at full size: dw(G) = dw(G on S) + dw(G off S)
    (Gc_d,) = _dev(wl.G - Gm)
    gc = tp.ladder_backward(A, w, Gc_d, L, nu)
    e_lin = rel_err(g["w"].cpu().numpy(), gm["w"].cpu().numpy() + gc["w"].cpu().numpy())
    print(f"ladder full size: out {e_out:.2e} dA {e_dA:.2e} dw(sample) {e_dw:.2e} linearity {e_lin:.2e}")
    assert e_out <= TOL and e_dA <= TOL and e_dw <= TOL and e_lin <= TOL


@pytest.mark.parametrize("L,nu,C,n", [(3, 5, 128, 37), (2, 3, 32, 11), (3, 2, 64, 5)])
def test_saved_rungs_match_recompute(L, nu, C, n):
    """The backward reading the rungs the forward kept equals the oracle (and the recomputing
    backward); the rungs themselves equal the oracle's B_2 .. B_{nu-1}."""
    wl = workloads.generate_ladder(spec=dict(n_nodes=n, L=L, C=C, nu=nu), seed=77)
    A, w, G = _dev(wl.A, wl.w, wl.G)
    rungs = tp.ladder_rungs(A, nu)
    out = tp.ladder_forward(A, w, L, nu, rungs=rungs).cpu().numpy()
    g = tp.ladder_backward(A, w, G, L, nu, rungs=rungs)
    g0 = tp.ladder_backward(A, w, G, L, nu)
    lv = ladder.levels(wl.A, wl.w, L, nu)
    dA, dw = ladder.backward(wl.A, wl.w, wl.G, L, nu)
    errs = {"out": rel_err(out, ladder.forward(wl.A, wl.w, L, nu)),
            "A": rel_err(g["A"].cpu().numpy(), dA), "w": rel_err(g["w"].cpu().numpy(), dw),
            "A vs recompute": rel_err(g["A"].cpu().numpy(), g0["A"].cpu().numpy().astype(np.float64)),
            "w vs recompute": rel_err(g["w"].cpu().numpy(), g0["w"].cpu().numpy().astype(np.float64))}
    for q in range(nu - 2):
        errs[f"B{q + 2}"] = rel_err(rungs[q].cpu().numpy(), lv[q + 1])
    print(f"rungs L={L} nu={nu} C={C} n={n}", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (k, v)
