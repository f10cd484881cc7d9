"""GPU parity of the full product ladder (per-path channel-mixing maps between the products): the
HIP library (through its C ABI) against the fp64 oracle (oracle/ladder.py, full_forward /
full_backward), element by element.

Small cases cover every lmax (0..3) and correlation order (2..5), every channel count the kernels
take (32, 64, 128), and node counts whose row counts leave ragged GEMM tiles (rows per l3 not a
multiple of 128; several and partial dL/dW row ranges).  At the benchmark size (4096
nodes, 128 channels, lmax 3, nu 5) the forward and dL/dA are checked on sampled nodes (both are
node-local) and dL/dW, a sum over all nodes, with an upstream gradient that is zero outside the
sample, plus its linearity in the upstream gradient at full size.  Tolerance: max relative error
1e-4 per output tensor (gpu_harness.rel_err)."""
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


def _check(n, L, C, nu, seed):
    wl = workloads.generate_full_ladder(spec=dict(n_nodes=n, L=L, C=C, nu=nu), seed=seed)
    A, W, G = _dev(wl.A, wl.W, wl.G)
    out = tp.full_ladder_forward(A, W, L, nu).cpu().numpy()
    g = tp.full_ladder_backward(A, W, G, L, nu)
    ref = ladder.full_forward(wl.A, wl.W, L, nu)
    dA, dW = ladder.full_backward(wl.A, wl.W, wl.G, L, nu)
    errs = {"out": rel_err(out, ref), "A": rel_err(g["A"].cpu().numpy(), dA),
            "W": rel_err(g["W"].cpu().numpy(), dW)}
    print(f"full ladder n={n} L={L} C={C} nu={nu}", {k: f"{v:.2e}" for k, v in errs.items()},
          flush=True)
    for k, v in errs.items():
        assert v <= TOL, (k, v)


@pytest.mark.parametrize("L", [0, 1, 2, 3])
@pytest.mark.parametrize("nu", [2, 3, 4, 5])
def test_small_parity_every_order(L, nu):
    _check(n=37, L=L, C=64, nu=nu, seed=10 * L + nu)


@pytest.mark.parametrize("C,n", [(32, 13), (128, 37), (128, 300)])
def test_small_parity_channels_and_ragged_tiles(C, n):
    _check(n=n, L=3, C=C, nu=5, seed=C + n)


def test_diagonal_maps_equal_the_path_reduced_ladder():
    """Through both C ABIs: W[s][p] = diag(w[s][p]) gives the path-reduced ladder."""
    import torch
    wl = workloads.generate_ladder(spec=dict(n_nodes=53, L=3, C=128, nu=4), seed=8)
    A, w, G = _dev(wl.A, wl.w, wl.G)
    W = torch.diag_embed(w).contiguous()
    out_full = tp.full_ladder_forward(A, W, 3, 4).cpu().numpy()
    out_red = tp.ladder_forward(A, w, 3, 4).cpu().numpy()
    gf = tp.full_ladder_backward(A, W, G, 3, 4)
    gr = tp.ladder_backward(A, w, G, 3, 4)
    diag = torch.diagonal(gf["W"], dim1=-2, dim2=-1).cpu().numpy()
    errs = {"out": rel_err(out_full, out_red.astype(np.float64)),
            "A": rel_err(gf["A"].cpu().numpy(), gr["A"].cpu().numpy().astype(np.float64)),
            "diag W": rel_err(diag, gr["w"].cpu().numpy().astype(np.float64))}
    print("diagonal maps vs path-reduced", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (k, v)


@pytest.mark.parametrize("L,nu,C,n", [(3, 5, 128, 37), (2, 3, 32, 11), (3, 2, 64, 5)])
def test_saved_rungs_match_recompute(L, nu, C, n):
    wl = workloads.generate_full_ladder(spec=dict(n_nodes=n, L=L, C=C, nu=nu), seed=78)
    A, W, G = _dev(wl.A, wl.W, wl.G)
    rungs = tp.ladder_rungs(A, nu)
    out = tp.full_ladder_forward(A, W, L, nu, rungs=rungs).cpu().numpy()
    g = tp.full_ladder_backward(A, W, G, L, nu, rungs=rungs)
    g0 = tp.full_ladder_backward(A, W, G, L, nu)
    lv = ladder.full_levels(wl.A, wl.W, L, nu)
    dA, dW = ladder.full_backward(wl.A, wl.W, wl.G, L, nu)
    errs = {"out": rel_err(out, ladder.full_forward(wl.A, wl.W, L, nu)),
            "A": rel_err(g["A"].cpu().numpy(), dA), "W": rel_err(g["W"].cpu().numpy(), dW)}
    for q in range(nu - 2):
        errs[f"B{q + 2}"] = rel_err(rungs[q].cpu().numpy(), lv[q + 1])
    print(f"full ladder rungs L={L} nu={nu} C={C} n={n}", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    # reading the rungs or recomputing them runs the same kernels on the same values
    assert bool((g["A"] == g0["A"]).all()) and bool((g["W"] == g0["W"]).all())


def test_kept_path_outputs_match_recompute():
    """A backward reading every step's path outputs from the forward equals the recomputing one
    bitwise (the same kernels on the same values), with and without kept rungs."""
    wl = workloads.generate_full_ladder(spec=dict(n_nodes=41, L=3, C=128, nu=5), seed=9)
    A, W, G = _dev(wl.A, wl.W, wl.G)
    saved = tp.full_ladder_saved(A, 3, 5)
    rungs = tp.ladder_rungs(A, 5)
    o1 = tp.full_ladder_forward(A, W, 3, 5, rungs=rungs, saved=saved)
    o2 = tp.full_ladder_forward(A, W, 3, 5)
    assert bool((o1 == o2).all())
    a = tp.full_ladder_backward(A, W, G, 3, 5, rungs=rungs, saved=saved)
    b = tp.full_ladder_backward(A, W, G, 3, 5)
    for k in ("A", "W"):
        assert bool((a[k] == b[k]).all()), k
    dA, dW = ladder.full_backward(wl.A, wl.W, wl.G, 3, 5)
    assert rel_err(a["A"].cpu().numpy(), dA) <= TOL and rel_err(a["W"].cpu().numpy(), dW) <= TOL


def test_gradient_subsets_and_determinism():
    wl = workloads.generate_full_ladder(spec=dict(n_nodes=41, L=3, C=128, nu=4), seed=4)
    L, nu = wl.L, wl.nu
    A, W, G = _dev(wl.A, wl.W, wl.G)
    full = tp.full_ladder_backward(A, W, G, L, nu)
    again = tp.full_ladder_backward(A, W, G, L, nu)
    only_A = tp.full_ladder_backward(A, W, G, L, nu, want_W=False)
    only_W = tp.full_ladder_backward(A, W, G, L, nu, want_A=False)
    assert set(only_A) == {"A"} and set(only_W) == {"W"}
    for k in ("A", "W"):
        assert bool((full[k] == again[k]).all()), k            # bitwise reproducible
    assert bool((only_A["A"] == full["A"]).all())
    assert bool((only_W["W"] == full["W"]).all())
    o1 = tp.full_ladder_forward(A, W, L, nu)
    o2 = tp.full_ladder_forward(A, W, L, nu)
    assert bool((o1 == o2).all())


def test_no_nodes_zeroes_dW():
    import torch
    L, nu, C = 2, 3, 32
    P = tp.ladder_num_paths(L)
    A = torch.zeros((0, (L + 1) ** 2, C), device="cuda")
    W = torch.randn((nu - 1, P, C, C), device="cuda")
    G = torch.zeros_like(A)
    dW = torch.full_like(W, 7.0)
    res = tp.full_ladder_backward(A, W, G, L, nu, outs={"W": dW})
    torch.cuda.synchronize()
    assert float(res["W"].abs().max()) == 0.0
    assert tp.full_ladder_forward(A, W, L, nu).shape == A.shape


def test_benchmark_size_sampled():
    wl = workloads.generate_full_ladder("ladder")
    L, nu = wl.L, wl.nu
    A, W, G = _dev(wl.A, wl.W, wl.G)
    rng = np.random.default_rng(6)
    S = np.sort(rng.choice(wl.n_nodes, size=16, replace=False))
    out = tp.full_ladder_forward(A, W, L, nu).cpu().numpy()
    g = tp.full_ladder_backward(A, W, G, L, nu)
    ref = ladder.full_forward(wl.A[S], wl.W, L, nu)
    dA_ref, dW_ref = ladder.full_backward(wl.A[S], wl.W, wl.G[S], L, nu)
    e_out = rel_err(out[S], ref)
    e_dA = rel_err(g["A"].cpu().numpy()[S], dA_ref)
    Gm = np.zeros_like(wl.G)
    Gm[S] = wl.G[S]
    (Gm_d,) = _dev(Gm)
    gm = tp.full_ladder_backward(A, W, Gm_d, L, nu)
    e_dW = rel_err(gm["W"].cpu().numpy(), dW_ref)
    rest = np.setdiff1d(np.arange(wl.n_nodes), S)
    assert float(np.abs(gm["A"].cpu().numpy()[rest]).max()) == 0.0
    (Gc_d,) = _dev(wl.G - Gm)
    gc = tp.full_ladder_backward(A, W, Gc_d, L, nu)
    e_lin = rel_err(g["W"].cpu().numpy(), gm["W"].cpu().numpy() + gc["W"].cpu().numpy())
    print(f"full ladder full size: out {e_out:.2e} dA {e_dA:.2e} dW(sample) {e_dW:.2e} "
          f"linearity {e_lin:.2e}")
    assert e_out <= TOL and e_dA <= TOL and e_dW <= TOL and e_lin <= TOL
