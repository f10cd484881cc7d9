"""Shared pieces of the GPU parity tests: device copies of a workload, library calls through the
C ABI (via the ctypes binding), fp64 oracle references and the parity metric."""
from __future__ import annotations

import numpy as np

import tensor_product_gnn_amd as tp
from oracle import conv
from tensor_product_gnn_amd import workloads

TOL = 1e-4  # max relative error against the fp64 oracle (fp32 path)
# With bf16 operands for the radial-MLP contractions the oracle rounds the same operands, but it
# rounds its fp64 values where the library rounds fp32 ones: an operand within fp32 rounding of a
# bf16 rounding boundary goes one bf16 ulp (2^-8 relative) the other way.  Perturbing the oracle's
# operands by fp32-sized relative noise (3e-7) before the rounding moves its results, on the small
# l <= 3 workload, by up to 6.9e-4 (out), 6.3e-4 (dL/dvec), 7.3e-4 (dL/dW1) and 1.9e-3 (dL/dW2,
# a sum over all edges) in the metric below; the bound keeps a factor above 2.5 over those.  (The
# bf16 operands themselves move the results by about 1.5e-2 from the unrounded fp64 values.)
TOL_BF16 = 5e-3


def rel_err(got, ref) -> float:
    """max_i |g_i - r_i| / max(|r_i|, rms(r)) over one output tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), rms)))


class Device:
    """A workload on the GPU plus the library handle for it."""

    def __init__(self, wl: workloads.Workload, sender_csr: bool = True, mlp_bf16: bool = False):
        import torch
        self.wl = wl
        s = wl.spec
        self.conv = tp.Conv(wl.irreps(), wl.irreps_sh(), wl.irreps(), n_radial=s["n_radial"],
                            hidden=s["hidden"], r_cut=s["r_cut"], mlp_bf16=mlp_bf16)
        self.g = tp.Graph.from_arrays(wl.n_nodes, wl.row_ptr, wl.src, wl.dst, sender_csr=sender_csr)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.vec, self.x, self.W1, self.W2, self.G = t(wl.vec), t(wl.x), t(wl.W1), t(wl.W2), t(wl.G)
        self.W_lin = t(np.stack(wl.W_lin)) if wl.W_lin is not None else None

    def forward(self):
        return self.conv.forward(self.g, self.vec, self.x, self.W1, self.W2)

    def backward(self, G=None, want_x=True, want_W=True):
        return self.conv.backward(self.g, self.vec, self.x, self.W1, self.W2,
                                  self.G if G is None else G, want_vec=True, want_x=want_x,
                                  want_W1=want_W, want_W2=want_W)


def problem(wl, mlp_bf16=False):
    return conv.Problem.from_workload(wl, mlp_bf16=mlp_bf16)


def receiver_edges(wl, receivers):
    return np.concatenate([np.arange(wl.row_ptr[d], wl.row_ptr[d + 1]) for d in receivers])


def sample_receivers(wl, k, seed=0):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(wl.n_nodes, size=min(k, wl.n_nodes), replace=False))


def sample_edges(wl, k, seed=0):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(wl.n_edges, size=min(k, wl.n_edges), replace=False))
