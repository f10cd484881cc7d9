"""tensor_product_gnn_amd — Python binding of libequitp, the E(3)-equivariant edge convolution for
MI355X (gfx950).

This module only marshals arguments: torch tensors provide device memory and the current HIP
stream, and every step of the computation runs in the library's HIP kernels (include/equitp.h
documents the operation, layouts and error behaviour).  If libequitp.so is missing the calls
raise; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libequitp.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "equitp.h")

STATUS = {0: "EQUITP_OK", -1: "EQUITP_INVALID_ARG", -2: "EQUITP_IRREPS_PARSE",
          -3: "EQUITP_UNSUPPORTED", -4: "EQUITP_HIP_ERROR", -5: "EQUITP_WORKSPACE_TOO_SMALL"}

_lib = None


class EquiTPError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}")


class GraphStruct(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_int32), ("n_edges", ctypes.c_int32),
                ("row_ptr", ctypes.c_void_p), ("src", ctypes.c_void_p), ("dst", ctypes.c_void_p),
                ("t_row_ptr", ctypes.c_void_p), ("t_perm", ctypes.c_void_p),
                ("path_mask", ctypes.c_void_p)]


def lib() -> ctypes.CDLL:
    """The loaded libequitp.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() or "
                           "python tensor_product_gnn_amd/csrc/build.py")
    # torch ships its own HIP runtime; it has to be in the process before the library resolves
    # libamdhip64, or the library binds to a second runtime and fails on torch's device memory
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    ip = ctypes.POINTER(ctypes.c_int)
    L.equitp_create.argtypes = [ctypes.c_char_p, ctypes.c_char_p, ctypes.c_char_p, i32, ctypes.POINTER(vp)]
    L.equitp_set_radial.argtypes = [vp, i32, f32]
    L.equitp_set_mlp_precision.argtypes = [vp, i32]
    L.equitp_query.argtypes = [vp, ip, ip, ip, ip, ip, ip, ip]
    L.equitp_path.argtypes = [vp, i32, ip, ip, ip]
    L.equitp_forward.argtypes = [vp, ctypes.POINTER(GraphStruct), vp, vp, vp, vp, vp, vp]
    L.equitp_backward_workspace.argtypes = [vp, i32, i32, ctypes.POINTER(sz)]
    L.equitp_backward.argtypes = [vp, ctypes.POINTER(GraphStruct), vp, vp, vp, vp, vp, vp, vp, vp,
                                  vp, vp, sz, vp]
    L.equitp_linear.argtypes = [i32, i32, i32, vp, vp, i32, vp, vp]
    L.equitp_build_csr_workspace.argtypes = [i32, i32, ctypes.POINTER(sz)]
    L.equitp_build_csr.argtypes = [i32, i32, vp, vp, vp, vp, sz, vp]
    L.equitp_cg_block.argtypes = [i32, i32, i32, ctypes.POINTER(ctypes.c_float)]
    L.equitp_ladder_num_paths.argtypes = [i32, ip]
    L.equitp_ladder_forward.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
    L.equitp_ladder_backward_workspace.argtypes = [i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.equitp_ladder_backward.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.equitp_full_ladder_workspace.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.equitp_mixed_create.argtypes = [ctypes.c_char_p, ctypes.c_char_p, i32, i32, f32, ctypes.POINTER(vp)]
    L.equitp_mixed_query.argtypes = [vp, ip, ip, ip, ip, ip, ip, ip]
    L.equitp_mixed_workspace.argtypes = [vp, i32, i32, i32, ctypes.POINTER(sz)]
    L.equitp_mixed_saved_floats.argtypes = [vp, i32, ctypes.POINTER(sz)]
    L.equitp_mixed_forward.argtypes = [vp, ctypes.POINTER(GraphStruct), vp, vp, vp, vp, vp, vp, vp, vp,
                                       sz, vp]
    L.equitp_mixed_backward.argtypes = [vp, ctypes.POINTER(GraphStruct), vp, vp, vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp, vp, vp, sz, vp]
    L.equitp_mixed_destroy.argtypes = [vp]
    L.equitp_full_ladder_saved_floats.argtypes = [i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.equitp_full_ladder_forward.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.equitp_full_ladder_backward.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.equitp_destroy.argtypes = [vp]
    L.equitp_destroy.restype = None
    L.equitp_status_string.argtypes = [i32]
    L.equitp_status_string.restype = ctypes.c_char_p
    L.equitp_profile_enable.argtypes = [i32]
    L.equitp_profile_only.argtypes = [ctypes.c_char_p]
    L.equitp_profile_get.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p), ip, ctypes.POINTER(ctypes.c_double)]
    for name in ("equitp_profile_enable", "equitp_profile_only", "equitp_profile_reset", "equitp_profile_count",
                 "equitp_profile_get", "equitp_create", "equitp_set_radial", "equitp_set_mlp_precision",
                 "equitp_query", "equitp_path",
                 "equitp_forward", "equitp_backward_workspace", "equitp_backward", "equitp_linear",
                 "equitp_build_csr_workspace", "equitp_build_csr", "equitp_cg_block",
                 "equitp_ladder_num_paths", "equitp_ladder_forward",
                 "equitp_ladder_backward_workspace", "equitp_ladder_backward"):
        getattr(L, name).restype = i32
    _lib = L
    return L


def header_functions() -> list:
    """Names of the functions include/equitp.h declares."""
    txt = open(HEADER_PATH).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(equitp_\w+)\s*\(", txt)))


def _check(status: int, what: str) -> None:
    if status != 0:
        raise EquiTPError(status, what)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    if stream is not None:
        return int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, name, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor on the GPU")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    return t


class Graph:
    """Device-resident edge list sorted by receiver, plus the sender CSR for input gradients."""

    def __init__(self, n_nodes: int, row_ptr, src, dst, t_row_ptr=None, t_perm=None,
                 path_mask=None):
        import torch
        self.n_nodes = int(n_nodes)
        self.row_ptr = _need(row_ptr, torch.int32, "row_ptr", 1)
        self.src = _need(src, torch.int32, "src", 1)
        self.dst = _need(dst, torch.int32, "dst", 1)
        self.n_edges = int(self.src.numel())
        if self.row_ptr.numel() != self.n_nodes + 1 or self.dst.numel() != self.n_edges:
            raise ValueError("graph arrays have inconsistent sizes")
        self.t_row_ptr = t_row_ptr
        self.t_perm = t_perm
        # per-edge path bitmask (int32 storage of the uint32 bits), or None
        self.path_mask = None if path_mask is None else _need(path_mask, torch.int32, "path_mask", 1)
        if self.path_mask is not None and self.path_mask.numel() != self.n_edges:
            raise ValueError("path_mask must have one entry per edge")
        self._sync()

    def _sync(self):
        self.struct = GraphStruct(self.n_nodes, self.n_edges, _ptr(self.row_ptr), _ptr(self.src),
                                  _ptr(self.dst), _ptr(self.t_row_ptr), _ptr(self.t_perm),
                                  _ptr(self.path_mask))

    @classmethod
    def from_arrays(cls, n_nodes, row_ptr, src, dst, device="cuda", sender_csr=True,
                    path_mask=None):
        """Copy host arrays (numpy) to the device; build the sender CSR with the library.
        path_mask: optional per-edge uint32 path bitmask."""
        import numpy as np
        import torch
        t = lambda a: torch.as_tensor(a, dtype=torch.int32).to(device).contiguous()
        pm = None
        if path_mask is not None:
            pm = torch.from_numpy(np.ascontiguousarray(np.asarray(path_mask, dtype=np.uint32)
                                                       .view(np.int32))).to(device)
        g = cls(n_nodes, t(row_ptr), t(src), t(dst), path_mask=pm)
        if sender_csr:
            g.t_row_ptr, g.t_perm = build_csr(g.src, n_nodes)
            g._sync()
        return g


def build_csr(key, n_nodes: int, stream=None):
    """(row_ptr [n_nodes + 1], perm [n]) grouping positions by key (stable)."""
    import torch
    key = _need(key, torch.int32, "key", 1)
    n = int(key.numel())
    nbytes = ctypes.c_size_t(0)
    _check(lib().equitp_build_csr_workspace(n_nodes, n, ctypes.byref(nbytes)), "build_csr_workspace")
    ws = torch.empty(max(1, nbytes.value), dtype=torch.uint8, device=key.device)
    row_ptr = torch.empty(n_nodes + 1, dtype=torch.int32, device=key.device)
    perm = torch.empty(max(1, n), dtype=torch.int32, device=key.device)
    _check(lib().equitp_build_csr(n_nodes, n, _ptr(key), _ptr(row_ptr), _ptr(perm), _ptr(ws),
                                  nbytes.value, _stream(stream)), "build_csr")
    return row_ptr, perm[:n]


class Conv:
    """One equivariant edge convolution (see include/equitp.h for the definition)."""

    def __init__(self, irreps_in: str, irreps_sh: str, irreps_out: str, n_radial: int = 8,
                 hidden: int = 64, r_cut: float = 5.0, mlp_bf16: bool = False):
        """mlp_bf16: bf16 operands (fp32 accumulation) for the radial-MLP W2 contractions."""
        h = ctypes.c_void_p()
        _check(lib().equitp_create(irreps_in.encode(), irreps_sh.encode(), irreps_out.encode(),
                                   n_radial, ctypes.byref(h)), "create")
        self._h = h
        _check(lib().equitp_set_radial(h, hidden, float(r_cut)), "set_radial")
        if mlp_bf16:
            _check(lib().equitp_set_mlp_precision(h, 1), "set_mlp_precision")
        self.mlp_bf16 = bool(mlp_bf16)
        vals = [ctypes.c_int() for _ in range(7)]
        _check(lib().equitp_query(h, *[ctypes.byref(v) for v in vals]), "query")
        (self.n_paths, self.channels, self.f_in, self.f_sh, self.f_out, self.w1_numel,
         self.w2_numel) = [v.value for v in vals]
        self.n_radial, self.hidden, self.r_cut = n_radial, hidden, float(r_cut)

    def __del__(self):
        if getattr(self, "_h", None) is not None and _lib is not None:
            _lib.equitp_destroy(self._h)
            self._h = None

    def paths(self):
        out = []
        for p in range(self.n_paths):
            a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
            _check(lib().equitp_path(self._h, p, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), "path")
            out.append((a.value, b.value, c.value))
        return out

    def forward(self, g: Graph, vec, x, W1, W2, out=None, stream=None):
        import torch
        _need(vec, torch.float32, "vec")
        _need(x, torch.float32, "x")
        _need(W1, torch.float32, "W1")
        _need(W2, torch.float32, "W2")
        if out is None:
            out = torch.empty((g.n_nodes, self.f_out, self.channels), dtype=torch.float32, device=x.device)
        _need(out, torch.float32, "out")
        _check(lib().equitp_forward(self._h, ctypes.byref(g.struct), _ptr(vec), _ptr(x), _ptr(W1),
                                    _ptr(W2), _ptr(out), _stream(stream)), "forward")
        return out

    def workspace_bytes(self, n_nodes: int, n_edges: int) -> int:
        b = ctypes.c_size_t(0)
        _check(lib().equitp_backward_workspace(self._h, n_nodes, n_edges, ctypes.byref(b)), "workspace")
        return b.value

    def backward(self, g: Graph, vec, x, W1, W2, grad_out, want_vec=True, want_x=False,
                 want_W1=True, want_W2=True, workspace=None, outs: Optional[dict] = None,
                 stream=None):
        """Returns a dict with the requested gradients (vec, x, W1, W2); only those whose want_*
        flag is set are computed, into the tensors given in `outs` or newly allocated ones."""
        import torch
        _need(grad_out, torch.float32, "grad_out")
        dev = x.device
        outs = dict(outs or {})
        if want_vec and "vec" not in outs:
            outs["vec"] = torch.empty((g.n_edges, 3), dtype=torch.float32, device=dev)
        if want_x and "x" not in outs:
            outs["x"] = torch.empty((g.n_nodes, self.f_in, self.channels), dtype=torch.float32, device=dev)
        if want_W1 and "W1" not in outs:
            outs["W1"] = torch.empty_like(W1)
        if want_W2 and "W2" not in outs:
            outs["W2"] = torch.empty_like(W2)
        nbytes = self.workspace_bytes(g.n_nodes, g.n_edges)
        if workspace is None:
            workspace = torch.empty(max(256, nbytes), dtype=torch.uint8, device=dev)
        want = {"vec": want_vec, "x": want_x, "W1": want_W1, "W2": want_W2}
        outs = {k: v for k, v in outs.items() if want.get(k, False)}
        _check(lib().equitp_backward(self._h, ctypes.byref(g.struct), _ptr(vec), _ptr(x), _ptr(W1),
                                     _ptr(W2), _ptr(grad_out), _ptr(outs.get("vec")),
                                     _ptr(outs.get("x")), _ptr(outs.get("W1")), _ptr(outs.get("W2")),
                                     _ptr(workspace), workspace.numel(), _stream(stream)), "backward")
        return outs


class MixedConv:
    """Edge convolution with its own channel count per rotation order (see include/equitp.h,
    equitp_mixed_*): per-path channelwise products, receiver sums kept per path, then a
    channel-mixing linear map per path into the output rank."""

    def __init__(self, irreps_in: str, irreps_out: str, n_radial: int = 8, hidden: int = 64,
                 r_cut: float = 5.0):
        h = ctypes.c_void_p()
        _check(lib().equitp_mixed_create(irreps_in.encode(), irreps_out.encode(), n_radial, hidden,
                                         float(r_cut), ctypes.byref(h)), "mixed_create")
        self._h = h
        vals = [ctypes.c_int() for _ in range(7)]
        _check(lib().equitp_mixed_query(h, *[ctypes.byref(v) for v in vals]), "mixed_query")
        (self.n_paths, self.f_in, self.f_out, self.w2_numel, self.wlin_numel, self.n_slices,
         self.n_launches) = [v.value for v in vals]
        self.n_radial, self.hidden, self.r_cut = n_radial, hidden, float(r_cut)

    def __del__(self):
        if getattr(self, "_h", None) is not None and _lib is not None:
            _lib.equitp_mixed_destroy(self._h)
            self._h = None

    def workspace_bytes(self, n_nodes: int, n_edges: int, backward: bool) -> int:
        b = ctypes.c_size_t(0)
        _check(lib().equitp_mixed_workspace(self._h, n_nodes, n_edges, int(backward), ctypes.byref(b)),
               "mixed_workspace")
        return b.value

    def _ws(self, g, backward, workspace, dev):
        import torch
        n = self.workspace_bytes(g.n_nodes, g.n_edges, backward)
        if workspace is None:
            workspace = torch.empty(max(256, n), dtype=torch.uint8, device=dev)
        return workspace

    def saved_tensor(self, n_nodes: int, device="cuda"):
        """An empty buffer for the path outputs a training forward keeps for its backward."""
        import torch
        n = ctypes.c_size_t(0)
        _check(lib().equitp_mixed_saved_floats(self._h, n_nodes, ctypes.byref(n)), "mixed_saved")
        return torch.empty(max(1, n.value), dtype=torch.float32, device=device)

    def forward(self, g: Graph, vec, x, W1, W2, Wlin, out=None, saved=None, workspace=None,
                stream=None):
        import torch
        for t, nm in ((vec, "vec"), (x, "x"), (W1, "W1"), (W2, "W2"), (Wlin, "Wlin")):
            _need(t, torch.float32, nm)
        if out is None:
            out = torch.empty((g.n_nodes, self.f_out), dtype=torch.float32, device=x.device)
        ws = self._ws(g, False, workspace, x.device)
        _check(lib().equitp_mixed_forward(self._h, ctypes.byref(g.struct), _ptr(vec), _ptr(x), _ptr(W1),
                                          _ptr(W2), _ptr(Wlin), _ptr(out), _ptr(saved), _ptr(ws),
                                          ws.numel(), _stream(stream)), "mixed_forward")
        return out

    def backward(self, g: Graph, vec, x, W1, W2, Wlin, grad_out, want=("vec", "x", "W1", "W2", "Wlin"),
                 workspace=None, outs: Optional[dict] = None, saved=None, stream=None):
        import torch
        _need(grad_out, torch.float32, "grad_out")
        dev = x.device
        outs = dict(outs or {})
        shapes = {"vec": (g.n_edges, 3), "x": tuple(x.shape), "W1": tuple(W1.shape),
                  "W2": tuple(W2.shape), "Wlin": tuple(Wlin.shape)}
        for k in want:
            if k not in outs:
                outs[k] = torch.empty(shapes[k], dtype=torch.float32, device=dev)
        outs = {k: v for k, v in outs.items() if k in want}
        ws = self._ws(g, True, workspace, dev)
        _check(lib().equitp_mixed_backward(self._h, ctypes.byref(g.struct), _ptr(vec), _ptr(x),
                                           _ptr(W1), _ptr(W2), _ptr(Wlin), _ptr(saved), _ptr(grad_out),
                                           _ptr(outs.get("vec")), _ptr(outs.get("x")),
                                           _ptr(outs.get("W1")), _ptr(outs.get("W2")),
                                           _ptr(outs.get("Wlin")), _ptr(ws), ws.numel(),
                                           _stream(stream)), "mixed_backward")
        return outs


def linear(feat, W, lmax: int, transpose: bool = False, out=None, stream=None):
    """Per-irrep channel mixing out[n, l*l+m, :] = feat[n, l*l+m, :] W_l (or W_l^T)."""
    import torch
    _need(feat, torch.float32, "feat", 3)
    _need(W, torch.float32, "W", 3)
    if out is None:
        out = torch.empty_like(feat)
    n, F, C = feat.shape
    if F != (lmax + 1) ** 2 or tuple(W.shape) != (lmax + 1, C, C):
        raise ValueError("shape mismatch")
    _check(lib().equitp_linear(n, lmax, C, _ptr(feat), _ptr(W), int(transpose), _ptr(out),
                               _stream(stream)), "linear")
    return out


def ladder_num_paths(lmax: int) -> int:
    n = ctypes.c_int(0)
    _check(lib().equitp_ladder_num_paths(lmax, ctypes.byref(n)), "ladder_num_paths")
    return n.value


def _ladder_shapes(A, w, lmax: int, nu: int):
    import torch
    _need(A, torch.float32, "A", 3)
    _need(w, torch.float32, "w", 3)
    n, F, C = A.shape
    if F != (lmax + 1) ** 2 or tuple(w.shape) != (nu - 1, ladder_num_paths(lmax), C):
        raise ValueError("shape mismatch")
    return n, C


def ladder_forward(A, w, lmax: int, nu: int, out=None, rungs=None, stream=None):
    """Node-local product ladder: out = B_2 + ... + B_nu with B_1 = A and
    B_s = sum_p w[s-2, p] (B_{s-1} (x)_p A).  A [N, (lmax+1)^2, C], w [nu-1, P, C].
    rungs: optional [nu-2, N, (lmax+1)^2, C] tensor the forward fills with B_2 .. B_{nu-1} for the
    backward (see ladder_rungs)."""
    import torch
    n, C = _ladder_shapes(A, w, lmax, nu)
    if out is None:
        out = torch.empty_like(A)
    if rungs is not None:
        _need(rungs, torch.float32, "rungs", 4)
        if tuple(rungs.shape) != (max(nu - 2, 0), n, (lmax + 1) ** 2, C):
            raise ValueError("rungs shape mismatch")
    _check(lib().equitp_ladder_forward(lmax, nu, n, C, _ptr(A), _ptr(w), _ptr(out), _ptr(rungs),
                                       _stream(stream)), "ladder_forward")
    return out


def ladder_rungs(A, nu: int):
    """An empty rungs tensor for ladder_forward / ladder_backward."""
    import torch
    n, F, C = A.shape
    return torch.empty((max(nu - 2, 0), n, F, C), dtype=torch.float32, device=A.device)


def ladder_workspace_bytes(lmax: int, nu: int, n_nodes: int, channels: int) -> int:
    b = ctypes.c_size_t(0)
    _check(lib().equitp_ladder_backward_workspace(lmax, nu, n_nodes, channels, ctypes.byref(b)),
           "ladder_workspace")
    return b.value


def ladder_backward(A, w, grad_out, lmax: int, nu: int, want_A=True, want_w=True,
                    workspace=None, outs: Optional[dict] = None, rungs=None, stream=None):
    """Returns {"A": dL/dA, "w": dL/dw} (the requested ones) for the loss <grad_out, out>.
    rungs: the tensor a forward filled (optional; without it the rungs are recomputed)."""
    import torch
    n, C = _ladder_shapes(A, w, lmax, nu)
    _need(grad_out, torch.float32, "grad_out", 3)
    outs = dict(outs or {})
    if want_A and "A" not in outs:
        outs["A"] = torch.empty_like(A)
    if want_w and "w" not in outs:
        outs["w"] = torch.empty_like(w)
    outs = {k: v for k, v in outs.items() if {"A": want_A, "w": want_w}.get(k, False)}
    nbytes = ladder_workspace_bytes(lmax, nu, n, C)
    if workspace is None:
        workspace = torch.empty(max(256, nbytes), dtype=torch.uint8, device=A.device)
    if rungs is not None:
        _need(rungs, torch.float32, "rungs", 4)
        if tuple(rungs.shape) != (max(nu - 2, 0), n, (lmax + 1) ** 2, C):
            raise ValueError("rungs shape mismatch")
    _check(lib().equitp_ladder_backward(lmax, nu, n, C, _ptr(A), _ptr(w), _ptr(rungs), _ptr(grad_out),
                                        _ptr(outs.get("A")), _ptr(outs.get("w")), _ptr(workspace),
                                        workspace.numel(), _stream(stream)), "ladder_backward")
    return outs


def _full_ladder_shapes(A, W, lmax: int, nu: int):
    import torch
    _need(A, torch.float32, "A", 3)
    _need(W, torch.float32, "W", 4)
    n, F, C = A.shape
    if F != (lmax + 1) ** 2 or tuple(W.shape) != (nu - 1, ladder_num_paths(lmax), C, C):
        raise ValueError("shape mismatch")
    return n, C


def _check_rungs(rungs, n, lmax, nu, C):
    import torch
    if rungs is not None:
        _need(rungs, torch.float32, "rungs", 4)
        if tuple(rungs.shape) != (max(nu - 2, 0), n, (lmax + 1) ** 2, C):
            raise ValueError("rungs shape mismatch")


def full_ladder_workspace_bytes(lmax: int, nu: int, n_nodes: int, channels: int,
                                backward: bool) -> int:
    b = ctypes.c_size_t(0)
    _check(lib().equitp_full_ladder_workspace(lmax, nu, n_nodes, channels, int(backward),
                                              ctypes.byref(b)), "full_ladder_workspace")
    return b.value


def full_ladder_saved(A, lmax: int, nu: int):
    """An empty buffer for every step's path outputs (full_ladder_forward / _backward `saved`)."""
    import torch
    n_nodes, _, C = A.shape
    n = ctypes.c_size_t(0)
    _check(lib().equitp_full_ladder_saved_floats(lmax, nu, n_nodes, C, ctypes.byref(n)), "full_ladder_saved")
    return torch.empty(max(1, n.value), dtype=torch.float32, device=A.device)


def full_ladder_forward(A, W, lmax: int, nu: int, out=None, rungs=None, saved=None, workspace=None,
                        stream=None):
    """Full product ladder: out = B_2 + ... + B_nu with B_1 = A and
    B_s[l3] = sum_{p -> l3} (B_{s-1} (x)_p A) W[s-2, p] (channel-mixing map per path).
    A [N, (lmax+1)^2, C], W [nu-1, P, C, C]; rungs as for ladder_forward."""
    import torch
    n, C = _full_ladder_shapes(A, W, lmax, nu)
    if out is None:
        out = torch.empty_like(A)
    _check_rungs(rungs, n, lmax, nu, C)
    nbytes = full_ladder_workspace_bytes(lmax, nu, n, C, False)
    if workspace is None:
        workspace = torch.empty(max(256, nbytes), dtype=torch.uint8, device=A.device)
    _check(lib().equitp_full_ladder_forward(lmax, nu, n, C, _ptr(A), _ptr(W), _ptr(out),
                                            _ptr(rungs), _ptr(saved), _ptr(workspace),
                                            workspace.numel(), _stream(stream)), "full_ladder_forward")
    return out


def full_ladder_backward(A, W, grad_out, lmax: int, nu: int, want_A=True, want_W=True,
                         workspace=None, outs: Optional[dict] = None, rungs=None, saved=None,
                         stream=None):
    """Returns {"A": dL/dA, "W": dL/dW} (the requested ones) for the loss <grad_out, out> of
    full_ladder_forward.  rungs: the tensor a forward filled (optional)."""
    import torch
    n, C = _full_ladder_shapes(A, W, lmax, nu)
    _need(grad_out, torch.float32, "grad_out", 3)
    outs = dict(outs or {})
    if want_A and "A" not in outs:
        outs["A"] = torch.empty_like(A)
    if want_W and "W" not in outs:
        outs["W"] = torch.empty_like(W)
    outs = {k: v for k, v in outs.items() if {"A": want_A, "W": want_W}.get(k, False)}
    _check_rungs(rungs, n, lmax, nu, C)
    nbytes = full_ladder_workspace_bytes(lmax, nu, n, C, True)
    if workspace is None:
        workspace = torch.empty(max(256, nbytes), dtype=torch.uint8, device=A.device)
    _check(lib().equitp_full_ladder_backward(lmax, nu, n, C, _ptr(A), _ptr(W), _ptr(rungs),
                                             _ptr(saved), _ptr(grad_out), _ptr(outs.get("A")),
                                             _ptr(outs.get("W")), _ptr(workspace),
                                             workspace.numel(), _stream(stream)),
           "full_ladder_backward")
    return outs


def profile_enable(on: bool = True) -> None:
    _check(lib().equitp_profile_enable(int(on)), "profile_enable")


def profile_only(names=None) -> None:
    """Time only the named units (a list of names, as profile_read reports them); None: all."""
    arg = ",".join(names).encode() if names else None
    _check(lib().equitp_profile_only(arg), "profile_only")


def profile_reset() -> None:
    _check(lib().equitp_profile_reset(), "profile_reset")


def profile_read() -> dict:
    """{kernel name: (launches, total ms)} for launches since the last reset (waits on events)."""
    out = {}
    for i in range(lib().equitp_profile_count()):
        nm, n, ms = ctypes.c_char_p(), ctypes.c_int(), ctypes.c_double()
        _check(lib().equitp_profile_get(i, ctypes.byref(nm), ctypes.byref(n), ctypes.byref(ms)), "profile_get")
        out[nm.value.decode()] = (n.value, ms.value)
    return out


def cg_block(l1: int, l2: int, l3: int):
    """The CG block the kernels use, as a numpy array [2l1+1, 2l2+1, 2l3+1] (host only)."""
    import numpy as np
    d = np.zeros((2 * l1 + 1) * (2 * l2 + 1) * (2 * l3 + 1), dtype=np.float32)
    _check(lib().equitp_cg_block(l1, l2, l3, d.ctypes.data_as(ctypes.POINTER(ctypes.c_float))), "cg_block")
    return d.reshape(2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1)
