"""Benchmark of the equivariant edge convolution on one MI355X.

A step is one forward plus one backward (gradients w.r.t. edge vectors and both radial-MLP
weight matrices) of the convolution on one batch of synthetic input already resident in HBM.
Default workload: 1024 nodes x 128 edges/node (131072 edges), 128 channels x (0e+1o+2e+3o),
spherical harmonics to l = 3, 8 Bessel functions, radial MLP width 64, fp32: the edge-convolution
shape of FlashCart Fig. 3(a) at maximum rank 3.

Prints one JSON line: whole-job edges/s, the roofline of the dominant kernel (per-launch durations
from HIP events recorded by the library on the launch stream during the timed steps) and the
fp64 CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "edges/sec fwd+bwd (128 ch, lmax=2/3, fp32) + % of HBM/FP32 roofline"
FP32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 (matrix cores; packed vector issue is the same)
HBM_PEAK_GBS = 8000.0

WORKLOADS = {
    "c2": dict(desc="1024 nodes x 128 random receivers/node (131072 edges), 128x(0e+1o+2e+3o), "
                    "SH lmax 3, 8 Bessel, MLP width 64, r_c 35 A; forward + backward to edge "
                    "vectors, W1 and W2", grads=("vec", "W1", "W2")),
    "c1": dict(desc="1024 nodes x 128 random receivers/node (131072 edges), 128x(0e+1o+2e), SH "
                    "lmax 2, 8 Bessel, MLP width 64, r_c 35 A; forward only", grads=()),
    "c3": dict(desc="5x5x5 diamond cell (1000 atoms, a 3.567 A, noise 0.05 A), 5 A cutoff, "
                    "128x(0e+1o+2e), lmax 2; interaction block: convolution, per-irrep 128x128 "
                    "linear, its data gradient, backward to edge vectors (forces)",
               grads=("vec",), block=True),
    "c4": dict(desc="32768 atoms, random sequential addition at 0.1 /A^3, 6 A cutoff "
                    "(~2.94M edges), 128x(0e+1o+2e+3o), lmax 3; forward + full backward",
               grads=("vec", "x", "W1", "W2")),
    "c2a": dict(desc="c2's graph and features with per-edge adaptive path subsets: each edge keeps "
                     "the paths with spherical-harmonic degree l2 <= its own degree (3 for the "
                     "shortest quarter of the edges down to 0 for the longest; 13.5 of 23 paths on "
                     "average), edges sorted by degree within each receiver; forward + backward to "
                     "edge vectors, W1 and W2", grads=("vec", "W1", "W2")),
    "ladder": dict(desc="node-local product ladder, 4096 nodes, 128x(0e+1o+2e+3o), lmax 3, "
                        "correlation order 5 (four path-reduced products); forward (keeping the rungs) + "
                        "backward to the atomic basis and the path weights", kind="ladder"),
    "c2m": dict(desc="c2's graph (1024 nodes x 128 edges) with the NequIP large-model multiplicities "
                     "128x0e+64x1o+32x2e+32x3o in and out, SH lmax 3, 8 Bessel, MLP width 64: per-path "
                     "products and receiver sums, a channel-mixing map per path; forward + backward "
                     "to edge vectors, W1, W2 and the maps", kind="mixed"),
    "full_ladder": dict(desc="node-local product ladder, full form: the same 4096 nodes, "
                             "128x(0e+1o+2e+3o), lmax 3, correlation order 5, with a 128x128 "
                             "channel-mixing map per step and path (23 paths) in place of the path "
                             "weights; forward (keeping the rungs and path outputs) + backward to "
                             "the atomic basis and the maps", kind="full_ladder"),
}


def ladder_flops(tp, lmax):
    """Algorithmic FLOP of one path-reduced product per (node, channel): per path, one FMA per CG
    entry (the sums over m2), one per (m1, m3) pair with entries (the contraction with the previous
    rung) and one per output component (the path weight)."""
    import numpy as np
    n = 0
    for l1 in range(lmax + 1):
        for l2 in range(lmax + 1):
            for l3 in range(abs(l1 - l2), min(l1 + l2, lmax) + 1):
                if (l1 + l2 + l3) % 2:
                    continue
                nz = tp.cg_block(l1, l2, l3) != 0
                n += int(nz.sum()) + int(nz.any(axis=1).sum()) + (2 * l3 + 1)
    return 2 * n


def path_flops(conv, tp, path_mask=None):
    """Algorithmic FLOP per edge of one forward tensor product and one forward radial MLP.  With
    per-edge path subsets only the paths an edge keeps are counted (averaged over the edges)."""
    import numpy as np
    C = conv.channels
    tp_p, mlp_p = [], []
    for (l1, l2, l3) in conv.paths():
        nnz = int(np.count_nonzero(tp.cg_block(l1, l2, l3)))
        tp_p.append(2 * (C * (min(nnz, (2 * l1 + 1) * (2 * l3 + 1)) + (2 * l3 + 1)) + nnz))
        mlp_p.append(2 * conv.hidden * C)
    share = np.ones(len(tp_p))
    if path_mask is not None:
        bits = (np.asarray(path_mask, dtype=np.int64)[:, None] >> np.arange(len(tp_p))) & 1
        share = bits.mean(axis=0)
    tp_flop = float(np.dot(share, tp_p))
    mlp_flop = 2 * conv.n_radial * conv.hidden + float(np.dot(share, mlp_p))
    return tp_flop, mlp_flop


def cpu_baseline(wl_name, grads, budget_s=25.0):
    """The fp64 oracle on the edges of the first few receivers of the same workload."""
    import numpy as np
    from oracle import conv as oc
    from tensor_product_gnn_amd import workloads
    wl = workloads.generate(wl_name)
    pb = oc.Problem.from_workload(wl)
    threads = 1
    try:
        import threadpoolctl
        threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:
        pass
    n_recv, t_used, n_e = 2, 0.0, 0
    while True:
        edges = np.arange(wl.row_ptr[0], wl.row_ptr[n_recv])
        t0 = time.perf_counter()
        oc.forward(pb, edges=edges)
        if grads:
            oc.backward(pb, edges=edges, want_dx=("x" in grads))
        t_used = time.perf_counter() - t0
        n_e = len(edges)
        if t_used * 2.2 > budget_s or n_recv >= 64:
            break
        n_recv *= 2
    return {"value": n_e / t_used, "unit": "edges/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{wl_name}: the {n_e} edges of receivers 0..{n_recv - 1}, fp64 numpy "
                      f"forward" + (f" + backward ({', '.join(grads)})" if grads else "") +
                      f", {t_used:.1f} s"}


# Source files each profiled unit is compiled from: a recorded HBM traffic figure is used only
# while their code (comments and whitespace left out, so that editing a comment keeps a record)
# hashes to what it hashed to when the counters were taken.
KERNEL_SOURCES = {
    "seg_fwd": ("conv_seg.hip", "common.h", "sh.h", "params.h", "cg_table.h"),
    "seg_dx": ("conv_seg.hip", "common.h", "sh.h", "params.h", "cg_table.h"),
    "bwd": ("conv_bwd.hip", "common.h", "sh.h", "params.h", "cg_table.h"),
    "ladder_fwd": ("ladder.hip", "common.h", "params.h", "cg_table.h"),
    "ladder_bwd": ("ladder.hip", "common.h", "params.h", "cg_table.h"),
    "mix_fwd": ("full_ladder.hip", "full_ladder.h", "common.h", "cg_table.h"),
    "mix_dt": ("full_ladder.hip", "full_ladder.h", "common.h", "cg_table.h"),
    "mix_dw": ("full_ladder.hip", "full_ladder.h", "common.h", "cg_table.h"),
    "full_tp": ("full_ladder.hip", "full_ladder.h", "common.h", "cg_table.h"),
    "full_tp_bwd": ("full_ladder.hip", "full_ladder.h", "common.h", "cg_table.h"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def code_tokens(text):
    """C/C++ source with its comments removed and whitespace runs collapsed (string literals are
    kept as written; the kernel sources hold no comment markers inside strings)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(unit):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[unit]:
        with open(os.path.join(ROOT, "tensor_product_gnn_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(unit, workload):
    """HBM bytes per launch of `unit` from the rocprofv3 FETCH_SIZE / WRITE_SIZE record, or None
    when there is no record or the kernel's sources changed since it was taken."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        if not ln.startswith("traffic-record:"):
            continue
        kv = dict(t.split("=", 1) for t in ln.split()[1:])
        if kv.get("unit") == unit and kv.get("workload") == workload and \
                kv.get("sources") == kernel_source_hash(unit):
            return float(kv["hbm_bytes"])
    return None


def summarize_rocprof(d, workload):
    """Markdown summary of a rocprofv3 run set under directory `d`: trace/ (kernel-trace --stats),
    fetch/ and write/ (--pmc FETCH_SIZE, WRITE_SIZE), cfetch/ and cwrite/ (the same counters over
    plain device copies of known size, for the KiB-to-bytes factor)."""
    import csv
    import glob

    def rows(sub, suffix):
        f = glob.glob(os.path.join(d, sub, "**", f"*{suffix}"), recursive=True)
        return list(csv.DictReader(open(f[0]))) if f else []

    out = [f"rocprofv3 summary, workload {workload}", ""]
    stats = rows("trace", "kernel_stats.csv")
    if stats:
        out += ["| kernel | calls | avg us | total ms | % |", "|---|---|---|---|---|"]
        for r in stats:
            out.append(f"| `{r['Name'][:110]}` | {r['Calls']} | "
                       f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['TotalDurationNs']) / 1e6:.3f}"
                       f" | {float(r['Percentage']):.2f} |")
        out.append("")

    def per_kernel(sub):
        acc = {}
        for r in rows(sub, "counter_collection.csv"):
            a = acc.setdefault(r["Kernel_Name"], [0, 0.0])
            a[0] += 1
            a[1] += float(r["Counter_Value"])
        return {k: v[1] / v[0] for k, v in acc.items()}

    copy_bytes = None
    factors = {}
    for cnt, sub, csub in (("FETCH_SIZE", "fetch", "cfetch"), ("WRITE_SIZE", "write", "cwrite")):
        cp = [v for k, v in per_kernel(csub).items() if "copyBuffer" in k]
        if cp:
            kib = max(cp)
            copy_bytes = float(os.environ.get("COPY_BYTES", 256 << 20))
            factors[cnt] = copy_bytes / (kib * 1024)
            out.append(f"{cnt}: plain copy of {copy_bytes / 2**20:.0f} MiB counts {kib:.0f} KiB -> "
                       f"factor {factors[cnt]:.3f} bytes per counted byte")
    out.append("")
    fetch, write = per_kernel("fetch"), per_kernel("write")
    if fetch or write:
        out += ["| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | HBM MB/dispatch "
                "(scaled) |", "|---|---|---|---|"]
        for k in sorted(set(fetch) | set(write)):
            f_, w_ = fetch.get(k, 0.0), write.get(k, 0.0)
            mb = (f_ * 1024 * factors.get("FETCH_SIZE", 1.0) +
                  w_ * 1024 * factors.get("WRITE_SIZE", 1.0)) / 1e6
            out.append(f"| `{k[:110]}` | {f_:.0f} | {w_:.0f} | {mb:.2f} |")
    return "\n".join(out)


def timed_run(step, args, candidates):
    """Warm-up; an untimed pass of up to five steps with HIP events around every library unit (the
    per-unit breakdown, and which of `candidates` takes the most time); then the timed steps with
    events around that dominant unit only, so the timed region carries the events the roofline
    figure needs and not the cost (a few microseconds of stream time each) of events around every
    small launch.  Returns the timed steps' elapsed seconds, {unit: (launches, total ms)} (the
    dominant unit as timed, the others from the untimed pass scaled to the timed step count) and
    the dominant unit's name."""
    import torch
    import tensor_product_gnn_amd as tp
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    n_prof = max(1, min(args.steps, 5))
    tp.profile_reset()
    tp.profile_only(None)
    tp.profile_enable(True)
    for _ in range(n_prof):
        step()
    torch.cuda.synchronize()
    tp.profile_enable(False)
    every = tp.profile_read()
    dom = max((k for k in every if k in candidates), key=lambda k: every[k][1])
    tp.profile_reset()
    tp.profile_only([dom])
    tp.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    tp.profile_enable(False)
    timed = tp.profile_read()
    tp.profile_only(None)
    prof = {k: (v[0] // n_prof * args.steps, v[1] / n_prof * args.steps) for k, v in every.items()}
    prof[dom] = timed[dom]
    return elapsed, prof, dom


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mlp-bf16", action="store_true",
                    help="mixed-precision variant: bf16 operands (fp32 accumulation) for the radial-MLP "
                         "W2 contractions; tensor product and sums stay fp32")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run plain device-to-device copies of this many MiB (HBM counter "
                         "calibration for rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    ap.add_argument("--summarize-rocprof", default="",
                    help="print a markdown summary of the rocprofv3 output under this directory "
                         "and exit (no GPU work)")
    args = ap.parse_args()
    if args.summarize_rocprof:
        print(summarize_rocprof(args.summarize_rocprof, args.workload))
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding is a design note, not an implemented path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import tensor_product_gnn_amd as tp
    from tensor_product_gnn_amd import workloads

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 5}))
        return

    spec = WORKLOADS[args.workload]
    if spec.get("kind") == "ladder":
        run_ladder(args, spec)
        return
    if spec.get("kind") == "full_ladder":
        run_full_ladder(args, spec)
        return
    if spec.get("kind") == "mixed":
        run_mixed(args, spec)
        return
    wl = workloads.generate(args.workload)
    s = wl.spec
    conv = tp.Conv(wl.irreps(), wl.irreps_sh(), wl.irreps(), n_radial=s["n_radial"],
                   hidden=s["hidden"], r_cut=s["r_cut"], mlp_bf16=args.mlp_bf16)
    grads = spec["grads"]
    block = spec.get("block", False)
    g = tp.Graph.from_arrays(wl.n_nodes, wl.row_ptr, wl.src, wl.dst, sender_csr=("x" in grads),
                             path_mask=wl.path_mask)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    vec, x, W1, W2, G = t(wl.vec), t(wl.x), t(wl.W1), t(wl.W2), t(wl.G)
    out = torch.empty((wl.n_nodes, conv.f_out, conv.channels), dtype=torch.float32, device="cuda")
    outs = {k: torch.empty_like(v) for k, v in (("vec", vec), ("x", x), ("W1", W1), ("W2", W2))
            if k in grads}
    ws = torch.empty(conv.workspace_bytes(wl.n_nodes, wl.n_edges), dtype=torch.uint8, device="cuda")
    want = {f"want_{k}": (k in grads) for k in ("vec", "x", "W1", "W2")}
    if block:
        W_lin = t(np.stack(wl.W_lin))
        y, G_conv = torch.empty_like(out), torch.empty_like(out)

    def step():
        conv.forward(g, vec, x, W1, W2, out=out)
        if block:
            # y = out W_l per irrep; upstream dL/dy = G, so dL/dout = G W_l^T
            tp.linear(out, W_lin, wl.L, out=y)
            tp.linear(G, W_lin, wl.L, transpose=True, out=G_conv)
        if grads:
            conv.backward(g, vec, x, W1, W2, G_conv if block else G, workspace=ws, outs=outs,
                          **want)

    elapsed, prof, dom = timed_run(step, args, ("seg_fwd", "bwd", "seg_dx", "linear"))

    E = wl.n_edges
    tp_flop, mlp_flop = path_flops(conv, tp, wl.path_mask)
    # algorithmic FLOP per edge of each profiled unit (recomputation is not counted):
    #   seg_fwd  forward tensor product + forward radial MLP
    #   bwd      dL/dw and dL/dY (one tensor product each), dL/dh and dL/dW2 (one MLP contraction
    #            each), dL/de and dL/dW1 (the small hidden-layer terms, inside mlp_flop); one
    #            launch of this unit is the group kernels of one backward pass
    #   seg_dx   dL/dx (one tensor product)
    #            (without weight gradients: dL/dw, dL/dY and dL/dh only, 2 TP + 1 MLP)
    #   linear   per-irrep channel mixing, 2 N F C^2 per launch (expressed per edge)
    ww = "W1" in grads or "W2" in grads
    lin_flop = 2 * wl.n_nodes * conv.f_out * conv.channels ** 2 / E
    kflop = {"seg_fwd": tp_flop + mlp_flop,
             "bwd": 2 * tp_flop + (2 if ww else 1) * mlp_flop,
             "seg_dx": tp_flop, "linear": lin_flop}
    step_flop = kflop["seg_fwd"] + (kflop["bwd"] if grads else 0) + \
        (kflop["seg_dx"] if "x" in grads else 0) + (2 * lin_flop if block else 0)
    n_l, ms = prof[dom]
    avg_s = ms / 1e3 / n_l
    achieved = kflop[dom] * E / avg_s / 1e12
    kernels = {k: {"launches": v[0], "avg_us": round(v[1] * 1e3 / v[0], 2)} for k, v in prof.items()}
    # the tensor-product (VALU) and radial-MLP (MFMA) shares of each unit's algorithmic FLOP
    ksplit = {"seg_fwd": (tp_flop, mlp_flop),
              "bwd": (2 * tp_flop, (2 if ww else 1) * mlp_flop),
              "seg_dx": (tp_flop, 0.0)}
    for k in kernels:
        if k in kflop:
            sec = prof[k][1] / 1e3 / prof[k][0]
            kernels[k]["tflops"] = round(kflop[k] * E / sec / 1e12, 2)
            kernels[k]["frac"] = round(kernels[k]["tflops"] / FP32_PEAK_TFLOPS, 4)
            if k in ksplit:
                kernels[k]["tp_frac"] = round(ksplit[k][0] * E / sec / 1e12 / FP32_PEAK_TFLOPS, 4)
                kernels[k]["mlp_frac"] = round(ksplit[k][1] * E / sec / 1e12 / FP32_PEAK_TFLOPS, 4)
    value = E * args.steps / elapsed
    # graph preprocessing, outside the timed step (once per graph): the sender CSR that dL/dx
    # needs, built on the GPU (stable radix sort of the senders), wall clock with synchronisation
    csr_reps = 10
    tp.build_csr(g.src, wl.n_nodes)   # first use loads the sort's kernels
    torch.cuda.synchronize()
    tc = time.perf_counter()
    for _ in range(csr_reps):
        tp.build_csr(g.src, wl.n_nodes)
    torch.cuda.synchronize()
    csr_us = (time.perf_counter() - tc) / csr_reps * 1e6
    res = {
        "metric": METRIC, "value": value, "unit": "edges/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32 + bf16 MLP operands" if args.mlp_bf16 else "fp32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {spec['desc']}", "nodes": wl.n_nodes,
                   "edges": E, "channels": conv.channels, "lmax": wl.L, "hidden": conv.hidden,
                   "n_radial": conv.n_radial, "n_paths": conv.n_paths},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved,
                     "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / FP32_PEAK_TFLOPS,
                     # (the recorded counters are for the fp32 kernels)
                     "traffic": None if args.mlp_bf16 else recorded_traffic(dom, args.workload),
                     "flop_per_edge": kflop[dom], "launch_avg_us": avg_s * 1e6},
        "step_roofline": {"flop_per_edge": step_flop,
                          "achieved_tflops": step_flop * E * args.steps / elapsed / 1e12,
                          "frac": step_flop * E * args.steps / elapsed / 1e12 / FP32_PEAK_TFLOPS},
        "kernels": kernels,
        "graph_prep": {"sender_csr_build_us": round(csr_us, 1), "edges": E,
                       "note": "once per graph, not part of a step"},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.workload, spec["grads"])
    print(json.dumps(res))


def ladder_cpu_baseline(budget_s=20.0):
    """The fp64 oracle (forward and backward) on the first nodes of the ladder workload."""
    import numpy as np
    from oracle import ladder as ol
    from tensor_product_gnn_amd import workloads
    wl = workloads.generate_ladder("ladder")
    threads = os.environ.get("OMP_NUM_THREADS") or os.cpu_count()
    n, t_used = 16, 0.0
    while True:
        t0 = time.perf_counter()
        ol.forward(wl.A[:n], wl.w, wl.L, wl.nu)
        ol.backward(wl.A[:n], wl.w, wl.G[:n], wl.L, wl.nu)
        t_used = time.perf_counter() - t0
        if t_used > budget_s / 3 or n >= wl.n_nodes:
            break
        n *= 2
    return {"value": n / t_used, "unit": "nodes/s", "cores": int(threads), "kind": "oracle",
            "sample": f"ladder: nodes 0..{n - 1} of 4096, fp64 numpy forward + backward (A, w), "
                      f"{t_used:.1f} s"}


def run_ladder(args, spec):
    """The node-local product ladder ("FlashCart", Fig. 3(b)): one step is one forward and one
    backward (dL/dA and dL/dw) over all nodes; value in nodes/s."""
    import numpy as np
    import torch
    import tensor_product_gnn_amd as tp
    from tensor_product_gnn_amd import workloads

    wl = workloads.generate_ladder("ladder")
    L, nu, N, C = wl.L, wl.nu, wl.n_nodes, wl.C
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    A, w, G = t(wl.A), t(wl.w), t(wl.G)
    out = torch.empty_like(A)
    outs = {"A": torch.empty_like(A), "w": torch.empty_like(w)}
    ws = torch.empty(max(256, tp.ladder_workspace_bytes(L, nu, N, C)), dtype=torch.uint8,
                     device="cuda")

    rungs = tp.ladder_rungs(A, nu)   # a training step keeps the rungs for the backward

    def step():
        tp.ladder_forward(A, w, L, nu, out=out, rungs=rungs)
        tp.ladder_backward(A, w, G, L, nu, workspace=ws, outs=outs, rungs=rungs)

    elapsed, prof, dom = timed_run(step, args, ("ladder_fwd", "ladder_bwd"))

    # algorithmic FLOP per node: forward nu-1 products; backward dL/dw, dL/dB and dL/dA, one
    # product each per step (the rungs B_2..B_{nu-1} come from the forward)
    pf = ladder_flops(tp, L) * C
    kflop = {"ladder_fwd": (nu - 1) * pf, "ladder_bwd": 3 * (nu - 1) * pf}
    step_flop = kflop["ladder_fwd"] + kflop["ladder_bwd"]
    n_l, ms = prof[dom]
    avg_s = ms / 1e3 / n_l
    achieved = kflop[dom] * N / avg_s / 1e12
    kernels = {k: {"launches": v[0], "avg_us": round(v[1] * 1e3 / v[0], 2)} for k, v in prof.items()}
    for k in kernels:
        if k in kflop:
            kernels[k]["tflops"] = round(kflop[k] * N / (prof[k][1] / 1e3 / prof[k][0]) / 1e12, 2)
            kernels[k]["frac"] = round(kernels[k]["tflops"] / FP32_PEAK_TFLOPS, 4)
    res = {
        "metric": "nodes/sec, node-local product ladder fwd+bwd (128 ch, lmax 3, nu 5, fp32) + % of "
                  "FP32 vector roofline",
        "value": N * args.steps / elapsed, "unit": "nodes/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": f"ladder: {spec['desc']}", "nodes": N, "channels": C, "lmax": L,
                   "nu": nu, "n_paths": tp.ladder_num_paths(L)},
        "roofline": {"bound": "alu", "kernel": dom, "achieved": achieved,
                     "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / FP32_PEAK_TFLOPS,
                     "traffic": recorded_traffic(dom, "ladder"),
                     "flop_per_node": kflop[dom], "launch_avg_us": avg_s * 1e6},
        "step_roofline": {"flop_per_node": step_flop,
                          "achieved_tflops": step_flop * N * args.steps / elapsed / 1e12,
                          "frac": step_flop * N * args.steps / elapsed / 1e12 / FP32_PEAK_TFLOPS},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = ladder_cpu_baseline()
    print(json.dumps(res))


def full_ladder_flops(tp, lmax, C):
    """Algorithmic FLOP per node of each full-ladder kernel, one launch (one step).  Products
    (per channel): one FMA per CG entry and one per (m1, m3) pair with entries, as in the
    path-reduced product without its weight; their backward: two FMAs per CG entry (dL/dB and
    dL/dA).  Each mixing GEMM (forward, dT, dW): 2 C^2 per row of path outputs, sum_p (2 l3 + 1)
    rows per node."""
    nnz = pairs = rows = 0
    for l1 in range(lmax + 1):
        for l2 in range(lmax + 1):
            for l3 in range(abs(l1 - l2), min(l1 + l2, lmax) + 1):
                if (l1 + l2 + l3) % 2:
                    continue
                nz = tp.cg_block(l1, l2, l3) != 0
                nnz += int(nz.sum())
                pairs += int(nz.any(axis=1).sum())
                rows += 2 * l3 + 1
    gemm = 2 * rows * C * C
    return {"full_tp": 2 * (nnz + pairs) * C, "full_tp_bwd": 4 * nnz * C,
            "mix_fwd": gemm, "mix_dt": gemm, "mix_dw": gemm}


def full_ladder_cpu_baseline(budget_s=20.0):
    """The fp64 oracle (forward and backward) on the first nodes of the full-ladder workload."""
    from oracle import ladder as ol
    from tensor_product_gnn_amd import workloads
    wl = workloads.generate_full_ladder("ladder")
    threads = 1
    try:
        import threadpoolctl
        threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:
        pass
    n, t_used = 16, 0.0
    while True:
        t0 = time.perf_counter()
        ol.full_forward(wl.A[:n], wl.W, wl.L, wl.nu)
        ol.full_backward(wl.A[:n], wl.W, wl.G[:n], wl.L, wl.nu)
        t_used = time.perf_counter() - t0
        if t_used > budget_s / 3 or n >= wl.n_nodes:
            break
        n *= 2
    return {"value": n / t_used, "unit": "nodes/s", "cores": int(threads), "kind": "oracle",
            "sample": f"full_ladder: nodes 0..{n - 1} of 4096, fp64 numpy forward + backward "
                      f"(A, W), {t_used:.1f} s"}


def run_full_ladder(args, spec):
    """The full product ladder ("FlashCart", Fig. 3(b), dashed curves): one step is one forward
    and one backward (dL/dA and dL/dW) over all nodes; value in nodes/s."""
    import numpy as np
    import torch
    import tensor_product_gnn_amd as tp
    from tensor_product_gnn_amd import workloads

    wl = workloads.generate_full_ladder("ladder")
    L, nu, N, C = wl.L, wl.nu, wl.n_nodes, wl.C
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    A, W, G = t(wl.A), t(wl.W), t(wl.G)
    out = torch.empty_like(A)
    outs = {"A": torch.empty_like(A), "W": torch.empty_like(W)}
    ws = torch.empty(max(256, tp.full_ladder_workspace_bytes(L, nu, N, C, True)),
                     dtype=torch.uint8, device="cuda")
    rungs = tp.ladder_rungs(A, nu)
    saved = tp.full_ladder_saved(A, L, nu)   # a training step keeps every step's path outputs

    def step():
        tp.full_ladder_forward(A, W, L, nu, out=out, rungs=rungs, saved=saved, workspace=ws)
        tp.full_ladder_backward(A, W, G, L, nu, workspace=ws, outs=outs, rungs=rungs, saved=saved)

    elapsed, prof, dom = timed_run(step, args,
                                   ("mix_fwd", "mix_dt", "mix_dw", "full_tp", "full_tp_bwd"))

    kflop = full_ladder_flops(tp, L, C)
    step_flop = sum(kflop[k] * prof[k][0] / args.steps for k in prof if k in kflop)
    n_l, ms = prof[dom]
    avg_s = ms / 1e3 / n_l
    achieved = kflop[dom] * N / avg_s / 1e12
    gemm = [k for k in ("mix_fwd", "mix_dt", "mix_dw") if k in prof]
    gemm_flop = sum(kflop[k] * N * prof[k][0] for k in gemm)
    gemm_s = sum(prof[k][1] / 1e3 for k in gemm)
    kernels = {k: {"launches": v[0], "avg_us": round(v[1] * 1e3 / v[0], 2)} for k, v in prof.items()}
    for k in kernels:
        if k in kflop:
            kernels[k]["tflops"] = round(kflop[k] * N / (prof[k][1] / 1e3 / prof[k][0]) / 1e12, 2)
            kernels[k]["frac"] = round(kernels[k]["tflops"] / FP32_PEAK_TFLOPS, 4)
            kernels[k]["share"] = round(prof[k][1] / 1e3 / elapsed, 4)
    res = {
        "metric": "nodes/sec, full node-local product ladder fwd+bwd (128 ch, lmax 3, nu 5, fp32) "
                  "+ % of FP32 matrix roofline",
        "value": N * args.steps / elapsed, "unit": "nodes/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": f"full_ladder: {spec['desc']}", "nodes": N, "channels": C,
                   "lmax": L, "nu": nu, "n_paths": tp.ladder_num_paths(L)},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved,
                     "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / FP32_PEAK_TFLOPS,
                     "traffic": recorded_traffic(dom, "full_ladder"),
                     "flop_per_node": kflop[dom], "launch_avg_us": avg_s * 1e6},
        "gemm_roofline": {"kernels": gemm, "achieved_tflops": gemm_flop / gemm_s / 1e12,
                          "frac": gemm_flop / gemm_s / 1e12 / FP32_PEAK_TFLOPS},
        "step_roofline": {"flop_per_node": step_flop,
                          "achieved_tflops": step_flop * N * args.steps / elapsed / 1e12,
                          "frac": step_flop * N * args.steps / elapsed / 1e12 / FP32_PEAK_TFLOPS},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = full_ladder_cpu_baseline()
    print(json.dumps(res))


def mixed_cpu_baseline(budget_s=20.0):
    """The fp64 mixed-multiplicity oracle on the edges into the first receivers of c2m."""
    import numpy as np
    from oracle import mixed as om
    from tensor_product_gnn_amd import workloads
    wl = workloads.generate_mixed("c2m")
    pb = om.Problem.from_workload(wl)
    rp = wl.graph.row_ptr
    threads = 1
    try:
        import threadpoolctl
        threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:
        pass
    n_recv = 1
    while True:
        edges = np.arange(rp[0], rp[n_recv])
        t0 = time.perf_counter()
        om.forward(pb, edges=edges)
        om.backward(pb, edges=edges)
        t_used = time.perf_counter() - t0
        if t_used * 2.2 > budget_s or n_recv >= 64:
            break
        n_recv *= 2
    return {"value": len(edges) / t_used, "unit": "edges/s", "cores": int(threads), "kind": "oracle",
            "sample": f"c2m: the {len(edges)} edges into receivers 0..{n_recv - 1}, fp64 numpy forward + "
                      f"backward (vec, x, W1, W2, maps), {t_used:.1f} s"}


def run_mixed(args, spec):
    """Edge convolution with mixed per-l multiplicities: one step is one forward and one backward
    (dL/dvec, dL/dW1, dL/dW2, dL/dWlin) on c2's graph; value in edges/s."""
    import numpy as np
    import torch
    import tensor_product_gnn_amd as tp
    from oracle import mixed as om
    from tensor_product_gnn_amd import workloads

    wl = workloads.generate_mixed("c2m")
    g0 = wl.graph
    conv = tp.MixedConv(wl.irreps(wl.mult_in), wl.irreps(wl.mult_out), n_radial=8, hidden=64,
                        r_cut=g0.spec["r_cut"])
    g = tp.Graph.from_arrays(g0.x.shape[0], g0.row_ptr, g0.src, g0.dst, sender_csr=False)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    vec, x, W1, W2, Wlin, G = t(g0.vec), t(wl.x), t(g0.W1), t(wl.W2), t(wl.Wlin), t(wl.G)
    N, E = g0.x.shape[0], len(g0.src)
    out = torch.empty((N, conv.f_out), dtype=torch.float32, device="cuda")
    want = ("vec", "W1", "W2", "Wlin")
    outs = {"vec": torch.empty((E, 3), device="cuda"), "W1": torch.empty_like(W1),
            "W2": torch.empty_like(W2), "Wlin": torch.empty_like(Wlin)}
    ws = torch.empty(max(256, conv.workspace_bytes(N, E, True)), dtype=torch.uint8, device="cuda")
    saved = conv.saved_tensor(N)   # a training step keeps the path outputs for the backward

    def step():
        conv.forward(g, vec, x, W1, W2, Wlin, out=out, saved=saved, workspace=ws)
        conv.backward(g, vec, x, W1, W2, Wlin, G, want=want, workspace=ws, outs=outs, saved=saved)

    elapsed, prof, dom = timed_run(step, args, ("bwd", "seg_fwd", "mixed_mix_fwd", "mixed_mix_dt",
                                                "mixed_mix_dw"))

    # algorithmic FLOP per edge (oracle.mixed.flops_per_edge: products, radial MLP, maps); the
    # units are whole passes: `seg_fwd` = the masked slice forwards of one forward pass (the
    # forward keeps the path outputs, so the backward does not run them again), `bwd` = the masked
    # slice backwards of one backward pass (dL/dw and dL/dY: two products; dL/dh and dL/dW2: two
    # MLP contractions)
    tpf, mlpf, linf = om.flops_per_edge(wl.mult_in, wl.mult_out, 8, 64, N, E)
    units = {"bwd": 2 * tpf + 2 * mlpf, "seg_fwd": tpf + mlpf,
             "mixed_mix_fwd": linf, "mixed_mix_dt": linf, "mixed_mix_dw": linf}
    per_step = {k: prof[k][1] / 1e3 / args.steps for k in prof}
    step_flop = (tpf + mlpf + linf) + (2 * tpf + 2 * mlpf + 2 * linf)
    dom_s = per_step[dom]
    achieved = units[dom] * E / dom_s / 1e12
    kernels = {k: {"launches": v[0], "avg_us": round(v[1] * 1e3 / v[0], 2),
                   "per_step_us": round(per_step[k] * 1e6, 1)} for k, v in prof.items()}
    res = {
        "metric": "edges/sec fwd+bwd, mixed multiplicities 128x0e+64x1o+32x2e+32x3o (lmax 3, fp32) "
                  "+ % of FP32 roofline",
        "value": E * args.steps / elapsed, "unit": "edges/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": f"c2m: {spec['desc']}", "nodes": N, "edges": E,
                   "mult_in": wl.mult_in, "mult_out": wl.mult_out, "n_paths": conv.n_paths,
                   "channel_slices": conv.n_slices, "launches_per_pass": conv.n_launches},
        "roofline": {"bound": "mfma", "kernel": f"{dom} (one pass: all its masked slice launches)",
                     "achieved": achieved, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / FP32_PEAK_TFLOPS,
                     "traffic": recorded_traffic(dom, "c2m") if dom == "bwd" else None,
                     "flop_per_edge": units[dom], "pass_us": dom_s * 1e6},
        "step_roofline": {"flop_per_edge": step_flop,
                          "achieved_tflops": step_flop * E * args.steps / elapsed / 1e12,
                          "frac": step_flop * E * args.steps / elapsed / 1e12 / FP32_PEAK_TFLOPS},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = mixed_cpu_baseline()
    print(json.dumps(res))


if __name__ == "__main__":
    main()
