"""Benchmark: one KAN layer training step (forward + backward) on one MI355X.

A step is the whole hot path over one batch: pack the coefficient operand,
forward contraction (basis generated in LDS), pack the transposed operand and
dy, dx contraction with its B' epilogue, and the batch-reduction contraction
for dC and dW_base.  Inputs are seeded synthetic tensors resident in HBM
before timing starts.  Prints one JSON line.

Default workload: one layer 4096 -> 4096, 65536 rows, G = 20 cubic, bf16 x /
C / W_base, float32 accumulation, silu base branch.  Other workloads:
``--workload c1 .. c5`` (c2 and c4 are two-layer chains), and ``g1`` / ``g2``,
the grouped spline activation (one spline per group of channels): a step is
its forward and its backward (dx, and dC reduced over every row), and the
line reports elements/s against the HBM roofline.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KAN layer fwd+bwd rows/sec and GFLOP/s; % of MFMA/HBM roofline, 1 GPU"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}     # MI355X dense MFMA (fp32: = vector fp32)
PEAK_HBM_GBS = 8000.0
WORKLOAD_TEXT = {
    "c1": "KAN layer 8->4, 32 rows, G=8 cubic on [-1,1], fp32, no base branch",
    "c2": "KAN net 784->64->10, 1024 rows, G=8 cubic on [-1,1], fp32, silu base branch",
    "c3": "KAN layer 1024->1024, 8192 rows, cubic on [-1,1], fp32, no base branch",
    "c4": "KAN channel mixer 768->3072->768, 12608 rows (64 x 197 tokens), G=5 cubic, bf16 "
          "x/C/W_base, fp32 accumulate, silu base branch",
    "c5": "KAN layer 4096->4096, 65536 rows, G=20 cubic on [-1,1], bf16 x/C/W_base, fp32 "
          "accumulate, silu base branch",
    "g1": "grouped spline activation, 25216 rows (128 x 197 tokens) x 3072 channels, 8 groups, "
          "G=5 cubic on [-1,1], bf16 x/C, fp32 y/dx/dC",
    "g2": "per-channel spline activation, 32768 rows (8 x 4096 tokens) x 2048 channels, 2048 "
          "groups, G=8 cubic on [-1,1], bf16 x/C, fp32 y/dx/dC",
    "s1": "2-D tensor-product spline layer, 8192 rows, 1024 inputs as 512 pairs -> 1024 outputs, "
          "G=5 bicubic on [-1,1]^2, bf16 x/C, fp32 accumulate",
}
SURFACE_METRIC = "2-D tensor-product KAN layer fwd+bwd rows/sec; % of MFMA roofline, 1 GPU"
GROUPED_METRIC = "grouped spline activation fwd+bwd elements/sec; % of HBM roofline, 1 GPU"
MFMA_FILES = ("kan_mfma.hip", "kan_device.h", "kan_sparse.h", "kan_internal.h", "kan_api.cpp")
GROUPED_FILES = ("kan_grouped.hip", "kan_device.h", "kan_internal.h", "kan_api.cpp")
GATHER_FILES = ("kan_gather.hip", "kan_device.h", "kan_internal.h", "kan_plan.cpp", "kan_api.cpp")
DIGEST_FILES = {"mfma": MFMA_FILES, "grouped": GROUPED_FILES, "gather": GATHER_FILES}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 10 for c5, else 20)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c5", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--G", type=int, default=None, help="grid size (c3 only: 8, 20 or 50)")
    ap.add_argument("--variant", default="auto", choices=["auto", "mfma", "gather"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=None)
    ap.add_argument("--code-digest", nargs="?", const="mfma", default=None, choices=sorted(DIGEST_FILES),
                    help="print the digest that ties a counter summary to the kernel source")
    ap.add_argument("--degree", type=int, default=3,
                    help="spline degree (1 .. 5) of the layer workloads and of --basis-forms")
    ap.add_argument("--basis-forms", type=int, default=0, metavar="POINTS",
                    help="time the local-span and truncated-power basis evaluations on POINTS inputs")
    ap.add_argument("--forward-forms", action="store_true",
                    help="time the bf16 matrix-core forward with its three operand generators "
                         "(2:4 sparse, span-based dense, truncated-power dense) on the bf16 layer shapes")
    ap.add_argument("--blas-reference", action="store_true",
                    help="time plain bf16 torch.matmul on the c5 contraction shapes and exit")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run one plain device copy of BYTES bytes (HBM counter calibration)")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 10 if args.workload == "c5" else 20
    return args


def basis_forms(n, steps, degree=3):
    """Dense B and dB of n float32 inputs on [-1, 1] (+ one grid width each
    side) from the local span form (kan_basis_eval) and from the truncated-power
    form (kan_basis_eval_tp), at G = 8, 20, 50 and the given degree: points/s
    and output GB/s."""
    import ctypes
    import torch
    from kolmogorov_arnold_network_amd import _lib as L
    g = torch.Generator(device="cuda:0").manual_seed(3)
    x = torch.rand(n, device="cuda:0", generator=g) * 2.5 - 1.25
    res = {}
    for G in (8, 20, 50):
        B = torch.empty(n, G + degree, device="cuda:0")
        dB = torch.empty_like(B)
        for name, fn in (("local_span", L.lib().kan_basis_eval), ("truncated_power", L.lib().kan_basis_eval_tp)):
            grid = L.kan_grid_t(-1.0, 1.0, G, degree)
            S = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            call = lambda: L.check(fn(ctypes.byref(grid), n, L.KAN_F32, ctypes.c_void_p(x.data_ptr()),
                                      ctypes.c_void_p(B.data_ptr()), ctypes.c_void_p(dB.data_ptr()), S), name)
            call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                call()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            out_bytes = 2 * n * (G + degree) * 4
            res["G%d_%s" % (G, name)] = {"ms": ms, "points_per_s": n / (ms * 1e-3),
                                          "output_GB_per_s": out_bytes / (ms * 1e-3) / 1e9,
                                          "hbm_frac": out_bytes / (ms * 1e-3) / 8e12}
    print(json.dumps({"basis_forms": res, "points": n, "steps": steps, "degree": degree}))


def forward_forms(steps):
    """The bf16 layer forward on the matrix cores with each of its three A
    operand generators -- the 2:4 structured-sparse one (default), the dense
    span-based one (KAN_FLAG_DENSE_FORWARD) and the dense truncated-power one
    (KAN_FLAG_TP_FORWARD) -- on the layer shapes of the bf16 workloads and of
    the grid sweep at bf16: ms per forward and the output's relative Frobenius
    distance from the span-based dense forward.  Inputs are drawn on the
    device: x ~ U(-1, 1), C ~ N(0, 0.02), W_base ~ N(0, 1/in)."""
    import torch
    from kolmogorov_arnold_network_amd import _lib as L
    from kolmogorov_arnold_network_amd import functional as F
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(11)
    res = []
    for name, N, I, O, G in (("768->3072 (12608 rows, G=5)", 12608, 768, 3072, 5),
                             ("3072->768 (12608 rows, G=5)", 12608, 3072, 768, 5),
                             ("1024->1024 (8192 rows, G=8)", 8192, 1024, 1024, 8),
                             ("1024->1024 (8192 rows, G=20)", 8192, 1024, 1024, 20),
                             ("1024->1024 (8192 rows, G=50)", 8192, 1024, 1024, 50),
                             ("4096->4096 (65536 rows, G=20)", 65536, 4096, 4096, 20)):
        x = (torch.rand(N, I, device=dev, generator=g) * 2 - 1).to(torch.bfloat16)
        C = (torch.randn(O, I, G + 3, device=dev, generator=g) * 0.02).to(torch.bfloat16)
        W = (torch.randn(O, I, device=dev, generator=g) / I ** 0.5).to(torch.bfloat16)
        grid = (-1.0, 1.0, G)
        row = {"layer": name}
        ys = {}
        for form, kw in (("sparse", {}), ("dense", {"dense_forward": True}), ("tp", {"tp_forward": True})):
            flags = F._fwd_flags(kw.get("dense_forward", False), kw.get("tp_forward", False))
            ws = F.workspace(F.layer_desc(x, C, W, grid, "mfma", flags), L.KAN_PASS_FORWARD, dev)
            y = F.kan_forward(x, C, W, grid, "mfma", ws=ws, **kw)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                F.kan_forward(x, C, W, grid, "mfma", ws=ws, out=y, **kw)
            e1.record()
            torch.cuda.synchronize()
            row[form + "_ms"] = e0.elapsed_time(e1) / steps
            ys[form] = y
        for form in ("sparse", "tp"):
            row[form + "_vs_dense"] = float((ys[form] - ys["dense"]).norm() / ys["dense"].norm())
        res.append(row)
        print(json.dumps(row), flush=True)
        del x, C, W, ys, y, ws
        torch.cuda.empty_cache()
    print(json.dumps({"forward_forms": res, "steps": steps}))


def blas_reference(steps):
    """Plain bf16 GEMMs of the c5 contraction shapes (forward, dx, dC) through
    torch.matmul, the vendor BLAS, on random data: the rate a library GEMM of
    the same size reaches on this GPU, for comparison with the fused
    contraction kernels."""
    import torch
    res = []
    for name, (M, N, K) in (("fwd", (65536, 4096, 98304)), ("dx", (65536, 98304, 4096)),
                            ("dC", (4096, 98304, 65536))):
        a = torch.randn(M, K, device="cuda:0", dtype=torch.bfloat16)
        b = torch.randn(K, N, device="cuda:0", dtype=torch.bfloat16)
        c = torch.empty(M, N, device="cuda:0", dtype=torch.bfloat16)
        torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res.append({"gemm": name, "M": M, "N": N, "K": K, "ms": ms,
                    "TFLOP_per_s": 2.0 * M * N * K / ms / 1e9})
        del a, b, c
        torch.cuda.empty_cache()
    print(json.dumps({"blas_reference": res, "steps": steps}))


def copy_probe(nbytes):
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": src.numel() * 4}))


def stage_names(nl):
    out = []
    for l in range(nl):
        out += ["L%d.pack_fwd" % l, "L%d.fwd" % l] + (["L%d.cast" % l] if l + 1 < nl else [])
    for l in range(nl - 1, -1, -1):
        out += ["L%d.pack_bwd" % l, "L%d.dx" % l, "L%d.dC" % l]
    return out


def main():
    args = parse()
    if args.code_digest:
        print(kernel_code_digest(DIGEST_FILES[args.code_digest]))
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.blas_reference:
        blas_reference(args.steps)
        return
    if args.forward_forms:
        forward_forms(args.steps)
        return
    if args.basis_forms:
        basis_forms(args.basis_forms, args.steps, args.degree)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the KAN layer path here has no multi-GPU "
              "mode (it would shard the rows, one process per GPU, and all-reduce dC and "
              "dW_base); run with "
              "--gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.workload.startswith("g"):
        grouped_bench(args)
        return
    if args.workload.startswith("s"):
        surface_bench(args)
        return

    import numpy as np
    import torch

    import workloads as wl
    from kolmogorov_arnold_network_amd import _lib as L
    from kolmogorov_arnold_network_amd import functional as F

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = wl.make_workload(args.workload, G=args.G, degree=args.degree)
    G, lo, hi = d["G"], d["lo"], d["hi"]
    grid = (lo, hi, G)
    dt = d["dtype"]
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    N = d["N"]
    widths = d["widths"]
    nl = len(widths) - 1
    base = d["base"]

    def dev_t(a, dtype):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dtype)

    x0 = dev_t(d["x"], tdt)
    layers = [(dev_t(C, tdt), dev_t(W, tdt)) for C, W in d["layers"]]
    dy = dev_t(d["dy"], torch.float32)
    # per-layer buffers, workspaces and descriptors, allocated once
    ys = [torch.empty((N, widths[l + 1]), dtype=torch.float32, device=dev) for l in range(nl)]
    # a float32 chain reads the previous layer's output in place; a bf16 chain
    # rounds it into a bf16 buffer first
    xs = [x0] + [torch.empty((N, widths[l + 1]), dtype=tdt, device=dev) if dt == "bf16" else ys[l]
                 for l in range(nl - 1)]
    gx = [torch.empty((N, widths[l]), dtype=torch.float32, device=dev) for l in range(nl)]
    gC = [torch.empty_like(C, dtype=torch.float32) for C, _ in layers]
    gW = [None if W is None else torch.empty_like(W, dtype=torch.float32) for _, W in layers]
    descs, wsf, wsb, descs_p = [], [], [], []
    for l, (C, W) in enumerate(layers):
        dsc = F.layer_desc(xs[l], C, W, grid, args.variant)
        descs.append(dsc)
        dp = F.layer_desc(xs[l], C, W, grid, args.variant, L.KAN_FLAG_PREPARED)
        descs_p.append(dp)
        wsf.append(F.workspace(dsc, L.KAN_PASS_FORWARD, dev))
        wsb.append(F.workspace(dsc, L.KAN_PASS_BACKWARD, dev))
    lib = L.lib()
    import ctypes
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = torch.cuda.current_stream(dev)
    S = ctypes.c_void_p(stream.cuda_stream)
    names = stage_names(nl)
    events = None

    def rec(k):
        if events is not None:
            events[k].record(stream)

    def step():
        k = 0
        rec(k)
        for l, (C, W) in enumerate(layers):
            dsc = ctypes.byref(descs[l])
            buf, n = wsf[l]
            L.check(lib.kan_prepare(dsc, 0, P(C), P(W), None, P(buf), n, S), "prepare fwd")
            k += 1; rec(k)
            L.check(lib.kan_forward(ctypes.byref(descs_p[l]), P(xs[l]), P(C), P(W), P(ys[l]), P(buf),
                                    n, S), "forward")
            k += 1; rec(k)
            if l + 1 < nl:
                if dt == "bf16":
                    L.check(lib.kan_cast_f32_to_bf16(P(ys[l]), P(xs[l + 1]), ys[l].numel(), S), "cast")
                k += 1; rec(k)
        g = dy
        for l in range(nl - 1, -1, -1):
            C, W = layers[l]
            dsc = ctypes.byref(descs[l])
            dpp = ctypes.byref(descs_p[l])
            buf, n = wsb[l]
            L.check(lib.kan_prepare(dsc, 1, P(C), P(W), P(g), P(buf), n, S), "prepare bwd")
            k += 1; rec(k)
            L.check(lib.kan_backward(dpp, P(xs[l]), P(C), P(W), P(g), P(gx[l]), None, None, P(buf), n,
                                     S), "backward dx")
            k += 1; rec(k)
            L.check(lib.kan_backward(dpp, P(xs[l]), P(C), P(W), P(g), None, P(gC[l]), P(gW[l]),
                                     P(buf), n, S), "backward dC")
            k += 1; rec(k)
            g = gx[l]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    per_step_events = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        events = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        per_step_events.append(events)
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    events = None
    stage_ms = {nm: 0.0 for nm in names}
    for evs in per_step_events:
        for k, nm in enumerate(names):
            stage_ms[nm] += evs[k].elapsed_time(evs[k + 1]) / args.steps
    ms_per_step = 1e3 * elapsed / args.steps
    step_ms = sorted(evs[0].elapsed_time(evs[-1]) for evs in per_step_events)
    median_ms = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (
        step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])
    # work counts: algorithmic = the D + 1 non-zero basis functions (+ silu) per
    # input in each of the three contractions (D = 3: 4); executed = the dense
    # I*(G+D+base) basis, except a structured-sparse forward, whose matrix
    # instructions run half of its 4 NG columns per input (the rule of
    # KAN_FLAG_DENSE_FORWARD in kan.h; cubic layers only)
    D = args.degree
    Kb = G + D + (1 if base else 0)
    ng = max(4, (Kb + 3) // 4)
    ng += ng & 1
    sparse = (D == 3 and dt == "bf16" and args.variant in ("auto", "mfma") and ng <= 8 and Kb >= 11
              and 8 * ng <= 3 * Kb)
    fwd_cols = 2 * ng if sparse else Kb
    alg = exe = 0.0
    for l in range(nl):
        I, O = widths[l], widths[l + 1]
        alg += 6.0 * N * I * O * (D + 1 + (1 if base else 0))
        exe += 2.0 * N * I * O * (fwd_cols + 2 * Kb)
    gemm_stages = [nm for nm in names if nm.split(".")[1] in ("fwd", "dx", "dC")]
    dom = max(gemm_stages, key=lambda nm: stage_ms[nm])
    dl = int(dom[1])
    I, O = widths[dl], widths[dl + 1]
    alg_dom = 2.0 * N * I * O * (D + 1 + (1 if base else 0))
    exe_dom = 2.0 * N * I * O * (fwd_cols if dom.endswith(".fwd") else Kb)
    # which kernel family ran the dominant stage: the variant asked for, or
    # AUTO's rule (include/kan.h, kan_variant_t): bf16 on the matrix cores;
    # float32 forward on the gather kernel, float32 backward by its cost estimate
    Kb_dom = G + D + (1 if base else 0)
    mfma_ok = Kb_dom <= 256 and (D == 3 or Kb_dom >= 4)
    if args.variant != "auto":
        mfma_path = args.variant == "mfma"
    elif dt == "bf16":
        mfma_path = mfma_ok
    elif dom.endswith(".fwd"):
        mfma_path = False
    else:
        nio = float(N) * I * O
        mfma_path = mfma_ok and 4.0 * nio * Kb_dom / 110e12 + 150e-6 < nio / 1.6e12
    peak = PEAK_TFLOPS[dt]
    t_dom = stage_ms[dom] * 1e-3
    roof = {
        "bound": "mfma" if mfma_path else "alu",
        "kernel": dom,
        "achieved": alg_dom / t_dom / 1e12,
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": alg_dom / t_dom / 1e12 / peak,
        "traffic": None,
        "executed_achieved": exe_dom / t_dom / 1e12 if mfma_path else None,
        "executed_frac": exe_dom / t_dom / 1e12 / peak if mfma_path else None,
        "dominant_ms": stage_ms[dom],
    }
    tr = read_traffic(args.workload, dom.split(".")[1], MFMA_FILES if mfma_path else GATHER_FILES)
    if tr is not None:
        roof["traffic"] = tr
    out = {
        "metric": METRIC,
        "value": N * 1e3 / ms_per_step,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "median_ms_per_step": median_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload] + (" (G=%d)" % G if args.workload == "c3" else "")
                   + (" (spline degree %d)" % D if D != 3 else ""),
                   "name": args.workload, "rows": N, "widths": widths, "G": G,
                   "base_branch": base, "variant": args.variant, "degree": D},
        "gflops_algorithmic": alg / (ms_per_step * 1e-3) / 1e9,
        "gflops_executed": exe / (ms_per_step * 1e-3) / 1e9,
        "sparse_forward": sparse,
        "stage_ms": stage_ms,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, args.cpu_rows)
    print(json.dumps(out))


def grouped_bench(args):
    """Forward and backward of the grouped spline activation, timed per stage
    with HIP events on the launch stream."""
    import ctypes

    import numpy as np
    import torch

    import workloads as wl
    from kolmogorov_arnold_network_amd import _lib as L
    from kolmogorov_arnold_network_amd import functional as F

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = wl.make_grouped(args.workload)
    N, I, groups, G = d["N"], d["I"], d["groups"], d["G"]
    K = G + 3
    tdt = torch.bfloat16 if d["dtype"] == "bf16" else torch.float32
    es = 2 if d["dtype"] == "bf16" else 4
    x = torch.from_numpy(d["x"]).to(dev).to(tdt)
    C = torch.from_numpy(d["C"]).to(dev).to(tdt)
    dy = torch.from_numpy(d["dy"]).to(dev)
    y = torch.empty((N, I), dtype=torch.float32, device=dev)
    dx = torch.empty((N, I), dtype=torch.float32, device=dev)
    dC = torch.empty((groups, K), dtype=torch.float32, device=dev)
    desc = F.group_desc(x, C, (d["lo"], d["hi"], G))
    nws = F.kan_group_workspace_size(desc)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    lib = L.lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = torch.cuda.current_stream(dev)
    S = ctypes.c_void_p(stream.cuda_stream)
    names = ["group.fwd", "group.bwd"]
    events = None

    def rec(k):
        if events is not None:
            events[k].record(stream)

    def step():
        rec(0)
        L.check(lib.kan_group_forward(ctypes.byref(desc), P(x), P(C), P(y), S), "group forward")
        rec(1)
        L.check(lib.kan_group_backward(ctypes.byref(desc), P(x), P(C), P(dy), P(dx), P(dC), P(ws), nws, S),
                "group backward")
        rec(2)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    per_step = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        events = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        per_step.append(events)
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stage_ms = {nm: sum(ev[k].elapsed_time(ev[k + 1]) for ev in per_step) / args.steps
                for k, nm in enumerate(names)}
    ms_per_step = 1e3 * elapsed / args.steps
    step_ms = sorted(ev[0].elapsed_time(ev[2]) for ev in per_step)
    median_ms = step_ms[len(step_ms) // 2]
    # algorithmic HBM bytes: every element of x read once and y written once
    # (forward); x and dy read and dx written once (backward); C once, dC once
    alg = {"group.fwd": N * I * (es + 4) + groups * K * es,
           "group.bwd": N * I * (es + 4 + 4) + groups * K * (es + 4)}
    dom = max(names, key=lambda nm: stage_ms[nm])
    achieved = alg[dom] / (stage_ms[dom] * 1e-3) / 1e9
    roof = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": read_traffic(args.workload, dom.replace(".", "_"),
                                                                     GROUPED_FILES),
            "algorithmic_bytes": alg[dom], "dominant_ms": stage_ms[dom],
            "stage_GBps": {nm: alg[nm] / (stage_ms[nm] * 1e-3) / 1e9 for nm in names}}
    out = {
        "metric": GROUPED_METRIC,
        "value": N * I * 1e3 / ms_per_step,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "median_ms_per_step": median_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": d["dtype"],
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "name": args.workload, "rows": N,
                   "channels": I, "groups": groups, "G": G},
        "stage_ms": stage_ms,
        "workspace_bytes": nws,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = grouped_cpu_baseline(d, args.cpu_rows)
    print(json.dumps(out))


def surface_bench(args):
    """One training step of the 2-D tensor-product layer: forward (packing
    included), dx (packing of C^T and dy included) and dC, timed per stage
    with HIP events on the launch stream."""
    import ctypes

    import numpy as np
    import torch

    import workloads as wl
    from kolmogorov_arnold_network_amd import _lib as L
    from kolmogorov_arnold_network_amd import functional as F

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = wl.make_surface(args.workload)
    N, P, O, G = d["N"], d["P"], d["O"], d["G"]
    K1 = G + 3
    tdt = torch.bfloat16 if d["dtype"] == "bf16" else torch.float32
    x = torch.from_numpy(d["x"]).to(dev).to(tdt)
    C = torch.from_numpy(d["C"]).to(dev).to(tdt)
    dy = torch.from_numpy(d["dy"]).to(dev)
    y = torch.empty((N, O), dtype=torch.float32, device=dev)
    dx = torch.empty((N, 2 * P), dtype=torch.float32, device=dev)
    dC = torch.empty(C.shape, dtype=torch.float32, device=dev)
    grid = (d["lo"], d["hi"], G)
    desc = F.surface_desc(x, C, grid)
    dprep = F.surface_desc(x, C, grid)
    dprep.flags = L.KAN_FLAG_PREPARED
    nf = F.kan_surface_workspace_size(desc, L.KAN_PASS_FORWARD)
    nb = F.kan_surface_workspace_size(desc, L.KAN_PASS_BACKWARD)
    wsf = torch.empty(max(nf, 1), dtype=torch.uint8, device=dev)
    wsb = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    lib = L.lib()
    Pt = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = torch.cuda.current_stream(dev)
    S = ctypes.c_void_p(stream.cuda_stream)
    names = ["surface.fwd", "surface.dx", "surface.dC"]
    events = None

    def rec(k):
        if events is not None:
            events[k].record(stream)

    def step():
        rec(0)
        L.check(lib.kan_surface_forward(ctypes.byref(desc), Pt(x), Pt(C), Pt(y), Pt(wsf), nf, S), "forward")
        rec(1)
        L.check(lib.kan_surface_backward(ctypes.byref(desc), Pt(x), Pt(C), Pt(dy), Pt(dx), None, Pt(wsb), nb, S),
                "backward dx")
        rec(2)
        L.check(lib.kan_surface_backward(ctypes.byref(dprep), Pt(x), Pt(C), Pt(dy), None, Pt(dC), Pt(wsb), nb, S),
                "backward dC")
        rec(3)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    per_step = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        events = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        per_step.append(events)
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stage_ms = {nm: sum(ev[k].elapsed_time(ev[k + 1]) for ev in per_step) / args.steps
                for k, nm in enumerate(names)}
    ms_per_step = 1e3 * elapsed / args.steps
    step_ms = sorted(ev[0].elapsed_time(ev[3]) for ev in per_step)
    median_ms = step_ms[len(step_ms) // 2]
    # algorithmic: the 16 non-zero products per (row, pair) in each of the
    # three contractions; executed: all (G+3)^2 columns of a pair
    alg_one = 2.0 * N * O * P * 16
    exe_one = 2.0 * N * O * P * K1 * K1
    dom = max(names, key=lambda nm: stage_ms[nm])
    peak = PEAK_TFLOPS[d["dtype"]]
    t_dom = stage_ms[dom] * 1e-3
    roof = {"bound": "mfma", "kernel": dom, "achieved": alg_one / t_dom / 1e12, "peak": peak,
            "unit": "TFLOP/s", "frac": alg_one / t_dom / 1e12 / peak,
            "traffic": read_traffic(args.workload, dom.split(".")[1]),
            "executed_achieved": exe_one / t_dom / 1e12, "executed_frac": exe_one / t_dom / 1e12 / peak,
            "dominant_ms": stage_ms[dom],
            "stage_executed_TFLOPs": {nm: exe_one / (stage_ms[nm] * 1e-3) / 1e12 for nm in names}}
    out = {
        "metric": SURFACE_METRIC,
        "value": N * 1e3 / ms_per_step,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "median_ms_per_step": median_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": d["dtype"],
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "name": args.workload, "rows": N, "pairs": P,
                   "outputs": O, "G": G},
        "gflops_algorithmic": 3 * alg_one / (ms_per_step * 1e-3) / 1e9,
        "gflops_executed": 3 * exe_one / (ms_per_step * 1e-3) / 1e9,
        "stage_ms": stage_ms,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = surface_cpu_baseline(d, args.cpu_rows)
    print(json.dumps(out))


def surface_cpu_baseline(d, rows=None):
    """The float64 NumPy oracle of the 2-D layer on a bounded sample of rows:
    y, dx and the rows' own dC contributions, timed on the host."""
    import oracle
    import workloads as wl
    N = d["N"]
    n = min(N, rows or 256)
    R = wl.sample_indices(N, n, 97)
    x, dy = d["x"][R].astype("float64"), d["dy"][R].astype("float64")
    t0 = time.perf_counter()
    oracle.surface_forward(x, d["C"], d["lo"], d["hi"], d["G"])
    oracle.surface_backward(x, d["C"], dy, d["lo"], d["hi"], d["G"])
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "rows/s", "cores": _cpu_threads(), "kind": "oracle",
            "sample": "%d of %d rows: forward, dx and the rows' own dC contributions in float64 "
                      "NumPy, %.1f s; CPU %s" % (n, N, dt, _cpu_model())}


def grouped_cpu_baseline(d, rows=None):
    """The float64 NumPy oracle of the grouped activation on a bounded sample
    of rows: y, dx and the rows' own dC contributions, timed on the host."""
    import oracle
    import workloads as wl
    N, I = d["N"], d["I"]
    n = min(N, rows or 4096)
    R = wl.sample_indices(N, n, 98)
    x, dy = d["x"][R].astype("float64"), d["dy"][R].astype("float64")
    t0 = time.perf_counter()
    oracle.grouped_forward(x, d["C"], d["lo"], d["hi"], d["G"])
    oracle.grouped_backward(x, d["C"], dy, d["lo"], d["hi"], d["G"])
    dt = time.perf_counter() - t0
    return {"value": n * I / dt, "unit": "elements/s", "cores": _cpu_threads(), "kind": "oracle",
            "sample": "%d of %d rows (%d elements): forward, dx and the rows' own dC contributions "
                      "in float64 NumPy, %.1f s; CPU %s" % (n, N, n * I, dt, _cpu_model())}


def _cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def kernel_code_digest(files=MFMA_FILES):
    """sha256 of a kernel family's source (the kernel file, the headers it
    includes and the launch planner) with // comments and blank lines
    removed: a counter summary stays valid across comment edits and goes stale
    with any change to the code."""
    import re
    csrc = os.path.join(ROOT, "kolmogorov_arnold_network_amd", "csrc")
    lines = []
    for name in files:
        lines += [re.sub(r"//.*", "", l).rstrip() for l in open(os.path.join(csrc, name)).read().splitlines()]
    return hashlib.sha256("\n".join(l for l in lines if l).encode()).hexdigest()


def read_traffic(workload, kernel, files=MFMA_FILES):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("code_sha256") != kernel_code_digest(files):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# rows per oracle sample: the sizes the parity tests check each workload on
# (c1, c2: every row; c3: 512; c4: 256; c5: 128)
SAMPLE_ROWS = {"c1": 32, "c2": 1024, "c3": 512, "c4": 256, "c5": 128}


def cpu_baseline(d, rows=None, budget_s=10.0):
    """The float64 NumPy oracle on bounded samples of the same workload: y, dx
    and the sample rows' own dC / dW_base contributions, timed on the host.
    Seeded subsets of the parity sample size are run one after another until
    about ``budget_s`` seconds have passed, with BLAS on every host thread;
    then one subset again with BLAS on a single thread."""
    import oracle
    import workloads as wl
    from threadpoolctl import threadpool_limits
    N = d["N"]
    n = min(N, rows or SAMPLE_ROWS[d["name"]])
    lo, hi, G = d["lo"], d["hi"], d["G"]
    bf = d["dtype"] == "bf16"
    k = d["layers"][0][0].shape[2] - G                     # spline degree

    def one(seed):
        R = wl.sample_indices(N, n, seed)
        t0 = time.perf_counter()
        acts = oracle.network_forward(d["x"][R], d["layers"], lo, hi, G, bf16_between=bf, k=k)
        oracle.network_backward(acts, d["layers"], d["dy"][R], lo, hi, G, k=k)
        return time.perf_counter() - t0

    cores = _cpu_threads()
    total, reps = 0.0, 0
    while reps == 0 or (total < budget_s and reps < 64):
        total += one(99 + reps)
        reps += 1
    with threadpool_limits(limits=1):
        t1 = one(99)
    model = _cpu_model()
    return {"value": reps * n / total, "unit": "rows/s", "cores": cores, "kind": "oracle",
            "single_core_value": n / t1,
            "sample": "%d seeded subset(s) of %d of %d rows (forward and backward: dx, and the rows' own "
                      "dC/dW_base contributions) in float64 NumPy, %.1f s on %d threads; one subset on 1 "
                      "thread, %.1f s; CPU %s" % (reps, n, N, total, cores, t1, model)}


if __name__ == "__main__":
    main()
