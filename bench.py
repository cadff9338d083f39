"""Throughput of one MatRIS-MoE interaction block (forward + force VJP) on one
MI355X, in atoms/s, with the roofline position of the dominant kernel and the
CPU oracle timed beside it.

One step = the whole path on one batch of synthetic structures: periodic
radius graph, edge embedding + aggregation, element-routed MoE (dispatch,
expert GEMMs, combine), readout, and the input gradient (expert GEMMs
transposed, aggregation transposed, edge/force part).  Inputs are resident in
HBM before the timed region starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config S]
                    [--block core|full|stack|train|full-train|stack-train]

``--block full`` times the complete block instead (Tri -> MoE0 -> neighbour
multi-head attention -> MoE1 -> readout, and its input gradient);
``--block stack`` times a model of ``--blocks`` complete blocks on one graph
(element embedding, the blocks, readout, forces and stress through all of
them), with the block weights drawn on the GPU from a seeded generator.
``--block train`` times one training step of the block: forward, forces, and
the parameter gradients of a loss on energies and forces (forward tangents
and the tangent of the input gradient), for seeded loss upstreams dL/dE and
dL/dF; ``--block full-train`` the same for the complete block and
``--block stack-train`` for the stack of ``--blocks`` complete blocks (all
parameter gradients, the element embedding's included).

Prints ONE JSON line.  ``--calibrate-copy`` instead runs a plain 1 GiB device
copy (for scaling hardware byte counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "atoms/s per interaction block (fwd+force VJP) on 1 MI355X; % HBM/MFMA roofline"
TRAIN_METRIC = ("atoms/s per interaction-block training step (fwd, forces, energy+force loss "
                "parameter gradients) on 1 MI355X")
MFMA_FP32_PEAK_TFLOPS = 157.3      # MI355X dense FP32 matrix peak
HBM_PEAK_GBS = 8000.0
# Unpacked FP32 vector peak: 256 CUs x 4 SIMDs x 16 lanes x 2 FLOP (FMA) x 2.4 GHz.  The
# 157.3 TFLOP/s vector figure counts packed FP32 (two lanes per instruction), which this
# library does not generate.
VALU_FP32_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
EXPERT_CLASSES = ("gemm_expert_up", "gemm_expert_down", "gemm_expert_vjp_down", "gemm_expert_vjp_up",
                  "gemm_expert_pair")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_expert_traffic_S.txt")


def _kernel_source_hash() -> str:
    p = os.path.join(ROOT, "element_routed_moe_amd", "csrc", "gemm.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def _traffic(kernel: str):
    """Bytes per launch from the committed hardware-counter summary, if it was
    taken on the current kernel source (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("gemm_source_sha256_16") != _kernel_source_hash():
        return None
    v = kv.get(f"{kernel}_bytes_per_launch")
    return float(v) if v else None


def calibrate_copy():
    import torch
    n = 1 << 28                       # 2^28 floats = 1 GiB
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 3}))


def host_cpu():
    """The host's CPUs as this process sees them: usable cores and the model name."""
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return ncpu, model


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        return 1


def cpu_baseline(cfg, inp, n_structs: int, full: bool = False):
    """The float64 NumPy oracle on the first n_structs structures of the workload."""
    import numpy as np
    from oracle import attention as OA
    from oracle import block as OB
    from oracle import graph as OG
    threads = blas_threads()
    ncpu, model = host_cpu()
    n = int(inp["struct_ptr"][n_structs])
    sub = dict(inp)
    sub["pos"] = inp["pos"][:n]
    sub["cell"] = inp["cell"][:n_structs]
    sub["struct_ptr"] = inp["struct_ptr"][:n_structs + 1]
    sub["z"] = inp["z"][:n]
    sub["h"] = inp["h"][:n]
    g_up = np.broadcast_to(inp["w_r"], (n, cfg.d_node)).astype(np.float64)
    t0 = time.perf_counter()
    gr = OG.radius_graph(sub["pos"], sub["cell"], sub["struct_ptr"], sub["cutoff"])
    if full:
        f = OA.full_block_forward(sub, gr)
        OA.full_block_vjp(sub, gr, f, g_up)
    else:
        f = OB.block_forward(sub, gr)
        OB.block_vjp(sub, gr, f, g_up)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "atoms/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n_structs} of {cfg.n_structs} structures ({n} atoms, "
                      f"{gr['src'].size} edges) of the {cfg.name} workload, float64 NumPy oracle"
                      f"{' of the complete block' if full else ''}, graph + forward + VJP in "
                      f"{dt:.2f} s",
            "host_cpus": ncpu, "cpu_model": model, "blas_threads": int(threads),
            "threads_note": "cores = the BLAS pool that runs the oracle's matrix products; its "
                            "scatter-adds (np.add.at), routing loop and graph loops run on one "
                            "thread"}


def cpu_baseline_train(cfg, inp, n_structs: int, Ebar, Fbar):
    """The float64 autograd oracle of the training gradient on the first n_structs structures."""
    import numpy as np
    import torch
    from oracle import graph as OG
    from oracle import train as TR
    n = int(inp["struct_ptr"][n_structs])
    sub = dict(inp)
    sub["pos"], sub["z"], sub["h"] = inp["pos"][:n], inp["z"][:n], inp["h"][:n]
    sub["cell"], sub["struct_ptr"] = inp["cell"][:n_structs], inp["struct_ptr"][:n_structs + 1]
    t0 = time.perf_counter()
    gr = OG.radius_graph(sub["pos"], sub["cell"], sub["struct_ptr"], sub["cutoff"])
    TR.loss_grads(sub, gr, np.asarray(Ebar[:n_structs], np.float64), np.asarray(Fbar[:n], np.float64))
    dt = time.perf_counter() - t0
    ncpu, model = host_cpu()
    return {"value": n / dt, "unit": "atoms/s", "cores": int(torch.get_num_threads()), "kind": "oracle",
            "host_cpus": ncpu, "cpu_model": model,
            "sample": f"first {n_structs} of {cfg.n_structs} structures ({n} atoms, {gr['src'].size} "
                      f"edges) of the {cfg.name} workload, float64 PyTorch-autograd oracle of the "
                      f"training gradient (graph, energy, forces, all parameter gradients) in {dt:.2f} s"}


def memory_kernel_fractions(cfg, E, kernel_ms):
    """Position of the core block's memory- and vector-bound kernels against their rooflines,
    from the per-class times of the breakdown steps (ms per step).

    Algorithmic work per step (N atoms, E edges, k experts per atom):
      combine (forward + VJP, 2 launches): reads k expert rows + u, writes h', per atom:
        2 x (k + 2) x 4 Dn bytes;
      embed_aggregate (1 launch): 16 basis FMAs + 1 modulating FMA per edge and channel,
        2 x 17 x E x De FLOP; HBM: 20 B of geometry and index per edge, the s row read
        (the gathered s rows counted once) and the a row written per atom (8 De B);
      edge_vjp (1 launch): about 41 FMA per edge and channel (e and de/dr rebuilt from the 16
        radial terms, the sender gradient, the edge scalar), 2 x 41 x E x De FLOP; HBM:
        20 B per edge, abar and s read and sbar written per atom (12 De B);
      route_dispatch (route + dispatch kernels): z read, tok_atom and slot written,
        (4 + 8 k) N bytes (latency-bound: the fraction only shows how far from HBM it is).
    """
    N, k, De, Dn = cfg.n_atoms, cfg.top_k, cfg.d_edge, cfg.d_node
    res = {}

    def hbm(name, nbytes):
        ms = kernel_ms.get(name)
        if not ms:
            return
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"bound": "hbm", "bytes_per_step": int(nbytes), "ms_per_step": ms,
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4)}

    def valu(name, flop, nbytes):
        ms = kernel_ms.get(name)
        if not ms:
            return
        tf = flop / (ms * 1e-3) / 1e12
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"bound": "alu", "flop_per_step": flop, "ms_per_step": ms,
                     "achieved": round(tf, 2), "peak": round(VALU_FP32_PEAK_TFLOPS, 2),
                     "unit": "TFLOP/s", "frac": round(tf / VALU_FP32_PEAK_TFLOPS, 4),
                     "hbm_bytes_per_step": int(nbytes), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}

    hbm("combine", 2 * (k + 2) * 4.0 * Dn * N)
    hbm("route_dispatch", (4 + 8 * k) * float(N))
    valu("embed_aggregate", 2.0 * 17 * E * De, 20.0 * E + 8.0 * De * N)
    valu("edge_vjp", 2.0 * 41 * E * De, 20.0 * E + 12.0 * De * N)
    res["note"] = ("alu peak = unpacked FP32 vector rate (256 CUs x 4 SIMD x 16 lanes x 2 FLOP x "
                   "2.4 GHz); times from the breakdown steps")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="S")
    ap.add_argument("--block", choices=("core", "full", "stack", "train", "full-train", "stack-train"),
                    default="core")
    ap.add_argument("--blocks", type=int, default=6)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-structs", type=int, default=32)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--breakdown-steps", type=int, default=3,
                    help="untimed steps after the timed ones, with every kernel launch timed, for "
                         "kernel_ms_per_step")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the block has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return

    import numpy as np
    import torch
    from element_routed_moe_amd import mlip, synth

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    cfg = synth.CONFIGS[args.config]
    train = args.block.endswith("train")
    full = args.block in ("full", "full-train")
    stack = args.block in ("stack", "stack-train")
    if train:
        # seeded loss upstreams: dL/dE ~ N(0,1) per structure, dL/dF ~ N(0,1) per component
        rng = np.random.default_rng(41)
        Ebar_h = rng.standard_normal(cfg.n_structs)
        Fbar_h = rng.standard_normal((cfg.n_atoms, 3)).astype(np.float32)
        Ebar = torch.tensor(Ebar_h, dtype=torch.float64, device="cuda")
        Fbar = torch.from_numpy(Fbar_h).to("cuda")
    if stack:
        shared, _ = synth.make_stack_inputs(cfg, 0)
        params = synth.device_stack_params(cfg, args.blocks, "cuda")
        blk = mlip.Stack(shared, params, device="cuda", train=train)
        inputs = shared
    elif train and not full:
        inputs = synth.make_inputs(cfg)
        blk = mlip.Block(inputs, device="cuda", train=True)
    else:
        inputs = synth.make_full_inputs(cfg) if full else synth.make_inputs(cfg)
        blk = (mlip.FullBlock(inputs, device="cuda", train=train) if full
               else mlip.Block(inputs, device="cuda"))

    def one_step():
        blk.step()
        if train:
            blk.train_grad(Ebar, Fbar)

    log(f"inputs resident for workload {cfg.name}: {cfg.n_atoms} atoms")
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    E = blk.graph["n_edges"]
    log(f"warmup done ({args.warmup} steps, {E} edges)")

    # In the timed steps only the matrix-core GEMM classes (the roofline's candidates) are bracketed
    # by HIP events: every timed launch costs two event records, which added about 0.13 ms to an
    # S step when all launches were timed.
    mlip.profile_reset()
    mlip.profile_select(EXPERT_CLASSES + ("gemm_expert_tan", "gemm_wgrad"))
    mlip.profile_enable(True)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        one_step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mlip.profile_enable(False)
    prof = mlip.profile_read()
    # per-class breakdown from extra, untimed steps with every launch timed, read step by step;
    # each class reports the median over the steps, so one disturbed step does not move it
    breakdown_steps = max(args.breakdown_steps, 0)
    mlip.profile_select(None)
    per_step = []
    for _ in range(breakdown_steps):
        mlip.profile_reset()
        mlip.profile_enable(True)
        one_step()
        torch.cuda.synchronize()
        mlip.profile_enable(False)
        per_step.append(mlip.profile_read())
    mlip.profile_reset()

    ms_per_step = wall * 1e3 / args.steps
    N = cfg.n_atoms
    value = N * args.steps / wall

    # the same step on the previous step's graph, as a model of several blocks reuses one graph
    nog_steps = 0 if train else args.steps
    nog_ms = None
    if nog_steps:
        blk.step(build_graph=False)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(nog_steps):
            blk.step(build_graph=False)
        torch.cuda.synchronize()
        nog_ms = (time.perf_counter() - t1) * 1e3 / nog_steps

    # dominant kernel: the matrix-core class with the largest summed time
    # (with --block full each class has two launches per step, one per MoE layer).
    # Algorithmic flops per launch: 2 M Dn H for every expert GEMM (M = N k
    # tokens); a training step's weight gradients are priced per step:
    # d W1 and d W2 each 2 terms x 2 M Dn H, d W_u and d W_d each 2 x 2 N De Dn.
    k = cfg.top_k
    Mtok = N * k
    flops = {c: 2.0 * Mtok * cfg.d_node * cfg.d_hidden for c in EXPERT_CLASSES + ("gemm_expert_tan",)}
    # the forward's Y = silu(P) W2 and the gradient's Q = (g W2^T) silu'(P) in one launch
    flops["gemm_expert_pair"] = 2 * 2.0 * Mtok * cfg.d_node * cfg.d_hidden
    Dn, H, Da = cfg.d_node, cfg.d_hidden, cfg.d_attn
    moe_wgrad = 2 * (2 * 2.0 * Mtok * Dn * H)                    # d W1, d W2: two terms each
    if full or stack:
        # per complete block: both MoE layers, W_qkv and W_o (two terms), W_T (two terms) and
        # W_s (one term when the block's input does not move, i.e. the first block)
        blk_w = 2 * moe_wgrad + 2 * 2.0 * N * Dn * 3 * Da + 2 * 2.0 * N * Da * Dn + 2 * 2.0 * N * Da * Dn
        nb = args.blocks if stack else 1
        wgrad_step = nb * (blk_w + 2.0 * N * Dn * Da) + (nb - 1) * 2.0 * N * Dn * Da
    else:
        wgrad_step = moe_wgrad + 2 * (2 * 2.0 * N * cfg.d_edge * Dn)
    classes = [c for c in flops if c in prof and prof[c]["launches"]]
    if "gemm_wgrad" in prof and prof["gemm_wgrad"]["launches"]:
        classes.append("gemm_wgrad")
        flops["gemm_wgrad"] = wgrad_step / (prof["gemm_wgrad"]["launches"] / args.steps)
    dom = max(classes, key=lambda c: prof[c]["total_ms"])
    avg_ms = prof[dom]["total_ms"] / max(prof[dom]["launches"], 1)
    achieved = flops[dom] / (avg_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
            "peak": MFMA_FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_FP32_PEAK_TFLOPS, 4),
            # the counters were taken on the core step of the S workload only
            "traffic": (_traffic(dom) if dom in EXPERT_CLASSES and args.config == "S" and args.block == "core"
                        else None),
            "avg_launch_ms": round(avg_ms, 4), "flop_per_launch": flops[dom]}
    if dom == "gemm_wgrad":
        roof["flop_per_launch_note"] = "mean over the step's weight-gradient launches"

    kernel_ms = {}
    if per_step:
        for name in per_step[0]:
            if per_step[0][name]["launches"]:
                kernel_ms[name] = round(float(np.median([p[name]["total_ms"] for p in per_step])), 4)
    out = {
        "metric": TRAIN_METRIC if train else METRIC, "value": round(value, 1), "unit": "atoms/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "atoms": N, "edges": int(E), "structures": cfg.n_structs,
                   "cutoff": cfg.cutoff, "d_edge": cfg.d_edge, "d_node": cfg.d_node,
                   "d_hidden": cfg.d_hidden, "experts": cfg.n_experts, "top_k": k,
                   "element_types": cfg.n_types,
                   "block": (("Tri + MoE0 + neighbour attention + MoE1" if full else
                              f"{args.blocks} x (Tri + MoE0 + neighbour attention + MoE1)" if stack
                              else "aggregation + MoE") + (", training gradient" if train else ""))},
        "edges_per_s": round(E * args.steps / wall, 1),
        "event_ms_per_step": round(ev0.elapsed_time(ev1) / args.steps, 4),
        "kernel_ms_per_step": kernel_ms,
        "kernel_ms_per_step_note": f"median over {breakdown_steps} untimed steps after the timed ones, every "
                                   "launch timed; the timed steps time only the matrix-core GEMM classes",
        "roofline": roof,
    }
    if nog_ms is not None:
        out["ms_per_step_without_graph_build"] = round(nog_ms, 4)
    moe_tabs = [blk.moe] if not (full or stack) else ([blk.moe0, blk.moe] if full else [])
    if moe_tabs:
        loads = []
        for tab in moe_tabs:
            cnt = np.diff(tab["exp_off"].cpu().numpy().astype(np.int64))
            act = cnt[cnt > 0]
            loads.append({"max": int(cnt.max()), "mean_active": round(float(act.mean()), 1),
                          "min_active": int(act.min()), "active_experts": int(act.size),
                          "mean_all": round(float(cnt.mean()), 1)})
        out["expert_tokens"] = loads[0] if len(loads) == 1 else {"moe0": loads[0], "moe1": loads[1]}
    if args.block == "core" and breakdown_steps:
        out["memory_kernels"] = memory_kernel_fractions(cfg, E, kernel_ms)
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")
    if full or stack:
        out["config"]["heads"] = cfg.n_heads
        out["config"]["d_attn"] = cfg.d_attn
    if stack or (train and full):
        # the float64 oracle of these at S widths is beyond a bounded CPU sample (tens of GB of
        # float64 expert weights and gradients); the per-block baselines are in the other lines
        args.no_cpu_baseline = True
    if train and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_train(cfg, inputs, 1, Ebar_h, Fbar_h)
    elif not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inputs, min(args.cpu_structs, cfg.n_structs), full)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
