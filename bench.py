"""Benchmark of the MoE layer forward on one MI355X.

One step = one moe_forward (route -> slot assignment -> dispatch -> expert FFN ->
combine) over one batch of seeded synthetic tokens already resident in HBM.
Default workload: the DeepSeek-R1-shaped routed experts on one GPU holding all
of them (T=4096, H=7168, E=256, k=8, SwiGLU 7168->2048->7168, dropless,
softmax then top-8 renormalised, router bias N(0,1), bf16 activations and
weights, fp32 router): the largest workload that fits one GPU.

Prints one JSON line: the layer's tokens/s, per-stage times, the roofline of
the expert FFN (algorithmic bytes over its launch time against 8 TB/s, with
the rocprofv3 HBM byte counts when they match the current kernel source) and
the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/s + expert-GEMM % MFMA peak + route/dispatch % HBM BW"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # fp32 matrix
PEAK_F64_TFLOPS = 78.6         # fp64 (vector and matrix)

WORKLOADS = {
    "1": "switch-tiny-fp32-T256-H64-E4-k1-F128-relu-cf1.25",
    "2": "switch-top1-bf16-T16384-H768-E64-k1-F3072-gelu-cf1.0",
    "3a": "ds7508-top4-bf16-T32768-H512-E12-k4-F2048-gelu-cf1.0",
    "3b": "ds7508-top4-bf16-T32768-H512-E12-k4-F2048-gelu-cf0.5",
    "3c": "ds7508-top4-bf16-T32768-H512-E12-k4-F2048-gelu-cf0.25",
    "4": "mixtral-top2-bf16-T8192-H4096-E8-k2-F14336-swiglu-dropless",
    "5": "deepseek-top8-bf16-T4096-H7168-E256-k8-F2048-swiglu-dropless",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash():
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "top_routing_expert_router_amd", "csrc", "ffn.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload):
    """HBM bytes per step of the expert-FFN stage (all its grouped-GEMM launches) from the
    committed rocprofv3 PMC summary, if it was taken on the current expert-FFN source; else None."""
    path = os.path.join(ROOT, "profiles", f"expert_ffn_pmc_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("ffn_hip_sha256_16") != src_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_step_expert_stage"])
    except (KeyError, ValueError):
        return None


# workloads measured briefly next to the main one (layer time and expert-FFN roofline)
EXTRA_WORKLOADS = ("2", "4")

EXPERT_KERNEL = "grouped_gemm"
EPI_COMBINE1 = 4  # epilogue argument of the second GEMM that also does the top-1 combine
COPY_BYTES = 256 << 20


def _gemm_epilogue(name):
    """Epilogue template argument of a tiled grouped-GEMM kernel name, else None."""
    import re

    m = re.search(r"grouped_gemm_(pipe|ring)_kernel<([^>]*)>", name)
    if not m:
        return None
    args = [a.strip() for a in m.group(2).split(",")]
    try:
        return int(args[5] if m.group(1) == "pipe" else args[4])
    except (IndexError, ValueError):
        return None


def _stage_kernel(name):
    """A launch of the expert-FFN stage (the forward's combine-fused second GEMM is not)."""
    return EXPERT_KERNEL in name and _gemm_epilogue(name) != EPI_COMBINE1


def _kernel_rows(db_path):
    import sqlite3

    db = sqlite3.connect(db_path)
    return db.execute("select name, duration from kernels order by start").fetchall()


def summarize_trace(db_path, cmd):
    """Per-kernel duration summary of a rocprofv3 --kernel-trace database (text)."""
    import collections

    agg = collections.OrderedDict()
    for name, dur in _kernel_rows(db_path):
        a = agg.setdefault(name, [0, 0.0, float("inf"), 0.0])
        a[0] += 1
        a[1] += dur
        a[2] = min(a[2], dur)
        a[3] = max(a[3], dur)
    total = sum(v[1] for v in agg.values())
    print(f"# rocprofv3 kernel-trace summary\n# command: {cmd}\n# durations in microseconds")
    print(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'share':>7}  kernel")
    for name, (c, t, mn, mx) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        print(f"{c:6d} {t / c / 1e3:10.2f} {mn / 1e3:10.2f} {mx / 1e3:10.2f} {100 * t / total:6.1f}%  {name[:110]}")


def summarize_pmc(fetch_db, write_db, workload, cmd):
    """HBM bytes of the expert-FFN kernels from FETCH_SIZE / WRITE_SIZE runs, each scaled by
    what the same counter reads for the plain device copy of COPY_BYTES run in that process."""
    import sqlite3

    def per_kernel(db_path, counter):
        db = sqlite3.connect(db_path)
        rows = db.execute("select name, counter_value from pmc_events where counter_name = ?", (counter,)).fetchall()
        out = {}
        for n, v in rows:
            out.setdefault(n, []).append(v)
        return out

    f = per_kernel(fetch_db, "FETCH_SIZE")
    w = per_kernel(write_db, "WRITE_SIZE")

    def copy_kib(d):
        vals = [v for n, vs in d.items() if "copy" in n.lower() or "elementwise" in n.lower() for v in vs
                if v * 1024 > COPY_BYTES / 8]
        return sorted(vals)[len(vals) // 2] if vals else None

    cf, cw = copy_kib(f), copy_kib(w)
    sf = COPY_BYTES / (cf * 1024) if cf else 1.0
    sw = COPY_BYTES / (cw * 1024) if cw else 1.0
    print(f"# rocprofv3 PMC summary: HBM bytes of the expert FFN launches\n# command: {cmd}")
    print(f"workload: {workload}")
    print(f"ffn_hip_sha256_16: {src_hash()}")
    print(f"copy_kernel_bytes: {COPY_BYTES}")
    print(f"fetch_scale_from_copy: {sf:.4f}   # copy reads {COPY_BYTES} B; FETCH_SIZE read {cf} KiB")
    print(f"write_scale_from_copy: {sw:.4f}   # copy writes {COPY_BYTES} B; WRITE_SIZE read {cw} KiB")
    tot = 0.0
    for n in sorted(set(f) | set(w)):
        if not _stage_kernel(n):
            continue
        fb = sum(f.get(n, [0])) / max(len(f.get(n, [1])), 1) * 1024 * sf
        wb = sum(w.get(n, [0])) / max(len(w.get(n, [1])), 1) * 1024 * sw
        tot += fb + wb
        print(f"kernel: {n[:90]}  read_bytes_per_launch: {fb:.4g}  write_bytes_per_launch: {wb:.4g}")
    print(f"hbm_bytes_per_step_expert_stage: {tot:.6g}")
    print("# the other kernels of the same runs (route, slot assignment, combine, the forward's second GEMM\n"
          "# with the top-1 combine folded in), bytes per launch")
    for n in sorted(set(f) | set(w)):
        if _stage_kernel(n) or "copy" in n.lower() or "elementwise" in n.lower():
            continue
        fb = sum(f.get(n, [0])) / max(len(f.get(n, [1])), 1) * 1024 * sf
        wb = sum(w.get(n, [0])) / max(len(w.get(n, [1])), 1) * 1024 * sw
        print(f"other_kernel: {n[:90]}  read_bytes_per_launch: {fb:.4g}  write_bytes_per_launch: {wb:.4g}")


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")


def summarize_mfma(db_path, workload, cmd, cus=256):
    """Matrix-core work of the grouped-GEMM launches from a rocprofv3 --pmc run of MFMA_COUNTERS.
    Each counter arrives as one row per hardware instance of a dispatch: the SQ counters are
    summed over the instances, GRBM_GUI_ACTIVE (the dispatch's active cycles, per instance)
    taken at its largest.  SQ_INSTS_VALU_MFMA_MOPS_BF16 counts units of 512 bf16 flops; the busy
    share is SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x CUs x 4 SIMDs.  Averages per launch."""
    import sqlite3

    db = sqlite3.connect(db_path)
    rows = db.execute("select dispatch_id, name, counter_name, counter_value, duration from pmc_events").fetchall()
    disp = {}
    for d, n, c, v, dur in rows:
        if EXPERT_KERNEL not in n:
            continue
        e = disp.setdefault(d, {"name": n, "dur": dur, "c": {}})
        if c == "GRBM_GUI_ACTIVE":
            e["c"][c] = max(e["c"].get(c, 0.0), v)
        else:
            e["c"][c] = e["c"].get(c, 0.0) + v
    per = {}
    for e in disp.values():
        per.setdefault(e["name"], []).append(e)
    print(f"# rocprofv3 PMC summary: matrix-core work of the grouped-GEMM launches\n# command: {cmd}")
    print(f"workload: {workload}")
    print(f"ffn_hip_sha256_16: {src_hash()}")
    for n in sorted(per):
        es = per[n]
        avg = lambda c: sum(e["c"].get(c, 0.0) for e in es) / len(es)
        flops = avg("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512
        gui = avg("GRBM_GUI_ACTIVE")
        busy = avg("SQ_VALU_MFMA_BUSY_CYCLES") / (gui * cus * 4) if gui else float("nan")
        dur_us = sum(e["dur"] for e in es) / len(es) / 1e3
        print(f"kernel: {n[:90]}  launches: {len(es)}  mfma_flops_per_launch: {flops:.4g}  "
              f"mfma_busy_frac: {busy:.4f}  gui_active_cycles: {gui:.4g}  us_under_counters: {dur_us:.1f}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="5", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the layer captured in a HIP graph instead of eager moe_forward calls")
    ap.add_argument("--no-extra", action="store_true", help="skip the brief runs of the other workloads")
    ap.add_argument("--core-only", action="store_true",
                    help="skip the extra measurements (for profiler runs: only the routed layer's launches)")
    ap.add_argument("--backward-only", action="store_true",
                    help="route once, then time moe_backward alone (--steps calls after one warm-up call)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain device copy of 256 MiB (the PMC byte-counter calibration)")
    ap.add_argument("--summarize-trace", metavar="DB", help="print the kernel summary of a rocprofv3 database")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="print expert-FFN HBM bytes from FETCH_SIZE / WRITE_SIZE rocprofv3 databases")
    ap.add_argument("--summarize-mfma", metavar="DB",
                    help="print the grouped-GEMM matrix-core counters of a rocprofv3 --pmc database")
    ap.add_argument("--cmd", default="", help="command line to record in a summary")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.cmd)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, WORKLOADS[args.config], args.cmd)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, WORKLOADS[args.config], args.cmd)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: the expert-parallel path across GPUs is designed, not built",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    from top_routing_expert_router_amd import binding as B
    from top_routing_expert_router_amd.synth import recipes

    run = recipes.RUNS[args.config]
    workload = WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    B.lib()  # fail loudly if the library is not built
    cfg = B.MoEConfig.from_run(run)
    bf16 = run.dtype == recipes.BF16
    tdt = torch.bfloat16 if bf16 else torch.float32
    eb = run.elem_bytes

    def up(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    t0 = time.time()
    x_h = recipes.gen_x(run)
    wg_h, bias_h = recipes.gen_router(run)
    def upload(which):
        out_f, in_f = (run.F, run.H) if which in ("w1", "w3") else (run.H, run.F)
        w = torch.empty((run.E, out_f, in_f), dtype=tdt, device=dev)
        per = max(1, (1 << 26) // (out_f * in_f))
        for e0 in range(0, run.E, per):
            es = list(range(e0, min(run.E, e0 + per)))
            p = recipes.gen_expert_weight(run, which, experts=es)
            blk = np.stack([p[e] for e in es])
            hb = torch.from_numpy(blk.view(np.int16)).view(torch.bfloat16) if blk.dtype == np.uint16 \
                else torch.from_numpy(blk)
            w[e0:e0 + len(es)].copy_(hb)
        return w

    x = up(x_h)
    wg, bias = up(wg_h), up(bias_h)
    w1 = upload("w1")
    w3 = upload("w3") if run.act == recipes.SWIGLU else None
    w2 = upload("w2")
    rmax = B.max_rows(cfg)
    plan = B.alloc_plan(cfg, dev)
    X = torch.empty((max(rmax, 1), run.H), dtype=tdt, device=dev)
    Y = torch.empty_like(X)
    y = torch.empty((run.T, run.H), dtype=tdt, device=dev)
    ws = B.alloc_workspace(cfg, dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s: {workload}, R_max={rmax}, ws={ws.numel() / 2**20:.1f} MiB")

    if args.backward_only:
        out = measure_backward(run, cfg, dev, up, x, wg, bias, w1, w3, w2, plan, ws, max(1, args.steps))
        print(json.dumps({"workload": workload, "backward": out}), flush=True)
        return

    def step():
        B.forward(cfg, x, wg, bias, w1, w3, w2, x, y, plan, X, Y, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- with --graph the layer's launches are captured once in a HIP graph and a
    # step is one replay (the same kernels on the same buffers; nothing the
    # library enqueues is a memset or an allocation).  Default: eager calls.
    graph = None
    if args.graph:
        try:
            gs = torch.cuda.Stream()
            gs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(gs):
                step()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=gs):
                step()
            torch.cuda.synchronize()
        except Exception as exc:  # capture unavailable: eager steps
            log(f"[bench] graph capture failed ({exc}); timing eager steps")
            graph = None
    run_step = graph.replay if graph is not None else step
    for _ in range(args.warmup):  # warm-up of the timed form as well (first replays upload the graph)
        run_step()

    def time_steps(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # ---- timed region: K whole-layer steps, back to back on one stream
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        run_step()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    ms_eager = time_steps(step) if graph is not None else ms_per_step
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step ({'graph replay' if graph else 'eager'})")

    # ---- per-step spread: the same K steps with an event between steps (no syncs)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(args.steps):
        run_step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    ms_median = per_step[len(per_step) // 2]

    # ---- per-stage durations: each stage entry point called K times back to back
    # (the plan and buffers of this batch stay valid across repeats), HIP events
    # recorded on the stream the kernels run on (torch's current stream)
    def timed(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps * 1e3

    stage_us = {
        "route": timed(lambda: B.route(cfg, x, wg, bias, plan, ws)),
        "dispatch": timed(lambda: B.dispatch(cfg, x, plan, X)),
        "expert_ffn": timed(lambda: B.expert_ffn(cfg, X, plan, w1, w3, w2, Y, ws)),
        "combine": timed(lambda: B.combine(cfg, Y, plan, x, y)),
    }

    # Extra measurements (cold stages, training terms, routing variants, shared
    # expert) are skipped with --core-only, which the profiler runs use so that
    # every launch they record belongs to the routed layer.
    stage_cold_us, losses_us, variants, shared_out, cold_sets, backward_out = None, None, None, None, None, None
    if not args.core_only:
        # cold: the stage runs back to back over rotating copies of its buffers, as many
        # sets as make 1 GiB of traffic per rotation (four times the 256 MB Infinity
        # Cache), so every call reads inputs that have left every cache while the GPU
        # stays busy (no idle-launch gap in the timed region)
        def timed_rotating(make_set, call, bytes_per_call):
            nsets = max(2, -(-(1 << 30) // max(int(bytes_per_call), 1)))
            sets = [make_set() for _ in range(nsets)]
            torch.cuda.synchronize()
            for st in sets:  # touch every set once
                call(*st)
            reps = max(2, args.steps // nsets + 1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                for st in sets:
                    call(*st)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / (reps * nsets) * 1e3
            del sets
            return us, nsets

        kept_now = plan["kept"].cpu().numpy()
        R_now = int(kept_now.sum())
        xb = run.T * run.H * eb
        cold_disp, ns_d = timed_rotating(lambda: (x.clone(), torch.empty_like(X)),
                                         lambda xs, Xs: B.dispatch(cfg, xs, plan, Xs), xb + R_now * run.H * eb)
        cold_comb, ns_c = timed_rotating(lambda: (Y.clone(), x.clone(), torch.empty_like(y)),
                                         lambda Ys, rs, ys: B.combine(cfg, Ys, plan, rs, ys),
                                         R_now * run.H * eb + 2 * xb)
        cold_route, ns_r = timed_rotating(lambda: (x.clone(),), lambda xs: B.route(cfg, xs, wg, bias, plan, ws),
                                          xb)
        stage_cold_us = {"route": cold_route, "dispatch": cold_disp, "combine": cold_comb}
        cold_sets = {"route": ns_r, "dispatch": ns_d, "combine": ns_c}

        # ---- router training terms (load-balancing loss, z-loss): route with the
        # optional losses output, against route without it
        plan_l = dict(plan)
        plan_l["losses"] = torch.empty(2, dtype=torch.float64, device=dev)
        losses_us = {"route_us": round(stage_us["route"], 2),
                     "route_with_losses_us": round(timed(lambda: B.route(cfg, x, wg, bias, plan_l, ws)), 2),
                     "losses": [float(v) for v in plan_l["losses"].cpu().tolist()]}

        # ---- routing variants: "probs" drop policy and sigmoid scores, route alone
        def route_time(c):
            ws_c = B.alloc_workspace(c, dev)
            plan_c = B.alloc_plan(c, dev)
            B.route(c, x, wg, bias, plan_c, ws_c)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(args.steps):
                B.route(c, x, wg, bias, plan_c, ws_c)
            e1.record()
            torch.cuda.synchronize()
            return round(e0.elapsed_time(e1) / args.steps * 1e3, 2), int(plan_c["n_dropped"].item())

        # ---- shared expert (one dense FFN of the routed experts' width on every token,
        # added to the routed output): the layer with it, and its FFN alone
        cfg_s = B.MoEConfig.from_run(run)
        cfg_s.shared_F = run.F
        sws = [up(recipes.gen_shared_weight(run, n, run.F)) if (n != "s3" or run.act == recipes.SWIGLU) else None
               for n in ("s1", "s3", "s2")]
        ws_s = B.alloc_workspace(cfg_s, dev)
        Ys = torch.empty((run.T, run.H), dtype=tdt, device=dev)
        fwd_s_us = timed(lambda: B.forward_shared(cfg_s, x, wg, bias, w1, w3, w2, *sws, x, y, plan, X, Y, ws_s))
        shared_ffn_us = timed(lambda: B.shared_expert(cfg_s, x, *sws, Ys, ws_s))
        shared_flops = 2.0 * run.T * run.H * run.F * run.m
        shared_out = {"workload": workload + f"+shared-F{run.F}", "ms_per_step": round(fwd_s_us / 1e3, 5),
                      "tokens_per_s": round(run.T / (fwd_s_us * 1e-6), 1), "shared_ffn_us": round(shared_ffn_us, 2),
                      "shared_ffn_tflops": round(shared_flops / (shared_ffn_us * 1e-6) / 1e12, 1)}
        del ws_s, Ys, sws

        backward_out = measure_backward(run, cfg, dev, up, x, wg, bias, w1, w3, w2, plan, ws,
                                        max(2, min(args.steps, 10)))

        variants = {}
        for name, kw in (("position", {}), ("probs", {"drop_policy": 1}), ("sigmoid", {"score_fn": 1})):
            c = B.MoEConfig.from_run(run)
            for key, val in kw.items():
                setattr(c, key, val)
            us, nd = route_time(c)
            variants[name] = {"route_us": us, "dropped": nd}

    log("[bench] stages (us): " + ", ".join(f"{s}={v:.1f}" for s, v in stage_us.items()))

    # ---- algorithmic work per step (from the plan of this batch)
    kept = plan["kept"].cpu().numpy()
    R = int(kept.sum())
    nonempty = int((kept > 0).sum())
    T, H, E, k, F, m = run.T, run.H, run.E, run.k, run.F, run.m
    ffn_flops = 2.0 * R * H * F * m
    ffn_bytes = nonempty * m * H * F * eb + 2.0 * R * H * eb
    route_bytes = T * H * eb + H * E * 4 + E * 4 + T * k * 12
    route_flops = 2.0 * T * H * E
    disp_bytes = T * H * eb + R * H * eb
    comb_bytes = R * H * eb + 2.0 * T * H * eb
    mfma_peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS

    def gbs(b, us):
        return b / (us * 1e-6) / 1e9

    t_ffn = stage_us["expert_ffn"]
    ffn_tflops = ffn_flops / (t_ffn * 1e-6) / 1e12
    ffn_gbs = gbs(ffn_bytes, t_ffn)
    t_mfma = ffn_flops / (mfma_peak * 1e12) * 1e6
    t_hbm = ffn_bytes / (PEAK_HBM_GBS * 1e9) * 1e6
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(ffn_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ffn_gbs / PEAK_HBM_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(ffn_tflops, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(ffn_tflops / mfma_peak, 4)}
    roof["traffic"] = read_traffic(workload)
    roof["kernel"] = "expert_ffn (grouped GEMM1 + GEMM2 launches)"
    roof["algorithmic_per_launch"] = {"flops": ffn_flops, "bytes": ffn_bytes}

    split_router = bf16 and H % 64 == 0
    if split_router:  # three bf16 pieces per router weight on the bf16 matrix cores
        route_roof_us = max(route_bytes / (PEAK_HBM_GBS * 1e3), 3 * route_flops / (PEAK_BF16_TFLOPS * 1e6))
        route_note = "split-bf16 router: roofline = max(bytes/HBM, 3 x 2THE / bf16 peak)"
    else:
        route_roof_us = max(route_bytes / (PEAK_HBM_GBS * 1e3), route_flops / (PEAK_F64_TFLOPS * 1e6))
        route_note = "binary64 router: roofline = max(bytes/HBM, 2THE / fp64 peak)"
    router_desc = ("fp32 logits: split-bf16 MFMA with a certified radius, binary64 recomputation of undecided "
                   "tokens" if split_router else "fp32 logits (binary64 accumulation)")
    stages_out = {
        "route": {"us": round(stage_us["route"], 2), "GB_s": round(gbs(route_bytes, stage_us["route"]), 1),
                  "hbm_frac": round(gbs(route_bytes, stage_us["route"]) / PEAK_HBM_GBS, 4),
                  "roofline_frac": round(route_roof_us / stage_us["route"], 4),
                  "note": route_note},
        "dispatch": {"us": round(stage_us["dispatch"], 2), "GB_s": round(gbs(disp_bytes, stage_us["dispatch"]), 1),
                     "hbm_frac": round(gbs(disp_bytes, stage_us["dispatch"]) / PEAK_HBM_GBS, 4)},
        "expert_ffn": {"us": round(t_ffn, 2), "TFLOP_s": round(ffn_tflops, 1),
                       "mfma_frac": round(ffn_tflops / mfma_peak, 4), "GB_s": round(ffn_gbs, 1),
                       "roofline_frac": round(max(t_mfma, t_hbm) / t_ffn, 4)},
        "combine": {"us": round(stage_us["combine"], 2), "GB_s": round(gbs(comb_bytes, stage_us["combine"]), 1),
                    "hbm_frac": round(gbs(comb_bytes, stage_us["combine"]) / PEAK_HBM_GBS, 4)},
    }
    if k == 1 and bf16 and H % 64 == 0 and F % 64 == 0:
        stages_out["combine"]["note"] = ("the stage entry point; moe_forward folds the top-1 combine into the second "
                                         "GEMM's epilogue on this shape")
    stages_cold = None
    if stage_cold_us is not None:
        cold_bytes = {"route": route_bytes, "dispatch": disp_bytes, "combine": comb_bytes}
        stages_cold = {n: {"us": round(v, 2), "GB_s": round(gbs(cold_bytes[n], v), 1),
                           "hbm_frac": round(gbs(cold_bytes[n], v) / PEAK_HBM_GBS, 4)}
                       for n, v in stage_cold_us.items()}
        stages_cold["note"] = ("back-to-back calls rotating over copies of the stage's buffers, "
                               f"{cold_sets} sets per rotation (>= 1 GiB of traffic, 4x the 256 MB Infinity "
                               "Cache): inputs come from HBM, no idle gaps")

    # ---- CPU baseline: the oracle on the machine's host cores, bounded sample
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(run, x_h, wg_h, bias_h, args.cpu_seconds)

    value = T / (ms_per_step * 1e-3)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_median": round(ms_median, 5),
        "ms_per_step_eager": round(ms_eager, 5),
        "launch": "HIP graph replay of moe_forward" if graph is not None else "eager moe_forward calls",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded SplitMix64/Box-Muller inputs, random-init weights)",
        "config": {"workload": workload, "T": T, "H": H, "E": E, "k": k, "F": F,
                   "act": ["relu", "gelu", "swiglu"][run.act],
                   "capacity": B.capacity(cfg), "R_kept": R, "dropped": T * k - R, "router": router_desc},
        "expert_gemm_tflops": round(ffn_tflops, 1),
        "expert_gemm_mfma_frac": round(ffn_tflops / mfma_peak, 4),
        "route_dispatch_hbm_frac": {"route": stages_out["route"]["hbm_frac"],
                                    "dispatch": stages_out["dispatch"]["hbm_frac"],
                                    "combine": stages_out["combine"]["hbm_frac"]},
        "stages": stages_out,
        "stages_cold": stages_cold,
        "router_training_terms": losses_us,
        "routing_variants": variants,
        "shared_expert": shared_out,
        "backward": backward_out,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if not args.core_only and not args.no_extra:
        out["extra_workloads"] = {n: extra_workload(n, 20, 10) for n in EXTRA_WORKLOADS if n != args.config}
        log("[bench] extra workloads: " + ", ".join(f"{n}={v['ms_per_step']:.3f} ms" for n, v in
                                                     out["extra_workloads"].items()))
    print(json.dumps(out), flush=True)


def measure_backward(run, cfg, dev, up, x, wg, bias, w1, w3, w2, plan, ws, calls):
    """moe_backward: the fp32 gradients in x, Wg, bias and the expert weights for an
    upstream gradient dy, the routing held fixed (it recomputes the forward's
    activations).  Routes once (with logits), then one warm-up call and `calls` timed
    calls.  Its floor: the weights of the non-empty experts read once and the fp32
    weight gradients written once (plus x, dy and dx)."""
    import torch

    from top_routing_expert_router_amd import binding as B
    from top_routing_expert_router_amd.synth import recipes

    eb = run.elem_bytes
    plan_b = dict(plan)
    plan_b["logits"] = torch.empty((run.T, run.E), dtype=torch.float32, device=dev)
    B.route(cfg, x, wg, bias, plan_b, ws)
    dy = up(recipes.gen_dy(run))
    grads = B.alloc_grads(cfg, dev)
    bws = torch.empty(max(B.backward_workspace_bytes(cfg), 1), dtype=torch.uint8, device=dev)
    B.backward(cfg, x, wg, w1, w3, w2, plan_b, dy, grads, bws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(calls):
        B.backward(cfg, x, wg, w1, w3, w2, plan_b, dy, grads, bws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / calls * 1e3
    kept = plan_b["kept"].cpu().numpy()
    R = int(kept.sum())
    floor = (int((kept > 0).sum()) * run.m * run.H * run.F * eb + run.E * run.m * run.H * run.F * 4 +
             3.0 * run.T * run.H * eb)
    flops = 2 * 2.0 * R * run.H * run.F * run.m  # data and weight gradients (no recomputation)
    out = {"ms": round(us / 1e3, 4), "tokens_per_s": round(run.T / (us * 1e-6), 1), "calls": calls,
           "floor_bytes": floor, "hbm_frac": round(floor / (us * 1e-6) / 8e12, 4),
           "gradient_tflops": round(flops / (us * 1e-6) / 1e12, 1), "workspace_GiB": round(bws.numel() / 2 ** 30, 2),
           "note": "fp32 gradients of x, Wg, bias, W1, W3, W2; activations recomputed from x"}
    log(f"[bench] backward: {us / 1e3:.2f} ms ({out['hbm_frac']:.3f} of the HBM floor)")
    if cfg.dtype == B.BF16 and run.H % 64 == 0 and run.F % 8 == 0:
        # training with the forward's pre-activations kept (moe_forward_save): the
        # forward with and without keeping them, and the backward given them
        R_max = max(B.max_rows(cfg), 1)
        act = torch.empty(B.saved_act_bytes(cfg), dtype=torch.uint8, device=dev)
        X = torch.empty((R_max, run.H), dtype=torch.bfloat16, device=dev)
        Y = torch.empty_like(X)
        y = torch.empty((run.T, run.H), dtype=torch.bfloat16, device=dev)

        def timed_calls(fn):
            fn()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(calls):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / calls * 1e3

        f_us = timed_calls(lambda: B.forward(cfg, x, wg, bias, w1, w3, w2, x, y, plan_b, X, Y, ws))
        fs_us = timed_calls(lambda: B.forward_save(cfg, x, wg, bias, w1, w3, w2, x, y, plan_b, X, Y, act, ws))
        kb_us = timed_calls(lambda: B.backward(cfg, x, wg, w1, w3, w2, plan_b, dy, grads, bws, act=act))
        out["kept_preactivations"] = {
            "backward_ms": round(kb_us / 1e3, 4), "hbm_frac": round(floor / (kb_us * 1e-6) / 8e12, 4),
            "forward_ms": round(f_us / 1e3, 4), "forward_save_ms": round(fs_us / 1e3, 4),
            "kept_GiB": round(act.numel() / 2 ** 30, 3),
            "note": "moe_forward_save keeps u (and v) for moe_backward, which then skips their recomputation"}
        log(f"[bench] backward with kept pre-activations: {kb_us / 1e3:.2f} ms "
            f"({out['kept_preactivations']['hbm_frac']:.3f} of the HBM floor); forward {f_us / 1e3:.3f} ms, "
            f"keeping them {fs_us / 1e3:.3f} ms")
        del act, X, Y, y
    del grads, bws, dy
    return out


def extra_workload(name, steps, warmup):
    """The same whole-layer measurement, briefer, on another workload: layer time, tokens/s,
    the expert-FFN stage (its grouped-GEMM launches) and its roofline fraction."""
    import numpy as np
    import torch

    from top_routing_expert_router_amd import binding as B
    from top_routing_expert_router_amd.synth import recipes

    run = recipes.RUNS[name]
    dev = torch.device("cuda:0")
    cfg = B.MoEConfig.from_run(run)
    bf16 = run.dtype == recipes.BF16
    tdt = torch.bfloat16 if bf16 else torch.float32
    eb = run.elem_bytes

    def up(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x = up(recipes.gen_x(run))
    wg, bias = (up(t) for t in recipes.gen_router(run))
    ws_ = {n: up(recipes.gen_expert_weight(run, n)) if (n != "w3" or run.act == recipes.SWIGLU) else None
           for n in ("w1", "w3", "w2")}
    plan = B.alloc_plan(cfg, dev)
    rmax = B.max_rows(cfg)
    X = torch.empty((max(rmax, 1), run.H), dtype=tdt, device=dev)
    Y = torch.empty_like(X)
    y = torch.empty((run.T, run.H), dtype=tdt, device=dev)
    ws = B.alloc_workspace(cfg, dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3

    layer_us = timed(lambda: B.forward(cfg, x, wg, bias, ws_["w1"], ws_["w3"], ws_["w2"], x, y, plan, X, Y, ws))
    B.dispatch(cfg, x, plan, X)  # the forward reads x through row_token and leaves X unwritten
    ffn_us = timed(lambda: B.expert_ffn(cfg, X, plan, ws_["w1"], ws_["w3"], ws_["w2"], Y, ws))
    kept = plan["kept"].cpu().numpy()
    R = int(kept.sum())
    flops = 2.0 * R * run.H * run.F * run.m
    byts = int((kept > 0).sum()) * run.m * run.H * run.F * eb + 2.0 * R * run.H * eb
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    t_mfma, t_hbm = flops / (peak * 1e12) * 1e6, byts / (PEAK_HBM_GBS * 1e9) * 1e6
    out = {"workload": WORKLOADS[name], "ms_per_step": round(layer_us / 1e3, 5),
           "tokens_per_s": round(run.T / (layer_us * 1e-6), 1), "expert_ffn_us": round(ffn_us, 2),
           "expert_ffn_tflops": round(flops / (ffn_us * 1e-6) / 1e12, 1),
           "expert_ffn_roofline": {"bound": "hbm" if t_hbm >= t_mfma else "mfma",
                                   "frac": round(max(t_mfma, t_hbm) / ffn_us, 4)}}
    del ws_, X, Y, y, ws, x
    torch.cuda.empty_cache()
    return out


def cpu_baseline(run, x_h, wg_h, bias_h, target_s):
    """Oracle tokens/s on the host cores: routing of the whole batch (capacity needs every
    token), the expert FFN of every row of a seeded sample of experts (only their weights
    are generated on the host), scaled to all kept rows, and the combine of every token."""
    import numpy as np

    import oracle
    from top_routing_expert_router_amd.synth import recipes

    C = None if run.dropless else oracle.capacity(run.T, run.k, run.E, run.cf, run.min_capacity)
    t0 = time.perf_counter()
    plan = oracle.route(x_h, run.dtype, wg_h, bias_h, run.k, run.gate_mode, C)
    t_route = time.perf_counter() - t0
    off, R = plan["offsets"], plan["R"]
    rows_of = np.diff(off)
    order = np.random.default_rng(run.run_id).permutation(np.nonzero(rows_of > 0)[0])
    # about target_s of FFN work at a first guess of 4 GFLOP/s per thread, at least one expert
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    flop_row = 2.0 * run.H * run.F * run.m
    budget = max(1, int(target_s * 4e9 * threads / flop_row))
    chosen, m = [], 0
    for e in order:
        if chosen and m + rows_of[e] > budget:
            break
        chosen.append(int(e))
        m += int(rows_of[e])
    Y = np.zeros((max(R, 1), run.H), np.float64)
    ws = {n: recipes.gen_expert_weight(run, n, experts=chosen) for n in (("w1", "w3", "w2") if run.m == 3 else
                                                                          ("w1", "w2"))}
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in chosen])
    ex = np.concatenate([np.full(rows_of[e], i, np.int32) for i, e in enumerate(chosen)])
    xin = x_h[plan["row_token"][rows]]
    cw = {n: np.stack([ws[n][e] for e in chosen]) for n in ws}
    t1 = time.perf_counter()
    Y[rows] = oracle.expert_rows(xin, ex, run.dtype, run.act, cw["w1"], cw.get("w3"), cw["w2"])
    t_ffn = time.perf_counter() - t1
    t2 = time.perf_counter()
    oracle.combine(Y[:max(R, 1)], plan, run.dtype, residual=x_h)
    t_comb = time.perf_counter() - t2
    total = t_route + t_ffn * (R / max(m, 1)) + t_comb
    return {"value": round(run.T / total, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"routing of all {run.T} tokens ({t_route:.2f}s); expert FFN of all {m} rows of {len(chosen)} "
                      f"seeded-random non-empty experts ({t_ffn:.2f}s), scaled to the {R} kept rows; combine of all "
                      f"{run.T} tokens ({t_comb:.2f}s); binary64 C oracle with OpenMP"}


if __name__ == "__main__":
    main()
