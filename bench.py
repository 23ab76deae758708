#!/usr/bin/env python3
"""Throughput of whole training steps run as one persistent kernel each, on one MI355X.

A step is one launch of the persistent kernel over the whole compiled program
(forward, MSE loss, explicit backward, in-place SGD).  The default workload is
the largest single-GPU configuration: the 16-layer fp16 residual MLP (batch
512, width 2048, h = h + relu(addmm(h, W_i, b_i)), MSE head to 2048 targets,
full backward, lr 1e-4; 47 contractions, 201.9 GFLOP per step).  Inputs are
seeded synthetic tensors already resident in HBM; parameters are updated in
place every step (state feedback) and the (x, target) batch rotates over 4
resident batches.  The timed region is 5 batches of back-to-back launches,
each bracketed by HIP events on the launch stream; the value is the median
batch's rate, and the raw batch times are kept.  The 4096-wide bf16 MLP gets
its own roofline block; the other workloads (2-layer fp32 MLP, 3-layer bf16
MLP with SGD, with AdamW and captured from torch.func, int8-weight GEMV stack
rotating 3 weight sets, with 4 decode rows and with Q8_0 activations) are
timed briefly under "others".

Prints one JSON line on stdout.  --gpus N with N > 1 is refused: the
kernel runs on one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
WORKLOAD_NAMES = {
    "c1": "mlp2-fp32-b64-128-256-10",
    "c2": "mlp3-bf16-b256-512-1024-1024-64",
    "c3": "gemv8-int8w-bf16x-4096x4096",
    "c4": "mlp3-bf16-b1024-4096-4096-4096-1024",
    "c5": "resmlp16-fp16-b512-w2048",
    "c2a": "mlp3-bf16-b256-512-1024-1024-64-adamw",
    "c3r4": "gemv8-int8w-bf16x-4x4096x4096",
    "c3q": "gemv8-int8w-q8x-4096x4096",
    "c2cap": "mlp3-bf16-b256-512-1024-1024-64-captured",
}


def config(name: str) -> dict:
    """The workload's configuration; c2a is C2 with AdamW (defaults 0.9,
    0.999, 1e-8, weight decay 1e-2) in place of SGD, at step t = 10; c3r4 is
    C3 with 4 decode rows; c3q is C3 with its activations quantised to Q8_0
    inside each product."""
    from persistent_whole_step_amd import programs
    if name == "c2a":
        return dict(programs.CONFIGS["c2"], optimizer=programs.AdamW(), adam_t=10)
    if name == "c3r4":
        return dict(programs.CONFIGS["c3"], rows=4)
    if name == "c3q":
        return dict(programs.CONFIGS["c3"], xq=True)
    if name == "c2cap":
        return dict(programs.CONFIGS["c2"], captured=True)
    return programs.CONFIGS[name]


def captured_mlp(cfg):
    """C2's step written as a torch.func training step and captured by the
    front end (state first, so the updated parameters commit in place).
    Returns the program and the permutation from the workload's input order
    (x, t, W1, b1, ...) to the captured order (W1, b1, ..., x, t)."""
    import torch
    from persistent_whole_step_amd import frontend
    dims, B, lr = cfg["dims"], cfg["batch"], cfg["lr"]
    L = len(dims) - 1

    def step(params, x, target):
        def loss(p):
            h = x
            for i in range(L):
                h = torch.addmm(p[2 * i + 1], h, p[2 * i])
                if i + 1 < L:
                    h = torch.relu(h)
            return ((h - target) ** 2).mean()
        g, v = torch.func.grad_and_value(loss)(params)
        return v, tuple(w - lr * gw for w, gw in zip(params, g))

    bf = torch.bfloat16
    params = tuple(t for i in range(L) for t in (torch.zeros(dims[i], dims[i + 1], dtype=bf),
                                                 torch.zeros(dims[i + 1], dtype=bf)))
    c = frontend._capture(step, (params, torch.zeros(B, dims[0], dtype=bf), torch.zeros(B, dims[-1], dtype=bf)))
    c.program.inplace = frontend._update_mapping(c)
    return c.program, list(range(2, 2 + 2 * L)) + [0, 1]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "persistent_whole_step_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def gemv_bytes(cfg) -> int:
    k, n, L, m = cfg["k"], cfg["n"], cfg["layers"], cfg.get("rows", 1)
    nb = (k + 31) // 32
    return L * (n * k + n * nb * 4 + n * 4 + m * k * 2 + m * n * 2)


class Runner:
    """Compiled program + resident input variants + prebuilt C descriptors."""

    def __init__(self, name: str, seed0: int = 0, **opts):
        import torch
        from persistent_whole_step_amd import programs, tk
        to_torch = tk.tensor_from_storage
        self.name = name
        self.cfg = config(name)
        order = None
        if self.cfg.get("captured"):
            self.prog, order = captured_mlp(self.cfg)
        else:
            self.prog = programs.build(self.cfg)
        reorder = (lambda ins: [ins[i] for i in order]) if order else (lambda ins: ins)
        self.p = tk.compile(self.prog.text(), device=0, **opts)
        self.stats = self.p.query()
        cfg = self.cfg
        if cfg["kind"] == "gemv":
            sets = [programs.inputs_for(cfg, seed0 + j) for j in range(3)]
            self.inputs = [[to_torch(a, s.dtype) for a, s in zip(ins, self.prog.inputs)] for ins in sets]
        else:
            wl = [to_torch(a, s.dtype) for a, s in zip(programs.inputs_for(cfg, seed0), programs.build(cfg).inputs)]
            self.inputs = [reorder(wl)]
            for j in range(1, 4):
                ins = programs.inputs_for(cfg, seed0 + 100 + j)
                dt = cfg.get("dtype", "bf16")
                self.inputs.append(reorder([to_torch(ins[0], dt), to_torch(ins[1], dt)] + wl[2:]))
        self.buffers = self.p.allocate(*self.inputs[0])
        self.variants = []
        for ins in self.inputs:
            bufs = tk.ExecutionBuffers(tuple(ins[self.p._inplace_map()[s]] if s in self.p._inplace_map() else o
                                             for s, o in enumerate(self.buffers.outputs)), self.buffers.workspace)
            self.p.validate_into(*ins, buffers=bufs)
            ci, co, cw = self.p._descs(ins, bufs)
            self.variants.append((ci, len(ins), co, len(bufs.outputs), cw))
        self.run_c = tk.lib().tk_run_into
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.tk = tk

    def close(self):
        """Free the compiled program and drop the resident tensors."""
        self.p.close()
        self.variants = []
        self.inputs = []
        self.buffers = None

    def step(self, i: int):
        ci, ni, co, no, cw = self.variants[i % len(self.variants)]
        rc = self.run_c(self.p._h, ci, ni, co, no, ctypes.byref(cw), self.stream)
        if rc != 0:
            raise self.tk.TkError(rc, self.tk.lib().tk_last_error().decode())

    def graph_time(self, replays: int, warmup: int = 3):
        """Steps/s of the steady-state loop replayed from a captured HIP graph
        (one launch per resident batch variant per replay)."""
        import torch
        tk = self.tk
        variants = []
        for ins in self.inputs:
            bufs = tk.ExecutionBuffers(tuple(ins[self.p._inplace_map()[s]] if s in self.p._inplace_map() else o
                                             for s, o in enumerate(self.buffers.outputs)), self.buffers.workspace)
            variants.append((ins, bufs))
        g = tk.StepGraph(self.p, variants)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record()
        for _ in range(replays):
            g.replay()
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        self.check_not_aborted()
        return replays * g.steps, wall, start.elapsed_time(end)

    def check_not_aborted(self):
        aborted, stage = self.p.workspace_status(self.buffers.workspace)
        if aborted:
            raise RuntimeError(f"{self.name}: a grid barrier timed out in stage {stage}")

    def time_batches(self, steps: int, warmup: int, batches: int = 5):
        """`steps` launches in `batches` equal batches of back-to-back launches,
        each bracketed by HIP events on the launch stream, after `warmup`
        untimed launches; the whole timed region is bracketed by device
        synchronisation.  Returns (wall seconds, [batch ms], steps per batch)."""
        import torch
        per = max(1, steps // batches)
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(batches)]
        t0 = time.perf_counter()
        i = 0
        for a, b in evs:
            a.record()
            for _ in range(per):
                self.step(i)
                i += 1
            b.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        self.check_not_aborted()
        return wall, [a.elapsed_time(b) for a, b in evs], per

    def stage_stamps(self):
        """In-situ stage timing of one launch (workgroup 0's stamps: items
        done, then barrier passed; the next stage's descriptors are staged
        inside the barrier, so the staging stamp equals the first and
        sum_staging_us is 0), in microseconds."""
        import torch
        self.p.set_debug(timestamps=True)
        for i in range(3):
            self.step(i)
        torch.cuda.synchronize()
        ts = self.p.read_timestamps(self.buffers.workspace)
        self.p.set_debug(timestamps=False)
        self.check_not_aborted()
        n = self.stats["n_stages"]
        items, staging, barrier = [], [], []
        for st in range(n):
            start, done, blob, bar = ts[4 * st:4 * st + 4]
            if done >= start:
                items.append((done - start) / 100.0)
            if st + 1 < n:
                staging.append((blob - done) / 100.0)
                barrier.append((bar - blob) / 100.0)
        med = lambda v: round(sorted(v)[len(v) // 2], 3) if v else None
        return {"stages": n, "sum_items_us": round(sum(items), 2), "sum_staging_us": round(sum(staging), 2),
                "sum_barrier_us": round(sum(barrier), 2), "median_barrier_us": med(barrier),
                "median_items_us": med(items),
                "note": "workgroup 0: barrier = waiting at the grid barrier after its own items, which includes "
                        "the slowest workgroup's lag"}

    def kernel_ms(self, n: int = 50) -> float:
        """Average duration of one launch, HIP events on the launch stream."""
        import torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(evs):
            a.record()
            self.step(i)
            b.record()
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in evs)
        return sum(ts) / len(ts)


def roofline(name: str, cfg, prog, kernel_ms: float, traffic):
    from persistent_whole_step_amd import programs
    if cfg["kind"] == "gemv":
        b = gemv_bytes(cfg)
        ach = b / (kernel_ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(ach, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic, "algorithmic_bytes": b}
    fl = programs.contraction_flops(prog)
    ach = fl / (kernel_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[cfg["dtype"]]
    return {"bound": "mfma", "achieved": round(ach, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(ach / peak, 5), "traffic": traffic, "algorithmic_flops": fl}


def traffic_for(name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, when
    it was taken on the current kernel sources (else null)."""
    path = os.path.join(ROOT, "profiles", f"tk_persistent_{WORKLOAD_NAMES[name]}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != source_hash():
        return None
    return d.get("bytes_per_launch")


def barrier_latency(n_small: int = 8, n_large: int = 264):
    """Per-barrier latency: slope of launch time over the number of stages of a
    chain of trivial one-element ops, launched on a full grid."""
    import torch
    from persistent_whole_step_amd import tk
    from persistent_whole_step_amd.programs import Program
    res = {}
    grid = None
    for n in (n_small, n_large):
        p = Program()
        x = p.input("x", "f32", (1,))
        v = x
        for _ in range(n):
            v = p.op("add", [v, 1.0], "f32")
        p.output(v)
        prog = tk.compile(p.text(), device=0, fuse_pointwise=0, force_grid=100000)
        grid = prog.query()["grid_size"]
        xt = torch.zeros(1, device="cuda:0")
        bufs = prog.allocate(xt)
        for _ in range(5):
            prog.run_into(xt, buffers=bufs)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        a.record()
        for _ in range(reps):
            prog.run_into(xt, buffers=bufs)
        b.record()
        torch.cuda.synchronize()
        res[n] = a.elapsed_time(b) / reps
        ab, _ = prog.workspace_status(bufs.workspace)
        if ab:
            raise RuntimeError("barrier microbenchmark aborted")
    per = (res[n_large] - res[n_small]) / (n_large - n_small) * 1e3
    return {"per_barrier_us": round(per, 3), "grid": grid, "launch_ms_%d_stages" % n_small: round(res[n_small], 4),
            "launch_ms_%d_stages" % n_large: round(res[n_large], 4)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_time(text, ins, runs: int):
    from oracle import oracle
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        oracle.run(text, [a.copy() for a in ins])
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[len(ts) // 2]


def cpu_baseline(name: str):
    """The oracle, as it stands, timed on this host's cores.  The headline
    workload is timed on a bounded sample: the same step with 2 of its 16
    residual layers (same batch and width), whose time is scaled to the whole
    step by the contraction FLOPs (the step's cost is in its contractions).
    C1-C3 (the oracle finishes them in seconds) are timed whole: all threads,
    median of 3, and one thread (median of 3; one run for C2)."""
    from oracle import oracle
    from persistent_whole_step_amd import programs
    threads = oracle.threads()
    cfg = config(name)
    res = {"unit": "steps/s", "kind": "oracle", "cpu": cpu_model(), "cores": threads}
    if cfg["kind"] == "residual" and cfg["layers"] > 2:
        small = dict(cfg, layers=2)
        prog, full = programs.build(small), programs.build(cfg)
        scale = programs.contraction_flops(full) / programs.contraction_flops(prog)
        t = _oracle_time(prog.text(), programs.inputs_for(small, 0), 1)
        res.update(value=round(1.0 / (t * scale), 6),
                   sample=f"one step of the same residual MLP with 2 of its {cfg['layers']} layers "
                          f"(batch {cfg['batch']}, width {cfg['width']}) in {t:.2f} s, scaled by the contraction "
                          f"FLOPs ({scale:.2f}x) to the whole step")
    else:
        prog = programs.build(cfg)
        t = _oracle_time(prog.text(), programs.inputs_for(cfg, 0), 3)
        res.update(value=round(1.0 / t, 4), sample=f"whole {WORKLOAD_NAMES[name]} steps, median of 3")
    per_config = {}
    for c in ("c1", "c2", "c3"):
        cc = config(c)
        prog = programs.build(cc)
        ins = programs.inputs_for(cc, 0)
        oracle.set_threads(threads)
        t_all = _oracle_time(prog.text(), ins, 3)
        oracle.set_threads(1)
        t_one = _oracle_time(prog.text(), ins, 1 if c == "c2" else 3)
        oracle.set_threads(threads)
        per_config[WORKLOAD_NAMES[c]] = {"steps_per_s_all_threads": round(1.0 / t_all, 3),
                                         "steps_per_s_one_thread": round(1.0 / t_one, 3)}
        log(f"[bench] oracle {c}: {per_config[WORKLOAD_NAMES[c]]}")
    res["whole_steps"] = per_config
    return res


def measure(name: str, steps: int, warmup: int, launch_mode: int, stamps: bool = False):
    """Time one workload: batched events, launch duration, roofline."""
    r = Runner(name, launch_mode=launch_mode)
    log(f"[bench] {name}: stages={r.stats['n_stages']} grid={r.stats['grid_size']}; timing {steps} steps")
    wall, batch_ms, per = r.time_batches(steps, warmup)
    med = sorted(batch_ms)[len(batch_ms) // 2]
    kms = r.kernel_ms()
    out = {
        "value": per / (med * 1e-3),
        "ms_per_step": med / per,
        "steps": per * len(batch_ms),
        "wall_steps_per_s": per * len(batch_ms) / wall,
        "batch_ms": [round(x, 4) for x in batch_ms],
        "steps_per_batch": per,
        "kernel_ms": kms,
        "roofline": roofline(name, r.cfg, r.prog, kms, traffic_for(name)),
        "stats": r.stats,
    }
    if stamps:
        out["stage_stamps"] = r.stage_stamps()
    return r, out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c5", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--others", default="c1,c2,c2a,c2cap,c3,c3r4,c3q",
                    help="comma list of extra workloads ('' for none)")
    ap.add_argument("--other-steps", type=int, default=100)
    ap.add_argument("--no-c4", action="store_true", help="skip the 4096-wide MLP's roofline block")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-barrier", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="report the eager launch loop only")
    ap.add_argument("--launch-mode", type=int, default=1, choices=(0, 1),
                    help="0: cooperative launch; 1: ordinary launch of the co-resident grid (default)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on one GPU only; sharding across GPUs is a design, not an implementation",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        sys.exit(1)
    from persistent_whole_step_amd import tk
    tk.lib()

    log(f"[bench] workload {args.config}: compiling")
    r, m = measure(args.config, args.steps, args.warmup, args.launch_mode, stamps=True)
    graph = None
    if args.launch_mode == 1 and not args.no_graph:
        # the steady-state loop replayed from a captured graph, state fed back
        # through the in-place updates
        n_rep = max(1, min(args.steps, 200) // len(r.inputs))
        gsteps, gwall, gev = r.graph_time(n_rep)
        graph = {"steps_per_s": round(gsteps / gwall, 2), "ms_per_step": round(gwall / gsteps * 1e3, 5),
                 "steps": gsteps, "event_ms_per_step": round(gev / gsteps, 5)}
    st = m["stats"]
    line = {
        "metric": "training steps/sec per program",
        "value": round(m["value"], 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": m["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r.cfg.get("dtype", "bf16"),
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.config], "batch": r.cfg.get("batch"),
                   "dims": r.cfg.get("dims"), "width": r.cfg.get("width"), "layers": r.cfg.get("layers"),
                   "lr": r.cfg.get("lr"), "parallelism": "single-gpu", "resident_batches": 4,
                   "stages": st["n_stages"], "grid_barriers": st["grid_barriers"], "grid": st["grid_size"],
                   "launch": "ordinary, co-resident grid" if args.launch_mode == 1 else "cooperative"},
        "timing": f"median of {len(m['batch_ms'])} event-timed batches of {m['steps_per_batch']} launches",
        "batch_ms": m["batch_ms"],
        "wall_steps_per_s": round(m["wall_steps_per_s"], 2),
        "graph_replay": graph,
        "kernel_ms": round(m["kernel_ms"], 5),
        "roofline": m["roofline"],
        "stage_stamps": m["stage_stamps"],
    }
    log(f"[bench] {args.config}: {m['value']:.1f} steps/s, kernel {m['kernel_ms'] * 1e3:.1f} us")
    r.close()
    del r
    torch.cuda.empty_cache()
    if not args.no_barrier:
        log("[bench] barrier microbenchmark")
        line["barrier"] = barrier_latency()
    if not args.no_c4 and args.config != "c4":
        log("[bench] 4096-wide MLP")
        r4, m4 = measure("c4", args.other_steps, 10, args.launch_mode, stamps=True)
        line["c4"] = {"workload": WORKLOAD_NAMES["c4"], "steps_per_s": round(m4["value"], 2),
                      "ms_per_step": round(m4["ms_per_step"], 5), "batch_ms": m4["batch_ms"],
                      "kernel_ms": round(m4["kernel_ms"], 5), "roofline": m4["roofline"],
                      "stage_stamps": m4["stage_stamps"]}
        r4.close()
        del r4
        torch.cuda.empty_cache()
    others = {}
    for name in [x for x in args.others.split(",") if x and x != args.config]:
        log(f"[bench] other workload {name}")
        o, mo = measure(name, args.other_steps, 10, args.launch_mode)
        rf = mo["roofline"]
        others[WORKLOAD_NAMES[name]] = {"steps_per_s": round(mo["value"], 2),
                                       "ms_per_step": round(mo["ms_per_step"], 4),
                                       "kernel_ms": round(mo["kernel_ms"], 4), "stages": mo["stats"]["n_stages"],
                                       "achieved": rf["achieved"], "unit": rf["unit"], "frac": rf["frac"]}
        log(f"[bench] {name}: {others[WORKLOAD_NAMES[name]]}")
        o.close()
        del o
        torch.cuda.empty_cache()
    if others:
        line["others"] = others
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline(args.config)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
