"""Benchmark of the sparse MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload skewed|prefill|decode|capacity|tiny]
                    [--reroute] [--no-others]

A step is one moe_forward (router, dispatch, expert GEMM1+GELU, GEMM2,
combine) over one batch of seeded synthetic inputs that are resident in HBM
before the timed region starts.  The default workload is the largest one a
single GPU holds: T = 16384 tokens, d = 4096, E = 64, k = 2, F = 14336 with a
Zipf-skewed router bias.  Unless --no-others is given, the prefill,
capacity-limited and decode workloads are then measured the same way (without
the CPU baseline) and reported under "other_workloads".  --reroute times moe_forward_reroute
instead: pairs over the expert capacity move to their token's next-best
expert with room rather than being dropped.  The headline times K steps captured in one
HIP graph and replayed.  Each stage entry point is then timed on its own: K
back-to-back launches, captured in a HIP graph and replayed between two HIP
events on the stream the kernels run on, which gives the kernels' average
duration without host gaps.  Prints one
JSON line: tokens/s of the whole layer, the roofline fraction of the dominant
kernel (of the published peak, and of the peak a plain copy and a large
vendor-library GEMM reach on the same GPU, "achievable"), per-stage times,
and the CPU oracle timed on a bounded sample of the same workload (a
baseline, not the target).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 MFMA/vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE-layer tokens/sec at 1 GPU; % bf16 MFMA peak (FFN) / % HBM peak (rest)"

# HBM bytes per launch of the expert GEMMs from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch), scaled by what the same counters read for a
# plain 1 GiB device copy (FETCH_SIZE x2.0, WRITE_SIZE x1.0); valid only for
# the GEMM code they were taken on (sha1 prefix of the source without its
# comments, gemm_code_sha1), else reported as null.
TRAFFIC_SOURCE_SHA1 = "17b1e6c718f5"
TRAFFIC_BYTES = {  # (workload, stage) -> (fetch KiB, write KiB) per dispatch, raw counter values
    ("skewed", "expert_up"): (7089269.9, 918918.2),
    ("skewed", "expert_down"): (6354849.7, 266148.9),
    ("prefill", "expert_up"): (468235.1, 180359.1),
    ("prefill", "expert_down"): (518053.5, 65572.1),
    ("capacity", "expert_up"): (751814.4, 285444.5),
    ("capacity", "expert_down"): (591858.4, 416824.2),
    ("decode", "expert_up"): (122263.1, 160.0),
    ("decode", "expert_down"): (122351.3, 224.0),
}
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0


def gemm_code_sha1(path):
    """sha1 prefix of a source file's code: line comments and blank lines
    dropped and each line stripped, so a change to the comments alone keeps
    the counters measured on that code."""
    import hashlib
    import re
    lines = []
    with open(path, encoding="utf-8") as f:
        for line in f:
            code = re.sub(r"//.*$", "", line).strip()
            if code:
                lines.append(code)
    return hashlib.sha1("\n".join(lines).encode()).hexdigest()[:12]


def gemm_traffic(workload, stage):
    sha = gemm_code_sha1(os.path.join(ROOT, "sparse_mixture_experts_04_amd", "csrc", "grouped_gemm.hip"))
    if sha != TRAFFIC_SOURCE_SHA1 or (workload, stage) not in TRAFFIC_BYTES:
        return None
    fetch, write = TRAFFIC_BYTES[(workload, stage)]
    return round((fetch * FETCH_SCALE + write * WRITE_SCALE) * 1024)


def gemm_kernel_name(w, capacity, stage, gathers):
    """The expert-GEMM kernel the library runs for this shape (its selection
    rule: bf16 with at most min(T, C) rows per expert picks the few-rows
    kernels; the up-projection of the 256x256 and decode kernels gathers X
    through perm where moe_expert_up_gather_supported says so)."""
    gelu = "true" if stage == "expert_up" else "false"
    K = w.d if stage == "expert_up" else w.F
    N = w.F if stage == "expert_up" else w.d
    if w.dtype != "bf16":
        return f"grouped_gemm_kernel<float, 64, 64, 2, 2, {gelu}>"
    bound = w.T if capacity < 0 else min(w.T, capacity)
    few = bound <= 16 or (bound <= 64 and w.T * w.k <= 16 * w.E)  # at most 16 rows per expert on average
    if K % 128 == 0 and N % 8 == 0 and few:
        g = 1 if bound <= 4 else 2 if bound <= 8 else 4
        return f"grouped_gemm_bf16_gemv<{gelu}, {g}, {'true' if gathers and stage == 'expert_up' else 'false'}>"
    if bound <= 64:
        return f"grouped_gemm_bf16_skinny<{gelu}, {1 if bound <= 16 else 2 if bound <= 32 else 4}>"
    return f"grouped_gemm_bf16_256<{gelu}, {'true' if gathers and stage == 'expert_up' else 'false'}, 8>"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; decode-sized workloads: their step count, 100)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="skewed")
    ap.add_argument("--no-others", action="store_true", help="measure only --workload")
    ap.add_argument("--cpu-sample", type=int, default=None, help="tokens (prefill-like) or steps (decode) for the oracle")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of one HIP-graph replay of the K steps")
    ap.add_argument("--reroute", action="store_true",
                    help="reroute over-capacity pairs to the next-best expert (moe_forward_reroute)")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the measured peaks (device copy, read-only stream, vendor GEMM)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (reference for HBM byte counters)")
    return ap.parse_args()


def to_dev(torch, a, dtype):
    if a is None:
        return None
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def stage_work(w, N, active, es, gathers, reroute=False):
    """Algorithmic FLOPs and bytes per launch of each stage (N kept pairs,
    `active` experts with rows).  With the gathered up-projection the
    dispatch moves indices only and the up-projection reads each pair's row
    of X in place of the copied row."""
    T, d, F, E, k = w.T, w.d, w.F, w.E, w.k
    rows = 0 if gathers else T * d * es + N * d * es
    order = T * E if reroute else 0  # the preference order, written by the router, read by the dispatch
    return {
        "route": {"flops": 2.0 * T * d * E, "bytes": T * d * es + d * E * es + T * k * 8 + order},
        "dispatch": {"flops": 0.0, "bytes": rows + T * k * 4 * 3 + order},
        "expert_up": {"flops": 2.0 * N * d * F, "bytes": active * F * d * es + N * d * es + N * F * es},
        "expert_down": {"flops": 2.0 * N * F * d, "bytes": active * d * F * es + N * F * es + N * d * es},
        "combine": {"flops": 0.0, "bytes": N * d * es + T * k * 8 + T * d * es},
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, sample, reroute=False):
    """The oracle, as it stands, on a bounded sample of the workload: the
    first `sample` tokens as one batch with the full expert weights (a
    prefill-like workload; default 512 tokens), or `sample` decode steps
    (default 4).  The sample is repeated until at least 10 s (at most about
    30 s) of CPU work has been timed."""
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    t0 = time.perf_counter()
    toks, reps = 0, 0
    if w.steps > 1:
        n = sample or 4
        while True:
            for s in range(n):
                X = workloads.decode_step_inputs(w, s)
                oracle.moe_forward(X, inp.Wg, inp.bias, inp.W1, inp.W2, w.k, inp.expert_capacity, w.dtype,
                                   reroute=reroute)
            toks += n * w.T
            reps += 1
            elapsed = time.perf_counter() - t0
            if elapsed >= 10.0 or elapsed + elapsed / reps > 30.0:
                break
        desc = f"{reps} x {n} decode steps of {w.T} tokens, full weights"
    else:
        n = min(sample or 512, w.T)
        cap = (-(-n // w.E) * w.k) if inp.expert_capacity >= 0 else -1
        while True:
            oracle.moe_forward(inp.X[:n], inp.Wg, inp.bias, inp.W1, inp.W2, w.k, cap, w.dtype, reroute=reroute)
            toks += n
            reps += 1
            elapsed = time.perf_counter() - t0
            if elapsed >= 10.0 or elapsed + elapsed / reps > 30.0:
                break
        desc = (f"{reps} x first {n} of {w.T} tokens as one batch, full expert weights"
                + (f", capacity {cap}" if cap >= 0 else "") + (", rerouted" if reroute and cap >= 0 else ""))
    dt = time.perf_counter() - t0
    return {"value": toks / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": desc, "seconds": round(dt, 2), "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count()}


def rotation_sets(w, T, d, F, k, es):
    """How many input sets the per-stage timings rotate over: enough that
    the smallest per-set input of a stage (the hidden states X, read by the
    router) summed over the sets exceeds 1 GiB, four times the 256 MB
    last-level (MALL) cache, so no stage time is served from it; at least 4,
    at most 32."""
    per_set = T * d * es
    return int(min(32, max(4, -(-(1 << 30) // max(per_set, 1)))))


def measure(torch, moe, workloads, name, steps, warmup, eager=False, reroute=False, with_cpu=False,
            cpu_sample=None):
    """Measure one workload: the whole-layer step rate, the per-stage kernel
    times and the roofline of the dominant expert GEMM."""
    w = workloads.WORKLOADS[name]
    t_gen = time.perf_counter()
    inp = workloads.generate(w)
    gen_s = time.perf_counter() - t_gen
    dt = w.dtype
    es = 2 if dt == "bf16" else 4
    if steps is None:
        steps = w.steps if w.steps > 1 else 20
    cfg = moe.config(w.T, w.d, w.F, w.E, w.k, inp.expert_capacity, dt)
    Wg, W1, W2 = to_dev(torch, inp.Wg, dt), to_dev(torch, inp.W1, dt), to_dev(torch, inp.W2, dt)
    bias = to_dev(torch, inp.bias, "f32")
    if w.steps > 1:
        xs = [to_dev(torch, workloads.decode_step_inputs(w, s), dt) for s in range(w.steps)]
    else:
        # Rotated copies of the one batch: the same tokens in another order
        # (the layer is equivariant under token permutations, so each copy
        # does the same work) at other addresses, for the stage timings.
        X0 = to_dev(torch, inp.X, dt)
        nrot = rotation_sets(w, w.T, w.d, w.F, w.k, es)
        xs = [X0] + [torch.roll(X0, shifts=(i * w.T) // nrot, dims=0).contiguous() for i in range(1, nrot)]
    reroute = bool(reroute)
    layer = moe.MoELayer(cfg, Wg, W1, W2, bias, reroute=reroute)
    b = layer.buf
    stream = torch.cuda.current_stream()

    # Whole-layer steps step through the decode steps' fresh hidden states;
    # a prefill-like layer repeats its one batch.
    step_x = xs if w.steps > 1 else xs[:1]
    for i in range(warmup):
        layer.forward(step_x[i % len(step_x)])
    torch.cuda.synchronize()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(run, n):
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        ev0.record(stream)
        run()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n, time.perf_counter() - w0

    def eager_steps():
        for i in range(steps):
            layer.forward(step_x[i % len(step_x)])

    eager_ms, eager_wall = timed(eager_steps, steps)
    graph_ms = None
    if not eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager_steps()
        graph.replay()  # untimed replay
        torch.cuda.synchronize()
        graph_ms, graph_wall = timed(graph.replay, steps)
        stream = torch.cuda.current_stream()
        del graph
    ms_step, wall = (eager_ms, eager_wall) if graph_ms is None else (graph_ms, graph_wall)

    # ---- per-stage kernel times: each stage entry point is launched K times
    # back to back (one graph replay) between two HIP events on the launch
    # stream, so the queue stays full and the interval is the kernels' own
    # time (no host gaps).
    # The launches rotate over several input sets prepared by forwards of the
    # benchmark's own batches (decode: consecutive steps, so the expert
    # weights streamed change from launch to launch; prefill-like: the
    # rotated copies, so activations are not served from the last-level
    # cache).
    names = ["route", "dispatch", "expert_up", "expert_down", "combine"]
    rws, rbytes = b.scratch_view(cfg, "route"), moe.moe_workspace_size(cfg, moe.MOE_OP_ROUTE)
    dws = b.scratch_view(cfg, "dispatch")
    dbytes = moe.moe_workspace_size(cfg, moe.MOE_OP_DISPATCH_REROUTE if reroute else moe.MOE_OP_DISPATCH)
    Xp_ws, H_ws, Yp_ws = b.workspace_view(cfg, "Xp"), b.workspace_view(cfg, "H"), b.workspace_view(cfg, "Yp")
    nsets = min(len(xs), 4) if w.steps > 1 else len(xs)
    gathers = moe.moe_expert_up_gather_supported(cfg)
    sets, per_step_N, per_step_active = [], [], []
    for si in range(nsets):
        layer.forward(xs[si])
        torch.cuda.synchronize()
        sets.append({"X": xs[si], "ids": b.topk_ids.clone(), "w": b.topk_w.clone(), "off": b.expert_offsets.clone(),
                     "order": b.expert_order.clone() if reroute else None,
                     "inv": b.inv_perm.clone(), "perm": b.perm.clone(),
                     "Xp": None if gathers else Xp_ws.clone(), "H": H_ws.clone(), "Yp": Yp_ws.clone()})
        off = b.expert_offsets.cpu().numpy()
        per_step_N.append(int(off[-1]))
        per_step_active.append(int((np.diff(off) > 0).sum()))
    # The stages as moe_forward runs them: where the up-projection gathers X
    # through perm, the dispatch writes indices only.
    stage_fn = {
        "route": lambda q: moe.moe_route(cfg, q["X"], Wg, bias, b.topk_ids, b.topk_w, rws, rbytes),
        "dispatch": lambda q: moe.moe_dispatch(cfg, q["ids"], q["X"], b.expert_counts, b.expert_offsets, b.perm,
                                               b.inv_perm, None if gathers else Xp_ws, dws, dbytes),
        "expert_up": (lambda q: moe.moe_expert_up_gather(cfg, q["X"], q["perm"], q["off"], W1, q["H"])) if gathers
        else (lambda q: moe.moe_expert_up(cfg, q["Xp"], q["off"], W1, q["H"])),
        "expert_down": lambda q: moe.moe_expert_down(cfg, q["H"], q["off"], W2, q["Yp"]),
        "combine": lambda q: moe.moe_combine(cfg, q["Yp"], q["inv"], q["w"], b.out),
    }
    if reroute:
        stage_fn["route"] = lambda q: moe.moe_route_ranked(cfg, q["X"], Wg, bias, b.topk_ids, b.topk_w,
                                                           b.expert_order, rws, rbytes)
        stage_fn["dispatch"] = lambda q: moe.moe_dispatch_reroute(
            cfg, q["ids"], q["order"], q["X"], b.expert_counts, b.expert_offsets, b.perm, b.inv_perm,
            None if gathers else Xp_ws, dws, dbytes)
    # The K launches of a stage are captured in one HIP graph and replayed
    # (eager launches with --eager): a stage of microsecond kernels (decode)
    # would otherwise time the host's per-call overhead, not the kernels.
    stage_ms = {}
    nst = max(steps, nsets)
    for n in names:
        fn = stage_fn[n]
        fn(sets[0])  # untimed
        run_all = lambda: [fn(sets[i % nsets]) for i in range(nst)]  # noqa: E731
        if eager:
            stage_ms[n], _ = timed(run_all, nst)
        else:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_all()
            g.replay()  # untimed replay
            torch.cuda.synchronize()
            stage_ms[n], _ = timed(g.replay, nst)
            del g

    N = float(np.mean(per_step_N))
    active = float(np.mean(per_step_active))
    work = stage_work(w, N, active, es, gathers, reroute)
    stages = {}
    for n in names:
        ms = stage_ms[n]
        f, by = work[n]["flops"], work[n]["bytes"]
        stages[n] = {"ms": round(ms, 5), "tflops": round(f / ms / 1e9, 2) if f else 0.0,
                     "gbs": round(by / ms / 1e6, 1),
                     "frac_hbm": round(by / ms / 1e6 / PEAK_HBM_GBS, 4)}
        if n.startswith("expert"):
            peak = PEAK_BF16_TFLOPS if dt == "bf16" else PEAK_F32_TFLOPS
            stages[n]["frac_mfma"] = round(f / ms / 1e9 / peak, 4)
    dom = max(["expert_up", "expert_down"], key=lambda n: stage_ms[n])
    ms = stage_ms[dom]
    if w.steps > 1 or N / max(active, 1) < 64:
        roof = {"bound": "hbm", "achieved": round(work[dom]["bytes"] / ms / 1e6, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        peak = PEAK_BF16_TFLOPS if dt == "bf16" else PEAK_F32_TFLOPS
        roof = {"bound": "mfma", "achieved": round(work[dom]["flops"] / ms / 1e9, 2), "peak": peak,
                "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = gemm_traffic(w.name + ("_reroute" if reroute else ""), dom)
    roof["algorithmic_bytes"] = round(work[dom]["bytes"])
    roof["kernel"] = gemm_kernel_name(w, inp.expert_capacity, dom, gathers)
    roof["ms"] = round(ms, 5)

    cpu = None
    if with_cpu:
        cpu = cpu_baseline(w, inp, cpu_sample, reroute)
        if w.name == "tiny":
            # The tiny layer's oracle also on one core (BLAS limited to one thread).
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                one = cpu_baseline(w, inp, cpu_sample, reroute)
            one["cores"] = 1
            cpu["one_core"] = one

    res = {
        "value": round(w.T / (ms_step / 1e3), 1),
        "steps": steps,
        "ms_per_step": round(ms_step, 5),
        "timing": "hip-graph replay of the K steps" if graph_ms is not None else "eager launches",
        "eager_ms_per_step": round(eager_ms, 5),
        "config": {"workload": w.name + ("_rerouted" if reroute and inp.expert_capacity >= 0 else ""), "T": w.T,
                   "d": w.d, "E": w.E, "k": w.k, "F": w.F, "expert_capacity": inp.expert_capacity,
                   "over_capacity": ("rerouted" if reroute else "dropped") if inp.expert_capacity >= 0 else "none",
                   "bias": w.bias, "seed": w.seed, "parallelism": "single GPU, all experts resident"},
        "dtype": dt,
        "roofline": roof,
        "cpu_baseline": cpu,
        "stages": stages,
        "stage_input_sets": nsets,
        "kept_pairs": N,
        "active_experts": active,
        "wall_s_timed_region": round(wall, 4),
        "input_gen_s": round(gen_s, 2),
    }
    del layer, sets, xs, W1, W2
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def achievable_peaks(torch):
    """Peaks measured on this GPU beside the published ones: HBM from a plain
    1 GiB device-to-device copy (read plus write bytes) and a read-only sum
    over 2 GiB (the better of the two), and MFMA from a square
    8192 x 8192 x 8192 bf16 matrix product through torch (the vendor GEMM
    library), each timed with HIP events over back-to-back launches."""
    stream = torch.cuda.current_stream()

    def per_launch_ms(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps

    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    copy_ms = per_launch_ms(lambda: dst.copy_(src), 10)
    copy_gbs = 2 * src.numel() * 4 / copy_ms / 1e6
    del dst
    big = torch.ones(1 << 29, dtype=torch.float32, device="cuda")  # 2 GiB, read only
    acc = torch.empty((), dtype=torch.float32, device="cuda")
    read_ms = per_launch_ms(lambda: torch.sum(big, dim=0, out=acc), 10)
    read_gbs = big.numel() * 4 / read_ms / 1e6
    del src, big, acc
    n = 8192
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    a = torch.randn((n, n), device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn((n, n), device="cuda", generator=g).to(torch.bfloat16)
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    mm_ms = per_launch_ms(lambda: torch.mm(a, b, out=c), 20)
    tflops = 2.0 * n ** 3 / mm_ms / 1e9
    del a, b, c
    torch.cuda.empty_cache()
    return {"hbm_gbs": round(max(copy_gbs, read_gbs), 1), "hbm_copy_gbs": round(copy_gbs, 1),
            "hbm_read_gbs": round(read_gbs, 1), "bf16_gemm_tflops": round(tflops, 1),
            "method": "HBM: the better of a 1 GiB fp32 device copy (2 GiB moved) and a sum over 2 GiB of fp32, "
                      "10 launches each; MFMA: torch.mm bf16 8192^3, 20 launches; HIP events"}


def add_achievable(roof, ach):
    """The roofline's achieved rate as a fraction of the measured peak of its bound."""
    ref = ach["hbm_gbs"] if roof["bound"] == "hbm" else ach["bf16_gemm_tflops"]
    if roof["unit"] in ("GB/s", "TFLOP/s") and ref > 0 and (roof["bound"] == "hbm" or roof["peak"] == PEAK_BF16_TFLOPS):
        roof["frac_of_achievable"] = round(roof["achieved"] / ref, 4)


def main():
    args = parse()
    if args.calibrate_copy:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel() * 4, "copies": 5}))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs the layer on one GPU holding all experts; --gpus N>1 is not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import sparse_mixture_experts_04_amd as moe
    import workloads

    head = measure(torch, moe, workloads, args.workload, args.steps, args.warmup, eager=args.eager,
                   reroute=args.reroute, with_cpu=not args.no_cpu, cpu_sample=args.cpu_sample)
    print(f"[bench] {head['config']['workload']}: {head['value']:.1f} tokens/s, "
          f"{head['roofline']['kernel']} at {head['roofline']['frac']:.4f} of peak", file=sys.stderr, flush=True)
    others = {}
    if not args.no_others and not args.reroute and args.workload == "skewed":
        for name in ("prefill", "capacity", "decode"):
            r = measure(torch, moe, workloads, name, None, args.warmup, eager=args.eager)
            others[name] = {k: r[k] for k in ("value", "ms_per_step", "steps", "roofline", "stages", "kept_pairs",
                                              "active_experts", "stage_input_sets")}
            others[name]["unit"] = "tokens/s"
            others[name]["config"] = r["config"]
            print(f"[bench] {name}: {r['value']:.1f} tokens/s, {r['roofline']['kernel']} at "
                  f"{r['roofline']['frac']:.4f} of peak", file=sys.stderr, flush=True)

    ach = None
    if not args.no_achievable:
        ach = achievable_peaks(torch)
        for r in [head] + list(others.values()):
            add_achievable(r["roofline"], ach)
            for st in r["stages"].values():
                st["frac_of_achievable_hbm"] = round(st["gbs"] / ach["hbm_gbs"], 4)

    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "timing": head["timing"],
        "eager_ms_per_step": head["eager_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded; random-init weights of the stated shapes)",
        "config": head["config"],
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "achievable": ach,  # null with --no-achievable
        "stages": head["stages"],
        "stage_input_sets": head["stage_input_sets"],
        "kept_pairs": head["kept_pairs"],
        "active_experts": head["active_experts"],
        "wall_s_timed_region": head["wall_s_timed_region"],
        "input_gen_s": head["input_gen_s"],
    }
    if others:
        line["other_workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
