"""Benchmark of the fused MoE-LoRA layer on one MI355X.

One step = one full layer call (route, align, gate_up shrink, gate_up GEMM +
expand + SiLU*up, down shrink, down GEMM + expand, top-k combine) on one
batch of seeded synthetic input already resident in HBM.  Prints one JSON
line with tokens/s, the roofline of the dominant kernel (timed live with
HIP events on the stream it runs on) and the CPU oracle's rate on a bounded
sample of the same workload, single-threaded and on all host cores.

The headline metric has two halves: HBM bandwidth for decode-sized batches
(the default workload, whose tokens/s is `value`) and MFMA utilisation for
prefill-sized batches; the default run therefore also times the 6400-token
prefill workload and reports it as the nested `prefill` object.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "MoE-LoRA layer tokens/s; achieved HBM GB/s (decode) / MFMA % of peak (prefill)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense; f32 = vector peak
STAGES = ("route_align", "shrink_gate_up", "gate_up", "shrink_down", "down", "combine")
DEFAULT_WORKLOAD = "decode_bf16"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=[w.name for w in synth.WORKLOADS])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-lora", action="store_true",
                    help="base MoE only: no LoRA pointers (the layer's early exit)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--prefill-steps", type=int, default=20,
                    help="timed calls of the prefill leg (0: no prefill leg)")
    ap.add_argument("--prefill-warmup", type=int, default=5)
    ap.add_argument("--fp8-steps", type=int, default=200,
                    help="timed calls of the E4M3-weight decode leg (0: none)")
    return ap.parse_args()


def _code_only(text):
    """Source text without comments and whitespace (kernel code is not
    expected to hold "//" or "/*" inside string literals)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return re.sub(r"\s+", "", text)


def kernel_source_hash(csrc=None):
    """Hash of the device-kernel code (everything in csrc but the host ABI
    file, comments and whitespace ignored), used to tell whether committed
    counters still apply."""
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "lora_expert_gemm_amd", "csrc")
    for n in sorted(os.listdir(csrc)):
        if n == "api.hip":
            continue
        with open(os.path.join(csrc, n)) as f:
            h.update(n.encode() + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, stage):
    """HBM bytes per launch of the kernel that ran `stage` (e.g. "gate_up")
    from the committed rocprofv3 counter summary (profiles/hbm_traffic.json),
    or None when there is none for this workload or the kernel sources
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source") != kernel_source_hash():
        return None
    v = t.get("workloads", {}).get(workload, {}).get(stage)
    return v["bytes"] if v else None


def hbm_bound(alg, stage, dtype):
    """Whether a stage is bound by HBM: its algorithmic FLOPs per byte below
    the ridge point (peak FLOP/s over peak bytes/s of the dtype's MFMA)."""
    ridge = MFMA_PEAK_TFLOPS[dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    return alg[f"{stage}_flop"] < ridge * alg[f"{stage}_bytes"]


def algorithmic(w, ids, aid, row_mode=False):
    """Bytes and FLOPs the method must move / compute for one call: weights of
    the experts and (adapter, expert) pairs routed to, x read, out written;
    FLOPs of the routed rows (padding and elementwise work excluded).  Per
    kernel: gate_up holds the base GEMM and the expand (its shrink runs
    before it); the down launch holds the base GEMM and the expand, or, with
    row-wise LoRA, the base GEMM and the down shrink (the expand then runs in
    the combine)."""
    s = 2 if w.dtype == "bf16" else 4
    sw = 1 if w.wdtype == "fp8" else s     # bytes of a base-weight element
    sc = 4 if w.wdtype == "fp8" else 0     # bytes of a row scale
    T, H, I, k, r = w.T, w.H, w.I, w.k, w.r
    valid = (ids >= 0) & (ids < w.E)
    experts = np.unique(ids[valid])
    tok_a = np.repeat(aid[:, None], k, axis=1)
    lora_rows = valid & (tok_a >= 0) & (tok_a < w.NA)
    pairs = np.unique(np.stack([tok_a[lora_rows], ids[lora_rows]], 1), axis=0) \
        if lora_rows.any() else np.zeros((0, 2))
    n_exp, n_pair, R, R_lora = len(experts), len(pairs), int(valid.sum()), int(lora_rows.sum())
    layer_bytes = n_exp * (3 * H * I * sw + (2 * I + H) * sc) + \
        s * (n_pair * r * (2 * H + 3 * I) + 2 * T * H)
    layer_flop = R * 6 * H * I + R_lora * 2 * r * (2 * H + 3 * I)
    # the dominant kernels: gate_up (base 2I x H per expert, expand 2I x r per
    # pair, x in, h out, z in) and down (H x I per expert, H x r per pair, h in,
    # y out)
    gu_bytes = n_exp * 2 * I * (H * sw + sc) + s * (n_pair * 2 * I * r + T * H + R * I) + \
        4 * R_lora * r
    gu_flop = R * 4 * H * I + R_lora * 4 * I * r
    if row_mode:  # A_d read, z_d written by the shrinks riding along
        dn_bytes = n_exp * H * (I * sw + sc) + s * (n_pair * I * r + R * I) + 4 * R * H + \
            4 * R_lora * r
        dn_flop = R * 2 * H * I + R_lora * 2 * I * r
    else:         # B_d read, z_d read by the expand
        dn_bytes = n_exp * H * (I * sw + sc) + s * (n_pair * H * r + R * I) + 4 * R * H + \
            4 * R_lora * r
        dn_flop = R * 2 * H * I + R_lora * 2 * H * r
    return dict(n_exp=n_exp, n_pair=n_pair, R=R, R_lora=R_lora, layer_bytes=layer_bytes,
                layer_flop=layer_flop, gate_up_bytes=gu_bytes, gate_up_flop=gu_flop,
                down_bytes=dn_bytes, down_flop=dn_flop)


def copy_calibration(mib):
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: 5 copies of {n} bytes")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, d, target_s):
    """The oracle (float64 C) on a bounded sample of the workload, once on one
    thread and once on every thread OpenMP gives it (tokens spread over
    threads, each token's arithmetic unchanged): its first n tokens, n
    chosen so each run takes about target_s / 2 seconds; when the whole
    workload is quicker than that, whole passes are repeated.  `value` and
    `cores` are the all-thread run's."""
    import oracle
    dt = oracle.BF16 if w.dtype == "bf16" else oracle.F32
    ids, wts = oracle.ref_route(d["logits"], w.k)

    def run(tokens):
        t0 = time.perf_counter()
        oracle.ref_forward(d["x"], ids, wts, d["adapter_ids"], d["W_gu"], d["W_d"],
                           d["A_gu"], d["B_gu"], d["A_d"], d["B_d"], inter=w.I, rank=w.r,
                           n_adapters=w.NA, dtype=dt, tokens=np.asarray(tokens, np.int32))
        return time.perf_counter() - t0

    def timed(threads, budget):
        used = oracle.set_threads(threads)
        t1 = run(list(range(min(w.T, used))))
        per_tok = t1 / min(w.T, used) * used   # one token's time on one thread
        n = int(max(1, min(w.T, budget / max(per_tok, 1e-6) * used)))
        el, passes = 0.0, 0
        while passes == 0 or (n == w.T and el < budget):
            el += run(list(range(n)))
            passes += 1
        what = f"tokens 0..{n - 1} of {w.T}" if n < w.T else f"all {w.T} tokens x {passes} passes"
        return used, n * passes / el, f"{what} of {w.name}; {el:.1f} s"

    try:
        _, v1, s1 = timed(1, target_s / 2)
        used, vn, sn = timed(0, target_s / 2)
    finally:
        oracle.set_threads(0)
    return {"value": vn, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"oracle (C, float64, OpenMP over tokens, {used} threads) on {sn}",
            "single_thread": {"value": v1, "cores": 1,
                              "sample": f"oracle (C, float64, 1 thread) on {s1}"},
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0))}


def ceilings(torch, stream):
    """What the same device reaches on plain work, timed here for context: a
    read-only stream (the vendor bf16 GEMV, torch.mv, over a 2 GiB matrix of
    131072 x 8192: bytes read per second; it out-streams torch's
    reductions, which reach 3.7-5.6 TB/s on the same bytes), a 1 GiB device
    copy (bytes read + written per second) and a bf16 8192^3 torch.matmul
    (the vendor GEMM)."""
    res = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def rate(fn, n, bytes_per):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return bytes_per * n / (e0.elapsed_time(e1) / 1e3)

    try:
        m = torch.ones((1 << 17, 8192), dtype=torch.bfloat16, device="cuda")   # 2 GiB
        v = torch.ones(8192, dtype=torch.bfloat16, device="cuda")
        res["read_GB/s"] = rate(lambda: torch.mv(m, v), 10, m.numel() * 2) / 1e9
        del m, v
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        res["copy_GB/s"] = rate(lambda: b.copy_(a), 10, 2 * a.numel()) / 1e9
        del a, b
        n = 8192
        x = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        y = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        res["gemm_bf16_TFLOP/s"] = rate(lambda: torch.matmul(x, y), 10, 2 * n ** 3) / 1e12
        del x, y
    except Exception as ex:  # context only
        res["error"] = str(ex)
    log(f"[bench] ceilings: {res}")
    return res


def graph_replay(torch, step, stream, steps):
    """The same layer call captured once in a HIP graph (no per-kernel launch
    cost on replay) and replayed `steps` times; ms per replay, or the error."""
    try:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()  # default priority
        cap.wait_stream(stream)
        with torch.cuda.graph(g, stream=cap):
            step(cap)
        stream.wait_stream(cap)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        log(f"[bench] hipGraph replay: {ms:.4f} ms/step")
        return {"ms_per_step": ms}
    except Exception as ex:  # reported, not fatal: the eager timing is the result
        log(f"[bench] hipGraph capture failed: {ex}")
        return {"ms_per_step": None, "error": str(ex)}


def measure(torch, L, w, steps, warmup, no_lora=False, graph_steps=None):
    """Time `steps` layer calls of workload w (after `warmup`), then the same
    calls with the library's per-stage events and as a hipGraph replay;
    returns the timings, the algorithmic counts of the call and the roofline
    of its dominant kernel."""
    log(f"[bench] generating {w}")
    d = synth.make_inputs(w)
    dtype = L.BF16_FP8W if w.wdtype == "fp8" else L.BF16 if w.dtype == "bf16" else L.F32
    plan = L.Plan(w.T, w.H, w.I, w.E, w.k, w.NA, w.r, dtype)
    info = plan.info(w.T)
    log(f"[bench] plan: {info}")

    def dev(a):
        a = a.view(np.int16) if a.dtype == np.uint16 else a
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    t = {n: dev(v) for n, v in d.items() if v is not None and not n.endswith("_scale")}
    if w.wdtype == "fp8":  # E4M3 codes and row scales in the ABI's one-buffer layout
        for n in ("W_gu", "W_d"):
            t[n] = dev(L.fp8_weight_buffer(d[n], d[n + "_scale"]))
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((w.T, w.H), dtype=torch.int16 if w.dtype == "bf16" else torch.float32,
                      device="cuda")
    stream = torch.cuda.current_stream()
    lora = [None] * 4 if no_lora else [t["A_gu"], t["B_gu"], t["A_d"], t["B_d"]]

    def step(st=None):
        L.moelora_forward(plan.handle, w.T, t["x"], t["logits"], None, None, t["adapter_ids"],
                          t["W_gu"], t["W_d"], *lora, out, ws, plan.workspace_bytes,
                          (st or stream).cuda_stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = ev0.elapsed_time(ev1) / steps
    log(f"[bench] {w.name}: {steps} steps: {ms:.4f} ms/step (wall {wall:.3f} s)")

    # per-stage times: events recorded by the library around each kernel
    # stage on the forward's own stream
    L.moelora_timing_begin(plan.handle, steps)
    for _ in range(steps):
        step()
    st_ms, n_calls = L.moelora_timing_end(plan.handle)
    stage = {n: v / n_calls for n, v in zip(STAGES, st_ms)}
    log("[bench] stages (ms/call): " + ", ".join(f"{n}={v:.4f}" for n, v in stage.items()))
    graph = graph_replay(torch, step, stream, graph_steps or steps)

    lay = plan.layout(w.T)
    torch.cuda.synchronize()
    ids = ws[lay["off_topk_ids"]: lay["off_topk_ids"] + 4 * w.T * w.k].cpu().numpy() \
        .view(np.int32).reshape(w.T, w.k)
    alg = algorithmic(w, ids, d["adapter_ids"] if not no_lora else np.full(w.T, -1, np.int32),
                      "lora_mode=row" in info)
    dom = max(("gate_up", "down"), key=lambda n: stage[n])
    roof = {**roofline(alg, dom, stage[dom], w.dtype), "kernel": dom,
            "traffic": None if no_lora else measured_traffic(w.name, dom),
            "launch_ms": stage[dom],
            "units_per_launch": {"experts": alg["n_exp"], "adapter_expert_pairs": alg["n_pair"],
                                 "routed_rows": alg["R"]}}
    layer_s = ms / 1e3
    layer = {"algo_bytes": alg["layer_bytes"], "algo_flop": alg["layer_flop"],
             "GB/s": alg["layer_bytes"] / layer_s / 1e9,
             "TFLOP/s": alg["layer_flop"] / layer_s / 1e12,
             "hbm_frac": alg["layer_bytes"] / layer_s / 1e9 / HBM_PEAK_GBS,
             "mfma_frac": alg["layer_flop"] / layer_s / 1e12 / MFMA_PEAK_TFLOPS[w.dtype]}
    kernels = {k: roofline(alg, k, stage[k], w.dtype) for k in ("gate_up", "down") if stage[k] > 0}
    del t, ws, out
    return dict(w=w, d=d, ms=ms, stage=stage, graph=graph, alg=alg, roof=roof, layer=layer,
                kernels=kernels, plan=info)


def roofline(alg, kernel, launch_ms, dtype):
    """Achieved rate of one kernel against the roofline its algorithmic
    intensity puts it under (HBM bytes, or MFMA FLOPs of the layer dtype)."""
    sec = launch_ms / 1e3
    if hbm_bound(alg, kernel, dtype):
        r = {"bound": "hbm", "achieved": alg[f"{kernel}_bytes"] / sec / 1e9,
             "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        r = {"bound": "mfma", "achieved": alg[f"{kernel}_flop"] / sec / 1e12,
             "peak": MFMA_PEAK_TFLOPS[dtype], "unit": "TFLOP/s"}
    r["frac"] = r["achieved"] / r["peak"]
    return r


def config_of(w, no_lora=False):
    return {"workload": w.name, "T": w.T, "H": w.H, "I": w.I, "E": w.E, "top_k": w.k,
            "adapters": w.NA, "rank": w.r,
            "adapter_ids": "none (no LoRA)" if no_lora else w.adapters}


def main():
    args = parse()
    if args.gpus != 1:
        log(f"bench.py measures one GPU only (the layer has no multi-GPU path; how it would "
            f"shard is described with the design); --gpus {args.gpus} is not supported")
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calib:
        copy_calibration(args.copy_calib)
        return
    import lora_expert_gemm_amd as L

    w = synth.workload(args.workload)
    m = measure(torch, L, w, args.steps, args.warmup, args.no_lora)
    ceil = ceilings(torch, torch.cuda.current_stream())
    roof = m["roof"]
    ref = ceil.get("read_GB/s" if roof["bound"] == "hbm" else "gemm_bf16_TFLOP/s")
    roof["frac_of_measured_ceiling"] = roof["achieved"] / ref if ref else None
    res = {
        "metric": METRIC,
        "value": w.T / (m["ms"] / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": config_of(w, args.no_lora),
        "roofline": roof,
        "layer": m["layer"],
        "kernels": m["kernels"],
        "stages_ms": m["stage"],
        "graph": m["graph"],
        "ceilings": ceil,
        "plan": m["plan"],
        "kernel_source": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline(w, m["d"], args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    del m
    if args.workload == DEFAULT_WORKLOAD and args.prefill_steps > 0 and not args.no_lora:
        # the metric's other half: MFMA utilisation of the prefill-sized batch
        pw = synth.workload("prefill_bf16")
        p = measure(torch, L, pw, args.prefill_steps, args.prefill_warmup)
        pr = p["roof"]
        pr["frac_of_measured_ceiling"] = (pr["achieved"] / ceil["gemm_bf16_TFLOP/s"]
                                          if ceil.get("gemm_bf16_TFLOP/s") else None)
        res["prefill"] = {
            "config": config_of(pw), "steps": args.prefill_steps,
            "warmup": args.prefill_warmup, "ms_per_step": p["ms"],
            "tokens_per_s": pw.T / (p["ms"] / 1e3), "roofline": pr, "layer": p["layer"],
            "kernels": p["kernels"], "stages_ms": p["stage"], "graph": p["graph"],
            "plan": p["plan"]}
        log(f"[bench] prefill: {p['ms']:.4f} ms/step, gate_up {pr['achieved']:.0f} TFLOP/s "
            f"({pr['frac']:.3f} of peak), layer {p['layer']['mfma_frac']:.3f} of MFMA peak")
    if args.workload == DEFAULT_WORKLOAD and args.fp8_steps > 0 and not args.no_lora:
        # the same decode step with E4M3 base weights and row scales
        fw = synth.workload("decode_fp8w")
        f = measure(torch, L, fw, args.fp8_steps, args.warmup)
        res["decode_fp8w"] = {
            "config": config_of(fw), "weights": "E4M3 codes + float32 row scales",
            "steps": args.fp8_steps, "ms_per_step": f["ms"], "tokens_per_s": fw.T / (f["ms"] / 1e3),
            "roofline": f["roof"], "layer": f["layer"], "kernels": f["kernels"],
            "stages_ms": f["stage"], "plan": f["plan"]}
        log(f"[bench] decode_fp8w: {f['ms']:.4f} ms/step, {f['roof']['kernel']} "
            f"{f['roof']['achieved']:.0f} GB/s ({f['roof']['frac']:.3f} of peak)")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
