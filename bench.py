#!/usr/bin/env python3
"""Throughput of the Titans memory hot path (chunked update + retrieval) on one GPU.

One step = one titans_mem_forward call over the whole workload (every
stream, every chunk: coefficient scan, key forward, backprop, masked
retrieval, state fold).  Inputs are synthetic (seeded generator), resident
in HBM before the timed region; outputs are preallocated.

Prints ONE JSON line: memory tokens/s (B*H*N per step time), the roofline
of the dominant kernel measured with HIP events on the launch stream, and
the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks (dense matrix cores; fp32 matrix = fp32 vector peak)
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
WORKLOAD_NAMES = ("linear", "mlp2_short", "headline", "long", "deep")


# dominant kernel of each path: (kernel function, the sources under csrc/ it is built from)
DOMINANT_KERNEL = {"mlp2_d64_h256_mfma": ("mlp2_group_kernel", ("tm_mlp2_group.hip",)),
                   "generic_f32": ("generic_kernel", ("tm_generic.hip", "tm_block_gemm.h")),
                   "input_side": ("input_kernel", ("tm_input.hip",)),
                   "retrieve_mlp2": ("mlp2_retrieve_kernel", ("tm_retrieve.hip",)),
                   "backward": ("backward_kernel", ("tm_backward.hip", "tm_generic.hip", "tm_block_gemm.h")),
                   "deep_bf16_mfma": ("deep_read_kernel", ("tm_deep.hip",)),
                   "linear_f32": ("linear_kernel", ("tm_linear.hip",))}


def _source_digest(srcs):
    import hashlib
    h = hashlib.sha256()
    for src in srcs:
        with open(os.path.join(ROOT, "test_learned_neural_amd", "csrc", src), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _summary_fields(path):
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.split()[0] if v.split() else ""
    return fields


def committed_counters(kernel_path, workload):
    """Counter figures per launch of the path's dominant kernel on ``workload``
    from the committed rocprofv3 summaries in profiles/ (HBM bytes from the
    FETCH_SIZE and WRITE_SIZE passes, scaled by a plain copy's readings;
    executed matrix FLOPs from SQ_INSTS_MFMA), each only while the kernel
    source hash recorded in it matches the current sources; None otherwise.
    The counters are not re-read in the run: the JSON names their file."""
    out = {"traffic": None, "traffic_source": None, "mfma_flops": None, "mfma_source": None}
    if kernel_path not in DOMINANT_KERNEL:
        return out
    kernel, srcs = DOMINANT_KERNEL[kernel_path]
    digest = _source_digest(srcs)
    for kind, field, key in (("hbm_traffic", "hbm_bytes_per_launch", "traffic"),
                             ("sq_counters", "mfma_flops_per_launch", "mfma_flops")):
        rel = os.path.join("profiles", f"{kernel}__{workload}__{kind}.txt")
        path = os.path.join(ROOT, rel)
        if not os.path.exists(path):
            continue
        fields = _summary_fields(path)
        if fields.get("kernel_source_sha256") != digest:
            continue
        try:
            out[key] = float(fields[field])
        except (KeyError, ValueError):
            continue
        out[key.replace("flops", "source") if key == "mfma_flops" else "traffic_source"] = rel
    return out


def counter_fields(kernel_path, workload, launch_s, peak):
    """The roofline object's counter-derived entries: `traffic` (HBM bytes
    per launch, or null), `traffic_source` (the committed summary it comes
    from) and `counters` (executed MFMA rate and counted HBM rate over this
    run's launch time)."""
    c = committed_counters(kernel_path, workload)
    ctr = {}
    if c["mfma_flops"] is not None:
        t = c["mfma_flops"] / launch_s / 1e12
        ctr.update(mfma_executed_tflops=t, mfma_executed_frac=t / peak, mfma_source=c["mfma_source"])
    if c["traffic"] is not None:
        ctr["hbm_counted_gbs"] = c["traffic"] / launch_s / 1e9
    return {"traffic": c["traffic"], "traffic_source": c["traffic_source"], "counters": ctr or None}


def algorithmic_work(cfg):
    """(FLOPs, HBM bytes) per memory token (one token of one stream) of the
    chunked method: key forward P, backprop P - d*n_1, two weighted
    reductions 2P, and retrieval 2P + b * sum(n_{l-1} + n_l) MACs; bytes
    are k, v, q, y, the three gates, and the state read/written once."""
    w = cfg.widths
    P = cfg.param_count
    b = cfg.chunk
    upd = 4 * P - w[0] * w[1]
    ret = 2 * P + b * sum(w[i] + w[i + 1] for i in range(cfg.n_layers))
    flops = 2 * (upd + ret)
    esz = 2 if cfg.io == "bf16" else 4
    byts = 4 * cfg.d * esz + 3 * 4 + 4 * P * 4 / cfg.N
    return flops, byts


def input_side_work(icfg):
    """(FLOPs, HBM bytes) per launch of the input side: the projection GEMM
    [B*N x D] . [D x 3*(H*d + H)], and x, the weights, k, v, q (bf16) and
    the gates (fp32) moved once."""
    R, C = icfg.B * icfg.N, icfg.channels
    flops = 2.0 * R * icfg.D * (3 * C + 3 * icfg.H)
    byts = R * icfg.D * 2 + 3 * (C + icfg.H) * icfg.D * 2 + R * 3 * C * 2 + R * 3 * icfg.H * 4
    return flops, byts


def bench_input_side(args, np, torch, tmm, wl):
    """The step before the memory (x -> k, v, q and the gates) on the
    headline workload's input side; returns the JSON object describing it."""
    icfg = wl.INPUT_CONFIGS["headline"]
    inp = wl.make_input_side(icfg, workers=min(16, len(os.sched_getaffinity(0))))

    def bf(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    x, wp, wg = bf(inp["x"]), bf(inp["w_proj"]), bf(inp["w_gate"])
    cw, bg = torch.from_numpy(inp["conv_w"]).cuda(), torch.from_numpy(inp["b_gate"]).cuda()
    scales = tuple(float(v) for v in inp["gate_scale"])
    out = tmm.input_side(x, wp, cw, wg, bg, scales, H=icfg.H, d=icfg.d)
    stream = torch.cuda.current_stream()
    desc = tmm.make_input_desc(icfg.B, icfg.N, icfg.D, icfg.H, icfg.d, icfg.conv_width)
    ptrs = [x.data_ptr(), wp.data_ptr(), cw.data_ptr(), wg.data_ptr(), bg.data_ptr()]
    optrs = [t.data_ptr() for t in out]

    def step():
        rc = tmm.raw_input(desc, *ptrs, scales, *optrs, stream.cuda_stream)
        if rc != tmm.OK:
            raise tmm.TitansMemError(rc, "titans_mem_input")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    wall0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    launch_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    flops, byts = input_side_work(icfg)
    achieved = flops / launch_s / 1e12
    tokens = icfg.B * icfg.N
    res = {"workload": icfg.name, "value": tokens / (wall / args.steps), "unit": "tokens/s",
           "ms_per_step": wall * 1e3 / args.steps, "dtype": "bf16",
           "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                        "frac": achieved / PEAK_TFLOPS["bf16"],
                        **counter_fields("input_side", icfg.name, launch_s, PEAK_TFLOPS["bf16"]),
                        "algorithmic_flops_per_launch": flops, "avg_launch_ms": launch_s * 1e3,
                        "hbm_achieved_gbs": byts / launch_s / 1e9, "hbm_peak_gbs": PEAK_HBM_GBS}}
    print(f"[bench] input side {icfg.name}: {launch_s * 1e3:.3f} ms/launch, {achieved:.1f} TFLOP/s "
          f"({achieved / PEAK_TFLOPS['bf16'] * 100:.1f}% of bf16 peak)", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        import oracle
        el, done = 0.0, 0
        for b in range(icfg.B):   # whole sequences until about half the CPU budget is spent
            one = {k: (v[b:b + 1] if k == "x" else v) for k, v in inp.items()}
            f = wl.input_side_f64(one)
            t1 = time.perf_counter()
            oracle.input_side(f["x"], f["w_proj"], f["conv_w"], f["w_gate"], f["b_gate"], f["gate_scale"],
                              H=icfg.H, d=icfg.d)
            el += time.perf_counter() - t1
            done += 1
            if el > args.cpu_seconds / 2:
                break
        res["cpu_baseline"] = {"value": done * icfg.N / el, "unit": "tokens/s",
                               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                               "sample": f"{done} of {icfg.B} sequences x {icfg.N} tokens, fp64 numpy matmuls, "
                                         f"{el:.2f} s"}
    return res


def backward_flops_per_token(cfg):
    """Algorithmic FLOPs of titans_mem_backward per memory token, with dL/dy
    given and the read after each write: the chunked state sweep that yields
    the chunk-start states (key forward, backprop, the two weighted
    reductions: 8 P - 2 d n_1), and the chunk-wise reverse sweep's products
    (key forward and backprop again, the reads' forward and backward, the
    fold's adjoint, the inner gradient's backward pass and the two state
    adjoints: 32 P - 6 d n_1), plus the [b x b] score products of the reads,
    b per token times 2 (sum_l n_{l-1} + sum_{l<L} n_l) + 4 sum_l (n_l + n_{l-1})."""
    w = cfg.widths
    L = len(w) - 1
    P = cfg.param_count
    first = w[0] * w[1]
    b = min(cfg.chunk, cfg.N)
    sweep = 8 * P - 2 * first
    reverse = 32 * P - 6 * first
    scores = b * (2 * (sum(w[:L]) + sum(w[1:L])) + 4 * sum(w[l] + w[l - 1] for l in range(1, L + 1)))
    return sweep + reverse + scores


def bench_backward(args, np, torch, tmm, wl, prefix=1024, steps=3):
    """Gradients through the memory (titans_mem_backward) on the headline
    memory shape, every stream, the first `prefix` tokens."""
    full = wl.WORKLOADS[args.workload]
    cfg = full.with_(N=prefix)
    prefix_name = full.name.replace(f"_n{full.N}_", f"_n{prefix}_")   # e.g. ..._n1024_c64_bf16
    inp = wl.make_inputs(cfg, workers=min(16, len(os.sched_getaffinity(0))))
    B, H, N, d, P = cfg.B, cfg.H, cfg.N, cfg.d, cfg.param_count
    if cfg.io == "bf16":
        tok = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).reshape(B, H, N, d).cuda()
    else:
        tok = lambda a: torch.from_numpy(a).reshape(B, H, N, d).cuda()
    per = lambda a, n: torch.from_numpy(a).reshape(B, H, n).cuda()
    k, v, q = tok(inp["k"]), tok(inp["v"]), tok(inp["q"])
    al, et, th = per(inp["alpha"], N), per(inp["eta"], N), per(inp["theta"], N)
    W0, S0 = per(inp["W0"], P), per(inp["S0"], P)
    gen = torch.Generator(device="cuda").manual_seed(7)
    dy = torch.randn(B, H, N, d, device="cuda", generator=gen)
    run = lambda: tmm.backward(k, v, q, al, et, th, W0, S0, cfg.chunk, hidden=cfg.hidden, n_layers=cfg.n_layers,
                               dy=dy)
    run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    wall0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    launch_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    tokens = B * H * N
    flops = backward_flops_per_token(cfg) * tokens
    achieved = flops / launch_s / 1e12
    res = {"workload": f"{cfg.name} (first {prefix} tokens of every stream)", "value": tokens / (wall / steps),
           "unit": "memory-tokens/s", "ms_per_step": wall * 1e3 / steps, "dtype": "f32", "steps": steps,
           "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS["f32"], "unit": "TFLOP/s",
                        "frac": achieved / PEAK_TFLOPS["f32"],
                        **counter_fields("backward", prefix_name, launch_s, PEAK_TFLOPS["f32"]),
                        "algorithmic_flops_per_launch": flops, "avg_launch_ms": launch_s * 1e3}}
    print(f"[bench] backward {cfg.name}, {prefix} tokens: {launch_s * 1e3:.1f} ms/launch, "
          f"{tokens / launch_s:.3g} memory-tokens/s, {achieved:.2f} TFLOP/s fp32", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        import oracle
        el, done = 0.0, 0
        for b, h in wl.stream_ids(cfg):   # whole streams until about half the CPU budget is spent
            f = wl.inputs_f64(cfg, wl.make_inputs(cfg, streams=[(b, h)]))
            dyn = dy[b, h].double().cpu().numpy()[None]
            t1 = time.perf_counter()
            oracle.backward(f["k"], f["v"], f["q"], f["alpha"], f["eta"], f["theta"], f["W0"], f["S0"], dyn, None,
                            None, d=d, hidden=cfg.hidden, n_layers=cfg.n_layers, chunk=cfg.chunk)
            el += time.perf_counter() - t1
            done += 1
            if el > args.cpu_seconds / 2:
                break
        res["cpu_baseline"] = {"value": done * N / el, "unit": "memory-tokens/s", "cores": torch.get_num_threads(),
                               "kind": "oracle",
                               "sample": f"{done} of {B * H} streams x {N} tokens, fp64 torch reverse mode, {el:.2f} s"}
    return res


def bench_retrieve(args, np, torch, tmm, wl, steps=10):
    """Retrieval at a fixed state (titans_mem_retrieve): y = M_W(q) for every
    token of every stream of the workload, W = the workload's initial state."""
    cfg = wl.WORKLOADS[args.workload]
    inp = wl.make_inputs(cfg, workers=min(16, len(os.sched_getaffinity(0))))
    B, H, N, d, P = cfg.B, cfg.H, cfg.N, cfg.d, cfg.param_count
    if cfg.io == "bf16":
        q = torch.from_numpy(inp["q"].view(np.int16)).view(torch.bfloat16).reshape(B, H, N, d).cuda()
    else:
        q = torch.from_numpy(inp["q"]).reshape(B, H, N, d).cuda()
    W = torch.from_numpy(inp["W0"]).reshape(B, H, P).cuda()
    y = tmm.retrieve(q, W, hidden=cfg.hidden, n_layers=cfg.n_layers)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    wall0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        tmm.retrieve(q, W, hidden=cfg.hidden, n_layers=cfg.n_layers, y_out=y)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    launch_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    tokens = B * H * N
    w = cfg.widths
    flops = 2.0 * tokens * P                       # one memory forward per token
    esz = 2 if cfg.io == "bf16" else 4
    byts = 2.0 * tokens * d * esz + B * H * P * 4  # q in, y out, the state once
    mfma = tmm.select_path(tmm.make_desc(B, H, N, d, cfg.hidden, cfg.n_layers, cfg.io), cfg.chunk) == \
        tmm.PATH_MLP2_D64_H256
    dt = "bf16" if mfma else "f32"
    achieved = flops / launch_s / 1e12
    res = {"workload": cfg.name, "value": tokens / (wall / steps), "unit": "memory-tokens/s",
           "ms_per_step": wall * 1e3 / steps, "dtype": dt, "steps": steps,
           "roofline": {"bound": "mfma" if mfma else "alu", "achieved": achieved, "peak": PEAK_TFLOPS[dt],
                        "unit": "TFLOP/s", "frac": achieved / PEAK_TFLOPS[dt],
                        **(counter_fields("retrieve_mlp2", cfg.name, launch_s, PEAK_TFLOPS[dt]) if mfma
                           else {"traffic": None, "traffic_source": None, "counters": None}),
                        "algorithmic_flops_per_launch": flops, "avg_launch_ms": launch_s * 1e3,
                        "hbm_achieved_gbs": byts / launch_s / 1e9, "hbm_peak_gbs": PEAK_HBM_GBS}}
    print(f"[bench] retrieve {cfg.name}: {launch_s * 1e3:.3f} ms/launch, {tokens / launch_s:.3g} memory-tokens/s, "
          f"{achieved:.1f} TFLOP/s", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        import oracle
        t1 = time.perf_counter()
        n = 0
        for s in range(B * H):   # whole streams, token by token, until about a quarter of the CPU budget
            Wn = inp["W0"][s].astype(np.float64)
            qn = wl.io_to_f64(inp["q"][s], cfg.io)
            for t in range(N):
                oracle.memory_apply(Wn, qn[t], d, cfg.hidden, cfg.n_layers)
            n += N
            if time.perf_counter() - t1 > args.cpu_seconds / 4:
                break
        el = time.perf_counter() - t1
        res["cpu_baseline"] = {"value": n / el, "unit": "memory-tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n // N} of {B * H} streams x {N} tokens, fp64 C memory forward, "
                                         f"{el:.2f} s"}
    return res


def bench_workloads(args, np, torch, tmm, wl):
    """Every other memory workload (the linear fp32 memory, 32 streams x
    4096, 16 streams x 1,048,576 tokens, the 4-layer deep memory): one
    warmup and two timed titans_mem_forward calls each, with HIP events on
    the launch stream; inputs resident in HBM.  Returns a list of objects
    (workload, kernel path, ms per call, memory-tokens/s, algorithmic
    roofline fraction against the path's peak)."""
    dev = torch.device("cuda:0")
    paths = {tmm.PATH_GENERIC_F32: ("generic_f32", "f32"), tmm.PATH_MLP2_D64_H256: ("mlp2_d64_h256_mfma", "f16"),
             tmm.PATH_DEEP_BF16: ("deep_bf16_mfma", "bf16")}
    out = []
    for name in ("linear", "mlp2_short", "long", "deep"):
        if name == args.workload:
            continue
        cfg = wl.WORKLOADS[name]
        t0 = time.time()
        inp = wl.make_inputs(cfg, workers=min(16, len(os.sched_getaffinity(0))))
        B, H, N, d, P = cfg.B, cfg.H, cfg.N, cfg.d, cfg.param_count

        def tok(a):
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if cfg.io == "bf16" else torch.from_numpy(a)
            return t.reshape(B, H, N, d).to(dev)

        def per(a, n):
            return torch.from_numpy(a).reshape(B, H, n).to(dev)

        k, v, q = tok(inp["k"]), tok(inp["v"]), tok(inp["q"])
        alpha, eta, theta = per(inp["alpha"], N), per(inp["eta"], N), per(inp["theta"], N)
        W0, S0 = per(inp["W0"], P), per(inp["S0"], P)
        del inp
        y, W_out, S_out = torch.empty_like(k), torch.empty_like(W0), torch.empty_like(S0)
        desc = tmm.make_desc(B, H, N, d, cfg.hidden, cfg.n_layers, cfg.io)
        path = tmm.select_path(desc, cfg.chunk)
        ws_bytes = tmm.workspace_bytes(desc, cfg.chunk)
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream(dev)

        def step():
            rc = tmm.raw_forward(desc, k.data_ptr(), v.data_ptr(), q.data_ptr(), alpha.data_ptr(), eta.data_ptr(),
                                 theta.data_ptr(), W0.data_ptr(), S0.data_ptr(), cfg.chunk, y.data_ptr(),
                                 W_out.data_ptr(), S_out.data_ptr(), ws.data_ptr(), ws_bytes, stream.cuda_stream)
            if rc != tmm.OK:
                raise tmm.TitansMemError(rc, "titans_mem_forward")

        step()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2)]
        for a, b in ev:
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        flops_tok, _ = algorithmic_work(cfg)
        pname, dt = paths.get(path, (str(path), "f32"))
        tflops = flops_tok * B * H * N / (ms / 1e3) / 1e12
        res = {"workload": cfg.name, "kernel_path": pname, "ms_per_call": ms,
               "memory_tokens_per_s": B * H * N / (ms / 1e3), "achieved_tflops": tflops,
               "peak_tflops": PEAK_TFLOPS[dt], "frac": tflops / PEAK_TFLOPS[dt]}
        out.append(res)
        print(f"[bench] {cfg.name}: {ms:.3f} ms per call on {pname} ({res['memory_tokens_per_s']:.3g} memory-tokens/s, "
              f"{tflops / PEAK_TFLOPS[dt] * 100:.1f}% of {dt} peak; inputs {time.time() - t0:.1f} s)",
              file=sys.stderr, flush=True)
        del k, v, q, alpha, eta, theta, W0, S0, y, W_out, S_out, ws
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="headline", choices=sorted(WORKLOAD_NAMES),
                    help="memory workload (default: the 2-layer d=64 h=256 memory over 128 streams x 16384 tokens)")
    ap.add_argument("--force-generic", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-input-side", action="store_true", help="skip the input-side leg")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-retrieve", action="store_true", help="skip the fixed-state retrieval leg")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other memory workloads (one line each in the `workloads` list)")
    ap.add_argument("--retrieve-only", action="store_true",
                    help="time only the fixed-state retrieval (titans_mem_retrieve) and print its JSON line")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the backward (gradients through the memory) and print its JSON line")
    ap.add_argument("--input-side-only", action="store_true",
                    help="time only the input side (x -> k, v, q, gates) and print its JSON line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES (three times), to scale "
                         "HBM byte counters, and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the memory's (batch, head) streams are independent "
              "and this benchmark runs them on a single device; --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        src = torch.empty(args.calibrate_copy, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": args.calibrate_copy, "copies": 3}))
        return

    from test_learned_neural_amd import titans_mem as tmm
    from test_learned_neural_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tmm.load()
    if args.retrieve_only:
        print(json.dumps({"metric": "retrieval memory tokens/sec at a fixed state, 1 GPU", "n_gpus": 1,
                          "higher_is_better": True, "data": "synthetic",
                          **bench_retrieve(args, np, torch, tmm, wl)}), flush=True)
        return
    if args.backward_only:
        print(json.dumps({"metric": "backward memory tokens/sec (gradients through the memory), 1 GPU", "n_gpus": 1,
                          "higher_is_better": True, "data": "synthetic",
                          **bench_backward(args, np, torch, tmm, wl)}), flush=True)
        return
    if args.input_side_only:
        print(json.dumps({"metric": "input-side tokens/sec (x -> k, v, q, gates), 1 GPU", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                          "data": "synthetic", **bench_input_side(args, np, torch, tmm, wl)}), flush=True)
        return
    cfg = wl.WORKLOADS[args.workload]
    t0 = time.time()
    inp = wl.make_inputs(cfg, workers=min(16, len(os.sched_getaffinity(0))))
    print(f"[bench] generated {cfg.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    B, H, N, d, P = cfg.B, cfg.H, cfg.N, cfg.d, cfg.param_count

    def tok(a):
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if cfg.io == "bf16" else torch.from_numpy(a)
        return t.reshape(B, H, N, d).to(dev)

    def per(a, n):
        return torch.from_numpy(a).reshape(B, H, n).to(dev)

    k, v, q = tok(inp["k"]), tok(inp["v"]), tok(inp["q"])
    alpha, eta, theta = per(inp["alpha"], N), per(inp["eta"], N), per(inp["theta"], N)
    W0, S0 = per(inp["W0"], P), per(inp["S0"], P)
    y = torch.empty_like(k)
    W_out = torch.empty_like(W0)
    S_out = torch.empty_like(S0)
    flags = tmm.FLAG_FORCE_GENERIC if args.force_generic else 0
    desc = tmm.make_desc(B, H, N, d, cfg.hidden, cfg.n_layers, cfg.io, flags=flags)
    path = tmm.select_path(desc, cfg.chunk)
    ws_bytes = tmm.workspace_bytes(desc, cfg.chunk)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        rc = tmm.raw_forward(desc, k.data_ptr(), v.data_ptr(), q.data_ptr(), alpha.data_ptr(),
                             eta.data_ptr(), theta.data_ptr(), W0.data_ptr(), S0.data_ptr(), cfg.chunk,
                             y.data_ptr(), W_out.data_ptr(), S_out.data_ptr(), ws.data_ptr(), ws_bytes,
                             stream.cuda_stream)
        if rc != tmm.OK:
            raise tmm.TitansMemError(rc, "titans_mem_forward")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = wall * 1e3 / args.steps
    mem_tokens = B * H * N
    value = mem_tokens / (ms_per_step / 1e3)
    flops_tok, bytes_tok = algorithmic_work(cfg)
    avg_launch_s = float(np.mean(launch_ms)) / 1e3
    # the arithmetic type of each path's products: fp32 (generic), scaled fp16
    # operands (the 2-layer d=64 kernel), bf16 operands (deep memories); sums fp32
    dtype = {tmm.PATH_GENERIC_F32: "f32", tmm.PATH_MLP2_D64_H256: "f16", tmm.PATH_DEEP_BF16: "bf16"}[path]
    achieved = flops_tok * mem_tokens / avg_launch_s / 1e12
    peak = PEAK_TFLOPS[dtype]
    bound = "mfma"   # every path runs its contractions on the matrix cores
    print(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step, event avg {np.mean(launch_ms):.3f} ms, "
          f"min {np.min(launch_ms):.3f} ms; {achieved:.1f} TFLOP/s; HBM {bytes_tok * mem_tokens / avg_launch_s / 1e9:.0f} GB/s",
          file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        f = wl.inputs_f64(cfg, {kk: vv for kk, vv in inp.items()})
        done = 0
        elapsed = 0.0
        streams_total = B * H
        batch = min(cores, streams_total)
        while done < streams_total and elapsed < args.cpu_seconds:
            sl = slice(done, min(done + batch, streams_total))
            t1 = time.perf_counter()
            oracle.forward(f["k"][sl], f["v"][sl], f["q"][sl], f["alpha"][sl], f["eta"][sl], f["theta"][sl],
                           f["W0"][sl], f["S0"][sl], d=d, hidden=cfg.hidden, n_layers=cfg.n_layers,
                           chunk=cfg.chunk, threads=batch)
            elapsed += time.perf_counter() - t1
            done = sl.stop
        cpu = {"value": done * N / elapsed, "unit": "memory-tokens/s", "cores": batch, "kind": "oracle",
               "sample": f"{done} of {streams_total} streams x {N} tokens, fp64 token-by-token, "
                         f"{batch} OpenMP threads, {elapsed:.1f} s"}
        print(f"[bench] cpu oracle: {cpu['value']:.3g} memory-tokens/s ({cpu['sample']})", file=sys.stderr,
              flush=True)

    kernel_path_name = {tmm.PATH_GENERIC_F32: "generic_f32",
                        tmm.PATH_MLP2_D64_H256: "mlp2_d64_h256_mfma",
                        tmm.PATH_DEEP_BF16: "deep_bf16_mfma"}.get(path, str(path))
    if path == tmm.PATH_GENERIC_F32 and cfg.n_layers == 1 and cfg.d <= 64 and cfg.d % 4 == 0 and cfg.chunk <= 64:
        kernel_path_name = "linear_f32"   # the generic path's linear-memory kernel
    out = {
        "metric": "memory tokens/sec (retrieve + chunked update), 1 GPU",
        "value": value,
        "unit": "memory-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "H": H, "N": N, "d": d, "hidden": cfg.hidden,
                   "n_layers": cfg.n_layers, "chunk": cfg.chunk, "io": cfg.io,
                   "kernel_path": kernel_path_name,
                   "sequence_tokens_per_s": B * N / (ms_per_step / 1e3)},
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, **counter_fields(kernel_path_name, cfg.name, avg_launch_s, peak),
                     "algorithmic_flops_per_launch": flops_tok * mem_tokens,
                     "avg_launch_ms": avg_launch_s * 1e3,
                     "hbm_achieved_gbs": bytes_tok * mem_tokens / avg_launch_s / 1e9,
                     "hbm_peak_gbs": PEAK_HBM_GBS},
        "cpu_baseline": cpu,
    }
    if not args.no_input_side:
        out["input_side"] = bench_input_side(args, np, torch, tmm, wl)
    if not args.no_retrieve:
        out["retrieve"] = bench_retrieve(args, np, torch, tmm, wl)
    if not args.no_backward:
        out["backward"] = bench_backward(args, np, torch, tmm, wl)
    if not args.no_workloads:
        out["workloads"] = bench_workloads(args, np, torch, tmm, wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
