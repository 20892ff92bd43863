#!/usr/bin/env python3
"""Throughput of one ZONOS2 MoE feed-forward layer forward on one MI355X.

A step is one forward of the whole layer (RMSNorm + router + top-k, dispatch
permutation, grouped SwiGLU experts, combine) over one batch of seeded
synthetic hidden states, through the C ABI of libmoe_layer.so.  Inputs are
resident in HBM before timing starts.  Several independently allocated
copies of the layer are used in rotation so that consecutive steps do not
find the previous step's 576 MiB of expert weights in the 256 MiB MALL, as
consecutive MoE layers of the backbone would not.

Prints ONE JSON line: the metric, the step time, a roofline entry for the
dominant kernel (its algorithmic bytes or flops per launch over its average
duration, from HIP events recorded by the library on the forward's stream)
and the fp64 CPU oracle's throughput on a bounded sample of the same workload,
with the oracle's routing of every benched batch checked against the GPU's
(near-ties counted and reported).  The default line (the decode workload)
also carries `prefill`: the T=4096 and T=16384 prefill workloads' step time,
tokens/s, whole-layer fraction of the bf16 MFMA peak and their gate/up
grouped GEMM's time and fraction.

With --fp8 the expert weights are E4M3 codes with per-row fp32 scales
(moe_layer_create_fp8): decode streams half the weight bytes.  With --w8a8
the activations are quantised to E4M3 as well (moe_layer_create_w8a8) and the
expert GEMMs run on the fp8 MFMA, priced against the dense fp8 peak.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config {0,1,2,3,4}]
                       [--fp8 | --w8a8]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
import warnings

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
METRIC = "MoE-layer tokens/s at 1 GPU; HBM GB/s (decode) and MFMA % of peak (prefill)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# sources that decide the dominant kernel's memory traffic (its counters are
# void once any of them changes)
DOMINANT_SOURCES = {"k_gateup_stream": ["k_expert_stream.hip", "common.hpp", "kernels.hpp"],
                    "k_gateup_f32": ["k_expert_f32.hip", "common.hpp", "kernels.hpp"],
                    "k_expert_gemm<0>": ["k_expert_gemm.hip", "common.hpp", "kernels.hpp"]}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_ffn_amd", "csrc")
    for f in DOMINANT_SOURCES[kernel]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def dominant_kernel_name(cfg, act8: bool = False) -> str:
    if cfg.dtype == "f32":
        return "k_gateup_f32"
    return "k_gateup_stream" if cfg.T * cfg.k <= 64 else "k_expert_gemm<0>"


def kernel_short_name(name: str) -> str:
    """'void moe::k_x<0, moe::(anonymous namespace)::Geo<8, 1> >(args)' -> 'k_x<0, Geo<8, 1> >'."""
    import re
    name = re.sub(r"^void ", "", name).replace("(anonymous namespace)::", "")
    depth, end = 0, len(name)
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            end = i
            break
    return name[:end].replace("moe::", "").strip()


def _matches(short: str, kernel: str) -> bool:
    """Does a profiled kernel name belong to the kernel named `kernel` ('k_x' or 'k_x<0>')?"""
    if short == kernel or short.startswith(kernel + "<"):
        return True
    return kernel.endswith(">") and short.startswith(kernel[:-1] + ",")


def _counter_means(run_dir: str) -> dict:
    """Mean counter value (KiB) per dispatch of each kernel in a rocprofv3 --pmc run."""
    import csv
    import re
    sums: dict = {}
    for r in csv.DictReader(open(os.path.join(run_dir, "run_counter_collection.csv"))):
        name = r["Kernel_Name"]
        key = "torch_neg" if "neg_kernel" in name else kernel_short_name(name)
        s = sums.setdefault(key, [0.0, 0])
        s[0] += float(r["Counter_Value"])
        s[1] += 1
    return {k: v[0] / v[1] for k, v in sums.items()}


def ingest_counters(pmc_dir: str) -> None:
    """Turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs into profiles/traffic.json.

    Expects pmc_dir/copy_fetch and pmc_dir/copy_write (bench.py
    --copy-calibration 1024 under --pmc FETCH_SIZE, resp. WRITE_SIZE) and
    pmc_dir/c<N>_fetch, pmc_dir/c<N>_write for each --config N profiled
    (c<N>fp8_fetch, c<N>fp8_write for --config N --fp8; c<N>w8a8_* for
    --w8a8); the entries of workloads it does not hold are kept.  Each
    counter is scaled by the bytes the copy kernel really moves over what the
    same counter reads for it."""
    from synth.configs import WORKLOADS
    copy_bytes = 1024 << 20
    cf = _counter_means(os.path.join(pmc_dir, "copy_fetch"))["torch_neg"] * 1024
    cw = _counter_means(os.path.join(pmc_dir, "copy_write"))["torch_neg"] * 1024
    ffac, wfac = copy_bytes / cf, copy_bytes / cw
    # workloads not profiled in this directory keep their earlier entries
    out = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            out = json.load(f)
    out["_calibration"] = {"copy_bytes_each_way": copy_bytes, "fetch_counter_bytes": cf,
                           "write_counter_bytes": cw, "fetch_factor": round(ffac, 5),
                           "write_factor": round(wfac, 5)}
    for cid, tag in [(c, t) for c in (0, 1, 2, 3, 4) for t in ("", "fp8", "w8a8")]:
        fd, wd = (os.path.join(pmc_dir, f"c{cid}{tag}_{x}") for x in ("fetch", "write"))
        if not (os.path.isdir(fd) and os.path.isdir(wd)):
            continue
        cfg = WORKLOADS[cid]
        wname = cfg.name + {"": "", "fp8": "_fp8w", "w8a8": "_w8a8"}[tag]
        fm, wm = _counter_means(fd), _counter_means(wd)
        kernels = {}
        for kname in fm:
            if kname.startswith("k_") and kname in wm and \
                    not kname.startswith(("k_pack", "k_prep", "k_mfma_rate")):
                kernels[kname] = {"fetch_bytes": round(fm[kname] * 1024 * ffac),
                                  "write_bytes": round(wm[kname] * 1024 * wfac)}
        dom = dominant_kernel_name(cfg, act8=tag == "w8a8")
        dk = next(k for k in kernels if _matches(k, dom))
        out[wname] = {"kernel": dom, "source_hash": kernel_source_hash(dom),
                      "bytes_per_launch": kernels[dk]["fetch_bytes"] + kernels[dk]["write_bytes"],
                      "kernels": kernels}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def dominant_kernel(cfg, counts, fp8: bool = False, act8: bool = False):
    """Dominant kernel of a forward and its algorithmic work per launch.

    Decode-sized batches (T*k <= 64) take the weight-streaming path whose
    gate/up kernel moves 2/3 of the bytes; larger batches take the tiled
    grouped GEMM whose gate/up launch does 2/3 of the flops.  fp8 weights:
    one byte per weight plus one fp32 scale per row.  fp8 activations (act8):
    decode sizes stream the fp8 weights as above; larger batches run the fp8
    MFMA GEMMs, priced against the fp8 peak."""
    d, F, k, T = cfg.d, cfg.F, cfg.k, cfg.T
    n = T * k
    touched = int((counts > 0).sum())
    if cfg.dtype == "f32":
        # fp32 layers: gate and up rows of each touched expert, 4 bytes each
        per_expert = 2 * F * d * 4
        return {"slot": "experts_gate_up", "kernel": "k_gateup_f32", "bound": "hbm",
                "unit": "GB/s", "units": touched, "per_unit": per_expert,
                "unit_name": "touched expert (fp32 W_gate + W_up bytes)",
                "work": touched * per_expert, "work_unit": "bytes"}
    if n <= 64:
        # W_gate + W_up bytes of one expert
        per_expert = 2 * F * d + 2 * F * 4 if fp8 else 2 * F * d * 2
        work = touched * per_expert + n * d * 2 + n * F * 2
        return {"slot": "experts_gate_up", "kernel": "k_gateup_stream", "bound": "hbm",
                "unit": "GB/s", "units": touched, "per_unit": per_expert,
                "unit_name": "touched expert (W_gate + W_up bytes%s)" % (
                    ": E4M3 codes + row scales" if fp8 else ""), "work": work,
                "work_unit": "bytes"}
    per_assign = 2 * 2 * F * d                      # gate and up: 2 flops x F x d each
    work = n * per_assign
    # the same launch's algorithmic HBM bytes: the touched experts' gate and up
    # rows (fp8 banks: codes + row scales), each routed row's operand tile read
    # once (E4M3 with fp8 activations) and its bf16 activations written once
    wgu = 2 * F * d + 2 * F * 4 if act8 else 2 * F * d * 2
    hbm = touched * wgu + n * d * (1 if act8 else 2) + n * F * 2
    return {"slot": "experts_gate_up", "kernel": "k_expert_gemm<0>", "bound": "mfma",
            "peak": PEAK_FP8_TFLOPS if act8 else PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "units": n, "per_unit": per_assign,
            "unit_name": "routed assignment (gate+up flops)", "work": work, "work_unit": "flops",
            "hbm_bytes": hbm}


def layer_work(cfg, counts, fp8: bool = False):
    touched = int((counts > 0).sum())
    d, F, n = cfg.d, cfg.F, cfg.T * cfg.k
    es = 4 if cfg.dtype == "f32" else 2
    wexp = 3 * F * d + (2 * F + d) * 4 if fp8 else 3 * F * d * es  # expert weight bytes
    bytes_ = touched * wexp + 2 * cfg.T * d * es + cfg.E * d * es + cfg.E * 4 + d * es
    flops = n * 6 * F * d + 2 * cfg.T * d * cfg.E
    return bytes_, flops, touched


def routing_check(inputs, sel_gpu) -> dict:
    """The oracle's routing (O1-O3, every token) of a benched batch against the
    GPU's: tokens whose top-k margin is below 1e-3 (near-ties, either route
    is correct), how many of them the GPU routed differently, and how many
    other tokens it routed differently (must be 0)."""
    import numpy as np
    from oracle import moe_oracle as O
    from synth import gen
    cfg = inputs["cfg"]
    vals = gen.values_f32(inputs)
    x = O.rmsnorm(vals["hidden"], vals["gain"], cfg.eps)
    _, sc = O.router_scores(x, vals["w_router"], vals["bias"])
    sel_o, margin = O.select_topk(sc, cfg.k)
    firm = margin >= O.MARGIN_TOL
    same = (np.asarray(sel_gpu) == sel_o).all(axis=1)
    return {"workload": cfg.name, "tokens": int(cfg.T), "near_ties": int(np.sum(~firm)),
            "near_tie_flips": int(np.sum(~same & ~firm)),
            "firm_mismatches": int(np.sum(~same & firm))}


def cpu_baseline(inputs, seconds: float, fp8: dict | None = None, act8: bool = False):
    """The fp64 oracle as it stands, on the host cores, over a bounded sample."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import moe_oracle as O
    from synth import gen
    cfg = inputs["cfg"]
    vals = gen.values_f32(inputs)
    if fp8 is not None:  # the oracle on the dequantised fp8 expert weights
        for name in ("w_gate", "w_up", "w_down"):
            vals[name] = O.fp8_weights(fp8[name], fp8["s" + name[1:]])
    ncores = len(os.sched_getaffinity(0))
    sample = None if cfg.T <= 64 else np.sort(
        np.random.default_rng(0).choice(cfg.T, size=64, replace=False))
    ntok = cfg.T if sample is None else len(sample)
    with threadpool_limits(limits=ncores):
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
        reps, t0 = 0, time.perf_counter()
        while True:
            O.oracle_forward(vals, tokens=sample, fp8_act=act8)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds or reps >= 10000:
                break
    with threadpool_limits(limits=1):
        reps1, t1 = 0, time.perf_counter()
        while True:
            O.oracle_forward(vals, tokens=sample, fp8_act=act8)
            reps1 += 1
            el1 = time.perf_counter() - t1
            if el1 >= seconds / 3 or reps1 >= 10000:
                break
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         model)
    except OSError:
        pass
    what = (f"full batch of {cfg.T} tokens" if sample is None else
            f"{ntok} sampled tokens of {cfg.T} (routing of all {cfg.T} tokens included)")
    return {"value": round(reps * ntok / el, 2), "unit": "tokens/s", "cores": int(threads),
            "cpu_model": model, "single_thread_value": round(reps1 * ntok / el1, 2),
            "kind": "oracle",
            "sample": f"{reps} oracle forwards (fp64 NumPy) of the {cfg.name} workload: {what}; "
                      f"{el:.1f} s; single-thread: {reps1} forwards in {el1:.1f} s",
            "host_cpus": ncores}


def hw_context(dev) -> dict:
    """Measured rates of this part, as context for the roofline fractions
    (which use the published peaks): a 1 GiB device copy (HBM read + write)
    and a vendor bf16 GEMM (torch.matmul, hipBLASLt) of the prefill gate/up
    shape."""
    import torch

    def best_ms(fn, reps=5):
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts)

    out = {}
    n = 1 << 30
    src = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ms = best_ms(lambda: dst.copy_(src))
    out["hbm_copy_GBps"] = round(2 * n / (ms * 1e-3) / 1e9, 1)
    del src, dst
    a = torch.randn(4096, 2048, device=dev).to(torch.bfloat16)
    b = torch.randn(2048, 6144, device=dev).to(torch.bfloat16)
    c = torch.matmul(a, b)
    ms = best_ms(lambda: torch.matmul(a, b, out=c))
    out["vendor_gemm_bf16_4096x6144x2048_TFLOPs"] = round(2 * 4096 * 6144 * 2048 / (ms * 1e-3) / 1e12, 1)
    return out


def per_forward(layers, hidden, outs, n: int) -> dict:
    """Distribution of single-forward times (an event pair around each forward)."""
    import torch
    nl = len(layers)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record()
        layers[i % nl].forward(hidden, out=outs[i % nl])
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    q = lambda f: round(t[min(len(t) - 1, int(f * len(t)))], 3)  # noqa: E731
    return {"p10": q(0.1), "median": q(0.5), "p90": q(0.9), "n": n}


def graph_timing(layers, hidden, outs, K: int) -> dict:
    """One forward per layer copy captured into a HIP graph, replayed ~K/nl times."""
    import torch
    nl = len(layers)
    torch.cuda.synchronize()
    for L, o in zip(layers, outs):
        L.forward(hidden, out=o)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for L, o in zip(layers, outs):
            L.forward(hidden, out=o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for L, o in zip(layers, outs):
            L.forward(hidden, out=o)
    for o in outs:
        o.zero_()
    g.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(o, r) for o, r in zip(outs, ref))
    reps = max(1, K // nl)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * nl)
    del g
    return {"ms_per_step": ms, "matches_eager": bool(same)}


def run_stack(args):
    """Per-frame latency of the FFN half of the full 28-layer backbone at decode.

    Layers (digest item 5): 3 dense, 24 MoE (16 experts; top-1, the last one
    top-2), 1 dense; a dense layer is the one-expert case.  d_model=2048,
    d_ff=3072, T=32 (32 streams x one frame).  Weights are drawn on the GPU
    (seeded torch generator, the layer distributions of the workloads); no
    oracle runs here (the stack's parity is in tests/test_gpu_stack.py).
    --fp8 / --w8a8: every layer's expert weights quantised per row on the GPU
    (E4M3, scale max|row| / 448), with bf16 or fp8 activations.
    """
    import torch
    from moe_ffn_amd import MoELayer, MoEStack, load_library
    load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d, F, E, T = 2048, 3072, 16, 32
    plan = [(1, 1)] * 3 + [(E, 1)] * 23 + [(E, 2)] + [(1, 1)]
    g = torch.Generator(device=dev)
    layers = []
    t0 = time.perf_counter()
    for l, (ne, k) in enumerate(plan):
        g.manual_seed(1000 + l)
        def rnd(*shape, std=1.0):
            return (torch.randn(*shape, generator=g, device=dev) * std).to(torch.bfloat16)
        w = {"rms_gain": (1.0 + torch.randn(d, generator=g, device=dev) * 0.1 ** 0.5).to(torch.bfloat16),
             "w_router": rnd(ne, d, std=d ** -0.5),
             "b_router": (torch.randn(ne, generator=g, device=dev) * 0.1 ** 0.5) if ne > 1
             else torch.zeros(1, device=dev),
             "w_gate": rnd(ne, F, d, std=d ** -0.5), "w_up": rnd(ne, F, d, std=d ** -0.5),
             "w_down": rnd(ne, d, F, std=F ** -0.5)}
        sc = None
        if args.fp8:
            sc = {}
            for name, sname in (("w_gate", "gate"), ("w_up", "up"), ("w_down", "down")):
                w32 = w[name].float()
                amax = w32.abs().amax(dim=-1)
                s_ = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
                w[name] = (w32 / s_[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
                sc[sname] = s_.contiguous()
        layers.append(MoELayer(d, F, ne, k, "bf16", w, T, fp8_scales=sc, fp8_act=args.w8a8))
        del w, sc
    torch.cuda.synchronize()
    log(f"[bench] {len(layers)} layers created in {time.perf_counter() - t0:.1f} s")
    g.manual_seed(7)
    h0 = torch.randn(T, d, generator=g, device=dev).to(torch.bfloat16)
    # routing of every layer on this frame (eager loop), for the bytes touched
    touched, h = [], h0
    for L in layers:
        y, r = L.forward(h, routing=True)
        touched.append(int((r["counts"] > 0).sum()))
        h = (h.float() + y.float()).to(torch.bfloat16)
    stack = MoEStack(layers, max_tokens=T)
    out = stack.forward(h0)
    torch.cuda.synchronize()
    same_as_loop = bool(torch.equal(out.view(torch.int16), h.view(torch.int16)))
    per_expert = 3 * F * d + (2 * F + d) * 4 if args.fp8 else 3 * F * d * 2
    wbytes = sum(t * per_expert for t in touched)
    K, W = args.steps, args.warmup
    for _ in range(W):
        stack.forward(h0, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        stack.forward(h0, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / K
    side = torch.cuda.Stream()
    gout = torch.empty_like(h0)
    stack.capture(h0, gout, side)
    stack.replay(side)
    side.synchronize()
    graph_same = bool(torch.equal(gout.view(torch.int16), out.view(torch.int16)))
    e0.record(side)
    for _ in range(K):
        stack.replay(side)
    e1.record(side)
    side.synchronize()
    ms_graph = e0.elapsed_time(e1) / K
    eda = None
    if args.eda is not None:  # the same pass with the router logits depth-averaged
        stack.set_eda(args.eda)
        for _ in range(W):
            stack.forward(h0, out=out)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(K):
            stack.forward(h0, out=out)
        e1.record()
        torch.cuda.synchronize()
        eda = {"alpha": args.eda, "us_per_frame_eager": round(e0.elapsed_time(e1) / K * 1e3, 2)}
        log(f"[bench] with depth-averaged router logits (alpha {args.eda}): "
            f"eager {eda['us_per_frame_eager']:.1f} us per frame")
    log(f"[bench] stack of {len(layers)} FFN layers: eager {ms_eager * 1e3:.1f} us, "
        f"graph {ms_graph * 1e3:.1f} us per frame of {T} tokens; experts touched per layer "
        f"{touched}; stack equals layer loop: {same_as_loop}, graph equals eager: {graph_same}")
    line = {"metric": "FFN-stack frames of 32 tokens per second (28 layers, decode)",
            "value": round(1e3 / ms_graph, 2), "unit": "frames/s", "n_gpus": 1, "steps": K,
            "warmup": W, "ms_per_step": round(ms_graph, 6), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3" if args.w8a8 else "bf16",
            "data": "synthetic: random-init weights drawn on the GPU (seeded), N(0,1) hidden states",
            "config": {"workload": "ffn_stack_28_layers_decode_T32_d2048_E16_F3072" +
                                   ("_w8a8" if args.w8a8 else "_fp8w" if args.fp8 else ""),
                       "layers": "3 dense, 23 MoE top-1, 1 MoE top-2, 1 dense", "T": T},
            "stack": {"us_per_frame_graph": round(ms_graph * 1e3, 2),
                      "us_per_frame_eager": round(ms_eager * 1e3, 2),
                      "tokens_per_s": round(T / (ms_graph * 1e-3), 1),
                      "weight_bytes_per_frame": wbytes,
                      "weight_GBps": round(wbytes / (ms_graph * 1e-3) / 1e9, 1),
                      "experts_touched": touched, "stack_equals_layer_loop": same_as_loop,
                      "graph_equals_eager": graph_same, "depth_averaged_router": eda}}
    stack.close()
    for L in layers:
        L.close()
    print(json.dumps(line), flush=True)


def make_layers(inp, n: int, fp8: bool, dev, act8: bool = False):
    """n independently allocated copies of the workload's layer (fp8: E4M3
    expert weights with row scales; act8: and E4M3 activations) and the fp8
    codes used (or None)."""
    import numpy as np
    import torch
    from moe_ffn_amd import MoELayer
    cfg = inp["cfg"]
    q8 = None
    if fp8:
        from synth.gen import fp8_expert_weights
        q8 = fp8_expert_weights(inp)

    def host(a):  # read-only cached inputs: the tensor is only read, for the copy
        with warnings.catch_warnings():
            warnings.filterwarnings("ignore", message="The given NumPy array is not writable")
            return torch.from_numpy(a)

    def tt(a, bf16=True):
        if bf16 and a.dtype == np.uint16:
            return host(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return host(np.ascontiguousarray(a, np.float32)).to(dev)

    w = {"rms_gain": tt(inp["gain"]), "w_router": tt(inp["w_router"]),
         "b_router": tt(inp["bias"], False)}
    scales = None
    if q8 is None:
        w.update({n_: tt(inp[n_]) for n_ in ("w_gate", "w_up", "w_down")})
    else:
        w.update({n_: host(q8[n_]).to(dev) for n_ in ("w_gate", "w_up", "w_down")})
        scales = {n_: tt(q8["s_" + n_], False) for n_ in ("gate", "up", "down")}
    layers = [MoELayer(cfg.d, cfg.F, cfg.E, cfg.k, cfg.dtype, w, cfg.T, rms_eps=cfg.eps,
                       fp8_scales=scales, fp8_act=act8)
              for _ in range(n)]
    del w, scales
    hidden = tt(inp["hidden"])
    torch.cuda.synchronize()
    return layers, hidden, q8


def time_steps(layers, hidden, outs, K: int, per_kernel: bool):
    """K forwards rotating over the layer copies, bracketed by synchronisations
    and HIP events on the forwards' stream.  Returns (ms per step, per-kernel
    ms per forward from the events the library attaches to each kernel's own
    dispatch, or None)."""
    import torch
    nl = len(layers)
    if per_kernel:
        for L in layers:
            L.timing_start((K + nl - 1) // nl)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for i in range(K):
        layers[i % nl].forward(hidden, out=outs[i % nl])
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    slots = None
    if per_kernel:
        slots, nf = {}, 0
        for L in layers:
            sl, n = L.timing_stop()
            nf += n
            for k_, v in sl.items():
                slots[k_] = slots.get(k_, 0.0) + v
        slots = {k_: v / nf for k_, v in slots.items()}
    return ms / K, slots


def roofline_entry(dom: dict, dom_ms: float, traffic) -> dict:
    if dom["work_unit"] == "bytes":
        achieved, peak = dom["work"] / (dom_ms * 1e-3) / 1e9, PEAK_HBM_GBPS
    else:
        achieved, peak = dom["work"] / (dom_ms * 1e-3) / 1e12, dom.get("peak", PEAK_BF16_TFLOPS)
    out = {"bound": dom["bound"], "achieved": round(achieved, 2), "peak": peak,
           "unit": dom["unit"], "frac": round(achieved / peak, 4), "traffic": traffic,
           "kernel": dom["kernel"], "avg_launch_us": round(dom_ms * 1e3, 3),
           "per_unit": dom["per_unit"], "units_per_launch": dom["units"],
           "unit_name": dom["unit_name"]}
    if "hbm_bytes" in dom:
        # a grouped GEMM with few tokens per expert can take longer to read its
        # weights at the HBM peak than to do its flops at the MFMA peak: the
        # roofline's bound is then HBM, and both sides are reported
        gbps = dom["hbm_bytes"] / (dom_ms * 1e-3) / 1e9
        t_mfma = dom["work"] / (peak * 1e12)
        t_hbm = dom["hbm_bytes"] / (PEAK_HBM_GBPS * 1e9)
        out["hbm_side"] = {"algorithmic_bytes": dom["hbm_bytes"], "achieved_GBps": round(gbps, 1),
                           "peak_GBps": PEAK_HBM_GBPS, "frac": round(gbps / PEAK_HBM_GBPS, 4)}
        out["roofline_bound"] = "hbm" if t_hbm > t_mfma else "mfma"
        out["roofline_frac"] = round(max(t_mfma, t_hbm) / (dom_ms * 1e-3), 4)
    return out


def counter_traffic(wname: str, kernel: str):
    """HBM bytes per launch of the kernel from profiles/traffic.json, if the
    kernel's sources still hash to the value recorded with the counters."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f).get(wname, {})
        if tr.get("kernel") == kernel and tr.get("source_hash") == kernel_source_hash(kernel):
            return tr.get("bytes_per_launch")
    except (OSError, ValueError):
        return None
    return None


def prefill_summary(cid: int, args, dev, w8a8: bool = False) -> tuple[dict, dict, object]:
    """Step time, whole-layer MFMA fraction and the gate/up GEMM's time and
    fraction of one prefill workload (a sub-object of the default line);
    w8a8: the layer with fp8 weights and activations, its fractions against
    the fp8 peak (at decode sizes: its weight stream against HBM).
    Returns (summary, inputs, GPU routing choice)."""
    import torch
    from synth import make_inputs
    inp = make_inputs(cid)
    cfg = inp["cfg"]
    layers, hidden, _ = make_layers(inp, args.instances, w8a8, dev, w8a8)
    outs = [torch.empty_like(hidden) for _ in layers]
    _, r = layers[0].forward(hidden, routing=True)
    sel = r["sel"].cpu().numpy()
    counts = r["counts"].cpu().numpy()
    dom = dominant_kernel(cfg, counts, w8a8, w8a8)
    lbytes, lflops, touched = layer_work(cfg, counts, w8a8)
    peak = PEAK_FP8_TFLOPS if w8a8 else PEAK_BF16_TFLOPS
    K = args.prefill_steps
    for i in range(max(5, K // 10)):
        layers[i % len(layers)].forward(hidden, out=outs[i % len(layers)])
    ms, _ = time_steps(layers, hidden, outs, K, False)
    ms_ev, slots = time_steps(layers, hidden, outs, K, True)
    wname = cfg.name + ("_w8a8" if w8a8 else "")
    rl = roofline_entry(dom, slots[dom["slot"]], counter_traffic(wname, dom["kernel"]))
    for L in layers:
        L.close()
    out = {"workload": wname, "T": cfg.T, "top_k": cfg.k, "steps": K,
           "tokens_per_s": round(cfg.T / (ms * 1e-3), 1), "us_per_step": round(ms * 1e3, 3),
           "mfma_frac_layer": round(lflops / (ms * 1e-3) / 1e12 / peak, 4),
           "mfma_peak_TFLOPs": peak,
           "algorithmic_flops": lflops, "algorithmic_bytes": lbytes,
           "experts_touched": touched,
           "gemm_gate_up": {"kernel": dom["kernel"], "us": rl["avg_launch_us"],
                            "achieved": rl["achieved"], "unit": rl["unit"], "frac": rl["frac"],
                            "traffic": rl["traffic"],
                            **{k_: rl[k_] for k_ in ("hbm_side", "roofline_bound",
                                                      "roofline_frac") if k_ in rl}},
           "kernel_us": {k_: round(v * 1e3, 3) for k_, v in slots.items()},
           "us_per_step_with_kernel_events": round(ms_ev * 1e3, 3)}
    log(f"[bench] {wname}: {out['us_per_step']:.1f} us/step, {out['tokens_per_s'] / 1e6:.2f} M "
        f"tokens/s, layer {100 * out['mfma_frac_layer']:.1f}% of the {'fp8' if w8a8 else 'bf16'} "
        f"peak; gate/up {rl['avg_launch_us']:.1f} us = {100 * rl['frac']:.1f}% of its roofline")
    return out, inp, sel


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=1, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--instances", type=int, default=3)
    ap.add_argument("--prefill-steps", type=int, default=200,
                    help="steps of each prefill workload in the default line's `prefill` entry")
    ap.add_argument("--no-prefill", action="store_true",
                    help="leave the prefill and fp8-activation workloads out of the decode line")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the copy / vendor-GEMM context measurements")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run only a plain device copy (dst = -src, MIB MiB read and MIB MiB\n"
                         "written) five times, to scale the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--fp8", action="store_true",
                    help="expert weights as E4M3 codes with per-row scales")
    ap.add_argument("--w8a8", action="store_true",
                    help="E4M3 weights and E4M3 activations (fp8 MFMA GEMMs)")
    ap.add_argument("--stack", action="store_true",
                    help="time the FFN half of the full 28-layer backbone at decode instead")
    ap.add_argument("--eda", type=float, default=None, metavar="ALPHA",
                    help="with --stack: also time the pass with the router logits depth-averaged")
    ap.add_argument("--ingest-counters", metavar="DIR",
                    help="no GPU: write profiles/traffic.json from rocprofv3 --pmc runs in DIR")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(args.ingest_counters)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the layer runs data-parallel with no exchange between "
              "GPUs, so N GPUs give N times one GPU's throughput; run it with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.w8a8:
        args.fp8 = True
    if args.stack:
        if args.steps == 2000:
            args.steps = 100
        run_stack(args)
        return

    import torch
    from synth import make_inputs
    from moe_ffn_amd import load_library

    load_library()  # fails loudly if the HIP library is not built
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    if args.fp8 and args.config == 0:
        raise SystemExit("--fp8 and --w8a8 need a bf16 workload (--config 1..4)")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)

    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"kernel": "elementwise neg (torch)",
                                               "bytes_read": nbytes, "bytes_written": nbytes,
                                               "launches": 5}}), flush=True)
        return

    t_gen = time.perf_counter()
    inp = make_inputs(args.config)
    cfg = inp["cfg"]
    wname = cfg.name + ("_w8a8" if args.w8a8 else "_fp8w" if args.fp8 else "")
    layers, hidden, q8 = make_layers(inp, args.instances, args.fp8, dev, args.w8a8)
    outs = [torch.empty_like(hidden) for _ in layers]
    log(f"[bench] inputs and {len(layers)} layers for {wname} in {time.perf_counter() - t_gen:.1f} s")

    _, r = layers[0].forward(hidden, routing=True)
    counts = r["counts"].cpu().numpy()
    sel_gpu = r["sel"].cpu().numpy()
    dom = dominant_kernel(cfg, counts, args.fp8, args.w8a8)
    lbytes, lflops, touched = layer_work(cfg, counts, args.fp8)
    log(f"[bench] {touched} experts touched; dominant kernel {dom['kernel']}")

    K, W = args.steps, args.warmup
    nl = len(layers)
    for i in range(W):
        layers[i % nl].forward(hidden, out=outs[i % nl])
    torch.cuda.synchronize()

    ms_step, _ = time_steps(layers, hidden, outs, K, False)
    log(f"[bench] {K} steps: {ms_step * 1e3:.2f} us/step")
    pf = per_forward(layers, hidden, outs, min(K, 1000))
    log(f"[bench] per forward: p10 {pf['p10']} median {pf['median']} p90 {pf['p90']} us")
    gr = graph_timing(layers, hidden, outs, K)
    log(f"[bench] HIP graph of {nl} forwards: {gr['ms_per_step'] * 1e3:.2f} us/step, "
        f"replay equals eager: {gr['matches_eager']}")
    ms_step_ev, slots = time_steps(layers, hidden, outs, K, True)
    log(f"[bench] with per-kernel events: {ms_step_ev * 1e3:.2f} us/step; "
        + ", ".join(f"{k_} {v * 1e3:.2f} us" for k_, v in slots.items()))
    for L in layers:
        L.close()
    del layers, outs

    value = cfg.T / (ms_step * 1e-3)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if cfg.dtype == "f32" else "fp8e4m3" if args.w8a8 else "bf16",
        "data": "synthetic: seeded N(0,1) hidden states and random-init weights of the stated "
                "distributions (no checkpoint or dataset)",
        "config": {"workload": wname, "T": cfg.T, "d_model": cfg.d, "d_ff": cfg.F,
                   "n_experts": cfg.E, "top_k": cfg.k, "router_bias": cfg.bias,
                   "expert_weights": "fp8_e4m3_row_scaled" if args.fp8 else cfg.dtype,
                   "expert_activations": "fp8_e4m3_row_scaled" if args.w8a8 else cfg.dtype,
                   "experts_touched": touched, "layer_instances": nl,
                   "device": props.name, "compute_units": props.multi_processor_count},
        "roofline": roofline_entry(dom, slots[dom["slot"]], counter_traffic(wname, dom["kernel"])),
        "layer": {"algorithmic_bytes": lbytes, "algorithmic_flops": lflops,
                  "hbm_GBps": round(lbytes / (ms_step * 1e-3) / 1e9, 1),
                  "mfma_frac": round(lflops / (ms_step * 1e-3) / 1e12 /
                                     (PEAK_FP8_TFLOPS if args.w8a8 else PEAK_BF16_TFLOPS), 4),
                  "mfma_peak_TFLOPs": PEAK_FP8_TFLOPS if args.w8a8 else PEAK_BF16_TFLOPS,
                  "us_per_step_with_kernel_events": round(ms_step_ev * 1e3, 3),
                  "per_forward_us": pf,
                  "graph": {"us_per_step": round(gr["ms_per_step"] * 1e3, 3),
                            "forwards_per_graph": nl, "replay_equals_eager": gr["matches_eager"]},
                  "kernel_us": {k_: round(v * 1e3, 3) for k_, v in slots.items()}},
    }
    checked = [(inp, sel_gpu)]
    if args.config == 1 and not args.fp8 and not args.no_prefill:
        line["prefill"] = {}
        for cid in (2, 4):
            summ, pinp, psel = prefill_summary(cid, args, dev)
            line["prefill"][f"T{pinp['cfg'].T}"] = summ
            checked.append((pinp, psel))
        # the same workloads with fp8 weights and activations (R20): the same
        # router, so the routing checked above covers them
        line["w8a8"] = {}
        for cid in (1, 2, 4):
            summ, pinp, _ = prefill_summary(cid, args, dev, w8a8=True)
            line["w8a8"][f"T{pinp['cfg'].T}"] = summ
    if not args.no_context:
        torch.cuda.synchronize()
        line["context"] = hw_context(dev)
        log(f"[bench] context: {line['context']}")
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, q8, args.w8a8)
        line["cpu_baseline"]["routing_check"] = [routing_check(i, s_) for i, s_ in checked]
        log(f"[bench] routing against the oracle: {line['cpu_baseline']['routing_check']}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
