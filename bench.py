"""Benchmark of the dropless sparse-MoE forward on one MI355X.

A step is one whole forward pass on resident inputs: router top-k + softmax,
sparse map, gathered gate+up GEMM with SwiGLU, down GEMM storing the
router-weighted per-route rows, and the ordered combine into bf16 tokens --
the three C-ABI calls back to back on one stream. The default workload is the Mixtral-8x7B-shaped layer
(S=4096, D=4096, F=14336, E=8, k=2) with seeded synthetic inputs.

Prints one JSON line with the whole-job throughput (tokens/s), the
roofline of the dominant kernel (timed live with HIP events on its own
stream over the timed region) and the fp64 CPU oracle timed on a bounded
sample of the same workload on this host.

--op ffn_bwd times the backward of the expert FFN (moe_scatter_ffn_bwd: dx,
dW1, dW3, dW2 and the router-weight gradient, with the gate+up forward
recomputed inside) on the configuration's routing; its line reports the
algorithmic backward TFLOP/s (12 S k D F, the recomputation not counted).

--op train times one training step of the layer's experts on the
configuration's routing: the training-mode forward (which keeps a, b and h)
followed by the backward fed those activations (no recomputation);
algorithmic 18 S k D F FLOP (forward 6, backward 12).

--op map_sweep times the sparse map alone on the ids of the top-4 of iid
N(0, 1) logits over 128 experts, S in {2^13, 2^16, 2^19, 2^21} (median of
20 launches each), against its algorithmic bytes 12 S k + 8 E.

--op pl_fwd / pl_bwd time the general ParallelLinear primitive instead, on
the expert up-projection of the chosen configuration (x [S, D] read by
index, W [E, D, F], router gates, output grouped [S*k, F]): the forward, or
the backward producing dx, dw and dgates. Their line reports algorithmic
TFLOP/s and the roofline of their dominant kernel.
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

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
METRIC = "MoE-layer fwd tokens/s + % bf16 MFMA peak (Mixtral-shape, S=4096, 1 GPU)"
KERNEL_SOURCES = ["sparse_mixture_experts_gemv_amd/csrc/gemm.hpp", "sparse_mixture_experts_gemv_amd/csrc/gemm_pp.hpp",
                  "sparse_mixture_experts_gemv_amd/csrc/common.hpp", "sparse_mixture_experts_gemv_amd/csrc/ffn.hip"]


def kernel_source_hash() -> str:
    """Hash of the gate+up kernel's sources with comments and blank lines removed (a comment
    edit does not invalidate counters taken on the same code)."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p)) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for line in text.splitlines():
            code = re.sub(r"//.*", "", line).strip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def layer_flops(S, D, F, E, k, with_router=True):
    return 6.0 * S * k * D * F + (2.0 * S * D * E if with_router else 0.0)


def roofline_entry(kernel: str, flops: float, nbytes: float, seconds: float, per: str = "launch") -> dict:
    """Roofline object for one kernel: against the MFMA peak or the HBM peak,
    whichever floor (flops / peak, bytes / bandwidth) is longer."""
    if nbytes / (PEAK_HBM_GBS * 1e9) > flops / (PEAK_BF16_TFLOPS * 1e12):
        achieved = nbytes / seconds / 1e9
        return {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                f"algorithmic_bytes_per_{per}": nbytes, f"avg_{per}_us": round(seconds * 1e6, 2)}
    achieved = flops / seconds / 1e12
    return {"kernel": kernel, "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
            f"algorithmic_flops_per_{per}": flops, f"avg_{per}_us": round(seconds * 1e6, 2)}


def warm_up(step, n: int, min_seconds: float) -> int:
    """At least `n` untimed steps and at least `min_seconds` of them: under sustained MFMA load the
    GPU's clock settles over the first tens of milliseconds, and the timed steps should see the
    steady state. Returns the number of steps run."""
    import torch

    done = 0
    t0 = time.perf_counter()
    while done < n or time.perf_counter() - t0 < min_seconds:
        for _ in range(8 if done >= n else 1):
            step()
            done += 1
        torch.cuda.synchronize()
    return done


def timed(step, steps: int, stream):
    """ms per step over `steps` back-to-back steps, bracketed by HIP events on `stream`, plus the
    wall-clock seconds of the region (synchronised on both sides)."""
    import torch

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, time.perf_counter() - wall0


def profiled(step, steps: int, stream):
    """The same loop with per-kernel HIP-event pairs recorded around every launch (moe_profile_*):
    {kernel: (total ms, launches)} and the ms per step of this loop."""
    import sparse_mixture_experts_gemv_amd as smoe

    smoe.profile_start(steps * 32)
    ms, _ = timed(step, steps, stream)
    return smoe.profile_stop(), ms


def host_cpu_info() -> dict:
    """What the CPU baseline ran on: the host's logical CPUs, the CPUs this process may use, the
    threads the oracle is given (the CPU share of this process: OMP_NUM_THREADS when set, else the
    affinity count) and the CPU model."""
    nproc = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = nproc
    share = affinity
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        share = min(share, int(env))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": nproc, "affinity": affinity, "threads": share, "model": model}


def touched_experts(offsets) -> int:
    """Experts with at least one route, from the map's offsets (read back after timing)."""
    o = offsets.cpu()
    return int(((o[1:] - o[:-1]) > 0).sum().item())


def load_traffic(workload: str, per_launch_units: float):
    """HBM bytes per launch of the gate+up kernel from committed rocprofv3 PMC
    counters, or None when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"pmc_ffn_gate_up_gemm_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != kernel_source_hash() or d.get("routes") != per_launch_units:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, p, target_s: float = 15.0):
    """The fp64 oracle (route + map + FFN) on a bounded sample of tokens."""
    import numpy as np
    import torch

    import oracle
    import workloads as wl

    o = oracle.get()
    host = host_cpu_info()
    nthreads = host["threads"]
    rng = np.random.default_rng(0)
    order = rng.permutation(cfg.S)
    wg = wl.bf16_bits(p["wg"].cpu())
    w1 = wl.bf16_bits(p["w1"].cpu())
    w3 = wl.bf16_bits(p["w3"].cpu())
    w2 = wl.bf16_bits(p["w2"].cpu())
    done, t_used = 0, 0.0
    while t_used < target_s and done < cfg.S:
        n = min(nthreads * 2, cfg.S - done)
        toks = np.sort(order[done:done + n])
        x = wl.bf16_bits(p["x"][torch.from_numpy(toks).to(p["x"].device)].cpu())
        t0 = time.perf_counter()
        if "ids" in p:
            ids = p["ids"].cpu().numpy()[toks]
            w = p["weights"].cpu().numpy()[toks].astype(np.float64)
        else:
            ids, w, _ = o.route(x, wg, cfg.k)
        o.sparse_map(ids, cfg.E)
        o.ffn(x, w1, w3, w2, ids, w, nthreads=nthreads)
        t_used += time.perf_counter() - t0
        done += n
    return {"value": done / t_used, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{done} random tokens of the {cfg.name} workload (route + map + FFN, fp64, "
                      f"{nthreads} threads, {t_used:.1f} s)",
            "host": host}


def pl_cpu_baseline(cfg, p, ids, gates, op, target_s: float = 15.0):
    """The fp64 oracle's ParallelLinear (forward or backward) on a bounded sample of tokens."""
    import numpy as np
    import torch

    import oracle
    import workloads as wl

    o = oracle.get()
    rng = np.random.default_rng(0)
    order = rng.permutation(cfg.S)
    # the backward's dw is [E, D, F'] fp64 per call, so it runs on the first F' = 512 output columns
    Fs = cfg.F if op == "pl_fwd" else min(cfg.F, 512)
    w = wl.bf16_bits(p["w1"][:, :, :Fs].contiguous().cpu())
    done, t_used, flops = 0, 0.0, 0.0
    n = 2
    while t_used < target_s and done < cfg.S:
        toks = np.sort(order[done:done + n])
        x = wl.bf16_bits(p["x"][torch.from_numpy(toks).to(p["x"].device)].cpu())
        sid = ids[toks]
        g = gates[toks].astype(np.float64)
        t0 = time.perf_counter()
        if op == "pl_fwd":
            o.parallel_linear(x, w, sid, g, False, True)
            flops += 2.0 * sid.size * cfg.D * Fs
        else:
            dy = wl.bf16_bits(torch.ones(sid.size, Fs, dtype=torch.bfloat16))
            o.parallel_linear_bwd(x, w, sid, dy, g, False, True)
            flops += 4.0 * sid.size * cfg.D * Fs  # the dx and dw products, as counted for the GPU
        t_used += time.perf_counter() - t0
        done += n
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} random tokens of the {cfg.name} up-projection ({op}, D_out {Fs}, fp64, 1 thread, "
                      f"{t_used:.1f} s)"}


def bench_parallel_linear(args, cfg, p):
    """ParallelLinear on the up-projection: x [S, D] by index, W1 [E, D, F], gates, grouped output."""
    import torch

    import sparse_mixture_experts_gemv_amd as smoe

    S, D, F, E, k = cfg.S, cfg.D, cfg.F, cfg.E, cfg.k
    x, w = p["x"], p["w1"]
    if "ids" in p:
        ids, gates = p["ids"], p["weights"]
    else:
        ids, gates = smoe.moe_route_topk(x, p["wg"], k)
    _, offsets, _, src = smoe.moe_sparse_map(ids, E)
    N = S * k
    ws = torch.empty(smoe.parallel_linear_workspace_bytes(S, k, D, F, E), dtype=torch.uint8, device="cuda")
    y = torch.empty((N, F), dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(7)
    dy = torch.randn((N, F), generator=g, device="cuda").to(torch.bfloat16)
    Et = touched_experts(offsets)
    # algorithmic bytes per launch: weights of the touched experts once, the
    # activations once, outputs once (dW: every expert's fp32 gradient)
    pl_bytes = {"pl_gemm": Et * D * F * 2.0 + S * D * 2.0 + N * F * 2.0,
                "pl_dx_gemm": Et * D * F * 2.0 + N * F * 2.0 + N * D * 4.0,
                "pl_wgrad_gemm": E * D * F * (2.0 if args.dw_bf16 else 4.0) + S * D * 2.0 + N * F * 2.0}
    if args.op == "pl_fwd":
        def step():
            smoe.moe_parallel_linear_fwd(x, w, gates, offsets, src, k, False, True, y, ws)
        flops = 2.0 * N * D * F
        dominant, dom_flops = "pl_gemm", 2.0 * N * D * F
    else:
        def step():
            smoe.moe_parallel_linear_bwd(x, w, gates, offsets, src, dy, k, False, True, workspace=ws,
                                         dw_dtype=torch.bfloat16 if args.dw_bf16 else torch.float32)
        flops = 4.0 * N * D * F  # dx and dw products (dgates is a by-product of the dx rows)
        dominant, dom_flops = None, 2.0 * N * D * F  # the slower of the dx and dw GEMMs
    stream = torch.cuda.current_stream()
    warm_up(step, args.warmup, args.warmup_seconds)
    ms, wall = timed(step, args.steps, stream)
    kern, _ = profiled(step, args.steps, stream)
    if dominant is None:
        dominant = max(("pl_dx_gemm", "pl_wgrad_gemm"), key=lambda n: kern[n][0] / kern[n][1])
    dom_ms = kern[dominant][0] / kern[dominant][1]
    rec = {
        "metric": f"ParallelLinear {'forward' if args.op == 'pl_fwd' else 'backward'} TFLOP/s (up-projection)",
        "value": round(flops / (ms / 1e3) / 1e12, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} ParallelLinear up-projection ({args.op}; scattered in, grouped out, "
                               f"gated{', bf16 dW' if args.op == 'pl_bwd' and args.dw_bf16 else ''})", "S": S,
                   "D_in": D, "D_out": F, "E": E, "k": k},
        "roofline": roofline_entry(dominant, dom_flops, pl_bytes[dominant], dom_ms / 1e3),
        "kernels": {n: {"avg_us": round(1e3 * tot / c, 2), "launches": c} for n, (tot, c) in kern.items()},
        "wall_s_timed_region": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        print("bench: timing the fp64 CPU oracle on a sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = pl_cpu_baseline(cfg, p, ids.cpu().numpy(), gates.cpu().numpy(), args.op,
                                              args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def ffn_bwd_cpu_baseline(cfg, p, ids, gates, target_s: float = 15.0):
    """The fp64 oracle's FFN backward on a bounded sample of tokens (its weight gradients are
    [E, D, F'] fp64 per call, so it runs on the first F' = 256 columns of F)."""
    import numpy as np
    import torch

    import oracle
    import workloads as wl

    o = oracle.get()
    order = np.random.default_rng(0).permutation(cfg.S)
    Fs = min(cfg.F, 256)
    w1 = wl.bf16_bits(p["w1"][:, :, :Fs].contiguous().cpu())
    w3 = wl.bf16_bits(p["w3"][:, :, :Fs].contiguous().cpu())
    w2 = wl.bf16_bits(p["w2"][:, :Fs, :].contiguous().cpu())
    done, t_used, flops = 0, 0.0, 0.0
    while t_used < target_s and done < cfg.S:
        toks = np.sort(order[done:done + 2])
        x = wl.bf16_bits(p["x"][torch.from_numpy(toks).to(p["x"].device)].cpu())
        dout = wl.bf16_bits(torch.ones(toks.size, cfg.D, dtype=torch.bfloat16))
        t0 = time.perf_counter()
        o.ffn_bwd(x, w1, w3, w2, ids[toks], gates[toks].astype(np.float64), dout)
        t_used += time.perf_counter() - t0
        flops += 12.0 * toks.size * cfg.k * cfg.D * Fs
        done += toks.size
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} random tokens of the {cfg.name} FFN backward (F {Fs} of {cfg.F}, fp64, 1 thread, "
                      f"{t_used:.1f} s)"}


def bench_ffn_bwd(args, cfg, p, train=False):
    """moe_scatter_ffn_bwd with every output on the configuration's routing and a random dout;
    with train, each step is the training-mode forward plus the backward on its saved activations."""
    import torch

    import sparse_mixture_experts_gemv_amd as smoe

    S, D, F, E, k = cfg.S, cfg.D, cfg.F, cfg.E, cfg.k
    if "ids" in p:
        ids, gates = p["ids"], p["weights"]
    else:
        ids, gates = smoe.moe_route_topk(p["x"], p["wg"], k)
    _, offsets, _, src = smoe.moe_sparse_map(ids, E)
    ws = torch.empty(smoe.scatter_ffn_bwd_workspace_bytes(S, D, F, E, k), dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(7)
    dout = (torch.randn((S, D), generator=g, device="cuda") * 0.1).to(torch.bfloat16)
    dw_dtype = torch.bfloat16 if args.dw_bf16 else torch.float32
    dw_bytes = 2 if args.dw_bf16 else 4

    if train:
        saved = torch.empty(smoe.saved_activations_numel(S, F, k), dtype=torch.bfloat16, device="cuda")
        fws = torch.empty(smoe.scatter_ffn_workspace_bytes(S, D, F, E, k), dtype=torch.uint8, device="cuda")
        out = torch.empty((S, D), dtype=torch.bfloat16, device="cuda")

        def step():
            smoe.moe_scatter_ffn_fwd(p["x"], p["w1"], p["w3"], p["w2"], gates, offsets, src, out, fws, saved=saved)
            smoe.moe_scatter_ffn_bwd(p["x"], p["w1"], p["w3"], p["w2"], gates, offsets, src, dout, workspace=ws,
                                     saved=saved, dw_dtype=dw_dtype)
    else:
        def step():
            smoe.moe_scatter_ffn_bwd(p["x"], p["w1"], p["w3"], p["w2"], gates, offsets, src, dout, workspace=ws,
                                     dw_dtype=dw_dtype)

    N = S * k
    flops = (18.0 if train else 12.0) * N * D * F
    gemm_flops = {"bwd_recompute_gemm": 4.0 * N * D * F, "bwd_dh_gemm": 2.0 * N * D * F,
                  "bwd_wgrad_gemm": 6.0 * N * D * F, "bwd_dx_gemm": 4.0 * N * D * F,
                  "ffn_gate_up_gemm": 4.0 * N * D * F, "ffn_down_scatter_gemm": 2.0 * N * D * F}
    stream = torch.cuda.current_stream()
    warm_up(step, args.warmup, args.warmup_seconds)
    ms, wall = timed(step, args.steps, stream)
    kern, _ = profiled(step, args.steps, stream)
    # the GEMM kind with the most time per step (the weight gradients run as two launches per step)
    per_step = {n: kern[n][0] / args.steps for n in gemm_flops if n in kern}
    dominant = max(per_step, key=per_step.get)
    Et = touched_experts(offsets)
    w_gu, w_dn = Et * 2.0 * D * F * 2, Et * 1.0 * F * D * 2  # touched W1+W3, W2 (bf16)
    gemm_bytes = {  # per step: weights once, activations and outputs once
        "bwd_recompute_gemm": w_gu + S * D * 2.0 + N * 3.0 * F * 2,
        "ffn_gate_up_gemm": w_gu + S * D * 2.0 + N * 3.0 * F * 2,
        "bwd_dh_gemm": w_dn + S * D * 2.0 + 2 * N * 2.0 * F * 2,
        "bwd_wgrad_gemm": E * 3.0 * D * F * dw_bytes + 2 * N * D * 2.0 + N * 3.0 * F * 2,
        "bwd_dx_gemm": w_gu + N * 2.0 * F * 2 + N * D * 4.0,
        "ffn_down_scatter_gemm": w_dn + N * F * 2.0 + N * D * 4.0}
    rec = {
        "metric": ("MoE expert-FFN training step TFLOP/s (forward keeping activations + backward)" if train else
                   "MoE expert-FFN backward TFLOP/s (dx, dW1, dW3, dW2, router-weight gradient)"),
        "value": round(flops / (ms / 1e3) / 1e12, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"{cfg.name} expert FFN training step (forward + backward, saved activations)"
                                if train else f"{cfg.name} expert FFN backward (SwiGLU, gate+up recomputed)")
                               + (", bf16 weight gradients" if args.dw_bf16 else ", fp32 weight gradients"),
                   "S": S, "D": D, "F": F, "E": E, "k": k},
        "tokens_per_s": round(S / (ms / 1e3), 1),
        "roofline": roofline_entry(dominant, gemm_flops[dominant], gemm_bytes[dominant], per_step[dominant] / 1e3,
                                   per="step"),
        "kernels": {n: {"avg_us": round(1e3 * tot / c, 2), "launches": c} for n, (tot, c) in kern.items()},
        "wall_s_timed_region": round(wall, 3),
    }
    if not args.no_cpu_baseline and not train:
        print("bench: timing the fp64 CPU oracle on a sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = ffn_bwd_cpu_baseline(cfg, p, ids.cpu().numpy(), gates.cpu().numpy(), args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def bench_map_sweep(args):
    """The sparse map alone: ids = top-4 of iid N(0, 1) logits [S, 128] (drawn on the GPU, not timed)."""
    import torch

    import sparse_mixture_experts_gemv_amd as smoe

    E, k = 128, 4
    rows = []
    for lg in (13, 16, 19, 21):
        S = 1 << lg
        g = torch.Generator(device="cuda").manual_seed(lg)
        ids = torch.randn((S, E), generator=g, device="cuda").topk(k, dim=1).indices.to(torch.int32).contiguous()
        out = (torch.empty(E, dtype=torch.int32, device="cuda"), torch.empty(E + 1, dtype=torch.int32, device="cuda"),
               torch.empty(S * k, dtype=torch.int32, device="cuda"), torch.empty(S * k, dtype=torch.int32, device="cuda"))
        ws = torch.empty(smoe.sparse_map_workspace_bytes(S, k, E), dtype=torch.uint8, device="cuda")
        for _ in range(5):
            smoe.moe_sparse_map(ids, E, out, ws)
        times = []
        for _ in range(20):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            smoe.moe_sparse_map(ids, E, out, ws)
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e3)
        us = sorted(times)[len(times) // 2]
        smoe.profile_start(64)
        for _ in range(10):
            smoe.moe_sparse_map(ids, E, out, ws)
        kern = smoe.profile_stop()
        nbytes = 12.0 * S * k + 8.0 * E
        rows.append({"S": S, "median_us": round(us, 2), "GB_s": round(nbytes / us / 1e3, 1),
                     "hbm_frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4),
                     "kernels_us": {n: round(1e3 * tot / c, 2) for n, (tot, c) in kern.items()}})
    big = rows[-1]
    rec = {"metric": "sparse map bandwidth (ids from top-4 of N(0,1) logits, E = 128)", "value": big["GB_s"],
           "unit": "GB/s", "n_gpus": 1, "higher_is_better": True, "dtype": "int32", "data": "synthetic",
           "config": {"workload": "sparse map alone, E = 128, k = 4, S = 2^13 .. 2^21"},
           "roofline": {"kernel": "sparse map (3 launches)", "bound": "hbm", "achieved": big["GB_s"],
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": big["hbm_frac"], "traffic": None},
           "sweep": rows}
    print(json.dumps(rec), flush=True)


def bench_route(args):
    """The router alone (moe_route_topk) on the three routed workloads, beside the
    cost of a plain read of the same token rows and of the split partial logits
    (a library reduction over the tensor), each timed as a HIP graph of 20 calls
    so that no host gap is counted."""
    import torch

    import sparse_mixture_experts_gemv_amd as smoe
    from workloads import CONFIGS

    def graph_us(fn, reps=20, replays=10):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(replays):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e3 / reps)
        return sorted(times)[len(times) // 2]

    rows = []
    for name in ("mixtral", "gptoss", "dsv3"):
        cfg = CONFIGS[name]
        S, D, E, k = cfg.S, cfg.D, cfg.E, cfg.k
        gen = torch.Generator(device="cuda").manual_seed(7)
        x = torch.randn((S, D), generator=gen, device="cuda").to(torch.bfloat16)
        wg = (torch.randn((D, E), generator=gen, device="cuda") * D ** -0.5).to(torch.bfloat16)
        ids = torch.empty((S, k), dtype=torch.int32, device="cuda")
        wts = torch.empty((S, k), dtype=torch.float32, device="cuda")
        wsb = smoe.route_workspace_bytes(S, E)
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")
        route_us = graph_us(lambda: smoe.moe_route_topk(x, wg, k, ids, wts, ws))
        read_x_us = graph_us(lambda: x.sum(dtype=torch.float32))
        smoe.profile_start(256)
        for _ in range(20):
            smoe.moe_route_topk(x, wg, k, ids, wts, ws)
        kern = smoe.profile_stop()
        row = {"workload": name, "S": S, "D": D, "E": E, "k": k, "route_us": round(route_us, 2),
               "kernels_us": {n: round(1e3 * tot / c, 2) for n, (tot, c) in kern.items()},
               "read_x_us": round(read_x_us, 2), "x_MB": round(S * D * 2 / 1e6, 1)}
        nbytes = S * D * 2.0 + D * E * 2.0 + S * k * 8.0
        row["algorithmic_MB"] = round(nbytes / 1e6, 1)
        row["hbm_frac"] = round(nbytes / route_us / 1e3 / PEAK_HBM_GBS, 4)
        row["read_x_hbm_frac"] = round(S * D * 2.0 / read_x_us / 1e3 / PEAK_HBM_GBS, 4)
        if wsb:
            part = torch.randn(wsb // 4, generator=gen, device="cuda")
            row["read_partials_us"] = round(graph_us(lambda: part.sum()), 2)
            row["partials_MB"] = round(wsb / 1e6, 1)
        rows.append(row)
        print(f"bench: route {name}: {row}", file=sys.stderr, flush=True)
        del x, wg, ws
    rec = {"metric": "router (logits, top-k, softmax) against a plain read of its input",
           "value": rows[0]["hbm_frac"], "unit": "fraction of 8 TB/s (mixtral)", "n_gpus": 1,
           "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "router alone on the mixtral, gptoss and dsv3 shapes"}, "rows": rows}
    print(json.dumps(rec), flush=True)


def bench_vendor_gemm(args):
    """Context for the GEMM rooflines: the vendor library's dense bf16 GEMM (torch.matmul,
    contiguous 2-D operands) on the shapes of the Mixtral layer's two expert GEMMs, as one
    dense product over all S*k routed rows and as a loop of per-expert products of S*k/E
    rows. No gather, no SwiGLU, no weighted rows: a reference point, not the method."""
    import torch

    from workloads import CONFIGS

    cfg = CONFIGS["mixtral"]
    S, D, F, E, k = cfg.S, cfg.D, cfg.F, cfg.E, cfg.k
    M = S * k
    gen = torch.Generator(device="cuda").manual_seed(11)

    def timed_us(fn, reps=10, rounds=10):
        # each call is hundreds of microseconds of GPU work, far above the host's
        # launch cost, so back-to-back eager calls keep the GPU busy
        t_end = time.time() + 0.5  # settle the clock under load
        while time.time() < t_end:
            fn()
            torch.cuda.synchronize()
        times = []
        for _ in range(rounds):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e3 / reps)
        return sorted(times)[len(times) // 2]

    rows = []
    for name, K, N in (("gate+up (W1 and W3 side by side)", D, 2 * F), ("down", F, D)):
        a = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
        w = (torch.randn((K, N), generator=gen, device="cuda") * K ** -0.5).to(torch.bfloat16)
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        flops = 2.0 * M * K * N
        dense_us = timed_us(lambda: torch.matmul(a, w, out=c))
        me = M // E
        a_e = [a[e * me:(e + 1) * me] for e in range(E)]
        c_e = [c[e * me:(e + 1) * me] for e in range(E)]
        w_e = [w] * E  # the same weights for every expert: a loop of E products of M / E rows

        def loop():
            for e in range(E):
                torch.matmul(a_e[e], w_e[e], out=c_e[e])

        loop_us = timed_us(loop)
        row = {"gemm": name, "M": M, "K": K, "N": N, "TFLOP": round(flops / 1e12, 4),
               "dense_us": round(dense_us, 1), "dense_tflops": round(flops / dense_us / 1e6, 1),
               "dense_frac": round(flops / dense_us / 1e6 / PEAK_BF16_TFLOPS, 4),
               "per_expert_loop_us": round(loop_us, 1), "per_expert_loop_tflops": round(flops / loop_us / 1e6, 1)}
        rows.append(row)
        print(f"bench: vendor gemm {row}", file=sys.stderr, flush=True)
        del a, w, c, a_e, c_e
    rec = {"metric": "vendor dense bf16 GEMM on the Mixtral expert-GEMM shapes (context)",
           "value": rows[0]["dense_tflops"], "unit": "TFLOP/s", "n_gpus": 1, "higher_is_better": True,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "torch.matmul on [S*k, K] x [K, N], mixtral shapes"}, "rows": rows}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default="mixtral", help="tiny | mixtral | gptoss | dsv3 | qwen2")
    ap.add_argument("--S", type=int, default=None, help="token count (default: the configuration's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--op", default="layer", choices=["layer", "ffn_bwd", "train", "pl_fwd", "pl_bwd", "map_sweep", "route", "vendor_gemm"],
                    help="layer: the MoE forward (default); ffn_bwd: the expert FFN backward; "
                         "pl_fwd / pl_bwd: ParallelLinear up-projection")
    ap.add_argument("--dw-bf16", action="store_true",
                    help="ffn_bwd / train / pl_bwd: weight gradients stored as bf16 (the *_bf16w entry points)")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing of the forward")
    ap.add_argument("--no-combines", action="store_true",
                    help="skip timing the forward with the atomic combine beside the default one")
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="warm-up runs at least this long as well as at least --warmup steps")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run three device-to-device copies of BYTES (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the dropless MoE forward here runs on a single MI355X "
              "(expert- or token-parallel sharding is not built). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_mixture_experts_gemv_amd as smoe
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings scale
        # the same counters of the MoE kernels to bytes
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "launches": 3}))
        return
    if args.op == "route":
        bench_route(args)
        return
    if args.op == "vendor_gemm":
        bench_vendor_gemm(args)
        return
    if args.op == "map_sweep":
        bench_map_sweep(args)
        return
    cfg = wl.CONFIGS[args.config]
    if args.S:
        cfg = cfg.with_S(args.S)
    S, D, F, E, k = cfg.S, cfg.D, cfg.F, cfg.E, cfg.k
    print(f"bench: {cfg.describe()} steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)
    p = wl.make_problem(cfg, S=S, device="cuda")
    if args.op in ("ffn_bwd", "train"):
        bench_ffn_bwd(args, cfg, p, train=args.op == "train")
        return
    if args.op != "layer":
        bench_parallel_linear(args, cfg, p)
        return
    layer = smoe.MoELayer(p["wg"], p["w1"], p["w3"], p["w2"], k, S)
    topk = (p["ids"], p["weights"]) if "ids" in p else None
    stream = torch.cuda.current_stream()

    def step():
        layer.forward(p["x"], topk=topk)

    warm = warm_up(step, args.warmup, args.warmup_seconds)
    # the headline: K steps with nothing but the forward passes in the stream
    ms, wall = timed(step, args.steps, stream)
    # per-kernel durations from a second loop of K steps with HIP events around every launch
    kern, ms_profiled = profiled(step, args.steps, stream)

    combines = None
    if not args.no_combines:
        # the other combine on the same inputs: the fp32 atomic scatter-add (smaller workspace)
        alt = smoe.MoELayer(p["wg"], p["w1"], p["w3"], p["w2"], k, S, atomic=True)

        def step_atomic():
            alt.forward(p["x"], topk=topk)

        warm_up(step_atomic, args.warmup, args.warmup_seconds)
        ms_atomic, _ = timed(step_atomic, args.steps, stream)
        kern_atomic, _ = profiled(step_atomic, args.steps, stream)
        del alt
        per = lambda kk: {n: round(1e3 * tot / c, 2) for n, (tot, c) in kk.items()}
        combines = {"rows": {"ms_per_step": round(ms, 4), "kernels_us": per(kern)},
                    "atomic": {"ms_per_step": round(ms_atomic, 4), "kernels_us": per(kern_atomic)}}

    graph_ms = None
    if not args.no_graph:
        # the same forward captured once as a HIP graph and replayed: no per-kernel launch cost
        layer.capture(p["x"], topk)
        warm_up(layer.replay, args.warmup, args.warmup_seconds)
        graph_ms, _ = timed(layer.replay, args.steps, stream)

    flops = layer_flops(S, D, F, E, k, with_router=topk is None)
    tokens_per_s = S / (ms / 1e3)
    kernels = {name: {"avg_us": 1e3 * tot / n, "launches": n} for name, (tot, n) in kern.items()}
    gu_ms = kern["ffn_gate_up_gemm"][0] / kern["ffn_gate_up_gemm"][1]
    gu_flops = 4.0 * S * k * D * F
    # algorithmic bytes of the gate+up launch: the touched experts' W1 and W3
    # once, x once, h written once (the touched count is read back after the
    # timed region)
    touched = int((layer.map[0] > 0).sum().item())
    gu_bytes = touched * 2.0 * D * F * 2 + S * D * 2.0 + S * k * F * 2.0
    # the roofline that bounds this launch: the larger of its MFMA and HBM floors
    hbm_bound = gu_bytes / (PEAK_HBM_GBS * 1e9) > gu_flops / (PEAK_BF16_TFLOPS * 1e12)
    traffic = load_traffic(cfg.name, S * k)
    if hbm_bound:
        achieved = gu_bytes / (gu_ms / 1e3) / 1e9
        roof = {"kernel": "ffn_gate_up_gemm", "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": gu_bytes, "touched_experts": touched,
                "avg_launch_us": round(gu_ms * 1e3, 2)}
    else:
        achieved = gu_flops / (gu_ms / 1e3) / 1e12
        roof = {"kernel": "ffn_gate_up_gemm", "bound": "mfma", "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "algorithmic_flops_per_launch": gu_flops, "avg_launch_us": round(gu_ms * 1e3, 2)}
    rec = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} MoE layer forward (dropless, SwiGLU experts)", "S": S, "D": D, "F": F,
                   "E": E, "k": k, "routing": "router top-k" if topk is None else "Zipf(1.2) expert draws"},
        "layer_tflops": round(flops / (ms / 1e3) / 1e12, 1),
        "layer_mfma_frac": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "roofline": roof,
        "kernels": {n: {"avg_us": round(v["avg_us"], 2), "launches": v["launches"]} for n, v in kernels.items()},
        "ms_per_step_profiled_loop": round(ms_profiled, 4),
        "warmup_steps_run": warm,
        "wall_s_timed_region": round(wall, 3),
    }
    if combines is not None:
        rec["combines"] = combines
    if graph_ms is not None:
        rec["graph_replay"] = {"ms_per_step": round(graph_ms, 4), "tokens_per_s": round(S / (graph_ms / 1e3), 1)}
    if not args.no_cpu_baseline:
        print("bench: timing the fp64 CPU oracle on a sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(cfg, p, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
