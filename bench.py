"""Benchmark of the fused MoE router on one MI355X.

One step = one pass of the whole router hot path over one batch: the top-k
forward (score function + selection + dense probs / routing map /
intermediate), the top-k backward, the aux-loss score forward and its
backward, on the headline workload (T=8192 tokens, E=2304 experts, K=36,
fp32 softmax logits ~ N(0, std 2)).

Throughput is effective bandwidth, counted as in the fused-router page's
"Performance" paragraph ("[Common] Optimize fused router forward/backward
kernels", NVIDIA TransformerEngine pull request 3012): the minimum bytes a
kernel must move (read its inputs once, write its outputs once) divided by
its time.  Algorithmic bytes per element: forward 13 (fp32 logits + probs,
1-byte map, fp32 intermediate), backward 13, aux forward 13, aux backward
12.  `value` = all bytes of a step / step time.

Inputs are resident in HBM before the timed region.  Every kernel reads
buffers last touched several kernels earlier: the step's kernels use
different sets out of >= 2 GiB of rotating buffer sets, so neither the
L2 nor the 256 MB Infinity Cache holds them (pass --warm to reuse one set).

Prints one JSON line.  --gpus above 1 exits: this router is benchmarked on
one GPU.
"""
import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective HBM GB/s (and % of 8 TB/s) for router fwd/bwd at T=8192, E/K sweep"
PEAK_GBPS = 8000.0          # MI355X HBM3E
BYTES_PER_ELEM = {"topk_fwd": 13, "topk_bwd": 13, "aux_fwd": 13, "aux_bwd": 12}
BF16_BYTES_PER_ELEM = {"topk_fwd": 9, "topk_bwd": 9, "aux_fwd": 9, "aux_bwd": 8}
# Load-balancing loss passes (tokens per expert from the aux map, the loss over
# the aux scores, its gradient): bytes per element of [T,E] plus per-expert
# and scalar terms, fp32 scores.
LOSS_KINDS = ["tokens_per_expert", "aux_loss_fwd", "aux_loss_bwd"]


def loss_bytes(kind, T, E, esz):
    if kind == "tokens_per_expert":
        return T * E * 1 + E * 8           # map read, counts written
    return T * E * esz + E * 8 + 4         # scores read (or grad written), counts, scalar


# GPU kernel symbol of each pass: the top-k and aux passes share kernels, so
# a profiler reports one average per symbol over both passes.
KERNEL_SYMBOL = {"topk_fwd": "fwd_kernel", "topk_bwd": "bwd_kernel",
                 "aux_fwd": "fwd_kernel", "aux_bwd": "bwd_kernel",
                 "tokens_per_expert": "count_kernel", "aux_loss_fwd": "loss_kernel",
                 "aux_loss_bwd": "loss_bwd_kernel", "shared_gate": "shared_gate_kernel",
                 "topk_fwd_grouped": "grouped_fwd_kernel"}
# B300 figures of the fused-router page for this exact shape (context only).
PAGE_B300_GBPS = {"topk_fwd": 964, "topk_bwd": 2766, "aux_fwd": 891, "aux_bwd": 4201}


# Sources each kernel symbol is built from (for the freshness check of the
# committed counter summaries).
_ROUTER_SOURCES = ["router_api.cpp", "router_device.h", "router_io.h", "router_kernels.h",
                   "router_launch.h", "router_params.h", "router_lpt16.hip", "router_lpt32.hip",
                   "router_lpt64a.hip", "router_lpt64b.hip", "router_lpt64c.hip",
                   "router_scalar.hip", "router_scalar2.hip"]
_LOSS_SOURCES = ["router_api.cpp", "router_device.h", "router_io.h", "router_params.h",
                 "router_loss.hip"]
_GATE_SOURCES = ["router_api.cpp", "router_device.h", "router_io.h", "router_params.h",
                 "router_topk_wave.h", "router_gate.hip"]
_GROUPED_SOURCES = ["router_api.cpp", "router_device.h", "router_io.h", "router_kernels.h",
                    "router_params.h", "router_grouped.h", "router_grouped.hip"]
_ROUTE_SOURCES = ["router_api.cpp", "router_device.h", "router_io.h", "router_params.h",
                  "router_topk_wave.h", "router_route.hip"]
SYMBOL_SOURCES = {"fwd_kernel": _ROUTER_SOURCES, "bwd_kernel": _ROUTER_SOURCES,
                  "loss_kernel": _LOSS_SOURCES, "count_kernel": _LOSS_SOURCES,
                  "loss_bwd_kernel": _LOSS_SOURCES, "shared_gate_kernel": _GATE_SOURCES,
                  "grouped_fwd_kernel": _GROUPED_SOURCES, "route_maps_kernel": _ROUTE_SOURCES}


def path_threshold_desc(router):
    """The top-k path setting as reported in the JSON line."""
    t = router.get_topk_path_threshold()
    if t == router.TOPK_PATH_AUTO:
        return "auto (argmax rounds for K < 5 / 4 / 2 at <= 4 / <= 8 / more elements per lane)"
    return t


def kernel_source_hash(symbol="fwd_kernel"):
    h = hashlib.sha256()
    for name in sorted(SYMBOL_SOURCES[symbol]):
        with open(os.path.join(ROOT, "score_function_top_amd", "csrc", name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _summary(path, symbol):
    """key: value lines of a committed counter summary, or None when it is
    missing or was taken on other kernel sources than the current ones."""
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.split("#")[0].strip()
    if vals.get("kernel_source_hash") != kernel_source_hash(symbol):
        return None
    return vals


def read_traffic(kind, workload="c4_2304x36"):
    """Measured HBM bytes per launch of pass `kind` from its own committed
    profiler summary, if that was taken on the current kernel sources."""
    vals = _summary(os.path.join(ROOT, "profiles", f"hbm_traffic_{kind}_{workload}.txt"),
                    KERNEL_SYMBOL[kind])
    try:
        return float(vals["hbm_bytes_per_launch"]) if vals else None
    except (KeyError, ValueError):
        return None


def read_valu(kind, workload="c4_2304x36"):
    """VALU issue of pass `kind` from its committed counter summary
    (SQ_ACTIVE_INST_VALU in 4-cycle units per launch, and VALU instructions
    per wave), if it was taken on the current kernel sources."""
    vals = _summary(os.path.join(ROOT, "profiles", f"valu_{kind}_{workload}.txt"),
                    KERNEL_SYMBOL[kind])
    try:
        return {"active_valu_quads_per_launch": float(vals["active_valu_quads_per_launch"]),
                "valu_insts_per_wave": float(vals["valu_insts_per_wave"]),
                "simds": int(vals["simds"])} if vals else None
    except (KeyError, ValueError):
        return None


def valu_busy(valu, us, clock_khz):
    """Share of the kernel's time the VALUs issue: SQ_ACTIVE_INST_VALU x 4
    cycles over (SIMDs x duration x engine clock)."""
    if not valu or not clock_khz:
        return None
    valu_us = valu["active_valu_quads_per_launch"] * 4 / valu["simds"] / (clock_khz * 1e-3)
    return {"valu_us_per_launch": round(valu_us, 2), "busy": round(valu_us / us, 3),
            "valu_insts_per_wave": valu["valu_insts_per_wave"]}


def environment(torch, router):
    """GPU, clocks, ROCm and the build the timed library came from."""
    env = {"gpu": torch.cuda.get_device_name(0),
           "arch": torch.cuda.get_device_properties(0).gcnArchName,
           "torch_hip": torch.version.hip}
    try:
        env.update(router.device_query())
    except router.RouterError:
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    info = os.path.join(ROOT, "score_function_top_amd", "librouter.build.json")
    try:
        with open(info) as f:
            b = json.load(f)
        env["hipcc"] = b.get("hipcc")
        env["hipcc_flags"] = " ".join(b.get("flags", []))
        env["built_from_git"] = b.get("git")
    except (OSError, ValueError):
        env["build_info"] = None
    return env


def oracle_gbps(synth, wl, thr, kinds, T=None):
    """Oracle GB/s (median of 3 runs, same byte formula as the GPU) per
    pass over the first T tokens of `wl`."""
    import numpy as np
    import oracle
    T = T or wl.T
    x64 = wl.logits()[1][:T]
    g64 = wl.grad()[1][:T]
    bias = wl.bias()
    b64 = None if bias is None else bias.astype(np.float64)
    bpe = BYTES_PER_ELEM if wl.dtype == synth.F32 else BF16_BYTES_PER_ELEM
    out = {}
    S = M = AS = None
    for kind in kinds:
        walls = []
        for _ in range(3):
            t0 = time.perf_counter()
            if kind == "topk_fwd":
                _, M, S, _ = oracle.topk_fwd(x64, wl.K, wl.score_fn, wl.renorm, wl.num_groups,
                                             wl.group_topk, wl.scaling_factor, b64, threads=thr)
            elif kind == "topk_bwd":
                oracle.topk_bwd(g64, S, M, wl.K, wl.score_fn, wl.renorm, wl.scaling_factor,
                                threads=thr)
            elif kind == "aux_fwd":
                _, _, AS = oracle.aux_fwd(x64, wl.K, wl.score_fn, wl.aux_renorm, threads=thr)
            else:
                oracle.aux_bwd(g64, AS, wl.score_fn, wl.aux_renorm, threads=thr)
            walls.append(time.perf_counter() - t0)
        nb = T * wl.E * bpe[kind] + (wl.E * 4 if (kind == "topk_fwd" and bias is not None)
                                     else 0)
        out[kind] = round(nb / float(np.median(walls)) / 1e9, 3)
    return out


SWEEP_ORACLE_TOKENS = 1024


def cpu_configs_and_sweep(synth):
    """The oracle beside the GPU on the five workloads and the E/K sweep
    (GB/s per pass)."""
    thr = max(1, min(os.cpu_count() or 1, 64))
    t0 = time.perf_counter()
    configs = {}
    for name, wl in synth.WORKLOADS.items():
        if wl.T * wl.E > 16384 * 2304:
            continue
        kinds = ["topk_fwd", "topk_bwd"] + (["aux_fwd", "aux_bwd"] if wl.aux else [])
        configs[name] = oracle_gbps(synth, wl, thr, kinds)
    sweep = {}
    for sf in (synth.SOFTMAX, synth.SIGMOID):
        for E in (256, 512, 2304):
            for K in (4, 8, 22, 36):
                wl = synth.sweep_workload(E, K, sf)
                sname = "softmax" if sf == synth.SOFTMAX else "sigmoid"
                sweep[f"{sname}_{E}x{K}"] = oracle_gbps(
                    synth, wl, thr, ["topk_fwd", "topk_bwd", "aux_fwd", "aux_bwd"],
                    T=SWEEP_ORACLE_TOKENS)
    return {"configs_GBps": configs, "sweep_GBps": sweep, "cores": thr, "kind": "oracle",
            "sample": f"whole workloads for the configs, the first {SWEEP_ORACLE_TOKENS} of "
                      f"8192 tokens per sweep cell",
            "note": f"fp64 C oracle on {thr} host threads, median of 3 runs per pass, same "
                    f"byte formulas as the GPU figures; {time.perf_counter() - t0:.1f} s"}


def cpu_baseline(wl, tokens):
    """The fp64 oracle (as it stands) over the first `tokens` tokens of the
    workload, all four passes, on this host's cores."""
    import numpy as np
    import oracle
    thr = max(1, min(os.cpu_count() or 1, 64))
    x_st, x64 = wl.logits()
    g_st, g64 = wl.grad()
    a_st, a64 = wl.aux_grad()
    x64, g64, a64 = x64[:tokens], g64[:tokens], a64[:tokens]
    walls = []
    t_start = time.perf_counter()
    while len(walls) < 3 or time.perf_counter() - t_start < 10.0:
        t0 = time.perf_counter()
        P, M, S, _ = oracle.topk_fwd(x64, wl.K, wl.score_fn, wl.renorm, threads=thr)
        oracle.topk_bwd(g64, S, M, wl.K, wl.score_fn, wl.renorm, wl.scaling_factor,
                        threads=thr)
        A, AM, AS = oracle.aux_fwd(x64, wl.K, wl.score_fn, wl.aux_renorm, threads=thr)
        oracle.aux_bwd(a64, AS, wl.score_fn, wl.aux_renorm, threads=thr)
        walls.append(time.perf_counter() - t0)
    dt = float(np.median(walls))
    bytes_ = tokens * wl.E * sum(BYTES_PER_ELEM.values())
    return {"value": round(bytes_ / dt / 1e9, 3), "unit": "GB/s", "cores": thr,
            "kind": "oracle",
            "sample": f"first {tokens} of {wl.T} tokens of the workload, all four passes "
                      f"(topk fwd, topk bwd, aux fwd, aux bwd), fp64 C oracle, median of "
                      f"{len(walls)} runs over >= 10 s ({dt:.2f} s wall each, {thr} threads), "
                      f"same byte formula as the GPU value"}


def graph_us_per_launch(torch, launches, replays=1):
    """Captures `launches` (callables that enqueue one kernel each on the
    current stream) into one HIP graph, replays it twice untimed, then
    `replays` times with one event pair around each replay, and returns the
    median over replays of the microseconds per launch.  Graph replay
    removes the host-side launch cost, which dominates kernels of a few
    microseconds."""
    return graph_us_stats(torch, launches, replays)["median"]


def graph_us_stats(torch, launches, replays=11):
    """As graph_us_per_launch; returns {"median", "p10", "p90", "replays",
    "launches"}: per-launch microseconds over the timed replays."""
    import numpy as np
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in launches[:3]:                # warm the launch path
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in launches:
            f()
    for _ in range(2):
        g.replay()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(replays)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 / len(launches) for a, b in evs])
    del g
    p10, p50, p90 = np.percentile(us, [10, 50, 90])
    return {"median": float(p50), "p10": float(p10), "p90": float(p90), "replays": replays,
            "launches": len(launches)}


# Launches per graph for the sweep and config cells: at least this many,
# cycling through every rotating buffer set.
CELL_LAUNCHES = 200
CELL_REPLAYS = 11


def cell_launches(f, sets):
    """max(CELL_LAUNCHES, len(sets)) launches of f cycling through the sets."""
    n = len(sets)
    return [lambda st=sets[i % n]: f(st) for i in range(max(CELL_LAUNCHES, n))]


def cell_result(nbytes, st):
    """us (median) and GB/s of a cell, with the spread over replays."""
    return {"us": round(st["median"], 2), "GBps": round(nbytes / st["median"] / 1e3, 1),
            "us_p10": round(st["p10"], 2), "us_p90": round(st["p90"], 2)}


def run_sweep(torch, router, synth, np):
    """Per-pass microseconds and effective GB/s over the T=8192 E/K grid of
    the router page's benchmark tables (softmax without renorm, sigmoid with
    renorm), cold caches (>= 2 GiB of rotating buffer sets per cell, every
    set used in each graph of launches)."""
    dev = torch.device("cuda:0")
    out = {}
    for sf in (synth.SOFTMAX, synth.SIGMOID):
        for E in (256, 512, 2304):
            for K in (4, 8, 22, 36):
                wl = synth.sweep_workload(E, K, sf)
                T = wl.T
                sname = "softmax" if sf == synth.SOFTMAX else "sigmoid"
                x = torch.from_numpy(wl.logits()[0]).to(dev)
                g = torch.from_numpy(wl.grad()[0]).to(dev)
                set_bytes = T * E * (4 * 3 + 4 + 1)
                n = max(4, -(-(2 << 30) // set_bytes))
                sets = []
                for _ in range(n):
                    st = {"x": x.clone(), "g": g.clone(),
                          "p": torch.empty_like(x), "dx": torch.empty_like(x),
                          "i": torch.empty_like(x),
                          "m": torch.empty(T, E, dtype=torch.bool, device=dev)}
                    sets.append(st)
                calls = {
                    "topk_fwd": lambda st: router.router_topk_fwd(
                        st["x"], K, sname, wl.renorm, out=(st["p"], st["m"], st["i"])),
                    "topk_bwd": lambda st: router.router_topk_bwd(
                        st["g"], st["i"], st["m"], K, sname, wl.renorm, out=st["dx"]),
                    "aux_fwd": lambda st: router.router_aux_scores(
                        st["x"], K, sname, wl.aux_renorm, out=(st["p"], st["m"], st["i"])),
                    "aux_bwd": lambda st: router.router_aux_scores_bwd(
                        st["g"], st["i"], sname, wl.aux_renorm, out=st["dx"]),
                }
                cell = {}
                for kind in ("topk_fwd", "topk_bwd", "aux_fwd", "aux_bwd"):
                    if kind.endswith("bwd"):          # backward inputs from its forward
                        for st in sets:
                            calls[kind.replace("bwd", "fwd")](st)
                    f = calls[kind]
                    st = graph_us_stats(torch, cell_launches(f, sets), CELL_REPLAYS)
                    cell[kind] = cell_result(T * E * BYTES_PER_ELEM[kind], st)
                out[f"{sname}_{E}x{K}"] = cell
                del sets, x, g
    return out


def workload_cells(torch, router, synth, np, wl, kinds=None):
    """Per-pass cells (us median / p10 / p90, GB/s) of one workload, cold:
    >= 2 GiB of rotating buffer sets, a HIP graph of max(200, sets)
    launches per pass, replayed CELL_REPLAYS times."""
    dev = torch.device("cuda:0")
    T, E, K = wl.T, wl.E, wl.K
    sname = "softmax" if wl.score_fn == synth.SOFTMAX else "sigmoid"
    esz = 4 if wl.dtype == synth.F32 else 2

    def host(arr):
        a = np.ascontiguousarray(arr)
        if wl.dtype == synth.F32:
            return torch.from_numpy(a)
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)

    x, g = host(wl.logits()[0]).to(dev), host(wl.grad()[0]).to(dev)
    bias = wl.bias()
    bd = None if bias is None else torch.from_numpy(bias).to(dev)
    set_bytes = T * E * (4 * esz + 4 + 1)
    n = max(4, -(-(2 << 30) // set_bytes))
    sets = [{"x": x.clone(), "g": g.clone(), "p": torch.empty_like(x),
             "dx": torch.empty_like(x),
             "i": torch.empty(T, E, dtype=torch.float32, device=dev),
             "m": torch.empty(T, E, dtype=torch.bool, device=dev)} for _ in range(n)]
    calls = {
        "topk_fwd": lambda st: router.router_topk_fwd(
            st["x"], K, sname, wl.renorm, wl.num_groups, wl.group_topk, wl.scaling_factor,
            bd, out=(st["p"], st["m"], st["i"])),
        "topk_bwd": lambda st: router.router_topk_bwd(
            st["g"], st["i"], st["m"], K, sname, wl.renorm, wl.scaling_factor, out=st["dx"]),
        "aux_fwd": lambda st: router.router_aux_scores(
            st["x"], K, sname, wl.aux_renorm, out=(st["p"], st["m"], st["i"])),
        "aux_bwd": lambda st: router.router_aux_scores_bwd(
            st["g"], st["i"], sname, wl.aux_renorm, out=st["dx"]),
    }
    if kinds is None:
        kinds = ["topk_fwd", "topk_bwd"] + (["aux_fwd", "aux_bwd"] if wl.aux else [])
    bpe = BYTES_PER_ELEM if wl.dtype == synth.F32 else BF16_BYTES_PER_ELEM
    cell = {}
    for kind in kinds:
        if kind.endswith("bwd"):
            for st in sets:
                calls[kind.replace("bwd", "fwd")](st)
        f = calls[kind]
        st = graph_us_stats(torch, cell_launches(f, sets), CELL_REPLAYS)
        nb = T * E * bpe[kind] + (E * 4 if (kind == "topk_fwd" and bias is not None) else 0)
        cell[kind] = cell_result(nb, st)
    del sets, x, g
    return cell


def run_configs(torch, router, synth, np):
    """Per-pass microseconds and effective GB/s of the five router workloads
    (bias, group-limited and bf16 variants included), cold caches, launches
    replayed from a HIP graph."""
    return {name: workload_cells(torch, router, synth, np, wl)
            for name, wl in synth.WORKLOADS.items()}


GRID_STUDY = ["c2_softmax_256x4", "c4_softmax_2304x36", "c5_group_sigmoid_256x8_bf16"]


def run_grid_study(torch, router, synth, np, names=GRID_STUDY):
    """The top-k forward and backward of each workload under both grid
    modes of the library: one block per token group ("full", the default)
    and the occupancy-sized persistent grid ("persistent")."""
    out = {}
    try:
        for name in names:
            wl = synth.WORKLOADS[name]
            res = {}
            for mode, label in ((router.GRID_FULL, "full"), (router.GRID_PERSISTENT, "persistent")):
                router.set_grid_mode(mode)
                for kind, c in workload_cells(torch, router, synth, np, wl,
                                              ["topk_fwd", "topk_bwd"]).items():
                    res.setdefault(kind, {})[label] = c
            out[name] = res
    finally:
        router.set_grid_mode(router.GRID_FULL)
    return out


# Fused shared-gate op of the aiter page on gfx950 (MI35X), microseconds per
# call at E=512, H=4096, top-10, one shared expert, bf16 (context only: its
# own table, "PROVISIONAL - single run").
PAGE_AITER_FUSED_US = {1: 14.6, 4: 13.9, 16: 15.2, 64: 14.8, 256: 15.8, 1024: 16.6,
                       4096: 23.5, 16384: 44.2}


def shared_gate_bytes(M, E=512, H=4096, K=10, S=1, esz=2):
    """Algorithmic bytes: gating and hidden rows read once, gate weights
    read once, K+S weights and ids written per token."""
    return M * E * esz + M * H * esz + S * H * esz + M * (K + S) * 8


def run_shared_gate(torch, router, synth, only_m=None):
    """Routed top-k with the shared-expert gate at the aiter page's shape
    (E=512 experts, hidden 4096, top-10, one shared expert, bf16) over its
    token sweep; calls replayed from a HIP graph; from M=1024 on the inputs
    rotate over >= 2 GiB of buffer sets (cold caches)."""
    dev = torch.device("cuda:0")
    E, H, K, S = 512, 4096, 10, 1
    out = {}
    for M in ((only_m,) if only_m else (1, 4, 16, 64, 256, 1024, 4096, 16384)):
        def dev_bf16(seed, shape, std):
            bits = synth.storage(synth.normal(seed, shape, std), synth.BF16)[0]
            return torch.from_numpy(bits.view("int16")).to(dev).view(torch.bfloat16)
        x0 = dev_bf16(9700 + M, (M, E), 1.0)
        h0 = dev_bf16(9701 + M, (M, H), 1.0)
        g = dev_bf16(9702, (S, H), 0.05)
        per = M * (E + H) * 2
        n = max(1, -(-(2 << 30) // per)) if M >= 1024 else 1
        sets = [(x0.clone(), h0.clone()) for _ in range(n)] if n > 1 else [(x0, h0)]
        w = torch.empty((M, K + S), dtype=torch.float32, device=dev)
        ids = torch.empty((M, K + S), dtype=torch.int32, device=dev)
        f = lambda st: router.router_topk_shared_gate(st[0], st[1], g, K, True, 1.0, E,
                                                      out=(w, ids))
        stt = graph_us_stats(torch, cell_launches(f, sets), CELL_REPLAYS)
        us = stt["median"]
        nb = shared_gate_bytes(M, E, H, K, S)
        out[f"M{M}"] = {"us_graph": round(us, 2), "us_p10": round(stt["p10"], 2),
                        "us_p90": round(stt["p90"], 2), "GBps": round(nb / us / 1e3, 1),
                        "frac_of_peak": round(nb / us / 1e3 / PEAK_GBPS, 4),
                        "algo_bytes": nb, "cold": n > 1,
                        "page_aiter_fused_us_context": PAGE_AITER_FUSED_US.get(M)}
        del sets, x0, h0
    return out


def copy_calibration(torch, dev, mib):
    """A plain device copy of `mib` MiB (the profiler's scale reference for
    byte counters), timed; None when mib is 0."""
    if not mib:
        return None
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        b.copy_(a)
    c0.record()
    for _ in range(10):
        b.copy_(a)
    c1.record()
    torch.cuda.synchronize()
    us = c0.elapsed_time(c1) * 100
    return {"bytes_read": n, "bytes_written": n, "us_avg": round(us, 2),
            "GBps": round(2 * n / us / 1e3, 1)}


# Read:write bytes per element of each pass (fp32), for the same-mix ceiling.
STREAM_MIX = {"topk_fwd": (4, 9), "topk_bwd": (9, 4), "aux_fwd": (4, 9), "aux_bwd": (8, 4),
              "copy": (4, 4), "read_only": (4, 0), "write_only": (0, 4),
              "map_read": (1, 0)}
# the stream mix whose bytes equal each aux-loss pass's (fp32 scores): the
# count reads the byte map, the loss reads the scores, its gradient writes
# them (the per-expert vectors are a few KB)
LOSS_STREAM = {"tokens_per_expert": "map_read", "aux_loss_fwd": "read_only",
               "aux_loss_bwd": "write_only"}


STREAM_UNITS = (1, 2, 4)   # 16-byte units per thread tried for each mix


def run_stream_ceiling(torch, router, T, E):
    """The bandwidth this device reaches for each pass's read:write mix with
    no arithmetic: the library's streaming kernel moving the pass's bytes
    (T*E elements), cold (rotating buffers of >= 2 GiB), timed like the
    config cells, with 1, 2 and 4 units per thread; the fastest is the
    ceiling (us_by_units keeps each).  GB/s and the share of the 8 TB/s
    peak."""
    dev = torch.device("cuda:0")
    out = {}
    for kind, (r, w) in STREAM_MIX.items():
        rb, wb = T * E * r, T * E * w
        n = max(4, -(-(2 << 30) // (rb + wb)))
        sets = [(torch.empty(max(rb, 16), dtype=torch.uint8, device=dev),
                 torch.empty(max(wb, 16), dtype=torch.uint8, device=dev)) for _ in range(n)]
        for a, _ in sets:
            a.fill_(1)
        best, by_units = None, {}
        for units in STREAM_UNITS:
            f = lambda st, u=units: router.stream_bandwidth(st[0], rb, st[1], wb, u)
            st = graph_us_stats(torch, cell_launches(f, sets), CELL_REPLAYS)
            by_units[str(units)] = round(st["median"], 2)
            if best is None or st["median"] < best[1]["median"]:
                best = (units, st)
        res = cell_result(rb + wb, best[1])
        res["frac_of_peak"] = round((rb + wb) / best[1]["median"] / 1e3 / PEAK_GBPS, 4)
        res["read_write_bytes_per_element"] = [r, w]
        res["units_per_thread"] = best[0]
        res["us_by_units"] = by_units
        out[kind] = res
        del sets
    if E % 256 == 0 and E <= 4096:
        # the forward's own pattern: one wave per row, the row read whole,
        # then two fp32 rows and one byte row written
        nb = T * E * 13
        n = max(4, -(-(2 << 30) // nb))
        sets = [(torch.empty(T, E, dtype=torch.float32, device=dev),
                 torch.empty(T, E, dtype=torch.float32, device=dev),
                 torch.empty(T, E, dtype=torch.float32, device=dev),
                 torch.empty(T, E, dtype=torch.uint8, device=dev)) for _ in range(n)]
        for st in sets:
            st[0].fill_(1.0)
        f = lambda st: router.row_stream_bandwidth(*st)
        st = graph_us_stats(torch, cell_launches(f, sets), CELL_REPLAYS)
        res = cell_result(nb, st)
        res["frac_of_peak"] = round(nb / st["median"] / 1e3 / PEAK_GBPS, 4)
        res["read_write_bytes_per_element"] = [4, 9]
        out["topk_fwd_row_pattern"] = res
        del sets
    return out


def run_decode_route(torch, router, synth, steps):
    """Latency of decode-shape routing with expert maps (one workgroup per
    call) at the onnxruntime page's shapes: T in 1..4 rows, E = 512 experts,
    K in {1, 2, 4, 6, 8, 10}, softmax with renormalisation, fp32 logits.
    us_graph: per call, median over replays of a HIP graph of CELL_LAUNCHES
    calls (p10/p90 beside it); us_eager:
    `steps` back-to-back calls on the stream, one event pair (host launch
    included when it is the bottleneck).  floor_us_graph: a one-element fill
    kernel the same way, the cost of any dependent kernel on this device."""
    dev = torch.device("cuda:0")
    out = {}
    for T in (1, 2, 3, 4):
        for K in (1, 2, 4, 6, 8, 10):
            x = torch.from_numpy(synth.storage(synth.normal(9000 + 10 * T + K, (T, 512)),
                                               synth.F32)[0]).to(dev)
            res = router.router_route_maps(x, K, "softmax", True)
            f = lambda: router.router_route_maps(x, K, "softmax", True, out=res)
            gst = graph_us_stats(torch, [f] * CELL_LAUNCHES, CELL_REPLAYS)
            g_us = gst["median"]
            for _ in range(3):
                f()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for _ in range(steps):
                f()
            b.record()
            torch.cuda.synchronize()
            out[f"T{T}_K{K}"] = {"us_graph": round(g_us, 2), "us_graph_p10": round(gst["p10"], 2),
                                 "us_graph_p90": round(gst["p90"], 2),
                                 "us_eager": round(a.elapsed_time(b) * 1e3 / steps, 2)}
    one = torch.zeros(1, device=dev)
    out["floor_us_graph"] = round(graph_us_per_launch(torch, [one.zero_] * CELL_LAUNCHES,
                                                      CELL_REPLAYS), 2)
    return out


def workload_by_name(synth, name):
    """One of the five workloads, or a sweep cell named
    sweep_<softmax|sigmoid>_<E>x<K> (T=8192; a _bf16 suffix stores the
    logits and gradients in bf16)."""
    if name in synth.WORKLOADS:
        return synth.WORKLOADS[name]
    parts = name.split("_")
    bf16 = len(parts) == 4 and parts[3] == "bf16"
    if (len(parts) == 3 or bf16) and parts[0] == "sweep" and parts[1] in ("softmax", "sigmoid"):
        E, K = (int(v) for v in parts[2].split("x"))
        wl = synth.sweep_workload(E, K, synth.SOFTMAX if parts[1] == "softmax"
                                  else synth.SIGMOID)
        if bf16:
            wl = dataclasses.replace(wl, name=name, dtype=synth.BF16)
        return wl
    raise SystemExit(f"bench.py: unknown workload {name}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c4_softmax_2304x36")
    ap.add_argument("--warm", action="store_true", help="reuse one buffer set")
    ap.add_argument("--sets", type=int, default=0, help="rotating buffer sets (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="oracle sample size in tokens (0: the whole batch)")
    ap.add_argument("--only", choices=["topk_fwd", "topk_bwd", "aux_fwd", "aux_bwd"] + LOSS_KINDS,
                    help="time only this kernel kind (for profiler runs)")
    ap.add_argument("--only-decode-route", action="store_true",
                    help="time only the decode routing (for profiler runs)")
    ap.add_argument("--only-shared-gate", action="store_true",
                    help="time only the shared-gate sweep (for profiler runs)")
    ap.add_argument("--shared-gate-tokens", type=int, default=0,
                    help="with --only-shared-gate: one token count instead of the sweep")
    ap.add_argument("--grid-mode", choices=["full", "persistent"], default="full",
                    help="the library's grid mode for the whole run (for profiler runs)")
    ap.add_argument("--grid-study", action="store_true",
                    help="time only the grid study (both grid modes; for profiler runs)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the T=8192 E/K sweep object")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also time a plain device copy of this size (profiler scale)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.exit("bench.py: the router is benchmarked on one GPU only; --gpus above 1 "
                 "is not supported (tokens shard with no exchange, so one GPU's share "
                 "at its real shape is the measurement)")

    import numpy as np
    import torch
    from score_function_top_amd import router, synth

    if args.grid_study:
        torch.cuda.set_device(0)
        print(json.dumps({"grid_study": run_grid_study(torch, router, synth, np)}), flush=True)
        return
    if args.only_decode_route:
        torch.cuda.set_device(0)
        print(json.dumps({"decode_route": run_decode_route(torch, router, synth, args.steps)}),
              flush=True)
        return
    if args.only_shared_gate:
        torch.cuda.set_device(0)
        res = {"shared_gate": run_shared_gate(torch, router, synth,
                                              args.shared_gate_tokens or None),
               "kernel_source_hash": {"gate": kernel_source_hash("shared_gate_kernel")}}
        copy = copy_calibration(torch, torch.device("cuda:0"), args.copy_calibration_mib)
        if copy:
            res["copy_calibration"] = copy
        print(json.dumps(res), flush=True)
        return

    router.set_grid_mode(router.GRID_PERSISTENT if args.grid_mode == "persistent"
                         else router.GRID_FULL)
    wl = workload_by_name(synth, args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T, E, K = wl.T, wl.E, wl.K
    sname = "softmax" if wl.score_fn == synth.SOFTMAX else "sigmoid"
    tdt = torch.float32 if wl.dtype == synth.F32 else torch.bfloat16
    esz = 4 if wl.dtype == synth.F32 else 2

    # ---- inputs: seeded on the host once, copied into every buffer set
    def host(arr):
        a = np.ascontiguousarray(arr)
        if wl.dtype == synth.F32:
            return torch.from_numpy(a)
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)

    x_h = host(wl.logits()[0])
    g_h = host(wl.grad()[0])
    a_h = host(wl.aux_grad()[0])
    bias = wl.bias()
    bias_d = None if bias is None else torch.from_numpy(bias).to(dev)
    set_bytes = T * E * (esz * 6 + 4 * 2 + 1 * 2) + T * E * esz  # 11 arrays per set
    n_sets = 1 if args.warm else (args.sets or max(4, -(-(2 << 30) // set_bytes)))

    def new_set():
        s = {k: torch.empty(T, E, dtype=tdt, device=dev)
             for k in ("x", "probs", "g", "dx", "ascores", "ag", "adx")}
        s.update({k: torch.empty(T, E, dtype=torch.float32, device=dev)
                  for k in ("inter", "ainter")})
        s.update({k: torch.empty(T, E, dtype=torch.bool, device=dev)
                  for k in ("map", "amap")})
        s["x"].copy_(x_h)
        s["g"].copy_(g_h)
        s["ag"].copy_(a_h)
        return s

    sets = [new_set() for _ in range(n_sets)]
    ws_bytes = router.router_aux_loss_workspace_bytes(T, E)
    cws_bytes = router.router_tokens_per_expert_workspace_bytes(T, E)
    for s in sets:
        s["cnt"] = torch.zeros(E, dtype=torch.int64, device=dev)
        s["cws"] = torch.zeros(cws_bytes, dtype=torch.uint8, device=dev)
        s["loss"] = torch.empty((), dtype=torch.float32, device=dev)
        s["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    grad_loss = torch.ones(1, dtype=torch.float32, device=dev)

    def launch(kind, s):
        if kind == "topk_fwd":
            router.router_topk_fwd(s["x"], K, sname, wl.renorm, wl.num_groups, wl.group_topk,
                                   wl.scaling_factor, bias_d,
                                   out=(s["probs"], s["map"], s["inter"]))
        elif kind == "topk_bwd":
            router.router_topk_bwd(s["g"], s["inter"], s["map"], K, sname, wl.renorm,
                                   wl.scaling_factor, out=s["dx"])
        elif kind == "aux_fwd":
            router.router_aux_scores(s["x"], K, sname, wl.aux_renorm,
                                     out=(s["ascores"], s["amap"], s["ainter"]))
        elif kind == "aux_bwd":
            router.router_aux_scores_bwd(s["ag"], s["ainter"], sname, wl.aux_renorm,
                                         out=s["adx"])
        elif kind == "tokens_per_expert":
            router.router_tokens_per_expert(s["amap"], out=s["cnt"], workspace=s["cws"])
        elif kind == "aux_loss_fwd":
            router.router_aux_loss_fwd(s["ascores"], s["cnt"], T, K, synth.AUX_LOSS_COEFF,
                                       out=s["loss"], workspace=s["ws"])
        else:   # aux_loss_bwd: the gradient lands in the aux-backward output buffer
            router.router_aux_loss_bwd(grad_loss, s["cnt"], T, T, K, synth.AUX_LOSS_COEFF,
                                       dtype=tdt, out=s["adx"])

    all_kinds = ["topk_fwd", "topk_bwd", "aux_fwd", "aux_bwd"] + LOSS_KINDS
    step_kinds = all_kinds[:4]
    kinds = [args.only] if args.only else step_kinds
    # kernel k of step i works on set (i + k) % n: with n >= 4 every input was
    # last touched a full rotation of other buffers earlier (the backward
    # passes read the forward outputs of earlier steps)
    for s in sets:                       # produce every set's forward outputs
        launch("topk_fwd", s)
        launch("aux_fwd", s)
        launch("tokens_per_expert", s)
    torch.cuda.synchronize()

    def step(i):
        for kind in kinds:
            launch(kind, sets[(i + all_kinds.index(kind)) % n_sets])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: K whole steps, one event pair around them
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(args.warmup + i)
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)

    # ---- the same K steps replayed from one captured HIP graph
    graph_us = graph_us_per_launch(
        torch, [lambda i=i, kind=kind: launch(kind, sets[(i + all_kinds.index(kind)) % n_sets])
                for i in range(args.warmup, args.warmup + args.steps) for kind in kinds])
    ms_per_step_graph = graph_us * len(kinds) / 1e3

    # ---- per-kernel average launch duration: K back-to-back launches of one
    # kind (rotating sets, as in the step), one event pair around them
    per_kernel_us = {}
    per_launch_us = {}
    warm_us = {}
    timed_kinds = kinds if args.only else step_kinds + LOSS_KINDS
    for kind in timed_kinds:
        k0 = all_kinds.index(kind)
        for i in range(3):
            launch(kind, sets[(i + k0) % n_sets])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(args.steps):
            launch(kind, sets[(i + k0) % n_sets])
        b.record()
        torch.cuda.synchronize()
        per_kernel_us[kind] = a.elapsed_time(b) * 1e3 / args.steps
        # one event pair per launch: the spread of single launches
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i, (ea, eb) in enumerate(evs):
            ea.record()
            launch(kind, sets[(i + k0) % n_sets])
            eb.record()
        torch.cuda.synchronize()
        per_launch_us[kind] = np.array([ea.elapsed_time(eb) * 1e3 for ea, eb in evs])
        if kind in step_kinds and n_sets > 1:
            # warm: the same launches on one buffer set (its inputs and outputs
            # partly resident in the L2 and the Infinity Cache)
            s0 = sets[k0 % n_sets]
            launch(kind, s0)
            torch.cuda.synchronize()
            a.record()
            for i in range(args.steps):
                launch(kind, s0)
            b.record()
            torch.cuda.synchronize()
            warm_us[kind] = a.elapsed_time(b) * 1e3 / args.steps

    bpe = BYTES_PER_ELEM if wl.dtype == synth.F32 else BF16_BYTES_PER_ELEM
    kern = {}
    for kind in kinds:
        if kind in LOSS_KINDS:
            nbytes = loss_bytes(kind, T, E, esz)
        else:
            nbytes = T * E * bpe[kind] + (E * 4 if (kind == "topk_fwd" and bias is not None)
                                          else 0)
        avg = per_kernel_us[kind]
        p10, p50, p90 = np.percentile(per_launch_us[kind], [10, 50, 90])
        kern[kind] = {"us_avg": round(avg, 2), "algo_bytes": nbytes,
                      "GBps": round(nbytes / avg / 1e3, 1),
                      "frac_of_peak": round(nbytes / avg / 1e3 / PEAK_GBPS, 4),
                      "us_single_launch": {"p10": round(p10, 2), "median": round(p50, 2),
                                           "p90": round(p90, 2)}}
        if kind in warm_us:
            kern[kind]["warm"] = {"us_avg": round(warm_us[kind], 2),
                                  "GBps": round(nbytes / warm_us[kind] / 1e3, 1)}
        if args.workload == "c4_softmax_2304x36" and kind in PAGE_B300_GBPS:
            kern[kind]["page_b300_GBps_context"] = PAGE_B300_GBPS[kind]
    step_bytes = sum(k["algo_bytes"] for k in kern.values())
    ms_per_step = total_ms / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # roofline of the dominant kernel symbol: mean launch duration over its
    # passes (what a profiler reports for that symbol)
    by_sym = {}
    for kind in kinds:
        by_sym.setdefault(KERNEL_SYMBOL[kind], []).append(kind)
    dom = max(by_sym, key=lambda sym: sum(kern[k]["us_avg"] for k in by_sym[sym]))
    us = sum(kern[k]["us_avg"] for k in by_sym[dom]) / len(by_sym[dom])
    nb = sum(kern[k]["algo_bytes"] for k in by_sym[dom]) / len(by_sym[dom])
    # the symbol's traffic: the mean over its passes' own counter summaries
    # (all of them present and current), else null
    traffic = None
    if args.workload == "c4_softmax_2304x36" and not args.warm:
        tr = [read_traffic(k) for k in by_sym[dom]]
        traffic = round(sum(tr) / len(tr)) if all(t is not None for t in tr) else None
    env = environment(torch, router)
    roof = {"bound": "hbm", "kernel": dom, "passes": by_sym[dom], "us_avg": round(us, 2),
            "achieved": round(nb / us / 1e3, 1), "peak": PEAK_GBPS, "unit": "GB/s",
            "frac": round(nb / us / 1e3 / PEAK_GBPS, 4),
            "algo_bytes_per_launch": int(nb), "traffic": traffic}
    if args.workload == "c4_softmax_2304x36" and not args.warm:
        roof["valu"] = valu_busy(read_valu(by_sym[dom][0]), us, env.get("clock_khz"))
        # the committed counter summaries of every pass's kernel, where they
        # match the current sources
        for kind in kinds:
            if kind in LOSS_KINDS:
                continue
            kern[kind]["traffic"] = read_traffic(kind)
            kern[kind]["valu"] = valu_busy(read_valu(kind), kern[kind]["us_avg"],
                                           env.get("clock_khz"))

    copy = copy_calibration(torch, dev, args.copy_calibration_mib)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "graph_replay": {"ms_per_step": round(ms_per_step_graph, 4),
                         "value": round(step_bytes / (ms_per_step_graph * 1e-3) / 1e9, 1),
                         "note": "the same steps captured in one HIP graph and replayed"},
        "dtype": "f32" if wl.dtype == synth.F32 else "bf16",
        "data": "synthetic (seeded numpy PCG64 logits and gradients)",
        "config": {"workload": f"{wl.name} ({' + '.join(kinds)})",
                   "T": T, "E": E, "K": K, "score_function": sname,
                   "logits": f"N(0, std {wl.logit_std})", "renorm": wl.renorm,
                   "cache": "warm (one buffer set)" if args.warm else
                            f"cold ({n_sets} rotating buffer sets, "
                            f"{n_sets * set_bytes / 2**30:.2f} GiB)",
                   "path_threshold": path_threshold_desc(router)},
        "roofline": roof,
        "kernels": kern,
        "wall_s_timed_region": round(t_wall, 4),
        "device": torch.cuda.get_device_name(0),
        "environment": env,
        "kernel_source_hash": {"router": kernel_source_hash("fwd_kernel"),
                               "loss": kernel_source_hash("loss_kernel"),
                               "gate": kernel_source_hash("shared_gate_kernel"),
                               "grouped": kernel_source_hash("grouped_fwd_kernel"),
                               "route": kernel_source_hash("route_maps_kernel")},
    }
    if not args.only:
        loss = {}
        for kind in LOSS_KINDS:
            nb = loss_bytes(kind, T, E, esz)
            avg = per_kernel_us[kind]
            k0 = all_kinds.index(kind)
            g_us = graph_us_per_launch(
                torch, [lambda i=i: launch(kind, sets[(i + k0) % n_sets])
                        for i in range(args.steps)])
            sym = KERNEL_SYMBOL[kind]
            loss[kind] = {"kernels": [sym] + (["loss_final_kernel"] if sym == "loss_kernel"
                                              else []),
                          "us_avg": round(avg, 2), "us_graph": round(g_us, 2),
                          "algo_bytes": nb, "GBps": round(nb / avg / 1e3, 1),
                          "GBps_graph": round(nb / g_us / 1e3, 1),
                          "frac_of_peak": round(nb / avg / 1e3 / PEAK_GBPS, 4),
                          "traffic": read_traffic(kind) if not args.warm else None}
        out["aux_loss"] = loss
        out["aux_loss_note"] = (
            "load-balancing loss passes on the same workload (not part of the step): "
            "tokens per expert from the aux map, loss over the fp32 aux scores, and its "
            "gradient [T,E]; us_avg from back-to-back launches (HIP events on the launch "
            "stream), us_graph from a replayed HIP graph; a pass's time covers all of its "
            "kernels")
    if copy:
        out["copy_calibration"] = copy
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_tokens or T)
        if not args.only and not args.no_sweep:
            out["cpu_baseline_configs_sweep"] = cpu_configs_and_sweep(synth)
    if not args.only:
        out["decode_route"] = run_decode_route(torch, router, synth, args.steps)
        out["decode_route_note"] = (
            "decode-shape routing with expert maps (one workgroup): microseconds per call, "
            "T rows x E=512 experts x K, softmax renormalised, fp32")
        out["shared_gate"] = run_shared_gate(torch, router, synth)
        m16 = out["shared_gate"]["M16384"]
        m16["traffic"] = (read_traffic("shared_gate", "e512_h4096_m16384")
                          if not args.warm else None)
        out["shared_gate_note"] = (
            "routed softmax top-k with the shared-expert sigmoid gate: M tokens x E=512 x "
            "hidden 4096, top-10, one shared expert, bf16, renormalised; graph-replayed; "
            "GB/s = gating + hidden + gate rows read, weights and ids written")
    if not args.only and args.workload == "c4_softmax_2304x36":
        out["stream_ceiling"] = {f"T{T}_E{E}": run_stream_ceiling(torch, router, T, E),
                                 "T8192_E256": run_stream_ceiling(torch, router, 8192, 256)}
        # the dominant kernel against the two data-movement references of its
        # own pass mix: what the pass's bytes take with no arithmetic
        here = out["stream_ceiling"][f"T{T}_E{E}"]
        refs = {"stream_mix_us": here[roof["passes"][0]]["us"]}
        if roof["kernel"] == "fwd_kernel" and "topk_fwd_row_pattern" in here:
            refs["row_pattern_us"] = here["topk_fwd_row_pattern"]["us"]
        roof["ceilings"] = {k: v for k, v in refs.items()}
        roof["ceilings"].update({k.replace("_us", "_frac"): round(v / roof["us_avg"], 4)
                                 for k, v in refs.items()})
        if "aux_loss" in out and esz == 4:
            for kind, mix in LOSS_STREAM.items():
                c = here[mix]["us"]
                out["aux_loss"][kind]["stream_ceiling_us"] = c
                out["aux_loss"][kind]["stream_ceiling_frac"] = round(
                    c / out["aux_loss"][kind]["us_graph"], 4)
        out["stream_ceiling_note"] = (
            "the library's streaming kernel (16-byte non-temporal buffer loads and stores, no "
            "arithmetic; the fastest of 1, 2 and 4 units per thread, every load issued before "
            "its stores) moving each pass's bytes at its read:write mix over T*E elements, "
            "cold; the bandwidth a kernel with that mix can reach on this device, at the "
            "headline size and at the E=256 sweep cells' size (map_read: the byte map, the "
            "tokens-per-expert pass's bytes); topk_fwd_row_pattern moves "
            "the forward's bytes in the forward's own pattern (one wave per row, the row read "
            "whole, then two fp32 rows and a byte row written), no arithmetic")
    if not args.no_sweep and not args.only:
        out["grid_study"] = run_grid_study(torch, router, synth, np)
        out["grid_study_note"] = (
            "top-k forward and backward under the library's two grid modes: one block per "
            "token group (full, the default) and the occupancy-sized persistent grid "
            "(resident blocks per CU x CUs, waves loop over token groups); cells as configs")
        out["configs"] = run_configs(torch, router, synth, np)
        out["configs_note"] = (f"the five router workloads (c1..c5), cold: per pass a HIP graph "
                               f"of max({CELL_LAUNCHES}, sets) launches cycling through every "
                               f"rotating buffer set, replayed {CELL_REPLAYS} times; us = median "
                               f"per launch over the replays, p10/p90 beside it")
        t0 = time.perf_counter()
        out["sweep"] = run_sweep(torch, router, synth, np)
        out["sweep_note"] = (f"T=8192, per pass: us (median per launch over {CELL_REPLAYS} "
                             f"replays of a HIP graph of max({CELL_LAUNCHES}, sets) launches "
                             f"cycling through every rotating buffer set, >= 2 GiB: cold), "
                             f"p10/p90, GB/s from the median; softmax without renorm, sigmoid "
                             f"with renorm; {time.perf_counter() - t0:.1f} s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
