"""Host-side pieces of bench.py that the measurement relies on (CPU): the
workload names it accepts, the byte counts it divides by, the stream mixes
that stand for each pass, the source lists behind the profile-freshness
hash, and the one-GPU guard."""
import os
import re
import subprocess
import sys

import pytest

import bench
from score_function_top_amd import build, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_workload_names():
    for name, wl in synth.WORKLOADS.items():
        assert bench.workload_by_name(synth, name) is wl
    wl = bench.workload_by_name(synth, "sweep_sigmoid_2304x36")
    assert (wl.T, wl.E, wl.K, wl.score_fn, wl.dtype) == (8192, 2304, 36, synth.SIGMOID, synth.F32)
    wb = bench.workload_by_name(synth, "sweep_softmax_3072x8_bf16")
    assert (wb.E, wb.K, wb.score_fn, wb.dtype) == (3072, 8, synth.SOFTMAX, synth.BF16)
    assert wb.name == "sweep_softmax_3072x8_bf16"
    # the same seeds as the fp32 cell: only the storage type differs
    wf = bench.workload_by_name(synth, "sweep_softmax_3072x8")
    assert wb.seed_logits == wf.seed_logits and wb.seed_grad == wf.seed_grad
    for bad in ("sweep_softmax_3072x8_fp16", "sweep_relu_256x4", "c9_softmax_1x1"):
        with pytest.raises(SystemExit):
            bench.workload_by_name(synth, bad)


def test_pass_bytes():
    T, E = 8192, 2304
    # the router page's count: x + probs in the dtype, map 1 B, intermediate 4 B
    assert bench.STREAM_MIX["topk_fwd"] == (4, 9) and bench.STREAM_MIX["topk_bwd"] == (9, 4)
    assert bench.STREAM_MIX["aux_bwd"] == (8, 4)
    assert bench.loss_bytes("tokens_per_expert", T, E, 4) == T * E + E * 8
    assert bench.loss_bytes("aux_loss_fwd", T, E, 4) == T * E * 4 + E * 8 + 4
    # each aux-loss pass's stream stands for the pass's T*E bytes
    per_elem = {"tokens_per_expert": 1, "aux_loss_fwd": 4, "aux_loss_bwd": 4}
    for kind, mix in bench.LOSS_STREAM.items():
        r, w = bench.STREAM_MIX[mix]
        assert r + w == per_elem[kind], kind
    assert set(bench.STREAM_UNITS) <= {1, 2, 4, 8}


def test_hash_sources_cover_the_build():
    """Every kernel unit the build compiles is in the source list of the
    hash that marks committed counter summaries as current, so a kernel
    change cannot leave a stale summary looking fresh."""
    built = {s if isinstance(s, str) else s[0] for s in build.SOURCES}
    hashed = set()
    for files in bench.SYMBOL_SOURCES.values():
        hashed |= set(files)
    csrc = os.path.join(ROOT, "score_function_top_amd", "csrc")
    for f in hashed:
        assert os.path.exists(os.path.join(csrc, f)), f
    router_units = {f for f in built if re.match(r"router_(lpt\d+\w*|scalar\d*)\.hip$", f)}
    assert router_units and router_units <= set(bench._ROUTER_SOURCES)
    for unit, sym in (("router_loss.hip", "loss_kernel"), ("router_gate.hip", "shared_gate_kernel"),
                      ("router_grouped.hip", "grouped_fwd_kernel"),
                      ("router_route.hip", "route_maps_kernel")):
        assert unit in bench.SYMBOL_SOURCES[sym]
    # headers every kernel unit includes
    for sym in bench.SYMBOL_SOURCES:
        assert {"router_params.h", "router_io.h"} <= set(bench.SYMBOL_SOURCES[sym]), sym


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr
