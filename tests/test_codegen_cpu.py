"""Code-generation check of the HIP kernels (CPU only: hipcc cross-compiles
the kernel sources to gfx950 assembly, nothing runs).

A lane-divergent `if` compiles to `s_and_saveexec` ... `s_cbranch_execz L`,
and its join block L must restore the full lane mask (`s_or_b64 exec, exec,
...`) before any vector instruction that holds a value for every lane.  A
vector write placed ahead of that restore reaches only the lanes that took
the branch.  hipcc produced exactly that once in the element-wise 16-chunk
sigmoid forward: a register copy of one element's score sat ahead of the
restore of the branch that skipped the sigmoid on padding elements, so the
lanes holding padding stored another element's raw logit as the
intermediate.  The kernels now keep every such computation out of
lane-divergent branches; this test fails if any kernel's join block runs
vector instructions before its exec restore again.
"""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from score_function_top_amd import build

# kernel sources as (file, extra flags): the grouped kernels' file is built
# once per lane width
KERNEL_SOURCES = [(s, []) if isinstance(s, str) else (s[0], [f"-DROUTER_GROUPED_LPT={s[1]}"])
                  for s in build.SOURCES
                  if (s if isinstance(s, str) else s[0]).endswith(".hip")]


def join_block_writes(asm):
    """(kernel, label, instructions) for every join block (a target of
    s_cbranch_execz) with vector instructions ahead of its exec restore;
    lane reads/writes that ignore the mask (readlane, writelane) excepted."""
    lines = asm.split("\n")
    fn, targets, owner = None, set(), {}
    for line in lines:
        m = re.match(r"^(_Z\w+):", line)
        if m:
            fn = m.group(1)
        m = re.search(r"s_cbranch_execz (\.LBB\w+)", line)
        if m:
            targets.add(m.group(1))
            owner[m.group(1)] = fn
    found = []
    for i, line in enumerate(lines):
        m = re.match(r"^(\.LBB\w+):", line)
        if not m or m.group(1) not in targets:
            continue
        pre, restored = [], False
        for t in (x.strip() for x in lines[i + 1:i + 400]):
            if not t or t.startswith(";"):
                continue
            if re.match(r"s_or_b64 exec, exec, ", t):
                restored = True
                break
            if t.startswith((".LBB", "s_cbranch", "s_branch", "s_endpgm")) or "saveexec" in t:
                break  # the block ends without restoring this branch's mask
            pre.append(t)
        vec = [p for p in pre if p.startswith("v_")
               and not re.match(r"v_(readlane|readfirstlane|writelane)", p)]
        if restored and vec:
            found.append((owner[m.group(1)], m.group(1), vec))
    return found


def test_detector_flags_a_write_ahead_of_the_restore():
    asm = "\n".join([
        "_Zk:", "\ts_and_saveexec_b64 s[4:5], s[0:1]", "\ts_cbranch_execz .LBB0_2",
        "\tv_rcp_f32_e32 v0, v40", ".LBB0_2:", "\tv_mov_b32_e32 v174, v144",
        "\ts_or_b64 exec, exec, s[4:5]", "\ts_endpgm"])
    assert join_block_writes(asm) == [("_Zk", ".LBB0_2", ["v_mov_b32_e32 v174, v144"])]
    ok = asm.replace("\tv_mov_b32_e32 v174, v144\n\ts_or_b64 exec, exec, s[4:5]",
                     "\ts_or_b64 exec, exec, s[4:5]\n\tv_mov_b32_e32 v174, v144")
    assert join_block_writes(ok) == []
    # a skip target whose block never restores a mask is not this pattern
    skip = asm.replace("\ts_or_b64 exec, exec, s[4:5]\n", "")
    assert join_block_writes(skip) == []


def _asm(entry, out_dir):
    src, defs = entry
    out = os.path.join(out_dir, os.path.splitext(src)[0] + "".join(defs) + ".s")
    cmd = ["hipcc", *build.FLAGS, *defs, "--cuda-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{r.stderr[-2000:]}")
    return open(out).read()


def test_no_vector_writes_ahead_of_exec_restores(tmp_path):
    if subprocess.run(["which", "hipcc"], capture_output=True).returncode != 0:
        pytest.skip("hipcc not available")
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        asms = list(ex.map(lambda s: _asm(s, str(tmp_path)), KERNEL_SOURCES))
    bad = []
    for src, asm in zip(KERNEL_SOURCES, asms):
        bad += [(src[0],) + f for f in join_block_writes(asm)]
    assert not bad, "vector writes ahead of an exec restore:\n" + "\n".join(
        f"{s}: {k[:80]} {lbl} {ins[:3]}" for s, k, lbl, ins in bad[:20])
